// Host-side launchers of the gfx950 kernels (internal to libvit).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vit {

// Epilogue selector of the bf16 GEMM acc = A @ W^T.
enum EpiKind {
  EPI_BIAS_BF16 = 0,   // out_bf16[m,n] = acc + bias[n]
  EPI_GELU_BF16 = 1,   // out_bf16[m,n] = GELU(acc + bias[n])
  EPI_RESIDUAL = 2,    // out_f32[m,n] += ls[n] * (acc + bias[n])
  EPI_BIAS_F32 = 3,    // out_f32[m,n] = acc + bias[n]
  EPI_QKV = 4,         // head split into q (scaled), k, vt (transposed, permuted)
  EPI_PATCH = 5,       // residual row of patch token: acc + bias[n] + pos[1 + i][n]
  EPI_RESIDUAL_LN = 6, // EPI_RESIDUAL, then h = LayerNorm(out row) in bf16 (N = 384 only)
  EPI_CHAN_LN = 7,     // channel LayerNorm of the row (acc + bias), SiLU, optional second
                       // LayerNorm; bf16 into out + m * ldc + c0 (N = 128 or 256)
  EPI_BIAS_F32_G8 = 8, // out_f32 in column groups of 8: out[(n/8) * ldc + 8 m + n % 8] = acc + bias[n]
                       // (ldc >= 8 M; N a multiple of 8; 3x3 convolutions only)
};

struct EpiParams {
  int kind = EPI_BIAS_BF16;
  const float* bias = nullptr;
  const float* ls = nullptr;
  void* out = nullptr;   // [M, ldc]
  int ldc = 0;
  // EPI_QKV
  uint16_t* q = nullptr;
  uint16_t* k = nullptr;
  uint16_t* vt = nullptr;
  int tokens = 0;        // rows per image (N)
  int heads = 0;
  int nv = 0;            // row length of vt
  // EPI_PATCH: rows m = b * patches + i go to residual row b * tokens + 1 + regs + i
  const float* pos = nullptr;
  int patches = 0;
  int regs = 0;
  // EPI_RESIDUAL_LN, EPI_CHAN_LN
  const float* ln_g = nullptr;
  const float* ln_b = nullptr;
  float eps = 0.f;
  uint16_t* h = nullptr;
  // EPI_RESIDUAL_LN: a region (16-byte aligned, < 4 GiB) that workgroups on
  // the CUs the row tiles leave idle read into the caches, or null
  const void* prefetch = nullptr;
  size_t prefetch_bytes = 0;
  // EPI_CHAN_LN (out is bf16 here)
  int c0 = 0;
  bool silu = false;
  const float* ln2_g = nullptr;  // second LayerNorm (after SiLU) if non-null
  const float* ln2_b = nullptr;
};

// Widths for which launch_gemm / launch_gemm_conv3 fuse the channel LayerNorm.
constexpr bool chan_ln_fusable(int n) { return n == 128 || n == 256; }

// Widths for which launch_gemm fuses the LayerNorm after a residual update.
constexpr bool residual_ln_fusable(int n) { return n == 384; }

// 3x3 / stride 1 / pad 1 convolution as an implicit GEMM: A rows are the
// pixels of in [batch * gh * gw, ld_in] (channels c0 .. c0 + C, C a multiple
// of 64), columns in (ky, kx, c) order, read in place with zeros outside the
// grid; W [N, 9 C].  Epilogues EPI_BIAS_BF16 and EPI_BIAS_F32.
hipError_t launch_gemm_conv3(const uint16_t* in, int ld_in, int c0, int C, int batch, int gh, int gw,
                             const uint16_t* W, int N, const EpiParams& ep, hipStream_t s);

// fp8 (OCP E4M3) GEMM: out[m, n] = scale * sum_k A[m, k] W[n, k] + bias[n]
// (bias may be null) with A [M, K], W [N, K] as E4M3 codes, K a multiple of
// 128; out fp32 or bf16 [M, ldc].
hipError_t launch_gemm_fp8(const uint8_t* A, const uint8_t* W, int M, int N, int K, float scale, const float* bias,
                           void* out, int ldc, bool out_f32, hipStream_t s);

// E4M3 codes of x[i] * s_inv (product in fp32; nearest value, ties to even,
// saturated to +-448, sign kept, NaN -> 0x7F); x fp32 (x_bf16 == false) or bf16.
hipError_t launch_quantize_fp8(const void* x, bool x_bf16, size_t n, float s_inv, uint8_t* out, hipStream_t s);
// int8 codes of x * s_inv (nearest, ties to even, clamped to +-127, NaN -> 0).
hipError_t launch_quantize_int8(const void* x, bool x_bf16, size_t n, float s_inv, int8_t* out, hipStream_t s);
// int8 GEMM: out[m, n] = scale * sum_k A[m, k] W[n, k] + bias[n], the sums exact
// in int32 (K <= 131072), then converted to fp32; K a multiple of 128.
hipError_t launch_gemm_int8(const int8_t* A, const int8_t* W, int M, int N, int K, float scale, const float* bias,
                            void* out, int ldc, bool out_f32, hipStream_t s);

// amax[0] = max |x[i]| over n fp32 (or bf16) values (NaN ignored); amax is written, not accumulated.
hipError_t launch_absmax(const void* x, bool x_bf16, size_t n, float* amax, hipStream_t s);

// One-time per-device set-up of the GEMM epilogues (the GELU Phi table; a
// synchronous copy).  launch_gemm does it on first use; encoders call it at
// creation so that no later launch copies.
hipError_t prepare_gemm();

hipError_t launch_gemm(const uint16_t* A, const uint16_t* W, int M, int N, int K, const EpiParams& ep,
                       hipStream_t s);

// LayerNorm of rows of x [rows, dim] into bf16 (out_f32 == false) or fp32.
hipError_t launch_layernorm(const float* x, int rows, int dim, const float* g, const float* b, float eps,
                            void* y, bool out_f32, hipStream_t s);

// Taps: LayerNorm of the patch rows of x [batch, tokens, dim], written
// channel-first to taps + b * tap_stride + (d * patches + i).
hipError_t launch_tap(const float* x, int batch, int tokens, int first_patch, int patches, int dim,
                      const float* g, const float* b, float eps, float* taps, size_t tap_stride,
                      hipStream_t s);

// Patch features for scoring: LayerNorm then L2 normalisation of the patch
// rows, bf16 out [batch * patches, dim].
hipError_t launch_ln_l2(const float* x, int batch, int tokens, int first_patch, int patches, int dim,
                        const float* g, const float* b, float eps, uint16_t* feats, hipStream_t s);

// Descriptor: desc[b] = x[b * row_stride + 0..dim) / max(||.||, 1e-12).
hipError_t launch_descriptor(const float* x, int batch, size_t row_stride, int dim, float* desc,
                             hipStream_t s);

// 8-bit HWC frames [batch, sh, sw, 3] -> ImageNet-normalised fp32 CHW
// [batch, 3, dh, dw] (bilinear, half-pixel centres; bgr: channel order B, G, R).
hipError_t launch_preprocess(const uint8_t* frames, int batch, int sh, int sw, bool bgr, float* out, int dh, int dw,
                             hipStream_t s);

// im2col of fp32 images [batch, 3, H, W] into bf16 [batch * gh * gw, kpad]
// with columns in (c, ky, kx) order, zero beyond 3 p^2.  With x non-null the
// same launch also writes token rows 0..regs of every image of x [batch,
// tokens, dim]: CLS + pos0, then the registers reg [regs, dim].
hipError_t launch_patchify(const float* img, int batch, int H, int W, int p, int kpad, uint16_t* out, float* x,
                           int tokens, int dim, const float* cls, const float* pos0, const float* reg, int regs,
                           hipStream_t s);

// Bicubic (a = -0.75, half-pixel centres, clamped taps) resampling of the
// patch rows of a position table; row 0 copied.
hipError_t launch_pos_resample(const float* pos_in, int gh, int gw, float* pos_out, int th, int tw, int dim,
                               hipStream_t s);

// Attention core (see vit_op_attention); no workspace.  Extra workgroups
// read [prefetch, prefetch + prefetch_bytes) (16-byte aligned, < 4 GiB; may be null)
// and discard it, so that a later kernel finds it in the last-level cache.
hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int batch, int tokens,
                            int heads, int nv, uint16_t* o, const void* prefetch, size_t prefetch_bytes,
                            hipStream_t s);

// ---- semantic head (channels-last activations, one row per pixel)
// Taps [batch, ntaps, D, P] fp32 (channel-first) -> out bf16 [batch * P, ntaps * D].
hipError_t launch_taps_cl(const float* taps, int batch, int ntaps, int D, int P, uint16_t* out, hipStream_t s);
// GroupNorm (C = 8 * groups) per image, affine, exact GELU -> bf16 [batch * P, C].  x is
// group-major fp32 (EPI_BIAS_F32_G8's layout): group j's 8 channels of pixel row m at
// x + j * gstride + 8 m (gstride >= 8 * batch * P).
hipError_t launch_groupnorm_gelu(const float* x, size_t gstride, int batch, int P, int C, int groups, const float* g,
                                 const float* b, float eps, uint16_t* out, hipStream_t s);
// Bilinear resize (half-pixel centres) of class-minor in [batch * gh * gw, ldi]
// to out [batch, classes, H, W] fp32.
hipError_t launch_resize_nchw(const float* in, int ldi, int classes, int batch, int gh, int gw, float* out, int H,
                              int W, hipStream_t s);

// fp32 -> bf16 (nearest even) of n values.
hipError_t launch_to_bf16(const float* x, size_t n, uint16_t* y, hipStream_t s);

// Slide-mode crops: out[w] = img[:, y_w : y_w + side, x_w : x_w + side].
hipError_t launch_crops(const float* img, int H, int W, const int* corners_dev, int nwin, int side, float* out,
                        hipStream_t s);

// Whole mode: bilinear upsample of cos [gh*gw, ldc] (class-minor) to H x W,
// first argmax over classes; dense [C, H, W] written if non-null.
hipError_t launch_upsample_argmax(const float* cos, int gh, int gw, int classes, int ldc, int H, int W,
                                  int* labels, float* dense, hipStream_t s);

// Slide mode: per window upsample + softmax over classes, accumulate with
// overlap counts, average, first argmax.
hipError_t launch_slide_merge(const float* cos, int nwin, const int* corners_dev, int wg, int classes, int ldc,
                              int side, int H, int W, int* labels, float* dense, hipStream_t s);

// Transpose cos [rows = nimg * g, ldc] into [nimg, classes, g] (for the low-resolution output).
hipError_t launch_cos_out(const float* cos, int nimg, int g, int classes, int ldc, float* out, hipStream_t s);

}  // namespace vit
