/*
 * vit_ops.h - the individual kernels of the encoder block, exposed for
 * per-operation checking and for callers composing their own blocks.
 *
 * Same conventions as vit.h: raw device pointers owned by the caller, fp32
 * unless stated, bf16 = IEEE-754 binary32 truncated to its upper 16 bits
 * (stored as uint16, produced by round-to-nearest-even), work enqueued on
 * `stream` without synchronisation, 0 on success or a negative vit_status
 * with a message in vit_last_error().
 */
#ifndef VIT_OPS_H
#define VIT_OPS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Frame preprocessing, the step right before the encoder: 8-bit HWC frames
 * to the ImageNet-normalised RGB CHW input of the model card ("Model I/O":
 * mean (0.485, 0.456, 0.406), std (0.229, 0.224, 0.225)), resized like the
 * deployment article's service (cv2.resize default: bilinear, half-pixel
 * centres, edge pixels replicated) and scaled by 1/255.
 *   frames [batch, src_h, src_w, 3] uint8, rows packed (stride src_w * 3);
 *   bgr != 0: channels stored B, G, R (cv2 decode order), else R, G, B.
 *   images [batch, 3, dst_h, dst_w] fp32 (the d_images of vit_forward).
 *   The resampled values are not rounded back to 8 bits.
 *   batch and dst_h at most 65535; all sizes >= 1.  Device pointers, caller-
 *   owned; enqueue only.  VIT_ERR_ARG for NULL pointers, VIT_ERR_SHAPE for
 *   sizes out of range. */
int vit_op_preprocess(const void* frames, int batch, int src_h, int src_w, int bgr, float* images, int dst_h,
                      int dst_w, void* stream);

/* LayerNorm over the last axis (LibreYOLO DINOv2 diagram, "Encoder block":
 * LayerNorm eps 1e-6): y = (x - mean) / sqrt(var + eps) * g + b, biased var.
 *   x [rows, dim] fp32; g, b [dim]; y [rows, dim], bf16 if out_fp32 == 0 else fp32.
 *   dim must be a multiple of 64 and <= 4096; x, g, b, y 16-byte aligned. */
int vit_op_layernorm(const float* x, int rows, int dim, const float* g, const float* b, float eps,
                     void* y, int out_fp32, void* stream);

/* Epilogues of vit_op_linear. */
enum vit_epilogue {
  VIT_EPI_BIAS_BF16 = 0,   /* c_bf16[m,n] = bf16(acc + bias[n]) */
  VIT_EPI_GELU_BF16 = 1,   /* c_bf16[m,n] = bf16(GELU(acc + bias[n])), GELU(z) = z Phi(z) with the
                              normal CDF Phi linearly interpolated between points 1/64 apart
                              (|error of Phi| <= 7.4e-6; Phi = 0 / 1 beyond -6 / 6) */
  VIT_EPI_RESIDUAL = 2,    /* c_f32[m,n] += ls[n] * (acc + bias[n])  (LayerScale + residual) */
  VIT_EPI_BIAS_F32 = 3     /* c_f32[m,n] = acc + bias[n]  (bias may be NULL: 0) */
};

/* Linear layer acc = a @ w^T (torch.nn.Linear; LibreYOLO diagram "Encoder
 * block" Linear D->Hm and Hm->D, "Encoder self-attention" Linear output).
 *   a [M,K] bf16 row-major, w [N,K] bf16 row-major, bias [N] fp32,
 *   ls [N] fp32 (RESIDUAL only), c [M,N] (bf16 or fp32 per epilogue).
 *   K must be a multiple of 64; M, N >= 1. */
int vit_op_linear(const void* a, const void* w, const float* bias, int M, int N, int K,
                  int epilogue, const float* ls, void* c, void* stream);

/* Residual update and the LayerNorm after it, in one GEMM whose tiles span
 * whole rows (LibreYOLO DINOv2 diagram, "Encoder block": the output Linear
 * (or the second MLP Linear), LayerScale, residual add, then the next block
 * step's LayerNorm, eps inside the square root):
 *   x[m, :] += ls * (a[m, :] w^T + bias);   h[m, :] = LayerNorm(x[m, :]; g, b, eps)
 *   a [M, K] bf16, w [N, K] bf16, bias, ls, g, b [N] fp32, x [M, N] fp32
 *   (updated in place), h [M, N] bf16.  N must be 384 (VIT_ERR_UNSUPPORTED
 *   otherwise), K a positive multiple of 64; float vectors and x 16-byte
 *   aligned, h 8-byte aligned.  x and h equal, bit for bit, vit_op_linear
 *   with VIT_EPI_RESIDUAL followed by vit_op_layernorm. */
int vit_op_linear_residual_ln(const void* a, const void* w, const float* bias, const float* ls, int M, int N, int K,
                              float* x, const float* g, const float* b, float eps, void* h, void* stream);

/* Fused Q/K/V projection with the head split of the attention kernel
 * (LibreYOLO diagram, "Encoder self-attention": Linear Q/K/V, reshape heads).
 *   h [batch*tokens, D] bf16 (LayerNorm output), wqkv [3D, D] bf16 (rows: the
 *   D rows of wq, then wk, then wv), bqkv [3D] fp32, D = 64*heads.
 * Outputs (bf16), with Nv = tokens rounded up to a multiple of 64:
 *   q  [batch, heads, tokens, 64]  = (h wq^T + bq) * log2(e) / sqrt(64)
 *   k  [batch, heads, tokens, 64]  = h wk^T + bk
 *   vt [batch, heads, 64, Nv]      = (h wv^T + bv) transposed per head; token t
 *        is stored at column t with bits 2 and 3 of t exchanged (so the eight
 *        tokens one MFMA lane consumes are contiguous).  Columns >= tokens are
 *        not written. */
int vit_op_qkv(const void* h, const void* wqkv, const float* bqkv, int batch, int tokens,
               int heads, void* q, void* k, void* vt, void* stream);

/* Multi-head attention core, O = softmax(Q K^T / sqrt(64)) V per (batch, head)
 * with the softmax over keys (LibreYOLO diagram, "Encoder self-attention";
 * the logits stay fp32, model card "Build BF16, not FP16").
 *   q, k, vt as produced by vit_op_qkv (the columns >= tokens of vt are
 *   ignored, whatever they hold); o [batch, tokens, heads*64] bf16 (heads
 *   merged in channel order).  No scratch memory is used.  Every query's
 *   output comes from one pass over all keys, so an image's result does not
 *   depend on the batch it is in. */
int vit_op_attention(const void* q, const void* k, const void* vt, int batch, int tokens, int heads,
                     void* o, void* stream);

/* ---- low-precision (fp8) linear layer -------------------------------------
 * The encoder's Linear layers (LibreYOLO DINOv2 diagram, "Encoder block") with
 * both operands in 8-bit floating point, the OCP E4M3 format gfx950's matrix
 * cores read: 1 sign, 4 exponent (bias 7) and 3 mantissa bits; largest finite
 * magnitude 448; codes 0x7F / 0xFF are NaN; no infinity.  The DINOv2
 * deployment article discusses reduced-precision (INT8) engines; E4M3 is the
 * 8-bit format of these matrix cores.  Scales are per tensor. */

/* amax[0] = max_i |x[i]| (NaN ignored) over n values of x, fp32 (x_bf16 = 0)
 * or bf16 (x_bf16 = 1); amax is a device float, overwritten. */
int vit_op_absmax(const void* x, int x_bf16, size_t n, float* amax, void* stream);

/* E4M3 codes: out[i] = E4M3(x[i] * s_inv), the product rounded to fp32 first,
 * then the nearest E4M3 value with ties to the even mantissa, magnitudes past
 * 448 (and infinities) saturated to +-448, the sign kept (also when the value
 * rounds to zero), NaN -> 0x7F.  x fp32 or bf16 [n]; out uint8 [n], 4-byte
 * aligned.  A per-tensor scale s = amax / 448 maps the largest magnitude to
 * the largest code (s_inv = 1 / s). */
int vit_op_quantize_fp8(const void* x, int x_bf16, size_t n, float s_inv, void* out, void* stream);

/* out[m, n] = scale * sum_k A[m, k] W[n, k] + bias[n] with A [M, K] and W
 * [N, K] E4M3 codes (uint8, row-major, K contiguous), scale = s_a * s_w the
 * product of the operands' scales, bias [N] fp32 or NULL, out [M, N] fp32
 * (out_f32 = 1) or bf16.  K must be a multiple of 128.  Products of two E4M3
 * values are exact in fp32; the sums are fp32. */
int vit_op_linear_fp8(const void* a, const void* w, int M, int N, int K, float scale, const float* bias, void* out,
                      int out_f32, void* stream);

/* ---- low-precision (int8) linear layer ------------------------------------
 * The same Linear layer with 8-bit integer operands (the DINOv2 deployment
 * article's INT8 engines), on gfx950's int8 matrix cores
 * (v_mfma_i32_32x32x32_i8).  Quantisation is symmetric with one scale per
 * tensor: a scale s = amax / 127 (vit_op_absmax) maps the largest magnitude to
 * the largest code. */

/* int8 codes: out[i] = the integer nearest to x[i] * s_inv (the product rounded
 * to fp32 first), ties to even, clamped to [-127, 127] (infinities included;
 * the code -128 is never produced), NaN -> 0.  x fp32 or bf16 [n]; out int8
 * [n], 4-byte aligned; s_inv finite. */
int vit_op_quantize_int8(const void* x, int x_bf16, size_t n, float s_inv, void* out, void* stream);

/* out[m, n] = scale * sum_k A[m, k] W[n, k] + bias[n] with A [M, K] and W
 * [N, K] int8 codes (row-major, K contiguous), scale = s_a * s_w, bias [N]
 * fp32 or NULL, out [M, N] fp32 (out_f32 = 1) or bf16.  K must be a multiple
 * of 128 and at most 131072, so that the int32 sums (exact) cannot overflow;
 * each sum is then rounded to fp32 (nearest even) and out = fma(sum, scale,
 * bias) in fp32, rounded to bf16 (nearest even) for bf16 output. */
int vit_op_linear_int8(const void* a, const void* w, int M, int N, int K, float scale, const float* bias, void* out,
                       int out_f32, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VIT_OPS_H */
