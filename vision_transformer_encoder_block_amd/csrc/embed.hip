// Input side of the encoder on gfx950: 8-bit frame preprocessing (resize +
// ImageNet normalisation), im2col of the fp32 images into the bf16 patch
// matrix (the A operand of the patch-embedding GEMM), CLS/register rows of the
// token sequence, bicubic resampling of the position table, the slide-mode
// window crops and a plain fp32 -> bf16 conversion.
#include "common.h"
#include "kernels.h"

namespace vit {
namespace {

struct PatchArgs {
  const float* img;
  bf16_t* out;
  int H, W, p, kpad, gw, gh;
  uint32_t per_image;   // patch rows x 16-byte chunks of one image
  int patch_blocks;     // workgroups per image for the patch matrix
  FastDiv div_chunks, div_gw, div_pp, div_p;
  bool vec4;
  // token rows 0..regs (null x: none)
  float* x;
  int tokens, dim, regs;
  const float* cls;
  const float* pos0;
  const float* reg;
};

// grid (patch_blocks [+ 1 + regs], batch).  In the patch blocks one thread
// writes 8 consecutive columns (16 bytes) of one patch row.  The (c, ky, kx)
// of the first column is decoded once and then stepped; when the 8 columns
// lie in one image row (vec4: p a multiple of 8, W a multiple of 4 and img
// 16-byte aligned, checked on the host) they are two float4 loads.  Index
// arithmetic is 32-bit with multiply-high divisions (per-image counts below
// 2^31, checked on the host).  The blocks after them write the CLS row (CLS +
// pos[0]) and the register rows of the token sequence, which the patch
// embedding GEMM leaves alone.
__global__ __launch_bounds__(256) void patchify_kernel(PatchArgs a) {
  const int b = blockIdx.y;
  if ((int)blockIdx.x >= a.patch_blocks) {
    const int r = blockIdx.x - a.patch_blocks;  // 0 = CLS, 1..regs = registers
    float* row = a.x + ((size_t)b * a.tokens + r) * a.dim;
    for (int c = threadIdx.x; c < a.dim; c += blockDim.x)
      row[c] = r == 0 ? a.cls[c] + a.pos0[c] : a.reg[(size_t)(r - 1) * a.dim + c];
    return;
  }
  const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= a.per_image) return;
  const int p = a.p, W = a.W, H = a.H;
  const uint32_t prow = fdiv(idx, a.div_chunks);
  const int ch = (int)(idx - prow * (uint32_t)(a.kpad / 8));
  const uint32_t gy = fdiv(prow, a.div_gw);
  const int gx = (int)(prow - gy * (uint32_t)a.gw);
  const int kvalid = 3 * p * p;
  const int k0 = ch * 8;
  float v[8];
  if (k0 >= kvalid) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  } else {
    int c = (int)fdiv((uint32_t)k0, a.div_pp);
    const int r = k0 - c * p * p;
    int ky = (int)fdiv((uint32_t)r, a.div_p), kx = r - ky * p;
    const float* base = a.img + (size_t)b * 3 * H * W + (size_t)(gy * p) * W + gx * p;
    if (a.vec4 && k0 + 8 <= kvalid) {
      const float4* src = reinterpret_cast<const float4*>(base + ((size_t)c * H + ky) * W + kx);
      const float4 lo = src[0], hi = src[1];
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = (k0 + e < kvalid) ? base[((size_t)c * H + ky) * W + kx] : 0.f;
        if (++kx == p) {
          kx = 0;
          if (++ky == p) {
            ky = 0;
            ++c;
          }
        }
      }
    }
  }
  uint4 u = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
  *reinterpret_cast<uint4*>(a.out + ((size_t)b * a.gh * a.gw + prow) * a.kpad + ch * 8) = u;
}

// Cubic-convolution weight (a = -0.75) of a tap at distance d.
__device__ __forceinline__ float cubic_w(float d) {
  const float a = -0.75f;
  d = fabsf(d);
  if (d <= 1.f) return ((a + 2.f) * d - (a + 3.f)) * d * d + 1.f;
  if (d < 2.f) return ((a * d - 5.f * a) * d + 8.f * a) * d - 4.f * a;
  return 0.f;
}

// One thread per (output row, channel); 4 x 4 taps with edge clamping.
__global__ __launch_bounds__(256) void pos_resample_kernel(const float* __restrict__ in, int gh, int gw,
                                                           float* __restrict__ out, int th, int tw, int dim) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)(1 + th * tw) * dim;
  if (idx >= total) return;
  const int c = (int)(idx % dim);
  const int row = (int)(idx / dim);
  if (row == 0) {
    out[c] = in[c];
    return;
  }
  const int oy = (row - 1) / tw, ox = (row - 1) % tw;
  const float sy = (oy + 0.5f) * ((float)gh / th) - 0.5f;
  const float sx = (ox + 0.5f) * ((float)gw / tw) - 0.5f;
  const int y0 = (int)floorf(sy), x0 = (int)floorf(sx);
  float acc = 0.f;
  for (int ty = -1; ty <= 2; ++ty) {
    const float wy = cubic_w(sy - (float)(y0 + ty));
    const int yy = min(max(y0 + ty, 0), gh - 1);
    float racc = 0.f;
    for (int tx = -1; tx <= 2; ++tx) {
      const float wx = cubic_w(sx - (float)(x0 + tx));
      const int xx = min(max(x0 + tx, 0), gw - 1);
      racc += wx * in[(size_t)(1 + yy * gw + xx) * dim + c];
    }
    acc += wy * racc;
  }
  out[(size_t)row * dim + c] = acc;
}

__global__ __launch_bounds__(256) void crops_kernel(const float* __restrict__ img, int H, int W,
                                                    const int* __restrict__ corners, int side,
                                                    float* __restrict__ out) {
  const int w = blockIdx.z;
  const int c = blockIdx.y;
  const int y0 = corners[2 * w], x0 = corners[2 * w + 1];
  const size_t n = (size_t)side * side;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int yy = (int)(i / side), xx = (int)(i % side);
    out[(((size_t)w * 3 + c) * side + yy) * side + xx] = img[((size_t)c * H + y0 + yy) * W + x0 + xx];
  }
}

// Frame preprocessing.  Bilinear sample (half-pixel centres, coordinates
// clamped at the edges) of the three 8-bit channels, scaled by 1/255 and
// normalised with the ImageNet mean/std (RGB order), written to three planes.
// bgr: the frame stores B, G, R.
constexpr float kMean[3] = {0.485f, 0.456f, 0.406f};
constexpr float kInvStd[3] = {1.f / 0.229f, 1.f / 0.224f, 1.f / 0.225f};

// Byte j of source row 0 is r0[o0 + j] (row 1: r1[o1 + j]); o0 and o1 may be
// negative, but every byte read, o + 3 x + c, is an index into the rows' data.
__device__ __forceinline__ void preprocess_pixel(const uint8_t* r0, int o0, const uint8_t* r1, int o1, int x0, int x1,
                                                 float lx, float ly, bool bgr, float* o, size_t plane) {
#pragma unroll
  for (int oc = 0; oc < 3; ++oc) {
    const int c = bgr ? 2 - oc : oc;
    const float top = (1.f - lx) * (float)r0[o0 + x0 * 3 + c] + lx * (float)r0[o0 + x1 * 3 + c];
    const float bot = (1.f - lx) * (float)r1[o1 + x0 * 3 + c] + lx * (float)r1[o1 + x1 * 3 + c];
    const float v = (1.f - ly) * top + ly * bot;
    o[oc * plane] = (v * (1.f / 255.f) - kMean[oc]) * kInvStd[oc];
  }
}

// One workgroup per output row (y, image b).  The byte span of the two source
// rows that the row's samples touch is copied to LDS with 16-byte loads (span
// ends rounded out to 16 bytes, never used; a chunk that would reach past the
// frames' last byte is read byte by byte), then every thread blends output
// pixels x = tid, tid + 256, ...
// from LDS: the frames are read once, in wide coalesced loads, instead of
// twelve scattered byte loads per output pixel.
constexpr int kPreSpanMax = 12288;  // LDS bytes per source row (4096 RGB pixels)

__global__ __launch_bounds__(256) void preprocess_rows_kernel(const uint8_t* __restrict__ frames, uint32_t total_bytes,
                                                              int sh, int sw, float* __restrict__ out, int dh, int dw,
                                                              bool bgr) {
  __shared__ uint4 rows[2][kPreSpanMax / 16 + 1];
  const int y = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int y0, y1, xa, xb, xc, xd;
  float ly, lx;
  bilinear_tap(y, sh, dh, y0, y1, ly);
  bilinear_tap(0, sw, dw, xa, xb, lx);
  bilinear_tap(dw - 1, sw, dw, xc, xd, lx);
  const uint32_t frame = (uint32_t)b * (uint32_t)sh * (uint32_t)sw * 3u;
  const uint32_t span_lo = (uint32_t)xa * 3u, span_hi = (uint32_t)(xd + 1) * 3u;  // bytes within a row
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(frames, total_bytes);
  uint32_t base[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint32_t lo = frame + (uint32_t)(r ? y1 : y0) * (uint32_t)sw * 3u + span_lo;
    base[r] = lo & ~15u;
    const uint32_t n16 = (lo + (span_hi - span_lo) - base[r] + 15u) / 16u;
    for (uint32_t i = tid; i < n16; i += 256) {
      const uint32_t at = base[r] + 16u * i;
      if (at + 16u <= total_bytes) {
        rows[r][i] = buf_load16(rs, at);
      } else {  // the chunk that reaches past the frames' last byte: byte loads
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (uint32_t j = 0; j < 16u && at + j < total_bytes; ++j) w[j >> 2] |= (uint32_t)frames[at + j] << (8 * (j & 3));
        rows[r][i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
  __syncthreads();
  // LDS row r holds global bytes from base[r] on; source byte j of row r is
  // LDS byte j + (row start - base[r]), with row start - base[r] in
  // [-span_lo, 15 - span_lo], so bytes j >= span_lo land at LDS bytes >= 0
  const int o0 = (int)(frame + (uint32_t)y0 * (uint32_t)sw * 3u - base[0]);
  const int o1 = (int)(frame + (uint32_t)y1 * (uint32_t)sw * 3u - base[1]);
  const uint8_t* l0 = reinterpret_cast<const uint8_t*>(rows[0]);
  const uint8_t* l1 = reinterpret_cast<const uint8_t*>(rows[1]);
  const size_t plane = (size_t)dh * dw;
  float* o = out + (size_t)b * 3 * plane + (size_t)y * dw;
  for (int x = tid; x < dw; x += 256) {
    int x0, x1;
    bilinear_tap(x, sw, dw, x0, x1, lx);
    preprocess_pixel(l0, o0, l1, o1, x0, x1, lx, ly, bgr, o + x, plane);
  }
}

// Frames whose row span does not fit the LDS buffer (or whose batch needs
// offsets of 32 bits or more): one thread per output pixel, reading the
// frames directly.
__global__ __launch_bounds__(256) void preprocess_kernel(const uint8_t* __restrict__ frames, int sh, int sw,
                                                         float* __restrict__ out, int dh, int dw, bool bgr) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= dw) return;
  const int y = blockIdx.y, b = blockIdx.z;
  int y0, y1, x0, x1;
  float ly, lx;
  bilinear_tap(y, sh, dh, y0, y1, ly);
  bilinear_tap(x, sw, dw, x0, x1, lx);
  const uint8_t* f = frames + (size_t)b * sh * sw * 3;
  const size_t plane = (size_t)dh * dw;
  preprocess_pixel(f + (size_t)y0 * sw * 3, 0, f + (size_t)y1 * sw * 3, 0, x0, x1, lx, ly, bgr,
                   out + (size_t)b * 3 * plane + (size_t)y * dw + x, plane);
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ x, size_t n, bf16_t* __restrict__ y) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = f2bf(x[i]);
}

}  // namespace

hipError_t launch_patchify(const float* img, int batch, int H, int W, int p, int kpad, uint16_t* out, float* x,
                           int tokens, int dim, const float* cls, const float* pos0, const float* reg, int regs,
                           hipStream_t s) {
  if (batch < 1 || batch > 65535 || p < 1 || kpad % 8 != 0 || kpad < 3 * p * p || regs < 0) return hipErrorInvalidValue;
  const int gw = W / p, gh = H / p;
  const size_t per_image = (size_t)gh * gw * (kpad / 8);
  if (per_image >= (1ull << 31)) return hipErrorInvalidValue;
  PatchArgs a{};
  a.img = img;
  a.out = reinterpret_cast<bf16_t*>(out);
  a.H = H, a.W = W, a.p = p, a.kpad = kpad, a.gw = gw, a.gh = gh;
  a.per_image = (uint32_t)per_image;
  a.patch_blocks = (int)((per_image + 255) / 256);
  a.div_chunks = make_fastdiv((uint32_t)(kpad / 8));
  a.div_gw = make_fastdiv((uint32_t)(gw > 0 ? gw : 1));
  a.div_pp = make_fastdiv((uint32_t)(p * p));
  a.div_p = make_fastdiv((uint32_t)p);
  a.vec4 = (p % 8) == 0 && (W % 4) == 0 && (reinterpret_cast<uintptr_t>(img) % 16) == 0;
  a.x = x, a.tokens = tokens, a.dim = dim, a.regs = regs, a.cls = cls, a.pos0 = pos0, a.reg = reg;
  const int blocks = a.patch_blocks + (x ? 1 + regs : 0);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(patchify_kernel, dim3((unsigned)blocks, (unsigned)batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pos_resample(const float* pos_in, int gh, int gw, float* pos_out, int th, int tw, int dim,
                               hipStream_t s) {
  const size_t total = (size_t)(1 + th * tw) * dim;
  hipLaunchKernelGGL(pos_resample_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, pos_in, gh, gw,
                     pos_out, th, tw, dim);
  return hipGetLastError();
}

hipError_t launch_crops(const float* img, int H, int W, const int* corners_dev, int nwin, int side, float* out,
                        hipStream_t s) {
  hipLaunchKernelGGL(crops_kernel, dim3(64, 3, nwin), dim3(256), 0, s, img, H, W, corners_dev, side, out);
  return hipGetLastError();
}

hipError_t launch_preprocess(const uint8_t* frames, int batch, int sh, int sw, bool bgr, float* out, int dh, int dw,
                             hipStream_t s) {
  if (batch < 1 || sh < 1 || sw < 1 || dh < 1 || dw < 1 || batch > 65535 || dh > 65535)
    return hipErrorInvalidValue;
  // source byte span of one output row, rounded out to 16 bytes at both ends
  int xa, xb, xc, xd;
  float w;
  bilinear_tap(0, sw, dw, xa, xb, w);
  bilinear_tap(dw - 1, sw, dw, xc, xd, w);
  const size_t span = (size_t)(xd + 1 - xa) * 3 + 30;
  const size_t total = (size_t)batch * sh * sw * 3;
  if (span <= (size_t)kPreSpanMax && total + 64 < (1ull << 32)) {
    hipLaunchKernelGGL(preprocess_rows_kernel, dim3((unsigned)dh, (unsigned)batch), dim3(256), 0, s, frames,
                       (uint32_t)total, sh, sw, out, dh, dw, bgr);
  } else {
    hipLaunchKernelGGL(preprocess_kernel, dim3((unsigned)((dw + 255) / 256), dh, batch), dim3(256), 0, s, frames, sh,
                       sw, out, dh, dw, bgr);
  }
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* x, size_t n, uint16_t* y, hipStream_t s) {
  hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, n, y);
  return hipGetLastError();
}

}  // namespace vit
