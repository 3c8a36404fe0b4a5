// Zero-shot patch-text scoring tail on gfx950: bilinear upsampling of the
// per-patch class scores (half-pixel centres, source clamped at 0 and at the
// last row/column), fused with the per-pixel argmax over classes (whole mode)
// or with the per-window softmax, overlap accumulation, averaging and argmax
// (slide mode).  One thread per output pixel; the class-minor score layout
// makes the class loop read contiguous memory for each of the four source
// patches, and the [C, H, W] score volume is never materialised unless a
// dense output is requested.
#include "common.h"
#include "kernels.h"

namespace vit {
namespace {

constexpr int MAXW = 16;  // windows covering one pixel

struct Bilin {
  int i00, i01, i10, i11;  // source rows (patch indices)
  float w00, w01, w10, w11;
};

__device__ __forceinline__ void axis(int o, int n_out, int n_in, int& i0, int& i1, float& l) {
  float src = ((float)o + 0.5f) * ((float)n_in / (float)n_out) - 0.5f;
  src = fmaxf(src, 0.f);
  i0 = min((int)floorf(src), n_in - 1);
  i1 = min(i0 + 1, n_in - 1);
  l = src - (float)i0;
}

__device__ __forceinline__ Bilin bilin(int y, int x, int H, int W, int gh, int gw) {
  int y0, y1, x0, x1;
  float ly, lx;
  axis(y, H, gh, y0, y1, ly);
  axis(x, W, gw, x0, x1, lx);
  Bilin b;
  b.i00 = y0 * gw + x0;
  b.i01 = y0 * gw + x1;
  b.i10 = y1 * gw + x0;
  b.i11 = y1 * gw + x1;
  b.w00 = (1.f - ly) * (1.f - lx);
  b.w01 = (1.f - ly) * lx;
  b.w10 = ly * (1.f - lx);
  b.w11 = ly * lx;
  return b;
}

__device__ __forceinline__ float interp(const float* __restrict__ cos, int ldc, const Bilin& b, int c) {
  return b.w00 * cos[(size_t)b.i00 * ldc + c] + b.w01 * cos[(size_t)b.i01 * ldc + c] +
         b.w10 * cos[(size_t)b.i10 * ldc + c] + b.w11 * cos[(size_t)b.i11 * ldc + c];
}

__global__ __launch_bounds__(256) void upsample_argmax_kernel(const float* __restrict__ cos, int gh, int gw,
                                                              int classes, int ldc, int H, int W,
                                                              int* __restrict__ labels, float* __restrict__ dense) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= H * W) return;
  const int y = idx / W, x = idx - y * W;
  const Bilin b = bilin(y, x, H, W, gh, gw);
  float best = -INFINITY;
  int arg = 0;
  for (int c = 0; c < classes; ++c) {
    const float v = interp(cos, ldc, b, c);
    if (dense) dense[(size_t)c * H * W + idx] = v;
    if (v > best) {
      best = v;
      arg = c;
    }
  }
  labels[idx] = arg;
}

__global__ __launch_bounds__(256) void slide_merge_kernel(const float* __restrict__ cos, int nwin,
                                                          const int* __restrict__ corners, int wg, int classes,
                                                          int ldc, int side, int H, int W, int* __restrict__ labels,
                                                          float* __restrict__ dense) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= H * W) return;
  const int y = idx / W, x = idx - y * W;
  Bilin bl[MAXW];
  const float* base[MAXW];
  float mx[MAXW], inv_z[MAXW];
  int cnt = 0;
  for (int w = 0; w < nwin && cnt < MAXW; ++w) {
    const int y0 = corners[2 * w], x0 = corners[2 * w + 1];
    if (y < y0 || y >= y0 + side || x < x0 || x >= x0 + side) continue;
    bl[cnt] = bilin(y - y0, x - x0, side, side, wg, wg);
    base[cnt] = cos + (size_t)w * wg * wg * ldc;
    ++cnt;
  }
  for (int k = 0; k < cnt; ++k) {
    float m = -INFINITY;
    for (int c = 0; c < classes; ++c) m = fmaxf(m, interp(base[k], ldc, bl[k], c));
    float z = 0.f;
    for (int c = 0; c < classes; ++c) z += expf(interp(base[k], ldc, bl[k], c) - m);
    mx[k] = m;
    inv_z[k] = 1.0f / z;
  }
  const float inv_cnt = 1.0f / (float)cnt;
  float best = -INFINITY;
  int arg = 0;
  for (int c = 0; c < classes; ++c) {
    float acc = 0.f;
    for (int k = 0; k < cnt; ++k) acc += expf(interp(base[k], ldc, bl[k], c) - mx[k]) * inv_z[k];
    acc *= inv_cnt;
    if (dense) dense[(size_t)c * H * W + idx] = acc;
    if (acc > best) {
      best = acc;
      arg = c;
    }
  }
  labels[idx] = arg;
}

__global__ __launch_bounds__(256) void cos_out_kernel(const float* __restrict__ cos, int nimg, int g, int classes,
                                                      int ldc, float* __restrict__ out) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)nimg * classes * g;
  if (idx >= total) return;
  const int r = (int)(idx % g);
  const int c = (int)((idx / g) % classes);
  const int i = (int)(idx / ((size_t)g * classes));
  out[idx] = cos[((size_t)i * g + r) * ldc + c];
}

}  // namespace

hipError_t launch_upsample_argmax(const float* cos, int gh, int gw, int classes, int ldc, int H, int W, int* labels,
                                  float* dense, hipStream_t s) {
  const int n = H * W;
  hipLaunchKernelGGL(upsample_argmax_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cos, gh, gw, classes, ldc, H, W,
                     labels, dense);
  return hipGetLastError();
}

hipError_t launch_slide_merge(const float* cos, int nwin, const int* corners_dev, int wg, int classes, int ldc,
                              int side, int H, int W, int* labels, float* dense, hipStream_t s) {
  const int n = H * W;
  hipLaunchKernelGGL(slide_merge_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cos, nwin, corners_dev, wg, classes,
                     ldc, side, H, W, labels, dense);
  return hipGetLastError();
}

hipError_t launch_cos_out(const float* cos, int nimg, int g, int classes, int ldc, float* out, hipStream_t s) {
  const size_t total = (size_t)nimg * classes * g;
  hipLaunchKernelGGL(cos_out_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, cos, nimg, g, classes,
                     ldc, out);
  return hipGetLastError();
}

}  // namespace vit
