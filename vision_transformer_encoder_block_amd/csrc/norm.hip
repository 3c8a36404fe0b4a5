// Row normalisations for gfx950: LayerNorm (bf16 or fp32 out), LayerNormed
// channel-first taps, LayerNorm + L2 patch features, and the L2-normalised CLS
// descriptor.  One wave64 per row; lane l holds columns l, l + 64, ... so every
// load and store instruction of a wave touches one contiguous 256-byte run.
// Mean and variance use two passes over the row held in registers.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace vit {
namespace {

constexpr int MAXV = 64;  // columns per lane: dim <= 4096

template <int V>
__device__ __forceinline__ void ln_row(const float* __restrict__ xr, const float* __restrict__ g,
                                       const float* __restrict__ b, float eps, int dim, int lane, float (&y)[V]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    y[i] = xr[lane + 64 * i];
    s += y[i];
  }
  const float mean = wave_sum(s) / (float)dim;
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    y[i] -= mean;
    v += y[i] * y[i];
  }
  const float rstd = rsqrtf(wave_sum(v) / (float)dim + eps);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int c = lane + 64 * i;
    y[i] = y[i] * rstd * g[c] + b[c];
  }
}

template <int V, bool F32>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ x, int rows, int dim,
                                                        const float* __restrict__ g, const float* __restrict__ b,
                                                        float eps, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float v[V];
  ln_row<V>(x + (size_t)row * dim, g, b, eps, dim, lane, v);
  if (F32) {
    float* yr = reinterpret_cast<float*>(y) + (size_t)row * dim;
#pragma unroll
    for (int i = 0; i < V; ++i) yr[lane + 64 * i] = v[i];
  } else {
    bf16_t* yr = reinterpret_cast<bf16_t*>(y) + (size_t)row * dim;
#pragma unroll
    for (int i = 0; i < V; ++i) yr[lane + 64 * i] = f2bf(v[i]);
  }
}

// Taps: rt (<= 32) patch rows per workgroup are normalised into LDS, then
// written channel-first so that consecutive lanes store consecutive patches.
template <int V>
__global__ __launch_bounds__(256) void tap_kernel(const float* __restrict__ x, int tokens, int first_patch,
                                                  int patches, int dim, const float* __restrict__ g,
                                                  const float* __restrict__ b, float eps, float* __restrict__ taps,
                                                  size_t tap_stride, int rt) {
  extern __shared__ float tile[];  // [rt][dim + 1]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bimg = blockIdx.y;
  const int p0 = blockIdx.x * rt;
  const int ld = dim + 1;
  for (int r = wave; r < rt; r += 4) {
    const int i = p0 + r;
    if (i >= patches) break;
    float v[V];
    ln_row<V>(x + ((size_t)bimg * tokens + first_patch + i) * dim, g, b, eps, dim, lane, v);
#pragma unroll
    for (int k = 0; k < V; ++k) tile[r * ld + lane + 64 * k] = v[k];
  }
  __syncthreads();
  float* out = taps + (size_t)bimg * tap_stride;
  const int rows = min(rt, patches - p0);
  for (int idx = threadIdx.x; idx < rt * dim; idx += 256) {
    const int d = idx / rt, r = idx - d * rt;
    if (r < rows) out[(size_t)d * patches + p0 + r] = tile[r * ld + d];
  }
}

template <int V>
__global__ __launch_bounds__(256) void ln_l2_kernel(const float* __restrict__ x, int batch, int tokens,
                                                    int first_patch, int patches, int dim,
                                                    const float* __restrict__ g, const float* __restrict__ b,
                                                    float eps, bf16_t* __restrict__ feats) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= batch * patches) return;
  const int bimg = row / patches, i = row - bimg * patches;
  float v[V];
  ln_row<V>(x + ((size_t)bimg * tokens + first_patch + i) * dim, g, b, eps, dim, lane, v);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < V; ++k) s += v[k] * v[k];
  const float inv = 1.0f / fmaxf(sqrtf(wave_sum(s)), 1e-12f);
  bf16_t* fr = feats + (size_t)row * dim;
#pragma unroll
  for (int k = 0; k < V; ++k) fr[lane + 64 * k] = f2bf(v[k] * inv);
}

__global__ __launch_bounds__(64) void descriptor_kernel(const float* __restrict__ x, size_t row_stride, int dim,
                                                        float* __restrict__ desc) {
  const int lane = threadIdx.x;
  const float* xr = x + (size_t)blockIdx.x * row_stride;
  float s = 0.f;
  for (int c = lane; c < dim; c += 64) s += xr[c] * xr[c];
  const float inv = 1.0f / fmaxf(sqrtf(wave_sum(s)), 1e-12f);
  for (int c = lane; c < dim; c += 64) desc[(size_t)blockIdx.x * dim + c] = xr[c] * inv;
}

template <template <int> class Launch, class... Args>
hipError_t by_width(int dim, Args... args) {
  switch (dim / 64) {
    case 1: return Launch<1>::go(args...);
    case 2: return Launch<2>::go(args...);
    case 3: return Launch<3>::go(args...);
    case 4: return Launch<4>::go(args...);
    case 5: return Launch<5>::go(args...);
    case 6: return Launch<6>::go(args...);
    case 7: return Launch<7>::go(args...);
    case 8: return Launch<8>::go(args...);
    case 9: return Launch<9>::go(args...);
    case 10: return Launch<10>::go(args...);
    case 11: return Launch<11>::go(args...);
    case 12: return Launch<12>::go(args...);
    case 13: return Launch<13>::go(args...);
    case 14: return Launch<14>::go(args...);
    case 15: return Launch<15>::go(args...);
    case 16: return Launch<16>::go(args...);
    case 20: return Launch<20>::go(args...);
    case 24: return Launch<24>::go(args...);
    case 32: return Launch<32>::go(args...);
    case 48: return Launch<48>::go(args...);
    case 64: return Launch<64>::go(args...);
  }
  return hipErrorInvalidValue;
}

template <int V>
struct LnLaunch {
  static hipError_t go(const float* x, int rows, int dim, const float* g, const float* b, float eps, void* y,
                       bool f32, hipStream_t s) {
    const dim3 grid((rows + 3) / 4);
    if (f32)
      hipLaunchKernelGGL((layernorm_kernel<V, true>), grid, dim3(256), 0, s, x, rows, dim, g, b, eps, y);
    else
      hipLaunchKernelGGL((layernorm_kernel<V, false>), grid, dim3(256), 0, s, x, rows, dim, g, b, eps, y);
    return hipGetLastError();
  }
};

template <int V>
struct TapLaunch {
  static hipError_t go(const float* x, int batch, int tokens, int first_patch, int patches, int dim,
                       const float* g, const float* b, float eps, float* taps, size_t tap_stride, hipStream_t s) {
    const int rt = (int)std::min<size_t>(32, 65536 / ((size_t)(dim + 1) * sizeof(float)));
    const size_t lds = (size_t)rt * (dim + 1) * sizeof(float);
    const dim3 grid((patches + rt - 1) / rt, batch);
    hipLaunchKernelGGL((tap_kernel<V>), grid, dim3(256), lds, s, x, tokens, first_patch, patches, dim, g, b, eps,
                       taps, tap_stride, rt);
    return hipGetLastError();
  }
};

template <int V>
struct LnL2Launch {
  static hipError_t go(const float* x, int batch, int tokens, int first_patch, int patches, int dim,
                       const float* g, const float* b, float eps, uint16_t* feats, hipStream_t s) {
    const dim3 grid((batch * patches + 3) / 4);
    hipLaunchKernelGGL((ln_l2_kernel<V>), grid, dim3(256), 0, s, x, batch, tokens, first_patch, patches, dim, g, b,
                       eps, feats);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_layernorm(const float* x, int rows, int dim, const float* g, const float* b, float eps, void* y,
                            bool out_f32, hipStream_t s) {
  if (rows <= 0 || dim <= 0 || dim % 64 != 0 || dim > 64 * MAXV) return hipErrorInvalidValue;
  return by_width<LnLaunch>(dim, x, rows, dim, g, b, eps, y, out_f32, s);
}

hipError_t launch_tap(const float* x, int batch, int tokens, int first_patch, int patches, int dim, const float* g,
                      const float* b, float eps, float* taps, size_t tap_stride, hipStream_t s) {
  if (dim % 64 != 0 || patches <= 0) return hipErrorInvalidValue;
  return by_width<TapLaunch>(dim, x, batch, tokens, first_patch, patches, dim, g, b, eps, taps, tap_stride, s);
}

hipError_t launch_ln_l2(const float* x, int batch, int tokens, int first_patch, int patches, int dim, const float* g,
                        const float* b, float eps, uint16_t* feats, hipStream_t s) {
  if (dim % 64 != 0 || patches <= 0) return hipErrorInvalidValue;
  return by_width<LnL2Launch>(dim, x, batch, tokens, first_patch, patches, dim, g, b, eps, feats, s);
}

hipError_t launch_descriptor(const float* x, int batch, size_t row_stride, int dim, float* desc, hipStream_t s) {
  if (batch <= 0 || dim <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(descriptor_kernel, dim3(batch), dim3(64), 0, s, x, row_stride, dim, desc);
  return hipGetLastError();
}

}  // namespace vit
