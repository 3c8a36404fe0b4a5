// Row normalisations for gfx950: LayerNorm (bf16 or fp32 out), LayerNormed
// channel-first taps, LayerNorm + L2 patch features, and the L2-normalised CLS
// descriptor.  A LayerNorm row is spread over 16, 32 or 64 lanes with 16-byte
// accesses (several rows per wave for narrow rows); mean and variance use two
// passes over the row held in registers.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace vit {
namespace {

constexpr int MAXV = 64;  // columns per lane: dim <= 4096

// LayerNorm of one row held by a group of LPR lanes as V4 float4 groups each
// (lane sl of the group holds columns 4 (sl + LPR i) .. + 3).  Every lane of
// the wave must call it (the group sums shuffle).  All LayerNorms of the
// library, including the one fused into the residual GEMM epilogue, go
// through ln_group_normalize, so they agree bit for bit on the same row.
template <int V4, int LPR>
__device__ __forceinline__ void ln_vec(const float* __restrict__ xrow, const float* __restrict__ g,
                                       const float* __restrict__ b, float eps, int dim, int sl, float4 (&v)[V4]) {
  const float4* xr = reinterpret_cast<const float4*>(xrow);
  float4 gg[V4], bb[V4];
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    v[i] = xr[sl + LPR * i];
    gg[i] = reinterpret_cast<const float4*>(g)[sl + LPR * i];
    bb[i] = reinterpret_cast<const float4*>(b)[sl + LPR * i];
  }
  ln_group_normalize<V4, LPR>(v, gg, bb, eps, dim);
}

// Lane group shape for dim = 64 V: the widest group that divides the row into float4s.
template <int V>
struct LnShape {
  static constexpr int LPR = V % 4 == 0 ? 64 : (V % 2 == 0 ? 32 : 16);
  static constexpr int V4 = 16 * V / LPR;
  static constexpr int RPW = 64 / LPR;  // rows per wave
};

// Block LayerNorm: 64 / LPR rows per wave, 16-byte loads, 8-byte bf16 stores.
template <int V4, int LPR, bool F32>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ x, int rows, int dim,
                                                        const float* __restrict__ g, const float* __restrict__ b,
                                                        float eps, void* __restrict__ y) {
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int sl = lane % LPR;
  const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  float4 v[V4];
  // lanes past the last row normalise it again (the group sums need every lane)
  ln_vec<V4, LPR>(x + (size_t)min(row, rows - 1) * dim, g, b, eps, dim, sl, v);
  if (row >= rows) return;
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const size_t at = (size_t)row * (dim / 4) + sl + LPR * i;
    if (F32) {
      reinterpret_cast<float4*>(y)[at] = v[i];
    } else {
      reinterpret_cast<uint2*>(y)[at] = make_uint2(pack_bf16x2(v[i].x, v[i].y), pack_bf16x2(v[i].z, v[i].w));
    }
  }
}

// Taps: rt (<= 32) patch rows per workgroup are normalised into LDS, then
// written channel-first so that consecutive lanes store consecutive patches.
template <int V4, int LPR>
__global__ __launch_bounds__(256) void tap_kernel(const float* __restrict__ x, int tokens, int first_patch,
                                                  int patches, int dim, const float* __restrict__ g,
                                                  const float* __restrict__ b, float eps, float* __restrict__ taps,
                                                  size_t tap_stride, int rt) {
  constexpr int RPW = 64 / LPR;
  extern __shared__ float tile[];  // [rt][dim + 1]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sl = lane % LPR;
  const int bimg = blockIdx.y;
  const int p0 = blockIdx.x * rt;
  const int ld = dim + 1;
  for (int r0 = wave * RPW; r0 < rt; r0 += 4 * RPW) {  // uniform over the wave
    const int r = r0 + lane / LPR;
    const int i = p0 + r;
    float4 v[V4];
    ln_vec<V4, LPR>(x + ((size_t)bimg * tokens + first_patch + min(i, patches - 1)) * dim, g, b, eps, dim, sl, v);
    if (r < rt && i < patches) {
#pragma unroll
      for (int k = 0; k < V4; ++k) {
        float* t = tile + r * ld + 4 * (sl + LPR * k);
        t[0] = v[k].x, t[1] = v[k].y, t[2] = v[k].z, t[3] = v[k].w;
      }
    }
  }
  __syncthreads();
  float* out = taps + (size_t)bimg * tap_stride;
  const int rows = min(rt, patches - p0);
  for (int idx = threadIdx.x; idx < rt * dim; idx += 256) {
    const int d = idx / rt, r = idx - d * rt;
    if (r < rows) out[(size_t)d * patches + p0 + r] = tile[r * ld + d];
  }
}

template <int V4, int LPR>
__global__ __launch_bounds__(256) void ln_l2_kernel(const float* __restrict__ x, int batch, int tokens,
                                                    int first_patch, int patches, int dim,
                                                    const float* __restrict__ g, const float* __restrict__ b,
                                                    float eps, bf16_t* __restrict__ feats) {
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int sl = lane % LPR;
  const int rows = batch * patches;
  const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int rc = min(row, rows - 1);
  const int bimg = rc / patches, i = rc - bimg * patches;
  float4 v[V4];
  ln_vec<V4, LPR>(x + ((size_t)bimg * tokens + first_patch + i) * dim, g, b, eps, dim, sl, v);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < V4; ++k) s += (v[k].x * v[k].x + v[k].y * v[k].y) + (v[k].z * v[k].z + v[k].w * v[k].w);
  const float inv = 1.0f / fmaxf(sqrtf(group_sum<LPR>(s)), 1e-12f);
  if (row >= rows) return;
#pragma unroll
  for (int k = 0; k < V4; ++k)
    reinterpret_cast<uint2*>(feats)[(size_t)row * (dim / 4) + sl + LPR * k] =
        make_uint2(pack_bf16x2(v[k].x * inv, v[k].y * inv), pack_bf16x2(v[k].z * inv, v[k].w * inv));
}

// One wave per image.  F > 0: dim = 64 F, and the wave reads the whole row
// into registers before it reduces (all loads in flight at once); F = 0: any
// dim, a strided loop.  Both sum lane-wise in column order, so they agree bit
// for bit.
template <int F>
__global__ __launch_bounds__(64) void descriptor_kernel(const float* __restrict__ x, size_t row_stride, int dim,
                                                        float* __restrict__ desc) {
  const int lane = threadIdx.x;
  const float* xr = x + (size_t)blockIdx.x * row_stride;
  float* dr = desc + (size_t)blockIdx.x * dim;
  float s = 0.f;
  if constexpr (F > 0) {
    float v[F];
#pragma unroll
    for (int i = 0; i < F; ++i) v[i] = xr[lane + 64 * i];
#pragma unroll
    for (int i = 0; i < F; ++i) s += v[i] * v[i];
    const float inv = 1.0f / fmaxf(sqrtf(wave_sum(s)), 1e-12f);
#pragma unroll
    for (int i = 0; i < F; ++i) dr[lane + 64 * i] = v[i] * inv;
  } else {
    for (int c = lane; c < dim; c += 64) s += xr[c] * xr[c];
    const float inv = 1.0f / fmaxf(sqrtf(wave_sum(s)), 1e-12f);
    for (int c = lane; c < dim; c += 64) dr[c] = xr[c] * inv;
  }
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
    using L = LnShape<V>;
    const dim3 grid((rows + 4 * L::RPW - 1) / (4 * L::RPW));
    if (f32)
      hipLaunchKernelGGL((layernorm_kernel<L::V4, L::LPR, true>), grid, dim3(256), 0, s, x, rows, dim, g, b, eps, y);
    else
      hipLaunchKernelGGL((layernorm_kernel<L::V4, L::LPR, false>), grid, dim3(256), 0, s, x, rows, dim, g, b, eps, y);
    return hipGetLastError();
  }
};

template <int V>
struct TapLaunch {
  static hipError_t go(const float* x, int batch, int tokens, int first_patch, int patches, int dim,
                       const float* g, const float* b, float eps, float* taps, size_t tap_stride, hipStream_t s) {
    using L = LnShape<V>;
    const int rt = (int)std::min<size_t>(32, 65536 / ((size_t)(dim + 1) * sizeof(float)));
    const size_t lds = (size_t)rt * (dim + 1) * sizeof(float);
    const dim3 grid((patches + rt - 1) / rt, batch);
    hipLaunchKernelGGL((tap_kernel<L::V4, L::LPR>), grid, dim3(256), lds, s, x, tokens, first_patch, patches, dim, g,
                       b, eps, taps, tap_stride, rt);
    return hipGetLastError();
  }
};

template <int V>
struct LnL2Launch {
  static hipError_t go(const float* x, int batch, int tokens, int first_patch, int patches, int dim,
                       const float* g, const float* b, float eps, uint16_t* feats, hipStream_t s) {
    using L = LnShape<V>;
    const dim3 grid((batch * patches + 4 * L::RPW - 1) / (4 * L::RPW));
    hipLaunchKernelGGL((ln_l2_kernel<L::V4, L::LPR>), grid, dim3(256), 0, s, x, batch, tokens, first_patch, patches,
                       dim, g, b, eps, feats);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_layernorm(const float* x, int rows, int dim, const float* g, const float* b, float eps, void* y,
                            bool out_f32, hipStream_t s) {
  if (rows <= 0 || dim <= 0 || dim % 64 != 0 || dim > 64 * MAXV) return hipErrorInvalidValue;
  // float4 access of x, g, b and y
  if (((uintptr_t)x | (uintptr_t)g | (uintptr_t)b | (uintptr_t)y) % 16 != 0) return hipErrorInvalidValue;
  return by_width<LnLaunch>(dim, x, rows, dim, g, b, eps, y, out_f32, s);
}

hipError_t launch_tap(const float* x, int batch, int tokens, int first_patch, int patches, int dim, const float* g,
                      const float* b, float eps, float* taps, size_t tap_stride, hipStream_t s) {
  if (dim % 64 != 0 || patches <= 0 || dim > 64 * MAXV) return hipErrorInvalidValue;
  if (((uintptr_t)x | (uintptr_t)g | (uintptr_t)b) % 16 != 0) return hipErrorInvalidValue;
  return by_width<TapLaunch>(dim, x, batch, tokens, first_patch, patches, dim, g, b, eps, taps, tap_stride, s);
}

hipError_t launch_ln_l2(const float* x, int batch, int tokens, int first_patch, int patches, int dim, const float* g,
                        const float* b, float eps, uint16_t* feats, hipStream_t s) {
  if (dim % 64 != 0 || patches <= 0 || dim > 64 * MAXV) return hipErrorInvalidValue;
  if (((uintptr_t)x | (uintptr_t)g | (uintptr_t)b | (uintptr_t)feats) % 16 != 0) return hipErrorInvalidValue;
  return by_width<LnL2Launch>(dim, x, batch, tokens, first_patch, patches, dim, g, b, eps, feats, s);
}

hipError_t launch_descriptor(const float* x, int batch, size_t row_stride, int dim, float* desc, hipStream_t s) {
  if (batch <= 0 || dim <= 0) return hipErrorInvalidValue;
  if (dim == 384)
    hipLaunchKernelGGL(descriptor_kernel<6>, dim3(batch), dim3(64), 0, s, x, row_stride, dim, desc);
  else if (dim == 768)
    hipLaunchKernelGGL(descriptor_kernel<12>, dim3(batch), dim3(64), 0, s, x, row_stride, dim, desc);
  else if (dim == 1024)
    hipLaunchKernelGGL(descriptor_kernel<16>, dim3(batch), dim3(64), 0, s, x, row_stride, dim, desc);
  else
    hipLaunchKernelGGL(descriptor_kernel<0>, dim3(batch), dim3(64), 0, s, x, row_stride, dim, desc);
  return hipGetLastError();
}

}  // namespace vit
