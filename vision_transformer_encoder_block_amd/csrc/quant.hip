// 8-bit quantisation for the low-precision linear layers: per-tensor absolute
// maximum (to choose a scale) and the E4M3 or int8 codes of x * s_inv.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace vit {
namespace {

// E4M3 code of v: nearest value, ties to the even mantissa, magnitudes past
// 448 (and infinities) saturated, sign kept (also for results that round to
// zero), NaN -> 0x7F.  Done on the fp32 bits, so the result is exact.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  if (!(a == a)) return 0x7Fu;
  a = fminf(a, 448.f);
  if (a < 0.015625f)  // below 2^-6: multiples of 2^-9 (0x08, the smallest normal, is 8 of them)
    return sign | (uint32_t)rintf(a * 512.f);
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // keep 3 mantissa bits, ties to even
  return sign | (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);  // exponent 127 + E -> field E + 7
}

// int8 code of v: the nearest integer with ties to even (v_rndne), clamped to
// [-127, 127] first (infinities included; clamping before rounding gives the
// same code as rounding first), NaN -> 0.
__device__ __forceinline__ uint32_t int8_code(float v) {
  if (!(v == v)) return 0u;
  return (uint32_t)(int)rintf(fminf(fmaxf(v, -127.f), 127.f)) & 0xFFu;
}

__device__ __forceinline__ float load_any(const void* x, bool bf, size_t i) {
  return bf ? bf2f(reinterpret_cast<const bf16_t*>(x)[i]) : reinterpret_cast<const float*>(x)[i];
}

template <bool INT8>
__device__ __forceinline__ uint32_t code8(float v) {
  if constexpr (INT8) return int8_code(v);
  else return e4m3_code(v);
}

// Four consecutive values per thread.
template <bool INT8>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ x, bool bf, size_t n, float s_inv,
                                                       uint8_t* __restrict__ out) {
  const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= code8<INT8>(load_any(x, bf, i + j) * s_inv) << (8 * j);
    *reinterpret_cast<uint32_t*>(out + i) = w;
  } else {
    for (size_t j = i; j < n; ++j) out[j] = (uint8_t)code8<INT8>(load_any(x, bf, j) * s_inv);
  }
}

__global__ void zero_kernel(float* p) { *p = 0.f; }

// max |x| with NaN ignored; one atomic max per workgroup on the (non-negative)
// float bits, whose unsigned order is the float order.
__global__ __launch_bounds__(256) void absmax_kernel(const void* __restrict__ x, bool bf, size_t n,
                                                     float* __restrict__ amax) {
  __shared__ float red[4];
  float m = 0.f;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    m = fmaxf(m, fabsf(load_any(x, bf, i)));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(m));
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const void* x, bool x_bf16, size_t n, float s_inv, uint8_t* out, hipStream_t s) {
  if (!x || !out || n == 0 || reinterpret_cast<uintptr_t>(out) % 4) return hipErrorInvalidValue;
  const size_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, x_bf16, n,
                     s_inv, out);
  return hipGetLastError();
}

hipError_t launch_quantize_int8(const void* x, bool x_bf16, size_t n, float s_inv, int8_t* out, hipStream_t s) {
  if (!x || !out || n == 0 || reinterpret_cast<uintptr_t>(out) % 4) return hipErrorInvalidValue;
  const size_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, x_bf16, n,
                     s_inv, reinterpret_cast<uint8_t*>(out));
  return hipGetLastError();
}

hipError_t launch_absmax(const void* x, bool x_bf16, size_t n, float* amax, hipStream_t s) {
  if (!x || !amax || n == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(1), 0, s, amax);
  const size_t blocks = std::min<size_t>((n + 255) / 256, 2048);
  hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, x_bf16, n, amax);
  return hipGetLastError();
}

}  // namespace vit
