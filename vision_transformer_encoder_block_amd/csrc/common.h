// Shared device helpers for the gfx950 kernels: bf16 conversion, vector
// types, wave64 reductions and the MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vit {

// Compute units of an MI355X (8 XCDs of 32); launch shapes are sized for it.
constexpr int kComputeUnits = 256;

typedef uint16_t bf16_t;  // storage type of a bfloat16 value

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2v v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Buffer resource over `bytes` bytes at `p`: loads at offsets >= bytes return 0,
// which zero-fills out-of-range rows of a tile without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Direct-to-LDS loads.  A raw buffer descriptor (base, no stride, byte range,
// gfx9 data format word); loads at offsets >= `bytes` return zeros.
typedef int int32x4 __attribute__((ext_vector_type(4)));

// The words must be wave-uniform (the descriptor is an SGPR operand of the
// inline assembly below); readfirstlane states that to the compiler.
__device__ __forceinline__ int32x4 make_rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  int32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from `voff` into LDS at lds_base + 16 * lane (lds_base is
// wave-uniform, passed in M0).  Issued from inline assembly so that the
// compiler does not insert its own conservative waits; the caller waits with
// wait_vm<> before the barrier that publishes the data.  The instruction has no
// VGPR result.
__device__ __forceinline__ void dma16(int32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders memory operations for the compiler but does
// not drain outstanding loads (the caller waits for exactly what it needs).
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Sum / max of a value and its copy in the other 32-lane half of the wave.
__device__ __forceinline__ float half_swap_sum(float v) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float half_swap_max(float v) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

// Sum over the LPR lanes of a lane group (LPR a power of two <= 64).
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// LayerNorm (two-pass mean and biased variance, eps inside the square root,
// then the affine g, b) of one row of `dim` values held by a group of LPR
// lanes as V4 float4 groups each, in place; gg, bb are this lane's groups of
// g and b.  Every lane of the wave must call it (the group sums shuffle).
template <int V4, int LPR>
__device__ __forceinline__ void ln_group_normalize(float4 (&v)[V4], const float4 (&gg)[V4], const float4 (&bb)[V4],
                                                   float eps, int dim) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = group_sum<LPR>(s) / (float)dim;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    v[i].x -= mean, v[i].y -= mean, v[i].z -= mean, v[i].w -= mean;
    q += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
  }
  const float rstd = rsqrtf(group_sum<LPR>(q) / (float)dim + eps);
#pragma unroll
  for (int i = 0; i < V4; ++i)
    v[i] = make_float4(v[i].x * rstd * gg[i].x + bb[i].x, v[i].y * rstd * gg[i].y + bb[i].y,
                       v[i].z * rstd * gg[i].z + bb[i].z, v[i].w * rstd * gg[i].w + bb[i].w);
}

// Source index and weight of output position i along an axis (n_in -> n_out):
// the centre (i + 1/2) n_in / n_out - 1/2 is the exact rational
// ((2i + 1) n_in - n_out) / (2 n_out), split into its integer part and an
// exactly computed remainder, so the weight carries only the rounding of one
// division (a float coordinate near 700 would carry an ulp of 6e-5).
// Negative centres clamp to 0; indices past the edge clamp to n_in - 1.
__host__ __device__ __forceinline__ void bilinear_tap(int i, int n_in, int n_out, int& i0, int& i1, float& w) {
  const long long num = (long long)(2 * i + 1) * n_in - n_out;
  const long long den = 2LL * n_out;
  if (num <= 0) {
    i0 = 0;
    w = 0.f;
  } else {
    const long long q = num / den;
    i0 = (int)q;
    w = (float)(num - q * den) / (float)den;
  }
  i0 = i0 < n_in - 1 ? i0 : n_in - 1;
  i1 = i0 + 1 < n_in - 1 ? i0 + 1 : n_in - 1;
}

// Division by a runtime constant for 0 <= n < 2^31 (multiply-high + shift).
struct FastDiv {
  uint32_t mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1u << s) < d) ++s;
  uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{uint32_t(m), s};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.mul) + n) >> f.shift; }

// Reads n 16-byte chunks from p, the chunks split over nw workgroups (this
// is workgroup w), and discards them: the lines then sit in the last-level
// cache when a later kernel streams the region, instead of coming from HBM
// at its first touch.  Extra workgroups of a launch that leaves compute units
// idle run this beside the launch's real work.
__device__ __forceinline__ void prefetch_region(const uint4* p, uint32_t n, uint32_t w, uint32_t nw) {
  uint32_t acc = 0;
  const uint32_t stride = nw * blockDim.x;
#pragma unroll 8
  for (uint32_t i = w * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  asm volatile("" ::"v"(acc));  // keeps the loads
}

}  // namespace vit
