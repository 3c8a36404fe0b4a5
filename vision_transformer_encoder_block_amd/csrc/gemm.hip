// bf16 MFMA GEMM for gfx950: acc[m, n] = sum_k A[m, k] * W[n, k] with fused
// epilogues (bias, GELU, LayerScale + residual, head split, patch rows).
//
// Both operands are K-contiguous (activations [M, K], nn.Linear weights
// [N, K]), so each lane of v_mfma_f32_32x32x16_bf16 reads 16 contiguous bytes
// of one row for either operand.  A 256-thread workgroup (4 waves in 2 x 2)
// computes a BM x BN tile; K advances in steps of 64 through a double-buffered
// LDS tile whose 16-byte chunks are XOR-swizzled by row so that the eight rows
// read together by consecutive lanes hit distinct banks.  Global loads for the
// next K step are in flight while the MFMAs of the current step run.
// Workgroup ids are remapped so that each XCD (8 per chip, its own L2) owns a
// contiguous range of tiles, grouped along M for operand reuse.
#include "common.h"
#include "kernels.h"

namespace vit {
namespace {

constexpr int BK = 64;

// Division by a runtime constant for 0 <= n < 2^31 (multiply-high + shift).
struct FastDiv {
  uint32_t mul, shift;
};

FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1u << s) < d) ++s;
  uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{uint32_t(m), s};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.mul) + n) >> f.shift; }

// Exchange bits 2 and 3 of a token index (layout of vt, see vit_op_qkv).
__device__ __forceinline__ int vt_pos(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int n = tiles_m * tiles_n;
  constexpr int XCD = 8;
  const int per = (n + XCD - 1) / XCD;
  int tall = n % XCD;
  if (tall == 0) tall = XCD;
  const int xcd = bid % XCD, local = bid / XCD;
  int pid = xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
  constexpr int GROUP_M = 8;
  const int in_group = GROUP_M * tiles_n;
  const int group = pid / in_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int r = pid - group * in_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// ---------------------------------------------------------------- epilogues

struct EpiBiasBf16 {
  const float* bias;
  bf16_t* out;
  int ldc;
  struct Col { float b; };
  __device__ Col col(int n) const { return {bias ? bias[n] : 0.f}; }
  __device__ void store(int m, int n, float v, Col c) const { out[(size_t)m * ldc + n] = f2bf(v + c.b); }
};

struct EpiGeluBf16 {
  const float* bias;
  bf16_t* out;
  int ldc;
  struct Col { float b; };
  __device__ Col col(int n) const { return {bias[n]}; }
  __device__ void store(int m, int n, float v, Col c) const { out[(size_t)m * ldc + n] = f2bf(gelu_erf(v + c.b)); }
};

struct EpiResidual {
  const float* bias;
  const float* ls;
  float* out;
  int ldc;
  struct Col { float b, s; };
  __device__ Col col(int n) const { return {bias[n], ls[n]}; }
  __device__ void store(int m, int n, float v, Col c) const {
    float* p = out + (size_t)m * ldc + n;
    *p = *p + c.s * (v + c.b);
  }
};

struct EpiBiasF32 {
  const float* bias;
  float* out;
  int ldc;
  struct Col { float b; };
  __device__ Col col(int n) const { return {bias ? bias[n] : 0.f}; }
  __device__ void store(int m, int n, float v, Col c) const { out[(size_t)m * ldc + n] = v + c.b; }
};

struct EpiQKV {
  const float* bias;
  bf16_t* q;
  bf16_t* k;
  bf16_t* vt;
  int D, N, heads, nv;
  FastDiv divN;
  float qscale;
  struct Col { float b; int which, head, d; };
  __device__ Col col(int n) const {
    const int which = n / D;
    const int c = n - which * D;
    return {bias[n], which, c >> 6, c & 63};
  }
  __device__ void store(int m, int n, float v, Col c) const {
    const int b = (int)fdiv((uint32_t)m, divN);
    const int tok = m - b * N;
    const size_t bh = (size_t)b * heads + c.head;
    const float x = v + c.b;
    if (c.which == 0) {
      q[(bh * N + tok) * 64 + c.d] = f2bf(x * qscale);
    } else if (c.which == 1) {
      k[(bh * N + tok) * 64 + c.d] = f2bf(x);
    } else {
      vt[(bh * 64 + c.d) * nv + vt_pos(tok)] = f2bf(x);
    }
  }
};

struct EpiPatch {
  const float* bias;
  const float* pos;
  float* out;
  int D, tokens, patches, regs;
  FastDiv divP;
  struct Col { float b; };
  __device__ Col col(int n) const { return {bias[n]}; }
  __device__ void store(int m, int n, float v, Col c) const {
    const int b = (int)fdiv((uint32_t)m, divP);
    const int i = m - b * patches;
    const size_t row = (size_t)b * tokens + 1 + regs + i;
    out[row * D + n] = v + c.b + pos[(size_t)(1 + i) * D + n];
  }
};

// ---------------------------------------------------------------- kernel

template <int BM, int BN, class Epi>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                                        int M, int N, int K, int tiles_m, int tiles_n, Epi epi) {
  constexpr int TM = BM / 64, TN = BN / 64;           // 32x32 blocks per wave
  constexpr int A_CH = BM * 8 / 256, B_CH = BN * 8 / 256;  // 16-byte chunks per thread per K step
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");
  __shared__ uint4 As[2][BM * 8];
  __shared__ uint4 Bs[2][BN * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const uint4* a_src[A_CH];
  const uint4* b_src[B_CH];
  bool a_ok[A_CH], b_ok[B_CH];
  int a_dst[A_CH], b_dst[B_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) {
    const int cid = tid + c * 256, r = cid >> 3, qd = cid & 7;
    const int row = m0 + r;
    a_ok[c] = row < M;
    a_src[c] = reinterpret_cast<const uint4*>(A + (size_t)(a_ok[c] ? row : 0) * K) + qd;
    a_dst[c] = r * 8 + (qd ^ (r & 7));
  }
#pragma unroll
  for (int c = 0; c < B_CH; ++c) {
    const int cid = tid + c * 256, r = cid >> 3, qd = cid & 7;
    const int row = n0 + r;
    b_ok[c] = row < N;
    b_src[c] = reinterpret_cast<const uint4*>(W + (size_t)(b_ok[c] ? row : 0) * K) + qd;
    b_dst[c] = r * 8 + (qd ^ (r & 7));
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const uint4 zero = make_uint4(0, 0, 0, 0);
  uint4 ra[A_CH], rb[B_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) ra[c] = a_ok[c] ? a_src[c][0] : zero;
#pragma unroll
  for (int c = 0; c < B_CH; ++c) rb[c] = b_ok[c] ? b_src[c][0] : zero;
#pragma unroll
  for (int c = 0; c < A_CH; ++c) As[0][a_dst[c]] = ra[c];
#pragma unroll
  for (int c = 0; c < B_CH; ++c) Bs[0][b_dst[c]] = rb[c];
  __syncthreads();

  const int KT = K / BK;
  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
      const int off = (kt + 1) * (BK / 8);
#pragma unroll
      for (int c = 0; c < A_CH; ++c) ra[c] = a_ok[c] ? a_src[c][off] : zero;
#pragma unroll
      for (int c = 0; c < B_CH; ++c) rb[c] = b_ok[c] ? b_src[c][off] : zero;
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int qd = ks * 2 + lhalf;
      bf16x8 af[TM], bw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / 2) + i * 32 + lrow;
        af[i] = as_bf16x8(As[cur][r * 8 + (qd ^ (r & 7))]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * (BN / 2) + j * 32 + lrow;
        bw[j] = as_bf16x8(Bs[cur][r * 8 + (qd ^ (r & 7))]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16(af[i], bw[j], acc[i][j]);
    }
    if (kt + 1 < KT) {
#pragma unroll
      for (int c = 0; c < A_CH; ++c) As[cur ^ 1][a_dst[c]] = ra[c];
#pragma unroll
      for (int c = 0; c < B_CH; ++c) Bs[cur ^ 1][b_dst[c]] = rb[c];
    }
    __syncthreads();
  }

  // accumulator element e of block (i, j): row 8*(e/4) + 4*lhalf + e%4, column lrow
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + wn * (BN / 2) + j * 32 + lrow;
    if (n >= N) continue;
    const auto cv = epi.col(n);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * (BM / 2) + i * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
        if (m < M) epi.store(m, n, acc[i][j][e], cv);
      }
    }
  }
}

template <int BM, int BN, class Epi>
hipError_t run(const bf16_t* A, const bf16_t* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, Epi>), dim3(tiles_m * tiles_n), dim3(256), 0, s, A, W, M, N, K,
                     tiles_m, tiles_n, epi);
  return hipGetLastError();
}

template <class Epi>
hipError_t dispatch(const bf16_t* A, const bf16_t* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  // Few tiles: a smaller tile keeps more CUs busy.
  const long big_tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (big_tiles < 256) return run<64, 64>(A, W, M, N, K, epi, s);
  return run<128, 128>(A, W, M, N, K, epi, s);
}

}  // namespace

hipError_t launch_gemm(const uint16_t* A, const uint16_t* W, int M, int N, int K, const EpiParams& ep,
                       hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0 || K % BK != 0) return hipErrorInvalidValue;
  switch (ep.kind) {
    case EPI_BIAS_BF16:
      return dispatch(A, W, M, N, K, EpiBiasBf16{ep.bias, (bf16_t*)ep.out, ep.ldc}, s);
    case EPI_GELU_BF16:
      return dispatch(A, W, M, N, K, EpiGeluBf16{ep.bias, (bf16_t*)ep.out, ep.ldc}, s);
    case EPI_RESIDUAL:
      return dispatch(A, W, M, N, K, EpiResidual{ep.bias, ep.ls, (float*)ep.out, ep.ldc}, s);
    case EPI_BIAS_F32:
      return dispatch(A, W, M, N, K, EpiBiasF32{ep.bias, (float*)ep.out, ep.ldc}, s);
    case EPI_QKV: {
      const int D = N / 3;
      EpiQKV e{ep.bias, ep.q, ep.k, ep.vt, D, ep.tokens, ep.heads, ep.nv, make_fastdiv(ep.tokens),
               kLog2e * 0.125f};
      return dispatch(A, W, M, N, K, e, s);
    }
    case EPI_PATCH: {
      EpiPatch e{ep.bias, ep.pos, (float*)ep.out, ep.ldc, ep.tokens, ep.patches, ep.regs,
                 make_fastdiv(ep.patches)};
      return dispatch(A, W, M, N, K, e, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace vit
