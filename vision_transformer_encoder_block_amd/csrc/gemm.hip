// bf16 MFMA GEMM for gfx950: acc[m, n] = sum_k A[m, k] * W[n, k] with fused
// epilogues (bias, GELU, LayerScale + residual, head split, patch rows).
//
// Both operands are K-contiguous (activations [M, K], nn.Linear weights
// [N, K]), so each lane of v_mfma_f32_32x32x16_bf16 reads 16 contiguous bytes
// of one row for either operand.  A 256-thread workgroup (4 waves in 2 x 2)
// computes a BM x BN tile; K advances in steps of 64 through a double-buffered
// LDS tile.  Tiles are fetched with buffer loads whose range check returns 0
// for rows past M or N, so ragged edges need no branches.  In LDS the 16-byte
// chunk c of row r sits at chunk c ^ ((r >> 1) & 7): the 16 rows read together
// by 16 consecutive lanes of one ds_read_b128 then cover all 64 banks.
// Global loads for the next K step are in flight while the MFMAs of the
// current step run.  The epilogue stages each wave's accumulators through LDS
// so that every lane writes 4 consecutive columns of one row (coalesced
// 8- or 16-byte stores).  Workgroup ids are remapped so that each XCD (8 per
// chip, own L2) owns a contiguous range of tiles, grouped along M.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace vit {
namespace {

constexpr int BK = 64;
#ifndef GEMM_STAGES
#define GEMM_STAGES 3
#endif
#ifndef GEMM_STAGES_SMALL
#define GEMM_STAGES_SMALL 3
#endif

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

// Column of token t in vt: bits 2 and 3 exchanged (see vit_op_qkv).
__device__ __forceinline__ int vt_pos(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

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

__device__ __forceinline__ uint2 pack4_bf16(const float (&v)[4]) {
  return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// ---------------------------------------------------------------- epilogues
// store4(m, n, v, nvalid): columns n .. n + nvalid - 1 (nvalid <= 4) of row m.
// `vec` is true when row starts and n are aligned for a 4-wide vector store.

struct EpiBiasBf16 {
  const float* bias;
  bf16_t* out;
  int ldc;
  bool vec;
  __device__ void store4(int m, int n, float (&v)[4], int nvalid) const {
    bf16_t* p = out + (size_t)m * ldc + n;
    for (int i = 0; i < 4; ++i) v[i] += (bias && i < nvalid) ? bias[n + i] : 0.f;
    if (vec && nvalid == 4) {
      *reinterpret_cast<uint2*>(p) = pack4_bf16(v);
    } else {
      for (int i = 0; i < nvalid; ++i) p[i] = f2bf(v[i]);
    }
  }
};

struct EpiGeluBf16 {
  const float* bias;
  bf16_t* out;
  int ldc;
  bool vec;
  __device__ void store4(int m, int n, float (&v)[4], int nvalid) const {
    bf16_t* p = out + (size_t)m * ldc + n;
    if (vec && nvalid == 4) {
      const float4 b = *reinterpret_cast<const float4*>(bias + n);
      v[0] = gelu_erf(v[0] + b.x);
      v[1] = gelu_erf(v[1] + b.y);
      v[2] = gelu_erf(v[2] + b.z);
      v[3] = gelu_erf(v[3] + b.w);
      *reinterpret_cast<uint2*>(p) = pack4_bf16(v);
    } else {
      for (int i = 0; i < nvalid; ++i) p[i] = f2bf(gelu_erf(v[i] + bias[n + i]));
    }
  }
};

struct EpiResidual {
  const float* bias;
  const float* ls;
  float* out;
  int ldc;
  bool vec;
  __device__ void store4(int m, int n, float (&v)[4], int nvalid) const {
    float* p = out + (size_t)m * ldc + n;
    if (vec && nvalid == 4) {
      const float4 b = *reinterpret_cast<const float4*>(bias + n);
      const float4 s = *reinterpret_cast<const float4*>(ls + n);
      float4 r = *reinterpret_cast<float4*>(p);
      r.x += s.x * (v[0] + b.x);
      r.y += s.y * (v[1] + b.y);
      r.z += s.z * (v[2] + b.z);
      r.w += s.w * (v[3] + b.w);
      *reinterpret_cast<float4*>(p) = r;
    } else {
      for (int i = 0; i < nvalid; ++i) p[i] = p[i] + ls[n + i] * (v[i] + bias[n + i]);
    }
  }
};

struct EpiBiasF32 {
  const float* bias;
  float* out;
  int ldc;
  bool vec;
  __device__ void store4(int m, int n, float (&v)[4], int nvalid) const {
    float* p = out + (size_t)m * ldc + n;
    for (int i = 0; i < 4; ++i) v[i] += (bias && i < nvalid) ? bias[n + i] : 0.f;
    if (vec && nvalid == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      for (int i = 0; i < nvalid; ++i) p[i] = v[i];
    }
  }
};

// Q and K columns (n < 2D) of the fused projection: head-major rows of 64.
struct EpiQK {
  const float* bias;
  bf16_t* q;
  bf16_t* k;
  int D, N, heads;
  FastDiv divN;
  float qscale;
  bool vec;  // always true: D % 64 == 0 and n % 4 == 0
  __device__ void store4(int m, int n, float (&v)[4], int) const {
    const int which = n >= D;
    const int c = n - which * D;
    const int head = c >> 6, d = c & 63;
    const int b = (int)fdiv((uint32_t)m, divN);
    const int tok = m - b * N;
    const size_t row = ((size_t)b * heads + head) * N + tok;
    const float4 bb = *reinterpret_cast<const float4*>(bias + n);
    const float s = which ? 1.f : qscale;
    float o[4] = {(v[0] + bb.x) * s, (v[1] + bb.y) * s, (v[2] + bb.z) * s, (v[3] + bb.w) * s};
    *reinterpret_cast<uint2*>((which ? k : q) + row * 64 + d) = pack4_bf16(o);
  }
};

struct EpiPatch {
  const float* bias;
  const float* pos;
  float* out;
  int D, tokens, patches, regs;
  FastDiv divP;
  bool vec;  // always true: D % 64 == 0
  __device__ void store4(int m, int n, float (&v)[4], int) const {
    const int b = (int)fdiv((uint32_t)m, divP);
    const int i = m - b * patches;
    const size_t row = (size_t)b * tokens + 1 + regs + i;
    const float4 bb = *reinterpret_cast<const float4*>(bias + n);
    const float4 pp = *reinterpret_cast<const float4*>(pos + (size_t)(1 + i) * D + n);
    *reinterpret_cast<float4*>(out + row * D + n) =
        make_float4(v[0] + bb.x + pp.x, v[1] + bb.y + pp.y, v[2] + bb.z + pp.z, v[3] + bb.w + pp.w);
  }
};

// V columns, computed transposed (A = wv rows, W = token rows): element (m, n)
// is channel m of token row n, stored in vt.  Written straight from the
// accumulators: the 32 lanes of a row hold 32 consecutive tokens.
struct EpiVt {
  const float* bias;  // bv
  bf16_t* vt;
  int N, heads, nv;
  FastDiv divN;
  __device__ void store(int m, int n, float v) const {
    const int b = (int)fdiv((uint32_t)n, divN);
    const int tok = n - b * N;
    const int head = m >> 6, d = m & 63;
    vt[(((size_t)b * heads + head) * 64 + d) * nv + vt_pos(tok)] = f2bf(v + bias[m]);
  }
};

// ---------------------------------------------------------------- pipeline helpers

// One LDS object per (size, stage): the compiler then tracks the DMA writes
// of each stage separately and only waits for the stage it reads.
template <int BYTES, int STAGE>
__device__ __forceinline__ uint4* stage_lds() {
  __shared__ uint4 buf[BYTES / 16];
  return buf;
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// ---------------------------------------------------------------- kernel
// S-stage pipeline: K steps of 64 arrive in LDS by direct-to-LDS buffer loads
// (each wave instruction fills 1 KB = 8 rows x 128 B; every lane fetches the
// logical chunk that belongs at its swizzled slot) issued S - 1 steps ahead.

template <int BM, int BN, int S, bool kStaged, class Epi>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                                        int M, int N, int K, int tiles_m, int tiles_n, Epi epi) {
  constexpr int TM = BM / 64, TN = BN / 64;     // 32x32 blocks per wave
  constexpr int WTM = BM / 2, WTN = BN / 2;     // wave tile
  constexpr int A_IT = BM / 32, B_IT = BN / 32; // DMA instructions per wave per stage
  constexpr int L = A_IT + B_IT;
  constexpr int STAGE_BYTES = (BM + BN) * 128;
  static_assert(S >= 2 && (S - 1) * L < 64, "pipeline depth");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int32x4 ra_src = make_rsrc_words(A, (uint32_t)((size_t)M * K * 2));
  const int32x4 rb_src = make_rsrc_words(W, (uint32_t)((size_t)N * K * 2));
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // byte offset (at k = 0) of the chunk this lane fetches in each DMA instruction
  uint32_t a_off[A_IT], b_off[B_IT];
  {
    const int sub = lane >> 3, pc = lane & 7;
#pragma unroll
    for (int j = 0; j < A_IT; ++j) {
      const int row = (j * 4 + wave) * 8 + sub;
      a_off[j] = (uint32_t)(m0 + row) * (uint32_t)K * 2u + (uint32_t)swz(row, pc) * 16u;
    }
#pragma unroll
    for (int j = 0; j < B_IT; ++j) {
      const int row = (j * 4 + wave) * 8 + sub;
      b_off[j] = (uint32_t)(n0 + row) * (uint32_t)K * 2u + (uint32_t)swz(row, pc) * 16u;
    }
  }
  auto issue = [&](auto stage, int kt) {
    const uint32_t blk = lds_addr(stage_lds<STAGE_BYTES, decltype(stage)::value>());
    const uint32_t koff = (uint32_t)kt * (BK * 2);
#pragma unroll
    for (int j = 0; j < A_IT; ++j) dma16(ra_src, a_off[j] + koff, blk + (uint32_t)(j * 4 + wave_u) * 1024u);
#pragma unroll
    for (int j = 0; j < B_IT; ++j)
      dma16(rb_src, b_off[j] + koff, blk + (uint32_t)(BM * 128 + (j * 4 + wave_u) * 1024));
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int KT = K / BK;
  const int lrow = lane & 31, lhalf = lane >> 5;
  // Fragments of step ks + 1 are read from LDS while the MFMAs of step ks run.
  auto compute = [&](auto stage) {
    const uint4* Ac = stage_lds<STAGE_BYTES, decltype(stage)::value>();
    const uint4* Bc = Ac + BM * 8;
    bf16x8 af[2][TM], bw[2][TN];
    auto read = [&](int buf, int ks) {
      const int qd = ks * 2 + lhalf;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WTM + i * 32 + lrow;
        af[buf][i] = as_bf16x8(Ac[r * 8 + swz(r, qd)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WTN + j * 32 + lrow;
        bw[buf][j] = as_bf16x8(Bc[r * 8 + swz(r, qd)]);
      }
    };
    read(0, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) read(cur ^ 1, ks + 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16(af[cur][i], bw[cur][j], acc[i][j]);
    }
  };

  static_for<0, S - 1>([&](auto s) {
    if (decltype(s)::value < KT) issue(s, decltype(s)::value);
  });
  for (int kt0 = 0; kt0 < KT; kt0 += S) {
    static_for<0, S>([&](auto s) {
      constexpr int st = decltype(s)::value;
      const int kt = kt0 + st;
      if (kt < KT) {
        // this wave's loads of stage st are done once at most `later` stages are in flight
        const int later = min(S - 2, KT - 1 - kt);
        static_for<0, S - 1>([&](auto c) {
          if (later == decltype(c)::value) wait_vm<decltype(c)::value * L>();
        });
        barrier_keep_loads();  // every wave's loads of stage st have landed
        if (kt + S - 1 < KT) issue(std::integral_constant<int, (st + S - 1) % S>{}, kt + S - 1);
        compute(s);
      }
    });
  }
  __syncthreads();

  // accumulator element e of block (i, j): row 8*(e/4) + 4*lhalf + e%4, column lrow
  if constexpr (!kStaged) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * WTN + j * 32 + lrow;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm * WTM + i * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
          if (m < M && n < N) epi.store(m, n, acc[i][j][e]);
        }
    }
  } else {
    // Each wave stages one 32-row block of its tile at a time (row stride WTN + 8
    // floats: the two lane halves land on disjoint banks), then every lane
    // handles 4 consecutive columns of one row.  Waves 0-1 use the LDS of
    // stage 0, waves 2-3 that of stage 1.
    constexpr int LD = WTN + 8;
    constexpr int LPR = WTN / 4;        // lanes per staged row
    constexpr int RPP = 64 / LPR;       // rows per pass
    static_assert(2 * 32 * LD * 4 <= STAGE_BYTES, "staging must fit in one stage");
    float* stage = reinterpret_cast<float*>(wave < 2 ? stage_lds<STAGE_BYTES, 0>() : stage_lds<STAGE_BYTES, 1>()) +
                   (wave & 1) * 32 * LD;
    const int cl = (lane % LPR) * 4;
    const int n = n0 + wn * WTN + cl;
    const int nvalid = min(4, N - n);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) stage[((e >> 2) * 8 + lhalf * 4 + (e & 3)) * LD + j * 32 + lrow] = acc[i][j][e];
      __syncthreads();
#pragma unroll
      for (int pass = 0; pass < 32 / RPP; ++pass) {
        const int r = pass * RPP + lane / LPR;
        const int m = m0 + wm * WTM + i * 32 + r;
        if (m < M && nvalid > 0) {
          const float4 t = *reinterpret_cast<const float4*>(stage + r * LD + cl);
          float v[4] = {t.x, t.y, t.z, t.w};
          epi.store4(m, n, v, nvalid);
        }
      }
      __syncthreads();
    }
  }
}

template <int BM, int BN, int S, bool kStaged, class Epi>
hipError_t run(const bf16_t* A, const bf16_t* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, S, kStaged, Epi>), dim3(tiles_m * tiles_n), dim3(256), 0, s, A, W, M,
                     N, K, tiles_m, tiles_n, epi);
  return hipGetLastError();
}

template <bool kStaged, class Epi>
hipError_t dispatch(const bf16_t* A, const bf16_t* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  // Few tiles: a smaller tile keeps more CUs busy.
  const long big_tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (big_tiles < 256) return run<64, 64, GEMM_STAGES_SMALL, kStaged>(A, W, M, N, K, epi, s);
  return run<128, 128, GEMM_STAGES, kStaged>(A, W, M, N, K, epi, s);
}

}  // namespace

hipError_t launch_gemm(const uint16_t* A, const uint16_t* W, int M, int N, int K, const EpiParams& ep,
                       hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0 || K % BK != 0) return hipErrorInvalidValue;
  if ((size_t)(M + 128) * K * 2 >= (1ull << 32) || (size_t)(N + 128) * K * 2 >= (1ull << 32))
    return hipErrorInvalidValue;  // 32-bit buffer offsets
  const bool vec = ep.ldc % 4 == 0;
  switch (ep.kind) {
    case EPI_BIAS_BF16:
      return dispatch<true>(A, W, M, N, K, EpiBiasBf16{ep.bias, (bf16_t*)ep.out, ep.ldc, vec}, s);
    case EPI_GELU_BF16:
      return dispatch<true>(A, W, M, N, K, EpiGeluBf16{ep.bias, (bf16_t*)ep.out, ep.ldc, vec}, s);
    case EPI_RESIDUAL:
      return dispatch<true>(A, W, M, N, K, EpiResidual{ep.bias, ep.ls, (float*)ep.out, ep.ldc, vec}, s);
    case EPI_BIAS_F32:
      return dispatch<true>(A, W, M, N, K, EpiBiasF32{ep.bias, (float*)ep.out, ep.ldc, vec}, s);
    case EPI_QKV: {
      // N = 3D: Q and K columns as one GEMM, V columns as a transposed GEMM.
      const int D = N / 3;
      const FastDiv dn = make_fastdiv(ep.tokens);
      EpiQK eqk{ep.bias, ep.q, ep.k, D, ep.tokens, ep.heads, dn, kLog2e * 0.125f, true};
      hipError_t e = dispatch<true>(A, W, M, 2 * D, K, eqk, s);
      if (e != hipSuccess) return e;
      EpiVt ev{ep.bias + 2 * D, ep.vt, ep.tokens, ep.heads, ep.nv, dn};
      return dispatch<false>(W + (size_t)2 * D * K, A, D, M, K, ev, s);
    }
    case EPI_PATCH: {
      EpiPatch e{ep.bias, ep.pos, (float*)ep.out, ep.ldc, ep.tokens, ep.patches, ep.regs, make_fastdiv(ep.patches),
                 true};
      return dispatch<true>(A, W, M, N, K, e, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace vit
