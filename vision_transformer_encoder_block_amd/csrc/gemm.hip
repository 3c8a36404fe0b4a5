// bf16 MFMA GEMM for gfx950: acc[m, n] = sum_k A[m, k] * W[n, k] with fused
// epilogues (bias, GELU, LayerScale + residual, head split, patch rows).
//
// Both operands are K-contiguous (activations [M, K], nn.Linear weights
// [N, K]), so each lane of v_mfma_f32_32x32x16_bf16 reads 16 contiguous bytes
// of one row for either operand.  A workgroup of WGM x WGN waves computes a
// BM x BN tile.  K advances in steps of BK through S LDS stages filled by
// direct-to-LDS buffer loads (no VGPR staging); the buffer range check returns
// zeros for rows past M or N, so ragged edges need no branches.  In LDS the
// 16-byte chunks of a row are XOR-swizzled so that the 16 rows read by 16
// consecutive lanes of one ds_read_b128 hit distinct banks.  The epilogue
// stages each wave's accumulators through LDS so that every lane writes 4
// consecutive columns of one row (coalesced 8- or 16-byte stores).  Workgroup
// ids are remapped so that each XCD (8 per chip, own L2) owns a contiguous
// range of tiles, grouped along M.  Tile shapes were chosen by measurement on
// MI355X: small tiles with several workgroups resident per CU beat large tiles
// on the encoder's shapes (K = 384..4096, M = 4101..16404).
#include "common.h"
#include "kernels.h"

#include <type_traits>

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
  struct Col { float b; };
  __device__ Col col(int n) const { return {bias ? bias[n] : 0.f}; }
  __device__ void store(int m, int n, float v, const Col& c) const { out[(size_t)m * ldc + n] = f2bf(v + c.b); }
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
  struct Col { float b; };
  __device__ Col col(int n) const { return {bias[n]}; }
  __device__ void store(int m, int n, float v, const Col& c) const { out[(size_t)m * ldc + n] = f2bf(gelu_erf(v + c.b)); }
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
  struct Col { float b, s; };
  __device__ Col col(int n) const { return {bias[n], ls[n]}; }
  __device__ void store(int m, int n, float v, const Col& c) const {
    float* p = out + (size_t)m * ldc + n;
    *p = *p + c.s * (v + c.b);
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
  struct Col { float b; };
  __device__ Col col(int n) const { return {bias ? bias[n] : 0.f}; }
  __device__ void store(int m, int n, float v, const Col& c) const { out[(size_t)m * ldc + n] = v + c.b; }
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
  struct Col { float b, s; int which, head, d; };
  __device__ Col col(int n) const {
    const int which = n >= D;
    const int c = n - which * D;
    return {bias[n], which ? 1.f : qscale, which, c >> 6, c & 63};
  }
  __device__ void store(int m, int n, float v, const Col& c) const {
    const int b = (int)fdiv((uint32_t)m, divN);
    const int tok = m - b * N;
    const size_t row = ((size_t)b * heads + c.head) * N + tok;
    (c.which ? k : q)[row * 64 + c.d] = f2bf((v + c.b) * c.s);
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
  struct Col { float b; };
  __device__ Col col(int n) const { return {bias[n]}; }
  __device__ void store(int m, int n, float v, const Col& c) const {
    const int b = (int)fdiv((uint32_t)m, divP);
    const int i = m - b * patches;
    const size_t row = (size_t)b * tokens + 1 + regs + i;
    out[row * D + n] = v + c.b + pos[(size_t)(1 + i) * D + n];
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
  struct Col { int b, col; };  // image and vt column of token row n
  __device__ Col col(int n) const {
    const int b = (int)fdiv((uint32_t)n, divN);
    return {b, vt_pos(n - b * N)};
  }
  __device__ void store(int m, int n, float v, const Col& c) const {
    const int head = m >> 6, d = m & 63;
    vt[(((size_t)c.b * heads + head) * 64 + d) * nv + c.col] = f2bf(v + bias[m]);
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
// S-stage pipeline: K steps of BK arrive in LDS by direct-to-LDS buffer loads
// (each wave instruction fills 1 KB; every lane fetches the logical chunk that
// belongs at its swizzled slot).  All S stages are requested up front; at the
// end of step kt each wave waits for its own loads of step kt + 1, one barrier
// publishes them (and retires step kt's buffer), the buffer is refilled with
// step kt + S, the first fragments of step kt + 1 are read, and only then do
// the last MFMAs of step kt issue, so the LDS latency of the next step hides
// under them.

// Chunk swizzle for rows of BK bf16 (BK / 8 chunks of 16 bytes): the 16 rows
// read by 16 consecutive lanes of one ds_read_b128 hit distinct 4-bank groups.
template <int BKT>
__device__ __forceinline__ int swz_k(int r, int c) {
  if constexpr (BKT == 64) return c ^ ((r >> 1) & 7);
  else return c ^ (r & 15);
}

template <int BM, int BN, int BKT, int WGM, int WGN, int S, bool kStaged, class Epi>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(const bf16_t* __restrict__ A,
                                                                  const bf16_t* __restrict__ W, int M, int N, int K,
                                                                  int tiles_m, int tiles_n, Epi epi) {
  constexpr int NW = WGM * WGN;                     // waves per workgroup
  constexpr int WTM = BM / WGM, WTN = BN / WGN;     // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;       // 32x32 blocks per wave
  constexpr int CPR = BKT / 8;                      // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                     // rows per DMA instruction
  constexpr int A_IT = BM / (RPI * NW), B_IT = BN / (RPI * NW);  // DMA instructions per wave per stage
  constexpr int L = A_IT + B_IT;
  constexpr int KS = BKT / 16;                      // MFMA k-steps per stage
  constexpr int STAGE_BYTES = (BM + BN) * BKT * 2;
  static_assert(BKT == 64 || BKT == 128, "BK");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(A_IT * RPI * NW == BM && B_IT * RPI * NW == BN, "DMA split");
  static_assert(S >= 2 && S * L < 64, "pipeline depth");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int32x4 ra_src = make_rsrc_words(A, (uint32_t)((size_t)M * K * 2));
  const int32x4 rb_src = make_rsrc_words(W, (uint32_t)((size_t)N * K * 2));
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // byte offset (at k = 0) of the chunk this lane fetches in each DMA instruction
  uint32_t a_off[A_IT], b_off[B_IT];
  {
    const int sub = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int j = 0; j < A_IT; ++j) {
      const int row = (j * NW + wave) * RPI + sub;
      a_off[j] = (uint32_t)(m0 + row) * (uint32_t)K * 2u + (uint32_t)swz_k<BKT>(row, pc) * 16u;
    }
#pragma unroll
    for (int j = 0; j < B_IT; ++j) {
      const int row = (j * NW + wave) * RPI + sub;
      b_off[j] = (uint32_t)(n0 + row) * (uint32_t)K * 2u + (uint32_t)swz_k<BKT>(row, pc) * 16u;
    }
  }
  auto issue = [&](auto stage, int kt) {
    const uint32_t blk = lds_addr(stage_lds<STAGE_BYTES, decltype(stage)::value>());
    const uint32_t koff = (uint32_t)kt * (BKT * 2);
#pragma unroll
    for (int j = 0; j < A_IT; ++j) dma16(ra_src, a_off[j] + koff, blk + (uint32_t)(j * NW + wave_u) * 1024u);
#pragma unroll
    for (int j = 0; j < B_IT; ++j)
      dma16(rb_src, b_off[j] + koff, blk + (uint32_t)(BM * BKT * 2 + (j * NW + wave_u) * 1024));
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int KT = K / BKT;
  const int lrow = lane & 31, lhalf = lane >> 5;
  bf16x8 af[2][TM], bw[2][TN];
  auto read = [&](auto stage, int buf, int ks) {
    const uint4* Ac = stage_lds<STAGE_BYTES, decltype(stage)::value>();
    const uint4* Bc = Ac + BM * CPR;
    const int qd = ks * 2 + lhalf;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WTM + i * 32 + lrow;
      af[buf][i] = as_bf16x8(Ac[r * CPR + swz_k<BKT>(r, qd)]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WTN + j * 32 + lrow;
      bw[buf][j] = as_bf16x8(Bc[r * CPR + swz_k<BKT>(r, qd)]);
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16(af[buf][i], bw[buf][j], acc[i][j]);
  };
  // wait until at most `later` stages of this wave's loads are in flight
  // (the ones issued after the stage being waited for)
  auto wait_stages = [&](int later) {
    static_for<0, S>([&](auto c) {
      if (later == decltype(c)::value) wait_vm<decltype(c)::value * L>();
    });
  };

  static_for<0, S>([&](auto s) {
    if (decltype(s)::value < KT) issue(s, decltype(s)::value);
  });
  wait_stages(min(S - 1, KT - 1));  // steps 1 .. S-1 may still be in flight
  barrier_keep_loads();
  read(std::integral_constant<int, 0>{}, 0, 0);

  for (int kt0 = 0; kt0 < KT; kt0 += S) {
    static_for<0, S>([&](auto s) {
      constexpr int st = decltype(s)::value;
      constexpr int nx = (st + 1) % S;
      const int kt = kt0 + st;
      if (kt < KT) {
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
          read(s, (ks + 1) & 1, ks + 1);
          mma(ks & 1);
        }
        if (kt + 1 < KT) {
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave is done reading step kt
          wait_stages(min(S - 2, KT - 2 - kt));  // steps kt + 2 .. kt + S - 1 may be in flight
          barrier_keep_loads();                  // step kt + 1 visible, step kt's buffer free
          if (kt + S < KT) issue(s, kt + S);
          read(std::integral_constant<int, nx>{}, KS & 1, 0);
        }
        mma((KS - 1) & 1);
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
          if (m < M && n < N) epi.store(m, n, acc[i][j][e], epi.col(n));
        }
    }
  } else {
    // Each wave stages one 32-row block of its tile at a time (row stride WTN + 8
    // floats: the two lane halves land on disjoint banks), then every lane
    // handles 4 consecutive columns of one row.  The staging areas live in the
    // (now idle) LDS of the pipeline stages.
    constexpr int LD = WTN + 8;
    constexpr int LPR = WTN / 4;                   // lanes per staged row
    constexpr int RPP = 64 / LPR;                  // rows per pass
    constexpr int PASSES = (32 + RPP - 1) / RPP;
    constexpr int WAVE_BYTES = 32 * LD * 4;
    constexpr int WPB = STAGE_BYTES / WAVE_BYTES;  // waves per stage object
    static_assert(LPR <= 64, "staging pass shape");
    static_assert(WPB >= 1 && WPB * S >= NW, "staging must fit in the stage LDS");
    float* stage = nullptr;
    static_for<0, S>([&](auto s) {
      if (wave / WPB == decltype(s)::value)
        stage = reinterpret_cast<float*>(stage_lds<STAGE_BYTES, decltype(s)::value>()) + (wave % WPB) * 32 * LD;
    });
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
      for (int pass = 0; pass < PASSES; ++pass) {
        const int r = pass * RPP + lane / LPR;
        const int m = m0 + wm * WTM + i * 32 + r;
        if (lane < RPP * LPR && r < 32 && m < M && nvalid > 0) {
          const float4 t = *reinterpret_cast<const float4*>(stage + r * LD + cl);
          float v[4] = {t.x, t.y, t.z, t.w};
          epi.store4(m, n, v, nvalid);
        }
      }
      __syncthreads();
    }
  }
}

// Tile configuration: BM x BN tile, WGM x WGN waves, S pipeline stages.
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int S_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, S = S_;
};

template <class C, bool kStaged, class Epi>
hipError_t run(const bf16_t* A, const bf16_t* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  if (K % C::BK != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<C::BM, C::BN, C::BK, C::WGM, C::WGN, C::S, kStaged, Epi>), dim3(tiles_m * tiles_n),
                     dim3(64 * C::WGM * C::WGN), 0, s, A, W, M, N, K, tiles_m, tiles_n, epi);
  return hipGetLastError();
}

// Tile shapes measured on MI355X over the encoder's GEMMs (M = 4101..16404,
// N = 384..4096, K = 384..4096): 128 x 128 is best or equal on most; 64 x 128
// wins on short-K products with few tiles (more resident workgroups per CU);
// 256 x 256 wins only on very large products.
using CfgMid = Cfg<128, 128, 64, 2, 2, 2>;
using CfgSmall = Cfg<64, 128, 64, 2, 2, 2>;
using CfgBig = Cfg<256, 256, 64, 2, 4, 2>;

template <bool kStaged, class Epi>
hipError_t dispatch(const bf16_t* A, const bf16_t* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  const long mid_tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  if ((long)M * N >= 32L * 1024 * 1024) return run<CfgBig, kStaged>(A, W, M, N, K, epi, s);
  if (K <= 512 && mid_tiles < 512) return run<CfgSmall, kStaged>(A, W, M, N, K, epi, s);
  return run<CfgMid, kStaged>(A, W, M, N, K, epi, s);
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
