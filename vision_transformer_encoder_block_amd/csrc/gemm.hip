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
// consecutive columns of one row (coalesced 8- or 16-byte stores); all of its
// reads (LDS, bias, residual) are issued before its first store, because
// loads and stores share one completion counter and a load waited for after
// a store would wait for the store too.  V columns of the fused Q/K/V
// projection leave through a transposing variant of the staging.  Workgroup
// ids are remapped so that each XCD (8 per chip, own L2) owns a contiguous
// range of tiles, grouped along M.  Tile shapes were chosen by measurement on
// MI355X: small tiles with several workgroups resident per CU beat large tiles
// on most of the encoder's shapes (K = 384..4096, M = 4101..16404); 256 x 256
// tiles win where they fill whole rounds of the CUs.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

namespace vit {
namespace {

constexpr int BK = 64;

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

// Columns n .. n + nvalid - 1 (nvalid <= 4; nothing read for nvalid <= 0).
// `vec` is uniform over the launch: N % 4 == 0 and the pointers are aligned,
// so every group a lane touches is whole and one vector access serves it
// (a uniform branch: no divergent control flow around the loads).
__device__ __forceinline__ float4 load4(const float* p, int nvalid, bool vec) {
  if (vec) return *reinterpret_cast<const float4*>(p);
  float t[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < 4; ++i)
    if (i < nvalid) t[i] = p[i];
  return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void store4_bf16(bf16_t* p, const float (&v)[4], int nvalid, bool vec) {
  if (vec) {
    *reinterpret_cast<uint2*>(p) = pack4_bf16(v);
  } else {
    for (int i = 0; i < nvalid; ++i) p[i] = f2bf(v[i]);
  }
}
__device__ __forceinline__ void store4_f32(float* p, const float (&v)[4], int nvalid, bool vec) {
  if (vec) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    for (int i = 0; i < nvalid; ++i) p[i] = v[i];
  }
}

// ---------------------------------------------------------------- GELU
// GELU(x) = x * Phi(x) with Phi, the standard normal CDF, read from a table at
// the points x_i = -6 + i / 64 (i = 0 .. 768) and linearly interpolated: the
// interpolation error is at most h^2/8 * max|Phi''| = 7.4e-6 (h = 1/64,
// max|Phi''| = phi(1)), and outside [-6, 6] Phi is 0 or 1 to within 1e-9.
// Entry i holds (Phi(x_i), Phi(x_{i+1}) - Phi(x_i)); the table is built on
// the host from erfc in double precision and copied once per device.  It is
// stored padded with zero entries to whole 1 KB blocks, the unit in which the
// GEMM copies it into LDS.
constexpr int kPhiPoints = 769;
constexpr int kPhiBlocks = (kPhiPoints * 8 + 1023) / 1024;  // 7
constexpr int kPhiPadded = kPhiBlocks * 128;                 // 896 entries
__device__ float2 g_phi_table[kPhiPadded];

__device__ __forceinline__ float gelu_table(float x, const float2* tab) {
  // t in [0, 768]; NaN converts to index 0 and propagates through f
  const float t = __builtin_amdgcn_fmed3f(fmaf(x, 64.f, 384.f), 0.f, 768.f);
  const float2 e = tab[(int)t];
  return x * fmaf(__builtin_amdgcn_fractf(t), e.y, e.x);
}

// ---------------------------------------------------------------- epilogues
// Staged epilogues: every lane owns 4 consecutive columns n .. n + 3 (nvalid
// of them inside the matrix) of several rows m of the tile.
//   col4(n, nvalid)   column constants (bias, LayerScale), read once per tile
//   pre(m, n, nvalid) row data read before any store of the pass group
//   finish4(v, col, row) the output values (all passes before any store)
//   write4(m, n, v, nvalid[, col]) the stores
// Output and parameter pointers may alias as far as the compiler knows, so
// reads placed after a store would wait for it; this split keeps all reads
// ahead of all stores.  `vec` (host-checked alignment) selects vector accesses.
struct NoRow {};

// Orders one wave's LDS staging writes and reads between the 32-row blocks
// of a row or transposed epilogue.  Each wave stages into its own area, and
// one wave's LDS instructions execute in order, so no workgroup barrier is
// needed; the wavefront-scope fences keep the compiler from moving the LDS
// accesses across it.  A workgroup barrier's release fence would also wait
// for the wave's outstanding global stores of the previous block (ViT-L/16 b1
// Q/K/V and fc1 -1.1 us each, b4 -4.9 and -5.3 us, outputs bit-identical).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct EpiBiasBf16 {
  const float* bias;
  bf16_t* out;
  int ldc;
  bool vec;
  using Col = float4;
  using Row = NoRow;
  __device__ Col col4(int n, int nvalid) const { return bias ? load4(bias + n, nvalid, vec) : make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ Row pre(int, int, int) const { return {}; }
  __device__ void finish4(float (&v)[4], const Col& b, const Row&) const {
    v[0] += b.x, v[1] += b.y, v[2] += b.z, v[3] += b.w;
  }
  __device__ void write4(int m, int n, const float (&v)[4], int nvalid) const {
    store4_bf16(out + (size_t)m * ldc + n, v, nvalid, vec);
  }
};

struct EpiGeluBf16 {
  const float* bias;
  bf16_t* out;
  int ldc;
  bool vec;
  const float2* phi;  // device copy of the Phi table
  using Col = float4;
  using Row = NoRow;
  __device__ static float2* lds_phi() {
    __shared__ float2 t[kPhiPadded];
    return t;
  }
  // Starts the copy of the table into LDS at kernel start with direct-to-LDS
  // loads (one 1 KB block per wave instruction).  Called before the operand
  // loads of the first stages: loads complete in issue order, so the wait for
  // stage 0 covers the table too and the barrier that publishes stage 0
  // publishes it, with no load latency of its own before the pipeline starts.
  __device__ void prologue(int wave, int lane, int nwaves) const {
    const int32x4 r = make_rsrc_words(phi, (uint32_t)(kPhiPadded * 8));
    const uint32_t base = lds_addr(lds_phi());
    for (int j = wave; j < kPhiBlocks; j += nwaves)
      dma16(r, (uint32_t)(j * 1024 + lane * 16), base + (uint32_t)(j * 1024));
  }
  __device__ Col col4(int n, int nvalid) const { return load4(bias + n, nvalid, vec); }
  __device__ Row pre(int, int, int) const { return {}; }
  __device__ void finish4(float (&v)[4], const Col& b, const Row&) const {
    const float2* t = lds_phi();
    v[0] = gelu_table(v[0] + b.x, t);
    v[1] = gelu_table(v[1] + b.y, t);
    v[2] = gelu_table(v[2] + b.z, t);
    v[3] = gelu_table(v[3] + b.w, t);
  }
  __device__ void write4(int m, int n, const float (&v)[4], int nvalid) const {
    store4_bf16(out + (size_t)m * ldc + n, v, nvalid, vec);
  }
};

struct EpiResidual {
  const float* bias;
  const float* ls;
  float* out;
  int ldc;
  bool vec;
  struct Col { float4 b, s; };
  using Row = float4;  // current residual
  __device__ Col col4(int n, int nvalid) const { return {load4(bias + n, nvalid, vec), load4(ls + n, nvalid, vec)}; }
  __device__ Row pre(int m, int n, int nvalid) const { return load4(out + (size_t)m * ldc + n, nvalid, vec); }
  __device__ void finish4(float (&v)[4], const Col& c, const Row& r) const {
    v[0] = r.x + c.s.x * (v[0] + c.b.x);
    v[1] = r.y + c.s.y * (v[1] + c.b.y);
    v[2] = r.z + c.s.z * (v[2] + c.b.z);
    v[3] = r.w + c.s.w * (v[3] + c.b.w);
  }
  __device__ void write4(int m, int n, const float (&v)[4], int nvalid) const {
    store4_f32(out + (size_t)m * ldc + n, v, nvalid, vec);
  }
};

struct EpiBiasF32 {
  const float* bias;
  float* out;
  int ldc;
  bool vec;
  using Col = float4;
  using Row = NoRow;
  __device__ Col col4(int n, int nvalid) const { return bias ? load4(bias + n, nvalid, vec) : make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ Row pre(int, int, int) const { return {}; }
  __device__ void finish4(float (&v)[4], const Col& b, const Row&) const {
    v[0] += b.x, v[1] += b.y, v[2] += b.z, v[3] += b.w;
  }
  __device__ void write4(int m, int n, const float (&v)[4], int nvalid) const {
    store4_f32(out + (size_t)m * ldc + n, v, nvalid, vec);
  }
};

// fp32 output in groups of 8 columns (the GroupNorm groups of the head):
// column n of row m at out[(n / 8) * gstride + 8 m + n % 8], so one group's
// values over all rows form one contiguous run.  N is a multiple of 8 and
// out, bias are 16-byte aligned, so every lane's 4 columns are one store.
struct EpiBiasF32G8 {
  const float* bias;
  float* out;
  size_t gstride;
  using Col = float4;
  using Row = NoRow;
  __device__ Col col4(int n, int nvalid) const { return bias ? load4(bias + n, nvalid, true) : make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ Row pre(int, int, int) const { return {}; }
  __device__ void finish4(float (&v)[4], const Col& b, const Row&) const {
    v[0] += b.x, v[1] += b.y, v[2] += b.z, v[3] += b.w;
  }
  __device__ void write4(int m, int n, const float (&v)[4], int) const {
    *reinterpret_cast<float4*>(out + (size_t)(n >> 3) * gstride + (size_t)m * 8 + (n & 7)) =
        make_float4(v[0], v[1], v[2], v[3]);
  }
};

// 8-bit products: acc is the fp32 sum of products of E4M3 values, or the
// exact int32 sum of int8 products converted to fp32; `scale` (the product of
// the two operands' dequantisation scales) restores the units:
// out = acc * scale + bias (one fused multiply-add), in fp32 or bf16.
template <bool F32>
struct EpiScale {
  float scale;
  const float* bias;
  void* out;
  int ldc;
  bool vec;
  using Col = float4;
  using Row = NoRow;
  __device__ Col col4(int n, int nvalid) const { return bias ? load4(bias + n, nvalid, vec) : make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ Row pre(int, int, int) const { return {}; }
  __device__ void finish4(float (&v)[4], const Col& b, const Row&) const {
    v[0] = fmaf(v[0], scale, b.x), v[1] = fmaf(v[1], scale, b.y);
    v[2] = fmaf(v[2], scale, b.z), v[3] = fmaf(v[3], scale, b.w);
  }
  __device__ void write4(int m, int n, const float (&v)[4], int nvalid) const {
    if constexpr (F32) store4_f32((float*)out + (size_t)m * ldc + n, v, nvalid, vec);
    else store4_bf16((bf16_t*)out + (size_t)m * ldc + n, v, nvalid, vec);
  }
};

// Q and K columns (n < 2D) of the fused projection: head-major rows of 64.
// D % 64 == 0, so the 4 columns of a lane never straddle a head.
struct EpiQK {
  const float* bias;
  bf16_t* q;
  bf16_t* k;
  int D, N, heads;
  FastDiv divN;
  float qscale;
  bool vec;
  struct Col { float4 b; float s; bf16_t* dst; int d; };
  using Row = NoRow;
  __device__ Col col4(int n, int nvalid) const {
    const int which = n >= D;
    const int c = n - which * D;
    return {load4(bias + n, nvalid, vec), which ? 1.f : qscale, (which ? k : q) + (size_t)(c >> 6) * N * 64, c & 63};
  }
  __device__ Row pre(int, int, int) const { return {}; }
  __device__ void finish4(float (&v)[4], const Col& c, const Row&) const {
    v[0] = (v[0] + c.b.x) * c.s;
    v[1] = (v[1] + c.b.y) * c.s;
    v[2] = (v[2] + c.b.z) * c.s;
    v[3] = (v[3] + c.b.w) * c.s;
  }
  __device__ void write4(int m, int, const float (&v)[4], int nvalid, const Col& c) const {
    const int b = (int)fdiv((uint32_t)m, divN);
    const int tok = m - b * N;
    store4_bf16(c.dst + ((size_t)b * heads * N + tok) * 64 + c.d, v, nvalid, vec);
  }
};

// All three projections in one GEMM (N = 3D).  Tiles of Q and K columns go
// through the staged row path of EpiQK; tiles of V columns (n >= 2D: tile
// uniform because 2D is a multiple of the tile width) are transposed through
// LDS: each lane takes one token and half-waves take channel pairs, so 32
// lanes write 32 consecutive vt columns of one channel row.
struct EpiQKV : EpiQK {
  bf16_t* vt;
  int nv;
  __device__ bool tile_transposed(int n0) const { return n0 >= 2 * D; }
  __device__ float tbias(int n) const { return bias[min(n, 3 * D - 1)]; }
  // value v of V channel ch (0 <= ch < D) of token row m
  struct TRow { bf16_t* base; bool ok; };
  __device__ TRow trow(int m, int M) const {
    const int b = (int)fdiv((uint32_t)m, divN);
    const int tok = m - b * N;
    return {vt + (size_t)b * heads * 64 * nv + vt_pos(tok), m < M};
  }
  __device__ void tstore(const TRow& r, int ch, float v) const {
    if (r.ok && ch < D) r.base[(size_t)ch * nv] = f2bf(v);
  }
};

// write4 with or without the column constants
template <class E>
__device__ __forceinline__ auto write4_any(const E& e, int m, int n, const float (&v)[4], int nvalid,
                                           const typename E::Col& c, int) -> decltype(e.write4(m, n, v, nvalid, c)) {
  return e.write4(m, n, v, nvalid, c);
}
template <class E>
__device__ __forceinline__ void write4_any(const E& e, int m, int n, const float (&v)[4], int nvalid,
                                           const typename E::Col&, long) {
  e.write4(m, n, v, nvalid);
}

template <class E, class = void>
struct HasPrologue : std::false_type {};
template <class E>
struct HasPrologue<E, std::void_t<decltype(&E::prologue)>> : std::true_type {};
template <class E, class = void>
struct HasRowLN : std::false_type {};
template <class E>
struct HasRowLN<E, std::void_t<decltype(E::kD)>> : std::true_type {};
template <class E, class = void>
struct HasPrefetch : std::false_type {};
template <class E>
struct HasPrefetch<E, std::void_t<decltype(E::pf_chunks)>> : std::true_type {};
template <class E, class = void>
struct HasChanLN : std::false_type {};
template <class E>
struct HasChanLN<E, std::void_t<decltype(E::kC)>> : std::true_type {};
template <class E, class = void>
struct HasTransposed : std::false_type {};
template <class E>
struct HasTransposed<E, std::void_t<decltype(&E::tile_transposed)>> : std::true_type {};

// Residual update followed by the next LayerNorm, for a tile that spans whole
// rows (N = kD): out[m, :] += ls * (acc + bias), then h[m, :] = LN(out[m, :])
// in bf16.  The arithmetic of both steps is that of EpiResidual and of the
// standalone LayerNorm kernel, so x and h are bit-identical to the unfused pair.
struct EpiResidualLN {
  static constexpr int kD = 384;
  const float* bias;
  const float* ls;
  float* out;  // residual x [M, kD] fp32
  const float* g;
  const float* b;
  float eps;
  bf16_t* h;   // [M, kD] bf16
  // workgroups past the tile grid read this region (16-byte chunks) into the
  // caches: the next GEMMs' weights, on the CUs the row tiles leave idle
  const uint4* pf = nullptr;
  uint32_t pf_chunks = 0;
};

// Channel LayerNorm of whole rows (N = kC channels of a pixel), the semantic
// head's ConvX block: y = LN(acc + bias) (biased variance, eps inside the
// square root, affine), then SiLU y / (1 + e^-y) if `silu`, then a second
// LayerNorm if g2 is non-null; bf16 into out[m * ld + c0 + n].
template <int C>
struct EpiChanLN {
  static constexpr int kC = C;
  const float* bias;  // may be null
  const float* g;
  const float* b;
  float eps;
  bool silu;
  const float* g2;    // may be null
  const float* b2;
  bf16_t* out;
  int ld, c0;
};

// Patch rows of the embedding GEMM: row m = b * patches + i goes to residual
// row b * tokens + 1 + regs + i with its position embedding pos[1 + i] added.
struct EpiPatch {
  const float* bias;
  const float* pos;
  float* out;
  int D, tokens, patches, regs;
  FastDiv divP;
  bool vec;
  using Col = float4;
  using Row = float4;  // position embedding of the patch
  __device__ Col col4(int n, int nvalid) const { return load4(bias + n, nvalid, vec); }
  __device__ Row pre(int m, int n, int nvalid) const {
    const int b = (int)fdiv((uint32_t)m, divP);
    return load4(pos + (size_t)(1 + m - b * patches) * D + n, nvalid, vec);
  }
  __device__ void finish4(float (&v)[4], const Col& bb, const Row& pp) const {
    v[0] += bb.x + pp.x;
    v[1] += bb.y + pp.y;
    v[2] += bb.z + pp.z;
    v[3] += bb.w + pp.w;
  }
  __device__ void write4(int m, int n, const float (&v)[4], int nvalid) const {
    const int b = (int)fdiv((uint32_t)m, divP);
    const size_t row = (size_t)b * tokens + 1 + regs + (m - b * patches);
    store4_f32(out + row * D + n, v, nvalid, vec);
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

// Chunk swizzle for rows of CPR chunks of 16 bytes: the 16 rows read by 16
// consecutive lanes of one ds_read_b128 hit distinct 4-bank groups.
template <int CPR>
__device__ __forceinline__ int swz_c(int r, int c) {
  if constexpr (CPR == 4) return c ^ ((r >> 2) & 3);
  else if constexpr (CPR == 8) return c ^ ((r >> 1) & 7);
  else return c ^ (r & 15);
}

// Matrix-core operand formats.
//   bf16: v_mfma_f32_32x32x16_bf16; a lane's fragment is one 16-byte chunk
//         (8 values) of its row.
//   fp8 (OCP E4M3): v_mfma_f32_32x32x64_f8f6f4 without block scales; a lane's
//         fragment is two chunks (32 values).  Lanes l and l + 32 hold the two
//         halves of the 64 k values of row l % 32, in the same arrangement for
//         A and B, which is all the dot products need.
//   int8: v_mfma_i32_32x32x32_i8; a lane's fragment is one chunk (16 values),
//         the byte layout of the bf16 case.  The int32 accumulators travel in
//         the fp32 accumulator registers bit for bit (kIntAcc) and become fp32
//         values after the main loop; integer sums are exact, so any split of
//         the k values over the lanes gives the same result.
typedef int int32x8 __attribute__((ext_vector_type(8)));
typedef int int32x16 __attribute__((ext_vector_type(16)));
struct MmaBf16 {
  static constexpr int ES = 2, KPM = 16, CPF = 1;  // bytes per value, k per MFMA, chunks per fragment
  static constexpr bool kIntAcc = false;
  using Frag = bf16x8;
  __device__ static Frag frag(const uint4& c0, const uint4&) { return as_bf16x8(c0); }
  __device__ static f32x16 mma(Frag a, Frag b, f32x16 c) { return mfma32x32x16(a, b, c); }
};
struct MmaFp8 {
  static constexpr int ES = 1, KPM = 64, CPF = 2;
  static constexpr bool kIntAcc = false;
  using Frag = int32x8;
  __device__ static Frag frag(const uint4& c0, const uint4& c1) {
    Frag f;
    f[0] = (int)c0.x, f[1] = (int)c0.y, f[2] = (int)c0.z, f[3] = (int)c0.w;
    f[4] = (int)c1.x, f[5] = (int)c1.y, f[6] = (int)c1.z, f[7] = (int)c1.w;
    return f;
  }
  __device__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};
struct MmaI8 {
  static constexpr int ES = 1, KPM = 32, CPF = 1;
  static constexpr bool kIntAcc = true;
  using Frag = int32x4;
  __device__ static Frag frag(const uint4& c0, const uint4&) {
    Frag f;
    f[0] = (int)c0.x, f[1] = (int)c0.y, f[2] = (int)c0.z, f[3] = (int)c0.w;
    return f;
  }
  __device__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, __builtin_bit_cast(int32x16, c), 0, 0, 0));
  }
};

// Addressing of the A operand.  Linear: row m of A holds its K values
// contiguously (A is [M, K]).
struct AMapLinear {
  static constexpr bool kConv = false;
};
// 3x3 / stride 1 / zero padding 1 convolution read in place (implicit GEMM):
// column k = (ky * 3 + kx) * C + c of row m, the pixel (y, x) of image b on a
// gh x gw grid, is in[(b * gh * gw + (y + ky - 1) * gw + x + kx - 1) * ld + c0 + c],
// and zero where that pixel lies outside the grid.  C is a multiple of the K
// step, so every step reads one tap; outside pixels get an offset past the
// end of the buffer, which the range check of the direct-to-LDS load turns
// into zeros.
struct AMapConv3 {
  static constexpr bool kConv = true;
  int gh, gw, ld, c0, C;
  uint32_t bytes;  // size of `in` in bytes
};

// XR = 32: the workgroups of row tile xt_tm also compute the 1..32 rows at the
// end of A that follow the last full row tile (M mod BM <= 32), with the W tile
// they already hold; each wave of the first two wave rows (wm = 0, 1) takes a
// 32 x 32 block of those rows, at the columns of its wm-th 32-column block
// (a 64-column wave tile has two).  This saves a row of tiles that would
// each stream a whole W tile for a few rows.  Row tile 0 takes them: it is
// dispatched first, so its longer workgroups do not form the kernel's tail.
template <int BM, int BN, int BKT, int WGM, int WGN, int S, class Epi, class AM = AMapLinear, class MT = MmaBf16,
          int XR = 0>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(const bf16_t* __restrict__ A,
                                                                  const bf16_t* __restrict__ W, int M, int N, int K,
                                                                  int tiles_m, int tiles_n, Epi epi, AM am = {},
                                                                  int xt_tm = -1) {
  constexpr int NW = WGM * WGN;                     // waves per workgroup
  constexpr int WTM = BM / WGM, WTN = BN / WGN;     // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;       // 32x32 blocks per wave
  constexpr int ES = MT::ES;                        // bytes per operand value
  constexpr int CPR = BKT * ES / 16;                // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                     // rows per DMA instruction (1 KB)
  // The DMA instructions of one stage (A rows, then W rows, RPI rows each)
  // go round-robin to the waves: instruction k is wave k % NW's (k / NW)-th.
  constexpr int A_INS = BM / RPI, TOT = (BM + BN) / RPI;
  constexpr int LHI = (TOT + NW - 1) / NW;          // per wave and stage, at most
  constexpr int L = TOT / NW;                       // ... at least (the waits count these)
  constexpr bool A_SPLIT = A_INS % NW == 0;         // instruction i of every wave reads the same operand
  constexpr int KS = BKT / MT::KPM;                 // MFMA k-steps per stage
  constexpr int STAGE_BYTES = (BM + BN + XR) * BKT * ES;  // A rows, W rows, then the extra A rows
  static_assert(XR == 0 || (XR == 32 && !HasRowLN<Epi>::value && !HasChanLN<Epi>::value && !HasTransposed<Epi>::value && !AM::kConv &&
                            (WGM == 2 || WGM == 4) && WTN == 64 && XR / (64 / (BKT * MT::ES / 16)) <= WGM * WGN),
                "extra rows: plain row epilogues, one 32-column block per wave of the first two wave rows");
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "BK");
  static_assert(!AM::kConv || ES == 2, "implicit convolution reads bf16 activations");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(A_INS * RPI == BM && TOT * RPI == BM + BN && L >= 1, "DMA split");
  static_assert(S >= 2 && S * LHI < 64, "pipeline depth");

  if constexpr (HasPrefetch<Epi>::value) {
    const int tiles = tiles_m * tiles_n;
    if ((int)blockIdx.x >= tiles) {  // workgroup-uniform
      prefetch_region(epi.pf, epi.pf_chunks, blockIdx.x - tiles, gridDim.x - tiles);
      return;
    }
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const bool xt = XR > 0 && tm == xt_tm;  // workgroup-uniform
  const int xr0 = tiles_m * BM;             // first of the extra rows

  static_assert(!AM::kConv || A_SPLIT, "implicit convolution needs whole A instructions per wave");
  uint32_t a_bytes = (uint32_t)((size_t)M * K * ES);
  if constexpr (AM::kConv) a_bytes = am.bytes;
  const int32x4 ra_src = make_rsrc_words(A, a_bytes);
  const int32x4 rb_src = make_rsrc_words(W, (uint32_t)((size_t)N * K * ES));
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  if constexpr (HasPrologue<Epi>::value) epi.prologue(wave_u, lane, NW);
  // byte offset (at k = 0) of the chunk this lane fetches in each of its DMA
  // instructions; instruction k fills LDS bytes [1024 k, 1024 (k + 1)) of the
  // stage (A's BM rows first, so W's rows start at BM * BKT * ES = 1024 A_INS)
  uint32_t g_off[LHI];
  // implicit convolution: the A row's image offset (b * gh * gw) and pixel
  // (y, x); rows past M get a y that no tap brings inside the grid
  constexpr int A_PER_WAVE = AM::kConv ? A_INS / NW : 0;
  int cpb[A_PER_WAVE > 0 ? A_PER_WAVE : 1], cy[A_PER_WAVE > 0 ? A_PER_WAVE : 1], cx[A_PER_WAVE > 0 ? A_PER_WAVE : 1];
  {
    const int sub = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int i = 0; i < LHI; ++i) {
      const int k = min(i * NW + wave, TOT - 1);
      const bool is_a = A_SPLIT ? i < A_INS / NW : k < A_INS;
      const int row = (is_a ? k : k - A_INS) * RPI + sub;
      g_off[i] = (uint32_t)((is_a ? m0 : n0) + row) * (uint32_t)K * (uint32_t)ES + (uint32_t)swz_c<CPR>(row, pc) * 16u;
      if constexpr (AM::kConv) {
        if (i < A_PER_WAVE) {
          const int m = m0 + row;
          const int P = am.gh * am.gw;
          const int b = m / P, pix = m - b * P;
          cpb[i] = b * P;
          cy[i] = m < M ? pix / am.gw : -4;
          cx[i] = pix - (pix / am.gw) * am.gw;
          g_off[i] = (uint32_t)swz_c<CPR>(row, pc) * 16u;  // chunk within the step
        }
      }
    }
  }
  // extra rows: instruction x (of XR / RPI) is wave x's; LDS block TOT + x
  uint32_t gx_off = 0;
  if constexpr (XR > 0) {
    const int row = wave * RPI + lane / CPR;
    gx_off = (uint32_t)(xr0 + row) * (uint32_t)K * (uint32_t)ES + (uint32_t)swz_c<CPR>(row, lane % CPR) * 16u;
  }
  auto issue = [&](auto stage, int kt) {
    const uint32_t blk = lds_addr(stage_lds<STAGE_BYTES, decltype(stage)::value>());
    const uint32_t koff = (uint32_t)kt * (BKT * ES);
    int ky = 0, kx = 0, cbase = 0;
    if constexpr (AM::kConv) {
      const int kel = kt * BKT;
      const int tap = kel / am.C;
      ky = tap / 3 - 1;
      kx = tap - 3 * (tap / 3) - 1;
      cbase = am.c0 + kel - tap * am.C;
    }
#pragma unroll
    for (int i = 0; i < LHI; ++i) {
      const int k = i * NW + wave_u;
      if (LHI == L || k < TOT) {  // wave-uniform
        const bool is_a = A_SPLIT ? i < A_INS / NW : k < A_INS;
        if constexpr (AM::kConv) {
          if (i < A_PER_WAVE) {
            const int y = cy[i] + ky, x = cx[i] + kx;
            const bool in = (unsigned)y < (unsigned)am.gh && (unsigned)x < (unsigned)am.gw;
            const uint32_t off =
                in ? (uint32_t)((cpb[i] + y * am.gw + x) * am.ld + cbase) * 2u + g_off[i] : 0x80000000u;
            dma16(ra_src, off, blk + (uint32_t)k * 1024u);
            continue;
          }
        }
        dma16(is_a ? ra_src : rb_src, g_off[i] + koff, blk + (uint32_t)k * 1024u);
      }
    }
    if constexpr (XR > 0) {
      // rows past M come back as zeros through the range check
      if (xt && wave_u < XR / RPI) dma16(ra_src, gx_off + koff, blk + (uint32_t)(TOT + wave_u) * 1024u);
    }
  };

  f32x16 acc[TM][TN], acc_x;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc_x[e] = 0.f;

  const int KT = K / BKT;
  const int lrow = lane & 31, lhalf = lane >> 5;
  typename MT::Frag af[2][TM], bw[2][TN], ax[2];
  auto read = [&](auto stage, int buf, int ks) {
    const uint4* Ac = stage_lds<STAGE_BYTES, decltype(stage)::value>();
    const uint4* Bc = Ac + BM * CPR;
    const int qd = (ks * 2 + lhalf) * MT::CPF;   // first chunk of this lane's fragment
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WTM + i * 32 + lrow;
      af[buf][i] = MT::frag(Ac[r * CPR + swz_c<CPR>(r, qd)], Ac[r * CPR + swz_c<CPR>(r, qd + MT::CPF - 1)]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WTN + j * 32 + lrow;
      bw[buf][j] = MT::frag(Bc[r * CPR + swz_c<CPR>(r, qd)], Bc[r * CPR + swz_c<CPR>(r, qd + MT::CPF - 1)]);
    }
    if constexpr (XR > 0) {
      if (xt && wm < 2) {
        const uint4* Xc = Bc + BN * CPR;
        ax[buf] = MT::frag(Xc[lrow * CPR + swz_c<CPR>(lrow, qd)], Xc[lrow * CPR + swz_c<CPR>(lrow, qd + MT::CPF - 1)]);
      }
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = MT::mma(af[buf][i], bw[buf][j], acc[i][j]);
    // columns wn * WTN + wm * 32 + [0, 32): the wm-th of the wave's B blocks,
    // chosen by a select (an index by the runtime wm would go through memory)
    if constexpr (XR > 0) {
      if (xt && wm < 2) acc_x = MT::mma(ax[buf], wm ? bw[buf][1] : bw[buf][0], acc_x);
    }
  };
  // wait until at most `later` stages of this wave's loads are in flight
  // (the ones issued after the stage being waited for); with L the smaller
  // per-wave count this is exact or stricter than needed
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
  if constexpr (MT::kIntAcc) {  // int32 sums -> fp32 (round to nearest even), whole vectors at a time
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_convertvector(__builtin_bit_cast(int32x16, acc[i][j]), f32x16);
  }

  // accumulator element e of block (i, j): row 8*(e/4) + 4*lhalf + e%4, column lrow
  if constexpr (HasChanLN<Epi>::value) {
    // Whole pixel rows: stage acc + bias of the BM x kC tile (row stride
    // kC + 4 floats), then the waves normalise the rows two at a time (32
    // lanes per row, kC / 128 float4 per lane).
    constexpr int D = Epi::kC;
    static_assert(BN == D && BM == 32 * WGM && TM == 1, "row tile shape");
    constexpr int LDR = D + 4;
    constexpr int RPS = 32 * LDR * 4 <= STAGE_BYTES ? 32 : 16;  // staged rows per stage buffer
    static_assert(RPS * LDR * 4 <= STAGE_BYTES && BM <= RPS * S, "staging must fit in the stage LDS");
    constexpr int LPR = 32, V4 = D / (4 * LPR), PAIRS = BM / 2, PASSES = (PAIRS + NW - 1) / NW;
    float* rows_lds[S];
    static_for<0, S>([&](auto c) { rows_lds[decltype(c)::value] = reinterpret_cast<float*>(stage_lds<STAGE_BYTES, decltype(c)::value>()); });
    auto row_ptr = [&](int r) { return rows_lds[r / RPS] + (r % RPS) * LDR; };
    {
      float bcol[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) bcol[j] = epi.bias ? epi.bias[wn * WTN + j * 32 + lrow] : 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          row_ptr(wm * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3))[wn * WTN + j * 32 + lrow] = acc[0][j][e] + bcol[j];
    }
    __syncthreads();
    const int sl = lane & 31;
    const bool second = epi.g2 != nullptr;  // uniform
    float4 gv[V4], bv[V4], g2v[V4], b2v[V4];
#pragma unroll
    for (int i = 0; i < V4; ++i) {
      gv[i] = reinterpret_cast<const float4*>(epi.g)[sl + LPR * i];
      bv[i] = reinterpret_cast<const float4*>(epi.b)[sl + LPR * i];
      g2v[i] = second ? reinterpret_cast<const float4*>(epi.g2)[sl + LPR * i] : make_float4(1.f, 1.f, 1.f, 1.f);
      b2v[i] = second ? reinterpret_cast<const float4*>(epi.b2)[sl + LPR * i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 v[PASSES][V4];
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const float* src = row_ptr(min(pass * NW + wave, PAIRS - 1) * 2 + (lane >> 5));
#pragma unroll
      for (int i = 0; i < V4; ++i) v[pass][i] = *reinterpret_cast<const float4*>(src + 4 * (sl + LPR * i));
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      if (PAIRS % NW != 0 && pass * NW + wave >= PAIRS) break;  // wave-uniform
      const int m = m0 + (pass * NW + wave) * 2 + (lane >> 5);
      ln_group_normalize<V4, LPR>(v[pass], gv, bv, epi.eps, D);
      if (epi.silu) {
#pragma unroll
        for (int i = 0; i < V4; ++i) {
          float4& t = v[pass][i];
          t = make_float4(t.x / (1.f + expf(-t.x)), t.y / (1.f + expf(-t.y)), t.z / (1.f + expf(-t.z)),
                          t.w / (1.f + expf(-t.w)));
        }
      }
      if (second) ln_group_normalize<V4, LPR>(v[pass], g2v, b2v, epi.eps, D);
      if (m < M) {
        bf16_t* orow = epi.out + (size_t)m * epi.ld + epi.c0;
#pragma unroll
        for (int i = 0; i < V4; ++i)
          reinterpret_cast<uint2*>(orow)[sl + LPR * i] =
              make_uint2(pack_bf16x2(v[pass][i].x, v[pass][i].y), pack_bf16x2(v[pass][i].z, v[pass][i].w));
      }
    }
    return;
  }
  if constexpr (HasRowLN<Epi>::value) {
    // Whole rows: stage acc + bias of the BM x kD tile (row stride kD + 4
    // floats; RPS consecutive rows per pipeline stage buffer), then the waves
    // finish the rows two at a time (32 lanes x 3 float4 per row, the lane
    // groups of the standalone LayerNorm).  All reads come before the first store.
    constexpr int D = Epi::kD;
    static_assert(BN == D && BM == 32 * WGM && TM == 1, "row tile shape");
    constexpr int LDR = D + 4;
    constexpr int RPS = 32 * LDR * 4 <= STAGE_BYTES ? 32 : 16;  // staged rows per stage buffer
    static_assert(RPS * LDR * 4 <= STAGE_BYTES && BM <= RPS * S, "staging must fit in the stage LDS");
    // row pair p = pass * NW + wave (rows 2p, 2p + 1, one per lane half)
    constexpr int LPR = 32, V4 = D / (4 * LPR), PAIRS = BM / 2, PASSES = (PAIRS + NW - 1) / NW;
    float* rows_lds[S];
    static_for<0, S>([&](auto c) { rows_lds[decltype(c)::value] = reinterpret_cast<float*>(stage_lds<STAGE_BYTES, decltype(c)::value>()); });
    auto row_ptr = [&](int r) { return rows_lds[r / RPS] + (r % RPS) * LDR; };
    {
      float bcol[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) bcol[j] = epi.bias[wn * WTN + j * 32 + lrow];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          row_ptr(wm * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3))[wn * WTN + j * 32 + lrow] = acc[0][j][e] + bcol[j];
    }
    __syncthreads();
    const int sl = lane & 31;
    float4 sv[V4], gv[V4], bv[V4];
#pragma unroll
    for (int i = 0; i < V4; ++i) {
      sv[i] = reinterpret_cast<const float4*>(epi.ls)[sl + LPR * i];
      gv[i] = reinterpret_cast<const float4*>(epi.g)[sl + LPR * i];
      bv[i] = reinterpret_cast<const float4*>(epi.b)[sl + LPR * i];
    }
    float4 v[PASSES][V4], xo[PASSES][V4];
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int r = min(pass * NW + wave, PAIRS - 1) * 2 + (lane >> 5);
      const int mc = min(m0 + r, M - 1);
      const float* src = row_ptr(r);
#pragma unroll
      for (int i = 0; i < V4; ++i) {
        v[pass][i] = *reinterpret_cast<const float4*>(src + 4 * (sl + LPR * i));
        xo[pass][i] = reinterpret_cast<const float4*>(epi.out + (size_t)mc * D)[sl + LPR * i];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      if (PAIRS % NW != 0 && pass * NW + wave >= PAIRS) break;  // wave-uniform
      const int m = m0 + (pass * NW + wave) * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < V4; ++i) {
        float4& t = v[pass][i];
        t = make_float4(xo[pass][i].x + sv[i].x * t.x, xo[pass][i].y + sv[i].y * t.y,
                        xo[pass][i].z + sv[i].z * t.z, xo[pass][i].w + sv[i].w * t.w);
        if (m < M) reinterpret_cast<float4*>(epi.out + (size_t)m * D)[sl + LPR * i] = t;
      }
      ln_group_normalize<V4, LPR>(v[pass], gv, bv, epi.eps, D);
      if (m < M) {
#pragma unroll
        for (int i = 0; i < V4; ++i)
          reinterpret_cast<uint2*>(epi.h + (size_t)m * D)[sl + LPR * i] =
              make_uint2(pack_bf16x2(v[pass][i].x, v[pass][i].y), pack_bf16x2(v[pass][i].z, v[pass][i].w));
      }
    }
    return;
  }
  if constexpr (HasTransposed<Epi>::value) {
    if (epi.tile_transposed(n0)) {
      // Stage token rows x WTN columns (channels) with the bias added, then
      // read them transposed: 32 rows at a time where the waves' areas fit the
      // stages (row stride WTN + 2 floats; lane -> row, half-wave -> column
      // parity), else 16 (row stride WTN + 4; lane % 16 -> row, lane / 16 ->
      // column residue mod 4).  Either way the reads hit 64 distinct banks.
      constexpr int TSR = (STAGE_BYTES / (32 * (WTN + 2) * 4)) * S >= NW ? 32 : 16;
      constexpr int LDT = TSR == 32 ? WTN + 2 : WTN + 4;
      constexpr int TG = 64 / TSR;  // column residue classes
      constexpr int WAVE_BYTES = TSR * LDT * 4;
      constexpr int WPB = STAGE_BYTES / WAVE_BYTES;
      static_assert(WPB >= 1 && WPB * S >= NW, "staging must fit in the stage LDS");
      float* stage = nullptr;
      static_for<0, S>([&](auto s) {
        if (wave / WPB == decltype(s)::value)
          stage = reinterpret_cast<float*>(stage_lds<STAGE_BYTES, decltype(s)::value>()) + (wave % WPB) * TSR * LDT;
      });
      const int nw0 = n0 + wn * WTN;
      float bcol[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) bcol[j] = epi.tbias(nw0 + j * 32 + lrow);
      const int ch0 = nw0 - 2 * epi.D;
      const int trl = lane % TSR, tg = lane / TSR;
      constexpr int EHT = TSR / 2;  // accumulator elements per staged part
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int h = 0; h < 32 / TSR; ++h) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = h * EHT; e < h * EHT + EHT; ++e)
              stage[((e >> 2) * 8 + lhalf * 4 + (e & 3) - h * TSR) * LDT + j * 32 + lrow] = acc[i][j][e] + bcol[j];
          wave_sync();
          const auto tr = epi.trow(m0 + wm * WTM + i * 32 + h * TSR + trl, M);
          float tv[WTN / TG];
#pragma unroll
          for (int c = 0; c < WTN / TG; ++c) tv[c] = stage[trl * LDT + TG * c + tg];
#pragma unroll
          for (int c = 0; c < WTN / TG; ++c) epi.tstore(tr, ch0 + TG * c + tg, tv[c]);
          wave_sync();
        }
      }
      return;
    }
  }
  if constexpr (!HasRowLN<Epi>::value && !HasChanLN<Epi>::value) {
    // Each wave stages SR rows of one 32-row block of its tile at a time (32, or
    // 16 where the waves' 32-row areas would not fit the stages; row stride
    // WTN + 8 floats: the two lane halves land on disjoint banks), then every
    // lane handles 4 consecutive columns of PASSES rows.  The staging areas
    // live in the (now idle) LDS of the pipeline stages.
    constexpr int LD = WTN + 8;
    constexpr int LPR = WTN / 4;                   // lanes per staged row
    constexpr int RPP = 64 / LPR;                  // rows per pass
    constexpr int SR = (STAGE_BYTES / (32 * LD * 4)) * S >= NW ? 32 : 16;  // rows staged at a time
    constexpr int PASSES = (SR + RPP - 1) / RPP;
    constexpr int WAVE_BYTES = SR * LD * 4;
    constexpr int WPB = STAGE_BYTES / WAVE_BYTES;  // waves per stage object
    static_assert(LPR <= 64, "staging pass shape");
    static_assert(WPB >= 1 && WPB * S >= NW, "staging must fit in the stage LDS");
    float* stage = nullptr;
    static_for<0, S>([&](auto s) {
      if (wave / WPB == decltype(s)::value)
        stage = reinterpret_cast<float*>(stage_lds<STAGE_BYTES, decltype(s)::value>()) + (wave % WPB) * SR * LD;
    });
    const int cl = (lane % LPR) * 4;
    const int n = n0 + wn * WTN + cl;
    const int nvalid = min(4, N - n);
    const bool lane_ok = lane < RPP * LPR && nvalid > 0;
    // Reads are issued for every lane at in-range addresses (idle lanes read
    // the tile's first columns or the last row) so that no branch surrounds them.
    const int n_rd = lane_ok ? n : n0;
    const int nvalid_rd = lane_ok ? nvalid : min(4, N - n0);
    const typename Epi::Col cc = epi.col4(n_rd, nvalid_rd);
    // One staged block of SR rows (rows row0 + [0, SR)): this lane's 4 columns at
    // column nl (ok: inside the block and the matrix), with the read-side
    // column nl_rd / count nv_rd and the column constants c.
    auto emit = [&](int row0, int nl, int nv, bool ok, int nl_rd, int nv_rd, const typename Epi::Col& c) {
      float v[PASSES][4];
      typename Epi::Row rw[PASSES];
      const int mb = row0 + lane / LPR;
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
        const int r = min(pass * RPP + lane / LPR, SR - 1);
        const float4 t = *reinterpret_cast<const float4*>(stage + r * LD + cl);
        v[pass][0] = t.x;
        v[pass][1] = t.y;
        v[pass][2] = t.z;
        v[pass][3] = t.w;
        rw[pass] = epi.pre(min(mb + pass * RPP, M - 1), nl_rd, nv_rd);
      }
      // Loads and stores share vmcnt: an epilogue without global reads per
      // block waits only for its LDS reads, not for the previous block's stores.
      if constexpr (std::is_same<typename Epi::Row, NoRow>::value)
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the staged values are in
      else
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): every read of this block is in
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) epi.finish4(v[pass], c, rw[pass]);
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
        const int r = pass * RPP + lane / LPR;
        if (ok && r < SR && mb + pass * RPP < M) write4_any(epi, mb + pass * RPP, nl, v[pass], nv, c, 0);
      }
    };
    // accumulator element e holds row 8 (e / 4) + 4 lhalf + e % 4 of its block:
    // rows [16 h, 16 h + 16) are elements 8 h .. 8 h + 7
    constexpr int EH = SR / 2;  // elements per staged part
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int h = 0; h < 32 / SR; ++h) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = h * EH; e < h * EH + EH; ++e)
            stage[((e >> 2) * 8 + lhalf * 4 + (e & 3) - h * SR) * LD + j * 32 + lrow] = acc[i][j][e];
        wave_sync();
        emit(m0 + wm * WTM + i * 32 + h * SR, n, nvalid, lane_ok, n_rd, nvalid_rd, cc);
        wave_sync();
      }
    }
    if constexpr (XR > 0) {
      if (xt && wm < 2) {  // wave-uniform
        // the extra rows: staged in the first 32 columns of the wave's area
        static_assert(SR == 32, "extra rows are staged whole");
#pragma unroll
        for (int e = 0; e < 16; ++e) stage[((e >> 2) * 8 + lhalf * 4 + (e & 3)) * LD + lrow] = acc_x[e];
        wave_sync();
        const int nx = n0 + wn * WTN + wm * 32 + cl;
        const int nvx = min(4, N - nx);
        const bool okx = lane < RPP * LPR && cl < 32 && nvx > 0;
        const int nx_rd = okx ? nx : n0;
        const int nvx_rd = okx ? nvx : min(4, N - n0);
        const typename Epi::Col ccx = epi.col4(nx_rd, nvx_rd);
        emit(xr0, nx, nvx, okx, nx_rd, nvx_rd, ccx);
      }
    }
  }
}

// Tile configuration: BM x BN tile, WGM x WGN waves, S pipeline stages.
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int S_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, S = S_;
};

// 128- and 256-row tiles with plain row epilogues can take up to 32 rows past
// the last full row tile (see gemm_bf16_kernel's XR).
template <class C, class Epi, class AM, class MT>
constexpr bool takes_extra_rows() {
  return (C::BM == 128 || C::BM == 256) && (C::WGM == 2 || C::WGM == 4) && C::BN / C::WGN == 64 && !HasRowLN<Epi>::value &&
         !HasChanLN<Epi>::value && !HasTransposed<Epi>::value && !AM::kConv && std::is_same<MT, MmaBf16>::value;
}

template <class C, class Epi, class AM = AMapLinear, class MT = MmaBf16>
hipError_t run(const bf16_t* A, const bf16_t* W, int M, int N, int K, const Epi& epi, hipStream_t s, AM am = {},
               int extra_wgs = 0) {
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  if (K % C::BK != 0) return hipErrorInvalidValue;
  if constexpr (takes_extra_rows<C, Epi, AM, MT>()) {
    const int rem = M % C::BM;
    if (M > C::BM && rem > 0 && rem <= 32) {  // row tile 0 also computes the rem rows after the last full one
      const int full = M / C::BM;
      hipLaunchKernelGGL((gemm_bf16_kernel<C::BM, C::BN, C::BK, C::WGM, C::WGN, C::S, Epi, AM, MT, 32>),
                         dim3(full * tiles_n), dim3(64 * C::WGM * C::WGN), 0, s, A, W, M, N, K, full, tiles_n, epi, am,
                         0);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<C::BM, C::BN, C::BK, C::WGM, C::WGN, C::S, Epi, AM, MT>),
                     dim3(tiles_m * tiles_n + extra_wgs), dim3(64 * C::WGM * C::WGN), 0, s, A, W, M, N, K, tiles_m,
                     tiles_n, epi, am, -1);
  return hipGetLastError();
}

// Tile shapes measured on MI355X over the encoder's GEMMs (M = 4101..16404,
// N = 384..4096, K = 384..4096): 128 x 128 is best or equal on most; 64 x 128
// wins on short-K products with few tiles (more resident workgroups per CU);
// 256 x 256 wins only on very large products.
using CfgMid = Cfg<128, 128, 64, 2, 2, 2>;
using CfgSmall = Cfg<64, 128, 64, 2, 2, 2>;
using CfgBig = Cfg<256, 256, 64, 2, 4, 2>;
// 256 x 256 on 16 waves (64 x 64 wave tiles, four waves per SIMD at <= 128
// VGPRs), epilogue rows staged 16 at a time: the fused Q/K/V projection, which
// takes no extra rows (with them the 16-wave kernels spill)
using CfgBig16 = Cfg<256, 256, 64, 4, 4, 2>;
using CfgTiny = Cfg<64, 64, 64, 2, 2, 2>;
// 128 x 128 with 8 waves (32 x 64 wave tiles): two waves per SIMD for grids of
// at most one tile per CU with extra rows (ViT-L/16 b1 out-proj and fc2), where
// the second wave of a SIMD covers the first one's load waits, and four for
// short-K products with two workgroups per CU.  Without extra rows the eight
// waves stage their epilogue rows 16 at a time (32 would not fit the stages).
using CfgMidW8 = Cfg<128, 128, 64, 4, 2, 2>;
// fp8 operands: a K step of 128 values is the same 128-byte row slice as 64 bf16 values
using CfgMid8 = Cfg<128, 128, 128, 2, 2, 2>;
using CfgSmall8 = Cfg<64, 128, 128, 2, 2, 2>;
using CfgTiny8 = Cfg<64, 64, 128, 2, 2, 2>;

template <class Epi, class AM = AMapLinear>
hipError_t dispatch(const bf16_t* A, const bf16_t* W, int M, int N, int K, const Epi& epi, hipStream_t s,
                    AM am = {}) {
  const long mid_tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  if ((long)M * N >= 32L * 1024 * 1024) return run<CfgBig>(A, W, M, N, K, epi, s, am);
  if constexpr (takes_extra_rows<CfgBig, Epi, AM, MmaBf16>()) {
    // 256 x 256 tiles, the rows past the last full row tile taken by row tile
    // 0, when they fill at least 7/8 of the CUs and W holds >= 4M values:
    // half the operand bytes per FLOP of 128 x 128 (ViT-L/16 b1 fc1, 4101 x
    // 4096 x 1024: 16 x 16 tiles, 45.9 -> 42.3 us; b4 fc2, 16404 x 1024 x 4096:
    // 138.6 -> 132.9 us; b4 out-proj with W of 1M values was slower, 47.1 ->
    // 49.1 us; same-process A/B, outputs bit-identical)
    const long big_tiles = (long)(M / 256) * ((N + 255) / 256);
    if (M > 256 && M % 256 <= 32 && (long)K * N >= 4L * 1024 * 1024 && big_tiles >= 224)
      return run<CfgBig>(A, W, M, N, K, epi, s, am);
  }
  if (mid_tiles < 256) {  // fewer 128 x 128 tiles than compute units: 64 x 128, or 64 x 64 if that too is short
    const long small_tiles = (long)((M + 63) / 64) * ((N + 127) / 128);
    if (small_tiles >= 256) return run<CfgSmall>(A, W, M, N, K, epi, s, am);
    return run<CfgTiny>(A, W, M, N, K, epi, s, am);
  }
  if (K <= 512 && mid_tiles < 512) return run<CfgSmall>(A, W, M, N, K, epi, s, am);
  if constexpr (takes_extra_rows<CfgMidW8, Epi, AM, MmaBf16>()) {
    // ViT-L/16 b1 out-proj and fc2 (4101 x 1024, 256 tiles): 18.5 -> 18.1 us and
    // 47.6 -> 46.1 us, forward 6.019 -> 5.982 ms (same-process A/B, outputs
    // bit-identical)
    using C = CfgMidW8;
    const int tiles_n = (N + C::BN - 1) / C::BN, full = M / C::BM, rem = M % C::BM;
    if ((long)full * tiles_n <= 256 && full >= 1 && rem > 0 && rem <= 32) {
      hipLaunchKernelGGL((gemm_bf16_kernel<C::BM, C::BN, C::BK, C::WGM, C::WGN, C::S, Epi, AM, MmaBf16, 32>),
                         dim3(full * tiles_n), dim3(64 * C::WGM * C::WGN), 0, s, A, W, M, N, K, full, tiles_n, epi, am, 0);
      return hipGetLastError();
    }
  }
  if constexpr (!AM::kConv) {
    // short-K products with several tiles per CU (ViT-S fc1, 14272 x 1536 x
    // 384: 37.8 -> 34.6 us; DINOv2-S @518 b8 fc1: 29.5 -> 27.4 us; same-process
    // A/B, outputs bit-identical): two 8-wave workgroups per CU put four waves
    // on each SIMD, so one workgroup's epilogue overlaps the other's loads.
    // Longer K gained nothing (ViT-L b4 out-proj 48.7 -> 50.4 us).
    if (K <= 512) return run<CfgMidW8>(A, W, M, N, K, epi, s, am);
  }
  return run<CfgMid>(A, W, M, N, K, epi, s, am);
}

// Phi table of the GELU epilogue: built once per device (synchronous copy to
// the device symbol); returns the device address or nullptr on failure.
const float2* phi_table_device() {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static const float2* addr[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    float2 host[kPhiPadded] = {};
    double prev = 0.5 * std::erfc(6.0 / std::sqrt(2.0));  // Phi(-6)
    for (int i = 0; i < kPhiPoints; ++i) {
      const double x1 = -6.0 + (i + 1) / 64.0;
      const double next = i + 1 < kPhiPoints ? 0.5 * std::erfc(-x1 / std::sqrt(2.0)) : prev;
      host[i] = make_float2((float)prev, (float)(next - prev));
      prev = next;
    }
    void* p = nullptr;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_phi_table), host, sizeof(host)) != hipSuccess) return nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_phi_table)) != hipSuccess) return nullptr;
    addr[dev] = static_cast<const float2*>(p);
  }
  return addr[dev];
}

// Fused Q/K/V: the V tiles must not straddle the K|V boundary at 2D.  With
// K >= 1024 the 256 x 256 tiles pay from 8M outputs on (ViT-L/16 b1: 4101 x
// 3072, forward -1.4% in a same-process A/B; the per-output k order, and so
// the result, is that of every other tile shape).
hipError_t dispatch_qkv(const bf16_t* A, const bf16_t* W, int M, int N, int K, const EpiQKV& epi, hipStream_t s) {
  const long mid_tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  const long outs = (long)M * N;
  // 16 waves: ViT-L/16 b1 4101 x 3072 x 1024 37.3 -> 34.6 us, b4 132.3 -> 123.2 us
  // against 8 (same-process A/B, q and k bit-identical)
  if ((outs >= 32L * 1024 * 1024 || (K >= 1024 && outs >= 8L * 1024 * 1024)) && (2 * epi.D) % CfgBig16::BN == 0)
    return run<CfgBig16>(A, W, M, N, K, epi, s);
  if (K <= 512 && mid_tiles < 512) return run<CfgSmall>(A, W, M, N, K, epi, s);
  // short K: 8-wave tiles as in dispatch (DINOv2-S @518 b8, 10960 x 1152 x
  // 384: 22.3 -> 20.9 us; ViT-S b32 25.9 -> 25.6 us; same-process A/B)
  if (K <= 512) return run<CfgMidW8>(A, W, M, N, K, epi, s);
  return run<CfgMid>(A, W, M, N, K, epi, s);
}

using CfgRowLN = Cfg<64, EpiResidualLN::kD, 64, 2, 4, 2>;

// Channel LayerNorm epilogue: 32 pixel rows x all kC channels per workgroup.
template <int C, class AM>
hipError_t run_chan_ln(const bf16_t* A, const bf16_t* W, int M, int K, const EpiParams& ep, hipStream_t s, AM am) {
  const EpiChanLN<C> e{ep.bias, ep.ln_g, ep.ln_b, ep.eps, ep.silu, ep.ln2_g, ep.ln2_b, (bf16_t*)ep.out, ep.ldc, ep.c0};
  // 32-row tiles (about 1.3 workgroups per CU at 8 x 37 x 37 pixels) measured
  // faster than 64-row ones for every conv of the head (b8: 288 vs 298 us).
  // These short loops (18-24 k-steps) wait on their loads: a third stage for
  // the 128-channel tiles (60 KB, still two workgroups per CU) took the b8
  // head from 298 to 268 us; the 256-channel tiles stay at two (a third, 108
  // KB, leaves one workgroup per CU: 281 us).
  return run<Cfg<32, C, 64, 1, 4, (C == 128 ? 3 : 2)>>(A, W, M, C, K, e, s, am);
}

// Checks shared by the linear and convolution forms of EPI_CHAN_LN.
template <class AM>
hipError_t dispatch_chan_ln(const bf16_t* A, const bf16_t* W, int M, int N, int K, const EpiParams& ep, hipStream_t s,
                            AM am = {}) {
  auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  if (!chan_ln_fusable(N) || !ep.out || !ep.ln_g || !ep.ln_b || !al16(ep.ln_g) || !al16(ep.ln_b) ||
      (ep.ln2_g && (!ep.ln2_b || !al16(ep.ln2_g) || !al16(ep.ln2_b))) || ep.ldc % 4 || ep.c0 % 4 || ep.c0 < 0 ||
      ep.c0 + N > ep.ldc || reinterpret_cast<uintptr_t>(ep.out) % 8)
    return hipErrorInvalidValue;
  if (N == 128) return run_chan_ln<128>(A, W, M, K, ep, s, am);
  return run_chan_ln<256>(A, W, M, K, ep, s, am);
}

// 8-bit tiles (fp8 or int8 operands, 128 values per K step), chosen by the
// same rules as the bf16 ones (no 256 x 256 tile: its 8-bit fragments would
// not fit the registers)
template <class MT, class Epi>
hipError_t dispatch_8bit(const void* A, const void* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  const auto a = reinterpret_cast<const bf16_t*>(A);
  const auto w = reinterpret_cast<const bf16_t*>(W);
  const long mid_tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (mid_tiles < 256) {
    const long small_tiles = (long)((M + 63) / 64) * ((N + 127) / 128);
    if (small_tiles >= 256) return run<CfgSmall8, Epi, AMapLinear, MT>(a, w, M, N, K, epi, s);
    return run<CfgTiny8, Epi, AMapLinear, MT>(a, w, M, N, K, epi, s);
  }
  if (K <= 1024 && mid_tiles < 512) return run<CfgSmall8, Epi, AMapLinear, MT>(a, w, M, N, K, epi, s);
  return run<CfgMid8, Epi, AMapLinear, MT>(a, w, M, N, K, epi, s);
}

}  // namespace

hipError_t prepare_gemm() { return phi_table_device() ? hipSuccess : hipErrorInvalidValue; }

hipError_t launch_gemm(const uint16_t* A, const uint16_t* W, int M, int N, int K, const EpiParams& ep,
                       hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0 || K % BK != 0) return hipErrorInvalidValue;
  if ((size_t)(M + 128) * K * 2 >= (1ull << 32) || (size_t)(N + 128) * K * 2 >= (1ull << 32))
    return hipErrorInvalidValue;  // 32-bit buffer offsets
  auto al = [](const void* p, size_t n) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % n == 0; };
  const bool par16 = N % 4 == 0 && al(ep.bias, 16) && al(ep.ls, 16);
  switch (ep.kind) {
    case EPI_BIAS_BF16: {
      const bool vec = ep.ldc % 4 == 0 && par16 && al(ep.out, 8);
      return dispatch(A, W, M, N, K, EpiBiasBf16{ep.bias, (bf16_t*)ep.out, ep.ldc, vec}, s);
    }
    case EPI_GELU_BF16: {
      const bool vec = ep.ldc % 4 == 0 && par16 && al(ep.out, 8);
      const float2* phi = phi_table_device();
      if (!phi) return hipErrorInvalidValue;
      return dispatch(A, W, M, N, K, EpiGeluBf16{ep.bias, (bf16_t*)ep.out, ep.ldc, vec, phi}, s);
    }
    case EPI_RESIDUAL: {
      const bool vec = ep.ldc % 4 == 0 && par16 && al(ep.out, 16);
      return dispatch(A, W, M, N, K, EpiResidual{ep.bias, ep.ls, (float*)ep.out, ep.ldc, vec}, s);
    }
    case EPI_BIAS_F32: {
      const bool vec = ep.ldc % 4 == 0 && par16 && al(ep.out, 16);
      return dispatch(A, W, M, N, K, EpiBiasF32{ep.bias, (float*)ep.out, ep.ldc, vec}, s);
    }
    case EPI_QKV: {
      const int D = N / 3;
      const FastDiv dn = make_fastdiv(ep.tokens);
      const bool vec = par16 && al(ep.q, 8) && al(ep.k, 8);
      EpiQKV e;
      static_cast<EpiQK&>(e) = EpiQK{ep.bias, ep.q, ep.k, D, ep.tokens, ep.heads, dn, kLog2e * 0.125f, vec};
      e.vt = ep.vt;
      e.nv = ep.nv;
      return dispatch_qkv(A, W, M, N, K, e, s);
    }
    case EPI_RESIDUAL_LN: {
      if (N != EpiResidualLN::kD || ep.ldc != N) return hipErrorInvalidValue;
      auto al16 = [&](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
      if (!al16(ep.bias) || !al16(ep.ls) || !al16(ep.out) || !al16(ep.ln_g) || !al16(ep.ln_b) || !ep.h ||
          reinterpret_cast<uintptr_t>(ep.h) % 8 != 0)
        return hipErrorInvalidValue;
      EpiResidualLN e{ep.bias, ep.ls, (float*)ep.out, ep.ln_g, ep.ln_b, ep.eps, (bf16_t*)ep.h};
      // One 64-row tile per CU (its two stages fill most of the LDS); where
      // the tiles leave CUs idle, up to that many extra workgroups read the
      // prefetch region there, about 8 chunks of 16 bytes per lane, so that
      // they finish well within the tiles' time.
      const int tiles = (M + CfgRowLN::BM - 1) / CfgRowLN::BM;
      int extra = 0;
      if (ep.prefetch && ep.prefetch_bytes >= 16 && tiles < kComputeUnits) {
        if (reinterpret_cast<uintptr_t>(ep.prefetch) % 16 != 0 || ep.prefetch_bytes >= (1ull << 32))
          return hipErrorInvalidValue;
        const uint32_t chunks = (uint32_t)(ep.prefetch_bytes / 16);
        constexpr uint32_t per_wg = 64u * CfgRowLN::WGM * CfgRowLN::WGN * 8u;
        extra = (int)std::min<uint32_t>((uint32_t)(kComputeUnits - tiles), (chunks + per_wg - 1) / per_wg);
        e.pf = static_cast<const uint4*>(ep.prefetch);
        e.pf_chunks = chunks;
      }
      return run<CfgRowLN>(A, W, M, N, K, e, s, AMapLinear{}, extra);
    }
    case EPI_CHAN_LN:
      return dispatch_chan_ln(A, W, M, N, K, ep, s, AMapLinear{});
    case EPI_PATCH: {
      const bool vec = par16 && al(ep.pos, 16) && al(ep.out, 16);
      EpiPatch e{ep.bias, ep.pos, (float*)ep.out, ep.ldc, ep.tokens, ep.patches, ep.regs, make_fastdiv(ep.patches),
                 vec};
      return dispatch(A, W, M, N, K, e, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_fp8(const uint8_t* A, const uint8_t* W, int M, int N, int K, float scale, const float* bias,
                           void* out, int ldc, bool out_f32, hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || ldc < N || !out) return hipErrorInvalidValue;
  if ((size_t)(M + 256) * K >= (1ull << 32) || (size_t)(N + 256) * K >= (1ull << 32)) return hipErrorInvalidValue;
  auto al = [](const void* p, size_t n) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % n == 0; };
  const bool vec = N % 4 == 0 && ldc % 4 == 0 && al(bias, 16) && al(out, out_f32 ? 16 : 8);
  if (out_f32) return dispatch_8bit<MmaFp8>(A, W, M, N, K, EpiScale<true>{scale, bias, out, ldc, vec}, s);
  return dispatch_8bit<MmaFp8>(A, W, M, N, K, EpiScale<false>{scale, bias, out, ldc, vec}, s);
}

hipError_t launch_gemm_int8(const int8_t* A, const int8_t* W, int M, int N, int K, float scale, const float* bias,
                            void* out, int ldc, bool out_f32, hipStream_t s) {
  // K * 127^2 < 2^31: the int32 sums cannot overflow
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || K > 131072 || ldc < N || !out) return hipErrorInvalidValue;
  if ((size_t)(M + 256) * K >= (1ull << 32) || (size_t)(N + 256) * K >= (1ull << 32)) return hipErrorInvalidValue;
  auto al = [](const void* p, size_t n) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % n == 0; };
  const bool vec = N % 4 == 0 && ldc % 4 == 0 && al(bias, 16) && al(out, out_f32 ? 16 : 8);
  if (out_f32) return dispatch_8bit<MmaI8>(A, W, M, N, K, EpiScale<true>{scale, bias, out, ldc, vec}, s);
  return dispatch_8bit<MmaI8>(A, W, M, N, K, EpiScale<false>{scale, bias, out, ldc, vec}, s);
}

hipError_t launch_gemm_conv3(const uint16_t* in, int ld_in, int c0, int C, int batch, int gh, int gw,
                             const uint16_t* W, int N, const EpiParams& ep, hipStream_t s) {
  if (C <= 0 || C % BK || c0 < 0 || c0 % 8 || ld_in % 8 || c0 + C > ld_in || batch < 1 || gh < 1 || gw < 1 || N <= 0)
    return hipErrorInvalidValue;
  const size_t M = (size_t)batch * gh * gw, K = (size_t)9 * C;
  const size_t bytes = M * ld_in * 2;
  if (bytes >= (1ull << 31) || (M + 128) * K * 2 >= (1ull << 32) || (size_t)(N + 128) * K * 2 >= (1ull << 32))
    return hipErrorInvalidValue;  // 32-bit buffer offsets; 0x80000000 marks the zero padding
  auto al = [](const void* p, size_t n) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % n == 0; };
  const bool par16 = N % 4 == 0 && al(ep.bias, 16);
  const AMapConv3 am{gh, gw, ld_in, c0, C, (uint32_t)bytes};
  switch (ep.kind) {
    case EPI_BIAS_BF16: {
      const bool vec = ep.ldc % 4 == 0 && par16 && al(ep.out, 8);
      return dispatch(in, W, (int)M, N, (int)K, EpiBiasBf16{ep.bias, (bf16_t*)ep.out, ep.ldc, vec}, s, am);
    }
    case EPI_BIAS_F32: {
      const bool vec = ep.ldc % 4 == 0 && par16 && al(ep.out, 16);
      return dispatch(in, W, (int)M, N, (int)K, EpiBiasF32{ep.bias, (float*)ep.out, ep.ldc, vec}, s, am);
    }
    case EPI_CHAN_LN:
      return dispatch_chan_ln(in, W, (int)M, N, (int)K, ep, s, am);
    case EPI_BIAS_F32_G8:
      if (N % 8 || !ep.out || !al(ep.out, 16) || !al(ep.bias, 16) || ep.ldc < 0 || (size_t)ep.ldc < 8 * M)
        return hipErrorInvalidValue;
      // 64 x 128 tiles with a third stage (72 KB, two workgroups per CU): the
      // head's smoothing conv (K = 2304, 344 tiles at b8) waits on its loads;
      // the third stage took the b8 head from 258.6 to 251.1 us
      return run<Cfg<64, 128, 64, 2, 2, 3>>(in, W, (int)M, N, (int)K,
                                            EpiBiasF32G8{ep.bias, (float*)ep.out, (size_t)ep.ldc}, s, am);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace vit
