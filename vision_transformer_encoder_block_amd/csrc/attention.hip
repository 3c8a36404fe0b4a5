// Fused multi-head attention for gfx950, head size 64:
//   O = softmax_keys(Q K^T / sqrt(64)) V   per (image, head)
// computed flash-style without storing the N x N logits.
//
// Each wave owns 32 queries.  It computes the TRANSPOSED logits S^T = K Q^T
// with v_mfma_f32_32x32x16_bf16 (keys on the MFMA rows, queries on the
// columns), so every lane holds 32 logits of ONE query: the per-query running
// max and sum are lane-local plus one exchange with the partner lane (lane ^
// 32) that holds the other keys of the same query.  The probabilities then
// feed O^T = V^T P^T straight from the accumulator registers (no LDS round
// trip): the key order inside each 16-key MFMA step is the accumulator's
// order, and V^T is stored with bits 2 and 3 of the token index exchanged so
// that the eight keys one lane needs are 16 contiguous bytes.
//
// Q arrives pre-multiplied by log2(e)/8, so p = exp2(s - m) with s, m, the
// running max and sum all fp32: logits of ~2.5e6 (the DINOv3 attention sink)
// stay finite.  The reference max m is moved lazily (only when a tile max
// exceeds it by more than 8), which keeps every p <= 2^8 and skips most
// rescales of the output accumulators.  After the first tile the
// probabilities are formed before any tile max; the max is taken (and the
// tile recomputed) only where a lane's sum of p exceeds 2^8, which any p above
// 2^8 implies, so the outputs are those of the max-first order.
// K and V^T tiles of 64 keys are staged in LDS (double-buffered, 16-byte
// chunks XOR-swizzled by row) and shared by the 4 waves of a workgroup; rows
// past the sequence end are read as zeros through buffer range checks.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace vit {
namespace {

constexpr int QT = 128;  // queries per workgroup (4 waves x 32)
constexpr int KT = 64;   // keys per tile

// Inverse of the token permutation used by vt (an involution).
__device__ __forceinline__ int vt_tok(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// LDS position of 16-byte chunk c of row r: the 16 rows read by 16 lanes of one
// ds_read_b128 cover all 64 banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// One workgroup: NW waves x 32 query rows starting at 32 NW qt, against all
// N keys; it writes the normalised output of its rows.
struct AttnArgs {
  const bf16_t* Q;
  const bf16_t* K;
  const bf16_t* Vt;
  bf16_t* O;
  int N, H, nv;
  int qtiles;      // query tiles per (b, h); the grid is 1-D
  int B;
  int split;       // 1: the last query tile holds 1..32 queries and its waves split the keys
  int n_attn;      // workgroups that compute attention; the ones after them prefetch
  const uint4* pf; // region the prefetch workgroups read into the caches (or null)
  uint32_t pf_chunks;  // its length in 16-byte chunks
};

// Workgroup id -> (query tile, head, image).  Workgroups are handed
// to the 8 XCDs round-robin by id; the ids are renumbered so that each XCD
// gets a contiguous run of (image, head) pairs and all query tiles of a pair
// meet the same K and V^T in that XCD's L2.
__device__ __forceinline__ void full_coords(int bid, int qtiles, int H, int B, int& qt, int& h, int& b) {
  constexpr int XCD = 8;
  const int n = qtiles * H * B;
  const int per = (n + XCD - 1) / XCD;
  int tall = n % XCD;
  if (tall == 0) tall = XCD;
  const int xcd = bid % XCD, local = bid / XCD;
  const int pid = xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
  qt = pid % qtiles;
  const int bh = pid / qtiles;
  h = bh % H;
  b = bh / H;
}

// At most 168 VGPRs (3 waves per SIMD): three 4-wave workgroups per CU keep
// e.g. a ViT-S/16 @336 batch of 32 (768 workgroups) resident in one round.
template <int NW>
__global__ __launch_bounds__(64 * NW, 12 / NW) void attention_kernel(AttnArgs a) {
  constexpr int S = 3;         // K / V^T tile stages in LDS
  constexpr int IPW = 8 / NW;  // DMA instructions per wave per K (or V^T) tile
  constexpr int L = 2 * IPW;   // ... per tile of both
  static_assert(S * L < 64, "vmcnt range");
  __shared__ uint4 KV[S][2][KT * 8];  // [stage][K | V^T][16-byte chunk]

  // Workgroups past the attention grid read weights that the next kernels
  // will stream (attention itself needs little of the memory system).
  if ((int)blockIdx.x >= a.n_attn) {  // workgroup-uniform
    prefetch_region(a.pf, a.pf_chunks, blockIdx.x - a.n_attn, gridDim.x - a.n_attn);
    return;
  }
  const int N = a.N, H = a.H, nv = a.nv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int qt, h, b;
  full_coords(blockIdx.x, a.qtiles, H, a.B, qt, h, b);
  const size_t bh = (size_t)b * H + h;
  const bf16_t* Qp = a.Q + bh * N * 64;
  const bf16_t* Kp = a.K + bh * N * 64;
  const bf16_t* Vp = a.Vt + bh * 64 * nv;
  const int lrow = lane & 31, lhalf = lane >> 5;
  // A last query tile with only 1..32 queries would leave one wave doing the
  // whole key range while three idle: instead all NW waves take its 32 query
  // rows, wave w the key half w % 2 of the tiles of parity w / 2, and they
  // merge their partial results at the end.  Whether a tile splits depends on
  // the sequence length only, so outputs do not depend on the batch.
  static_assert(NW == 4, "the key split pairs 2 tile parities with 2 key halves");
  const bool split = a.split && qt == a.qtiles - 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int kb_own = wave_u & 1, par = wave_u >> 1;
  const int row0 = split ? qt * 32 * NW : qt * 32 * NW + wave * 32;
  const int qrow = row0 + lrow;
  const bool idle = __builtin_amdgcn_readfirstlane(row0) >= N;

  // rows past N read as zeros through the buffer range checks
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qp, (uint32_t)N * 128u);
  const int32x4 rk_w = make_rsrc_words(Kp, (uint32_t)N * 128u);
  const int32x4 rv_w = make_rsrc_words(Vp, (uint32_t)nv * 128u);
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(buf_load16(rq, (uint32_t)qrow * 128u + ks * 32 + lhalf * 16));

  // K and V^T tiles (64 rows of 8 chunks of 16 bytes) arrive by direct-to-LDS
  // buffer loads: each wave instruction fills 8 rows (1 KB); the lane at slot
  // (row, p) fetches the logical chunk p ^ ((row >> 1) & 7), which is where the
  // swizzled reads below look for it.  K rows past N come back as zeros; the
  // V^T columns of keys >= N (padding of unspecified content) are zeroed in
  // LDS once the ragged last tile has landed, so they meet p = 0 as zeros.
  const uint32_t kv_base = lds_addr(&KV[0][0][0]);
  uint32_t k_off[IPW], v_off[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int row = (j * NW + wave) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    k_off[j] = (uint32_t)row * 128u + c * 16u;
    v_off[j] = (uint32_t)row * (uint32_t)nv * 2u + c * 16u;
  }
  auto issue = [&](int t, int stage) {
    const uint32_t k0 = (uint32_t)t * KT;
    const uint32_t kb = kv_base + (uint32_t)stage * (2 * KT * 8 * 16);
#pragma unroll
    for (int j = 0; j < IPW; ++j) dma16(rk_w, k_off[j] + k0 * 128u, kb + (uint32_t)(j * NW + wave_u) * 1024u);
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      dma16(rv_w, v_off[j] + k0 * 2u, kb + KT * 8 * 16 + (uint32_t)(j * NW + wave_u) * 1024u);
  };
  // wait until at most `later` tiles of this wave's loads are in flight
  auto wait_tiles = [&](int later) {
    if (later <= 0) wait_vm<0>();
    else if (later == 1) wait_vm<L>();
    else wait_vm<2 * L>();
  };
  static_assert(S <= 3, "wait_tiles covers up to two tiles in flight");
  // Zero the V^T entries of keys >= N in the stage holding tile t (called by
  // every thread after the barrier that publishes it; a barrier follows).
  auto fix_last = [&](int t, int stage) {
    uint4* vs = KV[stage][1];
    const int k0 = t * KT;
    for (int cid = tid; cid < 64 * 8; cid += 64 * NW) {
      const int r = cid >> 3, c = cid & 7;
      const int p0 = k0 + c * 8;
      uint4& u = vs[r * 8 + swz(r, c)];
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (vt_tok(p0 + e) >= N) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      u = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  float m_run = 0.f, l_run = 0.f;
  f32x16 o[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[0][e] = o[1][e] = 0.f;
  // Fifth MFMA k-step of S^T: ones (keys) x -m_run (queries) subtracts the
  // reference max inside the accumulation.  -m_run is split into three bf16
  // parts (8 + 8 + 8 significant bits cover fp32's 24, so the split is exact);
  // they sit in k-slots 0..2, held by the lower lane half.
  bf16x8 ones, mneg;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ones[e] = (__bf16)((lhalf == 0 && e < 3) ? 1.f : 0.f);
    mneg[e] = (__bf16)0.f;
  }
  auto set_mneg = [&](float m) {
    const float n = -m;
    const __bf16 h0 = (__bf16)n;
    const float r1 = n - (float)h0;
    const __bf16 h1 = (__bf16)r1;
    const __bf16 h2 = (__bf16)(r1 - (float)h1);
    mneg[0] = lhalf == 0 ? h0 : (__bf16)0.f;
    mneg[1] = lhalf == 0 ? h1 : (__bf16)0.f;
    mneg[2] = lhalf == 0 ? h2 : (__bf16)0.f;
  };

  const int nt = (N + KT - 1) / KT;  // key tiles; only the last is ragged
#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if (i < nt) issue(i, i);
  // Every load so far is waited for here (tile 0, which is needed, and the
  // tiles issued with it): the explicit vmcnt(0) also tells the compiler that
  // the Q fragments have landed, so it places no vmcnt waits for them in the
  // loop, where they would also wait for the K / V^T tiles in flight.
  wait_vm<0>();
  barrier_keep_loads();
  if (KT > N) {
    fix_last(0, 0);
    __syncthreads();
  }

  // Issue priority falls as a wave gets through its key range (3 at the
  // start, 2 past a quarter, 1 past half, 0 past three quarters).  The
  // arbiter otherwise favours the oldest waves; their workgroup finishes
  // first and leaves the CU with fewer waves to hide latency for the rest.
  __builtin_amdgcn_s_setprio(3);
  // The work of one wave on one key tile: NKB 32-key halves starting at half
  // kb0 (2 and 0 for a whole tile).  `first` marks the wave's first tile, where
  // the tile max always sets m_run.
  auto compute = [&](auto nkb_c, int t, int stage, int kb0, bool first) __attribute__((always_inline)) {
    constexpr int NKB = decltype(nkb_c)::value;
    const uint4* Ks = KV[stage][0];
    const uint4* Vs = KV[stage][1];

    // S^T for keys t*64 + kb*32 + [0, 32): element e <-> key 8*(e/4) + 4*lhalf + e%4.
    // All K fragments are read before the MFMAs, and the V fragments right
    // after them, so the LDS latency of both hides under MFMA and softmax work.
    // vf[db][j] and pf[j] belong to the 16-key step 2 kb0 + j of the tile.
    bf16x8 vf[2][2 * NKB];
    f32x16 s[NKB];
    // s = S^T - m_run (the first tile runs with m_run = 0); keys past N
    // (last tile only) get -inf.  The V fragments are read right after the
    // K fragments on the first call.
    auto logits = [&](bool read_v) {
      bf16x8 kf[NKB][4];
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const int r = (kb0 + kk) * 32 + lrow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[kk][ks] = as_bf16x8(Ks[r * 8 + swz(r, ks * 2 + lhalf)]);
      }
      if (read_v) {
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int r = db * 32 + lrow;
#pragma unroll
          for (int j = 0; j < 2 * NKB; ++j) vf[db][j] = as_bf16x8(Vs[r * 8 + swz(r, (2 * kb0 + j) * 2 + lhalf)]);
        }
      }
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kk][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) s[kk] = mfma32x32x16(kf[kk][ks], qf[ks], s[kk]);
        s[kk] = mfma32x32x16(ones, mneg, s[kk]);
      }
      if ((t + 1) * KT > N) {
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = t * KT + (kb0 + kk) * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
            if (key >= N) s[kk][e] = -INFINITY;
          }
      }
    };
    // probabilities p = 2^s, packed as the B operand of the key steps of
    // P V; returns this lane's sum of its 16 NKB (a tree of pairwise adds)
    bf16x8 pf[2 * NKB];
    auto probs = [&]() {
      float ps[2 * NKB];
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(s[kk][half * 8 + e]);
          ps[kk * 2 + half] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
          uint4 u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[6], p[7]));
          pf[kk * 2 + half] = as_bf16x8(u);
        }
      }
      if constexpr (NKB == 2) return (ps[0] + ps[1]) + (ps[2] + ps[3]);
      else return ps[0] + ps[1];
    };
    // The tile max moves the reference max m_run (and rescales O and l)
    // only when some query's tile max exceeds it by more than 8, so every
    // p = 2^(s - m_run) <= 2^8; the first tile always sets it.  Numerator and
    // denominator share m_run, so the final O / l is unchanged.
    auto rescale_by_max = [&]() {
      // tile max of this lane's logits: maxima of groups of three
      // (v_max3_f32), then of the group maxima
      auto sv = [&](int f) { return s[f >> 4][f & 15]; };
      float mt;
      if constexpr (NKB == 2) {
        float g3[11];
#pragma unroll
        for (int i = 0; i < 10; ++i) g3[i] = fmaxf(fmaxf(sv(3 * i), sv(3 * i + 1)), sv(3 * i + 2));
        g3[10] = fmaxf(sv(30), sv(31));
        const float u0 = fmaxf(fmaxf(g3[0], g3[1]), g3[2]), u1 = fmaxf(fmaxf(g3[3], g3[4]), g3[5]);
        const float u2 = fmaxf(fmaxf(g3[6], g3[7]), g3[8]), u3 = fmaxf(g3[9], g3[10]);
        mt = fmaxf(fmaxf(fmaxf(u0, u1), u2), u3);
      } else {
        float g3[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) g3[i] = fmaxf(fmaxf(sv(3 * i), sv(3 * i + 1)), sv(3 * i + 2));
        mt = fmaxf(fmaxf(fmaxf(g3[0], g3[1]), g3[2]), fmaxf(fmaxf(g3[3], g3[4]), sv(15)));
      }
      mt = half_swap_max(mt);
      if (first || __builtin_amdgcn_ballot_w64(mt > 8.0f)) {
        const float shift = first ? mt : fmaxf(mt, 0.f);
        const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-shift);
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          o[0][e] *= alpha;
          o[1][e] *= alpha;
        }
        m_run += shift;
        set_mneg(m_run);
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[kk][e] -= shift;
      }
    };
    // After the first tile, probabilities first, against the current m_run:
    // the tile max is only needed when some p may exceed 2^8, and a lane's
    // sum of its p exceeding 2^8 is necessary for that (rare once m_run has
    // settled).  Such a tile is recomputed from the K tile still in LDS, with
    // the max-based rescale above; as the rescale decision is the max test
    // either way, the results do not depend on which path ran.
    logits(true);
    float lsum = first ? 0.f : probs();
    if (first || __builtin_amdgcn_ballot_w64(lsum > 256.0f)) {
      // read K again rather than keep s or the K fragments in registers
      // through the fast path (the clobber stops the compiler reusing them)
      asm volatile("" ::: "memory");
      logits(false);
      rescale_by_max();
      lsum = probs();
    }
    l_run += lsum;
    // O^T[d, q] += V^T[d, keys] P^T[keys, q]; d = db*32 + row of the MFMA
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 2 * NKB; ++j) o[db] = mfma32x32x16(vf[db][j], pf[j], o[db]);
  };
  // The K / V^T pipeline after the work on tile i: refill the stage read in
  // the previous step (every wave passed the barrier after it), then wait for
  // this wave's part of tile i + 1 and publish it; the barrier also retires
  // this step's stage.
  auto advance = [&](int i) __attribute__((always_inline)) {
    if (i + 1 < nt) {
      if (i + S - 1 < nt) issue(i + S - 1, (i + S - 1) % S);
      wait_tiles(min(S - 2, nt - 2 - i));
      barrier_keep_loads();
      if ((i + 2) * KT > N) {
        fix_last(i + 1, (i + 1) % S);
        __syncthreads();
      }
    }
  };
  auto priority = [&](int i) __attribute__((always_inline)) {
    if (4 * i >= nt && 4 * (i - 1) < nt) __builtin_amdgcn_s_setprio(2);
    if (2 * i >= nt && 2 * (i - 1) < nt) __builtin_amdgcn_s_setprio(1);
    if (4 * i >= 3 * nt && 4 * (i - 1) < 3 * nt) __builtin_amdgcn_s_setprio(0);
  };
  // A split wave has keys at all only if its first key half starts before N
  // (only the last tile is ragged).
  const bool split_busy = split && par < nt && par * KT + kb_own * 32 < N;

  if (split) {  // workgroup-uniform
    for (int i = 0; i < nt; ++i) {
      priority(i);
      if ((i & 1) == par && i * KT + kb_own * 32 < N)
        compute(std::integral_constant<int, 1>{}, i, i % S, kb_own, i == par);
      advance(i);
    }
  } else {
    // One key tile; the first is peeled off the loop (the tile max always
    // sets m_run there).  Waves whose 32 query rows all lie past N
    // (wave-uniform) only load and sync.
    auto step = [&](int i, auto first_c) __attribute__((always_inline)) {
      priority(i);
      if (!idle) compute(std::integral_constant<int, 2>{}, i, i % S, 0, decltype(first_c)::value);
      advance(i);
    };
    step(0, std::true_type{});
    for (int i = 1; i < nt; ++i) step(i, std::false_type{});
  }

  if (split) {
    // Merge the NW partial results (each relative to its own m_run) into wave
    // 0 through LDS, in wave order: O = sum_w 2^(m_w - M) O_w, l likewise,
    // M = max_w m_w over the waves that saw keys (wave 0 always does).
    constexpr int F = 34;  // floats per lane: m, l, O^T (2 x 16)
    static_assert(NW * F * 64 * 4 <= (int)sizeof(KV), "merge buffer");
    float* mb = reinterpret_cast<float*>(&KV[0][0][0]);
    __syncthreads();  // every wave is done reading the last K / V^T stage
    float* mine = mb + wave * F * 64 + lane;
    mine[0] = split_busy ? m_run : -INFINITY;
    mine[64] = l_run;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) mine[(2 + db * 16 + e) * 64] = o[db][e];
    __syncthreads();
    if (wave != 0) return;
    float mw[NW], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = mb[w * F * 64 + lane];
      M = fmaxf(M, mw[w]);
    }
    l_run = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[0][e] = o[1][e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* src = mb + w * F * 64 + lane;
      const float sc = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
      l_run += sc * src[64];
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] += sc * src[(2 + db * 16 + e) * 64];
    }
  }

  const float l = half_swap_sum(l_run);
  const float inv = 1.0f / l;
  if (qrow < N) {
    bf16_t* op = a.O + ((size_t)b * N + qrow) * (size_t)(H * 64) + h * 64;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = db * 32 + i * 8 + lhalf * 4;
        uint2 u = make_uint2(pack_bf16x2(o[db][i * 4 + 0] * inv, o[db][i * 4 + 1] * inv),
                             pack_bf16x2(o[db][i * 4 + 2] * inv, o[db][i * 4 + 3] * inv));
        *reinterpret_cast<uint2*>(op + d) = u;
      }
  }
}

}  // namespace

// Every query tile runs against the whole key range in one pass (a partly
// filled last tile included: with 33..127 queries its idle waves only take
// part in the loads and barriers, with 1..32 its waves split the keys and
// merge in LDS), so no workspace is needed.
hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int batch, int tokens,
                            int heads, int nv, uint16_t* o, const void* prefetch, size_t prefetch_bytes,
                            hipStream_t s) {
  if (batch <= 0 || tokens <= 0 || heads <= 0 || nv < tokens || nv % 64 != 0) return hipErrorInvalidValue;
  if ((size_t)nv * 128 >= (1ull << 32)) return hipErrorInvalidValue;
  if (prefetch != nullptr && (reinterpret_cast<uintptr_t>(prefetch) % 16 != 0 || prefetch_bytes >= (1ull << 32)))
    return hipErrorInvalidValue;
  const int qtiles = (tokens + QT - 1) / QT;
  const int rem = tokens % QT;
  const int n_attn = qtiles * heads * batch;
  // About 32 chunks of 16 bytes per prefetching lane, at most 64 workgroups.
  // They run beside the attention workgroups only if the whole grid is
  // resident at once (three workgroups per CU); otherwise they would wait for
  // a free slot and lengthen the launch.
  constexpr int kResident = 3 * kComputeUnits;
  const uint32_t chunks = prefetch ? (uint32_t)(prefetch_bytes / 16) : 0u;
  int n_pf = chunks ? (int)std::min<uint32_t>(64u, (chunks + 256u * 32u - 1) / (256u * 32u)) : 0;
  if (n_attn + n_pf > kResident) n_pf = 0;
  AttnArgs a{q, k, vt, o, tokens, heads, nv, qtiles, batch, rem > 0 && rem <= 32 ? 1 : 0,
             n_attn, static_cast<const uint4*>(prefetch), chunks};
  hipLaunchKernelGGL((attention_kernel<4>), dim3(n_attn + n_pf), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace vit
