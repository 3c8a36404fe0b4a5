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
// rescales of the output accumulators.
// K and V^T tiles of 64 keys are staged in LDS (double-buffered, 16-byte
// chunks XOR-swizzled by row) and shared by the 4 waves of a workgroup; rows
// past the sequence end are read as zeros through buffer range checks.
#include "common.h"
#include "kernels.h"

namespace vit {
namespace {

constexpr int QT = 128;  // queries per workgroup (4 waves x 32)
constexpr int KT = 64;   // keys per tile

// Inverse of the token permutation used by vt (an involution).
__device__ __forceinline__ int vt_tok(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// LDS position of 16-byte chunk c of row r: the 16 rows read by 16 lanes of one
// ds_read_b128 cover all 64 banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

__global__ __launch_bounds__(256) void attention_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                                        const bf16_t* __restrict__ Vt, bf16_t* __restrict__ O,
                                                        int N, int H, int nv) {
  __shared__ uint4 Ks[2][KT * 8];
  __shared__ uint4 Vs[2][64 * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * H + h;
  const bf16_t* Qp = Q + bh * N * 64;
  const bf16_t* Kp = K + bh * N * 64;
  const bf16_t* Vp = Vt + bh * 64 * nv;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int qrow = blockIdx.x * QT + wave * 32 + lrow;

  // rows past N read as zeros through the buffer range checks
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qp, (uint32_t)N * 128u);
  const __amdgpu_buffer_rsrc_t rk_src = make_rsrc(Kp, (uint32_t)N * 128u);
  const __amdgpu_buffer_rsrc_t rv_src = make_rsrc(Vp, (uint32_t)nv * 128u);
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(buf_load16(rq, (uint32_t)qrow * 128u + ks * 32 + lhalf * 16));

  // cooperative tile loads: 512 chunks of K and 512 of V^T, 2 + 2 per thread
  int k_row[2], k_q[2], k_dst[2], v_row[2], v_q[2], v_dst[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int cid = tid + c * 256;
    k_row[c] = cid >> 3;
    k_q[c] = cid & 7;
    k_dst[c] = k_row[c] * 8 + swz(k_row[c], k_q[c]);
    v_row[c] = cid >> 3;  // channel d
    v_q[c] = cid & 7;     // 8 stored token positions
    v_dst[c] = v_row[c] * 8 + swz(v_row[c], v_q[c]);
  }
  auto load_tile = [&](int t, uint4* rk, uint4* rv) {
    const int k0 = t * KT;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      rk[c] = buf_load16(rk_src, (uint32_t)(k0 + k_row[c]) * 128u + k_q[c] * 16);
      const int p0 = k0 + v_q[c] * 8;  // < nv: nv is a multiple of 64
      uint4 u = buf_load16(rv_src, ((uint32_t)v_row[c] * nv + p0) * 2u);
      if (k0 + KT > N) {  // last tile: zero the positions of keys >= N
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (vt_tok(p0 + e) >= N) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        u = make_uint4(w[0], w[1], w[2], w[3]);
      }
      rv[c] = u;
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[0][e] = o[1][e] = 0.f;

  const int ntiles = (N + KT - 1) / KT;
  uint4 rk[2], rv[2];
  load_tile(0, rk, rv);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    Ks[0][k_dst[c]] = rk[c];
    Vs[0][v_dst[c]] = rv[c];
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1, rk, rv);

    // S^T for keys t*64 + kb*32 + [0, 32): element e <-> key 8*(e/4) + 4*lhalf + e%4
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
      const int r = kb * 32 + lrow;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int qd = ks * 2 + lhalf;
        s[kb] = mfma32x32x16(as_bf16x8(Ks[cur][r * 8 + swz(r, qd)]), qf[ks], s[kb]);
      }
    }
    if ((t + 1) * KT > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = t * KT + kb * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
          if (key >= N) s[kb][e] = -INFINITY;
        }
    }
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = (kb == 0); e < 16; ++e) mt = fmaxf(mt, s[kb][e]);
    mt = half_swap_max(mt);
    // Lazy rescaling: the reference max m_run only moves (and O, l are only
    // rescaled) when some query's tile max exceeds it by more than 8, so
    // p = exp2(s - m_run) <= 2^8.  Tile 0 always moves it (m_run = -inf, and
    // tile 0 holds key 0).  Numerator and denominator share m_run, so the
    // final O / l is unchanged.
    const bool grow = mt > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        o[0][e] *= alpha;
        o[1][e] *= alpha;
      }
    }
    const float m_use = m_run;
    // probabilities, packed as the B operand of the 4 key steps of P V
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(s[kb][half * 8 + e] - m_use);
          l_run += p[e];
        }
        uint4 u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                             pack_bf16x2(p[6], p[7]));
        pf[kb * 2 + half] = as_bf16x8(u);
      }
    }
    // O^T[d, q] += V^T[d, keys] P^T[keys, q]; d = db*32 + row of the MFMA
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int r = db * 32 + lrow;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int qd = ks * 2 + lhalf;
        o[db] = mfma32x32x16(as_bf16x8(Vs[cur][r * 8 + swz(r, qd)]), pf[ks], o[db]);
      }
    }

    if (t + 1 < ntiles) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Ks[cur ^ 1][k_dst[c]] = rk[c];
        Vs[cur ^ 1][v_dst[c]] = rv[c];
      }
    }
    __syncthreads();
  }

  const float l = half_swap_sum(l_run);
  const float inv = 1.0f / l;
  if (qrow < N) {
    bf16_t* op = O + ((size_t)b * N + qrow) * (size_t)(H * 64) + h * 64;
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

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int batch, int tokens,
                            int heads, int nv, uint16_t* o, hipStream_t s) {
  if (batch <= 0 || tokens <= 0 || heads <= 0 || nv < tokens || nv % 64 != 0) return hipErrorInvalidValue;
  if ((size_t)nv * 128 >= (1ull << 32)) return hipErrorInvalidValue;
  dim3 grid((tokens + QT - 1) / QT, heads, batch);
  hipLaunchKernelGGL(attention_kernel, grid, dim3(256), 0, s, q, k, vt, o, tokens, heads, nv);
  return hipGetLastError();
}

}  // namespace vit
