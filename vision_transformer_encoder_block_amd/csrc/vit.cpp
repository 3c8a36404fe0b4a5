// Host runtime and C ABI of the ViT encoder library: configuration presets,
// buffer planning, weight packing (fp32 blob -> bf16 GEMM operands, fp32 vectors),
// the per-block launch sequence on the caller's stream, and the per-op entry
// points.  The library never allocates device memory: weights and workspace are
// caller-owned buffers carved into 256-byte-aligned regions.  The one exception
// is vit_forward_static, whose activations live in a file-scope device array
// of fixed size (for callers that cannot allocate).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "host_error.h"
#include "kernels.h"
#include "vit.h"
#include "vit_ops.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return VIT_ERR_HIP;
}

#define VIT_HIP(call, what)                 \
  do {                                      \
    hipError_t e_ = (call);                 \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr size_t kAlign = 256;
constexpr size_t kLastLevelCacheBytes = 256ull << 20;  // MI355X Infinity Cache
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int round_up(int x, int m) { return (x + m - 1) / m * m; }

uint16_t host_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

bool width_supported(int dim) {
  if (dim <= 0 || dim % 64) return false;
  const int v = dim / 64;
  return v <= 16 || v == 20 || v == 24 || v == 32 || v == 48 || v == 64;
}

// Window starts along one axis: ceil((n - side) / stride) + 1 windows every
// `stride` pixels, the last one moved back to end at the border.
std::vector<int> window_starts(int n, int side, int stride) {
  std::vector<int> out;
  const int count = (n > side ? (n - side + stride - 1) / stride : 0) + 1;
  for (int i = 0; i < count; ++i) {
    const int end = std::min(i * stride + side, n);
    out.push_back(std::max(end - side, 0));
  }
  return out;
}

struct Geom {
  int img_h = 0, img_w = 0, gh = 0, gw = 0, P = 0, N = 0, nv = 0;
  const float* pos = nullptr;
};

// Linear offsets (bytes) of the packed weight regions.
struct WeightLayout {
  size_t patch_w, patch_b, cls, reg, pos_native, pos_main, pos_win, norm_g, norm_b, total;
  struct Blk {
    size_t ln1_g, ln1_b, wqkv, bqkv, wo, bo, ls1, ln2_g, ln2_b, w1, b1, w2, b2, ls2;
  };
  std::vector<Blk> blocks;
};

struct WorkLayout {
  size_t x, h, q, k, vt, o, f, cols, crops, feats, clsb, cos, corners, total;
  int ldc_cos;
};

// Device pointers of the encoder's activations (one set of buffers per forward).
struct Acts {
  float* x = nullptr;                     // residual stream fp32 [rows, D]
  uint16_t* h = nullptr;                  // LayerNorm output bf16 [rows, D]
  uint16_t *q = nullptr, *k = nullptr;    // bf16 [images, heads, N, 64]
  uint16_t* vt = nullptr;                 // bf16 [images, heads, 64, nv]
  uint16_t* o = nullptr;                  // attention output bf16 [rows, D]
  uint16_t* f = nullptr;                  // MLP hidden bf16 [rows, Hm]
  uint16_t* cols = nullptr;               // im2col bf16 [patch rows, kpad]
};

struct Plan {
  vit_config cfg;
  int D, Hm, R, p, kpad, L, heads;
  Geom main, win;
  int nwin = 0;
  std::vector<int> corners;  // (y, x) pairs
  int ntaps = 0;
  size_t host_floats = 0;
  WeightLayout wl;
  WorkLayout ws;
};

// Offsets of the activation buffers for `rows` token rows, `vt_elems` V^T
// values and `prows` patch rows, from byte 0 of a region; returns the end.
size_t layout_acts(const Plan& pl, size_t rows, size_t vt_elems, size_t prows, WorkLayout& s) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t D = pl.D, Hm = pl.Hm;
  s.x = take(rows * D * 4);
  s.h = take(rows * D * 2);
  s.q = take(rows * D * 2);
  s.k = take(rows * D * 2);
  s.vt = take(vt_elems * 2);
  s.o = take(rows * D * 2);
  s.f = take(rows * Hm * 2);
  s.cols = take(prows * pl.kpad * 2);
  return off;
}

Acts acts_at(char* base, const WorkLayout& s) {
  Acts a;
  a.x = (float*)(base + s.x);
  a.h = (uint16_t*)(base + s.h);
  a.q = (uint16_t*)(base + s.q);
  a.k = (uint16_t*)(base + s.k);
  a.vt = (uint16_t*)(base + s.vt);
  a.o = (uint16_t*)(base + s.o);
  a.f = (uint16_t*)(base + s.f);
  a.cols = (uint16_t*)(base + s.cols);
  return a;
}

int make_geom(const Plan& pl, int img_h, int img_w, Geom& g) {
  g.img_h = img_h;
  g.img_w = img_w;
  g.gh = img_h / pl.p;
  g.gw = img_w / pl.p;
  g.P = g.gh * g.gw;
  g.N = g.P + 1 + pl.R;
  g.nv = round_up(g.N, 64);
  return VIT_OK;
}

int build_plan(const vit_config* c, Plan& pl) {
  if (!c) return fail(VIT_ERR_ARG, "vit_config is NULL");
  pl.cfg = *c;
  if (c->patch < 2 || c->patch > 32) return fail(VIT_ERR_ARG, "patch must be in [2, 32]");
  if (c->img_h <= 0 || c->img_w <= 0 || c->img_h % c->patch || c->img_w % c->patch)
    return fail(VIT_ERR_SHAPE, "image size must be a positive multiple of the patch size");
  if (c->dim <= 0 || !width_supported(c->dim))
    return fail(VIT_ERR_UNSUPPORTED, "dim must be 64 * {1..16, 20, 24, 32, 48, 64}");
  if (c->heads * 64 != c->dim) return fail(VIT_ERR_UNSUPPORTED, "heads must equal dim / 64 (64-channel heads)");
  if (c->mlp_hidden <= 0 || c->mlp_hidden % 64) return fail(VIT_ERR_UNSUPPORTED, "mlp_hidden must be a multiple of 64");
  if (c->depth < 0 || c->extra_blocks < 0 || c->depth + c->extra_blocks > 256)
    return fail(VIT_ERR_ARG, "depth and extra_blocks must be >= 0 (at most 256 blocks)");
  if (c->registers < 0 || c->registers > 16) return fail(VIT_ERR_ARG, "registers must be in [0, 16]");
  if (c->max_batch < 1 || c->max_batch > 4096) return fail(VIT_ERR_ARG, "max_batch must be in [1, 4096]");
  if (!(c->ln_eps > 0.f) || !std::isfinite(c->ln_eps)) return fail(VIT_ERR_ARG, "ln_eps must be positive");
  if (c->pos_grid_h < 1 || c->pos_grid_w < 1) return fail(VIT_ERR_ARG, "pos grid must be >= 1 x 1");
  if (c->max_classes < 0 || c->max_classes > 65536) return fail(VIT_ERR_ARG, "max_classes must be in [0, 65536]");
  const int L = c->depth + c->extra_blocks;
  if (L < 32 && (c->tap_mask >> L) != 0) return fail(VIT_ERR_ARG, "tap_mask selects a block beyond the last one");
  pl.D = c->dim;
  pl.Hm = c->mlp_hidden;
  pl.R = c->registers;
  pl.p = c->patch;
  pl.L = L;
  pl.heads = c->heads;
  pl.kpad = round_up(3 * c->patch * c->patch, 64);
  pl.ntaps = __builtin_popcount(c->tap_mask);
  make_geom(pl, c->img_h, c->img_w, pl.main);
  if ((long)pl.main.N * c->max_batch > (1L << 30) / c->dim) return fail(VIT_ERR_SIZE, "image batch too large");
  pl.nwin = 0;
  pl.corners.clear();
  if (c->window > 0) {
    if (c->window % c->patch || c->window > c->img_h || c->window > c->img_w || c->window_stride < 1)
      return fail(VIT_ERR_SHAPE, "window must be a multiple of patch, fit the image, and stride >= 1");
    // a stride longer than the window leaves pixels no window covers (their
    // overlap count would be 0)
    if (c->window_stride > c->window)
      return fail(VIT_ERR_SHAPE, "window_stride must not exceed window (every pixel needs a window)");
    make_geom(pl, c->window, c->window, pl.win);
    const auto ys = window_starts(c->img_h, c->window, c->window_stride);
    const auto xs = window_starts(c->img_w, c->window, c->window_stride);
    for (int y : ys)
      for (int x : xs) {
        pl.corners.push_back(y);
        pl.corners.push_back(x);
      }
    pl.nwin = (int)(ys.size() * xs.size());
    // coverage bound of the merge kernel (16 windows per pixel)
    auto cover = [&](const std::vector<int>& st, int n) {
      int mx = 0;
      for (int i = 0; i < n; ++i) {
        int k = 0;
        for (int s : st) k += (i >= s && i < s + c->window);
        mx = std::max(mx, k);
      }
      return mx;
    };
    if (cover(ys, c->img_h) * cover(xs, c->img_w) > 16) return fail(VIT_ERR_UNSUPPORTED, "more than 16 windows overlap");
  } else if (c->window < 0 || c->window_stride < 0) {
    return fail(VIT_ERR_ARG, "window and window_stride must be >= 0");
  }

  // host blob size
  const size_t D = pl.D, Hm = pl.Hm, R = pl.R, p = pl.p;
  const size_t npos = 1 + (size_t)c->pos_grid_h * c->pos_grid_w;
  const size_t per_block = 2 * D + 4 * (D * D + D) + D + 2 * D + (Hm * D + Hm) + (D * Hm + D) + D;
  pl.host_floats = D * 3 * p * p + D + D + R * D + npos * D + (size_t)L * per_block + 2 * D;

  // packed weights
  WeightLayout& w = pl.wl;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  w.patch_w = take(D * pl.kpad * 2);
  w.patch_b = take(D * 4);
  w.cls = take(D * 4);
  w.reg = take(std::max<size_t>(R, 1) * D * 4);
  w.pos_native = take(npos * D * 4);
  const bool main_native = c->pos_grid_h == pl.main.gh && c->pos_grid_w == pl.main.gw;
  w.pos_main = main_native ? w.pos_native : take((1 + (size_t)pl.main.P) * D * 4);
  w.pos_win = 0;
  if (pl.nwin) {
    const bool win_native = c->pos_grid_h == pl.win.gh && c->pos_grid_w == pl.win.gw;
    w.pos_win = win_native ? w.pos_native : take((1 + (size_t)pl.win.P) * D * 4);
  }
  w.blocks.resize(L);
  for (int l = 0; l < L; ++l) {
    auto& b = w.blocks[l];
    b.ln1_g = take(D * 4);
    b.ln1_b = take(D * 4);
    b.wqkv = take(3 * D * D * 2);
    b.bqkv = take(3 * D * 4);
    b.wo = take(D * D * 2);
    b.bo = take(D * 4);
    b.ls1 = take(D * 4);
    b.ln2_g = take(D * 4);
    b.ln2_b = take(D * 4);
    b.w1 = take(Hm * D * 2);
    b.b1 = take(Hm * 4);
    b.w2 = take(D * Hm * 2);
    b.b2 = take(D * 4);
    b.ls2 = take(D * 4);
  }
  w.norm_g = take(D * 4);
  w.norm_b = take(D * 4);
  w.total = off;

  // workspace
  WorkLayout& s = pl.ws;
  const size_t rows_main = (size_t)c->max_batch * pl.main.N;
  const size_t rows_win = (size_t)pl.nwin * (pl.nwin ? pl.win.N : 0);
  const size_t rows = std::max(rows_main, rows_win);
  const size_t vt_main = (size_t)c->max_batch * D * pl.main.nv;
  const size_t vt_win = pl.nwin ? (size_t)pl.nwin * D * pl.win.nv : 0;
  const size_t prow_main = (size_t)c->max_batch * pl.main.P;
  const size_t prow_win = pl.nwin ? (size_t)pl.nwin * pl.win.P : 0;
  const size_t prows = std::max(prow_main, prow_win);
  off = layout_acts(pl, rows, std::max(vt_main, vt_win), prows, s);
  s.ldc_cos = round_up(std::max(c->max_classes, 1), 4);
  if (c->max_classes > 0) {
    const size_t frows = std::max((size_t)pl.main.P, prow_win);
    s.crops = pl.nwin ? take((size_t)pl.nwin * 3 * c->window * c->window * 4) : 0;
    s.feats = take(frows * D * 2);
    s.clsb = take((size_t)c->max_classes * D * 2);
    s.cos = take(frows * s.ldc_cos * 4);
    s.corners = take(std::max<size_t>(pl.corners.size(), 2) * 4);
  } else {
    s.crops = s.feats = s.clsb = s.cos = s.corners = 0;
  }
  s.total = off;
  return VIT_OK;
}

struct BlockW {
  const float *ln1_g, *ln1_b;
  const uint16_t* wqkv;
  const float* bqkv;
  const uint16_t* wo;
  const float *bo, *ls1, *ln2_g, *ln2_b;
  const uint16_t* w1;
  const float* b1;
  const uint16_t* w2;
  const float *b2, *ls2;
};

}  // namespace

struct vit_model {
  Plan pl;
  int device = 0;        // the device holding the weights (current at vit_create)
  char* wbase = nullptr;
  char* sbase = nullptr;  // bound workspace, or NULL (then only vit_forward_static runs)
  const uint16_t* patch_w = nullptr;
  const float *patch_b = nullptr, *cls = nullptr, *reg = nullptr, *norm_g = nullptr, *norm_b = nullptr;
  std::vector<BlockW> blocks;
  Acts act;               // activations in the bound workspace
  float *crops = nullptr, *cos = nullptr;
  uint16_t *feats = nullptr, *clsb = nullptr;
  int* corners = nullptr;
};

// ------------------------------------------------------------------ static scratch
// The activations of vit_forward_static.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is taken once per
// device with hipGetSymbolAddress (that device current) and only that address
// is passed to kernels.
static constexpr size_t kScratchBytes = (size_t)VIT_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `dev`, which must be the current device;
// resolved on the first call for that device.
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(VIT_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    if (!p || (uintptr_t)p % kAlign) return fail(VIT_ERR_HIP, "static scratch address is not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VIT_OK;
}

// Patch embedding, blocks and the final step for `batch` images of geometry g.
// final_feats == false: final LayerNorm into tokens_out (fp32 [batch, N, D]);
// final_feats == true: LayerNorm + L2 of the patch rows into m->feats (bf16).
int run_encoder(vit_model* m, const Acts& a, const Geom& g, const float* images, int batch, float* tokens_out,
                float* taps, bool final_feats, hipStream_t st) {
  const Plan& pl = m->pl;
  const int D = pl.D, Hm = pl.Hm, N = g.N;
  const int M = batch * N;
  const float eps = pl.cfg.ln_eps;
  // im2col of the images, and the CLS and register rows of x (the patch GEMM writes the others)
  VIT_HIP(vit::launch_patchify(images, batch, g.img_h, g.img_w, pl.p, pl.kpad, a.cols, a.x, N, D, m->cls, g.pos,
                               m->reg, pl.R, st),
          "patchify");
  vit::EpiParams pe;
  pe.kind = vit::EPI_PATCH;
  pe.bias = m->patch_b;
  pe.pos = g.pos;
  pe.out = a.x;
  pe.ldc = D;
  pe.tokens = N;
  pe.patches = g.P;
  pe.regs = pl.R;
  VIT_HIP(vit::launch_gemm(a.cols, m->patch_w, batch * g.P, D, pl.kpad, pe, st), "patch embedding");
  int tap_i = 0;
  // For D = 384 the residual GEMMs also apply the LayerNorm that follows them
  // (out projection -> LN2, fc2 -> LN1 of the next block), so h arrives ready.
  const bool fuse_ln = vit::residual_ln_fusable(D);
  for (int l = 0; l < pl.L; ++l) {
    const BlockW& w = m->blocks[l];
    if (!fuse_ln || l == 0)
      VIT_HIP(vit::launch_layernorm(a.x, M, D, w.ln1_g, w.ln1_b, eps, a.h, false, st), "ln1");
    vit::EpiParams eq;
    eq.kind = vit::EPI_QKV;
    eq.bias = w.bqkv;
    eq.q = a.q;
    eq.k = a.k;
    eq.vt = a.vt;
    eq.tokens = N;
    eq.heads = pl.heads;
    eq.nv = g.nv;
    VIT_HIP(vit::launch_gemm(a.h, w.wqkv, M, 3 * D, D, eq, st), "qkv");
    // While attention runs (it needs little of the memory system), spare
    // workgroups of its launch read this block's remaining weights (out
    // projection, fc1, fc2) and the next block's Q/K/V weights, which lie
    // contiguous in the weight buffer.  Weights larger than the last-level
    // cache (256 MB on an MI355X) are evicted by the rest of a forward, so
    // each GEMM would otherwise fetch its weights from HBM at first use;
    // smaller models keep theirs cached and skip the extra reads.
    const void* pf = nullptr;
    size_t pf_bytes = 0;
    if (pl.wl.total > kLastLevelCacheBytes) {
      const char* pf_end = l + 1 < pl.L ? (const char*)(m->blocks[l + 1].wqkv + (size_t)3 * D * D)
                                        : (const char*)(w.w2 + (size_t)D * Hm);
      pf = w.wo;
      pf_bytes = (size_t)(pf_end - (const char*)w.wo);
    }
    VIT_HIP(vit::launch_attention(a.q, a.k, a.vt, batch, N, pl.heads, g.nv, a.o, pf, pf_bytes, st),
            "attention");
    vit::EpiParams eo;
    eo.kind = fuse_ln ? vit::EPI_RESIDUAL_LN : vit::EPI_RESIDUAL;
    eo.bias = w.bo;
    eo.ls = w.ls1;
    eo.out = a.x;
    eo.ldc = D;
    eo.ln_g = w.ln2_g;
    eo.ln_b = w.ln2_b;
    eo.eps = eps;
    eo.h = a.h;
    // The row-LayerNorm GEMMs run one 64-row tile per CU; on the CUs they leave
    // idle, extra workgroups read the weights of the GEMMs that follow (here
    // fc1 and fc2, contiguous), which the rest of a forward evicts from the
    // last-level cache between uses.
    eo.prefetch = w.w1;
    eo.prefetch_bytes = (size_t)((const char*)(w.w2 + (size_t)D * Hm) - (const char*)w.w1);
    VIT_HIP(vit::launch_gemm(a.o, w.wo, M, D, D, eo, st), "out projection");
    if (!fuse_ln) VIT_HIP(vit::launch_layernorm(a.x, M, D, w.ln2_g, w.ln2_b, eps, a.h, false, st), "ln2");
    vit::EpiParams e1;
    e1.kind = vit::EPI_GELU_BF16;
    e1.bias = w.b1;
    e1.out = a.f;
    e1.ldc = Hm;
    VIT_HIP(vit::launch_gemm(a.h, w.w1, M, Hm, D, e1, st), "fc1");
    vit::EpiParams e2;
    const bool fuse_next = fuse_ln && l + 1 < pl.L;
    e2.kind = fuse_next ? vit::EPI_RESIDUAL_LN : vit::EPI_RESIDUAL;
    e2.bias = w.b2;
    e2.ls = w.ls2;
    e2.out = a.x;
    e2.ldc = D;
    if (fuse_next) {
      e2.ln_g = m->blocks[l + 1].ln1_g;
      e2.ln_b = m->blocks[l + 1].ln1_b;
      e2.eps = eps;
      e2.h = a.h;
      // the next block's LN1 parameters, Q/K/V and out-projection weights
      const BlockW& nx = m->blocks[l + 1];
      e2.prefetch = nx.ln1_g;
      e2.prefetch_bytes = (size_t)((const char*)(nx.wo + (size_t)D * D) - (const char*)nx.ln1_g);
    }
    VIT_HIP(vit::launch_gemm(a.f, w.w2, M, D, Hm, e2, st), "fc2");
    if (taps && l < 32 && ((pl.cfg.tap_mask >> l) & 1u)) {
      const size_t per_img = (size_t)pl.ntaps * D * g.P;
      VIT_HIP(vit::launch_tap(a.x, batch, N, 1 + pl.R, g.P, D, m->norm_g, m->norm_b, eps,
                              taps + (size_t)tap_i * D * g.P, per_img, st),
              "tap");
      ++tap_i;
    }
  }
  if (final_feats) {
    VIT_HIP(vit::launch_ln_l2(a.x, batch, N, 1 + pl.R, g.P, D, m->norm_g, m->norm_b, eps, m->feats, st),
            "patch features");
  } else {
    VIT_HIP(vit::launch_layernorm(a.x, M, D, m->norm_g, m->norm_b, eps, tokens_out, true, st), "final norm");
  }
  return VIT_OK;
}

const vit_config kPresets[5] = {
    // img_h img_w p  dim depth extra heads Hm   R  maxb eps   taps  pos grid  win  stride classes
    {224, 224, 16, 384, 12, 0, 6, 1536, 4, 1, 1e-6f, 0u, 14, 14, 0, 0, 0},
    {336, 336, 16, 384, 12, 0, 6, 1536, 4, 32, 1e-6f, 0u, 21, 21, 0, 0, 0},
    {518, 518, 14, 384, 12, 0, 6, 1536, 0, 8, 1e-6f, (1u << 2) | (1u << 5) | (1u << 8) | (1u << 11), 37, 37, 0, 0, 0},
    {1024, 1024, 16, 1024, 24, 0, 16, 4096, 4, 4, 1e-6f, 0u, 64, 64, 0, 0, 0},
    {512, 1024, 16, 1024, 24, 2, 16, 4096, 4, 1, 1e-6f, 0u, 32, 64, 384, 192, 150},
};

}  // namespace

extern "C" {

const char* vit_last_error(void) { return g_err.c_str(); }

int vit_config_preset(int cfg_id, vit_config* out) {
  if (!out) return fail(VIT_ERR_ARG, "out is NULL");
  if (cfg_id < 1 || cfg_id > 5) return fail(VIT_ERR_ARG, "preset id must be 1..5");
  *out = kPresets[cfg_id - 1];
  return VIT_OK;
}

int vit_plan(const vit_config* cfg, vit_sizes* out) {
  if (!out) return fail(VIT_ERR_ARG, "out is NULL");
  Plan pl;
  const int r = build_plan(cfg, pl);
  if (r) return r;
  out->weight_bytes = pl.wl.total;
  out->workspace_bytes = pl.ws.total;
  out->host_floats = pl.host_floats;
  out->tokens = pl.main.N;
  out->window_tokens = pl.nwin ? pl.win.N : 0;
  out->windows = pl.nwin;
  out->taps = pl.ntaps;
  return VIT_OK;
}

int vit_create(const vit_config* cfg, const float* host_params, size_t host_floats, void* d_weights,
               size_t weight_bytes, void* d_workspace, size_t workspace_bytes, void* stream, vit_model** out) {
  if (!out) return fail(VIT_ERR_ARG, "out is NULL");
  *out = nullptr;
  Plan pl;
  int r = build_plan(cfg, pl);
  if (r) return r;
  if (!host_params || !d_weights) return fail(VIT_ERR_ARG, "NULL parameter or weight pointer");
  // no workspace (NULL, 0 bytes): only vit_forward_static, whose activations
  // live in the library's static array, can run on the model
  const bool bound = d_workspace != nullptr;
  if (!bound && workspace_bytes != 0) return fail(VIT_ERR_ARG, "NULL workspace with a nonzero size");
  if (host_floats != pl.host_floats)
    return fail(VIT_ERR_SIZE, "parameter blob has " + std::to_string(host_floats) + " floats, expected " +
                                  std::to_string(pl.host_floats));
  if (weight_bytes < pl.wl.total) return fail(VIT_ERR_SIZE, "weight buffer smaller than vit_plan's weight_bytes");
  if (bound && workspace_bytes < pl.ws.total)
    return fail(VIT_ERR_SIZE, "workspace smaller than vit_plan's workspace_bytes");
  if (((uintptr_t)d_weights | (uintptr_t)d_workspace) % kAlign)
    return fail(VIT_ERR_ARG, "device buffers must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (vit::prepare_gemm() != hipSuccess) return fail(VIT_ERR_HIP, "GEMM tables could not be set up");
  int device = 0;
  VIT_HIP(hipGetDevice(&device), "hipGetDevice");
  {  // the static scratch's address on this device, resolved once at set-up
    void* unused = nullptr;
    r = scratch_on(device, &unused);
    if (r) return r;
  }

  const size_t D = pl.D, Hm = pl.Hm, R = pl.R, p = pl.p;
  const WeightLayout& wl = pl.wl;
  std::vector<unsigned char> stage(wl.total, 0);
  const float* src = host_params;
  auto put_f32 = [&](size_t at, size_t n) {
    std::memcpy(stage.data() + at, src, n * 4);
    src += n;
  };
  auto put_bf16 = [&](size_t at, size_t n) {
    uint16_t* d = reinterpret_cast<uint16_t*>(stage.data() + at);
    for (size_t i = 0; i < n; ++i) d[i] = host_bf16(src[i]);
    src += n;
  };
  {  // patch weight rows padded to kpad columns
    const size_t kv = 3 * p * p;
    uint16_t* d = reinterpret_cast<uint16_t*>(stage.data() + wl.patch_w);
    for (size_t o = 0; o < D; ++o)
      for (size_t k = 0; k < kv; ++k) d[o * pl.kpad + k] = host_bf16(src[o * kv + k]);
    src += D * kv;
  }
  put_f32(wl.patch_b, D);
  put_f32(wl.cls, D);
  put_f32(wl.reg, R * D);
  put_f32(wl.pos_native, (1 + (size_t)pl.cfg.pos_grid_h * pl.cfg.pos_grid_w) * D);
  for (int l = 0; l < pl.L; ++l) {
    const auto& b = wl.blocks[l];
    put_f32(b.ln1_g, D);
    put_f32(b.ln1_b, D);
    put_bf16(b.wqkv, D * D);                   // wq
    put_f32(b.bqkv, D);                        // bq
    put_bf16(b.wqkv + D * D * 2, D * D);       // wk
    put_f32(b.bqkv + D * 4, D);                // bk
    put_bf16(b.wqkv + 2 * D * D * 2, D * D);   // wv
    put_f32(b.bqkv + 2 * D * 4, D);            // bv
    put_bf16(b.wo, D * D);
    put_f32(b.bo, D);
    put_f32(b.ls1, D);
    put_f32(b.ln2_g, D);
    put_f32(b.ln2_b, D);
    put_bf16(b.w1, Hm * D);
    put_f32(b.b1, Hm);
    put_bf16(b.w2, D * Hm);
    put_f32(b.b2, D);
    put_f32(b.ls2, D);
  }
  put_f32(wl.norm_g, D);
  put_f32(wl.norm_b, D);
  if ((size_t)(src - host_params) != pl.host_floats) return fail(VIT_ERR_ARG, "internal: blob walk mismatch");

  auto* m = new (std::nothrow) vit_model();
  if (!m) return fail(VIT_ERR_ARG, "out of host memory");
  m->pl = pl;
  m->device = device;
  m->wbase = (char*)d_weights;
  m->sbase = (char*)d_workspace;
  char* W = m->wbase;
  m->patch_w = (const uint16_t*)(W + wl.patch_w);
  m->patch_b = (const float*)(W + wl.patch_b);
  m->cls = (const float*)(W + wl.cls);
  m->reg = (const float*)(W + wl.reg);
  m->norm_g = (const float*)(W + wl.norm_g);
  m->norm_b = (const float*)(W + wl.norm_b);
  m->pl.main.pos = (const float*)(W + wl.pos_main);
  if (pl.nwin) m->pl.win.pos = (const float*)(W + wl.pos_win);
  m->blocks.resize(pl.L);
  for (int l = 0; l < pl.L; ++l) {
    const auto& b = wl.blocks[l];
    BlockW& w = m->blocks[l];
    w.ln1_g = (const float*)(W + b.ln1_g);
    w.ln1_b = (const float*)(W + b.ln1_b);
    w.wqkv = (const uint16_t*)(W + b.wqkv);
    w.bqkv = (const float*)(W + b.bqkv);
    w.wo = (const uint16_t*)(W + b.wo);
    w.bo = (const float*)(W + b.bo);
    w.ls1 = (const float*)(W + b.ls1);
    w.ln2_g = (const float*)(W + b.ln2_g);
    w.ln2_b = (const float*)(W + b.ln2_b);
    w.w1 = (const uint16_t*)(W + b.w1);
    w.b1 = (const float*)(W + b.b1);
    w.w2 = (const uint16_t*)(W + b.w2);
    w.b2 = (const float*)(W + b.b2);
    w.ls2 = (const float*)(W + b.ls2);
  }
  char* S = m->sbase;
  const WorkLayout& ws = pl.ws;
  if (bound) m->act = acts_at(S, ws);
  if (bound && pl.cfg.max_classes > 0) {
    m->crops = pl.nwin ? (float*)(S + ws.crops) : nullptr;
    m->feats = (uint16_t*)(S + ws.feats);
    m->clsb = (uint16_t*)(S + ws.clsb);
    m->cos = (float*)(S + ws.cos);
    m->corners = (int*)(S + ws.corners);
  }

  auto bail = [&](int code) {
    delete m;
    return code;
  };
  hipError_t e = hipMemcpyAsync(d_weights, stage.data(), wl.total, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return bail(hip_fail(e, "weight upload"));
  if (bound) {
    e = hipMemsetAsync(d_workspace, 0, pl.ws.total, st);
    if (e != hipSuccess) return bail(hip_fail(e, "workspace clear"));
  }
  const float* pos_native = (const float*)(W + wl.pos_native);
  if (wl.pos_main != wl.pos_native) {
    e = vit::launch_pos_resample(pos_native, pl.cfg.pos_grid_h, pl.cfg.pos_grid_w, (float*)(W + wl.pos_main),
                                 pl.main.gh, pl.main.gw, (int)D, st);
    if (e != hipSuccess) return bail(hip_fail(e, "position resampling"));
  }
  if (pl.nwin && wl.pos_win != wl.pos_native) {
    e = vit::launch_pos_resample(pos_native, pl.cfg.pos_grid_h, pl.cfg.pos_grid_w, (float*)(W + wl.pos_win),
                                 pl.win.gh, pl.win.gw, (int)D, st);
    if (e != hipSuccess) return bail(hip_fail(e, "position resampling"));
  }
  if (m->corners && !pl.corners.empty()) {
    e = hipMemcpyAsync(m->corners, pl.corners.data(), pl.corners.size() * 4, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return bail(hip_fail(e, "window corners upload"));
  }
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return bail(hip_fail(e, "create synchronisation"));
  *out = m;
  return VIT_OK;
}

int vit_forward(vit_model* m, const float* d_images, int batch, float* d_tokens, float* d_taps, void* stream) {
  if (!m || !d_images || !d_tokens) return fail(VIT_ERR_ARG, "NULL model, image or token pointer");
  if (batch < 1 || batch > m->pl.cfg.max_batch) return fail(VIT_ERR_SIZE, "batch must be in [1, max_batch]");
  if ((uintptr_t)d_tokens % 16) return fail(VIT_ERR_ARG, "d_tokens must be 16-byte aligned");
  if (!m->sbase) return fail(VIT_ERR_ARG, "model created without a workspace (use vit_forward_static)");
  return run_encoder(m, m->act, m->pl.main, d_images, batch, d_tokens, d_taps, false, (hipStream_t)stream);
}

int vit_forward_static(vit_model* m, const float* d_images, int batch, float* d_tokens, float* d_taps,
                       void* stream) {
  if (!m || !d_images || !d_tokens) return fail(VIT_ERR_ARG, "NULL model, image or token pointer");
  if (batch < 1 || batch > m->pl.cfg.max_batch) return fail(VIT_ERR_SIZE, "batch must be in [1, max_batch]");
  if ((uintptr_t)d_tokens % 16) return fail(VIT_ERR_ARG, "d_tokens must be 16-byte aligned");
  const Plan& pl = m->pl;
  WorkLayout s;
  const size_t need = layout_acts(pl, (size_t)batch * pl.main.N, (size_t)batch * pl.D * pl.main.nv,
                                  (size_t)batch * pl.main.P, s);
  if (need > kScratchBytes)
    return fail(VIT_ERR_SIZE, "batch " + std::to_string(batch) + " needs " + std::to_string(need) +
                                  " bytes of activations; the static scratch holds " + std::to_string(kScratchBytes));
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    base = m->device >= 0 && m->device < kMaxDevices ? g_scratch_ptr[m->device] : nullptr;
  }
  if (!base) return fail(VIT_ERR_HIP, "static scratch not resolved for the model's device");
  return run_encoder(m, acts_at((char*)base, s), pl.main, d_images, batch, d_tokens, d_taps, false,
                     (hipStream_t)stream);
}

int vit_descriptor(vit_model* m, const float* d_tokens, int batch, float* d_desc, void* stream) {
  if (!m || !d_tokens || !d_desc) return fail(VIT_ERR_ARG, "NULL model, token or descriptor pointer");
  if (batch < 1 || batch > m->pl.cfg.max_batch) return fail(VIT_ERR_SIZE, "batch must be in [1, max_batch]");
  const int D = m->pl.D;
  VIT_HIP(vit::launch_descriptor(d_tokens, batch, (size_t)m->pl.main.N * D, D, d_desc, (hipStream_t)stream),
          "descriptor");
  return VIT_OK;
}

int vit_patch_scores(vit_model* m, const float* d_image, const float* d_class_emb, int classes, int mode,
                     int* d_labels, float* d_cos, float* d_dense, void* stream) {
  if (!m || !d_image || !d_class_emb || !d_labels) return fail(VIT_ERR_ARG, "NULL model, image, class or label pointer");
  const Plan& pl = m->pl;
  if (pl.cfg.max_classes <= 0) return fail(VIT_ERR_UNSUPPORTED, "model created with max_classes = 0");
  if (classes < 1 || classes > pl.cfg.max_classes) return fail(VIT_ERR_SIZE, "classes must be in [1, max_classes]");
  if (mode != 0 && mode != 1) return fail(VIT_ERR_ARG, "mode must be 0 (whole) or 1 (slide)");
  if (mode == 1 && pl.nwin == 0) return fail(VIT_ERR_UNSUPPORTED, "model created without a slide window");
  if (!m->sbase) return fail(VIT_ERR_ARG, "model created without a workspace");
  hipStream_t st = (hipStream_t)stream;
  const int D = pl.D, H = pl.cfg.img_h, W = pl.cfg.img_w, ldc = pl.ws.ldc_cos;
  VIT_HIP(vit::launch_to_bf16(d_class_emb, (size_t)classes * D, m->clsb, st), "class embeddings");
  vit::EpiParams ec;
  ec.kind = vit::EPI_BIAS_F32;
  ec.out = m->cos;
  ec.ldc = ldc;
  if (mode == 0) {
    int r = run_encoder(m, m->act, pl.main, d_image, 1, nullptr, nullptr, true, st);
    if (r) return r;
    VIT_HIP(vit::launch_gemm(m->feats, m->clsb, pl.main.P, classes, D, ec, st), "scores");
    VIT_HIP(vit::launch_upsample_argmax(m->cos, pl.main.gh, pl.main.gw, classes, ldc, H, W, d_labels, d_dense, st),
            "upsample");
    if (d_cos) VIT_HIP(vit::launch_cos_out(m->cos, 1, pl.main.P, classes, ldc, d_cos, st), "scores out");
  } else {
    const int side = pl.cfg.window;
    VIT_HIP(vit::launch_crops(d_image, H, W, m->corners, pl.nwin, side, m->crops, st), "crops");
    int r = run_encoder(m, m->act, pl.win, m->crops, pl.nwin, nullptr, nullptr, true, st);
    if (r) return r;
    VIT_HIP(vit::launch_gemm(m->feats, m->clsb, pl.nwin * pl.win.P, classes, D, ec, st), "scores");
    VIT_HIP(vit::launch_slide_merge(m->cos, pl.nwin, m->corners, pl.win.gh, classes, ldc, side, H, W, d_labels, d_dense,
                                    st),
            "slide merge");
    if (d_cos) VIT_HIP(vit::launch_cos_out(m->cos, pl.nwin, pl.win.P, classes, ldc, d_cos, st), "scores out");
  }
  return VIT_OK;
}

int vit_destroy(vit_model* m) {
  delete m;
  return VIT_OK;
}

// ------------------------------------------------------------------ per-op entry points

int vit_op_linear_residual_ln(const void* a, const void* w, const float* bias, const float* ls, int M, int N, int K,
                              float* x, const float* g, const float* b, float eps, void* h, void* stream) {
  if (!a || !w || !bias || !ls || !x || !g || !b || !h) return fail(VIT_ERR_ARG, "NULL pointer");
  if (M < 1 || K < 64 || K % 64) return fail(VIT_ERR_SHAPE, "M >= 1 and K a positive multiple of 64");
  if (!vit::residual_ln_fusable(N)) return fail(VIT_ERR_UNSUPPORTED, "the fused residual + LayerNorm needs N = 384");
  if (!(eps > 0.f)) return fail(VIT_ERR_ARG, "eps must be positive");
  if (((uintptr_t)bias | (uintptr_t)ls | (uintptr_t)x | (uintptr_t)g | (uintptr_t)b) % 16 || (uintptr_t)h % 8)
    return fail(VIT_ERR_ARG, "vectors and x must be 16-byte aligned, h 8-byte aligned");
  vit::EpiParams ep;
  ep.kind = vit::EPI_RESIDUAL_LN;
  ep.bias = bias;
  ep.ls = ls;
  ep.out = x;
  ep.ldc = N;
  ep.ln_g = g;
  ep.ln_b = b;
  ep.eps = eps;
  ep.h = (uint16_t*)h;
  VIT_HIP(vit::launch_gemm((const uint16_t*)a, (const uint16_t*)w, M, N, K, ep, (hipStream_t)stream),
          "linear + residual + layernorm");
  return VIT_OK;
}

int vit_op_preprocess(const void* frames, int batch, int src_h, int src_w, int bgr, float* images, int dst_h,
                      int dst_w, void* stream) {
  if (!frames || !images) return fail(VIT_ERR_ARG, "NULL pointer");
  if (batch < 1 || src_h < 1 || src_w < 1 || dst_h < 1 || dst_w < 1 || batch > 65535 || dst_h > 65535)
    return fail(VIT_ERR_SHAPE, "sizes must be >= 1, batch and dst_h <= 65535");
  if ((size_t)src_h * src_w * 3 >= (1ull << 31) || (size_t)dst_h * dst_w >= (1ull << 31))
    return fail(VIT_ERR_SHAPE, "frame or image too large");
  VIT_HIP(vit::launch_preprocess((const uint8_t*)frames, batch, src_h, src_w, bgr != 0, images, dst_h, dst_w,
                                 (hipStream_t)stream),
          "preprocess");
  return VIT_OK;
}

int vit_op_layernorm(const float* x, int rows, int dim, const float* g, const float* b, float eps, void* y,
                     int out_fp32, void* stream) {
  if (!x || !g || !b || !y) return fail(VIT_ERR_ARG, "NULL pointer");
  if (rows < 1 || !width_supported(dim)) return fail(VIT_ERR_SHAPE, "rows >= 1 and a supported dim required");
  if (!(eps > 0.f)) return fail(VIT_ERR_ARG, "eps must be positive");
  VIT_HIP(vit::launch_layernorm(x, rows, dim, g, b, eps, y, out_fp32 != 0, (hipStream_t)stream), "layernorm");
  return VIT_OK;
}

int vit_op_linear(const void* a, const void* w, const float* bias, int M, int N, int K, int epilogue, const float* ls,
                  void* c, void* stream) {
  if (!a || !w || !c) return fail(VIT_ERR_ARG, "NULL pointer");
  if (M < 1 || N < 1 || K < 64 || K % 64) return fail(VIT_ERR_SHAPE, "M, N >= 1 and K a positive multiple of 64");
  if (epilogue < 0 || epilogue > VIT_EPI_BIAS_F32) return fail(VIT_ERR_ARG, "unknown epilogue");
  if (epilogue != VIT_EPI_BIAS_F32 && epilogue != VIT_EPI_BIAS_BF16 && !bias) return fail(VIT_ERR_ARG, "bias is NULL");
  if (epilogue == VIT_EPI_RESIDUAL && !ls) return fail(VIT_ERR_ARG, "ls is NULL");
  vit::EpiParams ep;
  ep.kind = epilogue;  // the public and internal codes coincide for these four
  ep.bias = bias;
  ep.ls = ls;
  ep.out = c;
  ep.ldc = N;
  VIT_HIP(vit::launch_gemm((const uint16_t*)a, (const uint16_t*)w, M, N, K, ep, (hipStream_t)stream), "linear");
  return VIT_OK;
}

int vit_op_absmax(const void* x, int x_bf16, size_t n, float* amax, void* stream) {
  if (!x || !amax) return fail(VIT_ERR_ARG, "NULL pointer");
  if (n == 0) return fail(VIT_ERR_SHAPE, "n must be >= 1");
  VIT_HIP(vit::launch_absmax(x, x_bf16 != 0, n, amax, (hipStream_t)stream), "absmax");
  return VIT_OK;
}

int vit_op_quantize_fp8(const void* x, int x_bf16, size_t n, float s_inv, void* out, void* stream) {
  if (!x || !out) return fail(VIT_ERR_ARG, "NULL pointer");
  if (n == 0) return fail(VIT_ERR_SHAPE, "n must be >= 1");
  if ((uintptr_t)out % 4) return fail(VIT_ERR_ARG, "out must be 4-byte aligned");
  if (!std::isfinite(s_inv)) return fail(VIT_ERR_ARG, "s_inv must be finite");
  VIT_HIP(vit::launch_quantize_fp8(x, x_bf16 != 0, n, s_inv, (uint8_t*)out, (hipStream_t)stream), "quantize fp8");
  return VIT_OK;
}

int vit_op_linear_fp8(const void* a, const void* w, int M, int N, int K, float scale, const float* bias, void* out,
                      int out_f32, void* stream) {
  if (!a || !w || !out) return fail(VIT_ERR_ARG, "NULL pointer");
  if (M < 1 || N < 1 || K < 128 || K % 128) return fail(VIT_ERR_SHAPE, "M, N >= 1 and K a positive multiple of 128");
  if (!std::isfinite(scale)) return fail(VIT_ERR_ARG, "scale must be finite");
  VIT_HIP(vit::launch_gemm_fp8((const uint8_t*)a, (const uint8_t*)w, M, N, K, scale, bias, out, N, out_f32 != 0,
                               (hipStream_t)stream),
          "linear fp8");
  return VIT_OK;
}

int vit_op_quantize_int8(const void* x, int x_bf16, size_t n, float s_inv, void* out, void* stream) {
  if (!x || !out) return fail(VIT_ERR_ARG, "NULL pointer");
  if (n == 0) return fail(VIT_ERR_SHAPE, "n must be >= 1");
  if ((uintptr_t)out % 4) return fail(VIT_ERR_ARG, "out must be 4-byte aligned");
  if (!std::isfinite(s_inv)) return fail(VIT_ERR_ARG, "s_inv must be finite");
  VIT_HIP(vit::launch_quantize_int8(x, x_bf16 != 0, n, s_inv, (int8_t*)out, (hipStream_t)stream), "quantize int8");
  return VIT_OK;
}

int vit_op_linear_int8(const void* a, const void* w, int M, int N, int K, float scale, const float* bias, void* out,
                       int out_f32, void* stream) {
  if (!a || !w || !out) return fail(VIT_ERR_ARG, "NULL pointer");
  if (M < 1 || N < 1 || K < 128 || K % 128 || K > 131072)
    return fail(VIT_ERR_SHAPE, "M, N >= 1 and K a multiple of 128 in [128, 131072]");
  if (!std::isfinite(scale)) return fail(VIT_ERR_ARG, "scale must be finite");
  VIT_HIP(vit::launch_gemm_int8((const int8_t*)a, (const int8_t*)w, M, N, K, scale, bias, out, N, out_f32 != 0,
                                (hipStream_t)stream),
          "linear int8");
  return VIT_OK;
}

int vit_op_qkv(const void* h, const void* wqkv, const float* bqkv, int batch, int tokens, int heads, void* q, void* k,
               void* vt, void* stream) {
  if (!h || !wqkv || !bqkv || !q || !k || !vt) return fail(VIT_ERR_ARG, "NULL pointer");
  if (batch < 1 || tokens < 1 || heads < 1 || heads > 64) return fail(VIT_ERR_SHAPE, "bad batch/tokens/heads");
  const int D = heads * 64;
  vit::EpiParams eq;
  eq.kind = vit::EPI_QKV;
  eq.bias = bqkv;
  eq.q = (uint16_t*)q;
  eq.k = (uint16_t*)k;
  eq.vt = (uint16_t*)vt;
  eq.tokens = tokens;
  eq.heads = heads;
  eq.nv = round_up(tokens, 64);
  VIT_HIP(vit::launch_gemm((const uint16_t*)h, (const uint16_t*)wqkv, batch * tokens, 3 * D, D, eq,
                           (hipStream_t)stream),
          "qkv");
  return VIT_OK;
}

int vit_op_attention(const void* q, const void* k, const void* vt, int batch, int tokens, int heads, void* o,
                     void* stream) {
  if (!q || !k || !vt || !o) return fail(VIT_ERR_ARG, "NULL pointer");
  if (batch < 1 || tokens < 1 || heads < 1 || heads > 64) return fail(VIT_ERR_SHAPE, "bad batch/tokens/heads");
  VIT_HIP(vit::launch_attention((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)vt, batch, tokens, heads,
                                round_up(tokens, 64), (uint16_t*)o, nullptr, 0, (hipStream_t)stream),
          "attention");
  return VIT_OK;
}

}  // extern "C"

namespace vit {
int report_error(int code, const std::string& msg) { return fail(code, msg); }
}  // namespace vit
