// Host runtime and C ABI of the semantic head on the encoder's taps: config
// validation, buffer planning, weight packing (fp32 blob -> bf16 GEMM
// operands with 3x3 kernels reordered to (ky, kx, c) columns, the column
// order of the implicit-GEMM convolution; fp32 vectors) and the launch
// sequence on the caller's stream.  Like the encoder, the head
// never allocates device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "host_error.h"
#include "kernels.h"
#include "vit_head.h"

namespace {

using vit::report_error;

int hip_fail(hipError_t e, const char* what) {
  return report_error(VIT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define HEAD_HIP(call, what)                          \
  do {                                                \
    hipError_t e_ = (call);                           \
    if (e_ != hipSuccess) return hip_fail(e_, what);  \
  } while (0)

constexpr size_t kAlign = 256;
constexpr int kBottlenecks = 3;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

uint16_t host_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct HeadPlan {
  vit_head_config cfg;
  int P = 0, T = 0, W = 0, H2 = 0, C = 0;   // pixels per image, concat width, width, half, classes
  size_t host_floats = 0;
  // weights (byte offsets)
  size_t proj_w, proj_g, proj_b, out_w, out_g, out_b, fin_g, fin_b, lat_w, lat_b, sm_w, sm_b, gn_g, gn_b, pred_w,
      pred_b, wtotal;
  size_t bn_w[kBottlenecks][2], bn_g[kBottlenecks][2], bn_b[kBottlenecks][2];
  // workspace (byte offsets)
  size_t x0, f, y, t, p4, lat, g, grid, stotal;
};

int validate(const vit_head_config* c) {
  if (!c) return report_error(VIT_ERR_ARG, "vit_head_config is NULL");
  if (c->grid_h < 1 || c->grid_w < 1 || (long)c->grid_h * c->grid_w > (1L << 20))
    return report_error(VIT_ERR_SHAPE, "grid must be at least 1 x 1 and at most 2^20 pixels");
  if (c->dim < 64 || c->dim % 64) return report_error(VIT_ERR_UNSUPPORTED, "dim must be a positive multiple of 64");
  if (c->taps < 1 || c->taps > 16) return report_error(VIT_ERR_ARG, "taps must be in [1, 16]");
  if (c->width != 256)
    return report_error(VIT_ERR_UNSUPPORTED, "width must be 256 (the diagram's projector width at every size)");
  if (c->groups < 1 || c->width != 8 * c->groups) return report_error(VIT_ERR_UNSUPPORTED, "width must equal 8 * groups");
  if (c->classes < 1 || c->classes > 1024) return report_error(VIT_ERR_ARG, "classes must be in [1, 1024]");
  if (c->out_h < 1 || c->out_w < 1 || c->out_h > 65535 || c->out_w > 65535)
    return report_error(VIT_ERR_ARG, "out_h and out_w must be in [1, 65535]");
  if (c->max_batch < 1 || c->max_batch > 4096) return report_error(VIT_ERR_ARG, "max_batch must be in [1, 4096]");
  if ((long)c->max_batch * c->grid_h * c->grid_w * 9 * c->width > (1L << 31))
    return report_error(VIT_ERR_SIZE, "batch x grid too large");
  if (!(c->ln_eps > 0.f) || !std::isfinite(c->ln_eps) || !(c->gn_eps > 0.f) || !std::isfinite(c->gn_eps))
    return report_error(VIT_ERR_ARG, "epsilons must be positive");
  return VIT_OK;
}

int build_plan(const vit_head_config* c, HeadPlan& pl) {
  int r = validate(c);
  if (r) return r;
  pl.cfg = *c;
  pl.P = c->grid_h * c->grid_w;
  pl.T = c->taps * c->dim;
  pl.W = c->width;
  pl.H2 = c->width / 2;
  pl.C = c->classes;
  const size_t W = pl.W, H2 = pl.H2, T = pl.T, C = pl.C;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  pl.proj_w = take(W * T * 2);
  pl.proj_g = take(W * 4);
  pl.proj_b = take(W * 4);
  for (int i = 0; i < kBottlenecks; ++i)
    for (int j = 0; j < 2; ++j) {
      pl.bn_w[i][j] = take(H2 * 9 * H2 * 2);
      pl.bn_g[i][j] = take(H2 * 4);
      pl.bn_b[i][j] = take(H2 * 4);
    }
  pl.out_w = take(W * 5 * H2 * 2);
  pl.out_g = take(W * 4);
  pl.out_b = take(W * 4);
  pl.fin_g = take(W * 4);
  pl.fin_b = take(W * 4);
  pl.lat_w = take(W * W * 2);
  pl.lat_b = take(W * 4);
  pl.sm_w = take(W * 9 * W * 2);
  pl.sm_b = take(W * 4);
  pl.gn_g = take(W * 4);
  pl.gn_b = take(W * 4);
  pl.pred_w = take(C * W * 2);
  pl.pred_b = take(C * 4);
  pl.wtotal = off;
  pl.host_floats = W * T + 2 * W + kBottlenecks * 2 * (H2 * H2 * 9 + 2 * H2) + W * 5 * H2 + 4 * W + W * W + W +
                   W * W * 9 + W + 2 * W + C * W + C;

  const size_t M = (size_t)c->max_batch * pl.P;
  off = 0;
  pl.x0 = take(M * T * 2);
  pl.f = take(M * W * 4);
  pl.y = take(M * 5 * H2 * 2);
  pl.t = take(M * H2 * 2);
  pl.p4 = take(M * W * 2);
  pl.lat = take(M * W * 2);
  pl.g = take(M * W * 2);
  pl.grid = take(M * C * 4);
  pl.stotal = off;
  return VIT_OK;
}

}  // namespace

struct vit_head {
  HeadPlan pl;
  char* w = nullptr;   // weights
  char* s = nullptr;   // workspace
};

extern "C" {

int vit_head_config_preset(vit_head_config* out) {
  if (!out) return report_error(VIT_ERR_ARG, "out is NULL");
  *out = vit_head_config{37, 37, 384, 4, 256, 32, 19, 518, 518, 8, 1e-6f, 1e-5f};
  return VIT_OK;
}

int vit_head_plan(const vit_head_config* cfg, vit_head_sizes* out) {
  if (!out) return report_error(VIT_ERR_ARG, "out is NULL");
  HeadPlan pl;
  int r = build_plan(cfg, pl);
  if (r) return r;
  out->weight_bytes = pl.wtotal;
  out->workspace_bytes = pl.stotal;
  out->host_floats = pl.host_floats;
  return VIT_OK;
}

int vit_head_create(const vit_head_config* cfg, const float* host_params, size_t host_floats, void* d_weights,
                    size_t weight_bytes, void* d_workspace, size_t workspace_bytes, void* stream, vit_head** out) {
  if (!out) return report_error(VIT_ERR_ARG, "out is NULL");
  *out = nullptr;
  HeadPlan pl;
  int r = build_plan(cfg, pl);
  if (r) return r;
  if (!host_params || !d_weights || !d_workspace) return report_error(VIT_ERR_ARG, "NULL parameter or buffer pointer");
  if (host_floats != pl.host_floats)
    return report_error(VIT_ERR_SIZE, "parameter blob has " + std::to_string(host_floats) + " floats, expected " +
                                          std::to_string(pl.host_floats));
  if (weight_bytes < pl.wtotal) return report_error(VIT_ERR_SIZE, "weight buffer smaller than vit_head_plan's weight_bytes");
  if (workspace_bytes < pl.stotal)
    return report_error(VIT_ERR_SIZE, "workspace smaller than vit_head_plan's workspace_bytes");
  if (((uintptr_t)d_weights | (uintptr_t)d_workspace) % kAlign)
    return report_error(VIT_ERR_ARG, "device buffers must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (vit::prepare_gemm() != hipSuccess) return report_error(VIT_ERR_HIP, "GEMM tables could not be set up");

  std::vector<unsigned char> stage(pl.wtotal, 0);
  const float* src = host_params;
  auto put_f32 = [&](size_t at, size_t n) {
    std::memcpy(stage.data() + at, src, n * 4);
    src += n;
  };
  auto put_bf16 = [&](size_t at, size_t n) {  // [out, in, 1, 1] = GEMM [N, K]
    uint16_t* d = reinterpret_cast<uint16_t*>(stage.data() + at);
    for (size_t i = 0; i < n; ++i) d[i] = host_bf16(src[i]);
    src += n;
  };
  auto put_conv3 = [&](size_t at, size_t co, size_t ci) {  // [co, ci, 3, 3] -> [co, (ky, kx, ci)]
    uint16_t* d = reinterpret_cast<uint16_t*>(stage.data() + at);
    for (size_t o = 0; o < co; ++o)
      for (size_t c = 0; c < ci; ++c)
        for (size_t k = 0; k < 9; ++k) d[o * 9 * ci + k * ci + c] = host_bf16(src[(o * ci + c) * 9 + k]);
    src += co * ci * 9;
  };
  const size_t W = pl.W, H2 = pl.H2, T = pl.T, C = pl.C;
  put_bf16(pl.proj_w, W * T);
  put_f32(pl.proj_g, W);
  put_f32(pl.proj_b, W);
  for (int i = 0; i < kBottlenecks; ++i)
    for (int j = 0; j < 2; ++j) {
      put_conv3(pl.bn_w[i][j], H2, H2);
      put_f32(pl.bn_g[i][j], H2);
      put_f32(pl.bn_b[i][j], H2);
    }
  put_bf16(pl.out_w, W * 5 * H2);
  put_f32(pl.out_g, W);
  put_f32(pl.out_b, W);
  put_f32(pl.fin_g, W);
  put_f32(pl.fin_b, W);
  put_bf16(pl.lat_w, W * W);
  put_f32(pl.lat_b, W);
  put_conv3(pl.sm_w, W, W);
  put_f32(pl.sm_b, W);
  put_f32(pl.gn_g, W);
  put_f32(pl.gn_b, W);
  put_bf16(pl.pred_w, C * W);
  put_f32(pl.pred_b, C);
  if ((size_t)(src - host_params) != pl.host_floats) return report_error(VIT_ERR_ARG, "internal: blob walk mismatch");

  auto* h = new (std::nothrow) vit_head();
  if (!h) return report_error(VIT_ERR_ARG, "out of host memory");
  h->pl = pl;
  h->w = (char*)d_weights;
  h->s = (char*)d_workspace;
  hipError_t e = hipMemcpyAsync(d_weights, stage.data(), pl.wtotal, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "head weight upload");
  }
  *out = h;
  return VIT_OK;
}

int vit_head_forward(vit_head* h, const float* d_taps, int batch, float* d_logits, float* d_grid, void* stream) {
  if (!h || !d_taps || !d_logits) return report_error(VIT_ERR_ARG, "NULL head, taps or logits pointer");
  const HeadPlan& pl = h->pl;
  const vit_head_config& c = pl.cfg;
  if (batch < 1 || batch > c.max_batch) return report_error(VIT_ERR_SIZE, "batch must be in [1, max_batch]");
  if ((uintptr_t)d_taps % 16) return report_error(VIT_ERR_ARG, "taps must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const int M = batch * pl.P, W = pl.W, H2 = pl.H2, T = pl.T, C = pl.C, ldy = 5 * H2;
  char* w = h->w;
  char* s = h->s;
  auto bf = [](char* p, size_t at) { return reinterpret_cast<uint16_t*>(p + at); };
  auto f32 = [](char* p, size_t at) { return reinterpret_cast<float*>(p + at); };
  uint16_t *x0 = bf(s, pl.x0), *y = bf(s, pl.y), *t = bf(s, pl.t), *p4 = bf(s, pl.p4), *lat = bf(s, pl.lat),
           *g = bf(s, pl.g);
  float *f = f32(s, pl.f), *grid = f32(s, pl.grid);
  auto f32_out = [&](const float* bias, float* outp, int N) {
    vit::EpiParams ep;
    ep.kind = vit::EPI_BIAS_F32;
    ep.bias = bias;
    ep.out = outp;
    ep.ldc = N;
    return ep;
  };
  auto gemm_f32 = [&](const uint16_t* a, size_t wo, int N, int K, const float* bias, float* outp) {
    return vit::launch_gemm(a, bf(w, wo), M, N, K, f32_out(bias, outp, N), st);
  };

  // ConvX blocks (conv, channel LayerNorm, SiLU; the output block adds the
  // final LayerNorm): the GEMM epilogue normalises whole pixel rows and writes
  // bf16 at column c0 of a row of width ld
  auto convx = [&](size_t g_at, size_t b_at, uint16_t* outp, int ld, int c0, const float* g2 = nullptr,
                   const float* b2 = nullptr) {
    vit::EpiParams ep;
    ep.kind = vit::EPI_CHAN_LN;
    ep.ln_g = f32(w, g_at);
    ep.ln_b = f32(w, b_at);
    ep.eps = c.ln_eps;
    ep.silu = true;
    ep.ln2_g = g2;
    ep.ln2_b = b2;
    ep.out = outp;
    ep.ldc = ld;
    ep.c0 = c0;
    return ep;
  };
  auto conv3x = [&](const uint16_t* in, int ld_in, int c0_in, size_t wo, const vit::EpiParams& ep) {
    return vit::launch_gemm_conv3(in, ld_in, c0_in, H2, batch, c.grid_h, c.grid_w, bf(w, wo), H2, ep, st);
  };

  // Projector P4
  HEAD_HIP(vit::launch_taps_cl(d_taps, batch, c.taps, c.dim, pl.P, x0, st), "taps to channels-last");
  HEAD_HIP(vit::launch_gemm(x0, bf(w, pl.proj_w), M, W, T, convx(pl.proj_g, pl.proj_b, y, ldy, 0), st),
           "projector conv");
  for (int i = 0; i < kBottlenecks; ++i) {
    // input: b (channels H2 .. 2 H2) for the first, then the previous output
    HEAD_HIP(conv3x(y, ldy, H2 * (i + 1), pl.bn_w[i][0], convx(pl.bn_g[i][0], pl.bn_b[i][0], t, H2, 0)),
             "bottleneck conv 1");
    HEAD_HIP(conv3x(t, H2, 0, pl.bn_w[i][1], convx(pl.bn_g[i][1], pl.bn_b[i][1], y, ldy, H2 * (i + 2))),
             "bottleneck conv 2");
  }
  HEAD_HIP(vit::launch_gemm(y, bf(w, pl.out_w), M, W, ldy,
                            convx(pl.out_g, pl.out_b, p4, W, 0, f32(w, pl.fin_g), f32(w, pl.fin_b)), st),
           "projector output conv");
  // Task head
  {
    vit::EpiParams ep;
    ep.kind = vit::EPI_BIAS_BF16;
    ep.bias = f32(w, pl.lat_b);
    ep.out = lat;
    ep.ldc = W;
    HEAD_HIP(vit::launch_gemm(p4, bf(w, pl.lat_w), M, W, W, ep, st), "lateral conv");
  }
  {
    // written group-major (8 channels x all pixels per group), the layout the
    // GroupNorm reads as one contiguous run per (group, image)
    vit::EpiParams ep = f32_out(f32(w, pl.sm_b), f, 8 * M);
    ep.kind = vit::EPI_BIAS_F32_G8;
    HEAD_HIP(vit::launch_gemm_conv3(lat, W, 0, W, batch, c.grid_h, c.grid_w, bf(w, pl.sm_w), W, ep, st),
             "smoothing conv");
  }
  HEAD_HIP(vit::launch_groupnorm_gelu(f, (size_t)8 * M, batch, pl.P, W, c.groups, f32(w, pl.gn_g), f32(w, pl.gn_b),
                                      c.gn_eps, g, st),
           "GroupNorm + GELU");
  HEAD_HIP(gemm_f32(g, pl.pred_w, C, W, f32(w, pl.pred_b), grid), "predict conv");
  HEAD_HIP(vit::launch_resize_nchw(grid, C, C, batch, c.grid_h, c.grid_w, d_logits, c.out_h, c.out_w, st),
           "logit resize");
  if (d_grid)
    HEAD_HIP(vit::launch_resize_nchw(grid, C, C, batch, c.grid_h, c.grid_w, d_grid, c.grid_h, c.grid_w, st),
             "grid logits");
  return VIT_OK;
}

int vit_head_destroy(vit_head* h) {
  delete h;
  return VIT_OK;
}

int vit_op_conv3x3(const void* in, int ld_in, int c0, int cin, int batch, int gh, int gw, const void* w,
                   const float* bias, int n_out, float* out, void* stream) {
  if (!in || !w || !out) return report_error(VIT_ERR_ARG, "NULL pointer");
  if (cin < 64 || cin % 64 || c0 < 0 || c0 % 8 || ld_in % 8 || c0 + cin > ld_in)
    return report_error(VIT_ERR_SHAPE, "cin a positive multiple of 64, c0 and ld_in multiples of 8, c0 + cin <= ld_in");
  if (batch < 1 || gh < 1 || gw < 1 || n_out < 1) return report_error(VIT_ERR_SHAPE, "batch, grid and n_out must be >= 1");
  if ((uintptr_t)in % 16) return report_error(VIT_ERR_ARG, "in must be 16-byte aligned");
  vit::EpiParams ep;
  ep.kind = vit::EPI_BIAS_F32;
  ep.bias = bias;
  ep.out = out;
  ep.ldc = n_out;
  HEAD_HIP(vit::launch_gemm_conv3((const uint16_t*)in, ld_in, c0, cin, batch, gh, gw, (const uint16_t*)w, n_out, ep,
                                  (hipStream_t)stream),
           "conv3x3");
  return VIT_OK;
}

int vit_op_convx(const void* in, int ld_in, int c0, int cin, int batch, int gh, int gw, int ksize, const void* w,
                 int n_out, const float* g, const float* b, const float* g2, const float* b2, float eps, void* out,
                 int ld_out, int c0_out, void* stream) {
  if (!in || !w || !g || !b || !out || (g2 && !b2)) return report_error(VIT_ERR_ARG, "NULL pointer");
  if (ksize != 1 && ksize != 3) return report_error(VIT_ERR_ARG, "ksize must be 1 or 3");
  if (!vit::chan_ln_fusable(n_out)) return report_error(VIT_ERR_UNSUPPORTED, "n_out must be 128 or 256");
  if (cin < 64 || cin % 64 || c0 < 0 || c0 % 8 || ld_in % 8 || c0 + cin > ld_in)
    return report_error(VIT_ERR_SHAPE, "cin a positive multiple of 64, c0 and ld_in multiples of 8, c0 + cin <= ld_in");
  if (ksize == 1 && (c0 != 0 || ld_in != cin)) return report_error(VIT_ERR_SHAPE, "ksize 1 reads whole rows: c0 = 0, ld_in = cin");
  if (batch < 1 || gh < 1 || gw < 1) return report_error(VIT_ERR_SHAPE, "batch and grid must be >= 1");
  if (ld_out % 4 || c0_out < 0 || c0_out % 4 || c0_out + n_out > ld_out)
    return report_error(VIT_ERR_SHAPE, "ld_out and c0_out multiples of 4, c0_out + n_out <= ld_out");
  if (!(eps > 0.f)) return report_error(VIT_ERR_ARG, "eps must be positive");
  if ((uintptr_t)in % 16 || (uintptr_t)out % 8 || ((uintptr_t)g | (uintptr_t)b | (uintptr_t)g2 | (uintptr_t)b2) % 16)
    return report_error(VIT_ERR_ARG, "in and the vectors must be 16-byte aligned, out 8-byte aligned");
  vit::EpiParams ep;
  ep.kind = vit::EPI_CHAN_LN;
  ep.ln_g = g;
  ep.ln_b = b;
  ep.eps = eps;
  ep.silu = true;
  ep.ln2_g = g2;
  ep.ln2_b = b2;
  ep.out = out;
  ep.ldc = ld_out;
  ep.c0 = c0_out;
  const int M = batch * gh * gw;
  hipError_t e = ksize == 3 ? vit::launch_gemm_conv3((const uint16_t*)in, ld_in, c0, cin, batch, gh, gw,
                                                     (const uint16_t*)w, n_out, ep, (hipStream_t)stream)
                            : vit::launch_gemm((const uint16_t*)in, (const uint16_t*)w, M, n_out, cin, ep,
                                               (hipStream_t)stream);
  HEAD_HIP(e, "convx");
  return VIT_OK;
}

}  // extern "C"
