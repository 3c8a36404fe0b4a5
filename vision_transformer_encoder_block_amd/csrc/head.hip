// Kernels of the semantic head on the encoder's taps (LibreYOLO DINOv2
// diagram, "Projector P4", "Projector Bottleneck", "Projector output ConvX",
// "Task head").  Activations live channels-last, one row per pixel
// ([batch * gh * gw, C]), so 1x1 convs are plain GEMMs on the MFMA kernel and
// 3x3 convs are implicit GEMMs on it (the A loads gather the 3x3
// neighbourhood in place).  What remains here is the data movement and the
// per-pixel / per-group normalisations:
//   taps_cl_kernel        channel-first fp32 taps -> channels-last bf16 concat
//   groupnorm_gelu_kernel GroupNorm over (channels of a group x pixels) + GELU
//   resize_nchw_kernel    bilinear resize of class-minor logits to [B, C, H, W]
#include "common.h"
#include "kernels.h"

namespace vit {
namespace {

// One 64-channel x 64-pixel tile of one (image, tap) through LDS: reads are
// contiguous along pixels (the taps are channel-first), writes are 16 bytes
// (8 channels) per lane along the concatenated channels of a pixel row.
__global__ __launch_bounds__(256) void taps_cl_kernel(const float* __restrict__ taps, int ntaps, int D, int P,
                                                      uint16_t* __restrict__ out) {
  __shared__ float tile[64][65];
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int bt = blockIdx.z;              // b * ntaps + t
  const int b = bt / ntaps, t = bt - b * ntaps;
  const float* src = taps + ((size_t)bt * D + c0) * P;
  const int tid = threadIdx.x;
  const int col = tid & 63;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = (tid >> 6) + 4 * k;   // channel within the tile
    tile[r][col] = (p0 + col < P) ? src[(size_t)r * P + p0 + col] : 0.f;
  }
  __syncthreads();
  const int ldo = ntaps * D;
  const int chunk = tid & 7;            // 8 channels
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int pl = (tid >> 3) + 32 * pass;
    if (p0 + pl < P) {
      const int c = chunk * 8;
      uint4 u = make_uint4(pack_bf16x2(tile[c][pl], tile[c + 1][pl]), pack_bf16x2(tile[c + 2][pl], tile[c + 3][pl]),
                           pack_bf16x2(tile[c + 4][pl], tile[c + 5][pl]), pack_bf16x2(tile[c + 6][pl], tile[c + 7][pl]));
      *reinterpret_cast<uint4*>(out + ((size_t)b * P + p0 + pl) * ldo + t * D + c0 + c) = u;
    }
  }
}

// GroupNorm (8 channels per group) over the P pixels of one image, then the
// per-channel affine and the exact GELU; one workgroup per (group, image),
// two passes for the mean and the biased variance as in the definition.
// PPT > 0: each thread holds its pixels tid + 256 i (i < PPT) in registers,
// so the group is read from memory once; PPT = 0: three passes over memory
// (any P).  Both sum in the same order, so they give the same bits.
template <int PPT>
__global__ __launch_bounds__(256) void groupnorm_gelu_kernel(const float* __restrict__ x, int P, int C,
                                                             const float* __restrict__ g, const float* __restrict__ bta,
                                                             float eps, uint16_t* __restrict__ out) {
  __shared__ float red[4];
  const int grp = blockIdx.x, b = blockIdx.y;
  const int c0 = grp * 8;
  const float* base = x + (size_t)b * P * C + c0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto block_sum = [&](float s) {
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    const float t = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return t;
  };
  auto load = [&](int p, float (&v)[8]) {
    const float4 u = reinterpret_cast<const float4*>(base + (size_t)p * C)[0];
    const float4 w = reinterpret_cast<const float4*>(base + (size_t)p * C)[1];
    v[0] = u.x, v[1] = u.y, v[2] = u.z, v[3] = u.w, v[4] = w.x, v[5] = w.y, v[6] = w.z, v[7] = w.w;
  };
  auto add_sum = [](float& s, const float (&v)[8]) { s += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])); };
  auto add_sq = [](float& q, const float (&v)[8], float mean) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float d = v[i] - mean;
      q += d * d;
    }
  };
  const float n = 8.f * (float)P;
  float gs[8], bs[8];
  auto store = [&](int p, const float (&v)[8], float mean) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float z = (v[i] - mean) * gs[i] + bs[i];
      y[i] = 0.5f * z * (1.f + erff(z * 0.70710678118654752f));
    }
    *reinterpret_cast<uint4*>(out + ((size_t)b * P + p) * C + c0) =
        make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
  };
  if constexpr (PPT > 0) {
    float v[PPT][8];
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (tid + 256 * i < P) load(tid + 256 * i, v[i]);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (tid + 256 * i < P) add_sum(s, v[i]);
    const float mean = block_sum(s) / n;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (tid + 256 * i < P) add_sq(q, v[i], mean);
    const float rstd = rsqrtf(block_sum(q) / n + eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) gs[i] = g[c0 + i] * rstd, bs[i] = bta[c0 + i];
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (tid + 256 * i < P) store(tid + 256 * i, v[i], mean);
  } else {
    float v[8];
    float s = 0.f;
    for (int p = tid; p < P; p += 256) {
      load(p, v);
      add_sum(s, v);
    }
    const float mean = block_sum(s) / n;
    float q = 0.f;
    for (int p = tid; p < P; p += 256) {
      load(p, v);
      add_sq(q, v, mean);
    }
    const float rstd = rsqrtf(block_sum(q) / n + eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) gs[i] = g[c0 + i] * rstd, bs[i] = bta[c0 + i];
    for (int p = tid; p < P; p += 256) {
      load(p, v);
      store(p, v, mean);
    }
  }
}

// Bilinear resize (half-pixel centres, exact rational taps, clamped) of
// class-minor logits in [batch * gh * gw, ldi] to out [batch, classes, H, W];
// one thread per output pixel (flat index over H * W), looping over the
// classes; consecutive threads write consecutive pixels of each class plane.
__global__ __launch_bounds__(256) void resize_nchw_kernel(const float* __restrict__ in, int ldi, int classes, int gh,
                                                          int gw, float* __restrict__ out, int H, int W) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H * W) return;
  const int y = i / W, x = i - y * W, b = blockIdx.y;
  int y0, y1, x0, x1;
  float ly, lx;
  bilinear_tap(y, gh, H, y0, y1, ly);
  bilinear_tap(x, gw, W, x0, x1, lx);
  const float* base = in + (size_t)b * gh * gw * ldi;
  const float* r00 = base + (size_t)(y0 * gw + x0) * ldi;
  const float* r01 = base + (size_t)(y0 * gw + x1) * ldi;
  const float* r10 = base + (size_t)(y1 * gw + x0) * ldi;
  const float* r11 = base + (size_t)(y1 * gw + x1) * ldi;
  float* o = out + (size_t)b * classes * H * W + i;
  const size_t plane = (size_t)H * W;
  int c = 0;
  for (; c + 4 <= classes; c += 4) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float top = (1.f - lx) * r00[c + j] + lx * r01[c + j];
      const float bot = (1.f - lx) * r10[c + j] + lx * r11[c + j];
      v[j] = (1.f - ly) * top + ly * bot;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) o[(c + j) * plane] = v[j];
  }
  for (; c < classes; ++c) {
    const float top = (1.f - lx) * r00[c] + lx * r01[c];
    const float bot = (1.f - lx) * r10[c] + lx * r11[c];
    o[c * plane] = (1.f - ly) * top + ly * bot;
  }
}

}  // namespace

hipError_t launch_taps_cl(const float* taps, int batch, int ntaps, int D, int P, uint16_t* out, hipStream_t s) {
  if (batch < 1 || ntaps < 1 || D % 64 || P < 1 || (long)batch * ntaps > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(taps_cl_kernel, dim3((P + 63) / 64, D / 64, batch * ntaps), dim3(256), 0, s, taps, ntaps, D, P,
                     out);
  return hipGetLastError();
}

hipError_t launch_groupnorm_gelu(const float* x, int batch, int P, int C, int groups, const float* g, const float* b,
                                 float eps, uint16_t* out, hipStream_t s) {
  if (groups < 1 || C != 8 * groups || batch < 1 || batch > 65535 || P < 1) return hipErrorInvalidValue;
  const dim3 grid(groups, batch);
  switch ((P + 255) / 256) {  // pixels per thread held in registers (up to 8)
    case 1: hipLaunchKernelGGL(groupnorm_gelu_kernel<1>, grid, dim3(256), 0, s, x, P, C, g, b, eps, out); break;
    case 2: hipLaunchKernelGGL(groupnorm_gelu_kernel<2>, grid, dim3(256), 0, s, x, P, C, g, b, eps, out); break;
    case 3: hipLaunchKernelGGL(groupnorm_gelu_kernel<3>, grid, dim3(256), 0, s, x, P, C, g, b, eps, out); break;
    case 4: hipLaunchKernelGGL(groupnorm_gelu_kernel<4>, grid, dim3(256), 0, s, x, P, C, g, b, eps, out); break;
    case 5: hipLaunchKernelGGL(groupnorm_gelu_kernel<5>, grid, dim3(256), 0, s, x, P, C, g, b, eps, out); break;
    case 6: hipLaunchKernelGGL(groupnorm_gelu_kernel<6>, grid, dim3(256), 0, s, x, P, C, g, b, eps, out); break;
    case 7: hipLaunchKernelGGL(groupnorm_gelu_kernel<7>, grid, dim3(256), 0, s, x, P, C, g, b, eps, out); break;
    case 8: hipLaunchKernelGGL(groupnorm_gelu_kernel<8>, grid, dim3(256), 0, s, x, P, C, g, b, eps, out); break;
    default: hipLaunchKernelGGL(groupnorm_gelu_kernel<0>, grid, dim3(256), 0, s, x, P, C, g, b, eps, out);
  }
  return hipGetLastError();
}

hipError_t launch_resize_nchw(const float* in, int ldi, int classes, int batch, int gh, int gw, float* out, int H,
                              int W, hipStream_t s) {
  if (classes < 1 || ldi < classes || batch < 1 || batch > 65535 || H < 1 || W < 1 || (long)H * W > (1L << 30))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(resize_nchw_kernel, dim3((unsigned)(((long)H * W + 255) / 256), batch), dim3(256), 0, s, in, ldi,
                     classes, gh, gw, out, H, W);
  return hipGetLastError();
}

}  // namespace vit
