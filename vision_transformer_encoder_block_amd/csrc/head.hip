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
// per-channel affine and the exact GELU; one workgroup of 1024 threads per
// (group, image), two passes for the mean and the biased variance as in the
// definition.  The input is group-major, so the group's 8 P values of one
// image are one contiguous run of 2 P float4 (pixel q / 2, channels
// 4 (q % 2) .. + 3): each load instruction of a wave reads 1 KB of
// consecutive memory.  Sixteen waves per workgroup (four per SIMD) keep the
// exact-GELU arithmetic and the reductions from running at one wave per SIMD
// (b8 head: 265 -> 257 us against 256 threads).
// QPT > 0: each thread holds its float4 tid + 1024 i (i < QPT) in registers,
// so the group is read from memory once; QPT = 0: three passes over memory
// (any P).  Both sum in the same order, so they give the same bits.
template <int QPT>
__global__ __launch_bounds__(1024) void groupnorm_gelu_kernel(const float* __restrict__ x, size_t gstride, int P,
                                                             int C, const float* __restrict__ g,
                                                             const float* __restrict__ bta, float eps,
                                                             uint16_t* __restrict__ out) {
  __shared__ float red[16];
  const int grp = blockIdx.x, b = blockIdx.y;
  const int c0 = grp * 8;
  const float4* base = reinterpret_cast<const float4*>(x + grp * gstride + (size_t)b * P * 8);
  const int nq = 2 * P;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto block_sum = [&](float s) {
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < 16; ++i) t += red[i];
    __syncthreads();
    return t;
  };
  auto add_sum = [](float& s, const float4& v) { s += (v.x + v.y) + (v.z + v.w); };
  auto add_sq = [](float& q, const float4& v, float mean) {
    const float a = v.x - mean, c = v.y - mean, d = v.z - mean, e = v.w - mean;
    q += (a * a + c * c) + (d * d + e * e);
  };
  const float n = 8.f * (float)P;
  // this thread's four channels are 4 (q % 2) .. + 3 for every q = tid + 256 i
  const int cq = (tid & 1) * 4;
  float gs[4], bs[4];
  auto store = [&](int q, const float4& v, float mean) {
    const float in[4] = {v.x, v.y, v.z, v.w};
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = (in[i] - mean) * gs[i] + bs[i];
      y[i] = 0.5f * z * (1.f + erff(z * 0.70710678118654752f));
    }
    *reinterpret_cast<uint2*>(out + ((size_t)b * P + (q >> 1)) * C + c0 + cq) =
        make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
  };
  auto affine = [&](float rstd) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gs[i] = g[c0 + cq + i] * rstd, bs[i] = bta[c0 + cq + i];
  };
  if constexpr (QPT > 0) {
    float4 v[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i)
      if (tid + 1024 * i < nq) v[i] = base[tid + 1024 * i];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < QPT; ++i)
      if (tid + 1024 * i < nq) add_sum(s, v[i]);
    const float mean = block_sum(s) / n;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < QPT; ++i)
      if (tid + 1024 * i < nq) add_sq(q, v[i], mean);
    affine(rsqrtf(block_sum(q) / n + eps));
#pragma unroll
    for (int i = 0; i < QPT; ++i)
      if (tid + 1024 * i < nq) store(tid + 1024 * i, v[i], mean);
  } else {
    float s = 0.f;
    for (int q = tid; q < nq; q += 1024) add_sum(s, base[q]);
    const float mean = block_sum(s) / n;
    float q2 = 0.f;
    for (int q = tid; q < nq; q += 1024) add_sq(q2, base[q], mean);
    affine(rsqrtf(block_sum(q2) / n + eps));
    for (int q = tid; q < nq; q += 1024) store(q, base[q], mean);
  }
}

template <int Q>
void launch_gn(int qpt, dim3 grid, hipStream_t s, const float* x, size_t gstride, int P, int C, const float* g,
               const float* b, float eps, uint16_t* out) {
  if constexpr (Q > 0) {
    if (qpt == Q) {
      hipLaunchKernelGGL(groupnorm_gelu_kernel<Q>, grid, dim3(1024), 0, s, x, gstride, P, C, g, b, eps, out);
      return;
    }
    launch_gn<Q - 1>(qpt, grid, s, x, gstride, P, C, g, b, eps, out);
  } else {
    hipLaunchKernelGGL(groupnorm_gelu_kernel<0>, grid, dim3(1024), 0, s, x, gstride, P, C, g, b, eps, out);
  }
}

// Bilinear resize (half-pixel centres, exact rational taps, clamped) of
// class-minor logits in [batch * gh * gw, ldi] to out [batch, classes, H, W];
// one workgroup per output row y of one image.  The row's vertical blend of
// its two source rows, (1 - ly) r0 + ly r1 for every source column and class,
// is staged in LDS once (class-major); every output pixel of the row is then
// the horizontal blend of two staged values per class.  Consecutive threads
// write consecutive pixels of each class plane.
constexpr int kResizeLds = 4096;  // floats of staged row (16 KB): gw * classes <= this
__global__ __launch_bounds__(256) void resize_nchw_kernel(const float* __restrict__ in, int ldi, int classes, int gh,
                                                          int gw, float* __restrict__ out, int H, int W) {
  __shared__ float row[kResizeLds];
  const int y = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int y0, y1;
  float ly;
  bilinear_tap(y, gh, H, y0, y1, ly);
  const float* r0 = in + ((size_t)b * gh + y0) * gw * ldi;
  const float* r1 = in + ((size_t)b * gh + y1) * gw * ldi;
  const int n = gw * classes;
  for (int e = tid; e < n; e += 256) {
    const int xi = e / classes, c = e - xi * classes;
    row[c * gw + xi] = (1.f - ly) * r0[(size_t)xi * ldi + c] + ly * r1[(size_t)xi * ldi + c];
  }
  __syncthreads();
  float* o = out + ((size_t)b * classes * H + y) * W;
  const size_t plane = (size_t)H * W;
  for (int x = tid; x < W; x += 256) {
    int x0, x1;
    float lx;
    bilinear_tap(x, gw, W, x0, x1, lx);
    for (int c = 0; c < classes; ++c) o[c * plane + x] = (1.f - lx) * row[c * gw + x0] + lx * row[c * gw + x1];
  }
}

// The same resize for grids whose staged row would not fit (gw * classes >
// kResizeLds): one thread per output pixel, gathering its four source pixels'
// class vectors directly (horizontal blends first, then the vertical one).
__global__ __launch_bounds__(256) void resize_nchw_gather_kernel(const float* __restrict__ in, int ldi, int classes,
                                                                 int gh, int gw, float* __restrict__ out, int H, int W) {
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
  for (int c = 0; c < classes; ++c) {
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

hipError_t launch_groupnorm_gelu(const float* x, size_t gstride, int batch, int P, int C, int groups, const float* g,
                                 const float* b, float eps, uint16_t* out, hipStream_t s) {
  if (groups < 1 || C != 8 * groups || batch < 1 || batch > 65535 || P < 1 || gstride < (size_t)8 * batch * P ||
      reinterpret_cast<uintptr_t>(x) % 16 || gstride % 4)
    return hipErrorInvalidValue;
  // float4 per thread held in registers (up to 16, i.e. 8192 pixels), else
  // the loop over memory
  const int qpt = (2 * P + 1023) / 1024;
  launch_gn<16>(qpt <= 16 ? qpt : 0, dim3(groups, batch), s, x, gstride, P, C, g, b, eps, out);
  return hipGetLastError();
}

hipError_t launch_resize_nchw(const float* in, int ldi, int classes, int batch, int gh, int gw, float* out, int H,
                              int W, hipStream_t s) {
  if (classes < 1 || ldi < classes || batch < 1 || batch > 65535 || H < 1 || W < 1 || (long)H * W > (1L << 30) ||
      gh < 1 || gw < 1)
    return hipErrorInvalidValue;
  if ((long)gw * classes <= kResizeLds)
    hipLaunchKernelGGL(resize_nchw_kernel, dim3(H, batch), dim3(256), 0, s, in, ldi, classes, gh, gw, out, H, W);
  else
    hipLaunchKernelGGL(resize_nchw_gather_kernel, dim3((unsigned)(((long)H * W + 255) / 256), batch), dim3(256), 0, s,
                       in, ldi, classes, gh, gw, out, H, W);
  return hipGetLastError();
}

}  // namespace vit
