/*
 * vit_head.h - C ABI of the semantic head on the encoder's taps (MI355X, gfx950).
 *
 * The operation (LibreYOLO DINOv2 "n semantic" diagram, libreyolo.com):
 *   "Projector P4": the taps (LayerNormed patch features after blocks 3, 6,
 *   9, 12; vit_forward's d_taps) concatenated along channels; Conv2d 1x1
 *   taps*D -> width without bias, channel LayerNorm, SiLU; split into halves
 *   a, b; three Bottlenecks without shortcut, the first on b and each next one
 *   on the previous output ("Projector Bottleneck": Conv2d 3x3/1 pad 1 without
 *   bias, channel LayerNorm, SiLU, twice); concat a, b and the three outputs
 *   (5 * width / 2 channels); "Projector output ConvX" (Conv2d 1x1 -> width
 *   without bias, channel LayerNorm, SiLU); a final channel LayerNorm.
 *   "Task head": lateral Conv2d 1x1 width -> width with bias; smoothing
 *   Conv2d 3x3 pad 1 with bias; GroupNorm (groups); GELU (exact erf form);
 *   Dropout2d (identity in evaluation); predict Conv2d 1x1 width -> classes
 *   with bias; bilinear resize to out_h x out_w (align_corners=False).
 *   "Size equivalence": width 256 and taps 3/6/9/12 at every size.
 *
 * Readings where the diagram is silent: a channel LayerNorm normalises the
 * channels of each pixel (biased variance, eps inside the square root, here
 * ln_eps = 1e-6 like the encoder's) with a per-channel affine; GroupNorm uses
 * gn_eps = 1e-5 and a per-channel affine; the predict conv has a bias.
 *
 * Ownership, streams and errors follow vit.h: the caller allocates all device
 * memory; every call enqueues on `stream` and returns without synchronising
 * (except vit_head_create, which synchronises once after the upload); return
 * values are 0 or a negative vit_status, with vit_last_error() describing the
 * calling thread's last failure.  Calls on one vit_head must not overlap.
 *
 * Numerics: conv operands bf16 (nearest even) with fp32 accumulation; the
 * normalisation statistics, the logits and the resize are fp32; activations
 * between layers are stored as bf16.
 */
#ifndef VIT_HEAD_H
#define VIT_HEAD_H

#include <stddef.h>

#include "vit.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct vit_head vit_head;

typedef struct vit_head_config {
  int grid_h, grid_w;   /* patch grid of the taps (37 x 37 for DINOv2-S/14 @518) */
  int dim;              /* channels of one tap (encoder width D); multiple of 64 */
  int taps;             /* number of taps concatenated (4) */
  int width;            /* projector width: 256 (the diagram's, at every size) */
  int groups;           /* GroupNorm groups (32); width must equal 8 * groups */
  int classes;          /* predicted classes (19); 1..1024 */
  int out_h, out_w;     /* size of the resized logits (the image: 518 x 518) */
  int max_batch;        /* largest batch passed to vit_head_forward */
  float ln_eps;         /* channel LayerNorm epsilon (1e-6) */
  float gn_eps;         /* GroupNorm epsilon (1e-5) */
} vit_head_config;

typedef struct vit_head_sizes {
  size_t weight_bytes;     /* device bytes for the packed weights */
  size_t workspace_bytes;  /* device bytes for activations */
  size_t host_floats;      /* length of the fp32 parameter blob vit_head_create reads */
} vit_head_sizes;

/* The diagram's head for DINOv2-S/14 at 518 x 518 (grid 37 x 37, D 384, 4 taps,
 * width 256, 32 groups, 19 classes, logits 518 x 518), max_batch 8.  Pure host. */
int vit_head_config_preset(vit_head_config* out);

/* Validate `cfg` and report the buffer sizes it needs.  Pure host function. */
int vit_head_plan(const vit_head_config* cfg, vit_head_sizes* out);

/* Build a head from the fp32 blob `host_params` (host memory, `host_floats`
 * values), packing it into `d_weights` and binding `d_workspace` (device,
 * 256-byte aligned, at least vit_head_plan's sizes).  Conv weights are
 * rounded to bf16 (nearest even).  Synchronises `stream` before returning.
 *
 * Blob layout (fp32, concatenated in this order; conv weights [out, in, kh, kw]
 * as in torch.nn.Conv2d; W = width, H2 = width / 2, T = taps * dim):
 *   proj_w [W, T, 1, 1], proj_ln_g [W], proj_ln_b [W],
 *   for i = 1, 2, 3: bn{i}_w1 [H2, H2, 3, 3], bn{i}_ln1_g [H2], bn{i}_ln1_b [H2],
 *                    bn{i}_w2 [H2, H2, 3, 3], bn{i}_ln2_g [H2], bn{i}_ln2_b [H2],
 *   out_w [W, 5 * H2, 1, 1], out_ln_g [W], out_ln_b [W], final_ln_g [W], final_ln_b [W],
 *   lat_w [W, W, 1, 1], lat_b [W], smooth_w [W, W, 3, 3], smooth_b [W],
 *   gn_g [W], gn_b [W], pred_w [classes, W, 1, 1], pred_b [classes]. */
int vit_head_create(const vit_head_config* cfg, const float* host_params, size_t host_floats, void* d_weights,
                    size_t weight_bytes, void* d_workspace, size_t workspace_bytes, void* stream, vit_head** out);

/* Head forward for `batch` (1..max_batch) images.
 *   d_taps    device fp32 [batch, taps, dim, grid_h, grid_w] (vit_forward's d_taps), 16-byte aligned
 *   d_logits  device fp32 [batch, classes, out_h, out_w]: resized class logits
 *   d_grid    NULL, or device fp32 [batch, classes, grid_h, grid_w]: the logits
 *             before the resize
 * Enqueue only. */
int vit_head_forward(vit_head* h, const float* d_taps, int batch, float* d_logits, float* d_grid, void* stream);

/* Release the host-side handle (device buffers belong to the caller). */
int vit_head_destroy(vit_head* h);

/* One 3x3 / stride 1 / zero-padding 1 convolution of the head (diagram,
 * "Projector Bottleneck" and the task head's smoothing conv) as an implicit
 * GEMM on channels-last bf16 activations:
 *   out[m, n] = bias[n] + sum_{ky, kx, c} w[n, (ky * 3 + kx) * cin + c] *
 *               in[pixel (y + ky - 1, x + kx - 1) of image b, c0 + c]
 * for row m = pixel (y, x) of image b on a gh x gw grid; terms whose pixel
 * lies outside the grid are zero.
 *   in   device bf16 [batch * gh * gw, ld_in], 16-byte aligned; channels c0 .. c0 + cin
 *        (cin a positive multiple of 64, c0 and ld_in multiples of 8)
 *   w    device bf16 [n_out, 9 * cin] (torch's [n_out, cin, 3, 3] with columns in (ky, kx, c) order)
 *   bias device fp32 [n_out] or NULL (zero)
 *   out  device fp32 [batch * gh * gw, n_out]
 * Enqueue only. */
int vit_op_conv3x3(const void* in, int ld_in, int c0, int cin, int batch, int gh, int gw, const void* w,
                   const float* bias, int n_out, float* out, void* stream);

/* One ConvX unit of the head (diagram: Conv2d without bias, channel
 * LayerNorm, SiLU; the "Projector output ConvX" adds the final channel
 * LayerNorm) as one GEMM whose epilogue normalises the n_out channels of each
 * pixel:
 *   y[m, :] = SiLU(LN(conv(in)[m, :]; g, b, eps)), then y = LN(y; g2, b2, eps) if g2 != NULL,
 * with LN the biased-variance LayerNorm over the channels (eps inside the
 * square root, per-channel affine), written as bf16 to out[m * ld_out + c0_out + n].
 *   ksize 3: the 3x3 / stride 1 / zero-padding 1 convolution of vit_op_conv3x3
 *            (same in, ld_in, c0, cin and w layout);
 *   ksize 1: in [batch * gh * gw, cin] bf16 rows (ld_in == cin, c0 == 0), w [n_out, cin].
 *   n_out 128 or 256; g, b (and g2, b2) device fp32 [n_out], 16-byte aligned; eps > 0;
 *   out device bf16, 8-byte aligned; ld_out and c0_out multiples of 4, c0_out + n_out <= ld_out.
 * Enqueue only. */
int vit_op_convx(const void* in, int ld_in, int c0, int cin, int batch, int gh, int gw, int ksize, const void* w,
                 int n_out, const float* g, const float* b, const float* g2, const float* b2, float eps, void* out,
                 int ld_out, int c0_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VIT_HEAD_H */
