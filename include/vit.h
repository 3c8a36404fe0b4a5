/*
 * vit.h - C ABI of the MI355X (gfx950) ViT encoder forward pass.
 *
 * The operation (sources are web pages, cited by title and section):
 *   an image batch [B,3,H,W] (ImageNet-normalised, fp32, CHW) goes in
 *   (kornia/dinov3 model card, "Model I/O"); a token grid [B,N,D] of final
 *   LayerNorm outputs and an L2-normalised CLS descriptor [B,D] come out
 *   (same card, "Model I/O" and "Usage": descriptor = last_hidden_state[:,0],
 *   "L2-normed, cosine-ready").  In between: Conv2d patch embedding, learned
 *   CLS token, R register tokens placed between CLS and the patches, learned
 *   position embedding (bicubically resampled when the image grid differs
 *   from the stored grid), L pre-LN encoder blocks (LayerNorm eps 1e-6,
 *   multi-head self-attention with 64-channel heads and logits scaled by
 *   1/sqrt(64), LayerScale, residual; LayerNorm, Linear D->Hm, GELU,
 *   Linear Hm->D, LayerScale, residual) and a final LayerNorm (LibreYOLO
 *   DINOv2 diagram, figures "DINOv2-S encoder", "Encoder block", "Encoder
 *   self-attention"; DINOv2 ONNX/TensorRT article, class diagram).
 *
 * Ownership: the caller allocates ALL device memory (weights, workspace,
 * inputs, outputs) and passes raw device pointers; the library never
 * allocates device memory.  Host pointers are only read during the call.
 * Every call enqueues work on the caller's HIP stream (`stream`, a
 * hipStream_t passed as void*; NULL = the null stream) and returns without
 * synchronising, except vit_create, which synchronises the stream once after
 * uploading the packed weights.
 *
 * Errors: every function returns 0 (VIT_OK) or a negative vit_status.
 * Argument and shape errors are detected before anything is enqueued.  A
 * launch failure returns VIT_ERR_HIP.  Faults during execution surface at the
 * caller's next stream synchronisation.  vit_last_error() gives a message for
 * the calling thread's most recent failure.  No function throws or aborts.
 *
 * Numerics: GEMM operands are bf16 (round to nearest even), accumulation fp32;
 * the residual stream, LayerNorm statistics, softmax max/sum and all outputs
 * are fp32.  Attention logits are never stored in a 16-bit format, so the
 * ~2.5e6 logits reported for DINOv3 (model card, "Build BF16, not FP16")
 * stay finite.
 *
 * Thread safety: a vit_model owns one workspace; calls on one model must not
 * overlap in time (use one model per concurrent stream).
 */
#ifndef VIT_H
#define VIT_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vit_status {
  VIT_OK = 0,
  VIT_ERR_ARG = -1,         /* NULL pointer or out-of-range scalar */
  VIT_ERR_SHAPE = -2,       /* inconsistent geometry (e.g. H not a multiple of the patch) */
  VIT_ERR_SIZE = -3,        /* buffer smaller than vit_plan requires, or batch > max_batch */
  VIT_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  VIT_ERR_UNSUPPORTED = -5  /* valid but not implemented (e.g. head size != 64) */
};

typedef struct vit_model vit_model;

/* Model and geometry.  All fields are plain values. */
typedef struct vit_config {
  int img_h, img_w;          /* input image size; multiples of `patch` */
  int patch;                 /* patch side p (Conv2d kernel = stride = p), 2..32 */
  int dim;                   /* width D; multiple of 64 */
  int depth;                 /* backbone blocks L (>= 0) */
  int extra_blocks;          /* blocks appended after the backbone (dino.txt head: 2) */
  int heads;                 /* D / 64 (64-channel heads only) */
  int mlp_hidden;            /* Hm; multiple of 64 */
  int registers;             /* register tokens R, 0..16 */
  int max_batch;             /* largest batch passed to vit_forward */
  float ln_eps;              /* LayerNorm epsilon (1e-6) */
  unsigned tap_mask;         /* bit l-1 set: emit a tap after block l (l <= depth + extra_blocks) */
  int pos_grid_h, pos_grid_w;/* grid of the stored position table (1 + gh*gw rows) */
  int window, window_stride; /* slide-mode window side and stride in pixels (1 <= stride <= window); 0 = no slide mode */
  int max_classes;           /* largest class count for vit_patch_scores; 0 = no scoring */
} vit_config;

/* Sizes derived from a vit_config. */
typedef struct vit_sizes {
  size_t weight_bytes;       /* device bytes for the packed weights */
  size_t workspace_bytes;    /* device bytes for activations and scratch */
  size_t host_floats;        /* length of the fp32 parameter blob vit_create reads */
  int tokens;                /* N = (H/p)(W/p) + 1 + R at img_h x img_w */
  int window_tokens;         /* N of one slide window (0 without slide mode) */
  int windows;               /* number of slide windows on an img_h x img_w image */
  int taps;                  /* number of bits set in tap_mask */
} vit_sizes;

/* Fill `out` with one of the five workload presets:
 *   1 ViT-S/16 @224, R=4, max_batch 1        4 ViT-L/16 @1024, R=4, max_batch 4
 *   2 ViT-S/16 @336, R=4, max_batch 32       5 ViT-L/16 + 2 blocks @512x1024, R=4,
 *   3 DINOv2-S/14 @518, R=0, taps 3/6/9/12,     window 384 stride 192, 150 classes
 *     max_batch 8
 * Returns VIT_ERR_ARG for an unknown id or a NULL `out`. Pure host function. */
int vit_config_preset(int cfg_id, vit_config* out);

/* Validate `cfg` and report the buffer sizes it needs.  Pure host function. */
int vit_plan(const vit_config* cfg, vit_sizes* out);

/* Build a model from the fp32 parameter blob `host_params` (host memory,
 * `host_floats` values, layout below), packing it into `d_weights`
 * (device, >= weight_bytes) and binding `d_workspace` (device,
 * >= workspace_bytes).  Linear and patch weights are rounded to bf16 (nearest
 * even).  The workspace is cleared.  Synchronises `stream` before returning.
 * d_workspace may be NULL with workspace_bytes 0: the model then runs only
 * through vit_forward_static (vit_forward and vit_patch_scores return
 * VIT_ERR_ARG).  The model belongs to the device current at this call.
 *
 * Blob layout (fp32, row-major, concatenated in this order; Linear weights
 * are [out, in] as in torch.nn.Linear):
 *   patch_w [D,3,p,p], patch_b [D], cls [D], reg [R,D],
 *   pos [1 + pos_grid_h*pos_grid_w, D]  (row 0: CLS, then patches in raster order),
 *   then for each of the depth + extra_blocks blocks:
 *     ln1_g [D], ln1_b [D], wq [D,D], bq [D], wk [D,D], bk [D], wv [D,D], bv [D],
 *     wo [D,D], bo [D], ls1 [D], ln2_g [D], ln2_b [D], w1 [Hm,D], b1 [Hm],
 *     w2 [D,Hm], b2 [D], ls2 [D],
 *   norm_g [D], norm_b [D].
 * The buffers must stay allocated until vit_destroy and until all work
 * enqueued with the model has finished. */
int vit_create(const vit_config* cfg, const float* host_params, size_t host_floats,
               void* d_weights, size_t weight_bytes, void* d_workspace, size_t workspace_bytes,
               void* stream, vit_model** out);

/* Encoder forward for `batch` (1..max_batch) images.
 *   d_images  device fp32 [batch,3,img_h,img_w]
 *   d_tokens  device fp32 [batch,N,D], 16-byte aligned: final LayerNorm of every token
 *             (row 0 CLS, rows 1..R registers, then patches in raster order)
 *   d_taps    NULL, or device fp32 [batch, taps, D, H/p, W/p]: after each
 *             block selected by tap_mask, the final LayerNorm (backbone `norm`
 *             parameters) of the patch tokens, channel-first (LibreYOLO
 *             diagram: "Taps apply LayerNorm, remove CLS, reshape").
 * Enqueue only. */
int vit_forward(vit_model* m, const float* d_images, int batch, float* d_tokens, float* d_taps,
                void* stream);

/* Size of the library's static activation array (per device), see
 * vit_forward_static. */
#define VIT_STATIC_SCRATCH_BYTES (96u * 1024u * 1024u)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as vit_forward, same arguments and outputs (bit-identical), but the
 * activations live in a static device array of VIT_STATIC_SCRATCH_BYTES
 * (96 MiB) inside the library instead of the workspace bound at vit_create,
 * which may be NULL.  Nothing is allocated: each device that the library runs
 * on holds its own array from loading until the process ends, its address
 * taken once when the first model is created on that device.
 *   Limit: batch images need at most vit_plan's workspace_bytes with
 *   max_batch = batch (ViT-L/16 @1024: 94.2 MiB at batch 1; ViT-S/16 @336:
 *   4.2 MiB per image); a batch beyond 96 MiB returns VIT_ERR_SIZE, before
 *   anything is enqueued.
 *   Every call on one device shares that device's array and leaves its
 *   activations there: calls that overlap on one device (several streams or
 *   threads, or several models) race and must be serialised by the caller.
 *   The forward reads no activation it has not written in the same call, so
 *   the array needs no clearing.
 * Enqueue only. */
int vit_forward_static(vit_model* m, const float* d_images, int batch, float* d_tokens, float* d_taps,
                       void* stream);

/* CLS descriptor: d_desc[b] = tokens[b,0,:] / max(||tokens[b,0,:]||_2, 1e-12)
 * (model card, "Model I/O": the descriptor is the CLS token; "Usage":
 * L2-normed).  d_tokens as written by vit_forward; d_desc device fp32 [batch,D]. */
int vit_descriptor(vit_model* m, const float* d_tokens, int batch, float* d_desc, void* stream);

/* Zero-shot patch-text scoring of ONE image (dino.txt zero-shot segmentation
 * article, whole / slide modes).  Patch features are the final-LayerNormed
 * patch tokens after all depth + extra_blocks blocks, L2-normalised; the score
 * of class c at a patch is their dot product with d_class_emb[c].
 *   d_image      device fp32 [3,img_h,img_w]
 *   d_class_emb  device fp32 [classes,D] (unit vectors), classes <= max_classes
 *   mode 0 (whole): one forward; scores upsampled bilinearly (half-pixel
 *     centres) to img_h x img_w; label = first argmax over classes.
 *   mode 1 (slide): window x window crops every window_stride pixels, the last
 *     one moved back to the border, run as one batch; per window the upsampled
 *     scores are softmaxed over classes and accumulated with overlap counts;
 *     label = first argmax of the average.
 *   d_labels     device int32 [img_h,img_w]
 *   d_cos        NULL, or device fp32 low-resolution scores: whole [classes, H/p, W/p];
 *                slide [windows, classes, window/p, window/p]
 *   d_dense      NULL, or device fp32 [classes,img_h,img_w]: whole = upsampled
 *                scores, slide = averaged probabilities (large; for checking). */
int vit_patch_scores(vit_model* m, const float* d_image, const float* d_class_emb, int classes,
                     int mode, int* d_labels, float* d_cos, float* d_dense, void* stream);

/* Release the host-side handle (device buffers belong to the caller). */
int vit_destroy(vit_model* m);

/* Message for the calling thread's most recent failure ("" if none). */
const char* vit_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VIT_H */
