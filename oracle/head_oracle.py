"""Plain CPU oracle for the LibreYOLO DINOv2 semantic head on the four taps.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module.  The GPU product path never
calls it and shares no code with it.  Every step is written from the published
description in float64 NumPy; a matrix product (``@``) is the only library
primitive used for arithmetic (besides the erf GELU and the bilinear resize of
``vit_oracle``).

Source: the LibreYOLO DINOv2 "n semantic" diagram (libreyolo.com), sections

* "Projector P4": the four LayerNormed taps (after blocks 3, 6, 9, 12, each
  384 x 37 x 37) concatenated to 1536 channels; a 1x1 conv 1536 -> 256 without
  bias, channel LayerNorm, SiLU; a split into two halves a and b of 128
  channels; three Bottlenecks without shortcut; the concat of a, b and the
  three Bottleneck outputs (640 channels); the output ConvX; a final channel
  LayerNorm;
* "Projector Bottleneck": two 3x3 stride-1 convs 128 -> 128 with padding 1 and
  no bias, each followed by channel LayerNorm and SiLU, no residual;
* "Projector output ConvX": a 1x1 conv 640 -> 256 without bias, channel
  LayerNorm, SiLU;
* "Task head": lateral 1x1 conv 256 -> 256 with bias, smoothing 3x3 conv
  256 -> 256 with padding 1 and bias, GroupNorm with 32 groups, GELU,
  Dropout2d (identity in evaluation), predict 1x1 conv 256 -> 19, bilinear
  resize to 19 x 518 x 518 with align_corners=False;
* "Size equivalence": projector width 256 and taps 3, 6, 9, 12 at every size.

Readings where the diagram is silent (each also listed in the design notes):

* a channel LayerNorm normalises the channels of each pixel (biased variance,
  epsilon inside the square root) with a per-channel affine; its epsilon is
  1e-6, the only LayerNorm epsilon the diagram states;
* GroupNorm uses epsilon 1e-5 and a per-channel affine (PyTorch's defaults);
* the predict conv has a bias (PyTorch's default for Conv2d);
* GELU is the exact erf form, as in the encoder;
* the first Bottleneck takes the second half b, each later one the previous
  Bottleneck's output ("each receives the preceding output");
* the logits are resized to the encoder's input size.

Parity status: every function is pinned by ``tests/test_oracle_head.py``
(float64 PyTorch library routines, a torch.nn module written separately from
the diagram, closed forms, invariants and the diagram's printed shapes).
"""

from __future__ import annotations

import numpy as np
from scipy.special import expit

from .vit_oracle import bilinear_resize, gelu

F64 = np.float64

HEAD_LN_EPS = 1e-6      # channel LayerNorm (reading: the diagram's LayerNorm epsilon)
GROUPNORM_EPS = 1e-5    # GroupNorm (reading: PyTorch default)
GROUPS = 32             # "GroupNorm, 32 groups, 256 channels"
WIDTH = 256             # projector width ("Size equivalence")
HALF = 128              # C2f split ("a: 128 channels; b: 128 channels")
BOTTLENECKS = 3
CLASSES = 19            # "Predict Conv2d 1x1, 256 to 19 class logits"


def conv2d(x: np.ndarray, w: np.ndarray, b: np.ndarray | None = None, pad: int = 0) -> np.ndarray:
    """Stride-1 convolution of x [C, H, W] with w [Co, C, k, k] and zero padding ``pad``:
    out[o, y, x] = b[o] + sum_{c, ky, kx} w[o, c, ky, kx] * xpad[c, y + ky, x + kx]."""
    x = np.asarray(x, F64)
    w = np.asarray(w, F64)
    C, H, W = x.shape
    Co, Ci, kh, kw = w.shape
    assert Ci == C
    xp = np.zeros((C, H + 2 * pad, W + 2 * pad), F64)
    xp[:, pad:pad + H, pad:pad + W] = x
    Ho, Wo = H + 2 * pad - kh + 1, W + 2 * pad - kw + 1
    cols = np.empty((C, kh, kw, Ho, Wo), F64)
    for ky in range(kh):
        for kx in range(kw):
            cols[:, ky, kx] = xp[:, ky:ky + Ho, kx:kx + Wo]
    out = w.reshape(Co, C * kh * kw) @ cols.reshape(C * kh * kw, Ho * Wo)
    if b is not None:
        out += np.asarray(b, F64)[:, None]
    return out.reshape(Co, Ho, Wo)


def channel_layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = HEAD_LN_EPS) -> np.ndarray:
    """LayerNorm over the channels of every pixel of x [C, H, W], per-channel affine."""
    x = np.asarray(x, F64)
    mu = x.mean(axis=0, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=0, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(g, F64)[:, None, None] + np.asarray(b, F64)[:, None, None]


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x)."""
    x = np.asarray(x, F64)
    return x * expit(x)


def group_norm(x: np.ndarray, groups: int, g: np.ndarray, b: np.ndarray, eps: float = GROUPNORM_EPS) -> np.ndarray:
    """GroupNorm of x [C, H, W]: channels split into ``groups`` consecutive groups, each
    normalised over its channels and all pixels (biased variance), then a per-channel affine."""
    x = np.asarray(x, F64)
    C, H, W = x.shape
    xg = x.reshape(groups, (C // groups) * H * W)
    mu = xg.mean(axis=1, keepdims=True)
    var = ((xg - mu) ** 2).mean(axis=1, keepdims=True)
    y = ((xg - mu) / np.sqrt(var + eps)).reshape(C, H, W)
    return y * np.asarray(g, F64)[:, None, None] + np.asarray(b, F64)[:, None, None]


def conv_ln_silu(x: np.ndarray, w: np.ndarray, g: np.ndarray, b: np.ndarray, pad: int) -> np.ndarray:
    """Conv (no bias), channel LayerNorm, SiLU: the diagram's ConvX unit."""
    return silu(channel_layer_norm(conv2d(x, w, None, pad), g, b))


def bottleneck(x: np.ndarray, Ph: dict, i: int) -> np.ndarray:
    """Projector Bottleneck i (1-based): two 3x3 ConvX units, no residual."""
    y = conv_ln_silu(x, Ph[f"bn{i}_w1"], Ph[f"bn{i}_ln1_g"], Ph[f"bn{i}_ln1_b"], 1)
    return conv_ln_silu(y, Ph[f"bn{i}_w2"], Ph[f"bn{i}_ln2_g"], Ph[f"bn{i}_ln2_b"], 1)


def projector(taps: np.ndarray, Ph: dict, stats: dict | None = None) -> np.ndarray:
    """Projector P4 of one image: taps [4, D, gh, gw] -> [256, gh, gw]."""
    taps = np.asarray(taps, F64)
    n, D, gh, gw = taps.shape
    x = taps.reshape(n * D, gh, gw)                     # concat, tap 3 first
    y = conv_ln_silu(x, Ph["proj_w"], Ph["proj_ln_g"], Ph["proj_ln_b"], 0)
    a, b = y[:HALF], y[HALF:]
    parts = [a, b]
    cur = b
    for i in range(1, BOTTLENECKS + 1):
        cur = bottleneck(cur, Ph, i)
        parts.append(cur)
    cat = np.concatenate(parts, axis=0)                 # a, b, bottleneck 1, 2, 3
    if stats is not None:
        stats["c2f_concat"] = cat
    z = conv_ln_silu(cat, Ph["out_w"], Ph["out_ln_g"], Ph["out_ln_b"], 0)
    return channel_layer_norm(z, Ph["final_ln_g"], Ph["final_ln_b"])


def task_head_grid(p4: np.ndarray, Ph: dict) -> np.ndarray:
    """Task head up to the class logits at the patch grid: [256, gh, gw] -> [19, gh, gw]."""
    lat = conv2d(p4, Ph["lat_w"], Ph["lat_b"], 0)
    sm = conv2d(lat, Ph["smooth_w"], Ph["smooth_b"], 1)
    act = gelu(group_norm(sm, GROUPS, Ph["gn_g"], Ph["gn_b"]))   # Dropout2d: identity in evaluation
    return conv2d(act, Ph["pred_w"], Ph["pred_b"], 0)


def semantic_head(taps: np.ndarray, Ph: dict, out_h: int, out_w: int) -> dict:
    """The whole head for one image: taps [4, D, gh, gw] -> logits [19, out_h, out_w].

    Returns the projector output ``p4``, the grid logits ``grid`` and the resized ``logits``.
    """
    p4 = projector(taps, Ph)
    grid = task_head_grid(p4, Ph)
    return {"p4": p4, "grid": grid, "logits": bilinear_resize(grid, out_h, out_w)}
