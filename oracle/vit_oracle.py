"""Plain CPU oracle for the DINOv2/DINOv3 ViT encoder forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module.  The GPU product path never calls
it, and it shares no code with the HIP library: it implements every step again
from the published description, in float64 NumPy, without blocking, fusion or
reordering beyond what each definition states.  A matrix product (``@``) and
``scipy.special.erf`` are the only library primitives used for arithmetic.

Sources (web pages; sections named as they appear there):

* DINOv3 model card (aimarketly, "kornia/dinov3"): "Model I/O" (input
  [B,3,336,336], 4 register tokens between CLS and the patch grid, descriptor =
  CLS token of the last hidden state, L2-normed), "Build BF16, not FP16"
  (attention logits up to 2.5e6; fp16 overflow -> inf -> NaN).
* LibreYOLO DINOv2 "n semantic" diagram: "DINOv2-S encoder" (Conv2d patch
  embedding, flatten, learned CLS, concat, position embedding, bicubic
  interpolation, taps), "Encoder block" (pre-LN, eps 1e-6, layer scale, residual,
  MLP with GELU), "Encoder self-attention" (Linear Q/K/V, reshape heads, Q.K^T,
  divide by sqrt(64), softmax over keys, attention x V, merge heads, Linear
  output), "Taps apply LayerNorm, remove CLS, reshape".
* DINOv2 ONNX/TensorRT article (gitcode blog): DinoVisionTransformer class
  diagram (patch_embed, cls_token, pos_embed, register_tokens, blocks, norm),
  ``forward_features(x)["x_norm_clstoken"]``, model size table.
* DINOv2 ONNX/TensorRT deployment article: the FastAPI service's frame
  preprocessing (cv2 decode, BGR to RGB, cv2.resize, /255).
* dino.txt zero-shot segmentation article (hotelren): ViT-L/16 patch tokens
  after 2 extra attention blocks, per-patch L2 normalisation and cosine against
  class embeddings, whole mode (bilinear upsample, align_corners=False, argmax)
  and slide mode (side 384, stride 192, per-window softmax over classes,
  accumulate, divide by the overlap counts, argmax; 2 x 5 = 10 windows on a
  512 x 1024 image).

Readings where the pages are silent or ambiguous (each also listed in the
design notes): registers carry no position embedding; every Linear has a bias;
GELU is the exact erf form; the descriptor's L2 epsilon is 1e-12; taps use the
backbone's final LayerNorm parameters; the extra dino.txt blocks are ordinary
pre-LN blocks followed by the single final LayerNorm; bicubic resampling uses
the cubic-convolution kernel with a = -0.75 and half-pixel centres; slide
windows are full size with the last one moved back to end at the border;
frame preprocessing resamples the 8-bit values bilinearly without rounding
them back to 8 bits.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (library routines in float64, brute force on tiny
inputs, closed forms, invariants and the pages' printed shapes and counts).
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

F64 = np.float64

# ---------------------------------------------------------------------------
# number formats used only by the fp16 overflow demonstration


def to_format(x: np.ndarray, fmt: str | None) -> np.ndarray:
    """Round float64 values to ``fmt`` and return them as float64.

    ``fmt`` is None (no rounding), "fp32", "bf16" or "fp16".  fp16 follows IEEE
    binary16: round to nearest even, magnitudes beyond the largest finite value
    become +-inf.  bf16 keeps float32's 8-bit exponent and 8 significant bits
    (round to nearest even on the float32 bit pattern).
    """
    if fmt is None:
        return x
    if fmt == "fp32":
        return x.astype(np.float32).astype(F64)
    if fmt == "fp16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).astype(F64)
    if fmt == "bf16":
        f = x.astype(np.float32)
        bits = f.view(np.uint32).astype(np.uint64)
        keep = ((bits >> 16) & 1) + 0x7FFF
        bits = ((bits + keep) >> 16) << 16
        return bits.astype(np.uint32).view(np.float32).astype(F64)
    raise ValueError(f"unknown format {fmt!r}")


# ---------------------------------------------------------------------------
# patch embedding and token assembly


def patch_embed(images: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Conv2d with kernel = stride = p and a bias, flattened in raster order.

    ``images`` [B,3,H,W], ``w`` [D,3,p,p], ``b`` [D] -> [B, (H/p)*(W/p), D].
    Patch i = gy*gw + gx covers rows gy*p.. and cols gx*p..; its feature d is
    b[d] + sum over (c, ky, kx) of w[d,c,ky,kx] * x[c, gy*p+ky, gx*p+kx]
    (LibreYOLO diagram: "Conv2d 14x14 / 14, bias=True", "Flatten patch grid").
    """
    x = np.asarray(images, dtype=F64)
    B, C, H, W = x.shape
    D, C2, p, p2 = w.shape
    assert C == C2 and p == p2 and H % p == 0 and W % p == 0
    gh, gw = H // p, W // p
    # [B, C, gh, p, gw, p] -> [B, gh, gw, C, p, p]: one row per patch, (c, ky, kx) order
    cols = x.reshape(B, C, gh, p, gw, p).transpose(0, 2, 4, 1, 3, 5).reshape(B, gh * gw, C * p * p)
    return cols @ np.asarray(w, F64).reshape(D, C * p * p).T + np.asarray(b, F64)


def assemble_tokens(emb: np.ndarray, cls: np.ndarray, reg: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """[CLS + pos[0], registers (no position), patch_i + pos[1+i]] -> [B, 1+R+P, D].

    The position table covers CLS and the patches ("Position embedding 1,370 x
    384" for 1 CLS + 1369 patches); registers sit at indices 1..R between CLS
    and the patch grid (model card, "Model I/O").
    """
    B, Pn, D = emb.shape
    R = reg.shape[0]
    pos = np.asarray(pos, F64)
    assert pos.shape == (1 + Pn, D)
    t = np.empty((B, 1 + R + Pn, D), dtype=F64)
    t[:, 0] = np.asarray(cls, F64) + pos[0]
    t[:, 1:1 + R] = np.asarray(reg, F64)
    t[:, 1 + R:] = emb + pos[1:]
    return t


# ---------------------------------------------------------------------------
# block components


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * g + b over the last axis; var is the biased variance."""
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    return xc / np.sqrt(var + eps) * np.asarray(g, F64) + np.asarray(b, F64)


def gelu(x: np.ndarray) -> np.ndarray:
    """GELU in its exact form, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """x @ w^T + b with w in [out, in] layout."""
    return x @ np.asarray(w, F64).T + np.asarray(b, F64)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """exp(s - rowmax) / rowsum over the last axis (no special handling of inf/NaN)."""
    with np.errstate(invalid="ignore", over="ignore"):
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        return e / e.sum(axis=-1, keepdims=True)


def attention_weights(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """One head's softmax over keys of scale * q k^T: [N, M], rows summing to 1."""
    return softmax_rows((q @ k.T) * scale)


def sdpa(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, logit_format: str | None = None):
    """One head: softmax over keys of scale * q k^T, times v; q [N, c], k [M, c], v [M, c'].

    Returns (output [N, c'], max |logit|).  ``logit_format`` rounds the scaled
    logits to a float format before the softmax (fp16 overflow demonstration).
    """
    s = (q @ k.T) * scale
    smax = float(np.abs(s).max()) if s.size else 0.0
    s = to_format(s, logit_format)
    return softmax_rows(s) @ v, smax


def attention(h: np.ndarray, blk: dict, heads: int, logit_format: str | None = None,
              stats: dict | None = None) -> np.ndarray:
    """Multi-head self-attention of the LayerNormed tokens ``h`` [B, N, D].

    q, k, v = Linear(h); head j uses channels 64j .. 64j+63; per head
    S = q k^T / sqrt(64); P = softmax over keys; O = P v; heads merged back in
    channel order; output Linear.  ``logit_format`` rounds S to a float format
    before the softmax (used to show fp16 overflow); ``stats`` collects maxima.
    """
    B, N, D = h.shape
    hd = D // heads
    q = linear(h, blk["wq"], blk["bq"])
    k = linear(h, blk["wk"], blk["bk"])
    v = linear(h, blk["wv"], blk["bv"])
    o = np.empty_like(q)
    smax = 0.0
    scale = 1.0 / math.sqrt(hd)
    for bi in range(B):
        for j in range(heads):
            sl = slice(j * hd, (j + 1) * hd)
            o[bi, :, sl], m = sdpa(q[bi, :, sl], k[bi, :, sl], v[bi, :, sl], scale, logit_format)
            smax = max(smax, m)
    if stats is not None:
        _track(stats, "logits", smax)
        _track(stats, "q", np.abs(q).max())
        _track(stats, "k", np.abs(k).max())
        _track(stats, "v", np.abs(v).max())
        _track(stats, "attn_heads", np.nanmax(np.abs(o)) if np.isfinite(o).any() else float("nan"))
    return linear(o, blk["wo"], blk["bo"])


def mlp(h: np.ndarray, blk: dict, stats: dict | None = None) -> np.ndarray:
    """Linear D -> Hm, GELU, Linear Hm -> D."""
    z = linear(h, blk["w1"], blk["b1"])
    a = gelu(z)
    if stats is not None:
        _track(stats, "fc1", np.abs(z).max())
    return linear(a, blk["w2"], blk["b2"])


def block(t: np.ndarray, blk: dict, heads: int, eps: float, logit_format: str | None = None,
          stats: dict | None = None) -> np.ndarray:
    """Pre-LN encoder block: t += ls1 * Attn(LN1 t); t += ls2 * MLP(LN2 t)."""
    h1 = layer_norm(t, blk["ln1_g"], blk["ln1_b"], eps)
    a = attention(h1, blk, heads, logit_format, stats)
    t = t + np.asarray(blk["ls1"], F64) * a
    h2 = layer_norm(t, blk["ln2_g"], blk["ln2_b"], eps)
    m = mlp(h2, blk, stats)
    t = t + np.asarray(blk["ls2"], F64) * m
    if stats is not None:
        _track(stats, "ln1", np.abs(h1).max())
        _track(stats, "ln2", np.abs(h2).max())
        _track(stats, "attn_out", np.abs(a).max())
        _track(stats, "mlp_out", np.abs(m).max())
        _track(stats, "residual", np.abs(t).max())
    return t


def _track(stats: dict, name: str, value) -> None:
    """Keep the running maximum of ``value`` under ``name`` (NaN is sticky)."""
    value = float(value)
    old = stats.get(name)
    if old is None or math.isnan(value):
        stats[name] = value
    elif not math.isnan(old):
        stats[name] = max(old, value)
    if name == "logits":
        stats.setdefault("logits_per_block", []).append(value)


# ---------------------------------------------------------------------------
# whole forward pass


def descriptor(y_cls: np.ndarray, eps: float = 1e-12) -> np.ndarray:
    """CLS token of the final-LayerNormed tokens divided by max(||.||_2, eps)."""
    n = np.sqrt((y_cls * y_cls).sum(axis=-1, keepdims=True))
    return y_cls / np.maximum(n, eps)


def forward(images: np.ndarray, P: dict, cfg: dict, logit_format: str | None = None,
            stats: dict | None = None, pos: np.ndarray | None = None) -> dict:
    """Full encoder forward.

    Returns ``tokens`` [B, N, D] (final LayerNorm of every token), ``desc``
    [B, D] (L2-normalised CLS), and, if ``cfg['taps']`` lists block numbers,
    ``taps`` [B, len(taps), D, gh, gw]: after each listed block, the final
    LayerNorm of the patch tokens (CLS and registers removed) in channel-first
    grid layout.  ``pos`` overrides the stored position table (already at the
    image's grid).
    """
    x = np.asarray(images, F64)
    B, _, H, W = x.shape
    p = cfg["patch"]
    gh, gw = H // p, W // p
    R = cfg["registers"]
    eps = cfg["ln_eps"]
    emb = patch_embed(x, P["patch_w"], P["patch_b"])
    if pos is None:
        pos = P["pos"]
    t = assemble_tokens(emb, P["cls"], P["reg"], pos)
    if stats is not None:
        _track(stats, "embed", np.abs(t).max())
    taps = []
    tap_set = set(cfg.get("taps", ()))
    for li, blk in enumerate(P["blocks"]):
        t = block(t, blk, cfg["heads"], eps, logit_format, stats)
        if (li + 1) in tap_set:
            y = layer_norm(t[:, 1 + R:], P["norm_g"], P["norm_b"], eps)
            taps.append(y.reshape(B, gh, gw, -1).transpose(0, 3, 1, 2))
    y = layer_norm(t, P["norm_g"], P["norm_b"], eps)
    out = {"tokens": y, "desc": descriptor(y[:, 0])}
    if taps:
        out["taps"] = np.stack(taps, axis=1)
    return out


# ---------------------------------------------------------------------------
# resampling


def _cubic_weight(d: np.ndarray, a: float = -0.75) -> np.ndarray:
    """Cubic-convolution kernel W(d) with parameter a (Keys 1981)."""
    d = np.abs(d)
    w = np.zeros_like(d)
    near = d <= 1.0
    far = (d > 1.0) & (d < 2.0)
    w[near] = ((a + 2.0) * d[near] - (a + 3.0)) * d[near] ** 2 + 1.0
    w[far] = ((a * d[far] - 5.0 * a) * d[far] + 8.0 * a) * d[far] - 4.0 * a
    return w


def _bicubic_matrix(n_in: int, n_out: int) -> np.ndarray:
    """[n_out, n_in] matrix of one bicubic resampling pass (half-pixel centres, edge clamp)."""
    m = np.zeros((n_out, n_in), dtype=F64)
    for i in range(n_out):
        src = (i + 0.5) * n_in / n_out - 0.5
        x0 = math.floor(src)
        for tap in range(-1, 3):
            xi = x0 + tap
            wgt = float(_cubic_weight(np.array([src - xi]))[0])
            m[i, min(max(xi, 0), n_in - 1)] += wgt
    return m


def bicubic_resize(x: np.ndarray, out_h: int, out_w: int) -> np.ndarray:
    """Bicubic resampling of [C, h, w] to [C, out_h, out_w] (separable, rows then cols)."""
    C, h, w = x.shape
    my = _bicubic_matrix(h, out_h)
    mx = _bicubic_matrix(w, out_w)
    return np.einsum("yh,chw,xw->cyx", my, np.asarray(x, F64), mx, optimize=True)


def resample_pos(pos: np.ndarray, grid_from: tuple[int, int], grid_to: tuple[int, int]) -> np.ndarray:
    """Position table at ``grid_from`` -> ``grid_to``: CLS row kept, patch rows bicubic.

    The LibreYOLO diagram shows a "Bicubic interpolation" step on the position
    embedding ("37x37 unchanged" at the native grid).
    """
    gh, gw = grid_from
    th, tw = grid_to
    pos = np.asarray(pos, F64)
    D = pos.shape[1]
    g = pos[1:].reshape(gh, gw, D).transpose(2, 0, 1)
    r = bicubic_resize(g, th, tw).transpose(1, 2, 0).reshape(th * tw, D)
    return np.concatenate([pos[:1], r], axis=0)


def _bilinear_axis(n_in: int, n_out: int):
    """Source indices and weights of one bilinear pass (half-pixel centres, align_corners=False)."""
    i0 = np.empty(n_out, dtype=np.int64)
    i1 = np.empty(n_out, dtype=np.int64)
    lam = np.empty(n_out, dtype=F64)
    for i in range(n_out):
        src = max((i + 0.5) * n_in / n_out - 0.5, 0.0)
        x0 = min(int(math.floor(src)), n_in - 1)
        i0[i] = x0
        i1[i] = min(x0 + 1, n_in - 1)
        lam[i] = src - x0
    return i0, i1, lam


def bilinear_resize(x: np.ndarray, out_h: int, out_w: int) -> np.ndarray:
    """Bilinear resampling of [C, h, w] to [C, out_h, out_w] (align_corners=False)."""
    C, h, w = x.shape
    y0, y1, ly = _bilinear_axis(h, out_h)
    x0, x1, lx = _bilinear_axis(w, out_w)
    x = np.asarray(x, F64)
    rows = x[:, y0, :] * (1.0 - ly)[None, :, None] + x[:, y1, :] * ly[None, :, None]
    return rows[:, :, x0] * (1.0 - lx)[None, None, :] + rows[:, :, x1] * lx[None, None, :]


# ---------------------------------------------------------------------------
# frame preprocessing (the step right before the encoder)

IMAGENET_MEAN = (0.485, 0.456, 0.406)  # RGB; model card, "Model I/O"
IMAGENET_STD = (0.229, 0.224, 0.225)


def preprocess(frames: np.ndarray, out_h: int, out_w: int, bgr: bool = False) -> np.ndarray:
    """8-bit HWC frames [B, h, w, 3] -> ImageNet-normalised CHW images [B, 3, out_h, out_w].

    The deployment article's service decodes a frame (BGR), converts it to RGB
    and resizes it with cv2's default bilinear interpolation (half-pixel
    centres, edges clamped); the model card fixes the input as ImageNet-
    normalised RGB CHW with mean (0.485, 0.456, 0.406) and std (0.229, 0.224,
    0.225), with the 8-bit values scaled by 1/255.  Reading: the resize is the
    exact bilinear resampling of the 8-bit values, without rounding back to 8
    bits in between.
    """
    f = np.asarray(frames)
    if f.ndim != 4 or f.shape[-1] != 3 or f.dtype != np.uint8:
        raise ValueError("frames must be uint8 [B, h, w, 3]")
    if bgr:
        f = f[..., ::-1]
    mean = np.asarray(IMAGENET_MEAN, F64)[:, None, None]
    std = np.asarray(IMAGENET_STD, F64)[:, None, None]
    out = np.empty((f.shape[0], 3, out_h, out_w), dtype=F64)
    for i in range(f.shape[0]):
        chw = np.asarray(f[i], F64).transpose(2, 0, 1)
        out[i] = (bilinear_resize(chw, out_h, out_w) / 255.0 - mean) / std
    return out


# ---------------------------------------------------------------------------
# zero-shot patch-text scoring


def patch_features(images: np.ndarray, P: dict, cfg: dict, pos: np.ndarray | None = None) -> np.ndarray:
    """L2-normalised patch tokens [B, gh, gw, D] after all blocks and the final LayerNorm."""
    out = forward(images, P, cfg, pos=pos)
    B, _, H, W = images.shape
    p = cfg["patch"]
    f = out["tokens"][:, 1 + cfg["registers"]:]
    f = f / np.maximum(np.sqrt((f * f).sum(axis=-1, keepdims=True)), 1e-12)
    return f.reshape(B, H // p, W // p, -1)


def cosine_maps(feats: np.ndarray, class_emb: np.ndarray) -> np.ndarray:
    """cos[c, y, x] = class_emb[c] . feats[y, x] for one image's features [gh, gw, D]."""
    gh, gw, D = feats.shape
    return (np.asarray(class_emb, F64) @ feats.reshape(gh * gw, D).T).reshape(-1, gh, gw)


def scores_whole(image: np.ndarray, P: dict, cfg: dict, class_emb: np.ndarray) -> dict:
    """Whole mode: one forward; cosine maps upsampled to the image size; argmax over classes."""
    x = np.asarray(image, F64)[None]
    H, W = x.shape[2:]
    f = patch_features(x, P, cfg)[0]
    cos = cosine_maps(f, class_emb)
    up = bilinear_resize(cos, H, W)
    return {"cos": cos, "scores": up, "labels": up.argmax(axis=0)}


def slide_windows(img_h: int, img_w: int, side: int, stride: int) -> list[tuple[int, int]]:
    """Top-left corners of the slide-mode windows.

    Along each axis, ceil((n - side) / stride) + 1 windows start every
    ``stride`` pixels; the last one is moved back so that it ends at the
    border.  512 x 1024 with side 384 / stride 192 gives 2 x 5 = 10 windows.
    """
    def starts(n):
        count = max(-(-(n - side) // stride), 0) + 1
        out = []
        for i in range(count):
            end = min(i * stride + side, n)
            out.append(max(end - side, 0))
        return out
    return [(y, x) for y in starts(img_h) for x in starts(img_w)]


def scores_slide(image: np.ndarray, P: dict, cfg: dict, class_emb: np.ndarray) -> dict:
    """Slide mode: per window, cosine maps upsampled to the window, softmax over
    classes, accumulated into the image with overlap counts; average; argmax."""
    x = np.asarray(image, F64)
    _, H, W = x.shape
    side, stride = cfg["window"], cfg["window_stride"]
    p = cfg["patch"]
    wins = slide_windows(H, W, side, stride)
    pos_w = resample_pos(P["pos"], cfg["pos_grid"], (side // p, side // p))
    crops = np.stack([x[:, y:y + side, c:c + side] for (y, c) in wins])
    feats = patch_features(crops, P, cfg, pos=pos_w)
    C = class_emb.shape[0]
    probs = np.zeros((C, H, W), dtype=F64)
    counts = np.zeros((H, W), dtype=F64)
    cos_all = []
    for wi, (y, c) in enumerate(wins):
        cos = cosine_maps(feats[wi], class_emb)
        cos_all.append(cos)
        up = bilinear_resize(cos, side, side)
        probs[:, y:y + side, c:c + side] += softmax_rows(up.transpose(1, 2, 0)).transpose(2, 0, 1)
        counts[y:y + side, c:c + side] += 1.0
    probs /= counts
    return {"probs": probs, "counts": counts, "labels": probs.argmax(axis=0), "windows": wins,
            "cos": np.stack(cos_all)}
