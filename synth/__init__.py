"""Seeded synthetic inputs for the ViT encoder forward pass.

This module draws random numbers and lays them out under fixed names.  It holds
none of the encoder's arithmetic: both the CPU oracle (via the tests) and the
GPU library (via its Python binding) receive exactly the arrays produced here.

Workload presets describe the five benchmark configurations:

* ``vits16_224``  - ViT-S/16 DINOv3-style at 224x224 (1 CLS + 4 registers + 196
  patches = 201 tokens), fp32 weights, batch 1.
* ``vits16_336``  - ViT-S/16 at 336x336 (21x21 = 441 patches, 446 tokens),
  bf16-representable weights, batches 1 and 32, with the register-key attention
  sink that drives block-1 logits to about 2.5e6 (the DINOv3 model card, section
  "Build BF16, not FP16").
* ``vits14_518``  - DINOv2-S/14 at 518x518 (37x37 = 1369 patches + CLS = 1370
  tokens, no registers), batch 8, LayerNormed patch taps after blocks 3/6/9/12
  (the LibreYOLO DINOv2 diagram, "Tap stage" boxes).
* ``vitl16_1024`` - ViT-L/16 at 1024x1024 (4096 patches + 5 = 4101 tokens),
  batches 1 and 4.
* ``vitl16_text`` - ViT-L/16 plus 2 extra blocks, 512x1024 image, 150 class
  embeddings, whole and slide (384 window, 192 stride) scoring (the dino.txt
  zero-shot segmentation article, "whole" / "slide" section).

Parameter distributions: every Linear/conv weight and bias, the CLS token, the
registers and the position table are N(0, 0.02); LayerNorm gamma = 1 + N(0, 0.02)
and beta = N(0, 0.02); LayerScale is a constant (1e-5 unless overridden).  Images
are N(0, 1).  All draws use NumPy's PCG64 ``default_rng(seed)`` in the fixed order
documented in :func:`make_params`.
"""

from __future__ import annotations

import copy
import math

import numpy as np

__all__ = [
    "PRESETS",
    "preset",
    "tokens",
    "grid",
    "make_params",
    "make_images",
    "make_class_embeddings",
    "make_head_params",
    "make_taps",
    "round_bf16",
]

# Workload presets.  Keys mirror the C-ABI's vit_config fields.
PRESETS = {
    "vits16_224": dict(
        cfg_id=1, img_h=224, img_w=224, patch=16, dim=384, depth=12, extra_blocks=0,
        heads=6, mlp_hidden=1536, registers=4, ln_eps=1e-6, taps=(), window=0,
        window_stride=0, classes=0, bf16_params=False, sink=False, layerscale=1e-5,
        batches=(1,), seed=1001),
    "vits16_336": dict(
        cfg_id=2, img_h=336, img_w=336, patch=16, dim=384, depth=12, extra_blocks=0,
        heads=6, mlp_hidden=1536, registers=4, ln_eps=1e-6, taps=(), window=0,
        window_stride=0, classes=0, bf16_params=True, sink=True, layerscale=1e-5,
        batches=(1, 32), seed=1002),
    "vits14_518": dict(
        cfg_id=3, img_h=518, img_w=518, patch=14, dim=384, depth=12, extra_blocks=0,
        heads=6, mlp_hidden=1536, registers=0, ln_eps=1e-6, taps=(3, 6, 9, 12), window=0,
        window_stride=0, classes=0, bf16_params=True, sink=False, layerscale=1e-5,
        batches=(8,), seed=1003),
    "vitl16_1024": dict(
        cfg_id=4, img_h=1024, img_w=1024, patch=16, dim=1024, depth=24, extra_blocks=0,
        heads=16, mlp_hidden=4096, registers=4, ln_eps=1e-6, taps=(), window=0,
        window_stride=0, classes=0, bf16_params=True, sink=False, layerscale=1e-5,
        batches=(1, 4), seed=1004),
    "vitl16_text": dict(
        cfg_id=5, img_h=512, img_w=1024, patch=16, dim=1024, depth=24, extra_blocks=2,
        heads=16, mlp_hidden=4096, registers=4, ln_eps=1e-6, taps=(), window=384,
        window_stride=192, classes=150, bf16_params=True, sink=False, layerscale=1e-5,
        batches=(1,), seed=1005),
}

IMAGE_SEED_BASE = 2000
CLASS_SEED = 3000
SINK_SEED = 4000
HEAD_SEED = 5000
TAPS_SEED = 6000

# LibreYOLO DINOv2 semantic head (the diagram's "Projector P4" and "Task head")
HEAD = dict(width=256, half=128, bottlenecks=3, classes=19, taps=4)


def preset(name: str, **overrides) -> dict:
    """A copy of a preset with fields overridden (e.g. a smaller image or depth)."""
    cfg = copy.deepcopy(PRESETS[name])
    cfg["name"] = name
    cfg.update(overrides)
    cfg.setdefault("pos_grid", grid(cfg))
    return cfg


def grid(cfg: dict, img_h: int | None = None, img_w: int | None = None) -> tuple[int, int]:
    """Patch grid (rows, cols) of an image of the given (default: the preset's) size."""
    h = cfg["img_h"] if img_h is None else img_h
    w = cfg["img_w"] if img_w is None else img_w
    return h // cfg["patch"], w // cfg["patch"]


def tokens(cfg: dict, img_h: int | None = None, img_w: int | None = None) -> int:
    """Sequence length: patches + 1 CLS + registers."""
    gh, gw = grid(cfg, img_h, img_w)
    return gh * gw + 1 + cfg["registers"]


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept in float32.

    Used only to make stored parameters exactly representable in bf16 for the
    workloads whose weights are bf16.
    """
    a = np.array(a, dtype=np.float32, copy=True, order="C")
    if not np.isfinite(a).all():
        raise ValueError("round_bf16 expects finite values")
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return a


BLOCK_KEYS = ("ln1_g", "ln1_b", "wq", "bq", "wk", "bk", "wv", "bv", "wo", "bo", "ls1",
              "ln2_g", "ln2_b", "w1", "b1", "w2", "b2", "ls2")


def make_params(cfg: dict, seed: int | None = None) -> dict:
    """Random parameters for ``cfg``.

    Draw order (one PCG64 stream): patch_w [D,3,p,p], patch_b [D], cls [D],
    reg [R,D], pos [1+gh*gw, D] at ``cfg['pos_grid']``, then per block
    ln1_g, ln1_b, wq [D,D], bq, wk, bk, wv, bv, wo, bo, ln2_g, ln2_b,
    w1 [Hm,D], b1 [Hm], w2 [D,Hm], b2, then norm_g, norm_b.  Linear weights use
    the [out, in] layout.  LayerScale vectors are constants and draw nothing.
    """
    D, p, R, Hm = cfg["dim"], cfg["patch"], cfg["registers"], cfg["mlp_hidden"]
    gh, gw = cfg.get("pos_grid") or grid(cfg)
    rng = np.random.default_rng(cfg["seed"] if seed is None else seed)
    sd = np.float32(0.02)

    def normal(*shape):
        return rng.standard_normal(shape, dtype=np.float32) * sd

    def gamma(n):
        return np.float32(1.0) + normal(n)

    P = {}
    P["patch_w"] = normal(D, 3, p, p)
    P["patch_b"] = normal(D)
    P["cls"] = normal(D)
    P["reg"] = normal(R, D)
    P["pos"] = normal(1 + gh * gw, D)
    ls = np.full(D, cfg["layerscale"], dtype=np.float32)
    blocks = []
    for _ in range(cfg["depth"] + cfg["extra_blocks"]):
        b = {}
        b["ln1_g"] = gamma(D)
        b["ln1_b"] = normal(D)
        b["wq"] = normal(D, D)
        b["bq"] = normal(D)
        b["wk"] = normal(D, D)
        b["bk"] = normal(D)
        b["wv"] = normal(D, D)
        b["bv"] = normal(D)
        b["wo"] = normal(D, D)
        b["bo"] = normal(D)
        b["ls1"] = ls.copy()
        b["ln2_g"] = gamma(D)
        b["ln2_b"] = normal(D)
        b["w1"] = normal(Hm, D)
        b["b1"] = normal(Hm)
        b["w2"] = normal(D, Hm)
        b["b2"] = normal(D)
        b["ls2"] = ls.copy()
        blocks.append(b)
    P["blocks"] = blocks
    P["norm_g"] = gamma(D)
    P["norm_b"] = normal(D)

    if cfg.get("sink"):
        _plant_sink(cfg, P)
    if cfg.get("bf16_params"):
        P = _map_arrays(P, round_bf16)
    return P


def _map_arrays(P, fn):
    out = {}
    for k, v in P.items():
        if k == "blocks":
            out[k] = [{kk: fn(vv) for kk, vv in b.items()} for b in v]
        elif k.startswith("_"):
            out[k] = v
        else:
            out[k] = fn(v)
    return out


SINK_LOGIT = 2.5e6


def _plant_sink(cfg: dict, P: dict) -> None:
    """Give block 1, head 0 one key (register 0, token 1) whose logit is ~2.5e6.

    The DINOv3 model card (section "Build BF16, not FP16") reports scaled Q.K^T
    logits of 2.1e6-2.5e6 in the first block, absorbed by a register token,
    while every other tensor stays below 1800.  Random N(0, 0.02) weights give
    logits of order 0.1, so the sink is planted through parameters only:

    * a seeded sign vector e in {-1,+1}^64 and a seeded channel c*;
    * query bias of head 0 = a * e, so every query of head 0 is ~ a * e;
    * register 0 gets +1.0 added at channel c*; its LayerNorm output there is
      then about r* = sqrt(D / (1 + D * 0.02^2)) (the spike dominates the
      row variance);
    * key weight column c* of head 0 = (a / r*) * e, so register 0's key is
      ~ a * e and its scaled logit is ~ 64 a^2 / 8 = 8 a^2;
    * a = sqrt(2.5e6 / 8) * (1 + 0.05 u), u ~ U(-1, 1) the seeded factor.

    Other keys pick up z * (a / r*) * e with |z| the LayerNorm output of an
    ordinary token at c* (a few units), so the sink dominates by >1e6 and the
    softmax of head 0 in block 1 is one-hot on register 0 in any float format
    that does not overflow.
    """
    assert cfg["registers"] >= 1 and cfg["dim"] % 64 == 0
    D = cfg["dim"]
    rng = np.random.default_rng(SINK_SEED)
    e = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=64)
    c_star = int(rng.integers(0, D))
    u = float(rng.uniform(-1.0, 1.0))
    a = math.sqrt(SINK_LOGIT / 8.0) * (1.0 + 0.05 * u)
    r_star = math.sqrt(D / (1.0 + D * 0.02 * 0.02))
    blk = P["blocks"][0]
    blk["bq"][:64] = np.float32(a) * e
    P["reg"][0, c_star] += np.float32(1.0)
    blk["wk"][:64, c_star] = np.float32(a / r_star) * e
    P["_sink"] = dict(channel=c_star, a=a, r_star=r_star)


def make_images(cfg: dict, batch: int, seed: int | None = None,
                img_h: int | None = None, img_w: int | None = None) -> np.ndarray:
    """Images [batch, 3, H, W] float32 ~ N(0, 1) (stand-ins for ImageNet-normalised frames)."""
    h = cfg["img_h"] if img_h is None else img_h
    w = cfg["img_w"] if img_w is None else img_w
    s = IMAGE_SEED_BASE + cfg["cfg_id"] if seed is None else seed
    rng = np.random.default_rng(s)
    return rng.standard_normal((batch, 3, h, w), dtype=np.float32)


def make_class_embeddings(cfg: dict, classes: int | None = None, seed: int = CLASS_SEED) -> np.ndarray:
    """Class embeddings [C, D]: seeded Gaussian directions scaled to unit length.

    They stand in for the averaged, normalised text features of the dino.txt
    article (150 ADE20K classes); with bf16 parameters the stored values are
    rounded to bf16 after scaling, so their norms are 1 to within 2^-8.
    """
    C = cfg["classes"] if classes is None else classes
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((C, cfg["dim"])).astype(np.float64)
    g /= np.sqrt((g * g).sum(axis=1, keepdims=True))
    g = g.astype(np.float32)
    return round_bf16(g) if cfg.get("bf16_params") else g


def make_head_params(cfg: dict, seed: int = HEAD_SEED, classes: int | None = None) -> dict:
    """Random parameters of the semantic head on the taps of ``cfg`` (conv weights in
    the [out, in, kh, kw] layout of torch.nn.Conv2d).

    Draw order (one PCG64 stream): proj_w [256, 4D, 1, 1], proj_ln_g, proj_ln_b; for
    Bottleneck i = 1..3: bn{i}_w1 [128, 128, 3, 3], bn{i}_ln1_g, bn{i}_ln1_b,
    bn{i}_w2, bn{i}_ln2_g, bn{i}_ln2_b; out_w [256, 640, 1, 1], out_ln_g, out_ln_b,
    final_ln_g, final_ln_b; lat_w [256, 256, 1, 1], lat_b; smooth_w [256, 256, 3, 3],
    smooth_b; gn_g, gn_b; pred_w [C, 256, 1, 1], pred_b.  Weights and biases are
    N(0, 0.02), norm scales 1 + N(0, 0.02), norm shifts N(0, 0.02); rounded to bf16
    when the encoder's parameters are.
    """
    D = cfg["dim"]
    W, Hf, C = HEAD["width"], HEAD["half"], HEAD["classes"] if classes is None else classes
    rng = np.random.default_rng(seed)
    sd = np.float32(0.02)

    def normal(*shape):
        return rng.standard_normal(shape, dtype=np.float32) * sd

    def gamma(n):
        return np.float32(1.0) + normal(n)

    P = {}
    P["proj_w"] = normal(W, HEAD["taps"] * D, 1, 1)
    P["proj_ln_g"], P["proj_ln_b"] = gamma(W), normal(W)
    for i in range(1, HEAD["bottlenecks"] + 1):
        P[f"bn{i}_w1"] = normal(Hf, Hf, 3, 3)
        P[f"bn{i}_ln1_g"], P[f"bn{i}_ln1_b"] = gamma(Hf), normal(Hf)
        P[f"bn{i}_w2"] = normal(Hf, Hf, 3, 3)
        P[f"bn{i}_ln2_g"], P[f"bn{i}_ln2_b"] = gamma(Hf), normal(Hf)
    P["out_w"] = normal(W, (2 + HEAD["bottlenecks"]) * Hf, 1, 1)
    P["out_ln_g"], P["out_ln_b"] = gamma(W), normal(W)
    P["final_ln_g"], P["final_ln_b"] = gamma(W), normal(W)
    P["lat_w"], P["lat_b"] = normal(W, W, 1, 1), normal(W)
    P["smooth_w"], P["smooth_b"] = normal(W, W, 3, 3), normal(W)
    P["gn_g"], P["gn_b"] = gamma(W), normal(W)
    P["pred_w"], P["pred_b"] = normal(C, W, 1, 1), normal(C)
    if cfg.get("bf16_params"):
        P = {k: round_bf16(v) for k, v in P.items()}
    return P


def make_taps(cfg: dict, batch: int, seed: int = TAPS_SEED, gh: int | None = None, gw: int | None = None) -> np.ndarray:
    """Stand-in taps [batch, 4, D, gh, gw] float32 ~ N(0, 1) (LayerNormed features are
    of unit scale), for testing the head apart from the encoder."""
    g = grid(cfg)
    gh = g[0] if gh is None else gh
    gw = g[1] if gw is None else gw
    rng = np.random.default_rng(seed)
    return rng.standard_normal((batch, HEAD["taps"], cfg["dim"], gh, gw), dtype=np.float32)
