"""Pins of the semantic-head oracle (CPU only).

Each oracle function is checked against something other than itself: float64
PyTorch library routines (conv2d, layer_norm, group_norm, silu, interpolate),
closed forms, and a torch.nn module of the whole head written separately from
the LibreYOLO DINOv2 diagram ("Projector P4", "Projector Bottleneck",
"Projector output ConvX", "Task head").
"""

import numpy as np
import pytest
import torch
import torch.nn as nn
import torch.nn.functional as F

import synth
from oracle import head_oracle as H


RNG = np.random.default_rng(77)


def t64(a):
    return torch.from_numpy(np.asarray(a, np.float64))


@pytest.mark.parametrize("k,pad,bias", [(1, 0, False), (1, 0, True), (3, 1, False), (3, 1, True), (3, 0, True)])
def test_conv2d_matches_torch(k, pad, bias):
    x = RNG.standard_normal((5, 7, 6))
    w = RNG.standard_normal((4, 5, k, k))
    b = RNG.standard_normal(4) if bias else None
    got = H.conv2d(x, w, b, pad)
    ref = F.conv2d(t64(x)[None], t64(w), None if b is None else t64(b), padding=pad)[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_conv2d_brute_force_3x3_padding():
    # one output pixel at a corner, summed by hand: the zero padding drops row/col -1
    x = RNG.standard_normal((2, 4, 4))
    w = RNG.standard_normal((1, 2, 3, 3))
    out = H.conv2d(x, w, None, 1)
    s = sum(w[0, c, ky, kx] * x[c, ky - 1, kx - 1] for c in range(2) for ky in range(1, 3) for kx in range(1, 3))
    assert out[0, 0, 0] == pytest.approx(s, rel=1e-12)


def test_channel_layer_norm_matches_torch_and_invariant():
    x = RNG.standard_normal((12, 5, 4)) * 3 + 1
    g, b = RNG.standard_normal(12), RNG.standard_normal(12)
    got = H.channel_layer_norm(x, g, b, 1e-6)
    ref = F.layer_norm(t64(x).permute(1, 2, 0), (12,), t64(g), t64(b), 1e-6).permute(2, 0, 1).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # unit affine: every pixel's channels have mean 0 and variance var / (var + eps)
    y = H.channel_layer_norm(x, np.ones(12), np.zeros(12), 1e-6)
    var = x.var(axis=0)
    np.testing.assert_allclose(y.mean(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=0), var / (var + 1e-6), rtol=1e-12)


def test_group_norm_matches_torch():
    x = RNG.standard_normal((64, 5, 6)) * 2 - 0.5
    g, b = RNG.standard_normal(64), RNG.standard_normal(64)
    got = H.group_norm(x, 32, g, b, 1e-5)
    ref = F.group_norm(t64(x)[None], 32, t64(g), t64(b), 1e-5)[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_silu_closed_forms_and_torch():
    x = np.array([-30.0, -1.0, 0.0, 0.5, 30.0])
    got = H.silu(x)
    np.testing.assert_allclose(got, F.silu(t64(x)).numpy(), rtol=1e-14, atol=1e-300)
    assert got[2] == 0.0
    assert got[4] == pytest.approx(30.0, rel=1e-12)       # -> x for large x
    assert got[1] == pytest.approx(-1.0 / (1.0 + np.e), rel=1e-14)


# ------------------------------------------------------------------ torch.nn restatement of the diagram

class ChannelLN(nn.Module):
    def __init__(self, c, eps):
        super().__init__()
        self.ln = nn.LayerNorm(c, eps=eps)

    def forward(self, x):  # [B, C, H, W]
        return self.ln(x.permute(0, 2, 3, 1)).permute(0, 3, 1, 2)


class ConvX(nn.Module):
    def __init__(self, cin, cout, k):
        super().__init__()
        self.conv = nn.Conv2d(cin, cout, k, padding=k // 2, bias=False)
        self.norm = ChannelLN(cout, 1e-6)
        self.act = nn.SiLU()

    def forward(self, x):
        return self.act(self.norm(self.conv(x)))


class Bottleneck(nn.Module):
    def __init__(self, c):
        super().__init__()
        self.cv1 = ConvX(c, c, 3)
        self.cv2 = ConvX(c, c, 3)

    def forward(self, x):
        return self.cv2(self.cv1(x))   # no shortcut


class SemanticHead(nn.Module):
    def __init__(self, cin, width=256, classes=19):
        super().__init__()
        self.stem = ConvX(cin, width, 1)
        self.m = nn.ModuleList(Bottleneck(width // 2) for _ in range(3))
        self.out = ConvX(5 * (width // 2), width, 1)
        self.final = ChannelLN(width, 1e-6)
        self.lateral = nn.Conv2d(width, width, 1, bias=True)
        self.smooth = nn.Conv2d(width, width, 3, padding=1, bias=True)
        self.gn = nn.GroupNorm(32, width, eps=1e-5)
        self.gelu = nn.GELU()
        self.drop = nn.Dropout2d(0.1)
        self.pred = nn.Conv2d(width, classes, 1, bias=True)

    def forward(self, taps, size):
        x = torch.cat(list(taps.unbind(1)), dim=1)            # [B, 4D, gh, gw], tap 3 first
        y = list(self.stem(x).chunk(2, dim=1))                 # a, b
        for blk in self.m:
            y.append(blk(y[-1]))
        p4 = self.final(self.out(torch.cat(y, dim=1)))
        z = self.pred(self.drop(self.gelu(self.gn(self.smooth(self.lateral(p4))))))
        return p4, z, F.interpolate(z, size=size, mode="bilinear", align_corners=False)


def load(module, Ph):
    sd = {
        "stem.conv.weight": Ph["proj_w"], "stem.norm.ln.weight": Ph["proj_ln_g"], "stem.norm.ln.bias": Ph["proj_ln_b"],
        "out.conv.weight": Ph["out_w"], "out.norm.ln.weight": Ph["out_ln_g"], "out.norm.ln.bias": Ph["out_ln_b"],
        "final.ln.weight": Ph["final_ln_g"], "final.ln.bias": Ph["final_ln_b"],
        "lateral.weight": Ph["lat_w"], "lateral.bias": Ph["lat_b"],
        "smooth.weight": Ph["smooth_w"], "smooth.bias": Ph["smooth_b"],
        "gn.weight": Ph["gn_g"], "gn.bias": Ph["gn_b"],
        "pred.weight": Ph["pred_w"], "pred.bias": Ph["pred_b"],
    }
    for i in range(3):
        for j in (1, 2):
            sd[f"m.{i}.cv{j}.conv.weight"] = Ph[f"bn{i + 1}_w{j}"]
            sd[f"m.{i}.cv{j}.norm.ln.weight"] = Ph[f"bn{i + 1}_ln{j}_g"]
            sd[f"m.{i}.cv{j}.norm.ln.bias"] = Ph[f"bn{i + 1}_ln{j}_b"]
    module.load_state_dict({k: t64(v) for k, v in sd.items()})


@pytest.mark.parametrize("gh,gw,out", [(6, 5, (84, 70)), (9, 9, (126, 126))])
def test_head_matches_torch_module(gh, gw, out):
    cfg = synth.preset("vits14_518")
    Ph = synth.make_head_params(cfg)
    taps = synth.make_taps(cfg, 2, gh=gh, gw=gw)
    m = SemanticHead(4 * cfg["dim"]).double().eval()
    load(m, Ph)
    with torch.no_grad():
        p4, z, logits = m(t64(taps), out)
    for b in range(2):
        r = H.semantic_head(taps[b], Ph, *out)
        np.testing.assert_allclose(r["p4"], p4[b].numpy(), rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(r["grid"], z[b].numpy(), rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(r["logits"], logits[b].numpy(), rtol=1e-10, atol=1e-10)


def test_head_shapes_from_the_diagram():
    # cfg3 grid 37 x 37: the C2f concat has 640 channels, P4 is 256 x 37 x 37,
    # the logits 19 x 518 x 518 ("Size equivalence", "Task head")
    cfg = synth.preset("vits14_518")
    Ph = synth.make_head_params(cfg)
    taps = synth.make_taps(cfg, 1)
    assert taps.shape == (1, 4, 384, 37, 37)
    stats = {}
    p4 = H.projector(taps[0], Ph, stats)
    assert stats["c2f_concat"].shape == (640, 37, 37)
    assert p4.shape == (256, 37, 37)
    r = H.semantic_head(taps[0], Ph, 518, 518)
    assert r["grid"].shape == (19, 37, 37) and r["logits"].shape == (19, 518, 518)


def test_zero_bottleneck_weights_give_constant_channels():
    # with zero conv weights a ConvX unit outputs SiLU(beta) at every pixel, so the
    # third Bottleneck's channels are the closed form silu(bn3_ln2_b)
    cfg = synth.preset("vits14_518")
    Ph = dict(synth.make_head_params(cfg))
    for i in (1, 2, 3):
        Ph[f"bn{i}_w1"] = np.zeros_like(Ph[f"bn{i}_w1"])
        Ph[f"bn{i}_w2"] = np.zeros_like(Ph[f"bn{i}_w2"])
    taps = synth.make_taps(cfg, 1, gh=4, gw=4)
    stats = {}
    H.projector(taps[0], Ph, stats)
    cat = stats["c2f_concat"]
    b3 = Ph["bn3_ln2_b"].astype(np.float64)
    expect = b3 / (1.0 + np.exp(-b3))
    np.testing.assert_allclose(cat[512:640], np.broadcast_to(expect[:, None, None], (128, 4, 4)), rtol=1e-12)
