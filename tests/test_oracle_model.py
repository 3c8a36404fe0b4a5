"""Pins for the oracle's whole forward pass.

* shapes and counts the pages print (``tests/golden/page_facts.json``);
* a float64 torch.nn reference model (Conv2d, LayerNorm, MultiheadAttention,
  Linear, GELU modules) on a small configuration;
* closed forms (LayerScale = 0), invariants (descriptor norm, batch
  independence, tap 12 = final tokens) and the fp16 overflow demonstration on
  the ViT-S/16 @336 sink workload.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import vit_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def small_cfg(**kw):
    base = dict(img_h=48, img_w=32, dim=128, depth=2, heads=2, mlp_hidden=512, registers=4,
                layerscale=0.5, bf16_params=False, sink=False, taps=(), seed=77)
    base.update(kw)
    return synth.preset("vits16_224", **base)


# --------------------------------------------------------------------- page facts

def test_token_counts_from_pages():
    f = FACTS["vits16_336_input"]
    cfg = synth.preset("vits16_336")
    assert (cfg["img_h"], cfg["img_w"]) == tuple(f["value"][2:])
    assert synth.grid(cfg) == (f["grid_side"], f["grid_side"])
    assert cfg["registers"] == FACTS["vits16_registers"]["value"]
    assert synth.tokens(cfg) == 21 * 21 + 1 + 4 == 446
    d2 = FACTS["dinov2_s14_518"]
    cfg3 = synth.preset("vits14_518")
    assert synth.grid(cfg3) == tuple(d2["patch_grid"])
    assert synth.tokens(cfg3) == d2["tokens"] == d2["patches"] + 1
    assert cfg3["dim"] == d2["dim"] and cfg3["heads"] == d2["heads"]
    assert cfg3["dim"] // cfg3["heads"] == d2["head_dim"] == 64
    assert cfg3["mlp_hidden"] == d2["mlp_hidden"] and cfg3["depth"] == d2["blocks"]
    assert tuple(cfg3["taps"]) == tuple(d2["tap_blocks"])
    assert cfg3["ln_eps"] == d2["ln_eps"] and cfg3["registers"] == d2["registers"]
    # ViT-L/16: 16 heads of 64 channels
    cfg4 = synth.preset("vitl16_1024")
    assert cfg4["dim"] // cfg4["heads"] == 64 and cfg4["heads"] == FACTS["model_sizes"]["ViT-L/14"]["heads"]
    assert synth.tokens(cfg4) == 4101
    cfg5 = synth.preset("vitl16_text")
    assert synth.tokens(cfg5) == 32 * 64 + 5 == 2053
    assert synth.tokens(cfg5, 384, 384) == 24 * 24 + 5 == 581
    assert cfg5["extra_blocks"] == FACTS["dinotxt_slide"]["extra_blocks"]


def _param_count(D, depth, Hm, p, npos, R):
    per_block = 4 * (D * D + D) + (Hm * D + Hm) + (D * Hm + D) + 4 * D + 2 * D
    return D * 3 * p * p + D + D + R * D + npos * D + depth * per_block + 2 * D


def test_parameter_counts_match_model_table():
    # the architecture (4 DxD projections + DxHm + HmxD per block) reproduces the
    # printed parameter counts to within their rounding
    for name, (D, depth) in {"ViT-S/14": (384, 12), "ViT-B/14": (768, 12),
                             "ViT-L/14": (1024, 24), "ViT-G/14": (1536, 40)}.items():
        row = FACTS["model_sizes"][name]
        assert (row["dim"], row["depth"]) == (D, depth)
        n = _param_count(D, depth, 4 * D, 14, 1370, 0)
        assert abs(n / 1e6 - row["params_millions"]) / row["params_millions"] < 0.06, (name, n)


def test_param_shapes_from_generator():
    cfg = synth.preset("vits14_518")
    P = synth.make_params(cfg)
    assert P["pos"].shape == (1370, 384)
    assert P["patch_w"].shape == (384, 3, 14, 14)
    blk = P["blocks"][0]
    assert blk["w1"].shape == (1536, 384) and blk["w2"].shape == (384, 1536)
    assert len(P["blocks"]) == 12 and P["reg"].shape == (0, 384)


# --------------------------------------------------------------------- torch.nn reference

class TorchViT(torch.nn.Module):
    """float64 reference assembled from torch.nn library modules."""

    def __init__(self, cfg, P):
        super().__init__()
        D, p, H = cfg["dim"], cfg["patch"], cfg["heads"]
        dt = torch.float64
        self.cfg = cfg
        self.conv = torch.nn.Conv2d(3, D, p, stride=p, dtype=dt)
        self.P = P
        self.blocks = torch.nn.ModuleList()
        with torch.no_grad():
            self.conv.weight.copy_(t64(P["patch_w"]))
            self.conv.bias.copy_(t64(P["patch_b"]))
            for b in P["blocks"]:
                m = torch.nn.ModuleDict(dict(
                    ln1=torch.nn.LayerNorm(D, eps=cfg["ln_eps"], dtype=dt),
                    attn=torch.nn.MultiheadAttention(D, H, bias=True, batch_first=True, dtype=dt),
                    ln2=torch.nn.LayerNorm(D, eps=cfg["ln_eps"], dtype=dt),
                    fc1=torch.nn.Linear(D, cfg["mlp_hidden"], dtype=dt),
                    fc2=torch.nn.Linear(cfg["mlp_hidden"], D, dtype=dt)))
                m["ln1"].weight.copy_(t64(b["ln1_g"])); m["ln1"].bias.copy_(t64(b["ln1_b"]))
                m["ln2"].weight.copy_(t64(b["ln2_g"])); m["ln2"].bias.copy_(t64(b["ln2_b"]))
                m["attn"].in_proj_weight.copy_(t64(np.concatenate([b["wq"], b["wk"], b["wv"]])))
                m["attn"].in_proj_bias.copy_(t64(np.concatenate([b["bq"], b["bk"], b["bv"]])))
                m["attn"].out_proj.weight.copy_(t64(b["wo"])); m["attn"].out_proj.bias.copy_(t64(b["bo"]))
                m["fc1"].weight.copy_(t64(b["w1"])); m["fc1"].bias.copy_(t64(b["b1"]))
                m["fc2"].weight.copy_(t64(b["w2"])); m["fc2"].bias.copy_(t64(b["b2"]))
                m.ls1 = t64(b["ls1"]); m.ls2 = t64(b["ls2"])
                self.blocks.append(m)
            self.norm = torch.nn.LayerNorm(D, eps=cfg["ln_eps"], dtype=dt)
            self.norm.weight.copy_(t64(P["norm_g"])); self.norm.bias.copy_(t64(P["norm_b"]))

    def forward(self, x):
        P, B = self.P, x.shape[0]
        e = self.conv(x).flatten(2).transpose(1, 2)
        pos = t64(P["pos"])
        cls = (t64(P["cls"]) + pos[0]).expand(B, 1, -1)
        reg = t64(P["reg"]).expand(B, -1, -1)
        t = torch.cat([cls, reg, e + pos[1:]], dim=1)
        for m in self.blocks:
            h = m["ln1"](t)
            a, _ = m["attn"](h, h, h, need_weights=False)
            t = t + m.ls1 * a
            t = t + m.ls2 * m["fc2"](F.gelu(m["fc1"](m["ln2"](t))))
        y = self.norm(t)
        return y, F.normalize(y[:, 0], dim=-1)


@pytest.mark.parametrize("kw", [dict(), dict(patch=14, img_h=42, img_w=28, registers=0)])
def test_forward_matches_torch_nn_model(kw):
    cfg = small_cfg(**kw)
    P = synth.make_params(cfg)
    x = synth.make_images(cfg, 2)
    got = O.forward(x, P, cfg)
    with torch.no_grad():
        y, d = TorchViT(cfg, P)(t64(x))
    np.testing.assert_allclose(got["tokens"], y.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(got["desc"], d.numpy(), rtol=1e-9, atol=1e-12)


# --------------------------------------------------------------------- closed forms / invariants

def test_layerscale_zero_reduces_to_embedding_norm():
    cfg = small_cfg(layerscale=0.0)
    P = synth.make_params(cfg)
    x = synth.make_images(cfg, 1)
    got = O.forward(x, P, cfg)["tokens"]
    e = F.conv2d(t64(x), t64(P["patch_w"]), t64(P["patch_b"]), stride=cfg["patch"]).flatten(2).transpose(1, 2)
    pos = t64(P["pos"])
    t = torch.cat([(t64(P["cls"]) + pos[0])[None, None], t64(P["reg"])[None], e + pos[1:]], 1)
    ref = F.layer_norm(t, (cfg["dim"],), t64(P["norm_g"]), t64(P["norm_b"]), eps=cfg["ln_eps"])
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_descriptor_is_normalised_cls_and_batch_independent():
    cfg = small_cfg()
    P = synth.make_params(cfg)
    x = synth.make_images(cfg, 3)
    out = O.forward(x, P, cfg)
    d = out["desc"]
    np.testing.assert_allclose(np.linalg.norm(d, axis=1), 1.0, atol=1e-14)
    y0 = out["tokens"][:, 0]
    cos = (d * y0).sum(1) / np.linalg.norm(y0, axis=1)
    digits = FACTS["descriptor_is_cls"]["printed_digits"]
    assert np.all(np.round(cos, digits) == FACTS["descriptor_is_cls"]["cosine_pooler_vs_cls"])
    single = O.forward(x[1:2], P, cfg)
    np.testing.assert_allclose(single["tokens"][0], out["tokens"][1], rtol=1e-12, atol=1e-13)
    assert O.descriptor(np.zeros((1, 4)))[0].tolist() == [0, 0, 0, 0]


def test_taps_use_final_norm_and_tap12_equals_tokens():
    cfg = small_cfg(depth=4, taps=(1, 2, 4), registers=0, patch=14, img_h=42, img_w=28)
    P = synth.make_params(cfg)
    x = synth.make_images(cfg, 2)
    out = O.forward(x, P, cfg)
    gh, gw = synth.grid(cfg)
    assert out["taps"].shape == (2, 3, cfg["dim"], gh, gw)
    last = out["tokens"][:, 1:].reshape(2, gh, gw, -1).transpose(0, 3, 1, 2)
    assert np.array_equal(out["taps"][:, 2], last)
    # an intermediate tap equals LayerNorm of that block's residual (depth-truncated model)
    P1 = dict(P, blocks=P["blocks"][:1])
    one = O.forward(x, P1, dict(cfg, taps=()))["tokens"][:, 1:]
    np.testing.assert_allclose(out["taps"][:, 0], one.reshape(2, gh, gw, -1).transpose(0, 3, 1, 2),
                               rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------- the fp16 overflow facts

@pytest.fixture(scope="module")
def sink_run():
    cfg = synth.preset("vits16_336")
    P = synth.make_params(cfg)
    x = synth.make_images(cfg, 1)
    stats = {}
    ref = O.forward(x, P, cfg, stats=stats)
    return cfg, P, x, stats, ref


def test_sink_logits_reach_published_magnitude(sink_run):
    cfg, P, x, stats, ref = sink_run
    f = FACTS["fp16_overflow"]
    per_block = stats["logits_per_block"]
    assert 0.9 * f["max_abs_logit_natural_image"] <= per_block[0] <= 1.1 * f["max_abs_logit_natural_image"]
    assert per_block[0] > f["max_abs_logit_min"]
    assert max(per_block[1:]) < f["other_tensors_below"]
    for name, v in stats.items():
        if name not in ("logits", "logits_per_block"):
            assert v < f["other_tensors_below"], (name, v)
    params_max = max(np.abs(a).max() for a in [P["patch_w"], P["cls"], P["reg"], P["pos"]] +
                     [a for b in P["blocks"] for a in b.values()])
    assert params_max < f["other_tensors_below"]
    assert np.isfinite(ref["tokens"]).all()


def test_sink_softmax_is_one_hot_on_register_zero(sink_run):
    cfg, P, x, stats, ref = sink_run
    blk = P["blocks"][0]
    emb = O.patch_embed(x, P["patch_w"], P["patch_b"])
    t = O.assemble_tokens(emb, P["cls"], P["reg"], P["pos"])
    h = O.layer_norm(t, blk["ln1_g"], blk["ln1_b"], cfg["ln_eps"])
    q = O.linear(h, blk["wq"], blk["bq"])[0, :, :64]
    k = O.linear(h, blk["wk"], blk["bk"])[0, :, :64]
    s = q @ k.T / 8.0
    p = O.softmax_rows(s)
    assert np.all(p[:, 1] == 1.0)
    assert np.all(np.delete(p, 1, axis=1) == 0.0)
    second = np.sort(s, axis=1)[:, -2]
    assert np.min(s[:, 1] - second) > 1e6      # margin far above bf16 logit error


def test_fp16_logits_give_nan_everywhere_bf16_stays_finite(sink_run):
    cfg, P, x, stats, ref = sink_run
    out16 = O.forward(x, P, cfg, logit_format="fp16")
    assert np.isnan(out16["tokens"]).all() and np.isnan(out16["desc"]).all()
    for fmt in ("bf16", "fp32"):
        o = O.forward(x, P, cfg, logit_format=fmt)
        assert np.isfinite(o["tokens"]).all()
        cos = float((o["desc"] * ref["desc"]).sum())
        assert cos > 0.9999


# --------------------------------------------------------------------- zero-shot scoring

def _text_cfg():
    return small_cfg(img_h=64, img_w=96, window=48, window_stride=24, classes=7, depth=1,
                     extra_blocks=1, pos_grid=(4, 6))


def test_whole_mode_properties():
    cfg = _text_cfg()
    P = synth.make_params(cfg)
    T = synth.make_class_embeddings(cfg)
    x = synth.make_images(cfg, 1)[0]
    r = O.scores_whole(x, P, cfg, T)
    assert r["cos"].shape == (7, 4, 6) and r["scores"].shape == (7, 64, 96)
    assert np.abs(r["cos"]).max() <= 1 + 1e-12
    np.testing.assert_array_equal(r["labels"], np.argmax(r["scores"], axis=0))
    ref = F.interpolate(t64(r["cos"])[None], size=(64, 96), mode="bilinear", align_corners=False)[0]
    np.testing.assert_allclose(r["scores"], ref.numpy(), atol=1e-12)
    # features are unit vectors: cos of a class embedding equal to a patch feature is 1
    f = O.patch_features(x[None], P, cfg)[0]
    r2 = O.scores_whole(x, P, cfg, f[1, 2][None])
    assert abs(r2["cos"][0, 1, 2] - 1.0) < 1e-12


def test_slide_mode_properties():
    cfg = _text_cfg()
    P = synth.make_params(cfg)
    T = synth.make_class_embeddings(cfg)
    x = synth.make_images(cfg, 1)[0]
    r = O.scores_slide(x, P, cfg, T)
    assert len(r["windows"]) == 2 * 3
    assert r["counts"].min() >= 1
    np.testing.assert_allclose(r["probs"].sum(axis=0), 1.0, atol=1e-12)
    np.testing.assert_array_equal(r["labels"], np.argmax(r["probs"], axis=0))
    # a single window covering the whole image reduces to softmax(whole-mode scores)
    cfg1 = dict(cfg, img_h=48, img_w=48, pos_grid=(3, 3))
    P1 = synth.make_params(cfg1)
    x1 = synth.make_images(cfg1, 1)[0]
    s = O.scores_slide(x1, P1, cfg1, T)
    w = O.scores_whole(x1, P1, cfg1, T)
    np.testing.assert_allclose(s["probs"], torch.softmax(t64(w["scores"]), 0).numpy(), atol=1e-12)
