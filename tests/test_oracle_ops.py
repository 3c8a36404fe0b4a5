"""Pins for the oracle's individual steps.

Each step is compared with something other than itself: a float64 PyTorch CPU
library routine computing the same operation, a brute-force loop on a tiny input,
or a closed-form property.  None of these tests touches the GPU library.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import vit_oracle as O

RNG = np.random.default_rng(12345)


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# --------------------------------------------------------------------- patch embed

@pytest.mark.parametrize("p,H,W,D", [(16, 32, 48, 8), (14, 28, 42, 5), (2, 4, 6, 3)])
def test_patch_embed_matches_conv2d(p, H, W, D):
    x = RNG.standard_normal((2, 3, H, W))
    w = RNG.standard_normal((D, 3, p, p))
    b = RNG.standard_normal(D)
    got = O.patch_embed(x, w, b)
    ref = F.conv2d(t64(x), t64(w), t64(b), stride=p)  # [B, D, gh, gw]
    ref = ref.flatten(2).transpose(1, 2).numpy()       # raster order of the grid
    assert got.shape == (2, (H // p) * (W // p), D)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_patch_embed_brute_force():
    p, H, W, D = 2, 4, 6, 3
    x = RNG.standard_normal((1, 3, H, W))
    w = RNG.standard_normal((D, 3, p, p))
    b = RNG.standard_normal(D)
    got = O.patch_embed(x, w, b)[0]
    gw = W // p
    for gy in range(H // p):
        for gx in range(gw):
            for d in range(D):
                acc = b[d]
                for c in range(3):
                    for ky in range(p):
                        for kx in range(p):
                            acc += w[d, c, ky, kx] * x[0, c, gy * p + ky, gx * p + kx]
                assert abs(got[gy * gw + gx, d] - acc) < 1e-12


def test_assemble_tokens_layout():
    B, Pn, D, R = 2, 6, 4, 4
    emb = RNG.standard_normal((B, Pn, D))
    cls = RNG.standard_normal(D)
    reg = RNG.standard_normal((R, D))
    pos = RNG.standard_normal((1 + Pn, D))
    t = O.assemble_tokens(emb, cls, reg, pos)
    assert t.shape == (B, 1 + R + Pn, D)
    for bi in range(B):
        assert np.array_equal(t[bi, 0], cls + pos[0])
        assert np.array_equal(t[bi, 1:1 + R], reg)          # registers: no position term
        assert np.array_equal(t[bi, 1 + R:], emb[bi] + pos[1:])


# --------------------------------------------------------------------- LayerNorm

def test_layer_norm_matches_torch():
    x = RNG.standard_normal((3, 7, 384)) * 3 + 1
    g = 1 + 0.1 * RNG.standard_normal(384)
    b = 0.1 * RNG.standard_normal(384)
    got = O.layer_norm(x, g, b, 1e-6)
    ref = F.layer_norm(t64(x), (384,), t64(g), t64(b), eps=1e-6).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_layer_norm_invariants_and_eps_placement():
    # gamma = 1, beta = 0: every row has mean 0 and variance var/(var + eps)
    x = RNG.standard_normal((5, 64)) * np.array([1e-4, 1e-3, 1e-2, 1, 10])[:, None]
    eps = 1e-6
    y = O.layer_norm(x, np.ones(64), np.zeros(64), eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=1), var / (var + eps), rtol=1e-10)
    # eps sits under the square root of the variance (not added to the std)
    row = np.array([[1.0, -1.0] * 32]) * 1e-3   # var = 1e-6 exactly
    y = O.layer_norm(row, np.ones(64), np.zeros(64), 1e-6)
    assert abs(y[0, 0] - 1e-3 / math.sqrt(2e-6)) < 1e-12


# --------------------------------------------------------------------- GELU

def test_gelu_matches_torch_exact_form():
    x = np.linspace(-8, 8, 2001)
    got = O.gelu(x)
    ref = F.gelu(t64(x), approximate="none").numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)
    # the tanh approximation differs by > 1e-5 somewhere: the oracle is not it
    tanh_form = F.gelu(t64(x), approximate="tanh").numpy()
    assert np.abs(got - tanh_form).max() > 1e-5


def test_gelu_special_values():
    assert O.gelu(np.array([0.0]))[0] == 0.0
    assert abs(O.gelu(np.array([10.0]))[0] - 10.0) < 1e-15
    assert abs(O.gelu(np.array([-10.0]))[0]) < 1e-20
    for z in (-2.5, -0.3, 0.7, 1.9):
        assert abs(O.gelu(np.array([z]))[0] - z * 0.5 * (1 + math.erf(z / math.sqrt(2)))) < 1e-15


# --------------------------------------------------------------------- attention

def _rand_block(D, Hm=8, scale=0.3):
    blk = {}
    for n in ("wq", "wk", "wv", "wo"):
        blk[n] = RNG.standard_normal((D, D)) * scale
    for n in ("bq", "bk", "bv", "bo"):
        blk[n] = RNG.standard_normal(D) * scale
    blk["w1"] = RNG.standard_normal((Hm, D)) * scale
    blk["b1"] = RNG.standard_normal(Hm) * scale
    blk["w2"] = RNG.standard_normal((D, Hm)) * scale
    blk["b2"] = RNG.standard_normal(D) * scale
    return blk


def test_attention_brute_force_tiny():
    B, N, heads, hd = 1, 5, 2, 64
    D = heads * hd
    h = RNG.standard_normal((B, N, D)) * 0.5
    blk = _rand_block(D, scale=0.1)
    got = O.attention(h, blk, heads)
    # plain loops: q/k/v, per-head softmax over keys, merge, output projection
    q = [[sum(h[0, n, i] * blk["wq"][o, i] for i in range(D)) + blk["bq"][o] for o in range(D)] for n in range(N)]
    k = [[sum(h[0, n, i] * blk["wk"][o, i] for i in range(D)) + blk["bk"][o] for o in range(D)] for n in range(N)]
    v = [[sum(h[0, n, i] * blk["wv"][o, i] for i in range(D)) + blk["bv"][o] for o in range(D)] for n in range(N)]
    merged = [[0.0] * D for _ in range(N)]
    for j in range(heads):
        for n in range(N):
            logits = [sum(q[n][j * hd + c] * k[m][j * hd + c] for c in range(hd)) / 8.0 for m in range(N)]
            mx = max(logits)
            ex = [math.exp(s - mx) for s in logits]
            tot = sum(ex)
            for c in range(hd):
                merged[n][j * hd + c] = sum(ex[m] / tot * v[m][j * hd + c] for m in range(N))
    ref = np.array([[sum(merged[n][i] * blk["wo"][o, i] for i in range(D)) + blk["bo"][o]
                     for o in range(D)] for n in range(N)])
    np.testing.assert_allclose(got[0], ref, rtol=1e-10, atol=1e-12)


def test_attention_matches_torch_multihead():
    B, N, heads, hd = 2, 11, 3, 64
    D = heads * hd
    h = RNG.standard_normal((B, N, D))
    blk = _rand_block(D, scale=0.05)
    got = O.attention(h, blk, heads)
    mha = torch.nn.MultiheadAttention(D, heads, bias=True, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        mha.in_proj_weight.copy_(t64(np.concatenate([blk["wq"], blk["wk"], blk["wv"]])))
        mha.in_proj_bias.copy_(t64(np.concatenate([blk["bq"], blk["bk"], blk["bv"]])))
        mha.out_proj.weight.copy_(t64(blk["wo"]))
        mha.out_proj.bias.copy_(t64(blk["bo"]))
        ref, _ = mha(t64(h), t64(h), t64(h), need_weights=False)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_softmax_rows_sum_to_one():
    s = RNG.standard_normal((4, 9, 33)) * 50
    p = O.softmax_rows(s)
    assert np.abs(p.sum(-1) - 1).max() <= 1e-12
    np.testing.assert_allclose(p, torch.softmax(t64(s), -1).numpy(), rtol=1e-12, atol=1e-300)


def test_attention_invariant_to_key_bias():
    # adding a vector to every key shifts every logit of a query row by one constant
    B, N, heads, hd = 1, 7, 2, 64
    D = heads * hd
    h = RNG.standard_normal((B, N, D))
    blk = _rand_block(D, scale=0.05)
    a = O.attention(h, blk, heads)
    blk2 = dict(blk, bk=blk["bk"] + RNG.standard_normal(D))
    b = O.attention(h, blk2, heads)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)


def test_attention_permutation_equivariant():
    B, N, heads, hd = 1, 8, 2, 64
    D = heads * hd
    h = RNG.standard_normal((B, N, D))
    blk = _rand_block(D, scale=0.05)
    perm = RNG.permutation(N)
    a = O.attention(h, blk, heads)
    b = O.attention(h[:, perm], blk, heads)
    np.testing.assert_allclose(a[:, perm], b, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------- formats

def test_to_format_fp16_and_bf16():
    x = np.array([65504.0, 65520.0, 7e4, -2.5e6, 1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9, 3.14159, 2.5e6])
    f16 = O.to_format(x, "fp16")
    assert f16[0] == 65504.0 and np.isinf(f16[1]) and np.isinf(f16[2]) and f16[3] == -np.inf
    bf = O.to_format(x, "bf16")
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf, ref)
    assert np.isfinite(bf).all()
    assert bf[4] == 1.0 and bf[5] == 1.0 + 2 ** -7        # ties to even


# --------------------------------------------------------------------- resampling

@pytest.mark.parametrize("shape,out", [((3, 4, 6), (9, 5)), ((2, 24, 24), (384, 384)), ((1, 7, 3), (7, 3))])
def test_bilinear_matches_torch(shape, out):
    x = RNG.standard_normal(shape)
    got = O.bilinear_resize(x, *out)
    ref = F.interpolate(t64(x)[None], size=out, mode="bilinear", align_corners=False)[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_bilinear_constant_and_identity():
    c = np.full((2, 5, 7), 3.25)
    np.testing.assert_allclose(O.bilinear_resize(c, 13, 29), 3.25, atol=1e-15)
    x = RNG.standard_normal((2, 5, 7))
    np.testing.assert_array_equal(O.bilinear_resize(x, 5, 7), x)


@pytest.mark.parametrize("shape,out", [((3, 32, 64), (24, 24)), ((2, 14, 14), (16, 16)), ((1, 5, 9), (5, 9))])
def test_bicubic_matches_torch(shape, out):
    x = RNG.standard_normal(shape)
    got = O.bicubic_resize(x, *out)
    ref = F.interpolate(t64(x)[None], size=out, mode="bicubic", align_corners=False)[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_bicubic_identity_and_constant():
    x = RNG.standard_normal((4, 37, 37))
    np.testing.assert_allclose(O.bicubic_resize(x, 37, 37), x, rtol=0, atol=1e-14)
    c = np.full((1, 32, 64), -0.5)
    np.testing.assert_allclose(O.bicubic_resize(c, 24, 24), -0.5, atol=1e-14)


def test_resample_pos_keeps_cls_row():
    pos = RNG.standard_normal((1 + 6 * 8, 5))
    r = O.resample_pos(pos, (6, 8), (3, 4))
    assert r.shape == (1 + 12, 5)
    assert np.array_equal(r[0], pos[0])
    assert np.allclose(O.resample_pos(pos, (6, 8), (6, 8)), pos, atol=1e-14)


# --------------------------------------------------------------------- slide windows

def test_slide_windows_count_and_coverage():
    wins = O.slide_windows(512, 1024, 384, 192)
    assert len(wins) == 10
    assert sorted({y for y, _ in wins}) == [0, 128]
    assert sorted({x for _, x in wins}) == [0, 192, 384, 576, 640]
    cover = np.zeros((512, 1024), dtype=int)
    for y, x in wins:
        assert 0 <= y and y + 384 <= 512 and 0 <= x and x + 384 <= 1024
        cover[y:y + 384, x:x + 384] += 1
    assert cover.min() >= 1 and cover.max() <= 6
    assert O.slide_windows(384, 384, 384, 192) == [(0, 0)]


def test_sdpa_matches_torch_with_scale():
    q = RNG.standard_normal((13, 64))
    k = RNG.standard_normal((21, 64))
    v = RNG.standard_normal((21, 64))
    for scale in (0.125, math.log(2.0)):
        got, smax = O.sdpa(q, k, v, scale)
        ref = F.scaled_dot_product_attention(t64(q)[None], t64(k)[None], t64(v)[None], scale=scale)[0].numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
        assert smax == pytest.approx(np.abs(q @ k.T).max() * scale)


# --------------------------------------------------------------------- frame preprocessing

def _facts():
    import json, os
    return json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_preprocess_constants_are_the_cards():
    f = _facts()["imagenet_normalisation"]
    assert tuple(O.IMAGENET_MEAN) == tuple(f["mean"]) and tuple(O.IMAGENET_STD) == tuple(f["std"])


@pytest.mark.parametrize("frame,out", [((2, 37, 53), (45, 31)), ((1, 72, 128), (33, 33)), ((1, 20, 20), (64, 48))])
def test_preprocess_matches_torch(frame, out):
    """Resize + normalise against torch's bilinear interpolate (align_corners=False)
    on the 0..1-scaled frame, a routine the oracle does not use."""
    f = RNG.integers(0, 256, size=frame + (3,), dtype=np.uint8)
    got = O.preprocess(f, *out)
    t = torch.from_numpy(f.astype(np.float64)).permute(0, 3, 1, 2) / 255.0
    r = F.interpolate(t, size=out, mode="bilinear", align_corners=False)
    mean = torch.tensor([0.485, 0.456, 0.406], dtype=torch.float64)[None, :, None, None]
    std = torch.tensor([0.229, 0.224, 0.225], dtype=torch.float64)[None, :, None, None]
    np.testing.assert_allclose(got, ((r - mean) / std).numpy(), rtol=1e-12, atol=1e-12)


def test_preprocess_special_cases():
    # same size: no resampling, only the per-channel normalisation
    f = RNG.integers(0, 256, size=(1, 6, 9, 3), dtype=np.uint8)
    got = O.preprocess(f, 6, 9)
    for c, (m, s) in enumerate(zip((0.485, 0.456, 0.406), (0.229, 0.224, 0.225))):
        np.testing.assert_allclose(got[0, c], (f[0, :, :, c] / 255.0 - m) / s, rtol=0, atol=1e-14)
    # BGR input is the RGB result of the channel-reversed frame
    np.testing.assert_array_equal(O.preprocess(f, 4, 5, bgr=True), O.preprocess(f[..., ::-1].copy(), 4, 5))
    # a horizontal ramp v = 2x halved: output column j samples x = 2j + 0.5, i.e. v = 4j + 1
    ramp = np.zeros((1, 4, 128, 3), dtype=np.uint8)
    ramp[0, :, :, :] = (2 * np.arange(128, dtype=np.uint8))[None, :, None]
    got = O.preprocess(ramp, 4, 64)
    want = ((4 * np.arange(64) + 1) / 255.0 - 0.485) / 0.229
    np.testing.assert_allclose(got[0, 0, 2], want, rtol=0, atol=1e-12)
    # a 2-pixel row doubled: edge pixels replicate, the inner samples weigh 3:1
    two = np.array([[[[40, 40, 40], [200, 200, 200]]]], dtype=np.uint8)
    got = O.preprocess(two, 1, 4)[0, 1, 0] * 0.224 + 0.456
    np.testing.assert_allclose(got * 255.0, [40, 80, 160, 200], rtol=0, atol=1e-9)

