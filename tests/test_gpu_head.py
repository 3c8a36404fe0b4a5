"""GPU parity of the semantic head on the taps (LibreYOLO DINOv2 diagram,
"Projector P4" and "Task head") against the float64 oracle.

The head runs every conv on bf16 operands with fp32 accumulation and stores
the activations between layers as bf16; each of its ten stored activations
(taps, stem, six Bottleneck convs, projector output, lateral, GroupNorm output)
carries a relative rounding of at most 2^-9, and every one is followed by a
normalisation or a conv that keeps the activation scale near 1.  Summed over
the ten, that is 10 * 2^-9 = 1.95e-2 of the logit scale in the worst case; the
fp32 GEMM sums add far less (K <= 2304 terms at 2^-24).  The bound is 2e-2 of
the largest |logit|.
"""

import numpy as np
import pytest
import torch

import synth
import vision_transformer_encoder_block_amd as vit
from gpu_util import f32_dev, host, require_gpu, say
from oracle import head_oracle as H

pytestmark = pytest.mark.gpu

REL_TOL = 2e-2


def run_head(hcfg, Ph, taps):
    head = vit.SemanticHead(hcfg, Ph)
    logits, grid = head.forward(f32_dev(taps), want_grid=True)
    out = host(logits), host(grid)
    head.close()
    return out


def oracle_head(taps, Ph, out_h, out_w):
    refs = [H.semantic_head(taps[b], Ph, out_h, out_w) for b in range(taps.shape[0])]
    return np.stack([r["logits"] for r in refs]), np.stack([r["grid"] for r in refs])


def check(name, got, ref):
    assert got.shape == ref.shape
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    scale = np.abs(ref).max()
    say(f"{name}: max |gpu - oracle| = {err:.3e}, max |logit| = {scale:.3e}, ratio {err / scale:.3e}")
    assert err <= REL_TOL * scale


def check_labels(got, ref):
    """Argmax over classes agrees wherever the oracle's top-two margin exceeds twice the bound."""
    tol = REL_TOL * np.abs(ref).max()
    srt = np.sort(ref, axis=1)
    clear = (srt[:, -1] - srt[:, -2]) > 2 * tol
    agree = np.argmax(got, axis=1) == np.argmax(ref, axis=1)
    say(f"labels: {clear.mean():.3f} of pixels clear of ties, all of them agree: {agree[clear].all()}")
    assert agree[clear].all()


@pytest.mark.parametrize("batch,gh,gw,out", [(2, 6, 5, (84, 70)), (3, 13, 11, (100, 90)), (1, 1, 1, (7, 5)),
                                             (1, 20, 17, (42, 30)),    # GroupNorm: 1 float4 per thread
                                             (1, 50, 45, (33, 61)),    # GroupNorm: 5 float4 per thread
                                             (1, 64, 128, (70, 60)),   # GroupNorm: 8192 pixels, 16 per thread
                                             (1, 96, 90, (50, 40)),    # GroupNorm: > 8192 pixels (loop)
                                             (1, 3, 240, (5, 500))])   # 240 x 19 classes: the gather resize
def test_head_matches_oracle_small_grids(batch, gh, gw, out):
    require_gpu()
    cfg = synth.preset("vits14_518")
    say(f"semantic head, batch {batch}, grid {gh}x{gw} -> {out}")
    Ph = synth.make_head_params(cfg)
    taps = synth.make_taps(cfg, batch, gh=gh, gw=gw)
    got, got_grid = run_head(vit.head_config(gh, gw, out[0], out[1], batch), Ph, taps)
    ref, ref_grid = oracle_head(taps, Ph, *out)
    check("grid logits", got_grid, ref_grid)
    check("resized logits", got, ref)


def test_head_full_geometry_b8():
    require_gpu()
    cfg = synth.preset("vits14_518")
    say("semantic head, batch 8, grid 37x37 -> 518x518")
    Ph = synth.make_head_params(cfg)
    taps = synth.make_taps(cfg, 8)
    hcfg = vit.head_config_preset()
    got, got_grid = run_head(hcfg, Ph, taps)
    ref, ref_grid = oracle_head(taps, Ph, 518, 518)
    check("grid logits", got_grid, ref_grid)
    check("resized logits", got, ref)
    check_labels(got, ref)


def test_head_on_encoder_taps():
    """The encoder's own taps (DINOv2-S/14 @518, batch 2) through the head."""
    require_gpu()
    cfg = synth.preset("vits14_518")
    say("DINOv2-S/14 @518 b2 encoder taps -> semantic head")
    P = synth.make_params(cfg)
    Ph = synth.make_head_params(cfg)
    x = synth.make_images(cfg, 2)
    enc = vit.Encoder(cfg, P, max_batch=2)
    _, taps = enc.forward(f32_dev(x), with_taps=True)
    head = vit.SemanticHead(vit.head_config(37, 37, 518, 518, 2), Ph)
    logits, grid = head.forward(taps, want_grid=True)
    got, got_grid, taps_h = host(logits), host(grid), host(taps)
    head.close()
    enc.close()
    ref, ref_grid = oracle_head(taps_h, Ph, 518, 518)
    check("grid logits", got_grid, ref_grid)
    check("resized logits", got, ref)


def test_head_batch_invariance():
    """Each image's logits do not depend on the rest of the batch (bit for bit)."""
    require_gpu()
    cfg = synth.preset("vits14_518")
    Ph = synth.make_head_params(cfg)
    taps = synth.make_taps(cfg, 3, gh=9, gw=10)
    head = vit.SemanticHead(vit.head_config(9, 10, 40, 44, 3), Ph)
    all3 = host(head.forward(f32_dev(taps)))
    for b in range(3):
        one = host(head.forward(f32_dev(taps[b:b + 1])))
        np.testing.assert_array_equal(all3[b:b + 1], one)
    head.close()


def test_head_rejects_bad_calls():
    require_gpu()
    cfg = synth.preset("vits14_518")
    Ph = synth.make_head_params(cfg)
    head = vit.SemanticHead(vit.head_config(4, 4, 8, 8, 2), Ph)
    taps = f32_dev(synth.make_taps(cfg, 3, gh=4, gw=4))
    out = torch.empty((3, 19, 8, 8), device="cuda")
    with pytest.raises(vit.VitError):
        head.forward(taps, logits_out=out)      # batch 3 > max_batch 2
    r = vit.lib().vit_head_forward(head.handle, vit._ptr(taps), 0, vit._ptr(out), None, None)
    assert r == -3
    head.close()
    with pytest.raises(vit.VitError):
        vit.SemanticHead(vit.head_config(4, 4, 8, 8, 2), np.zeros(10, np.float32))


def _round_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("batch,gh,gw,ld,c0,cin,n_out,bias", [
    (2, 5, 7, 640, 128, 128, 128, False),    # a Bottleneck input slice of the C2f concat
    (1, 37, 37, 256, 0, 256, 256, True),     # the smoothing conv at the full grid
    (3, 1, 1, 128, 0, 128, 64, True),        # every neighbour is padding
    (2, 9, 4, 192, 64, 64, 19, False),       # ragged N
])
def test_conv3x3_matches_oracle(batch, gh, gw, ld, c0, cin, n_out, bias):
    """vit_op_conv3x3 (implicit GEMM) against the oracle's convolution.  Inputs and
    weights are bf16 values, so every product is exact in fp32 and the only error
    is the fp32 sum of 9 cin terms: |err| <= 9 cin 2^-24 sum |w x| (+ the bias add)."""
    require_gpu()
    say(f"conv3x3 batch {batch} grid {gh}x{gw} ld {ld} c0 {c0} cin {cin} -> {n_out}")
    rng = np.random.default_rng(gh * 100 + cin)
    x = _round_bf16(rng.standard_normal((batch * gh * gw, ld)))
    w4 = _round_bf16(rng.standard_normal((n_out, cin, 3, 3)) * 0.05)
    b = torch.from_numpy(rng.standard_normal(n_out).astype(np.float32)) if bias else None
    wk = w4.permute(0, 2, 3, 1).reshape(n_out, 9 * cin).contiguous()      # (ky, kx, c) columns
    out = torch.empty((batch * gh * gw, n_out), device="cuda")
    vit.vit_op_conv3x3(x.cuda(), ld, c0, cin, batch, gh, gw, wk.cuda(), None if b is None else b.cuda(), n_out, out)
    got = host(out)
    xs = x.double().numpy()[:, c0:c0 + cin].reshape(batch, gh, gw, cin).transpose(0, 3, 1, 2)
    w64 = w4.double().numpy()
    ref = np.stack([H.conv2d(xs[i], w64, None if b is None else b.double().numpy(), 1) for i in range(batch)])
    ref = ref.transpose(0, 2, 3, 1).reshape(batch * gh * gw, n_out)
    absref = np.stack([H.conv2d(np.abs(xs[i]), np.abs(w64), None, 1) for i in range(batch)])
    absref = absref.transpose(0, 2, 3, 1).reshape(batch * gh * gw, n_out)
    bound = 9 * cin * 2.0 ** -24 * absref + 2.0 ** -24 * np.abs(ref) + 1e-30
    err = np.abs(got - ref)
    say(f"max err / bound = {(err / bound).max():.3f}")
    assert (err <= bound).all()


@pytest.mark.parametrize("batch,gh,gw,ld,c0,cin,n_out,bias", [
    (2, 5, 7, 640, 128, 128, 128, False), (1, 37, 37, 256, 0, 256, 256, True), (3, 1, 1, 128, 0, 128, 64, True),
    (2, 9, 4, 192, 64, 64, 19, True)])
def test_conv3x3_exact_groups(batch, gh, gw, ld, c0, cin, n_out, bias):
    """The implicit-GEMM 3x3 conv bit for bit.  Inputs and weights of magnitude
    [1, 2) (8 significant bits) make the 16 products of one MFMA sum exactly
    (20 bits, as in the encoder's GEMM test), and the zero padding adds exact
    zeros, so the result must equal the fp32 accumulation of the 16-wide k
    groups of the (ky, kx, c) ordered columns in k order, then the bias add: a
    wrong neighbour, a tap read from the wrong row or a missing zero breaks it."""
    require_gpu()
    say(f"conv3x3 exact groups batch {batch} grid {gh}x{gw} ld {ld} c0 {c0} cin {cin} -> {n_out}")
    rng = np.random.default_rng(gh * 101 + cin + n_out)
    unit = lambda shape: (1.0 + rng.integers(0, 128, shape) / 128.0) * np.where(rng.integers(0, 2, shape) == 1, -1, 1)
    M = batch * gh * gw
    xv, wv = unit((M, ld)), unit((n_out, 9 * cin))
    x, wk = _round_bf16(xv), _round_bf16(wv)
    assert np.array_equal(x.double().numpy(), xv) and np.array_equal(wk.double().numpy(), wv)
    b = rng.standard_normal(n_out).astype(np.float32) if bias else np.zeros(n_out, np.float32)
    out = torch.empty((M, n_out), device="cuda")
    vit.vit_op_conv3x3(x.cuda(), ld, c0, cin, batch, gh, gw, wk.cuda(), torch.from_numpy(b).cuda() if bias else None,
                       n_out, out)
    got = host(out)
    img = xv[:, c0:c0 + cin].reshape(batch, gh, gw, cin)
    pad = np.zeros((batch, gh + 2, gw + 2, cin))
    pad[:, 1:-1, 1:-1] = img
    cols = np.concatenate([pad[:, ky:ky + gh, kx:kx + gw].reshape(M, cin) for ky in range(3) for kx in range(3)], axis=1)
    acc = np.zeros((M, n_out), np.float32)
    for g in range(0, 9 * cin, 16):
        acc = (acc.astype(np.float64) + cols[:, g:g + 16] @ wv[:, g:g + 16].T).astype(np.float32)
    model = (acc.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    diff = got != model
    say(f"  {diff.mean():.6f} of outputs differ from the accumulation model")
    assert not diff.any(), (np.argwhere(diff)[:5], np.abs(got - model).max())


def _ln_error(z, e_max, g, eps):
    """Bound on the change of LN(z) (channels on axis 1, per-channel affine g)
    when every input of a row moves by at most e_max of that row: the mean moves
    by <= e_max and sigma by <= e_max, so each output moves by
    <= |g| (2 e_max + |y| e_max) / sigma, y the normalised value; plus the fp32
    arithmetic of the statistics (2^-20 relative, generous)."""
    mu = z.mean(axis=1, keepdims=True)
    sig = np.sqrt(((z - mu) ** 2).mean(axis=1, keepdims=True) + eps)
    y = (z - mu) / sig
    return np.abs(g) * ((2 + np.abs(y)) * e_max / sig + 2.0 ** -20 * (1 + np.abs(y)))


@pytest.mark.parametrize("ksize,batch,gh,gw,ld,c0,cin,n_out,second,ld_out,c0_out", [
    (3, 2, 37, 37, 640, 128, 128, 128, False, 640, 384),   # a Bottleneck conv: C2f slice in, C2f slice out
    (3, 1, 5, 7, 128, 0, 128, 128, False, 128, 0),          # Bottleneck conv 1 into its temporary
    (1, 2, 9, 11, 1536, 0, 1536, 256, False, 640, 0),       # the projector conv (4 taps concatenated)
    (1, 1, 37, 37, 640, 0, 640, 256, True, 256, 0),         # the output ConvX with the final LayerNorm
    (3, 3, 1, 1, 256, 0, 256, 256, False, 256, 0),          # every neighbour is padding
])
def test_convx_matches_oracle(ksize, batch, gh, gw, ld, c0, cin, n_out, second, ld_out, c0_out):
    """vit_op_convx (conv, channel LayerNorm, SiLU, optional second LayerNorm, in
    one GEMM epilogue) against the oracle's conv_ln_silu.  Inputs and weights are
    bf16 values: the conv's only error is its fp32 sum (<= taps cin 2^-24
    sum |w x| per output), which each LayerNorm passes on scaled by 1/sigma and
    SiLU by at most 1.1; the bf16 output adds 2^-8 |y|."""
    require_gpu()
    say(f"convx k{ksize} batch {batch} grid {gh}x{gw} cin {cin} -> {n_out} second LN {second}")
    rng = np.random.default_rng(gh * 31 + cin + n_out)
    M = batch * gh * gw
    x = _round_bf16(rng.standard_normal((M, ld)))
    w4 = _round_bf16(rng.standard_normal((n_out, cin, ksize, ksize)) * 0.05)
    g = (1 + 0.02 * rng.standard_normal(n_out)).astype(np.float32)
    b = (0.02 * rng.standard_normal(n_out)).astype(np.float32)
    g2 = (1 + 0.02 * rng.standard_normal(n_out)).astype(np.float32)
    b2 = (0.02 * rng.standard_normal(n_out)).astype(np.float32)
    wk = w4.permute(0, 2, 3, 1).reshape(n_out, ksize * ksize * cin).contiguous()
    out = torch.zeros((M, ld_out), dtype=torch.bfloat16, device="cuda")
    dev = lambda a: torch.from_numpy(a).cuda()
    vit.vit_op_convx(x.cuda(), ld, c0, cin, batch, gh, gw, ksize, wk.cuda(), n_out, dev(g), dev(b),
                     dev(g2) if second else None, dev(b2) if second else None, H.HEAD_LN_EPS, out, ld_out, c0_out)
    got = host(out)
    xs = x.double().numpy()[:, c0:c0 + cin].reshape(batch, gh, gw, cin).transpose(0, 3, 1, 2)
    w64 = w4.double().numpy()
    pad = ksize // 2
    conv = np.stack([H.conv2d(xs[i], w64, None, pad) for i in range(batch)]).transpose(0, 2, 3, 1).reshape(M, n_out)
    absconv = np.stack([H.conv2d(np.abs(xs[i]), np.abs(w64), None, pad)
                        for i in range(batch)]).transpose(0, 2, 3, 1).reshape(M, n_out)
    e1 = (ksize * ksize * cin * 2.0 ** -24 * absconv).max(axis=1, keepdims=True)
    # the oracle's ConvX on channels-first images, back to rows
    ref = np.stack([H.conv_ln_silu(xs[i], w64, g, b, pad) for i in range(batch)])
    bound = 1.1 * _ln_error(conv, e1, g.astype(np.float64)[None], H.HEAD_LN_EPS)
    if second:
        ref = np.stack([H.channel_layer_norm(ref[i], g2, b2) for i in range(batch)])
        s = np.stack([H.conv_ln_silu(xs[i], w64, g, b, pad) for i in range(batch)]).transpose(0, 2, 3, 1).reshape(M, n_out)
        bound = _ln_error(s, bound.max(axis=1, keepdims=True), g2.astype(np.float64)[None], H.HEAD_LN_EPS)
    ref = ref.transpose(0, 2, 3, 1).reshape(M, n_out)
    bound = bound + 2.0 ** -8 * np.abs(ref) + 1e-30
    err = np.abs(got[:, c0_out:c0_out + n_out] - ref)
    say(f"max err / bound = {(err / bound).max():.3f}")
    assert (err <= bound).all()
    # columns outside [c0_out, c0_out + n_out) are not written
    assert not got[:, :c0_out].any() and not got[:, c0_out + n_out:].any()
