"""GPU parity of the int8 linear layer against the quantised oracle.

Codes are integers decided from the same float32 product on both sides, so they
must agree bit for bit.  The products of int8 codes are integers and their sums
are exact in int32 (K * 127^2 < 2^31), so the whole layer is determined: each
sum is rounded once to fp32 (nearest even), then out = fma(sum, scale, bias)
rounds once more, and bf16 output once more.  The kernel must equal that model
bit for bit; against the float64 oracle the error is then at most
2^-24 |scale| |sum| + 2^-24 |y| (+ 2^-8 |y| for bf16 output).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import vision_transformer_encoder_block_amd as vit
from gpu_util import host, require_gpu, say
from oracle import quant_oracle as Q

pytestmark = pytest.mark.gpu


def codes_dev(q):
    return torch.from_numpy(np.ascontiguousarray(q, np.int8)).cuda()


SPECIAL = np.array([0.0, -0.0, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, 127.4, 127.5, 128.0, -127.5, -200.0,
                    np.inf, -np.inf, np.nan, 1e-30, -1e-30, 3.0], np.float32)


@pytest.mark.parametrize("n,s_inv", [(1, 1.0), (3, 0.5), (4099, 1.0), (1 << 20, 0.37)])
def test_quantize_int8_codes_bit_exact(n, s_inv):
    require_gpu()
    rng = np.random.default_rng(n + 1)
    x = (rng.standard_normal(n) * 60).astype(np.float32)
    x[: min(n, SPECIAL.size)] = SPECIAL[: min(n, SPECIAL.size)]
    out = torch.empty(n, dtype=torch.int8, device="cuda")
    vit.vit_op_quantize_int8(torch.from_numpy(x).cuda(), n, s_inv, out)
    got = out.cpu().numpy()
    ref = Q.quantize_int8(x, s_inv)
    bad = np.flatnonzero(got != ref)
    say(f"quantize int8 n={n}: {bad.size} mismatches")
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])
    assert got.min() >= -127


def test_quantize_int8_from_bf16_bit_exact():
    require_gpu()
    rng = np.random.default_rng(6)
    xb = torch.from_numpy((rng.standard_normal(100003) * 30).astype(np.float32)).to(torch.bfloat16)
    out = torch.empty(xb.numel(), dtype=torch.int8, device="cuda")
    vit.vit_op_quantize_int8(xb.cuda(), xb.numel(), 2.5, out)
    np.testing.assert_array_equal(out.cpu().numpy(), Q.quantize_int8(xb.float().numpy(), 2.5))


def fma_model(acc, scale, bias):
    """fp32(fma(fp32(acc), scale, bias)) for exact integer sums acc, with the
    fused multiply-add evaluated exactly (rationals) and rounded once."""
    a32 = acc.astype(np.float64).astype(np.float32)            # int64 -> fp32, nearest even
    s = Fraction(float(np.float32(scale)))
    out = np.empty(acc.shape, np.float32)
    b = np.zeros(acc.shape[1], np.float32) if bias is None else np.asarray(bias, np.float32)
    bf = [Fraction(float(v)) for v in b]
    flat_a, flat_o = a32.reshape(-1), out.reshape(-1)
    N = acc.shape[1]
    for i, v in enumerate(flat_a):
        exact = Fraction(float(v)) * s + bf[i % N]
        # nearest float32 of a rational: round via float64 when that is exact, else by bracketing
        f64 = float(exact)
        c = np.float32(f64)
        if Fraction(f64) != exact or Fraction(float(c)) != exact:
            lo = np.float32(f64)
            cand = [np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))]
            c = min(cand, key=lambda z: (abs(Fraction(float(z)) - exact),
                                         int(np.array(z, np.float32).view(np.uint32)) & 1))
        flat_o[i] = c
    return out


def check_linear(qa, qw, scale, bias, out_f32, rows=None):
    M, K = qa.shape
    N = qw.shape[0]
    out = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    b = None if bias is None else torch.from_numpy(bias).cuda()
    vit.vit_op_linear_int8(codes_dev(qa), codes_dev(qw), M, N, K, scale, b, out)
    got = host(out)
    idx = np.arange(M) if rows is None else rows
    acc = Q.int8_products(qa[idx], qw)
    ref = Q.linear_int8(qa[idx], scale, qw, 1.0, bias)
    model = fma_model(acc, scale, bias)
    if not out_f32:
        model = host(torch.from_numpy(model).to(torch.bfloat16)).astype(np.float32)
    bound = 2.0 ** -24 * abs(scale) * np.abs(acc) + 2.0 ** -24 * np.abs(ref) \
        + (0 if out_f32 else 2.0 ** -8 * np.abs(ref)) + 1e-30
    err = np.abs(got[idx] - ref)
    same = (got[idx] == model.astype(np.float64)).mean()
    say(f"linear int8 {M}x{N}x{K} {'fp32' if out_f32 else 'bf16'}: max err / bound {(err / bound).max():.3f}, "
        f"{same:.5f} of outputs equal to the model")
    assert (err <= bound).all()
    np.testing.assert_array_equal(got[idx], model.astype(np.float64))


@pytest.mark.parametrize("M,N,K,out_f32,with_bias", [
    (1, 1, 128, True, False), (64, 64, 128, True, True), (300, 200, 384, True, True), (300, 200, 384, False, True),
    (1000, 130, 1536, True, False), (129, 1024, 256, False, False), (257, 130, 4096, True, True)])
def test_linear_int8_matches_model_bit_for_bit(M, N, K, out_f32, with_bias):
    require_gpu()
    rng = np.random.default_rng(M * 5 + N + K)
    qa = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, (N, K)).astype(np.int8)
    bias = rng.standard_normal(N).astype(np.float32) * 100 if with_bias else None
    check_linear(qa, qw, 3.0e-5, bias, out_f32)


@pytest.mark.parametrize("M,N,K", [(14272, 1536, 384), (14272, 384, 1536), (4101, 4096, 1024)])
def test_linear_int8_encoder_shapes_sampled(M, N, K):
    """The encoder's fc1 / fc2 shapes (ViT-S/16 @336 b32, ViT-L/16 @1024 b1) in
    int8, checked bit for bit on sampled rows (incl. the first and last tiles)."""
    require_gpu()
    rng = np.random.default_rng(K + 1)
    qa = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, (N, K)).astype(np.int8)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], rng.integers(0, M, 12)]))
    check_linear(qa, qw, 1.0 / 4096, rng.standard_normal(N).astype(np.float32), True, rows)


def test_linear_int8_extreme_sums():
    """Every product at +-127^2: sums up to 4096 * 16129 = 66M, past fp32's 2^24,
    so the conversion to fp32 rounds; sign patterns give every row a different sum."""
    require_gpu()
    rng = np.random.default_rng(29)
    M, N, K = 130, 70, 4096
    qa = np.where(rng.random((M, K)) < 0.5, -127, 127).astype(np.int8)
    qa[0] = 127
    qw = np.where(rng.random((N, K)) < 0.5, -127, 127).astype(np.int8)
    qw[0] = 127
    check_linear(qa, qw, 1.0, None, True)
    assert Q.int8_products(qa[:1], qw[:1])[0, 0] == K * 16129


def test_int8_rejects_bad_shapes():
    require_gpu()
    a = torch.zeros((4, 256), dtype=torch.int8, device="cuda")
    out = torch.empty((4, 4), device="cuda")
    for K in (0, 64, 200):
        with pytest.raises(vit.VitError):
            vit.vit_op_linear_int8(a, a, 4, 4, K, 1.0, None, out)
    with pytest.raises(vit.VitError):
        vit.vit_op_linear_int8(a, a, 4, 4, 256, float("nan"), None, out)


def test_quantized_int8_linear_end_to_end():
    """absmax -> per-tensor scales amax / 127 -> codes -> int8 GEMM, against the oracle on the same steps."""
    require_gpu()
    rng = np.random.default_rng(31)
    M, N, K = 500, 384, 384
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.02).astype(np.float32)
    xd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    amax = torch.empty(2, device="cuda")
    vit.vit_op_absmax(xd, x.size, amax[0:1])
    vit.vit_op_absmax(wd, w.size, amax[1:2])
    ax, aw = host(amax)
    sx, sw = np.float32(ax / 127.0), np.float32(aw / 127.0)
    qx = torch.empty((M, K), dtype=torch.int8, device="cuda")
    qw = torch.empty((N, K), dtype=torch.int8, device="cuda")
    vit.vit_op_quantize_int8(xd, x.size, float(np.float32(1.0) / sx), qx)
    vit.vit_op_quantize_int8(wd, w.size, float(np.float32(1.0) / sw), qw)
    qx_h, qw_h = qx.cpu().numpy(), qw.cpu().numpy()
    np.testing.assert_array_equal(qx_h, Q.quantize_int8(x, np.float32(1.0) / sx))
    np.testing.assert_array_equal(qw_h, Q.quantize_int8(w, np.float32(1.0) / sw))
    assert np.abs(qx_h).max() == 127 and np.abs(qw_h).max() == 127
    check_linear(qx_h, qw_h, float(np.float32(sx * sw)), bias, True)
    out = torch.empty((M, N), device="cuda")
    vit.vit_op_linear_int8(qx, qw, M, N, K, float(np.float32(sx * sw)), torch.from_numpy(bias).cuda(), out)
    y = x.astype(np.float64) @ w.T.astype(np.float64) + bias
    rel = np.abs(host(out) - y).max() / np.abs(y).max()
    say(f"int8 vs float64 linear: max error {rel:.3e} of max |y|")
    assert rel < 0.05
