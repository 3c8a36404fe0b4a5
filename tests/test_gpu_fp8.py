"""GPU parity of the fp8 (OCP E4M3) linear layer against the quantised oracle.

Codes are integers decided from the same float32 product on both sides, so they
must agree bit for bit.

The GEMM multiplies E4M3 values, whose products are exact.  With codes of
magnitude [1, 4) every 64-product group sums exactly in 16 bits, so the only
rounding is the fp32 accumulation across groups: those cases take a bound
derived from that alone and must match a model of the accumulation bit for bit
(test_linear_fp8_exact_groups).  Measured on the gfx950 matrix core, a single
product and any sum whose products lie within a few octaves are exact as well.  Each instruction adds its 64 products with a
limited number of bits below the largest of them: when one group mixes
magnitudes far apart, its error measured up to 2^-11.1 of its largest product
(random codes over the whole E4M3 range).  The bound is therefore, per output,
scale * (sum over the K / 64 groups of 2^-10 max_group |a w|
         + K 2^-24 sum |a w|)          (fp32 accumulation across groups)
+ 2^-23 |y| for the final scaling, and 2^-8 |y| more for bf16 output.
"""

import numpy as np
import pytest
import torch

import vision_transformer_encoder_block_amd as vit
from gpu_util import host, require_gpu, say
from oracle import quant_oracle as Q

pytestmark = pytest.mark.gpu


def codes_dev(q):
    return torch.from_numpy(np.ascontiguousarray(q, np.uint8)).cuda()


SPECIAL = np.array([0.0, -0.0, 1e-12, -1e-12, np.nan, np.inf, -np.inf, 448.0, 464.0, 465.0, -500.0, 3.625, 3.375,
                    2.0 ** -9, 1.5 * 2.0 ** -9, 2.0 ** -10, 0.0159, 240.0, 248.0, 256.0], np.float32)


@pytest.mark.parametrize("n,s_inv", [(1, 1.0), (3, 0.5), (4099, 7.3), (1 << 20, 0.013)])
def test_quantize_codes_bit_exact(n, s_inv):
    require_gpu()
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 60).astype(np.float32)
    x[: min(n, SPECIAL.size)] = SPECIAL[: min(n, SPECIAL.size)]
    out = torch.empty(n, dtype=torch.uint8, device="cuda")
    vit.vit_op_quantize_fp8(torch.from_numpy(x).cuda(), n, s_inv, out)
    got = out.cpu().numpy()
    ref = Q.quantize_e4m3(x, s_inv)
    bad = np.flatnonzero(got != ref)
    say(f"quantize n={n}: {bad.size} mismatches")
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_quantize_from_bf16_bit_exact():
    require_gpu()
    rng = np.random.default_rng(2)
    xb = torch.from_numpy((rng.standard_normal(100003) * 30).astype(np.float32)).to(torch.bfloat16)
    out = torch.empty(xb.numel(), dtype=torch.uint8, device="cuda")
    vit.vit_op_quantize_fp8(xb.cuda(), xb.numel(), 2.5, out)
    np.testing.assert_array_equal(out.cpu().numpy(), Q.quantize_e4m3(xb.float().numpy(), 2.5))


def test_absmax():
    require_gpu()
    rng = np.random.default_rng(4)
    x = rng.standard_normal(5_000_001).astype(np.float32)
    x[123456] = -77.25
    x[7] = np.nan
    amax = torch.empty(1, device="cuda")
    xd = torch.from_numpy(x).cuda()
    vit.vit_op_absmax(xd, x.size, amax)
    assert host(amax)[0] == 77.25
    vit.vit_op_absmax(xd[:100], 100, amax)      # overwritten, not accumulated
    assert host(amax)[0] == np.nanmax(np.abs(x[:100]))


def random_codes(rng, shape):
    """Finite E4M3 codes of both signs (no NaN codes)."""
    c = rng.integers(0, 0x7F, shape).astype(np.uint8)
    return c | (rng.integers(0, 2, shape).astype(np.uint8) << 7)


def check_linear(qa, qw, scale, bias, out_f32, rows=None):
    M, K = qa.shape
    N = qw.shape[0]
    out = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    b = None if bias is None else torch.from_numpy(bias).cuda()
    vit.vit_op_linear_fp8(codes_dev(qa), codes_dev(qw), M, N, K, scale, b, out)
    got = host(out)
    idx = np.arange(M) if rows is None else rows
    ref = Q.linear_fp8(qa[idx], scale, qw, 1.0, bias)
    A, Wd = np.abs(Q.dequantize_e4m3(qa[idx], 1.0)), np.abs(Q.dequantize_e4m3(qw, 1.0))
    absp = A @ Wd.T
    group_max = np.zeros_like(absp)           # sum over 64-wide K groups of the largest |a w|
    for g in range(0, K, 64):
        for r in range(A.shape[0]):
            group_max[r] += (A[r, None, g:g + 64] * Wd[:, g:g + 64]).max(axis=1)
    bound = scale * (2.0 ** -10 * group_max + K * 2.0 ** -24 * absp) + 2.0 ** -23 * np.abs(ref) \
        + (0 if out_f32 else 2.0 ** -8 * np.abs(ref)) + 1e-30
    err = np.abs(got[idx] - ref)
    say(f"linear fp8 {M}x{N}x{K} {'fp32' if out_f32 else 'bf16'}: max err / bound = {(err / bound).max():.3f}")
    assert (err <= bound).all()


@pytest.mark.parametrize("M,N,K,out_f32,with_bias", [
    (1, 1, 128, True, False), (64, 64, 128, True, True), (300, 200, 384, True, True), (300, 200, 384, False, True),
    (1000, 130, 1536, True, False), (129, 1024, 256, False, False)])
def test_linear_fp8_matches_oracle(M, N, K, out_f32, with_bias):
    require_gpu()
    rng = np.random.default_rng(M * 7 + N + K)
    qa, qw = random_codes(rng, (M, K)), random_codes(rng, (N, K))
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    check_linear(qa, qw, 0.01, bias, out_f32)


@pytest.mark.parametrize("M,N,K", [(14272, 1536, 384), (14272, 384, 1536), (4101, 4096, 1024)])
def test_linear_fp8_encoder_shapes_sampled(M, N, K):
    """The encoder's fc1 / fc2 shapes (ViT-S/16 @336 b32, ViT-L/16 @1024 b1) in fp8,
    checked on sampled rows (incl. the first and last tiles)."""
    require_gpu()
    rng = np.random.default_rng(K)
    qa, qw = random_codes(rng, (M, K)), random_codes(rng, (N, K))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], rng.integers(0, M, 60)]))
    check_linear(qa, qw, 1.0 / 64, rng.standard_normal(N).astype(np.float32), True, rows)


def narrow_codes(rng, shape):
    """E4M3 codes of magnitude in [1, 4) (exponent fields 7 and 8, any mantissa), both signs."""
    c = rng.integers(0x38, 0x48, shape).astype(np.uint8)
    return c | (rng.integers(0, 2, shape).astype(np.uint8) << 7)


def group_accumulation_model(qa, qw, scale, bias):
    """The kernel's arithmetic when every 64-product group sums exactly: E4M3
    values of magnitude [1, 4) have 4 significant bits, so their products have
    at most 8 and lie in [1, 16); a group of 64 then sums to less than 2^10
    with its lowest bit at 2^-6, 16 bits that any adder of fp32 width or more
    holds exactly.  The instructions add their group sums to the fp32
    accumulator in k order, one rounding (to nearest even) per group; the
    epilogue is one fp32 fma (acc * scale + bias)."""
    A, W = Q.dequantize_e4m3(qa, 1.0), Q.dequantize_e4m3(qw, 1.0)
    K = A.shape[1]
    acc = np.zeros((A.shape[0], W.shape[0]), np.float32)
    for g in range(0, K, 64):
        acc = (acc.astype(np.float64) + A[:, g:g + 64] @ W[:, g:g + 64].T).astype(np.float32)
    y = acc.astype(np.float64) * np.float64(np.float32(scale))
    if bias is not None:
        y = y + bias.astype(np.float64)
    return y.astype(np.float32), np.abs(A) @ np.abs(W).T


@pytest.mark.parametrize("M,N,K,out_f32", [(300, 200, 1536, True), (257, 130, 4096, True), (300, 200, 1536, False)])
def test_linear_fp8_exact_groups(M, N, K, out_f32):
    """Codes whose group sums are exact: the only error left is the fp32
    accumulation across the K / 64 groups, a bound that follows from the
    arithmetic alone, |err| <= scale (K / 64 - 1) 2^-24 sum |a w| + 2^-24 |y|
    (+ 2^-8 |y| for bf16 out).  Beyond the bound, the kernel must reproduce the
    model of that accumulation above bit for bit (also after the bf16 rounding):
    a wrong group order, a dropped or doubled group, a wrong scale or an extra
    rounding step all break it."""
    require_gpu()
    rng = np.random.default_rng(M + N + K)
    qa, qw = narrow_codes(rng, (M, K)), narrow_codes(rng, (N, K))
    bias = rng.standard_normal(N).astype(np.float32)
    scale = 0.01
    out = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    vit.vit_op_linear_fp8(codes_dev(qa), codes_dev(qw), M, N, K, scale, torch.from_numpy(bias).cuda(), out)
    got = host(out).astype(np.float64)
    model, absp = group_accumulation_model(qa, qw, scale, bias)
    ref = Q.linear_fp8(qa, scale, qw, 1.0, bias)
    bound = np.float32(scale) * (K // 64 - 1) * 2.0 ** -24 * absp + 2.0 ** -24 * np.abs(ref) \
        + (0 if out_f32 else 2.0 ** -8 * np.abs(ref)) + 1e-30
    err = np.abs(got - ref)
    model64 = model.astype(np.float64)
    if not out_f32:
        model64 = host(torch.from_numpy(model).to(torch.bfloat16)).astype(np.float64)
    off = np.abs(got - model64) / np.maximum(np.spacing(np.abs(model).astype(np.float32)).astype(np.float64), 1e-45)
    say(f"fp8 exact groups {M}x{N}x{K} {'fp32' if out_f32 else 'bf16'}: max err / bound {(err / bound).max():.3f}, "
        f"{(got == model64).mean():.4f} of outputs equal to the accumulation model, max {off.max():.1f} fp32 units off")
    assert (err <= bound).all()
    assert off.max() == 0.0


def test_quantized_linear_end_to_end():
    """absmax -> per-tensor scales -> codes -> fp8 GEMM, against the oracle on the same steps."""
    require_gpu()
    rng = np.random.default_rng(17)
    M, N, K = 500, 384, 384
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.02).astype(np.float32)
    xd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    amax = torch.empty(2, device="cuda")
    vit.vit_op_absmax(xd, x.size, amax[0:1])
    vit.vit_op_absmax(wd, w.size, amax[1:2])
    ax, aw = host(amax)
    assert ax == np.abs(x).max() and aw == np.abs(w).max()
    sx, sw = np.float32(ax / 448.0), np.float32(aw / 448.0)
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    vit.vit_op_quantize_fp8(xd, x.size, float(np.float32(1.0) / sx), qx)
    vit.vit_op_quantize_fp8(wd, w.size, float(np.float32(1.0) / sw), qw)
    qx_h, qw_h = qx.cpu().numpy(), qw.cpu().numpy()
    np.testing.assert_array_equal(qx_h, Q.quantize_e4m3(x, np.float32(1.0) / sx))
    np.testing.assert_array_equal(qw_h, Q.quantize_e4m3(w, np.float32(1.0) / sw))
    check_linear(qx_h, qw_h, float(np.float32(sx * sw)), bias, True)
    # and the quantised layer stays close to the full-precision one (E4M3 keeps 3 mantissa bits)
    out = torch.empty((M, N), device="cuda")
    vit.vit_op_linear_fp8(qx, qw, M, N, K, float(np.float32(sx * sw)), torch.from_numpy(bias).cuda(), out)
    y = x.astype(np.float64) @ w.T.astype(np.float64) + bias
    rel = np.abs(host(out) - y).max() / np.abs(y).max()
    say(f"fp8 vs float64 linear: max error {rel:.3e} of max |y|")
    assert rel < 0.1
