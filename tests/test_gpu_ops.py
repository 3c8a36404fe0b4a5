"""Per-kernel parity: each C-ABI op on the GPU against the oracle on identical
(bf16-rounded) inputs, at sizes spanning several tiles with ragged tails.

Tolerances follow from the arithmetic (see the design notes): products of two
bf16 values are exact in fp32, so a K-term fp32 sum is within
K * 2^-24 * sum|a_k w_k| of the exact value; a bf16 output adds half an ulp,
at most 2^-8 |y|.  The attention core is judged by the rule in
tests/attention_gate.py: a worst-case bound per output plus a per-head rms gate,
both scaled to the outputs and the values they average.
"""

import math

import numpy as np
import pytest
import torch

import synth
import vision_transformer_encoder_block_amd as vit
from oracle import vit_oracle as O
from tests.attention_gate import accepted, attention_check, logit_factor, workload_qkv
from tests.gpu_util import bf16_dev, exact_ln_rows, f32_dev, host, require_gpu, say, vt_position

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(2024)
U24 = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# ------------------------------------------------------------------ LayerNorm

@pytest.mark.parametrize("rows,dim", [(1, 64), (7, 384), (446, 384), (1001, 1024), (33, 768)])
@pytest.mark.parametrize("out_fp32", [0, 1])
def test_layernorm(rows, dim, out_fp32):
    say(f"layernorm rows={rows} dim={dim} fp32={out_fp32}")
    x = RNG.standard_normal((rows, dim)).astype(np.float32) * 2 + 0.3
    g = (1 + 0.02 * RNG.standard_normal(dim)).astype(np.float32)
    b = (0.02 * RNG.standard_normal(dim)).astype(np.float32)
    y = torch.empty((rows, dim), dtype=torch.float32 if out_fp32 else torch.bfloat16, device="cuda")
    vit.vit_op_layernorm(f32_dev(x), rows, dim, f32_dev(g), f32_dev(b), 1e-6, y, out_fp32)
    got = host(y)
    ref = O.layer_norm(x.astype(np.float64), g, b, 1e-6)
    tol = (2.0 ** -8 * np.abs(ref) if not out_fp32 else 0) + 2e-5 * (1 + np.abs(ref))
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()


def _exact_ln_rows(rows, dim):
    """Rows whose LayerNorm is exact (gpu_util.exact_ln_rows); y = fl32(d/8 * g + b)
    with one fused multiply-add, d/8 exact."""
    return exact_ln_rows(RNG, rows, dim)


@pytest.mark.parametrize("rows,dim", [(5, 64), (33, 384), (7, 768), (41, 1024), (3, 1536)])
def test_layernorm_exact(rows, dim):
    """The LayerNorm kernel bit for bit on rows where every step is exact
    (see _exact_ln_rows), fp32 and bf16 outputs; it also pins rsqrt(64) = 1/8."""
    say(f"layernorm exact rows={rows} dim={dim}")
    x, d = _exact_ln_rows(rows, dim)
    g = (1 + 0.02 * RNG.standard_normal(dim)).astype(np.float32)
    b = (0.02 * RNG.standard_normal(dim)).astype(np.float32)
    model = ((d / 8.0) * g.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    y32 = torch.empty((rows, dim), dtype=torch.float32, device="cuda")
    vit.vit_op_layernorm(f32_dev(x), rows, dim, f32_dev(g), f32_dev(b), 1e-6, y32, 1)
    assert np.array_equal(host(y32), model), np.abs(host(y32) - model).max()
    y16 = torch.empty((rows, dim), dtype=torch.bfloat16, device="cuda")
    vit.vit_op_layernorm(f32_dev(x), rows, dim, f32_dev(g), f32_dev(b), 1e-6, y16, 0)
    assert np.array_equal(host(y16), host(torch.from_numpy(model).to(torch.bfloat16)))


@pytest.mark.parametrize("M", [64, 446, 1000])
def test_linear_residual_ln_exact(M):
    """The LayerNorm half of the fused residual + LN epilogue bit for bit: with
    A = 0 and a zero bias the update adds exactly 0, so x keeps the exact rows of
    _exact_ln_rows and h must be bf16(fl32(d/8 * g + b))."""
    say(f"linear residual ln exact M={M}")
    N = K = 384
    x, d = _exact_ln_rows(M, N)
    a_d, _ = bf16_dev(np.zeros((M, K)))
    w_d, _ = bf16_dev(RNG.standard_normal((N, K)) * 0.05)
    ls = np.full(N, 1e-5, np.float32)
    g = (1 + 0.02 * RNG.standard_normal(N)).astype(np.float32)
    b = (0.02 * RNG.standard_normal(N)).astype(np.float32)
    xd = f32_dev(x)
    h = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    vit.vit_op_linear_residual_ln(a_d, w_d, f32_dev(np.zeros(N, np.float32)), f32_dev(ls), M, N, K, xd, f32_dev(g),
                                  f32_dev(b), 1e-6, h)
    assert np.array_equal(host(xd), x)
    model = ((d / 8.0) * g.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    assert np.array_equal(host(h), host(torch.from_numpy(model).to(torch.bfloat16)))


WIDTHS = [64 * v for v in list(range(1, 17)) + [20, 24, 32, 48, 64]]


@pytest.mark.parametrize("dim", WIDTHS)
def test_layernorm_every_supported_width(dim):
    """Each supported width has its own lane layout (float4s per lane, lanes per
    row): 37 rows (two rows per wave for narrow widths, a ragged last pair) at
    every one, bf16 output."""
    say(f"layernorm width {dim}")
    rows = 37
    x = RNG.standard_normal((rows, dim)).astype(np.float32) * 1.5 - 0.2
    g = (1 + 0.02 * RNG.standard_normal(dim)).astype(np.float32)
    b = (0.02 * RNG.standard_normal(dim)).astype(np.float32)
    y = torch.empty((rows, dim), dtype=torch.bfloat16, device="cuda")
    vit.vit_op_layernorm(f32_dev(x), rows, dim, f32_dev(g), f32_dev(b), 1e-6, y, 0)
    ref = O.layer_norm(x.astype(np.float64), g, b, 1e-6)
    assert np.all(np.abs(host(y) - ref) <= 2.0 ** -8 * np.abs(ref) + 2e-5 * (1 + np.abs(ref)))


# ------------------------------------------------------------------ GEMM epilogues

SHAPES = [(1, 64, 64), (5, 150, 384), (130, 384, 384), (446, 1152, 384), (1000, 1536, 384), (257, 384, 1536),
          (4101, 1024, 128), (300, 96, 768),
          (3000, 3000, 640),   # 128 x 128 tiles, ragged in M and N
          (4160, 2000, 320),   # 8-wave 128 x 128 tiles (K <= 512) staging 16 rows at a time, ragged in M and N
          (4100, 8200, 192),   # 256 x 256 tiles (M N >= 32M), ragged in M and N
          # 128 x 128 tiles whose last full row tile also takes the 1..32 rows after it
          (4101, 4096, 128), (4128, 3072, 192), (3969, 2048, 256), (4100, 1024, 1024),
          # 256 x 256 tiles (>= 224 of them, W of >= 4M values) with 5 or 32 such rows
          (1285, 16384, 256), (1056, 16384, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("epi", [vit.EPI_BIAS_BF16, vit.EPI_GELU_BF16, vit.EPI_RESIDUAL, vit.EPI_BIAS_F32])
def test_linear(M, N, K, epi):
    say(f"linear M={M} N={N} K={K} epi={epi}")
    a_d, a = bf16_dev(RNG.standard_normal((M, K)) * 0.7)
    w_d, w = bf16_dev(RNG.standard_normal((N, K)) * 0.05)
    bias = (0.1 * RNG.standard_normal(N)).astype(np.float32)
    ls = (0.5 + RNG.standard_normal(N)).astype(np.float32)
    z = O.linear(a, w, bias)
    s_abs = np.abs(a) @ np.abs(w).T
    acc_err = K * U24 * s_abs + 1e-7
    if epi == vit.EPI_BIAS_BF16:
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ref, tol = z, 2.0 ** -8 * np.abs(z) + acc_err
    elif epi == vit.EPI_GELU_BF16:
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ref = O.gelu(z)
        tol = 2.0 ** -8 * np.abs(ref) + 1.13 * acc_err + 2e-6
    elif epi == vit.EPI_RESIDUAL:
        r0 = RNG.standard_normal((M, N)).astype(np.float32)
        out = f32_dev(r0)
        ref = r0 + ls * z
        tol = np.abs(ls) * acc_err + 4 * U24 * (np.abs(r0) + np.abs(ls * z))
    else:
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ref, tol = z, acc_err + 2 * U24 * np.abs(z)
    vit.vit_op_linear(a_d, w_d, f32_dev(bias), M, N, K, epi, f32_dev(ls), out)
    got = host(out)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], np.abs(got - ref).max())


def _unit_bf16(shape):
    """bf16 values of magnitude [1, 2): random sign and 7-bit mantissa."""
    m = RNG.integers(0, 128, shape)
    return (1.0 + m / 128.0) * np.where(RNG.integers(0, 2, shape) == 1, -1.0, 1.0)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("epi", [vit.EPI_BIAS_F32, vit.EPI_BIAS_BF16])
def test_linear_exact_groups(M, N, K, epi):
    """The GEMM's rounding, reproduced bit for bit.  With operands of magnitude
    [1, 2) (8 significant bits) each product has at most 16 and lies in [1, 4),
    so the 16 products one 32 x 32 x 16 MFMA adds sum to less than 2^6 with
    their lowest bit at 2^-14: 20 bits, exact in any adder of fp32 width.  The
    only roundings left are the fp32 accumulator taking each 16-wide k group in
    k order (to nearest even) and the epilogue's bias add, then the bf16 store.
    Every tile shape (64 x 64 .. 256 x 256, the extra rows of row tile 0,
    ragged edges) must give exactly that; a wrong k order, a dropped or doubled
    k group, or an extra rounding breaks it."""
    say(f"linear exact groups M={M} N={N} K={K} epi={epi}")
    a = _unit_bf16((M, K))
    w = _unit_bf16((N, K))
    a_d, a_r = bf16_dev(a)
    w_d, w_r = bf16_dev(w)
    assert np.array_equal(a_r, a) and np.array_equal(w_r, w)
    bias = (0.1 * RNG.standard_normal(N)).astype(np.float32)
    acc = np.zeros((M, N), np.float32)
    for g in range(0, K, 16):
        acc = (acc.astype(np.float64) + a[:, g:g + 16] @ w[:, g:g + 16].T).astype(np.float32)
    model = (acc.astype(np.float64) + bias.astype(np.float64)).astype(np.float32)
    if epi == vit.EPI_BIAS_F32:
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    else:
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        model = host(torch.from_numpy(model).to(torch.bfloat16))
    vit.vit_op_linear(a_d, w_d, f32_dev(bias), M, N, K, epi, None, out)
    got = host(out)
    diff = got != model
    say(f"  {diff.mean():.6f} of outputs differ from the accumulation model")
    assert not diff.any(), (np.argwhere(diff)[:5], np.abs(got - model).max())


@pytest.mark.parametrize("M,N,K", [(5, 150, 384), (1000, 1536, 384), (4101, 1024, 128), (4100, 1024, 1024),
                                   (4101, 1024, 1024), (4160, 2000, 320), (1285, 16384, 256)])
def test_linear_residual_exact_groups(M, N, K):
    """The residual epilogue x += ls * (acc + b) bit for bit, with the operands
    of test_linear_exact_groups and LayerScale values that are powers of two
    (so ls * t is exact and a fused or a separate multiply-add give the same
    bits): one rounding for acc + b, one for the update."""
    say(f"linear residual exact groups M={M} N={N} K={K}")
    a, w = _unit_bf16((M, K)), _unit_bf16((N, K))
    a_d, _ = bf16_dev(a)
    w_d, _ = bf16_dev(w)
    bias = (0.1 * RNG.standard_normal(N)).astype(np.float32)
    ls = (2.0 ** RNG.integers(-17, 2, N) * np.where(RNG.integers(0, 2, N) == 1, -1.0, 1.0)).astype(np.float32)
    r0 = RNG.standard_normal((M, N)).astype(np.float32)
    acc = np.zeros((M, N), np.float32)
    for g in range(0, K, 16):
        acc = (acc.astype(np.float64) + a[:, g:g + 16] @ w[:, g:g + 16].T).astype(np.float32)
    t = (acc.astype(np.float64) + bias).astype(np.float32)
    model = (r0.astype(np.float64) + ls.astype(np.float64) * t).astype(np.float32)
    x = f32_dev(r0)
    vit.vit_op_linear(a_d, w_d, f32_dev(bias), M, N, K, vit.EPI_RESIDUAL, f32_dev(ls), x)
    got = host(x)
    diff = got != model
    say(f"  {diff.mean():.6f} of outputs differ from the model")
    assert not diff.any(), (np.argwhere(diff)[:5], np.abs(got - model).max())


@pytest.mark.parametrize("batch,tokens,heads", [(2, 201, 6), (1, 446, 6), (3, 70, 2), (1, 4101, 16), (20, 446, 6)])
def test_qkv_exact_groups(batch, tokens, heads):
    """The fused Q/K/V projection bit for bit on operands whose k groups sum
    exactly (see test_linear_exact_groups): q = bf16((acc + b) * log2(e)/8) with
    two fp32 roundings, k = bf16(acc + b), and v = bf16(acc + b) at its permuted
    v^T column; 4101 x 16 heads takes the 256 x 256 tiles."""
    say(f"qkv exact groups batch={batch} tokens={tokens} heads={heads}")
    D = 64 * heads
    M = batch * tokens
    h, w = _unit_bf16((M, D)), _unit_bf16((3 * D, D))
    h_d, _ = bf16_dev(h)
    w_d, _ = bf16_dev(w)
    bias = (0.1 * RNG.standard_normal(3 * D)).astype(np.float32)
    nv = (tokens + 63) // 64 * 64
    q = torch.empty((batch, heads, tokens, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    vt = torch.zeros((batch, heads, 64, nv), dtype=torch.bfloat16, device="cuda")
    vit.vit_op_qkv(h_d, w_d, f32_dev(bias), batch, tokens, heads, q, k, vt)
    acc = np.zeros((M, 3 * D), np.float32)
    for g in range(0, D, 16):
        acc = (acc.astype(np.float64) + h[:, g:g + 16] @ w[:, g:g + 16].T).astype(np.float32)
    t = (acc.astype(np.float64) + bias).astype(np.float32)
    c = np.float32(math.log2(math.e) / 8.0)
    qs = (t[:, :D].astype(np.float64) * np.float64(c)).astype(np.float32)
    to_bf = lambda x: host(torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16))
    ref_q = to_bf(qs).reshape(batch, tokens, heads, 64).transpose(0, 2, 1, 3)
    ref_k = to_bf(t[:, D:2 * D]).reshape(batch, tokens, heads, 64).transpose(0, 2, 1, 3)
    ref_v = to_bf(t[:, 2 * D:]).reshape(batch, tokens, heads, 64).transpose(0, 2, 3, 1)   # [b, h, d, t]
    gq, gk, gv = host(q), host(k), host(vt)
    cols = vt_position(np.arange(tokens))
    assert np.array_equal(gq, ref_q)
    assert np.array_equal(gk, ref_k)
    assert np.array_equal(gv[:, :, :, cols], ref_v)


def _phi_table():
    """The GELU epilogue's table, built the way the library builds it on the
    host: Phi at -6 + i/64 (i < 769) from the C library's erfc in double, each
    entry (Phi_i, Phi_(i+1) - Phi_i) rounded to float (the last difference 0)."""
    tab = np.zeros((769, 2), np.float32)
    prev = 0.5 * math.erfc(6.0 / math.sqrt(2.0))
    for i in range(769):
        x1 = -6.0 + (i + 1) / 64.0
        nxt = 0.5 * math.erfc(-x1 / math.sqrt(2.0)) if i + 1 < 769 else prev
        tab[i] = (np.float32(prev), np.float32(nxt - prev))
        prev = nxt
    return tab


@pytest.mark.parametrize("M,N,K", [(1000, 1536, 384), (446, 1152, 384), (257, 384, 1536), (4101, 1024, 128),
                                   (4160, 2000, 320)])
def test_linear_gelu_exact_groups(M, N, K):
    """The GELU epilogue bit for bit.  Operands of magnitude [1, 2) / 16 keep
    every 16-product group exact (as in test_linear_exact_groups) and put the
    pre-activations z = fl32(acc + b) mostly inside the table's [-6, 6].  The
    kernel then computes t = clamp(fma(z, 64, 384), 0, 768), Phi =
    fma(fract(t), d_i, Phi_i) with i = int(t), y = fl32(z Phi) and rounds to
    bf16; the model below does the same on the same table.  (The fused
    products are exact in float64, so only a double rounding at a float
    midpoint, about one output in 2^29, could tell them apart.)"""
    say(f"linear gelu exact groups M={M} N={N} K={K}")
    a, w = _unit_bf16((M, K)) / 16.0, _unit_bf16((N, K)) / 16.0
    a_d, a_r = bf16_dev(a)
    w_d, w_r = bf16_dev(w)
    assert np.array_equal(a_r, a) and np.array_equal(w_r, w)
    bias = (0.5 * RNG.standard_normal(N)).astype(np.float32)
    acc = np.zeros((M, N), np.float32)
    for g in range(0, K, 16):
        acc = (acc.astype(np.float64) + a[:, g:g + 16] @ w[:, g:g + 16].T).astype(np.float32)
    z = (acc.astype(np.float64) + bias).astype(np.float32)
    tab = _phi_table()
    t = np.clip((z.astype(np.float64) * 64.0 + 384.0).astype(np.float32), np.float32(0), np.float32(768))
    i = t.astype(np.int32)
    f = (t - np.floor(t)).astype(np.float32)
    phi = (f.astype(np.float64) * tab[i, 1].astype(np.float64) + tab[i, 0].astype(np.float64)).astype(np.float32)
    y = (z.astype(np.float64) * phi.astype(np.float64)).astype(np.float32)
    model = host(torch.from_numpy(y).to(torch.bfloat16))
    inside = ((t > 0) & (t < 768)).mean()
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    vit.vit_op_linear(a_d, w_d, f32_dev(bias), M, N, K, vit.EPI_GELU_BF16, None, out)
    got = host(out)
    diff = got != model
    say(f"  {inside:.3f} of pre-activations inside the table, {diff.mean():.7f} of outputs differ from the model")
    assert inside > 0.9
    assert not diff.any(), (np.argwhere(diff)[:5], np.abs(got - model).max())


def test_gelu_epilogue_wide_range():
    """GELU over pre-activations spanning [-8, 8] (every step of 1/16, exact in
    bf16), so the clamped ends of the epilogue's Phi lookup are exercised:
    a = x in column 0, w = 1 in column 0, so acc = x exactly."""
    say("gelu epilogue wide range")
    x = np.arange(-128, 129, dtype=np.float64) / 16.0
    M, N, K = x.size, 64, 64
    a = np.zeros((M, K))
    a[:, 0] = x
    w = np.zeros((N, K))
    w[:, 0] = 1.0
    a_d, a_r = bf16_dev(a)
    w_d, _ = bf16_dev(w)
    assert np.array_equal(a_r[:, 0], x)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    vit.vit_op_linear(a_d, w_d, f32_dev(np.zeros(N, np.float32)), M, N, K, vit.EPI_GELU_BF16,
                      f32_dev(np.ones(N, np.float32)), out)
    ref = O.gelu(np.repeat(x[:, None], N, 1))
    got = host(out)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6), np.abs(got - ref).max()


@pytest.mark.parametrize("M,K", [(1, 64), (130, 384), (446, 1536), (14272, 384)])
def test_linear_residual_ln(M, K):
    """Residual update + the LayerNorm after it in one kernel: against the
    oracle, and bit for bit against the two separate entry points."""
    say(f"linear + residual + layernorm M={M} K={K}")
    N = 384
    a_d, a = bf16_dev(RNG.standard_normal((M, K)) * 0.7)
    w_d, w = bf16_dev(RNG.standard_normal((N, K)) * 0.05)
    bias = (0.1 * RNG.standard_normal(N)).astype(np.float32)
    ls = (0.5 + RNG.standard_normal(N)).astype(np.float32)
    g = (1.0 + 0.1 * RNG.standard_normal(N)).astype(np.float32)
    b = (0.1 * RNG.standard_normal(N)).astype(np.float32)
    r0 = RNG.standard_normal((M, N)).astype(np.float32)
    x = f32_dev(r0)
    h = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    vit.vit_op_linear_residual_ln(a_d, w_d, f32_dev(bias), f32_dev(ls), M, N, K, x, f32_dev(g), f32_dev(b), 1e-6, h)
    z = O.linear(a, w, bias)
    ref_x = r0 + ls * z
    tol_x = np.abs(ls) * K * U24 * (np.abs(a) @ np.abs(w).T) + 4 * U24 * (np.abs(r0) + np.abs(ls * z)) + 1e-7
    gx = host(x)
    assert np.all(np.abs(gx - ref_x) <= tol_x), np.abs(gx - ref_x).max()
    ref_h = O.layer_norm(gx.astype(np.float64), g, b, 1e-6)
    assert np.all(np.abs(host(h) - ref_h) <= 2.0 ** -8 * np.abs(ref_h) + 2e-5 * (1 + np.abs(ref_h)))
    # the unfused pair on the same inputs
    x2 = f32_dev(r0)
    h2 = torch.empty_like(h)
    vit.vit_op_linear(a_d, w_d, f32_dev(bias), M, N, K, vit.EPI_RESIDUAL, f32_dev(ls), x2)
    vit.vit_op_layernorm(x2, M, N, f32_dev(g), f32_dev(b), 1e-6, h2, 0)
    assert torch.equal(x, x2) and torch.equal(h.view(torch.int16), h2.view(torch.int16))


# ------------------------------------------------------------------ QKV head split

# the last three: 128-row tiles with a ragged last row tile of 5, 32 and 5 rows
# (ViT-L/16 @1024 b1), V^T columns included
@pytest.mark.parametrize("batch,tokens,heads", [(1, 5, 1), (2, 201, 6), (1, 446, 6), (3, 70, 2),
                                                (1, 133, 16), (2, 80, 10), (1, 4101, 16),
                                                (20, 446, 6)])  # 8-wave tiles, V^T staged 16 rows at a time
def test_qkv_split(batch, tokens, heads):
    say(f"qkv batch={batch} tokens={tokens} heads={heads}")
    D = 64 * heads
    M = batch * tokens
    h_d, h = bf16_dev(RNG.standard_normal((M, D)))
    w_d, w = bf16_dev(RNG.standard_normal((3 * D, D)) * 0.05)
    bias = (0.1 * RNG.standard_normal(3 * D)).astype(np.float32)
    nv = (tokens + 63) // 64 * 64
    q = torch.empty((batch, heads, tokens, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    vt = torch.zeros((batch, heads, 64, nv), dtype=torch.bfloat16, device="cuda")
    vit.vit_op_qkv(h_d, w_d, f32_dev(bias), batch, tokens, heads, q, k, vt)
    z = O.linear(h, w, bias).reshape(batch, tokens, 3, heads, 64)
    acc = (3 * D) * U24 * (np.abs(h) @ np.abs(w).T).reshape(batch, tokens, 3, heads, 64) + 1e-7
    c = math.log2(math.e) / 8.0
    ref_q = z[:, :, 0].transpose(0, 2, 1, 3) * c
    ref_k = z[:, :, 1].transpose(0, 2, 1, 3)
    ref_v = z[:, :, 2].transpose(0, 2, 3, 1)          # [b, h, d, t]
    gq, gk, gv = host(q), host(k), host(vt)
    assert np.all(np.abs(gq - ref_q) <= 2 ** -8 * np.abs(ref_q) + c * acc[:, :, 0].transpose(0, 2, 1, 3) + 1e-7)
    assert np.all(np.abs(gk - ref_k) <= 2 ** -8 * np.abs(ref_k) + acc[:, :, 1].transpose(0, 2, 1, 3))
    cols = vt_position(np.arange(tokens))
    gv_t = gv[:, :, :, cols]
    assert np.all(np.abs(gv_t - ref_v) <= 2 ** -8 * np.abs(ref_v) + acc[:, :, 2].transpose(0, 2, 3, 1))
    pad = np.setdiff1d(np.arange(nv), cols)
    assert np.all(gv[:, :, :, pad] == 0)  # not written


# ------------------------------------------------------------------ attention core

def _run_attention(q, k, v):
    """The kernel on float64 q, k, v [batch, heads, tokens, 64] (q pre-scaled by
    log2(e)/8); returns the bf16-rounded inputs it read and its output
    [batch, tokens, heads, 64]."""
    batch, heads, tokens, _ = q.shape
    nv = (tokens + 63) // 64 * 64
    q_d, q = bf16_dev(q)
    k_d, k = bf16_dev(k)
    v_d, v = bf16_dev(v)
    vt = torch.zeros((batch, heads, 64, nv), dtype=torch.bfloat16, device="cuda")
    vt[:, :, :, torch.from_numpy(vt_position(np.arange(tokens))).cuda()] = v_d.transpose(2, 3)
    o = torch.empty((batch, tokens, heads * 64), dtype=torch.bfloat16, device="cuda")
    vit.vit_op_attention(q_d, k_d, vt, batch, tokens, heads, o)
    return q, k, v, host(o).reshape(batch, tokens, heads, 64)


def _gate_heads(q, k, v, got):
    """Every (image, head) against the oracle under the attention rule."""
    worst = rms = 0.0
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            # q is pre-multiplied by log2(e)/8: softmax_2(q k^T) = softmax_e(ln2 * q k^T)
            ref, _ = O.sdpa(q[b, h], k[b, h], v[b, h], math.log(2.0))
            P = O.attention_weights(q[b, h], k[b, h], math.log(2.0))
            res = attention_check(got[b, :, h], ref, P, v[b, h], logit_factor(q[b, h], k[b, h]))
            worst, rms = max(worst, res["worst_ratio"]), max(rms, res["rms_ratio"])
            assert accepted(res), (b, h, res)
    say(f"  worst-case ratio {worst:.3f}, rms ratio {rms:.3f}")


@pytest.mark.parametrize("batch,tokens,heads", [
    (1, 1, 1), (1, 5, 1), (2, 31, 2), (1, 64, 1), (1, 65, 3), (2, 127, 1),
    (1, 129, 2), (2, 201, 6), (1, 446, 6), (1, 1370, 2), (1, 4101, 2), (2, 2053, 3), (1, 1100, 1),
    # last query tile with 33..64 rows (two busy waves), one row, none
    (1, 1064, 2), (2, 1153, 1), (1, 1024, 1), (1, 1280, 2),
    # last query tile of 1..32 rows, whose waves split the keys: 32 rows, 33
    # (not split), one key past a full tile, a last key tile of one key
    (1, 32, 1), (1, 160, 2), (1, 161, 1), (3, 4097, 1), (1, 2113, 2)])
def test_attention_matches_oracle(batch, tokens, heads):
    """N(0, 1) q and k: logits with a std of about 8 (log2 units), nearly one-hot rows."""
    say(f"attention N(0,1) batch={batch} tokens={tokens} heads={heads}")
    q, k, v, got = _run_attention(RNG.standard_normal((batch, heads, tokens, 64)),
                                  RNG.standard_normal((batch, heads, tokens, 64)),
                                  RNG.standard_normal((batch, heads, tokens, 64)))
    _gate_heads(q, k, v, got)


@pytest.mark.parametrize("batch,tokens,heads", [(1, 201, 6), (2, 446, 3), (1, 581, 4), (1, 1370, 2), (1, 2053, 2),
                                                (1, 4101, 2)])
@pytest.mark.parametrize("logit_std", [0.2, 2.0])
def test_attention_workload_logits(batch, tokens, heads, logit_std):
    """q, k, v as the encoder makes them (LayerNormed rows times N(0, 0.02)
    projections): near-uniform attention at a logit std of 0.2 (log2 units),
    and a peakier 2.0; every sequence length has a ragged last key tile."""
    say(f"attention workload logits std={logit_std} batch={batch} tokens={tokens} heads={heads}")
    q, k, v = workload_qkv(RNG, batch, tokens, heads, logit_std)
    _gate_heads(*_run_attention(q, k, v))


@pytest.mark.parametrize("batch,tokens,heads", [(1, 1, 1), (1, 5, 2), (2, 31, 2), (1, 64, 1), (1, 65, 3), (2, 129, 2),
                                                (2, 201, 6), (2, 446, 6), (1, 1370, 2), (1, 2053, 3), (1, 4101, 16),
                                                (1, 4097, 1), (1, 160, 2), (1, 161, 1)])
def test_attention_exact_powers_of_two(batch, tokens, heads):
    """The kernel bit for bit on inputs where every step is exact.  Each query
    is a unit vector e_r (r one of 8 channels), each key holds logits in
    {0, -1, -2, -3} on those channels, and keys 0, 32, 64 and 96 hold 0 on all
    of them, so every wave's first key block (whole tiles, or the 32-key halves
    of a key-split last query tile) contains the row maximum 0 and no rescale
    happens.  Then p = 2^s exactly, the values are bf16 of magnitude [1, 2)
    (7-bit mantissas), every partial sum of p v and of p is a multiple of 2^-10
    below 2^14 (24 bits) and so exact in fp32 in any order, and the output is
    bf16(fl32(O * fl32(1 / l))) with O = sum p v and l = sum p exact.  A wrong
    mask, key order, value column, query row or head, a dropped or doubled key
    tile, or a merge that weights the key-split partials wrongly breaks it."""
    say(f"attention exact powers of two batch={batch} tokens={tokens} heads={heads}")
    r = RNG.integers(0, 8, (batch, heads, tokens))
    q = np.zeros((batch, heads, tokens, 64))
    np.put_along_axis(q, r[..., None], 1.0, axis=3)
    k = np.zeros((batch, heads, tokens, 64))
    k[..., :8] = -RNG.integers(0, 4, (batch, heads, tokens, 8))
    for anchor in (0, 32, 64, 96):
        if anchor < tokens:
            k[:, :, anchor, :8] = 0.0
    v = (1.0 + RNG.integers(0, 128, (batch, heads, tokens, 64)) / 128.0) * \
        np.where(RNG.integers(0, 2, (batch, heads, tokens, 64)) == 1, -1.0, 1.0)
    qr, kr, vr, got = _run_attention(q, k, v)
    assert np.array_equal(qr, q) and np.array_equal(kr, k) and np.array_equal(vr, v)
    s = np.einsum("bhqc,bhkc->bhqk", q, k)                 # integers in [-3, 0]
    p = np.exp2(s)                                          # exact powers of two
    num = np.einsum("bhqk,bhkd->bhqd", p, v)                # exact (checked below)
    l = p.sum(axis=3)
    assert np.array_equal(num, np.round(num * 1024) / 1024)
    assert np.einsum("bhqk,bhkd->bhqd", p, np.abs(v)).max() < 2 ** 14
    inv = np.float32(1.0) / l.astype(np.float32)
    o32 = num.astype(np.float32) * inv[..., None]
    model = host(torch.from_numpy(np.ascontiguousarray(o32.transpose(0, 2, 1, 3))).to(torch.bfloat16))
    diff = got != model
    say(f"  {diff.mean():.6f} of outputs differ from the exact model")
    assert not diff.any(), (np.argwhere(diff)[:5], np.abs(got - model).max())
    # the model is the oracle's softmax attention up to the output rounding
    ref, _ = O.sdpa(q[0, 0], k[0, 0], v[0, 0], math.log(2.0))
    assert np.all(np.abs(model[0, :, 0] - ref) <= 2 ** -8 * np.abs(ref) + 1e-12)


# the spike in the first key tile, or in the third (it then moves the running
# max mid-row); at 150 tokens the last 22 queries sit in a key-split tile, and
# the merge must drop the partial results of the waves that never saw the spike
@pytest.mark.parametrize("tokens", [200, 150])
@pytest.mark.parametrize("spike", [3, 140])
def test_attention_large_logits_stay_finite(spike, tokens):
    # spike logit ~ 64 * 5000 * 8 * ln2 = 1.8e6, far beyond fp16's 65504; it wins every row
    say(f"attention large logits, spike at key {spike}, tokens {tokens}")
    e = RNG.choice([-1.0, 1.0], size=64)
    qr = 5000.0 * (e + 0.05 * RNG.standard_normal((1, 2, tokens, 64)))
    kr = RNG.standard_normal((1, 2, tokens, 64))
    kr[:, :, spike] = 8.0 * e
    q, k, v, got = _run_attention(qr, kr, RNG.standard_normal((1, 2, tokens, 64)))
    assert np.isfinite(got).all()
    for h in range(2):
        ref, smax = O.sdpa(q[0, h], k[0, h], v[0, h], math.log(2.0))
        assert smax > 1e6
        np.testing.assert_array_equal(ref, np.broadcast_to(v[0, h, spike], ref.shape))
        # one-hot rows: the output is that key's value row, rounded to bf16 (exact)
        np.testing.assert_allclose(got[0, :, h], ref, atol=2 ** -8 * np.abs(ref).max() + 1e-6)


# Logits (log2 units) about `jump` higher in every key tile after the first, for
# every query: 5 leaves each p <= 2^8 but lane sums of 32 p far above 2^8; 12
# and 40 exceed the running max by more than 8 and move it on the second tile.
@pytest.mark.parametrize("tokens", [300, 280])   # 280: the last 24 queries split the keys
@pytest.mark.parametrize("jump", [5.0, 12.0, 40.0])
def test_attention_rising_logits(jump, tokens):
    say(f"attention rising logits, jump {jump}, tokens {tokens}")
    batch, heads = 1, 2
    e = RNG.choice([-1.0, 1.0], size=64)
    qr = e + 0.05 * RNG.standard_normal((batch, heads, tokens, 64))
    kr = 0.02 * RNG.standard_normal((batch, heads, tokens, 64))
    kr[:, :, 64:] += jump / 64.0 * e
    _gate_heads(*_run_attention(qr, kr, RNG.standard_normal((batch, heads, tokens, 64))))


# ------------------------------------------------------------------ frame preprocessing

@pytest.mark.parametrize("batch,src,dst,bgr", [(2, (720, 1280), (336, 336), True), (1, (37, 53), (45, 31), False),
                                               (3, (100, 150), (224, 224), False), (1, (518, 518), (518, 518), True),
                                               (1, (1, 1), (3, 2), False),
                                               # rows of 5000 pixels: wider than the staged-row buffer
                                               (1, (40, 5000), (30, 700), True)])
def test_preprocess(batch, src, dst, bgr):
    say(f"preprocess batch={batch} {src} -> {dst} bgr={bgr}")
    frames = RNG.integers(0, 256, size=(batch,) + src + (3,), dtype=np.uint8)
    fd = torch.from_numpy(frames).cuda()
    out = torch.empty((batch, 3) + dst, dtype=torch.float32, device="cuda")
    vit.vit_op_preprocess(fd, batch, src[0], src[1], bgr, out, dst[0], dst[1])
    ref = O.preprocess(frames, *dst, bgr=bgr)
    # fp32 weights and sums on values <= 255, then /255/std (std >= 0.224)
    np.testing.assert_allclose(host(out), ref, rtol=0, atol=2e-5)

