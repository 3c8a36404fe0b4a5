"""Plain CPU oracle for the low-precision (fp8) linear layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the GPU library shares no code
with it.

What it computes: a Linear layer y = x W^T + b (the encoder's Linears,
LibreYOLO DINOv2 diagram "Encoder block") with both operands quantised to
8-bit floating point, the "low precision" the DINOv2 deployment article
discusses for its engines (INT8 / reduced-precision builds).  The format is the
OCP 8-bit E4M3 ("fp8 e4m3fn") format that gfx950's matrix cores read:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0: subnormals m / 8 * 2^-6; fields 1..15: (1 + m / 8) * 2^(e - 7);
* exponent 15 with mantissa 7 (codes 0x7F and 0xFF) is NaN; there is no
  infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.

Quantisation of a value x with a per-tensor reciprocal scale s_inv:
v = float32(x) * float32(s_inv) rounded once in float32 (the decision is taken
in the kernel's precision, as both sides must), then the nearest E4M3 value,
ties to the code with an even mantissa, saturated to +-448; NaN stays NaN.
Dequantisation multiplies the decoded value by the scale.  The quantised
product is the float64 matrix product of the dequantised operands.

Readings (listed in the design notes): per-tensor scales; saturation (not
NaN) for magnitudes past 448; ties to even.

The same layer with 8-bit integer operands (the INT8 builds the deployment
article mentions): symmetric per-tensor quantisation q = the integer nearest
to float32(x) * float32(s_inv), ties to even, clamped to [-127, 127] (the
code -128 is left unused so that the range is symmetric), NaN -> 0.  The
products are integers and their sums are exact, so the layer is
y = sa * sw * (qa qw^T) + b with the integer matrix product taken exactly.

Parity status: pinned by ``tests/test_oracle_quant.py`` (torch's float8_e4m3fn
cast for every value in range, the format's closed-form extremes, brute force
on tiny products; for int8, torch's qint8 quantisation in range, brute-force
nearest integers, saturation and the closed-form all-extreme product).
"""

from __future__ import annotations

import numpy as np

F64 = np.float64
E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The value of an 8-bit E4M3 code (NaN for 0x7F / 0xFF)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=F64)


def quantize_e4m3(x: np.ndarray, s_inv: float) -> np.ndarray:
    """Codes (uint8) of x * s_inv (product in float32): the nearest E4M3 value, ties to
    the code with an even mantissa, magnitudes past 448 saturated, the sign kept
    (also for results that round to zero); NaN gives 0x7F."""
    v = (np.asarray(x, np.float32) * np.float32(s_inv)).astype(F64)
    mags = E4M3_TABLE[:0x7F]                       # codes 0x00 .. 0x7E: 0 .. 448, increasing
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - mags[lo], mags[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def dequantize_e4m3(codes: np.ndarray, scale: float) -> np.ndarray:
    """Decoded values times the scale (float64)."""
    return E4M3_TABLE[np.asarray(codes, np.uint8)] * F64(scale)


def linear_fp8(qa: np.ndarray, sa: float, qw: np.ndarray, sw: float, bias: np.ndarray | None) -> np.ndarray:
    """y = dequant(qa) @ dequant(qw)^T + b with qa [M, K], qw [N, K] E4M3 codes."""
    y = dequantize_e4m3(qa, sa) @ dequantize_e4m3(qw, sw).T
    if bias is not None:
        y = y + np.asarray(bias, F64)
    return y


INT8_MAX = 127


def quantize_int8(x: np.ndarray, s_inv: float) -> np.ndarray:
    """Codes (int8) of x * s_inv (product in float32): the nearest integer, ties
    to even, clamped to [-127, 127] (infinities included); NaN gives 0."""
    v = (np.asarray(x, np.float32) * np.float32(s_inv)).astype(F64)
    q = np.clip(np.rint(np.nan_to_num(v, nan=0.0, posinf=INT8_MAX, neginf=-INT8_MAX)), -INT8_MAX, INT8_MAX)
    return q.astype(np.int8)


def dequantize_int8(codes: np.ndarray, scale: float) -> np.ndarray:
    """Codes times the scale (float64)."""
    return np.asarray(codes, F64) * F64(scale)


def int8_products(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """The exact integer sums qa qw^T (int64) of qa [M, K] and qw [N, K] codes."""
    return np.asarray(qa, np.int64) @ np.asarray(qw, np.int64).T


def linear_int8(qa: np.ndarray, sa: float, qw: np.ndarray, sw: float, bias: np.ndarray | None) -> np.ndarray:
    """y = sa * sw * (qa qw^T) + b with qa [M, K], qw [N, K] int8 codes."""
    y = int8_products(qa, qw).astype(F64) * (F64(sa) * F64(sw))
    if bias is not None:
        y = y + np.asarray(bias, F64)
    return y
