"""Acceptance rule for the attention core's bf16 output against the float64 oracle.

Host-side test helper: it takes the oracle's softmax weights and output for the
same bf16 q, k, v the kernel reads and decides whether the kernel's output is
within what its roundings allow.  The kernel forms the logits in fp32 from bf16
q and k (log2 units), the probabilities p = 2^(s - m) in fp32, rounds them to
bf16 for the P.V product, sums the fp32 p, and rounds o = (P.V) / l to bf16.
Against the exact softmax(q k^T) v of the same inputs that leaves:

* each probability rounded to bf16: p_j (1 + d_j), |d_j| <= u = 2^-8, the unit
  roundoff of bf16 with round-to-nearest-even;
* fp32 logits: an error of at most 70 * 2^-24 * (sum_c |q_c k_jc| + |m|) on
  s_j - m (64 products and the three parts of -m), which changes p_j by the
  factor 2^e, i.e. by at most L = ln2 * that + 2^-23 (exp2's own error);
* fp32 sums over the N keys in the numerator and the denominator: N * 2^-24
  relative each;
* the output rounded to bf16: |r| <= u.

Per output element (query i, channel c), with A = sum_j p_j |v_jc| (the
softmax weights p sum to 1):

    |o_gpu - o| <= u |o| + (1 + u) E,   E = (u (1 + 2L) + 2L + 2N 2^-24) A     (worst case)

The rounding errors d_j and r have random signs.  A rounding error is spread
evenly over half an ulp either side, and an ulp is at most 2u times the value,
so its variance is at most u^2/3 of the value squared; summed over the keys:

    E[err^2] <= (u^2 / 3) (o^2 + B^2),   B^2 = sum_j p_j^2 v_jc^2.

The statistical gate asks, per (image, head), that the rms error over all its
outputs be at most 1.25 times the rms that model predicts, plus the rms of the
non-rounding part (2L + 2N 2^-24) A.  The model bounds the expected square from
above, and over the thousands of outputs of one head the observed rms stays
within a few percent of its expectation, so 1.25 is margin for that spread: a
result that drifts by a fraction of the outputs' own size fails the gate at any
logit scale, where the worst-case bound alone passes errors as large as u * A
(for near-uniform attention over N keys, A is about sqrt(N) times |o|).
"""

from __future__ import annotations

import math

import numpy as np

U = 2.0 ** -8          # bf16 unit roundoff (round to nearest even)
U24 = 2.0 ** -24       # fp32 unit roundoff


def logit_factor(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """L per query row: the largest relative change of any p_j from the fp32
    logit arithmetic (q, k as the kernel reads them, logits in log2 units)."""
    s = q @ k.T
    qk = np.abs(q) @ np.abs(k).T
    m = np.abs(s).max(axis=1) + 8.0        # the kernel's reference max lags the row max by <= 8
    return math.log(2.0) * 70 * U24 * (qk.max(axis=1) + m) + 2 * U24


def attention_check(got: np.ndarray, ref: np.ndarray, P: np.ndarray, v: np.ndarray, L: np.ndarray) -> dict:
    """Compare one head's kernel output `got` [N, c] with the oracle `ref` [N, c]
    given the oracle's weights P [N, M] and the values v [M, c].

    Returns the worst-case verdict (`elementwise_ok`), the statistical one
    (`rms_ok`), and the numbers behind them."""
    n_keys = P.shape[1]
    A = P @ np.abs(v)
    B2 = (P * P) @ (v * v)
    E = (U * (1 + 2 * L[:, None]) + 2 * L[:, None] + 2 * n_keys * U24) * A
    bound = U * np.abs(ref) + (1 + U) * E + 1e-30
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(err ** 2)))
    model = float(np.sqrt(np.mean(U * U / 3.0 * (ref ** 2 + B2))))
    fixed = float(np.sqrt(np.mean(((2 * L[:, None] + 2 * n_keys * U24) * A) ** 2)))
    rms_bound = 1.25 * model + fixed
    return dict(elementwise_ok=bool(np.all(err <= bound)), rms_ok=bool(rms <= rms_bound),
                worst_ratio=float((err / bound).max()), rms=rms, rms_bound=rms_bound,
                rms_ratio=rms / rms_bound if rms_bound > 0 else 0.0,
                rel_rms=rms / max(float(np.sqrt(np.mean(ref ** 2))), 1e-300))


def accepted(res: dict) -> bool:
    return res["elementwise_ok"] and res["rms_ok"]


def workload_qkv(rng: np.random.Generator, batch: int, tokens: int, heads: int, logit_std: float, dim: int = 384):
    """q, k, v shaped like the encoder's: unit-scale token rows (LayerNorm
    outputs) times N(0, 0.02) projections plus N(0, 0.02) biases, per head.
    q and k are scaled by the same factor so that the logits q.k / 8 have about
    `logit_std` (log2 units); q is returned pre-multiplied by log2(e)/8, as the
    kernel takes it.  Returns float64 arrays [batch, heads, tokens, 64]."""
    x = rng.standard_normal((batch, tokens, dim))
    w = rng.standard_normal((3, heads, dim, 64)) * 0.02
    b = rng.standard_normal((3, heads, 1, 64)) * 0.02
    q = np.einsum("btd,hdc->bhtc", x, w[0]) + b[0]
    k = np.einsum("btd,hdc->bhtc", x, w[1]) + b[1]
    v = np.einsum("btd,hdc->bhtc", x, w[2]) + b[2]
    natural = 0.02 * 0.02 * dim            # std of q.k / 8 for the unscaled projections (64 terms / 8)
    g = math.sqrt(logit_std / (natural * math.log2(math.e)))
    return q * g * (math.log2(math.e) / 8.0), k * g, v
