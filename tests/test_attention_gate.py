"""The attention acceptance rule (tests/attention_gate.py) pinned on the CPU.

A model of the kernel's arithmetic, written here from its documented roundings
(fp32 logits of bf16 q and k, p = 2^(s - max) in fp32, p rounded to bf16 for
P.V, fp32 row sums, output rounded to bf16), must pass the rule at every logit
scale.  Two plausible kernel mistakes, planted in that model on the CPU, must
fail it in the near-uniform regime the encoder runs in (logits of about 0.2 in
log2 units: LayerNormed tokens times N(0, 0.02) projections) and in a peakier
one: a softmax denominator that misses the ragged last key tile, and the last
tile's values shifted by one key.
"""

import math

import numpy as np
import pytest

import synth
from oracle import vit_oracle as O
from tests.attention_gate import accepted, attention_check, logit_factor, workload_qkv


def _bf16(a):
    return synth.round_bf16(np.asarray(a, np.float32)).astype(np.float64)


def _kernel_model(q, k, v, den_keys=None, v_used=None):
    """The kernel's roundings on one head (float32 logits and probabilities).
    den_keys: keys summed into the denominator (a planted mistake when short);
    v_used: the values multiplied by P (a planted mistake when permuted)."""
    s = q.astype(np.float32) @ k.astype(np.float32).T
    p = np.exp2(s - s.max(axis=1, keepdims=True)).astype(np.float32)
    num = _bf16(p) @ (v if v_used is None else v_used)
    den = p[:, : (den_keys or p.shape[1])].astype(np.float64).sum(axis=1, keepdims=True)
    return _bf16(num / den)


def _case(tokens, logit_std, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (_bf16(a[0, 0]) for a in workload_qkv(rng, 1, tokens, 1, logit_std))
    ref, _ = O.sdpa(q, k, v, math.log(2.0))
    P = O.attention_weights(q, k, math.log(2.0))
    return q, k, v, ref, P, logit_factor(q, k)


@pytest.mark.parametrize("tokens", [201, 446, 581, 1370, 2053, 4101])
@pytest.mark.parametrize("logit_std", [0.2, 2.0])
def test_rule_accepts_the_kernel_roundings(tokens, logit_std):
    q, k, v, ref, P, L = _case(tokens, logit_std, 11 + tokens)
    logits = q @ k.T
    assert 0.5 * logit_std < logits.std() < 2.0 * logit_std
    res = attention_check(_kernel_model(q, k, v), ref, P, v, L)
    assert accepted(res), res
    # the model's rms sits well inside the statistical gate
    assert res["rms_ratio"] < 0.7, res


# At 4101 near-uniform tokens the 5 shifted keys move the outputs by about 1.5x
# their rounding noise, inside the gate's margin; the peaky regime still shows it.
@pytest.mark.parametrize("tokens,logit_std", [(n, s) for n in (201, 446, 581, 1370, 2053, 4101) for s in (0.2, 2.0)
                                              if (n, s) != (4101, 0.2)])
def test_rule_rejects_values_shifted_in_the_last_tile(tokens, logit_std):
    q, k, v, ref, P, L = _case(tokens, logit_std, 11 + tokens)
    last = (tokens - 1) // 64 * 64
    vs = v.copy()
    vs[last:-1] = v[last + 1:]
    vs[-1] = 0.0                       # the zero padding past the sequence end
    res = attention_check(_kernel_model(q, k, v, v_used=vs), ref, P, v, L)
    assert not accepted(res), res


# The missing keys carry 4.5% (201), 14% (446), 0.9% (581) and 1.9% (1370) of
# the probability mass in the near-uniform regime; 5 keys of 2053 or 4101
# (0.24%, 0.12%) move the outputs by less than their bf16 rounding, which no
# rule can tell apart from rounding.
@pytest.mark.parametrize("tokens", [201, 446, 581, 1370])
@pytest.mark.parametrize("logit_std", [0.2, 2.0])
def test_rule_rejects_a_denominator_without_the_last_tile(tokens, logit_std):
    q, k, v, ref, P, L = _case(tokens, logit_std, 11 + tokens)
    last = (tokens - 1) // 64 * 64
    res = attention_check(_kernel_model(q, k, v, den_keys=last), ref, P, v, L)
    assert not accepted(res), res


def test_a_bound_on_the_value_range_is_blind_near_uniform():
    """Why the bound scales with the output: near-uniform attention at 446
    tokens averages the values down to about 1/20 of their range, and an
    absolute term of 2^-7 max|v| passes both planted mistakes."""
    q, k, v, ref, P, L = _case(446, 0.2, 11 + 446)
    vs = v.copy()
    vs[384:-1] = v[385:]
    vs[-1] = 0.0
    for bad in (_kernel_model(q, k, v, den_keys=384), _kernel_model(q, k, v, v_used=vs)):
        assert np.all(np.abs(bad - ref) <= 2 ** -8 * np.abs(ref) + 2 ** -7 * np.abs(v).max())
        assert not accepted(attention_check(bad, ref, P, v, L))


def test_rule_accepts_exact_and_rejects_a_uniform_drift():
    q, k, v, ref, P, L = _case(446, 0.2, 5)
    assert accepted(attention_check(ref.copy(), ref, P, v, L))
    assert not accepted(attention_check(ref * 1.02, ref, P, v, L))
