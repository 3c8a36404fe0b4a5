"""Helpers shared by the GPU parity tests (marshalling only, no arithmetic of the method)."""

import sys

import numpy as np
import torch

import vision_transformer_encoder_block_amd as vit


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    vit.lib()  # raises LibraryMissing: no fallback exists


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_dev(a: np.ndarray):
    """Round to bf16 (nearest even) on the host and move to the GPU; also return the rounded values."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.cuda(), t.to(torch.float64).numpy()


def f32_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def bf16_view(t_uint8_or_bf16, shape):
    return t_uint8_or_bf16.view(torch.bfloat16).reshape(shape)


def vt_position(t: np.ndarray) -> np.ndarray:
    """Column of token t in the vt layout: bits 2 and 3 exchanged (documented in vit_ops.h)."""
    return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1)


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def exact_ln_rows(rng, rows: int, dim: int):
    """Input rows whose LayerNorm is exact in fp32: an integer mean m in [-3, 3]
    plus deviations in +-pairs of 4, 8 and 12 (5 : 8 : 3 pairs per 16), so the
    sum is exactly m dim, the mean exact, every deviation exact, the sum of
    squares exactly 64 dim, the variance exactly 64 and var + 1e-6 rounds back to
    64 (half an ulp there is 3.8e-6).  Returns the rows (float32) and their
    deviations d (float64): the normalised values are d / 8."""
    assert dim % 32 == 0
    per = dim // 32
    base = np.array([4] * 5 * per + [8] * 8 * per + [12] * 3 * per, dtype=np.float64)
    d = np.empty((rows, dim))
    for r in range(rows):
        half = base * np.where(rng.integers(0, 2, base.size) == 1, -1.0, 1.0)
        d[r] = rng.permutation(np.concatenate([half, -half]))
    assert np.all((d ** 2).sum(axis=1) == 64 * dim) and np.all(d.sum(axis=1) == 0)
    m = rng.integers(-3, 4, (rows, 1)).astype(np.float64)
    return (m + d).astype(np.float32), d
