"""Seeded synthetic inputs shared by the tests and the benchmark.

This module holds no arithmetic of the method: it only draws Gaussian
Q/K/V, prefix masks and the hand-written example inputs, and rounds fp32 to
bf16.  Both the oracle and the HIP path consume what it returns; neither is
imported here.

Recipe (stated once, used everywhere):
  * generator: numpy ``default_rng(seed)`` (PCG64), ``standard_normal`` in
    float32, drawn in the order Q, K, V, then the mask m, then any decode
    inputs;
  * optional scale 1/sqrt(d) applied in float32 (the N(0,1)/sqrt(d) workloads);
  * bf16 inputs: fp32 rounded to nearest-even bf16; both the oracle and the
    GPU see exactly those rounded values;
  * random prefix masks: m_i i.i.d. uniform integers in [0, n-1] inclusive.

Arrays are returned in their storage format: float32, or bf16 as raw
``uint16`` bit patterns.  ``to_torch`` turns either into a CPU torch tensor
of the matching dtype.
"""
from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding helper expects finite values")
    b = x.view(np.uint32)
    # finite values stay below 0xFF800000, so adding at most 0x8000 cannot wrap
    return ((b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_dtype(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x_f32)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f32(x: np.ndarray) -> np.ndarray:
    """Storage-format array -> float32 values (bf16 widened exactly)."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float32)


def to_torch(x: np.ndarray):
    """Storage-format array -> CPU torch tensor (float32, bfloat16, or an
    integer array such as a prefix mask, passed through unchanged)."""
    import torch
    if x.dtype in (np.int64, np.int32):
        return torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))


def from_torch(t) -> np.ndarray:
    """CPU/GPU torch tensor (float32 or bfloat16) -> storage-format numpy array."""
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.to(torch.float32).numpy().copy()


def gaussian(rng: np.random.Generator, shape, scale: float | None, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale is not None:
        x = x * np.float32(scale)
    return as_dtype(x, dtype)


def qkv(B, Hq, Hkv, n, d, dtype=F32, seed=0, scaled=False, rng=None):
    """Draw Q [B,Hq,n,d], K and V [B,Hkv,n,d] in that order.

    ``scaled`` selects N(0,1)/sqrt(d) instead of N(0,1).
    Returns (q, k, v, rng) so that later draws continue the same stream.
    """
    rng = rng or np.random.default_rng(seed)
    s = (1.0 / np.sqrt(d)) if scaled else None
    q = gaussian(rng, (B, Hq, n, d), s, dtype)
    k = gaussian(rng, (B, Hkv, n, d), s, dtype)
    v = gaussian(rng, (B, Hkv, n, d), s, dtype)
    return q, k, v, rng


def mask(n, kind, rng=None, seed=0):
    """Prefix mask of length n: 'causal' (arange), 'random' (uniform in [0, n-1]),
    'full' (every query sees all keys), 'first' (every query sees key 0 only)."""
    if kind == "causal":
        return np.arange(n, dtype=np.int64)
    if kind == "full":
        return np.full(n, n - 1, dtype=np.int64)
    if kind == "first":
        return np.zeros(n, dtype=np.int64)
    if kind == "random":
        rng = rng or np.random.default_rng(seed)
        return rng.integers(0, n, size=n, dtype=np.int64)
    raise ValueError(kind)


def hand_case(which: str):
    """The two worked examples of the nx_f32_linear_attention.nx page (gates 1
    and 2): n = d = 2, V rows [2,4] and [6,8]; gate 1 has all-zero Q and K,
    gate 2 has Q = K = the 2x2 identity.  Shapes [1,1,2,2], float32."""
    v = np.array([[2.0, 4.0], [6.0, 8.0]], dtype=np.float32)
    if which == "zero":
        q = np.zeros((2, 2), dtype=np.float32)
        k = np.zeros((2, 2), dtype=np.float32)
    elif which == "identity":
        q = np.eye(2, dtype=np.float32)
        k = np.eye(2, dtype=np.float32)
    else:
        raise ValueError(which)
    return (q.reshape(1, 1, 2, 2), k.reshape(1, 1, 2, 2), v.reshape(1, 1, 2, 2))
