"""Seeded synthetic inputs for kernelized linear attention.

This module is shared by the tests, the bench and the oracle checks. It holds
no arithmetic of the attention method itself: only random draws, a fixed
scaling of those draws, and rounding of float32 values to the bfloat16 grid
(round-to-nearest-even), so that the GPU path and the oracle consume exactly
the same numbers.

Recipes (shapes follow the workloads the attention pages discuss: one head
dimension d per head, queries/keys/values drawn i.i.d. Gaussian):

* ``gaussian_qkv``: q, k, v ~ N(0, 1) * scale, float32, optionally rounded to
  bf16.  The draw order is q, then k, then v, each a full [B, H, N, d] block
  from ``numpy.random.default_rng(seed)`` (PCG64).
* ``performer_W``: random projection for the positive-random-feature map,
  m x d, built from ceil(m/d) independent d x d orthogonal blocks (Q factor
  of a Gaussian matrix, sign-fixed so diag(R) > 0), each row rescaled to the
  length of an independent N(0, I_d) vector, then rounded to bf16 values.
* ``decode_tokens``: per-sequence / per-step token blocks seeded by
  ``default_rng([base, index])`` so that any subset can be regenerated alone.
* ``log_gates``: natural logs of gates alpha ~ U(lo, 1), float32, for the
  gated (GLA) variant; lo = 1/4 is the smallest gate the kernels accept.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits",
    "bits_to_f32",
    "gaussian",
    "gaussian_qkv",
    "performer_W",
    "decode_tokens",
    "log_gates",
    "WORKLOADS",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even).

    Returns float32 values that are exactly representable in bf16.
    """
    return bits_to_f32(bf16_bits(x))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of ``x`` rounded to nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step].view(np.uint32)
        nan = (u & 0x7FFFFFFF) > 0x7F800000
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
        flat_out[s:s + step] = r.astype(np.uint16)
    return out


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """float32 values of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def gaussian(rng: np.random.Generator, shape, scale: float = 1.0, bf16: bool = True) -> np.ndarray:
    """N(0,1) float32 draws times ``scale`` (in float32), optionally on the bf16 grid."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return bf16_round(x) if bf16 else x


def gaussian_qkv(B: int, H: int, N: int, d: int, seed: int, scale: float = 1.0,
                 bf16: bool = True):
    """q, k, v of shape [B, H, N, d], drawn in that order from one PCG64 stream."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = gaussian(rng, shape, scale, bf16)
    k = gaussian(rng, shape, scale, bf16)
    v = gaussian(rng, shape, scale, bf16)
    return q, k, v


def performer_W(m: int, d: int, seed: int, bf16: bool = True) -> np.ndarray:
    """m x d block-orthogonal Gaussian projection (float32, bf16 values by default)."""
    rng = np.random.default_rng(seed)
    blocks = []
    for _ in range(math.ceil(m / d)):
        g = rng.standard_normal((d, d))
        qm, rm = np.linalg.qr(g)
        qm = qm * np.sign(np.diag(rm))[None, :]
        blocks.append(qm.T)
    w = np.concatenate(blocks, axis=0)[:m]
    lengths = np.linalg.norm(rng.standard_normal((m, d)), axis=1)
    w = np.ascontiguousarray((w * lengths[:, None]).astype(np.float32))
    return bf16_round(w) if bf16 else w


def decode_tokens(base_seed: int, index: int, shape, scale: float = 1.0, bf16: bool = True):
    """q, k, v blocks for one decode sequence (prefill) or one decode step."""
    rng = np.random.default_rng([base_seed, index])
    q = gaussian(rng, shape, scale, bf16)
    k = gaussian(rng, shape, scale, bf16)
    v = gaussian(rng, shape, scale, bf16)
    return q, k, v


def log_gates(rng: np.random.Generator, shape, lo: float = 0.25) -> np.ndarray:
    """float32 log(alpha), alpha ~ U(lo, 1)."""
    return np.log(rng.uniform(lo, 1.0, shape)).astype(np.float32)


# Named synthetic workloads.  Every entry is plain data: shapes, seeds and the
# scaling applied to N(0,1) draws.
WORKLOADS = {
    # causal and non-causal parity case, fp32 inputs, elu+1 map
    "parity_small_f32": dict(B=1, H=1, N=256, d=32, dtype="f32", seed=42, scale=1.0,
                             fmap="elu1"),
    # causal prefill, bf16 inputs scaled by 1/sqrt(d), chunk 64
    "prefill_b4h8n2048d64": dict(B=4, H=8, N=2048, d=64, dtype="bf16", seed=1002,
                                 scale=1.0 / math.sqrt(64), fmap="elu1"),
    # long-context causal prefill, bf16 inputs scaled by 1/sqrt(d)
    "prefill_b1h16n65536d128": dict(B=1, H=16, N=65536, d=128, dtype="bf16", seed=1003,
                                    scale=1.0 / math.sqrt(128), fmap="elu1"),
    # recurrent decode: 256 sequences x 32 heads, d=64, 4096 prefill tokens then
    # 1000 single-token steps, N(0,1) bf16 tokens
    "decode_s256h32d64": dict(B=256, H=32, d=64, dtype="bf16", prefill=4096, steps=1000,
                              prefill_seed=1004, step_seed=2004, scale=1.0, fmap="elu1"),
    # positive random features, m=256, W seeded, q,k,v N(0,1) bf16
    "performer_b2h8n16384d64m256": dict(B=2, H=8, N=16384, d=64, m=256, dtype="bf16",
                                        seed=1005, w_seed=5005, scale=1.0,
                                        fmap="performer"),
}
