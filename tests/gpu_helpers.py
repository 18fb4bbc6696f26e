"""Helpers shared by the GPU parity tests (not a test module)."""

import sys

import numpy as np
import torch

import la_inputs

TOL = {"bf16": 2e-2, "f32": 1e-4}   # relative Frobenius error per (batch, head)
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dt: str) -> torch.Tensor:
    """Exact upload: x holds bf16-representable float32 values for dt == 'bf16'."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(TORCH_DT[dt]).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max over leading (batch, head) index of ||y - ref||_F / ||ref||_F."""
    y = y.reshape(-1, y.shape[-2], y.shape[-1]) if y.ndim > 2 else y[None]
    ref = ref.reshape(y.shape)
    num = np.linalg.norm((y - ref).reshape(y.shape[0], -1), axis=1)
    den = np.maximum(np.linalg.norm(ref.reshape(y.shape[0], -1), axis=1), 1e-30)
    return float(np.max(num / den))


def qkv(B, H, N, d, seed, dt, scale=1.0):
    return la_inputs.gaussian_qkv(B, H, N, d, seed=seed, scale=scale, bf16=(dt == "bf16"))
