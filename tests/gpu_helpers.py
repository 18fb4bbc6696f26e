"""Helpers shared by the GPU parity tests (not a test module)."""

import sys

import numpy as np
import torch

import la_inputs

TOL = {"bf16": 2e-2, "f32": 1e-4}   # relative error bars (see rel_err)
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
# per-row check: a row's reference norm is floored at this fraction of the
# RMS row norm of its (batch, head) slab, so near-zero rows are measured
# against the slab's scale rather than against themselves
ROW_FLOOR = 1e-3
# Outputs that are sums of terms of both signs (gradients; the identity map
# without normalization, where a row is sum_j (q_i.k_j) v_j) can cancel to a
# row far smaller than its terms, while rounding errors follow the size of the
# terms. Their rows are measured against at least half the slab's RMS row
# norm: a wrong row (a wrong carried state, a wrong tail) still fails, since
# its error is of the order of the row norms.
SIGNED_ROW_FLOOR = 0.5

# worst per-row error seen in this session (reported by conftest at the end),
# and the worst per call site
WORST_ROW = {"err": 0.0, "where": ""}
WORST_BY_SITE = {}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dt: str) -> torch.Tensor:
    """Exact upload: x holds bf16-representable float32 values for dt == 'bf16'."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(TORCH_DT[dt]).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def _slabs(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if y.ndim < 2:
        y = y[None, None]
    y = y.reshape(-1, y.shape[-2], y.shape[-1])
    return y, ref.reshape(y.shape)


def err_parts(y, ref, floor=ROW_FLOOR):
    """(frobenius, per_row, (slab, row, row norm / RMS row norm)) for y
    against ref, both [..., rows, cols].

    frobenius: max over (batch, head) slabs of ||y - ref||_F / ||ref||_F.
    per_row:   max over slabs and rows i of ||y_i - ref_i|| / max(||ref_i||, floor * RMS_i ||ref_i||).
    """
    Y, R = _slabs(y, ref)
    D = Y - R
    frob = np.linalg.norm(D.reshape(D.shape[0], -1), axis=1) / \
        np.maximum(np.linalg.norm(R.reshape(R.shape[0], -1), axis=1), 1e-30)
    rn = np.linalg.norm(R, axis=2)
    dn = np.linalg.norm(D, axis=2)
    rms = np.sqrt(np.mean(rn * rn, axis=1))
    row = dn / np.maximum(np.maximum(rn, floor * rms[:, None]), 1e-30)
    # NaN anywhere must fail the comparison: np.max propagates it
    w = np.unravel_index(int(np.nanargmax(row)) if np.isfinite(row).any() else 0, row.shape)
    ratio = float(rn[w] / rms[w[0]]) if rms[w[0]] > 0 else 0.0
    return float(np.max(frob)), float(np.max(row)), (int(w[0]), int(w[1]), ratio)


def err_parts_local(y, ref, block=64, frac=0.5):
    """Per-row error with a local floor: row i is measured against
    max(||ref_i||, frac * RMS row norm of its block of `block` rows). Returns
    (per_row, (slab, row, row norm / block RMS))."""
    Y, R = _slabs(y, ref)
    rn = np.linalg.norm(R, axis=2)
    n = rn.shape[1]
    pad = (-n) % block
    rp = np.concatenate([rn, np.full((rn.shape[0], pad), np.nan)], axis=1).reshape(rn.shape[0], -1, block)
    brms = np.sqrt(np.nanmean(rp * rp, axis=2))
    floor = np.repeat(brms, block, axis=1)[:, :n]
    row = np.linalg.norm(Y - R, axis=2) / np.maximum(np.maximum(rn, frac * floor), 1e-30)
    w = np.unravel_index(int(np.nanargmax(row)) if np.isfinite(row).any() else 0, row.shape)
    return float(np.max(row)), (int(w[0]), int(w[1]), float(rn[w] / floor[w]) if floor[w] > 0 else 0.0)


def note_row(row, at, where):
    """Record a per-row error for the end-of-session report."""
    detail = f"slab {at[0]} row {at[1]} (row norm {at[2]:.2g} x RMS)"
    if not row <= WORST_ROW["err"]:
        WORST_ROW["err"] = row
        WORST_ROW["where"] = f"{where} {detail}"
    old = WORST_BY_SITE.get(where)
    if old is None or not row <= old[0]:
        WORST_BY_SITE[where] = (row, detail)


def rel_err(y, ref, floor=ROW_FLOOR, where=""):
    """Larger of the per-slab Frobenius error and the per-row error (err_parts).

    The per-row term keeps one wrong row (a segment boundary, a ragged tail,
    a late position) from hiding in the norm of a long sequence."""
    frob, row, at = err_parts(y, ref, floor)
    note_row(row, at, where or caller(1))
    return float(np.max([frob, row]))


def rel_err_terms(y, ref, terms, frac=0.25, where=""):
    """Larger of the per-slab Frobenius error and a componentwise per-row
    error: row i is measured against max(||ref_i||, frac * ||terms_i||),
    where terms holds the same sums taken over the absolute values of their
    terms. For signed sums whose rows can cancel far below their terms (the
    identity map without normalization), this is the scale the rounding
    errors follow; a row that cancels by less than 1/frac is measured against
    itself."""
    Y, R = _slabs(y, ref)
    T = np.asarray(terms, dtype=np.float64).reshape(Y.shape)
    frob = np.max(np.linalg.norm((Y - R).reshape(Y.shape[0], -1), axis=1) /
                  np.maximum(np.linalg.norm(R.reshape(R.shape[0], -1), axis=1), 1e-30))
    rn = np.linalg.norm(R, axis=2)
    row = np.linalg.norm(Y - R, axis=2) / np.maximum(np.maximum(rn, frac * np.linalg.norm(T, axis=2)), 1e-30)
    w = np.unravel_index(int(np.nanargmax(row)) if np.isfinite(row).any() else 0, row.shape)
    rms = np.sqrt(np.mean(rn[w[0]] ** 2))
    note_row(float(np.max(row)), (int(w[0]), int(w[1]), float(rn[w] / rms) if rms > 0 else 0.0),
             where or caller(1))
    return float(np.max([frob, np.max(row)]))


def caller(depth=1):
    f = sys._getframe(depth + 1)
    return f"{f.f_code.co_filename.rsplit('/', 1)[-1]}:{f.f_code.co_name}:{f.f_lineno}"


def qkv(B, H, N, d, seed, dt, scale=1.0):
    return la_inputs.gaussian_qkv(B, H, N, d, seed=seed, scale=scale, bf16=(dt == "bf16"))
