"""la_forward_static, the entry point for callers that cannot allocate: the
same forward as la_forward, its workspace the library's fixed device array.

Checked through the C ABI against la_forward on the same inputs, on two calls
in a row (the second smaller, so it runs on what the first left in the array):
identical outputs and final states (same kernels, same plan), and within the
parity tolerance of the oracle."""

import math

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

import causal_linear_attention_02_amd as la  # noqa: E402
from gpu_helpers import TOL, log, qkv, rel_err, to_dev, to_host  # noqa: E402


def _pair(B, H, N, d, dt, causal, seed, rows=None):
    need = la.la_forward_workspace_size(B, H, N, d, causal=causal)
    log(f"case static workspace B{B} H{H} N{N} d{d} {dt} causal={causal}: la_forward needs {need} B "
        f"(fixed array {la.LA_STATIC_SCRATCH_BYTES} B)")
    assert need <= la.LA_STATIC_SCRATCH_BYTES
    q, k, v = qkv(B, H, N, d, seed, dt, 1 / math.sqrt(d))
    tq, tk, tv = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    y_ref, S_ref, z_ref = la.la_forward(tq, tk, tv, causal=causal, return_state=True)
    out = torch.empty_like(tq)
    S = torch.empty_like(S_ref)
    z = torch.empty_like(z_ref)
    st = la.lib.la_forward_static(la._ptr(tq), la._ptr(tk), la._ptr(tv), la._ptr(out), B, H, N, d,
                                  la.ctypes.byref(la.la_feature_map(la.LA_ELU1, 0, None)), int(causal), 1,
                                  la.LA_BF16 if dt == "bf16" else la.LA_F32, None, None,
                                  la._ptr(S) if causal else None, la._ptr(z) if causal else None,
                                  la._stream(None))
    assert st == la.LA_OK, la.la_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(out, y_ref)
    if causal:
        assert torch.equal(S, S_ref) and torch.equal(z, z_ref)
    idx = np.arange(N) if rows is None else rows
    ref = O.attention(q, k, v, "elu1", causal=causal, rows=idx)
    e = rel_err(to_host(out[:, :, idx]), ref)
    log(f"  identical to la_forward; rel err against the oracle {e:.3e}")
    assert e <= TOL[dt]


def test_static_workspace_two_calls_in_a_row():
    # first: 64 segments of 66 KB per head (B1 H4 N16384 d128: 16.9 MB of segment states)
    rows = np.unique(np.concatenate([np.arange(0, 16384, 257), np.arange(255, 16384, 256), [16383]]))
    _pair(1, 4, 16384, 128, "bf16", True, 61, rows=rows)
    # second, smaller: fewer, smaller segment states over what the first left behind
    _pair(2, 3, 64 * 11 + 7, 64, "bf16", True, 62)
    _pair(1, 2, 64 * 9 + 3, 32, "f32", False, 63)
