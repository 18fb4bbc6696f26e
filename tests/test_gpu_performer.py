"""GPU parity of the positive-random-feature map and the attention built on it.

phi(x) = exp(W x~ - |x~|^2 / 2) / sqrt(m), x~ = d^(-1/4) x ("Linear Attention",
marovi.ai, "Mapas de características"). W is a seeded block-orthogonal
Gaussian matrix. For bf16 inputs the library multiplies with W rounded to
bf16, so the oracle is given that rounded W; for fp32 inputs W is used as is.
Tolerance: relative Frobenius error per (batch, head) <= 2e-2 (bf16 inputs),
<= 1e-4 (fp32 inputs).
"""

import math

import numpy as np
import pytest

import la_inputs
import oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

import causal_linear_attention_02_amd as la  # noqa: E402
from gpu_helpers import TOL, log, qkv, rel_err, to_dev, to_host  # noqa: E402

PAIRS = [(32, 64), (32, 128), (64, 64), (64, 128), (64, 256), (128, 64), (128, 128)]


def _W(m, d, seed, dt, rounded=True):
    """(device W, the W the oracle must use)."""
    w = la_inputs.performer_W(m, d, seed, bf16=rounded)
    ref = la_inputs.bf16_round(w) if dt == "bf16" else w
    return torch.from_numpy(w).cuda(), ref.astype(np.float64)


@pytest.mark.parametrize("d,m", PAIRS)
@pytest.mark.parametrize("din,dout", [("bf16", "f32"), ("bf16", "bf16"), ("f32", "f32")])
def test_feature_map_performer(d, m, din, dout):
    log(f"case feature_map performer d{d} m{m} {din}->{dout}")
    rng = np.random.default_rng(d * 1000 + m)
    rows = 64 * 3 + 21  # several tiles and a ragged tail
    x = la_inputs.gaussian(rng, (rows, d), 1.0, bf16=(din == "bf16"))
    tW, Wref = _W(m, d, 400 + m, din, rounded=False)
    y = la.la_feature_map_apply(to_dev(x, din), feature_map="performer", W=tW,
                                out_dtype={"bf16": torch.bfloat16, "f32": torch.float32}[dout])
    torch.cuda.synchronize()
    ref = O.phi_performer(x.astype(np.float64), Wref)
    got = to_host(y)
    assert got.shape == (rows, m)
    if dout == "bf16":
        # one bf16 rounding of a value within 1e-5 (relative) of the reference
        np.testing.assert_allclose(got, ref, rtol=2 ** -8 + 2e-5, atol=0)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-4, atol=0)


def _check_forward(B, H, N, d, m, dt, causal, normalize, seed, S0=None, z0=None, state=False):
    log(f"case performer forward B{B} H{H} N{N} d{d} m{m} {dt} causal={causal} norm={normalize} "
        f"state_in={S0 is not None} state_out={state}")
    q, k, v = qkv(B, H, N, d, seed, dt, 1.0)
    tW, Wref = _W(m, d, seed + 1, dt)
    kw = {}
    if S0 is not None:
        kw = dict(S_in=torch.from_numpy(S0.astype(np.float32)).cuda(),
                  z_in=torch.from_numpy(z0.astype(np.float32)).cuda())
    res = la.la_forward(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), feature_map="performer", W=tW,
                        causal=causal, normalize=normalize, return_state=state, **kw)
    torch.cuda.synchronize()
    y = res[0] if state else res
    ref = O.attention(q, k, v, "performer", W=Wref, causal=causal, normalize=normalize, S0=S0, z0=z0)
    err = rel_err(to_host(y), ref)
    log(f"  rel err {err:.3e}")
    assert err <= TOL[dt], err
    if state:
        Sr, zr = O.final_state(k, v, "performer", W=Wref, S0=S0, z0=z0)
        eS = rel_err(to_host(res[1]), Sr)
        ez = rel_err(to_host(res[2])[..., None], zr[..., None])
        log(f"  state rel err S {eS:.3e} z {ez:.3e}")
        assert eS <= TOL[dt] and ez <= TOL[dt]


@pytest.mark.parametrize("d,m", PAIRS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_performer_forward_small(d, m, dt):
    for N in (1, 65, 200):
        for causal in (True, False):
            _check_forward(2, 2, N, d, m, dt, causal, True, seed=500 + N + d + m)


@pytest.mark.parametrize("d,m", PAIRS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_performer_forward_multisegment(d, m, dt):
    N = 64 * 40 - 17
    for causal in (True, False):
        for normalize in (True, False):
            _check_forward(1, 2, N, d, m, dt, causal, normalize, seed=61 + d + m)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_performer_state_in_and_out(dt):
    d, m, N = 64, 128, 64 * 9 + 5
    rng = np.random.default_rng(8)
    kk = la_inputs.gaussian(rng, (1, 2, 300, d), bf16=False)
    vv = la_inputs.gaussian(rng, (1, 2, 300, d), bf16=False)
    _, Wref = _W(m, d, 13 + 1, dt)
    S0, z0 = O.final_state(kk, vv, "performer", W=Wref)
    for causal in (True, False):
        _check_forward(1, 2, N, d, m, dt, causal, True, seed=13, S0=S0, z0=z0, state=True)


@pytest.mark.parametrize("d,m", PAIRS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_performer_decode(d, m, dt):
    log(f"case performer decode d{d} m{m} {dt}")
    B, H, N0, T = 2, 3, 90, 4
    q, k, v = qkv(B, H, N0 + T, d, 71 + d + m, dt)
    tW, Wref = _W(m, d, 3 + m, dt, rounded=False)
    S0, z0 = O.final_state(k[:, :, :N0], v[:, :, :N0], "performer", W=Wref)
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    Sr, zr = S0, z0
    for t in range(N0, N0 + T):
        y = la.la_decode_step(S, z, to_dev(q[:, :, t], dt), to_dev(k[:, :, t], dt), to_dev(v[:, :, t], dt),
                              feature_map="performer", W=tW)
        yr, Sr, zr = O.decode_step(Sr, zr, q[:, :, t], k[:, :, t], v[:, :, t], "performer", W=Wref)
        torch.cuda.synchronize()
        err = rel_err(to_host(y)[..., None, :], yr[..., None, :])
        assert err <= TOL[dt], (t, err)
    eS = rel_err(to_host(S), Sr)
    ez = rel_err(to_host(z)[..., None], zr[..., None])
    log(f"  final state rel err S {eS:.3e} z {ez:.3e}")
    assert eS <= 1e-4 and ez <= 1e-4


def test_performer_prefill_decode_handoff():
    log("case performer decode after prefill (hand-off)")
    d, m, N0, T = 64, 256, 64 * 5 + 3, 4
    q, k, v = qkv(1, 3, N0 + T, d, 91, "bf16")
    tW, Wref = _W(m, d, 92, "bf16")
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    _, S, z = la.la_forward(tq[:, :, :N0].contiguous(), tk[:, :, :N0].contiguous(), tv[:, :, :N0].contiguous(),
                            feature_map="performer", W=tW, return_state=True)
    ref = O.attention(q, k, v, "performer", W=Wref, causal=True)
    for t in range(N0, N0 + T):
        y = la.la_decode_step(S, z, tq[:, :, t].contiguous(), tk[:, :, t].contiguous(), tv[:, :, t].contiguous(),
                              feature_map="performer", W=tW)
        torch.cuda.synchronize()
        err = rel_err(to_host(y)[..., None, :], ref[:, :, t][..., None, :])
        assert err <= TOL["bf16"], (t, err)


def test_performer_unsupported_pair_rejected():
    d, m = 32, 256
    tW = torch.zeros((m, d), dtype=torch.float32, device="cuda")
    x = torch.zeros((4, 3, 64, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(NotImplementedError):
        la.la_forward(x, x.clone(), x.clone(), feature_map="performer", W=tW)


@pytest.mark.parametrize("d,m,causal", [(64, 256, True), (64, 256, False), (128, 128, True), (128, 128, False),
                                        (32, 64, True), (32, 64, False)])
def test_performer_fused_needs_states_only(d, m, causal):
    """bf16, causal or not, at every head dimension: the projection runs
    inside the chunked passes, so the exact bf16 workspace
    (la_forward_workspace_size with dtype) holds the segment states only,
    far below the fp32 figure, which also holds phi(q) and phi(k); fp32
    inputs are rejected with it."""
    log(f"case performer fused path, states-only workspace, d={d} m={m} causal={causal}")
    N = 64 * 40 - 17
    q, k, v = qkv(1, 2, N, d, 123, "bf16", 1.0)
    tW, Wref = _W(m, d, 124, "bf16")
    need = la.la_forward_workspace_size(1, 2, N, d, feature_map="performer", W=tW, causal=causal,
                                        dtype=torch.bfloat16)
    full = la.la_forward_workspace_size(1, 2, N, d, feature_map="performer", W=tW, causal=causal,
                                        dtype=torch.float32)
    assert 0 < need and need * 4 < full
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = la.la_forward(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), feature_map="performer", W=tW,
                      workspace=ws, causal=causal)
    torch.cuda.synchronize()
    ref = O.attention(q, k, v, "performer", W=Wref, causal=causal)
    err = rel_err(to_host(y), ref)
    log(f"  rel err {err:.3e}")
    assert err <= TOL["bf16"], err
    with pytest.raises(ValueError):  # LA_ERR_WORKSPACE
        la.la_forward(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), feature_map="performer", W=tW,
                      workspace=ws, causal=causal)
