"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerance: relative Frobenius error per (batch, head) <= 2e-2 for bf16
inputs and <= 1e-4 for fp32 inputs. Inputs are seeded and synthetic.
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


# ---------------------------------------------------------------------------
# feature map
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("din,dout", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
def test_feature_map_elu1(din, dout):
    log(f"case feature_map elu1 {din}->{dout}")
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((333, 64)) * 3).astype(np.float32)
    x[0, :8] = [0.0, -0.0, 1.0, -1.0, 80.0, -80.0, -1e30, 1e-30]
    if din == "bf16":
        x = la_inputs.bf16_round(x)
    y = la.la_feature_map_apply(to_dev(x, din), out_dtype={"bf16": torch.bfloat16, "f32": torch.float32}[dout])
    torch.cuda.synchronize()
    ref = O.phi_elu1(x.astype(np.float64))
    got = to_host(y)
    if dout == "bf16":
        ref = la_inputs.bf16_round(ref.astype(np.float32)).astype(np.float64)
        np.testing.assert_allclose(got, ref, rtol=2 ** -7, atol=0)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-30)


# ---------------------------------------------------------------------------
# forward: small shapes, every supported head dim, both precisions
# ---------------------------------------------------------------------------
def _check_forward(B, H, N, d, dt, causal, normalize, seed, scale=1.0, S0=None, z0=None, state=False):
    log(f"case forward B{B} H{H} N{N} d{d} {dt} causal={causal} norm={normalize} seed={seed} "
        f"state_in={S0 is not None} state_out={state}")
    q, k, v = qkv(B, H, N, d, seed, dt, scale)
    kw = {}
    if S0 is not None:
        kw = dict(S_in=torch.from_numpy(S0.astype(np.float32)).cuda(),
                  z_in=torch.from_numpy(z0.astype(np.float32)).cuda())
    res = la.la_forward(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), causal=causal, normalize=normalize,
                        return_state=state, **kw)
    torch.cuda.synchronize()
    y = res[0] if state else res
    ref = O.attention(q, k, v, "elu1", causal=causal, normalize=normalize, S0=S0, z0=z0)
    err = rel_err(to_host(y), ref)
    log(f"  rel err {err:.3e}")
    assert err <= TOL[dt], err
    if state:
        Sr, zr = O.final_state(k, v, "elu1", S0=S0, z0=z0)
        eS = rel_err(to_host(res[1]), Sr)
        ez = rel_err(to_host(res[2])[..., None], zr[..., None])
        log(f"  state rel err S {eS:.3e} z {ez:.3e}")
        assert eS <= TOL[dt] and ez <= TOL[dt]
    return err


def test_forward_parity_small_f32_config():
    """B1 H1 N256 d32 fp32 inputs (seed 42), all four causal/normalize combinations."""
    for causal in (True, False):
        for normalize in (True, False):
            _check_forward(1, 1, 256, 32, "f32", causal, normalize, seed=42)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 200])
def test_forward_parity_shapes(d, dt, N):
    for causal in (True, False):
        _check_forward(2, 3, N, d, dt, causal, True, seed=100 + N + d, scale=1.0 / math.sqrt(d))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_forward_parity_multisegment(d, dt):
    """Few sequences, long enough to be split into segments; ragged tail."""
    N = 64 * 40 - 17
    for causal in (True, False):
        for normalize in (True, False):
            _check_forward(1, 2, N, d, dt, causal, normalize, seed=7 + d, scale=1.0)


@pytest.mark.parametrize("nchunks", [60, 64])
def test_forward_parity_fold_threshold(nchunks):
    """One sequence at d = 64 cut into 15 segments (segment states 249.6 KB: the
    output pass adds the local sums of the segments before it, no carry scan)
    or 16 (266 KB: carry scan); carried-in state, final state, ragged tail."""
    d, N = 64, 64 * nchunks - 5
    rng = np.random.default_rng(nchunks)
    kk = la_inputs.gaussian(rng, (1, 1, 200, d), bf16=False)
    vv = la_inputs.gaussian(rng, (1, 1, 200, d), bf16=False)
    S0, z0 = O.final_state(kk, vv, "elu1")
    _check_forward(1, 1, N, d, "bf16", True, True, seed=900 + nchunks, scale=1 / 8, S0=S0, z0=z0, state=True)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_forward_state_in_and_out(dt):
    d, N = 64, 64 * 9 + 5
    rng = np.random.default_rng(3)
    kk = la_inputs.gaussian(rng, (1, 2, 300, d), bf16=False)
    vv = la_inputs.gaussian(rng, (1, 2, 300, d), bf16=False)
    S0, z0 = O.final_state(kk, vv, "elu1")
    for causal in (True, False):
        _check_forward(1, 2, N, d, dt, causal, True, seed=11, S0=S0, z0=z0, state=True)
        _check_forward(1, 2, N, d, dt, causal, True, seed=12, state=True)


def test_forward_zero_length_copies_state():
    log("case forward N=0 state hand-off")
    d = 64
    q = torch.zeros((2, 2, 0, d), dtype=torch.bfloat16, device="cuda")
    S0 = torch.randn(2, 2, d, d, device="cuda")
    z0 = torch.rand(2, 2, d, device="cuda")
    _, S, z = la.la_forward(q, q.clone(), q.clone(), S_in=S0, z_in=z0, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(z, z0)
    _, S, z = la.la_forward(q, q.clone(), q.clone(), return_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0 and torch.count_nonzero(z) == 0


def test_forward_deterministic():
    log("case forward determinism")
    q, k, v = qkv(1, 4, 64 * 33 + 3, 128, 9, "bf16", 1 / math.sqrt(128))
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    a = la.la_forward(tq, tk, tv)
    b = la.la_forward(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_forward_batch_independent_of_split():
    """A sequence gives the same result alone (many segments) and inside a large batch."""
    log("case forward split invariance")
    d, N = 64, 2048
    q, k, v = qkv(1, 64, N, d, 21, "bf16", 1 / 8)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    full = la.la_forward(tq, tk, tv)
    one = la.la_forward(tq[:, :1].contiguous(), tk[:, :1].contiguous(), tv[:, :1].contiguous())
    torch.cuda.synchronize()
    assert rel_err(to_host(one), to_host(full[:, :1])) < 1e-2


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_parity(d, dt):
    log(f"case decode d{d} {dt}")
    B, H, N0, T = 3, 5, 100, 6
    q, k, v = qkv(B, H, N0 + T, d, 31 + d, dt)
    S0, z0 = O.final_state(k[:, :, :N0], v[:, :, :N0], "elu1")
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    Sr, zr = S0, z0
    for t in range(N0, N0 + T):
        y = la.la_decode_step(S, z, to_dev(q[:, :, t], dt), to_dev(k[:, :, t], dt), to_dev(v[:, :, t], dt))
        yr, Sr, zr = O.decode_step(Sr, zr, q[:, :, t], k[:, :, t], v[:, :, t], "elu1")
        torch.cuda.synchronize()
        err = rel_err(to_host(y)[..., None, :], yr[..., None, :])
        assert err <= TOL[dt], (t, err)
    eS = rel_err(to_host(S), Sr)
    log(f"  final state rel err {eS:.3e}")
    assert eS <= 1e-5


def test_decode_unnormalized_and_prefill_handoff():
    log("case decode after prefill (hand-off)")
    d, N0, T = 64, 64 * 5 + 3, 5
    q, k, v = qkv(2, 4, N0 + T, d, 77, "bf16")
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    _, S, z = la.la_forward(tq[:, :, :N0].contiguous(), tk[:, :, :N0].contiguous(), tv[:, :, :N0].contiguous(),
                            return_state=True)
    ref = O.attention(q, k, v, "elu1", causal=True)
    for t in range(N0, N0 + T):
        y = la.la_decode_step(S, z, tq[:, :, t].contiguous(), tk[:, :, t].contiguous(), tv[:, :, t].contiguous())
        torch.cuda.synchronize()
        assert rel_err(to_host(y)[..., None, :], ref[:, :, t][..., None, :]) <= TOL["bf16"]
    Sx, zx = O.final_state(k, v, "elu1")
    y = la.la_decode_step(S.clone(), z.clone(), tq[:, :, -1].contiguous(), tk[:, :, -1].contiguous(),
                          tv[:, :, -1].contiguous(), normalize=False)
    torch.cuda.synchronize()
    _, Sr, zr = O.decode_step(Sx, zx, q[:, :, -1], k[:, :, -1], v[:, :, -1], "elu1")
    yr = np.einsum("bhc,bhce->bhe", O.phi_elu1(q[:, :, -1]), Sr)
    assert rel_err(to_host(y)[..., None, :], yr[..., None, :]) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# the denominator clamp: y = num / max(den, 1e-6)
# ---------------------------------------------------------------------------
# Rows whose phi(q) vanishes (q = -1e30: elu+1 gives phi = 0 exactly, so
# num = den = 0 and y = 0) or nearly vanishes (q = -30: phi = e^-30, den of
# order 1e-9, below the clamp, so y = num / 1e-6 instead of num / den, a value
# some 10^3 - 10^5 times smaller than the weighted mean of v). The clamped rows
# are compared as a group of their own, so that their small scale is not
# hidden under the per-row floor of the other rows.
def _clamp_rows(N):
    i = np.arange(N)
    return np.nonzero(i % 7 == 3)[0], np.nonzero(i % 7 == 5)[0]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_denominator_clamp_prefill(dt, causal):
    B, H, N, d = 1, 2, 64 * 5 + 11, 64
    log(f"case denominator clamp prefill B{B} H{H} N{N} d{d} {dt} causal={causal}")
    q, k, v = qkv(B, H, N, d, 501, dt, 1 / 8)
    zero_rows, tiny_rows = _clamp_rows(N)
    fill = (lambda x: la_inputs.bf16_round(np.float32(x))) if dt == "bf16" else np.float32
    q[:, :, zero_rows] = fill(-1e30)
    q[:, :, tiny_rows] = fill(-30.0)
    y = to_host(la.la_forward(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), causal=causal))
    ref = O.attention(q, k, v, "elu1", causal=causal)
    # the oracle's clamped rows really are clamped: far below the weighted means
    unclamped = O.attention(q, k, v, "elu1", causal=causal, normalize=False)
    den = np.einsum("bhnc,bhnc->bhn", O.phi_elu1(q.astype(np.float64)), np.cumsum(O.phi_elu1(k.astype(np.float64)),
                    axis=2) if causal else np.broadcast_to(O.phi_elu1(k.astype(np.float64)).sum(axis=2, keepdims=True),
                                                           k.shape))
    assert np.all(den[:, :, tiny_rows] < 1e-7) and np.all(den[:, :, zero_rows] == 0.0)
    np.testing.assert_allclose(ref[:, :, tiny_rows], unclamped[:, :, tiny_rows] / 1e-6, rtol=1e-12)
    assert not np.isnan(y).any()
    assert np.all(y[:, :, zero_rows] == 0.0)
    e_all = rel_err(y, ref)
    e_tiny = rel_err(y[:, :, tiny_rows], ref[:, :, tiny_rows])
    log(f"  rel err all rows {e_all:.3e}, clamped rows {e_tiny:.3e}")
    assert e_all <= TOL[dt] and e_tiny <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_denominator_clamp_decode(dt):
    B, H, d, N0 = 2, 3, 64, 300
    log(f"case denominator clamp decode B{B} H{H} d{d} {dt}")
    q, k, v = qkv(B, H, N0 + 1, d, 502, dt, 1 / 8)
    S0, z0 = O.final_state(k[:, :, :N0], v[:, :, :N0], "elu1")
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    qt = q[:, :, N0].copy()
    fill = (lambda x: la_inputs.bf16_round(np.float32(x))) if dt == "bf16" else np.float32
    qt[0, 1] = fill(-30.0)      # den = e^-30 * sum(z) ~ 1e-9: clamped
    qt[1, 2] = fill(-1e30)      # phi(q) = 0: y = 0
    y = to_host(la.la_decode_step(S, z, to_dev(qt, dt), to_dev(k[:, :, N0], dt), to_dev(v[:, :, N0], dt)))
    torch.cuda.synchronize()
    yr, _, zr = O.decode_step(S0, z0, qt, k[:, :, N0], v[:, :, N0], "elu1")
    assert float(O.phi_elu1(np.float64(qt[0, 1, 0])) * zr[0, 1].sum()) < 1e-7
    assert not np.isnan(y).any() and np.all(y[1, 2] == 0.0)
    e = rel_err(y[..., None, :], yr[..., None, :])
    e_tiny = rel_err(y[0, 1][None], yr[0, 1][None])
    log(f"  rel err {e:.3e}, clamped head {e_tiny:.3e}")
    assert e <= TOL[dt] and e_tiny <= TOL[dt]


@pytest.mark.parametrize("causal", [True, False])
def test_denominator_clamp_negative_identity(causal):
    """Identity map, normalized: positive keys, and every fifth query row
    negated, so those rows have a clearly negative denominator (clamped to
    1e-6: y = num * 1e6) while the others stay clearly positive."""
    B, H, N, d = 1, 2, 64 * 3 + 7, 32
    log(f"case denominator clamp, negative identity-map denominators causal={causal}")
    q, k, v = qkv(B, H, N, d, 503, "f32", 1.0)
    q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    neg = np.nonzero(np.arange(N) % 5 == 1)[0]
    q[:, :, neg] = -q[:, :, neg]
    y = to_host(la.la_forward(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), feature_map="identity",
                              causal=causal))
    ref = O.attention(q, k, v, "identity", causal=causal)
    num = O.attention(q, k, v, "identity", causal=causal, normalize=False)
    np.testing.assert_allclose(ref[:, :, neg], num[:, :, neg] * 1e6, rtol=1e-12)
    pos = np.setdiff1d(np.arange(N), neg)
    e_neg = rel_err(y[:, :, neg], ref[:, :, neg])
    e_pos = rel_err(y[:, :, pos], ref[:, :, pos])
    log(f"  rel err clamped rows {e_neg:.3e}, other rows {e_pos:.3e}")
    assert e_neg <= TOL["f32"] and e_pos <= TOL["f32"]
