"""GPU parity of gated linear attention (la_forward_gated, la_decode_step_gated).

Reference: the oracle's gated forms (definition / blockwise, pinned in
test_oracle_gated_pins.py) on the same seeded inputs and gates; gates
alpha ~ U(lo, 1) with lo down to 1/4, the smallest the chunked kernels
accept. Error: relative Frobenius norm per (batch, head) <= 2e-2 (bf16
inputs), <= 1e-4 (fp32 inputs).
"""

import numpy as np
import pytest

import la_inputs
import oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

import causal_linear_attention_02_amd as la  # noqa: E402
from gpu_helpers import TOL, log, qkv, rel_err, rel_err_terms, to_dev, to_host  # noqa: E402


def _g(shape, seed, lo):
    return la_inputs.log_gates(np.random.default_rng(seed + 313), shape, lo)


def _check(B, H, N, d, dt, seed, lo=0.25, fmap="elu1", normalize=True, state=False, scale=1.0):
    log(f"case gated forward B{B} H{H} N{N} d{d} {dt} {fmap} norm={normalize} lo={lo} state={state}")
    q, k, v = qkv(B, H, N, d, seed, dt, scale)
    if fmap == "identity" and normalize:
        q, k = np.abs(q), np.abs(k)
    lg = _g((B, H, N, d), seed, lo)
    kw, okw = {}, {}
    if state:
        rng = np.random.default_rng(seed + 17)
        S0 = (rng.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
        z0 = rng.uniform(0.5, 2.0, (B, H, d)).astype(np.float32)
        kw = dict(S_in=torch.from_numpy(S0).cuda(), z_in=torch.from_numpy(z0).cuda(), return_state=True)
        okw = dict(S0=S0, z0=z0)
    res = la.la_forward_gated(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), torch.from_numpy(lg).cuda(),
                              feature_map=fmap, normalize=normalize, **kw)
    torch.cuda.synchronize()
    y = res[0] if state else res
    yr, Sr, zr = O.gated_chunked(q, k, v, lg, fmap, normalize=normalize, chunk=64, **okw)
    if fmap == "identity" and not normalize:
        # signed sums over few tokens (the gates decay fast): a row can cancel
        # far below its terms, so rows are measured componentwise, against the
        # same sums over absolute values (a CPU emulation of the kernel's bf16
        # rounding reproduces its worst row, 2.6e-2 against the row norm,
        # 1.8e-3 against those sums)
        aS0 = None if not state else np.abs(okw["S0"])
        terms = O.gated_chunked(np.abs(q), np.abs(k), np.abs(v), lg, "identity", normalize=False, chunk=64,
                                S0=aS0, z0=None if not state else okw["z0"])[0]
        err = rel_err_terms(to_host(y), yr, terms)
    else:
        err = rel_err(to_host(y), yr)
    log(f"  rel err {err:.3e}")
    assert err <= TOL[dt], err
    if state:
        eS = rel_err(to_host(res[1]), Sr)
        ez = rel_err(to_host(res[2])[..., None], zr[..., None])
        log(f"  state rel err S {eS:.3e} z {ez:.3e}")
        assert eS <= TOL[dt] and ez <= TOL[dt]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gated_small(d, dt):
    for N in (1, 63, 64, 65, 200):
        _check(2, 2, N, d, dt, seed=700 + N + d)


def test_gated_small_matches_the_definition():
    """A short case against the definition itself (explicit weights per key and channel)."""
    B, H, N, d = 1, 2, 150, 64
    q, k, v = qkv(B, H, N, d, 5, "f32")
    lg = _g((B, H, N, d), 5, 0.25)
    y = la.la_forward_gated(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    err = rel_err(to_host(y), O.gated_attention(q, k, v, lg))
    assert err <= TOL["f32"], err


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("normalize", [True, False])
def test_gated_multisegment(d, dt, normalize):
    _check(1, 2, 64 * 40 - 17, d, dt, seed=41 + d, normalize=normalize)


@pytest.mark.parametrize("lo", [0.25, 0.9, 1.0])
def test_gated_gate_ranges(lo):
    # the smallest gate, gates close to 1, and no gating at all (alpha = 1)
    _check(1, 2, 64 * 24 + 5, 128, "bf16", seed=3, lo=lo)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gated_state_in_and_out(d, dt):
    _check(1, 2, 64 * 12 + 9, d, dt, seed=57 + d, state=True)
    _check(2, 1, 70, d, dt, seed=58 + d, state=True)


@pytest.mark.parametrize("d", [32, 128])
def test_gated_identity_map(d):
    _check(1, 2, 64 * 9 + 30, d, "bf16", seed=77 + d, fmap="identity", normalize=False)


def test_gated_ones_equal_ungated_forward():
    B, H, N, d = 1, 4, 64 * 20 + 3, 128
    q, k, v = qkv(B, H, N, d, 9, "bf16", d ** -0.5)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    yg = la.la_forward_gated(tq, tk, tv, torch.zeros((B, H, N, d), device="cuda"))
    y = la.la_forward(tq, tk, tv)
    torch.cuda.synchronize()
    assert rel_err(to_host(yg), to_host(y)) <= 1e-2


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gated_decode(d, dt):
    log(f"case gated decode d{d} {dt}")
    B, H, N0, T = 2, 3, 90, 4
    q, k, v = qkv(B, H, N0 + T, d, 71 + d, dt)
    lg = _g((B, H, N0 + T, d), 71 + d, 0.25)
    S0, z0 = O.gated_final_state(k[:, :, :N0], v[:, :, :N0], lg[:, :, :N0])
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    Sr, zr = S0, z0
    for t in range(N0, N0 + T):
        y = la.la_decode_step_gated(S, z, to_dev(q[:, :, t], dt), to_dev(k[:, :, t], dt), to_dev(v[:, :, t], dt),
                                    torch.from_numpy(np.ascontiguousarray(lg[:, :, t])).cuda())
        yr, Sr, zr = O.gated_decode_step(Sr, zr, q[:, :, t], k[:, :, t], v[:, :, t], lg[:, :, t])
        torch.cuda.synchronize()
        err = rel_err(to_host(y)[..., None, :], yr[..., None, :])
        assert err <= TOL[dt], (t, err)
    assert rel_err(to_host(S), Sr) <= 1e-4


def test_gated_prefill_decode_handoff():
    B, H, N0, T, d = 1, 3, 64 * 5 + 3, 4, 64
    q, k, v = qkv(B, H, N0 + T, d, 91, "bf16")
    lg = _g((B, H, N0 + T, d), 91, 0.25)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    tg = torch.from_numpy(lg).cuda()
    _, S, z = la.la_forward_gated(tq[:, :, :N0].contiguous(), tk[:, :, :N0].contiguous(),
                                  tv[:, :, :N0].contiguous(), tg[:, :, :N0].contiguous(), return_state=True)
    ref, _, _ = O.gated_chunked(q, k, v, lg)
    for t in range(N0, N0 + T):
        y = la.la_decode_step_gated(S, z, tq[:, :, t].contiguous(), tk[:, :, t].contiguous(),
                                    tv[:, :, t].contiguous(), tg[:, :, t].contiguous())
        torch.cuda.synchronize()
        assert rel_err(to_host(y)[..., None, :], ref[:, :, t][..., None, :]) <= TOL["bf16"]


def test_gated_full_b1h16n65536d128_sampled_heads():
    W = la_inputs.WORKLOADS["prefill_b1h16n65536d128"]
    B, H, N, d = W["B"], W["H"], W["N"], W["d"]
    log(f"case full gated forward B{B} H{H} N{N} d{d} bf16 (heads 0 and 15 checked)")
    q, k, v = la_inputs.gaussian_qkv(B, H, N, d, seed=W["seed"], scale=W["scale"], bf16=True)
    lg = _g((B, H, N, d), W["seed"], 0.9)
    y, S, z = la.la_forward_gated(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                  torch.from_numpy(lg).cuda(), return_state=True)
    torch.cuda.synchronize()
    for h in (0, 15):
        yr, Sr, zr = O.gated_chunked(q[:, h], k[:, h], v[:, h], lg[:, h])
        e = rel_err(to_host(y[:, h]), yr)
        eS = rel_err(to_host(S[:, h]), Sr)
        log(f"  head {h} rel err y {e:.3e} S {eS:.3e}")
        assert e <= TOL["bf16"] and eS <= TOL["bf16"]


def test_gated_odd_segment_count():
    """B1 H3 with 684 chunks (a ragged tail of 47 tokens): the state pass splits
    each sequence into 171 segments, and the output pass, which takes two of
    those per segment, ends on a segment of one. Every head, with a state in
    and out, against the oracle's blockwise form."""
    B, H, N, d = 1, 3, 64 * 684 - 17, 64
    log(f"case gated forward B{B} H{H} N{N} d{d} bf16 (171 state-pass segments)")
    q, k, v = qkv(B, H, N, d, 19, "bf16", 1.0)
    lg = _g((B, H, N, d), 19, 0.25)
    rng = np.random.default_rng(20)
    S0 = (rng.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    z0 = rng.uniform(0.5, 2.0, (B, H, d)).astype(np.float32)
    y, S, z = la.la_forward_gated(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                  torch.from_numpy(lg).cuda(), S_in=torch.from_numpy(S0).cuda(),
                                  z_in=torch.from_numpy(z0).cuda(), return_state=True)
    torch.cuda.synchronize()
    yr, Sr, zr = O.gated_chunked(q, k, v, lg, S0=S0, z0=z0)
    e = rel_err(to_host(y), yr)
    eS = rel_err(to_host(S), Sr)
    ez = rel_err(to_host(z)[..., None], zr[..., None])
    log(f"  rel err y {e:.3e} S {eS:.3e} z {ez:.3e}")
    assert e <= TOL["bf16"] and eS <= TOL["bf16"] and ez <= TOL["bf16"]


def test_gated_out_of_range_gate_is_flagged():
    """One gate below 1/4 in one head (token 200, channel 5): that head's
    outputs from the chunk of that token on are NaN, earlier rows and the
    other head match the oracle, and la_device_status reports it."""
    B, H, N, d = 1, 2, 64 * 8, 64
    log("case gated out-of-range gate")
    assert la.la_device_status() in (la.LA_OK, la.LA_ERR_INVALID_ARG)
    q, k, v = qkv(B, H, N, d, 95, "bf16", 1 / 8)
    lg = _g((B, H, N, d), 95, 0.25)
    lg[0, 0, 200, 5] = np.log(np.float32(0.05))
    y = to_host(la.la_forward_gated(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                    torch.from_numpy(lg).cuda()))
    torch.cuda.synchronize()
    assert la.la_device_status() == la.LA_ERR_INVALID_ARG
    assert np.isnan(y[0, 0, 256:]).all()
    ref = O.gated_attention(q, k, v, lg)
    assert rel_err(y[:, 1:], ref[:, 1:]) <= TOL["bf16"]
    assert rel_err(y[:, :1, :192], ref[:, :1, :192]) <= TOL["bf16"]
