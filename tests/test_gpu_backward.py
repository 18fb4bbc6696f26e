"""GPU parity of la_backward (gradients of causal linear attention).

Reference: the oracle's attention_backward (the vector-Jacobian product of
the definition, pinned by finite differences in test_oracle_backward_pins.py)
on the same seeded inputs. Error per (batch, head): Frobenius norm of the
difference over the reference's, <= 2e-2 for bf16 inputs and <= 1e-4 for
fp32 inputs (the forward's bar: the gradient passes use the same operand
precisions). Where the exact gradient vanishes (dq and dk of a one-token
normalized sequence: the output is v_0 whatever q and k are) the error is
measured against 1e-3 of the output cotangent's norm instead.

Beside that norm, every row is checked on its own (its error over its
reference norm), so that one wrong row cannot hide in the norm of a long
sequence. Gradient rows are sums of terms of both signs (dk_j = phi'(k_j)
sum_{i>=j} phi(q_i) g_i.(v_j - y_i), and alike), so a row can cancel far below
its terms while its rounding error follows the terms, and the size of the
terms falls by orders of magnitude along a sequence (g_i = dy_i / D_i with D_i
growing with i): on the long-context workload a dk row with 6 times the
head's RMS row norm sat among neighbours of 40-70 times it. Each row is
therefore measured against at least half the RMS row norm of its 64-token
block (gpu_helpers.err_parts_local). Rows whose exact gradient vanishes are
left to the norm check: in the normalized form the first output is v_0
whatever q_0 is, so row 0 of dq is exactly zero and the GPU returns rounding
noise there.
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
from gpu_helpers import TOL, caller, err_parts_local, log, note_row, qkv, to_dev, to_host  # noqa: E402


def _dout(B, H, N, d, seed, dt):
    rng = np.random.default_rng(seed + 7919)
    return la_inputs.gaussian(rng, (B, H, N, d), 1.0, bf16=(dt == "bf16"))


def _err(g, r, dy, vanishing=False, skip_row0=False):
    """Larger of: max over (batch, head) of ||g - r||_F / ||r||_F (or
    / (1e-3 ||dy||_F) for a gradient that vanishes exactly), and the per-row
    error of err_parts_local (not taken for a vanishing gradient; without
    row 0 when skip_row0)."""
    G = g.reshape(-1, g.shape[-2] * g.shape[-1])
    R = r.reshape(G.shape)
    Y = dy.reshape(G.shape[0], -1)
    num = np.linalg.norm(G - R, axis=1)
    den = 1e-3 * np.linalg.norm(Y, axis=1) if vanishing else np.maximum(np.linalg.norm(R, axis=1), 1e-30)
    frob = float(np.max(num / den))
    if vanishing:
        return frob
    g3 = g.reshape(-1, g.shape[-2], g.shape[-1])
    r3 = r.reshape(g3.shape)
    if skip_row0:
        if g3.shape[1] == 1:
            return frob
        # row 0 keeps its place in its block's scale but is not checked
        # itself: the GPU's value there is replaced by the reference
        g3 = np.concatenate([r3[:, :1], g3[:, 1:]], axis=1)
    row, at = err_parts_local(g3, r3)
    note_row(row, at, caller(1))
    return float(np.max([frob, row]))


def _gammas(H):
    """Per-head decays spanning the supported range [1/4, 1]."""
    return np.array([0.25, 0.7, 0.97, 1.0, 0.999, 0.5][:H], dtype=np.float32)


def _check(B, H, N, d, dt, seed, fmap="elu1", normalize=True, state=False, positive=False, decay=False):
    log(f"case backward B{B} H{H} N{N} d{d} {dt} {fmap} norm={normalize} state={state} decay={decay}")
    q, k, v = qkv(B, H, N, d, seed, dt, 1.0)
    if positive:  # identity map, normalized: positive q, k keep the denominators away from 0
        q, k = np.abs(q), np.abs(k)
    dy = _dout(B, H, N, d, seed, dt)
    kw, okw = {}, {}
    if state:
        rng = np.random.default_rng(seed + 11)
        S0 = rng.standard_normal((B, H, d, d)).astype(np.float32) * 0.5
        z0 = rng.uniform(0.5, 2.0, (B, H, d)).astype(np.float32)
        dS = rng.standard_normal((B, H, d, d)).astype(np.float32) * 0.1
        dz = rng.standard_normal((B, H, d)).astype(np.float32) * 0.1
        dev = lambda x: torch.from_numpy(x).cuda()  # noqa: E731
        kw = dict(S_in=dev(S0), z_in=dev(z0), dS_out=dev(dS), dz_out=dev(dz), return_state_grad=True)
        okw = dict(S0=S0, z0=z0, dS_N=dS, dz_N=dz)
    args = (to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(dy, dt))
    if decay:
        g = _gammas(H)
        res = la.la_backward_decay(*args, torch.from_numpy(g).cuda(), feature_map=fmap, normalize=normalize, **kw)
        okw["decay"] = g.astype(np.float64)
    else:
        res = la.la_backward(*args, feature_map=fmap, normalize=normalize, **kw)
    torch.cuda.synchronize()
    ref = O.attention_backward(q, k, v, dy, fmap, causal=True, normalize=normalize, **okw)
    names = ("dq", "dk", "dv", "dS_in", "dz_in")
    for i, got in enumerate(res):
        g = to_host(got)
        r = ref[i]
        if g.ndim == 3:   # dz_in [B, H, d]: one row per (batch, head)
            g, r = g[..., None, :], r[..., None, :]
        err = _err(g, r, dy, vanishing=(N == 1 and normalize and i < 2), skip_row0=(normalize and i == 0))
        log(f"  {names[i]} rel err {err:.3e}")
        assert err <= TOL[dt], (names[i], err)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_small(d, dt):
    for N in (1, 63, 64, 65, 200):
        _check(2, 2, N, d, dt, seed=900 + N + d)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("normalize", [True, False])
def test_backward_multisegment(d, dt, normalize):
    # 40 chunks with a ragged tail: several segments per sequence
    _check(1, 2, 64 * 40 - 17, d, dt, seed=31 + d, normalize=normalize)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_state_in_and_out(d, dt):
    _check(1, 2, 64 * 12 + 9, d, dt, seed=57 + d, state=True)
    _check(2, 1, 70, d, dt, seed=58 + d, state=True)   # single segment


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_identity_map(d, dt):
    _check(1, 2, 64 * 9 + 30, d, dt, seed=77 + d, fmap="identity", normalize=False)
    _check(1, 2, 64 * 9 + 30, d, dt, seed=78 + d, fmap="identity", normalize=True, positive=True)


def test_backward_empty_sequence_passes_state_gradient():
    d = 64
    dS = torch.randn(1, 2, d, d, device="cuda")
    dz = torch.randn(1, 2, d, device="cuda")
    x = torch.zeros(1, 2, 0, d, device="cuda", dtype=torch.bfloat16)
    _, _, _, dS_in, dz_in = la.la_backward(x, x.clone(), x.clone(), x.clone(), dS_out=dS, dz_out=dz,
                                           return_state_grad=True)
    torch.cuda.synchronize()
    assert torch.equal(dS_in, dS) and torch.equal(dz_in, dz)


def test_backward_full_b1h16n65536d128_sampled_heads():
    """The long-context workload in one call (the library's own segment
    split); every gradient of two heads against the recurrent form of the
    oracle's gradients (O(N d^2) per head, so whole heads fit in seconds)."""
    W = la_inputs.WORKLOADS["prefill_b1h16n65536d128"]
    B, H, N, d = W["B"], W["H"], W["N"], W["d"]
    log(f"case full backward B{B} H{H} N{N} d{d} bf16 (heads 0 and 15 checked)")
    q, k, v = la_inputs.gaussian_qkv(B, H, N, d, seed=W["seed"], scale=W["scale"], bf16=True)
    dy = _dout(B, H, N, d, W["seed"], "bf16")
    dq, dk, dv, dS, dz = la.la_backward(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                        to_dev(dy, "bf16"), return_state_grad=True)
    torch.cuda.synchronize()
    for h in (0, 15):
        ref = O.recurrent_backward(q[:, h], k[:, h], v[:, h], dy[:, h], "elu1")
        for name, got, r in zip(("dq", "dk", "dv", "dS_in"), (dq, dk, dv, dS), ref[:4]):
            err = _err(to_host(got[:, h]), r, dy[:, h], skip_row0=(name == "dq"))
            log(f"  head {h} {name} rel err {err:.3e}")
            assert err <= TOL["bf16"], (h, name, err)
        ez = _err(to_host(dz[:, h])[..., None, :], ref[4][..., None, :], dy[:, h])
        assert ez <= TOL["bf16"], (h, "dz_in", ez)


@pytest.mark.parametrize("decay", [False, True])
def test_backward_odd_segment_count(decay):
    """B1 H3 with 684 chunks (a ragged tail of 47 tokens): the state passes
    split each sequence into 171 segments, and the dq and dk/dv passes, which
    take two of those per segment, end on a segment of one. Every gradient of
    every head, with final-state cotangents, against the recurrent form of the
    oracle's gradients."""
    B, H, N, d = 1, 3, 64 * 684 - 17, 64
    log(f"case backward B{B} H{H} N{N} d{d} bf16 decay={decay} (171 state-pass segments)")
    q, k, v = qkv(B, H, N, d, 77, "bf16", 1.0)
    dy = _dout(B, H, N, d, 77, "bf16")
    rng = np.random.default_rng(78)
    dS = (rng.standard_normal((B, H, d, d)) * 0.1).astype(np.float32)
    dz = (rng.standard_normal((B, H, d)) * 0.1).astype(np.float32)
    args = (to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(dy, "bf16"))
    kw = dict(dS_out=torch.from_numpy(dS).cuda(), dz_out=torch.from_numpy(dz).cuda(), return_state_grad=True)
    g = _gammas(H)
    if decay:
        res = la.la_backward_decay(*args, torch.from_numpy(g).cuda(), **kw)
    else:
        res = la.la_backward(*args, **kw)
    torch.cuda.synchronize()
    for h in range(H):
        ref = O.recurrent_backward(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], dy[:, h:h + 1], "elu1",
                                   dS_N=dS[:, h:h + 1], dz_N=dz[:, h:h + 1],
                                   decay=g[h:h + 1].astype(np.float64) if decay else None)
        for name, got, r in zip(("dq", "dk", "dv", "dS_in"), res[:4], ref[:4]):
            err = _err(to_host(got[:, h:h + 1]), r, dy[:, h:h + 1], skip_row0=(name == "dq"))
            log(f"  head {h} {name} rel err {err:.3e}")
            assert err <= TOL["bf16"], (h, name, err)
        ez = _err(to_host(res[4][:, h:h + 1])[..., None, :], ref[4][..., None, :], dy[:, h:h + 1])
        assert ez <= TOL["bf16"], (h, "dz_in", ez)


# --- decay (per-head gamma): gradients of la_forward_decay ---------------------------------------------------


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_decay_small(d, dt):
    for N in (1, 63, 64, 65, 200):
        _check(1, 4, N, d, dt, seed=1900 + N + d, decay=True)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("normalize", [True, False])
def test_backward_decay_multisegment(d, dt, normalize):
    # 40 chunks with a ragged tail: several segments, the last one partial
    _check(1, 4, 64 * 40 - 17, d, dt, seed=131 + d, normalize=normalize, decay=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_decay_state_in_and_out(d, dt):
    _check(1, 4, 64 * 12 + 9, d, dt, seed=157 + d, state=True, decay=True)
    _check(2, 2, 70, d, dt, seed=158 + d, state=True, decay=True)   # single segment
    _check(1, 4, 64 * 12, d, dt, seed=159 + d, state=True, decay=True)   # whole chunks only


@pytest.mark.parametrize("d", [32, 64, 128])
def test_backward_decay_identity_map(d):
    _check(1, 4, 64 * 9 + 30, d, "bf16", seed=177 + d, fmap="identity", normalize=False, decay=True)
    _check(1, 4, 64 * 9 + 30, d, "f32", seed=178 + d, fmap="identity", normalize=True, positive=True, decay=True)


def test_backward_decay_one_equals_no_decay():
    q, k, v = qkv(1, 2, 700, 64, 5, "bf16", 1.0)
    dy = _dout(1, 2, 700, 64, 5, "bf16")
    args = [to_dev(x, "bf16") for x in (q, k, v, dy)]
    a = la.la_backward(*args)
    b = la.la_backward_decay(*args, torch.ones(2, device="cuda"))
    torch.cuda.synchronize()
    # the same arithmetic up to the order of the fp32 accumulations (the
    # decay passes scale and walk their states differently), which the
    # gradients see in full where they carry fp32 states as hi + lo operands:
    # 1e-4 on the norm of each head, 5e-3 on every row
    for i, (x, y) in enumerate(zip(a, b)):
        gx, gy = to_host(x), to_host(y)
        frob = float(np.max(np.linalg.norm((gy - gx).reshape(2, -1), axis=1) /
                            np.linalg.norm(gx.reshape(2, -1), axis=1)))
        err = _err(gy, gx, dy, skip_row0=(i == 0))
        assert frob <= 1e-4 and err <= 5e-3, (i, frob, err)


def test_backward_decay_empty_sequence_passes_state_gradient():
    d = 64
    dS = torch.randn(1, 2, d, d, device="cuda")
    dz = torch.randn(1, 2, d, device="cuda")
    x = torch.zeros(1, 2, 0, d, device="cuda", dtype=torch.bfloat16)
    _, _, _, dS_in, dz_in = la.la_backward_decay(x, x.clone(), x.clone(), x.clone(), torch.full((2,), 0.5, device="cuda"),
                                                 dS_out=dS, dz_out=dz, return_state_grad=True)
    torch.cuda.synchronize()
    assert torch.equal(dS_in, dS) and torch.equal(dz_in, dz)


def test_backward_decay_full_b1h16n65536d128_sampled_heads():
    """The long-context workload with one decay per head, 1 - 2^-(5+h), in one
    call; two heads checked against the recurrent form of the oracle's gradients."""
    W = la_inputs.WORKLOADS["prefill_b1h16n65536d128"]
    B, H, N, d = W["B"], W["H"], W["N"], W["d"]
    log(f"case full decay backward B{B} H{H} N{N} d{d} bf16 (heads 0 and 15 checked)")
    g = np.array([1.0 - 2.0 ** (-5 - h) for h in range(H)], dtype=np.float32)
    q, k, v = la_inputs.gaussian_qkv(B, H, N, d, seed=W["seed"], scale=W["scale"], bf16=True)
    dy = _dout(B, H, N, d, W["seed"], "bf16")
    dq, dk, dv, dS, dz = la.la_backward_decay(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                              to_dev(dy, "bf16"), torch.from_numpy(g).cuda(), return_state_grad=True)
    torch.cuda.synchronize()
    for h in (0, 15):
        ref = O.recurrent_backward(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], dy[:, h:h + 1], "elu1",
                                   decay=g[h:h + 1].astype(np.float64))
        for name, got, r in zip(("dq", "dk", "dv", "dS_in"), (dq, dk, dv, dS), ref[:4]):
            err = _err(to_host(got[:, h:h + 1]), r, dy[:, h:h + 1], skip_row0=(name == "dq"))
            log(f"  head {h} {name} rel err {err:.3e}")
            assert err <= TOL["bf16"], (h, name, err)
        ez = _err(to_host(dz[:, h:h + 1])[..., None, :], ref[4][..., None, :], dy[:, h:h + 1])
        assert ez <= TOL["bf16"], (h, "dz_in", ez)


def test_backward_decay_out_of_range_gamma_is_flagged():
    """gamma = 0.05 on one head: that head's gradients are NaN, the other
    head's match the oracle, la_device_status reports the violation."""
    B, H, N, d = 1, 2, 64 * 6 + 3, 64
    log("case backward decay out-of-range gamma")
    assert la.la_device_status() in (la.LA_OK, la.LA_ERR_INVALID_ARG)
    q, k, v = qkv(B, H, N, d, 93, "bf16", 1.0)
    dy = _dout(B, H, N, d, 93, "bf16")
    g = np.array([0.05, 0.8], dtype=np.float32)
    res = la.la_backward_decay(*(to_dev(x, "bf16") for x in (q, k, v, dy)), torch.from_numpy(g).cuda(),
                               return_state_grad=True)
    torch.cuda.synchronize()
    assert la.la_device_status() == la.LA_ERR_INVALID_ARG
    ref = O.attention_backward(q[:, 1:2], k[:, 1:2], v[:, 1:2], dy[:, 1:2], "elu1", causal=True, decay=0.8)
    for i, got in enumerate(res):
        gh = to_host(got)
        assert np.isnan(gh[:, 0]).all(), i
        r = ref[i]
        g1 = gh[:, 1:2]
        if g1.ndim == 3:
            g1, r = g1[..., None, :], r[..., None, :]
        err = _err(g1, r, dy[:, 1:2], skip_row0=(i == 0))
        assert err <= TOL["bf16"], (i, err)
