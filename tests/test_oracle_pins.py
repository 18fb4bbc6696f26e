"""Pins for the CPU oracle: checks against values fixed by the pages and by
mathematics, never against a retyped copy of the oracle's own formulas.

Each test names the mistake it is there to catch.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import la_inputs
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    """Golden-file number: a float, {"ln": a} = ln(a), {"sqrt2": c} = c*sqrt(2)."""
    if isinstance(x, dict) and "ln" in x:
        return math.log(x["ln"])
    if isinstance(x, dict) and "sqrt2" in x:
        return x["sqrt2"] * math.sqrt(2.0)
    return float(x)


def _mat(rows):
    return np.array([[_num(x) for x in r] for r in rows], dtype=np.float64)


def _frac(rows):
    return np.array([[float(Fraction(s)) for s in r] for r in rows])


# ---------------------------------------------------------------------------
# Hand-worked examples (tests/golden): pin mask, operand order, state sums
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def elu_example():
    g = _load("worked_example_elu1.json")
    return g, _mat(g["q"]), _mat(g["k"]), _mat(g["v"])


def test_elu_worked_example_definition(elu_example):
    g, q, k, v = elu_example
    for causal, norm, key in [(True, True, "causal_normalized"),
                              (True, False, "causal_unnormalized"),
                              (False, True, "noncausal_normalized"),
                              (False, False, "noncausal_unnormalized")]:
        y = O.attention(q, k, v, "elu1", causal=causal, normalize=norm)
        np.testing.assert_allclose(y, _frac(g[key]), rtol=1e-12, atol=1e-12, err_msg=key)


def test_elu_worked_example_other_forms(elu_example):
    g, q, k, v = elu_example
    exp_c = _frac(g["causal_normalized"])
    for C in (1, 2, 3):
        y, S, z = O.chunked(q, k, v, "elu1", chunk=C)
        np.testing.assert_allclose(y, exp_c, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S, _frac(g["final_S"]), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(z, [float(Fraction(s)) for s in g["final_z"]], rtol=1e-12)
    y, S, z = O.recurrent(q, k, v, "elu1")
    np.testing.assert_allclose(y, exp_c, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, _frac(g["final_S"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.cumsum_form(q, k, v, "elu1"), exp_c, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.cumsum_form(q, k, v, "elu1", normalize=False),
                               _frac(g["causal_unnormalized"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.attention_via_state(q, k, v, "elu1"),
                               _frac(g["noncausal_normalized"]), rtol=1e-12, atol=1e-12)
    S, z = O.final_state(k, v, "elu1")
    np.testing.assert_allclose(S, _frac(g["final_S"]), rtol=1e-12, atol=1e-12)


def test_elu_worked_example_initial_state(elu_example):
    """Catches a dropped S0 or z0 term (numerator or denominator)."""
    g, q, k, v = elu_example
    S0, z0 = np.array(g["S0"]), np.array(g["z0"])
    want = np.array([float(Fraction(s)) for s in g["causal_normalized_with_state_row0"]])
    for y in (O.attention(q, k, v, "elu1", S0=S0, z0=z0)[0],
              O.chunked(q, k, v, "elu1", chunk=2, S0=S0, z0=z0)[0][0],
              O.recurrent(q, k, v, "elu1", S0=S0, z0=z0)[0][0]):
        np.testing.assert_allclose(y, want, rtol=1e-12)


def test_performer_worked_example():
    """Catches a missing d^-1/4 scaling, |x|^2/2 term, 1/sqrt(m) or a q/k swap."""
    g = _load("worked_example_performer.json")
    W, q, k, v = _mat(g["W"]), _mat(g["q"]), _mat(g["k"]), _mat(g["v"])
    c1, ch = math.cosh(1.0), math.cosh(0.5)
    v1, v2 = v[0], v[1]
    y = O.attention(q, k, v, "performer", W, causal=True, normalize=True)
    np.testing.assert_allclose(y, [v1, (c1 * v1 + v2) / (c1 + 1)], rtol=1e-12, atol=1e-15)
    y = O.attention(q, k, v, "performer", W, causal=True, normalize=False)
    np.testing.assert_allclose(y, [math.exp(-2) * ch * v1, c1 * v1 + v2], rtol=1e-12, atol=1e-15)
    y = O.attention(q, k, v, "performer", W, causal=False, normalize=True)
    np.testing.assert_allclose(y, [(v1 + v2) / 2, (c1 * v1 + v2) / (c1 + 1)], rtol=1e-12, atol=1e-15)
    e = math.e
    np.testing.assert_allclose(O.phi_performer(k[0], W),
                               [math.sqrt(e) / math.sqrt(2), 1 / math.sqrt(e) / math.sqrt(2)], rtol=1e-14)


# ---------------------------------------------------------------------------
# Feature maps against fixed values and a library routine
# ---------------------------------------------------------------------------

def test_phi_elu1_values():
    np.testing.assert_allclose(O.phi_elu1([0.0, 1.0, -1.0, 2.5]), [1.0, 2.0, math.exp(-1), 3.5],
                               rtol=1e-15)
    assert O.phi_elu1(np.float32(-1e30)) == 0.0
    assert O.phi_elu1(-1e30) == 0.0
    assert np.all(O.phi_elu1(np.linspace(-50, 50, 1001)) > 0)


def test_phi_elu1_matches_torch_elu():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal(4096) * 3
    ref = (torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0) + 1.0).numpy()
    np.testing.assert_allclose(O.phi_elu1(x), ref, rtol=1e-14, atol=1e-15)


def test_phi_performer_positive_and_unbiased():
    """E_W[phi(x).phi(y)] = exp(x.y/sqrt(d)); pins the sampler and all constants."""
    d, m, seeds = 8, 64, 600
    rng = np.random.default_rng(11)
    x = rng.standard_normal(d) * 0.7
    y = rng.standard_normal(d) * 0.7
    target = math.exp(float(x @ y) / math.sqrt(d))
    est = []
    for s in range(seeds):
        W = la_inputs.performer_W(m, d, seed=10_000 + s, bf16=False)
        fx, fy = O.phi_performer(x, W), O.phi_performer(y, W)
        assert np.all(fx > 0) and np.all(fy > 0)
        est.append(float(fx @ fy))
    est = np.array(est)
    mean, se = est.mean(), est.std(ddof=1) / math.sqrt(seeds)
    assert abs(mean - target) < 4 * se + 1e-3 * target, (mean, target, se)
    # a map without the 1/sqrt(m) constant would be off by a factor m
    assert abs(mean * m - target) > 10 * se


def test_performer_approaches_softmax():
    """Normalized random-feature attention tends to softmax(QK^T/sqrt(d))V as m grows."""
    scipy_special = pytest.importorskip("scipy.special")
    d, N = 8, 16
    rng = np.random.default_rng(5)
    q = rng.standard_normal((N, d)) * 0.5
    k = rng.standard_normal((N, d)) * 0.5
    v = rng.standard_normal((N, d))
    mask = np.tril(np.ones((N, N), bool))
    logits = np.where(mask, q @ k.T / math.sqrt(d), -np.inf)
    ref = scipy_special.softmax(logits, axis=1) @ v
    errs = []
    for m in (16, 256, 4096):
        e = []
        for s in range(8):
            W = la_inputs.performer_W(m, d, seed=777 + 31 * s + m, bf16=False)
            y = O.attention(q, k, v, "performer", W, causal=True)
            e.append(np.linalg.norm(y - ref) / np.linalg.norm(ref))
        errs.append(np.mean(e))
    assert errs[0] > errs[1] > errs[2], errs
    assert errs[2] < 0.05, errs


# ---------------------------------------------------------------------------
# Closed forms and textbook reductions
# ---------------------------------------------------------------------------

def test_identity_map_reduces_to_textbook_products():
    """phi = identity, no denominator: causal = tril(QK^T) V, non-causal = (QK^T) V."""
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((33, 7)) for _ in range(3))
    np.testing.assert_allclose(O.attention(q, k, v, "identity", causal=True, normalize=False),
                               np.tril(q @ k.T) @ v, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(O.attention(q, k, v, "identity", causal=False, normalize=False),
                               (q @ k.T) @ v, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(O.chunked(q, k, v, "identity", normalize=False, chunk=8)[0],
                               np.tril(q @ k.T) @ v, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(O.recurrent(q, k, v, "identity", normalize=False)[0],
                               np.tril(q @ k.T) @ v, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("fmap", ["elu1", "performer"])
def test_closed_form_special_cases(fmap):
    rng = np.random.default_rng(21)
    N, d = 40, 16
    W = la_inputs.performer_W(32, d, seed=3, bf16=False) if fmap == "performer" else None
    q, k, v = (rng.standard_normal((N, d)) * 0.5 for _ in range(3))
    # first causal output equals the first value (inclusive diagonal)
    y = O.attention(q, k, v, fmap, W, causal=True)
    np.testing.assert_allclose(y[0], v[0], rtol=1e-12)
    # constant values give that constant
    c = rng.standard_normal(d)
    for causal in (True, False):
        y = O.attention(q, k, np.tile(c, (N, 1)), fmap, W, causal=causal)
        np.testing.assert_allclose(y, np.tile(c, (N, 1)), rtol=1e-11)
    # identical keys give plain prefix means (causal) / the mean (non-causal)
    kk = np.tile(k[0], (N, 1))
    y = O.attention(q, kk, v, fmap, W, causal=True)
    np.testing.assert_allclose(y, np.cumsum(v, 0) / np.arange(1, N + 1)[:, None], rtol=1e-11,
                               atol=1e-13)
    y = O.attention(q, kk, v, fmap, W, causal=False)
    np.testing.assert_allclose(y, np.tile(v.mean(0), (N, 1)), rtol=1e-11, atol=1e-13)


def test_denominator_clamp():
    """Zero weights (elu+1 of a huge negative input underflows to 0) give y = 0, not NaN."""
    q = np.full((4, 3), -1e30)
    k = np.ones((4, 3))
    v = np.ones((4, 3))
    y = O.attention(q, k, v, "elu1", causal=True)
    assert np.all(y == 0.0)
    y, _, _ = O.decode_step(np.zeros((3, 3)), np.zeros(3), q[0], k[0], v[0])
    assert np.all(y == 0.0)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_invariants():
    rng = np.random.default_rng(4)
    N, d = 50, 8
    q, k, v, v2 = (rng.standard_normal((N, d)) for _ in range(4))
    y = O.attention(q, k, v, "elu1", causal=True)
    # convex hull of the visible values, coordinate-wise
    lo = np.minimum.accumulate(v, axis=0)
    hi = np.maximum.accumulate(v, axis=0)
    assert np.all(y >= lo - 1e-12) and np.all(y <= hi + 1e-12)
    # linear in V for either normalization
    for norm in (True, False):
        a = O.attention(q, k, 2 * v - 3 * v2, "elu1", normalize=norm)
        b = 2 * O.attention(q, k, v, "elu1", normalize=norm) - 3 * O.attention(q, k, v2, "elu1",
                                                                                normalize=norm)
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)
    # scale invariance of the normalized output (positive identity features)
    qp, kp = np.abs(q) + 0.1, np.abs(k) + 0.1
    np.testing.assert_allclose(O.attention(3 * qp, kp, v, "identity"),
                               O.attention(qp, kp, v, "identity"), rtol=1e-12)
    # non-causal: permuting (k, v) pairs changes nothing, permuting queries permutes y
    p = rng.permutation(N)
    y0 = O.attention(q, k, v, "elu1", causal=False)
    np.testing.assert_allclose(O.attention(q, k[p], v[p], "elu1", causal=False), y0, rtol=1e-12)
    np.testing.assert_allclose(O.attention(q[p], k, v, "elu1", causal=False), y0[p], rtol=1e-12)


def test_heads_independent_and_rows_subset():
    q, k, v = la_inputs.gaussian_qkv(2, 3, 70, 16, seed=8, bf16=False)
    y = O.attention(q, k, v, "elu1")
    for b in range(2):
        for h in range(3):
            np.testing.assert_allclose(O.attention(q[b, h], k[b, h], v[b, h], "elu1"), y[b, h],
                                       rtol=1e-13)
    rows = [0, 5, 69, 33]
    np.testing.assert_allclose(O.attention(q, k, v, "elu1", rows=rows), y[:, :, rows], rtol=1e-13)


# ---------------------------------------------------------------------------
# Recurrent and parallel forms agree ([LT] "Comprobar la equivalencia ...")
# ---------------------------------------------------------------------------

def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("shape,seed", [((1, 64, 16), 7), ((1, 128, 32), 42),
                                        ((1, 1, 256, 32), 42)])
@pytest.mark.parametrize("fmap", ["elu1", "performer"])
@pytest.mark.parametrize("normalize", [True, False])
def test_forms_agree(shape, seed, fmap, normalize):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    d = shape[-1]
    W = la_inputs.performer_W(2 * d, d, seed=seed, bf16=False) if fmap == "performer" else None
    ref = O.attention(q, k, v, fmap, W, causal=True, normalize=normalize)
    yr, Sr, zr = O.recurrent(q, k, v, fmap, W, normalize=normalize)
    assert _rel(yr, ref) < 1e-12
    assert _rel(O.cumsum_form(q, k, v, fmap, W, normalize=normalize), ref) < 1e-12
    Sf, zf = O.final_state(k, v, fmap, W)
    for C in (1, 16, 64, 256):
        yc, Sc, zc = O.chunked(q, k, v, fmap, W, normalize=normalize, chunk=C)
        assert _rel(yc, ref) < 1e-12
        assert _rel(Sc, Sf) < 1e-12 and _rel(zc, zf) < 1e-12
    assert _rel(Sr, Sf) < 1e-12 and _rel(zr, zf) < 1e-12
    refn = O.attention(q, k, v, fmap, W, causal=False, normalize=normalize)
    assert _rel(O.attention_via_state(q, k, v, fmap, W, normalize=normalize), refn) < 1e-12


def test_noncausal_snippet_shape():
    rng = np.random.default_rng(42)
    q, k, v = (rng.standard_normal((2, 512, 64)) for _ in range(3))
    a = O.attention(q, k, v, "elu1", causal=False)
    b = O.attention_via_state(q, k, v, "elu1")
    assert _rel(a, b) < 1e-12


def test_decode_continues_prefill():
    """Prefill state + single-token steps == the definition over the whole sequence."""
    rng = np.random.default_rng(12)
    H, N0, T, d = 3, 40, 10, 16
    q, k, v = (rng.standard_normal((H, N0 + T, d)) for _ in range(3))
    ref = O.attention(q, k, v, "elu1", causal=True)
    S, z = O.final_state(k[:, :N0], v[:, :N0], "elu1")
    for t in range(N0, N0 + T):
        y, S, z = O.decode_step(S, z, q[:, t], k[:, t], v[:, t], "elu1")
        np.testing.assert_allclose(y, ref[:, t], rtol=1e-12)
    # split and resume: the definition with an initial state
    S0, z0 = O.final_state(k[:, :N0], v[:, :N0], "elu1")
    tail = O.attention(q[:, N0:], k[:, N0:], v[:, N0:], "elu1", S0=S0, z0=z0)
    np.testing.assert_allclose(tail, ref[:, N0:], rtol=1e-12)
    tail_nc = O.attention(q[:, N0:], k[:, N0:], v[:, N0:], "elu1", causal=False, S0=S0, z0=z0)
    full_nc_last = O.attention(q, k, v, "elu1", causal=True, rows=[N0 + T - 1])
    np.testing.assert_allclose(tail_nc[:, -1:], full_nc_last, rtol=1e-12)


# ---------------------------------------------------------------------------
# Input generators
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    # exact ties: lower 16 bits 0x8000, both parities of the kept bit
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40008000], dtype=np.uint32).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = la_inputs.bf16_round(x)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_performer_W_structure():
    m, d = 40, 16
    W = la_inputs.performer_W(m, d, seed=2, bf16=False).astype(np.float64)
    assert W.shape == (m, d)
    for b0 in range(0, m, d):
        blk = W[b0:b0 + d]
        G = blk @ blk.T
        off = G - np.diag(np.diag(G))
        assert np.max(np.abs(off)) < 1e-4 * np.max(np.diag(G))
    Wb = la_inputs.performer_W(m, d, seed=2)
    np.testing.assert_array_equal(la_inputs.bf16_round(Wb), Wb)


# ---------------------------------------------------------------------------
# Decay (RetNet item of "Variantes y extensiones"): S_t = gamma S_{t-1} + phi(k_t) v_t^T
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def decay_example():
    g = _load("worked_example_decay.json")
    e = _load("worked_example_elu1.json")
    return g, _mat(e["q"]), _mat(e["k"]), _mat(e["v"]), _mat(e["S0"]), np.array(e["z0"], dtype=np.float64)


def test_decay_worked_example(decay_example):
    """Hand-derived values with gamma = 1/2: catches a wrong exponent (i-j+1,
    j-i), an undecayed normalizer, or the decay applied after the update."""
    g, q, k, v, S0, z0 = decay_example
    gam = g["gamma"]
    for norm, key in [(True, "causal_normalized"), (False, "causal_unnormalized")]:
        want = _frac(g[key])
        np.testing.assert_allclose(O.attention(q, k, v, "elu1", normalize=norm, decay=gam), want, rtol=1e-12)
        np.testing.assert_allclose(O.recurrent(q, k, v, "elu1", normalize=norm, decay=gam)[0], want, rtol=1e-12)
        for c in (1, 2, 3):
            np.testing.assert_allclose(O.chunked(q, k, v, "elu1", normalize=norm, chunk=c, decay=gam)[0], want,
                                       rtol=1e-12, err_msg=f"chunk {c}")
    S, z = O.final_state(k, v, "elu1", decay=gam)
    np.testing.assert_allclose(S, _frac(g["final_S"]), rtol=1e-12)
    np.testing.assert_allclose(z, np.array([float(Fraction(x)) for x in g["final_z"]]), rtol=1e-12)
    for c in (1, 2):
        _, Sc, zc = O.chunked(q, k, v, "elu1", chunk=c, decay=gam)
        np.testing.assert_allclose(Sc, S, rtol=1e-12)
        np.testing.assert_allclose(zc, z, rtol=1e-12)
    Sw, zw = _frac(g["final_S_with_state"]), np.array([float(Fraction(x)) for x in g["final_z_with_state"]])
    for Sx, zx in (O.final_state(k, v, "elu1", S0=S0, z0=z0, decay=gam),
                   O.recurrent(q, k, v, "elu1", S0=S0, z0=z0, decay=gam)[1:],
                   O.chunked(q, k, v, "elu1", chunk=2, S0=S0, z0=z0, decay=gam)[1:]):
        np.testing.assert_allclose(Sx, Sw, rtol=1e-12)
        np.testing.assert_allclose(zx, zw, rtol=1e-12)
    want0 = np.array([float(Fraction(x)) for x in g["causal_normalized_with_state_row0"]])
    for y in (O.attention(q, k, v, "elu1", S0=S0, z0=z0, decay=gam)[0],
              O.recurrent(q, k, v, "elu1", S0=S0, z0=z0, decay=gam)[0][0],
              O.chunked(q, k, v, "elu1", chunk=2, S0=S0, z0=z0, decay=gam)[0][0]):
        np.testing.assert_allclose(y, want0, rtol=1e-12)


def test_decay_zero_and_one():
    """gamma = 0 keeps only the current token (normalized y_i = v_i); gamma = 1 is no decay."""
    q, k, v = la_inputs.gaussian_qkv(1, 2, 70, 8, seed=3, scale=1.0, bf16=False)
    for f in (lambda **kw: O.attention(q, k, v, "elu1", **kw),
              lambda **kw: O.recurrent(q, k, v, "elu1", **kw)[0],
              lambda **kw: O.chunked(q, k, v, "elu1", chunk=16, **kw)[0]):
        np.testing.assert_allclose(f(decay=0.0), v, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(f(decay=1.0), f(), rtol=1e-12, atol=1e-12)
    qf, kf = O.phi_elu1(q), O.phi_elu1(k)
    np.testing.assert_allclose(O.attention(q, k, v, "elu1", normalize=False, decay=0.0),
                               np.sum(qf * kf, axis=-1, keepdims=True) * v, rtol=1e-12)


def test_decay_equal_keys_is_a_first_order_filter():
    """All keys equal: y_i = sum_j gamma^(i-j) v_j / sum_j gamma^(i-j), the
    ratio of two first-order recursive filters (scipy.signal.lfilter)."""
    from scipy.signal import lfilter
    rng = np.random.default_rng(8)
    N, d, gam = 90, 6, 0.83
    # positive q, k keep the identity map's denominator positive (away from the clamp)
    q = rng.uniform(0.1, 1.0, (N, d))
    k = np.broadcast_to(rng.uniform(0.1, 1.0, (1, d)), (N, d))
    v = rng.standard_normal((N, d))
    want = lfilter([1.0], [1.0, -gam], v, axis=0) / lfilter([1.0], [1.0, -gam], np.ones((N, 1)), axis=0)
    for fmap in ("elu1", "identity"):
        np.testing.assert_allclose(O.attention(q, k, v, fmap, decay=gam), want, rtol=1e-10)
        np.testing.assert_allclose(O.chunked(q, k, v, fmap, chunk=32, decay=gam)[0], want, rtol=1e-10)


def test_decay_split_resume_per_head_and_decode():
    """The state after a prefix (decayed to its end) continues the sequence;
    each head keeps its own gamma; decode steps continue a decayed prefill."""
    q, k, v = la_inputs.gaussian_qkv(2, 3, 150, 16, seed=12, scale=0.7, bf16=False)
    gam = np.array([0.95, 0.6, 0.999])
    full = O.attention(q, k, v, "elu1", decay=gam)
    S, z = O.final_state(k[:, :, :100], v[:, :, :100], "elu1", decay=gam)
    tail = O.attention(q[:, :, 100:], k[:, :, 100:], v[:, :, 100:], "elu1", S0=S, z0=z, decay=gam)
    np.testing.assert_allclose(tail, full[:, :, 100:], rtol=1e-10, atol=1e-12)
    for h in range(3):
        one = O.attention(q[:, h], k[:, h], v[:, h], "elu1", decay=gam[h])
        np.testing.assert_allclose(one, full[:, h], rtol=1e-12)
    Sd, zd = S, z
    for t in range(100, 104):
        y, Sd, zd = O.decode_step(Sd, zd, q[:, :, t], k[:, :, t], v[:, :, t], "elu1", decay=gam[None, :])
        np.testing.assert_allclose(y, full[:, :, t], rtol=1e-10, atol=1e-12)
    with pytest.raises(ValueError):
        O.attention(q, k, v, "elu1", causal=False, decay=0.9)
