"""Pins of the oracle's gated forms (CPU only).

Gated linear attention ("Linear Attention", marovi.ai, "Variantes y
extensiones", GLA item) read as a per-token, per-channel gate on the
feature dimension. The gated forms share no code with the pinned ungated
and decay forms, and are pinned by:
* a hand-worked example with gates varying over tokens and channels
  (tests/golden/worked_example_gated.json), with and without an initial
  state, normalized and not, and the final state;
* special cases: log-gates 0 give the ungated definition; a gate constant
  over tokens and channels gives the decay form (itself pinned in
  test_oracle_pins.py);
* the forms against each other: definition, recurrent loop, blockwise at
  several block sizes, split/resume with the final state;
* a normalized output stays a weighted mean of the values (inside their
  per-coordinate range).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example_gated.json")


def _fr(x):
    return np.array([[float(Fraction(c)) for c in r] for r in x]) if isinstance(x[0], list) else \
        np.array([float(Fraction(c)) for c in x])


@pytest.fixture(scope="module")
def gold():
    with open(GOLD) as f:
        return json.load(f)


def _ex(g):
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    lg = np.log(_fr(g["alpha"]))
    return q, k, v, lg


def test_worked_example_outputs(gold):
    q, k, v, lg = _ex(gold)
    for fn in (O.gated_attention, lambda *a, **kw: O.gated_recurrent(*a, **kw)[0],
               lambda *a, **kw: O.gated_chunked(*a, chunk=2, **kw)[0]):
        np.testing.assert_allclose(fn(q, k, v, lg, "identity", normalize=False), _fr(gold["unnormalized"]),
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(fn(q, k, v, lg, "identity"), _fr(gold["normalized"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(fn(q, k, v, lg, "identity", S0=np.eye(2), z0=np.ones(2)),
                                   _fr(gold["normalized_with_state"]), rtol=0, atol=1e-12)


def test_worked_example_final_state(gold):
    q, k, v, lg = _ex(gold)
    S, z = O.gated_final_state(k, v, lg, "identity")
    np.testing.assert_allclose(S, _fr(gold["final_S"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(z, _fr(gold["final_z"]), rtol=0, atol=1e-12)
    S, z = O.gated_final_state(k, v, lg, "identity", S0=np.eye(2), z0=np.ones(2))
    np.testing.assert_allclose(S, _fr(gold["final_S_with_state"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(z, _fr(gold["final_z_with_state"]), rtol=0, atol=1e-12)
    _, S2, z2 = O.gated_recurrent(q, k, v, lg, "identity", S0=np.eye(2), z0=np.ones(2))
    np.testing.assert_allclose(S2, S, rtol=0, atol=1e-12)
    np.testing.assert_allclose(z2, z, rtol=0, atol=1e-12)


def _rand(seed, B=2, H=3, N=37, d=6, m=8, fmap="elu1"):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    dfeat = m if fmap == "performer" else d
    lg = np.log(rng.uniform(0.3, 1.0, (B, H, N, dfeat)))
    W = rng.standard_normal((m, d)) if fmap == "performer" else None
    return q, k, v, lg, W


@pytest.mark.parametrize("fmap", ["elu1", "identity", "performer"])
def test_zero_log_gates_are_the_ungated_definition(fmap):
    q, k, v, lg, W = _rand(1, fmap=fmap)
    if fmap == "identity":
        q, k = np.abs(q), np.abs(k)
    z = np.zeros_like(lg)
    for norm in (True, False):
        np.testing.assert_allclose(O.gated_attention(q, k, v, z, fmap, W=W, normalize=norm),
                                   O.attention(q, k, v, fmap, W=W, causal=True, normalize=norm), rtol=1e-12, atol=1e-12)


def test_uniform_gate_is_the_decay_form():
    q, k, v, _, _ = _rand(2)
    gam = np.array([0.5, 0.8, 0.95])                         # one per head
    lg = np.broadcast_to(np.log(gam)[None, :, None, None], q.shape).copy()
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((2, 3, 6, 6))
    z0 = rng.uniform(0.5, 1.5, (2, 3, 6))
    np.testing.assert_allclose(O.gated_attention(q, k, v, lg, S0=S0, z0=z0),
                               O.attention(q, k, v, causal=True, S0=S0, z0=z0, decay=gam), rtol=1e-11, atol=1e-12)
    S, z = O.gated_final_state(k, v, lg, S0=S0, z0=z0)
    Sd, zd = O.final_state(k, v, S0=S0, z0=z0, decay=gam)
    np.testing.assert_allclose(S, Sd, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(z, zd, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("fmap", ["elu1", "performer"])
@pytest.mark.parametrize("normalize", [True, False])
def test_forms_agree(fmap, normalize):
    q, k, v, lg, W = _rand(4, fmap=fmap)
    rng = np.random.default_rng(5)
    dfeat = 8 if fmap == "performer" else 6
    S0 = rng.standard_normal((2, 3, dfeat, 6))
    z0 = rng.uniform(0.5, 1.5, (2, 3, dfeat))
    ref = O.gated_attention(q, k, v, lg, fmap, W=W, normalize=normalize, S0=S0, z0=z0)
    yr, Sr, zr = O.gated_recurrent(q, k, v, lg, fmap, W=W, normalize=normalize, S0=S0, z0=z0)
    np.testing.assert_allclose(yr, ref, rtol=1e-10, atol=1e-12)
    Sf, zf = O.gated_final_state(k, v, lg, fmap, W=W, S0=S0, z0=z0)
    np.testing.assert_allclose(Sr, Sf, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(zr, zf, rtol=1e-10, atol=1e-12)
    for C in (1, 5, 16, 64):
        yc, Sc, zc = O.gated_chunked(q, k, v, lg, fmap, W=W, normalize=normalize, chunk=C, S0=S0, z0=z0)
        np.testing.assert_allclose(yc, ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(Sc, Sf, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(zc, zf, rtol=1e-10, atol=1e-12)


def test_split_resume_and_sampled_rows():
    q, k, v, lg, _ = _rand(6, N=50)
    full = O.gated_attention(q, k, v, lg)
    S, z = O.gated_final_state(k[:, :, :20], v[:, :, :20], lg[:, :, :20])
    tail = O.gated_attention(q[:, :, 20:], k[:, :, 20:], v[:, :, 20:], lg[:, :, 20:], S0=S, z0=z)
    np.testing.assert_allclose(tail, full[:, :, 20:], rtol=1e-10, atol=1e-12)
    rows = np.array([0, 7, 31, 49])
    np.testing.assert_allclose(O.gated_attention(q, k, v, lg, rows=rows), full[:, :, rows], rtol=0, atol=1e-13)


def test_decode_step_continues_the_prefill():
    q, k, v, lg, _ = _rand(7, N=30)
    y = O.gated_attention(q, k, v, lg)
    S, z = O.gated_final_state(k[:, :, :29], v[:, :, :29], lg[:, :, :29])
    yt, _, _ = O.gated_decode_step(S, z, q[:, :, 29], k[:, :, 29], v[:, :, 29], lg[:, :, 29])
    np.testing.assert_allclose(yt, y[:, :, 29], rtol=1e-11, atol=1e-12)


def test_normalized_output_is_a_weighted_mean():
    q, k, v, lg, _ = _rand(8)
    y = O.gated_attention(q, k, v, lg)
    for i in range(v.shape[2]):
        lo = v[:, :, :i + 1].min(axis=2)
        hi = v[:, :, :i + 1].max(axis=2)
        assert np.all(y[:, :, i] >= lo - 1e-12) and np.all(y[:, :, i] <= hi + 1e-12)
