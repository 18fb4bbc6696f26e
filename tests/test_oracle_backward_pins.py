"""Pins of the oracle's gradients (CPU only).

The pages give no gradient formulas ("Linear Attention", marovi.ai,
"Entrenamiento: forma paralela", says only that training back-propagates
through the parallel form), so the oracle's `attention_backward` and
`recurrent_backward` are pinned against things they do not share code with:

* central finite differences of the forward oracle (`attention`,
  `final_state`, themselves pinned in test_oracle_pins.py), on tiny inputs,
  for every feature map, causal and non-causal, normalized or not, with and
  without decay and an initial state / final-state cotangent;
* invariants of the normalized form: outputs are weighted means of the
  values, so shifting every value by c shifts every output by c and the
  value gradients sum to the output cotangents; with the identity map the
  outputs do not change when all queries (or all keys) are scaled, so
  sum(q * dq) = sum(k * dk) = 0;
* the textbook gradient of Y = tril(Q K^T) V (identity map, numerator only);
* the two oracle forms against each other (quadratic vs recurrent).
"""

import itertools

import numpy as np
import pytest

import oracle as O

MAPS = ("elu1", "identity", "performer")


def _inputs(fmap, seed, B=1, H=2, N=6, d=3, m=4, with_state=False):
    rng = np.random.default_rng(seed)
    if fmap == "identity":  # positive rows keep the denominators away from zero
        q = rng.uniform(0.3, 1.2, (B, H, N, d))
        k = rng.uniform(0.3, 1.2, (B, H, N, d))
    else:
        q = rng.standard_normal((B, H, N, d))
        k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    dy = rng.standard_normal((B, H, N, d))
    W = rng.standard_normal((m, d)) if fmap == "performer" else None
    dfeat = m if fmap == "performer" else d
    st = {}
    if with_state:
        st = dict(S0=rng.standard_normal((B, H, dfeat, d)), z0=rng.uniform(0.2, 1.0, (B, H, dfeat)),
                  dS_N=rng.standard_normal((B, H, dfeat, d)), dz_N=rng.standard_normal((B, H, dfeat)))
    return q, k, v, dy, W, st


def _loss(q, k, v, dy, W, fmap, causal, normalize, decay, st):
    y = O.attention(q, k, v, fmap, W=W, causal=causal, normalize=normalize, S0=st.get("S0"), z0=st.get("z0"),
                    decay=decay)
    L = float(np.sum(dy * y))
    if "dS_N" in st:
        S, z = O.final_state(k, v, fmap, W=W, S0=st["S0"], z0=st["z0"], decay=decay)
        L += float(np.sum(st["dS_N"] * S) + np.sum(st["dz_N"] * z))
    return L


def _fd(fn, x, h=1e-5):
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        x0 = x[idx]
        x[idx] = x0 + h
        lp = fn()
        x[idx] = x0 - h
        lm = fn()
        x[idx] = x0
        g[idx] = (lp - lm) / (2 * h)
    return g


def _close(a, b, rel=1e-7):
    scale = max(1.0, float(np.max(np.abs(b))))
    np.testing.assert_allclose(a, b, rtol=0, atol=rel * scale)


CASES = [(f, c, n, dc, s) for f, c, n, dc, s in itertools.product(MAPS, (True, False), (True, False),
                                                                 (None, "heads"), (False, True))
         if not (dc and not c)]


@pytest.mark.parametrize("fmap,causal,normalize,decay,with_state", CASES)
def test_backward_matches_finite_differences(fmap, causal, normalize, decay, with_state):
    seed = 100 + CASES.index((fmap, causal, normalize, decay, with_state))
    q, k, v, dy, W, st = _inputs(fmap, seed, with_state=with_state)
    gam = np.array([0.6, 0.85]) if decay else None
    dq, dk, dv, dS0, dz0 = O.attention_backward(q, k, v, dy, fmap, W=W, causal=causal, normalize=normalize,
                                                S0=st.get("S0"), z0=st.get("z0"), dS_N=st.get("dS_N"),
                                                dz_N=st.get("dz_N"), decay=gam)
    L = lambda: _loss(q, k, v, dy, W, fmap, causal, normalize, gam, st)  # noqa: E731
    _close(dq, _fd(L, q))
    _close(dk, _fd(L, k))
    _close(dv, _fd(L, v))
    if with_state:
        _close(dS0, _fd(L, st["S0"]))
        _close(dz0, _fd(L, st["z0"]))
    else:
        assert not np.any(dS0 != dS0)  # defined (finite) even without a state


@pytest.mark.parametrize("fmap", MAPS)
@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("decay", [None, "heads"])
@pytest.mark.parametrize("with_state", [False, True])
def test_recurrent_backward_matches_quadratic(fmap, normalize, decay, with_state):
    q, k, v, dy, W, st = _inputs(fmap, 77, N=23, d=5, m=6, with_state=with_state)
    gam = np.array([0.7, 0.95]) if decay else None
    kw = dict(W=W, normalize=normalize, S0=st.get("S0"), z0=st.get("z0"), dS_N=st.get("dS_N"),
              dz_N=st.get("dz_N"), decay=gam)
    a = O.attention_backward(q, k, v, dy, fmap, causal=True, **kw)
    b = O.recurrent_backward(q, k, v, dy, fmap, **kw)
    for x, y in zip(a, b):
        _close(x, y, rel=1e-11)


@pytest.mark.parametrize("fmap", MAPS)
@pytest.mark.parametrize("causal,decay", [(True, None), (True, "heads"), (False, None)])
def test_value_gradients_sum_to_output_cotangents(fmap, causal, decay):
    q, k, v, dy, W, _ = _inputs(fmap, 5, N=17, d=4, m=8)
    gam = np.array([0.5, 0.9]) if decay else None
    _, _, dv, _, _ = O.attention_backward(q, k, v, dy, fmap, W=W, causal=causal, normalize=True, decay=gam)
    _close(dv.sum(axis=2), dy.sum(axis=2), rel=1e-12)


@pytest.mark.parametrize("causal,decay", [(True, None), (True, "heads"), (False, None)])
def test_identity_map_scale_invariance(causal, decay):
    q, k, v, dy, _, _ = _inputs("identity", 9, N=19, d=4)
    gam = np.array([0.8, 0.6]) if decay else None
    dq, dk, _, _, _ = O.attention_backward(q, k, v, dy, "identity", causal=causal, normalize=True, decay=gam)
    for g in range(2):
        assert abs(np.sum(q[0, g] * dq[0, g])) < 1e-12 * max(1.0, np.abs(dq).max())
        assert abs(np.sum(k[0, g] * dk[0, g])) < 1e-12 * max(1.0, np.abs(dk).max())


def test_identity_numerator_textbook_gradient():
    """Y = tril(Q K^T) V: dQ = tril(dY V^T) K, dK = tril(dY V^T)^T Q, dV = tril(Q K^T)^T dY."""
    rng = np.random.default_rng(3)
    N, d = 11, 5
    q, k, v, dy = (rng.standard_normal((N, d)) for _ in range(4))
    dq, dk, dv, _, _ = O.attention_backward(q, k, v, dy, "identity", causal=True, normalize=False)
    P = np.tril(dy @ v.T)
    np.testing.assert_allclose(dq, P @ k, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk, P.T @ q, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv, np.tril(q @ k.T).T @ dy, rtol=1e-12, atol=1e-12)


def test_feature_map_vjp_finite_differences():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 5))
    x[0, 0] = 1e-3  # near the elu+1 branch point, both sides
    x[0, 1] = -1e-3
    x[0, 2] = 0.0   # the branch point itself: phi'(0) = 1 from both sides
    W = rng.standard_normal((7, 5))
    for fmap in MAPS:
        dphi = rng.standard_normal((3, 7 if fmap == "performer" else 5))
        g = O.feature_map_vjp(x, dphi, fmap, W=W)
        L = lambda: float(np.sum(dphi * O.feature_map(x, fmap, W=W)))  # noqa: E731
        _close(g, _fd(L, x, h=1e-6), rel=1e-6)  # at 0 the difference quotient is off by h/4
