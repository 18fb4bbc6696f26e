"""Pins of the oracle's degree-2 polynomial feature map (CPU only).

"Linear Attention" (marovi.ai), "Mapas de características", polynomial
bullet: phi(x) = (1, x, x (x) x, ...), truncated at low degree. Reading:
degree 2, unit coefficients, x (x) x row-major. The pins check it against
things that do not use the oracle's code:

* the kernel identity phi(q).phi(k) = 1 + q.k + (q.k)^2;
* the map's layout on a hand-worked example;
* causal and non-causal attention against a brute force that never forms
  phi: y_i = sum_j K(q_i.k_j) v_j / sum_j K(q_i.k_j), K(s) = 1 + s + s^2;
* a carried-in state equals the same tokens prepended to the sequence;
* the recurrent (decode) form against the brute force.
"""

import numpy as np
import pytest

import oracle as O


def _kern(s):
    return 1.0 + s + s * s


def _brute(q, k, v, causal, normalize):
    """One sequence [N, d]: the kernel applied to dot products, loop over (i, j)."""
    N = q.shape[0]
    y = np.zeros_like(v, dtype=np.float64)
    for i in range(N):
        num = np.zeros(v.shape[1])
        den = 0.0
        for j in range(i + 1 if causal else N):
            w = _kern(float(np.dot(q[i], k[j])))
            num += w * v[j]
            den += w
        y[i] = num / max(den, 1e-6) if normalize else num
    return y


def test_poly2_worked_example():
    # x = (2, 3): (1 | 2, 3 | 2*2, 2*3, 3*2, 3*3)
    np.testing.assert_array_equal(O.phi_poly2(np.array([2.0, 3.0])), [1, 2, 3, 4, 6, 6, 9])
    assert O.feature_dim(64, "poly2") == 1 + 64 + 64 * 64


def test_poly2_kernel_identity():
    rng = np.random.default_rng(5)
    for d in (1, 3, 8, 32):
        q, k = rng.standard_normal((2, 50, d))
        got = np.sum(O.phi_poly2(q) * O.phi_poly2(k), axis=-1)
        s = np.sum(q * k, axis=-1)
        np.testing.assert_allclose(got, 1.0 + s + s * s, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("normalize", [True, False])
def test_poly2_attention_matches_brute_force(causal, normalize):
    rng = np.random.default_rng(11 + 2 * causal + normalize)
    B, H, N, d = 1, 2, 23, 5
    q, k, v = rng.standard_normal((3, B, H, N, d)) * 0.7
    y = O.attention(q, k, v, "poly2", causal=causal, normalize=normalize)
    for h in range(H):
        np.testing.assert_allclose(y[0, h], _brute(q[0, h], k[0, h], v[0, h], causal, normalize),
                                   rtol=1e-11, atol=1e-11)


def test_poly2_carried_state_equals_prepended_tokens():
    rng = np.random.default_rng(21)
    N0, N, d = 9, 14, 4
    q, k, v = rng.standard_normal((3, 1, 1, N0 + N, d))
    S0, z0 = O.final_state(k[..., :N0, :], v[..., :N0, :], "poly2")
    assert S0.shape[-2:] == (1 + d + d * d, d)
    y = O.attention(q[..., N0:, :], k[..., N0:, :], v[..., N0:, :], "poly2", S0=S0, z0=z0)
    full = _brute(q[0, 0], k[0, 0], v[0, 0], True, True)
    np.testing.assert_allclose(y[0, 0], full[N0:], rtol=1e-11, atol=1e-11)


def test_poly2_recurrent_and_blockwise_match_brute_force():
    rng = np.random.default_rng(31)
    N, d = 70, 3
    q, k, v = rng.standard_normal((3, 1, 1, N, d))
    ref = _brute(q[0, 0], k[0, 0], v[0, 0], True, True)
    y, S, z = O.recurrent(q, k, v, "poly2")
    np.testing.assert_allclose(y[0, 0], ref, rtol=1e-10, atol=1e-10)
    yc, Sc, zc = O.chunked(q, k, v, "poly2", chunk=16)
    np.testing.assert_allclose(yc[0, 0], ref, rtol=1e-10, atol=1e-10)
    # the final state read out by a fresh query equals the brute force over all keys
    qn = rng.standard_normal(d)
    w = _kern(k[0, 0] @ qn)
    np.testing.assert_allclose(O.phi_poly2(qn) @ S[0, 0], w @ v[0, 0], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(O.phi_poly2(qn) @ z[0, 0], w.sum(), rtol=1e-10)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-10)


def test_poly2_denominator_is_bounded_below():
    # 1 + s + s^2 >= 3/4, so the normalizer of n keys is at least 3n/4
    rng = np.random.default_rng(41)
    q, k = rng.standard_normal((2, 200, 6))
    s = q @ k.T
    K = O.phi_poly2(q) @ O.phi_poly2(k).T
    np.testing.assert_allclose(K, _kern(s), rtol=1e-12, atol=1e-12)
    assert K.min() >= 0.75 - 1e-12
