"""CPU oracle for kernelized linear attention (NumPy, float64).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
CPU-baseline leg may import or run this module. The product (the HIP library
and its Python binding) never does; the two share no code.

Sources (the three pages on linear attention):
  [LA]  "Linear Attention" article (marovi.ai), sections "Reformulación con
        núcleos", "Mapas de características", "Forma recurrente e inferencia
        autorregresiva", "Entrenamiento: forma paralela".
  [LT]  "Linear Transformer (Transformers are RNNs)" glossary entry
        (visibilidadia.com), sections "La función ELU + 1", "Formulación
        matemática de la atención lineal", "La formulación recurrente paso a
        paso", "Comprobar la equivalencia entre cálculo recurrente y cálculo
        causal vectorizado".
  [UL]  "Linear Attention" glossary entry (ultralytics.com), "Ejemplo de
        código" (the output without a denominator).

Every input is upcast to float64 exactly; everything is computed in float64.

Readings taken where the pages are silent or disagree (each one is also
listed with its reasons in the design notes of the repository):
  * causal sums include the current token (j <= i): [LA] recurrent form and
    [LT] step-by-step form update the state before reading it out;
  * the denominator is clamped, y = num / max(den, EPS) with EPS = 1e-6, as
    the code examples of [LT] do; with positive feature maps the clamp only
    matters when den < 1e-6;
  * ``normalize=False`` returns the numerator alone ([LA] notes some
    implementations drop the denominator; [UL]'s example does);
  * elu+1 uses alpha = 1 and takes the exponential branch at x = 0 ([LT]
    "La función ELU + 1");
  * the polynomial map is truncated at degree 2 with unit coefficients,
    phi(x) = (1, x, x (x) x) with x (x) x row-major, so the kernel is
    1 + q.k + (q.k)^2 (always >= 3/4);
  * random features: phi(x) = exp(W x~ - |x~|^2/2) / sqrt(m) with
    x~ = d^(-1/4) x, so that E[phi(q).phi(k)] = exp(q.k / sqrt(d)), the
    kernel that [LA] "Reformulación con núcleos" writes for softmax;
  * an optional initial state (S0, z0) stands for tokens before the first
    one given: it adds phi(q_i).S0 to the numerator and phi(q_i).z0 to the
    denominator of every output;
  * gates ([LA] "Variantes y extensiones", GLA item): a data-dependent
    per-token, per-channel gate alpha_t on the feature dimension,
    S_t = diag(alpha_t) S_{t-1} + phi(k_t) v_t^T, z gated alike (given as
    log-gates); a constant gate equal over channels is the decay below;
  * decay ([LA] "Variantes y extensiones", RetNet item): the state recurs as
    S_t = gamma S_{t-1} + phi(k_t) v_t^T and the normalizer the same way,
    z_t = gamma z_{t-1} + phi(k_t); unrolled, token j enters output i with
    weight gamma^(i-j) and an initial state with weight gamma^(i+1). It is
    defined for the causal and recurrent forms only; gamma may differ per
    head (one value per leading index, or per head of a [B, H, ...] input).

Parity pins: every function here is checked by tests that do not reuse its
code (hand-derived worked examples, closed forms, library routines,
invariants); see tests/test_oracle_pins.py.
"""

from __future__ import annotations

import numpy as np

EPS = 1e-6

FMAPS = ("elu1", "performer", "identity", "poly2")


# ---------------------------------------------------------------------------
# Feature maps  ([LA] "Mapas de características"; [LT] "La función ELU + 1")
# ---------------------------------------------------------------------------

def phi_elu1(x):
    """elu(x) + 1 elementwise: x + 1 for x > 0, exp(x) for x <= 0 ([LT] "La función ELU + 1")."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_performer(x, W):
    """Positive random features ([LA] "Mapas de características", Performer bullet).

    phi(x) = exp(W x~ - |x~|^2 / 2) / sqrt(m), x~ = d^(-1/4) x, W of shape (m, d).
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    d = x.shape[-1]
    m = W.shape[0]
    xt = x * d ** -0.25
    u = xt @ W.T
    sq = np.sum(xt * xt, axis=-1, keepdims=True)
    return np.exp(u - 0.5 * sq) / np.sqrt(m)


def phi_identity(x):
    """phi(x) = x ([LA] "Mapas de características", identity bullet); used as a test device."""
    return np.asarray(x, dtype=np.float64)


def phi_poly2(x):
    """Degree-2 truncation of the polynomial map (1, x, x (x) x, ...)
    ([LA] "Mapas de características", polynomial bullet).

    Reading: no coefficients on the terms; the d x d block of x (x) x is laid
    out row-major, entry 1 + d + a d + b = x_a x_b. Then
    phi(q).phi(k) = 1 + q.k + (q.k)^2. d' = 1 + d + d^2.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    outer = x[..., :, None] * x[..., None, :]
    one = np.ones(x.shape[:-1] + (1,))
    return np.concatenate([one, x, outer.reshape(x.shape[:-1] + (d * d,))], axis=-1)


def feature_map(x, fmap="elu1", W=None):
    if fmap == "elu1":
        return phi_elu1(x)
    if fmap == "performer":
        if W is None:
            raise ValueError("performer map needs W")
        return phi_performer(x, W)
    if fmap == "identity":
        return phi_identity(x)
    if fmap == "poly2":
        return phi_poly2(x)
    raise ValueError(f"unknown feature map {fmap!r}")


def feature_dim(d, fmap="elu1", W=None):
    if fmap == "poly2":
        return 1 + d + d * d
    return int(np.asarray(W).shape[0]) if fmap == "performer" else d


def _finish(num, den, normalize):
    if not normalize:
        return num
    return num / np.maximum(den, EPS)[..., None]


def _bh(x):
    """View [B, H, N, d] (or [N, d]) input as float64 [G, N, d]."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 2:
        return x[None]
    return x.reshape(-1, x.shape[-2], x.shape[-1])


def _gammas(decay, shape, G):
    """Per-(batch, head) decay factors as float64 [G], or None for no decay.

    ``decay`` is a number, or an array broadcastable to the leading dims of
    ``shape`` (e.g. one value per head of a [B, H, N, d] input)."""
    if decay is None:
        return None
    lead = tuple(shape[:-2]) if len(shape) > 2 else (1,)
    g = np.broadcast_to(np.asarray(decay, dtype=np.float64), lead).reshape(-1)
    if g.size != G:
        raise ValueError("decay does not match the leading dimensions")
    return g


def _state(S0, z0, G, dfeat, dv):
    S = np.zeros((G, dfeat, dv)) if S0 is None else np.asarray(S0, np.float64).reshape(G, dfeat, dv).copy()
    z = np.zeros((G, dfeat)) if z0 is None else np.asarray(z0, np.float64).reshape(G, dfeat).copy()
    return S, z


# ---------------------------------------------------------------------------
# The definition  ([LA] "Reformulación con núcleos", first form of y_i)
# ---------------------------------------------------------------------------

def attention(q, k, v, fmap="elu1", W=None, causal=True, normalize=True,
              S0=None, z0=None, rows=None, decay=None):
    """y_i = sum_j (phi(q_i).phi(k_j)) v_j / sum_j phi(q_i).phi(k_j).

    The sums run over j <= i when ``causal`` (inclusive), else over all j.
    With ``decay`` (causal only) term j of output i is weighted gamma^(i-j)
    and the initial state gamma^(i+1).
    The N x N similarity matrix is formed explicitly (brute force). ``rows``
    restricts the computation to a subset of query positions, so long
    sequences can be checked at sampled outputs.
    Returns float64 of shape [..., len(rows) or N, d_v].
    """
    shape = np.asarray(q).shape
    Q, K, V = _bh(q), _bh(k), _bh(v)
    G, N, _ = Q.shape
    dv = V.shape[-1]
    idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    Kf = feature_map(K, fmap, W)
    Qf = feature_map(Q[:, idx], fmap, W)
    dfeat = Kf.shape[-1]
    S, z = _state(S0, z0, G, dfeat, dv)
    gam = _gammas(decay, shape, G)
    if gam is not None and not causal:
        raise ValueError("decay is defined for the causal form only")
    out = np.empty((G, idx.size, dv))
    lag = idx[:, None] - np.arange(N)[None, :]        # i - j
    for g in range(G):
        A = Qf[g] @ Kf[g].T                           # [R, N] similarities
        s0 = np.ones((idx.size, 1))
        if causal:
            A = np.where(lag >= 0, A, 0.0)
            if gam is not None:
                A = A * np.where(lag >= 0, gam[g] ** np.maximum(lag, 0), 0.0)
                s0 = (gam[g] ** (idx + 1.0))[:, None]
        num = A @ V[g] + s0 * (Qf[g] @ S[g])
        den = A.sum(axis=1) + s0[:, 0] * (Qf[g] @ z[g])
        out[g] = _finish(num, den, normalize)
    return out.reshape(shape[:-2] + (idx.size, dv))


def final_state(k, v, fmap="elu1", W=None, S0=None, z0=None, decay=None):
    """S = S0 + sum_j phi(k_j) v_j^T, z = z0 + sum_j phi(k_j) ([LA] "Reformulación con núcleos").

    With decay: S = gamma^N S0 + sum_j gamma^(N-1-j) phi(k_j) v_j^T (and z alike)."""
    shape = np.asarray(k).shape
    K, V = _bh(k), _bh(v)
    G, N = K.shape[0], K.shape[1]
    Kf = feature_map(K, fmap, W)
    S, z = _state(S0, z0, G, Kf.shape[-1], V.shape[-1])
    gam = _gammas(decay, shape, G)
    if gam is not None:
        wgt = gam[:, None] ** (N - 1.0 - np.arange(N))[None, :]     # [G, N]
        S = gam[:, None, None] ** N * S + np.einsum("gn,gnc,gne->gce", wgt, Kf, V)
        z = gam[:, None] ** N * z + np.einsum("gn,gnc->gc", wgt, Kf)
    else:
        S = S + np.einsum("gnc,gne->gce", Kf, V)
        z = z + Kf.sum(axis=1)
    lead = shape[:-2]
    return S.reshape(lead + S.shape[1:]), z.reshape(lead + z.shape[1:])


# ---------------------------------------------------------------------------
# Non-causal form through the two sums ([LA] "Reformulación con núcleos",
# second form; [LT] "Formulación matemática": Q'(K'^T V) / Q'(K'^T 1))
# ---------------------------------------------------------------------------

def attention_via_state(q, k, v, fmap="elu1", W=None, normalize=True, S0=None, z0=None):
    shape = np.asarray(q).shape
    Q = _bh(q)
    S, z = final_state(k, v, fmap, W, S0, z0)
    G = Q.shape[0]
    S = np.asarray(S).reshape(G, S.shape[-2], S.shape[-1])
    z = np.asarray(z).reshape(G, z.shape[-1])
    Qf = feature_map(Q, fmap, W)
    num = np.einsum("gnc,gce->gne", Qf, S)
    den = np.einsum("gnc,gc->gn", Qf, z)
    return _finish(num, den, normalize).reshape(shape[:-1] + (S.shape[-1],))


# ---------------------------------------------------------------------------
# Recurrent form ([LA] "Forma recurrente e inferencia autorregresiva";
# [LT] "La formulación recurrente paso a paso")
# ---------------------------------------------------------------------------

def decode_step(S, z, q, k, v, fmap="elu1", W=None, normalize=True, decay=None):
    """One token per head: S += phi(k) v^T, z += phi(k), then y = phi(q)^T S / phi(q).z.

    With decay: S = gamma S + phi(k) v^T, z = gamma z + phi(k) ([LA]
    "Variantes y extensiones"); gamma a number or an array over the leading
    dims of q. S: [..., d', d], z: [..., d'], q/k/v: [..., d]. Returns
    (y, S_new, z_new); the inputs are not modified.
    """
    S = np.asarray(S, np.float64)
    z = np.asarray(z, np.float64)
    qf = feature_map(np.asarray(q, np.float64), fmap, W)
    kf = feature_map(np.asarray(k, np.float64), fmap, W)
    v = np.asarray(v, np.float64)
    if decay is not None:
        gam = np.broadcast_to(np.asarray(decay, np.float64), z.shape[:-1])
        S = gam[..., None, None] * S
        z = gam[..., None] * z
    S_new = S + kf[..., :, None] * v[..., None, :]
    z_new = z + kf
    num = np.einsum("...c,...ce->...e", qf, S_new)
    den = np.einsum("...c,...c->...", qf, z_new)
    return _finish(num, den, normalize), S_new, z_new


def recurrent(q, k, v, fmap="elu1", W=None, normalize=True, S0=None, z0=None, decay=None):
    """Token-by-token loop over the sequence (every head at once).

    Returns (y, S_N, z_N).
    """
    shape = np.asarray(q).shape
    Q, K, V = _bh(q), _bh(k), _bh(v)
    G, N, _ = Q.shape
    dv = V.shape[-1]
    dfeat = feature_dim(Q.shape[-1], fmap, W)
    S, z = _state(S0, z0, G, dfeat, dv)
    gam = _gammas(decay, shape, G)
    y = np.empty((G, N, dv))
    for t in range(N):
        y[:, t], S, z = decode_step(S, z, Q[:, t], K[:, t], V[:, t], fmap, W, normalize, gam)
    lead = shape[:-2]
    return (y.reshape(shape[:-1] + (dv,)), S.reshape(lead + S.shape[1:]),
            z.reshape(lead + z.shape[1:]))


# ---------------------------------------------------------------------------
# Cumulative-sum form ([LT] "Comprobar la equivalencia ..."): per-token outer
# products, prefix sums along the sequence, contraction with phi(q). Tiny
# inputs only (materializes N x d' x d per head).
# ---------------------------------------------------------------------------

def cumsum_form(q, k, v, fmap="elu1", W=None, normalize=True):
    shape = np.asarray(q).shape
    Q, K, V = _bh(q), _bh(k), _bh(v)
    Qf = feature_map(Q, fmap, W)
    Kf = feature_map(K, fmap, W)
    kv = Kf[..., :, None] * V[..., None, :]          # [G, N, d', d]
    S = np.cumsum(kv, axis=1)
    z = np.cumsum(Kf, axis=1)
    num = np.einsum("gnc,gnce->gne", Qf, S)
    den = np.einsum("gnc,gnc->gn", Qf, z)
    return _finish(num, den, normalize).reshape(shape[:-1] + (V.shape[-1],))


# ---------------------------------------------------------------------------
# Blockwise form ([LA] "Entrenamiento: forma paralela"): the sequence is cut
# into blocks of C tokens; inside a block the masked quadratic similarity
# form, across blocks the running sums S, z.
# ---------------------------------------------------------------------------

def chunked(q, k, v, fmap="elu1", W=None, causal=True, normalize=True, chunk=64,
            S0=None, z0=None, decay=None):
    """Returns (y, S_N, z_N). For ``causal=False`` the full sums are formed first.

    With decay (causal only): inside a block of L tokens the similarity of
    rows i, j (block positions r_i, r_j) is weighted gamma^(r_i-r_j), the
    carried state enters row i with weight gamma^(r_i+1), and the state moves
    on as S <- gamma^L S + sum_j gamma^(L-1-r_j) phi(k_j) v_j^T.
    """
    if decay is not None and not causal:
        raise ValueError("decay is defined for the causal form only")
    if not causal:
        y = attention_via_state(q, k, v, fmap, W, normalize, S0, z0)
        S, z = final_state(k, v, fmap, W, S0, z0)
        return y, S, z
    shape = np.asarray(q).shape
    Q, K, V = _bh(q), _bh(k), _bh(v)
    G, N, _ = Q.shape
    dv = V.shape[-1]
    Qf = feature_map(Q, fmap, W)
    Kf = feature_map(K, fmap, W)
    S, z = _state(S0, z0, G, Qf.shape[-1], dv)
    gam = _gammas(decay, shape, G)
    y = np.empty((G, N, dv))
    for s in range(0, N, chunk):
        e = min(N, s + chunk)
        L = e - s
        qc, kc, vc = Qf[:, s:e], Kf[:, s:e], V[:, s:e]
        A = np.einsum("gic,gjc->gij", qc, kc)
        A = A * np.tril(np.ones((L, L)))[None]
        if gam is None:
            sin = np.ones((G, L))                                   # weight of the carried state
            kw = np.ones((G, L))                                    # weight of key j in the update
            carry = np.ones(G)
        else:
            r = np.arange(L, dtype=np.float64)
            A = A * gam[:, None, None] ** np.maximum(r[:, None] - r[None, :], 0.0)[None]
            sin = gam[:, None] ** (r[None, :] + 1.0)
            kw = gam[:, None] ** (L - 1.0 - r[None, :])
            carry = gam ** L
        num = np.einsum("gij,gje->gie", A, vc) + sin[:, :, None] * np.einsum("gic,gce->gie", qc, S)
        den = A.sum(axis=2) + sin * np.einsum("gic,gc->gi", qc, z)
        y[:, s:e] = _finish(num, den, normalize)
        S = carry[:, None, None] * S + np.einsum("gj,gjc,gje->gce", kw, kc, vc)
        z = carry[:, None] * z + np.einsum("gj,gjc->gc", kw, kc)
    lead = shape[:-2]
    return (y.reshape(shape[:-1] + (dv,)), S.reshape(lead + S.shape[1:]),
            z.reshape(lead + z.shape[1:]))


# ---------------------------------------------------------------------------
# Gradients. [LA] "Entrenamiento: forma paralela" says the parallel form
# exists so that training (back-propagation) is fast; the pages print no
# gradient formulas. The functions below are the vector-Jacobian products of
# the definitions above, derived by hand: with the outputs' cotangents dY
# (and optionally the final state's, dS_N and dz_N) they return the
# gradients of L = <dY, Y> + <dS_N, S_N> + <dz_N, z_N> with respect to q, k,
# v (and the initial state). They are pinned by central finite differences
# of `attention` / `final_state` in tests/test_oracle_backward_pins.py.
#
# Derivative of the clamp: d max(den, EPS) / d den = 1 when den >= EPS,
# else 0 (at the configurations tested den is far above EPS).
# ---------------------------------------------------------------------------

def feature_map_vjp(x, dphi, fmap="elu1", W=None):
    """Gradient with respect to x of <dphi, phi(x)> (row-wise maps).

    elu+1: phi'(x) = 1 for x > 0, exp(x) for x <= 0. identity: 1.
    random features: phi_c = exp(u_c - |x~|^2/2)/sqrt(m), u = W x~, x~ = d^(-1/4) x,
    so d phi_c / d x = d^(-1/4) phi_c (W_c - x~).
    """
    x = np.asarray(x, dtype=np.float64)
    dphi = np.asarray(dphi, dtype=np.float64)
    if fmap == "elu1":
        return dphi * np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))
    if fmap == "identity":
        return dphi.copy()
    if fmap == "performer":
        W = np.asarray(W, dtype=np.float64)
        d = x.shape[-1]
        s = d ** -0.25
        f = phi_performer(x, W)
        t = dphi * f                                   # [..., m]
        return s * (t @ W - (x * s) * t.sum(axis=-1, keepdims=True))
    raise ValueError(f"unknown feature map {fmap!r}")


def _cot_state(dS, dz, G, dfeat, dv):
    dS = np.zeros((G, dfeat, dv)) if dS is None else np.asarray(dS, np.float64).reshape(G, dfeat, dv)
    dz = np.zeros((G, dfeat)) if dz is None else np.asarray(dz, np.float64).reshape(G, dfeat)
    return dS, dz


def attention_backward(q, k, v, dy, fmap="elu1", W=None, causal=True, normalize=True,
                       S0=None, z0=None, dS_N=None, dz_N=None, decay=None):
    """Vector-Jacobian product of `attention` (and of `final_state` for the
    seeds dS_N, dz_N), with the N x N similarity matrix formed explicitly.

    Per head, with Qf = phi(Q), Kf = phi(K), the weights Gm (the causal mask,
    times gamma^(i-j) with decay), s0_i the weight of the initial state
    (gamma^(i+1) with decay, else 1) and w_j the weight of key j in the final
    state (gamma^(N-1-j), else 1):
      A = (Qf Kf^T) * Gm,  num = A V + s0 (Qf S0),  den = A 1 + s0 (Qf z0)
      dnum = dY / max(den, EPS),  dden = -<dY, num> / max(den, EPS)^2  (normalized)
      dnum = dY,                  dden = 0                             (not normalized)
      dM   = (dnum V^T + dden 1^T) * Gm
      dQf  = dM Kf + s0 (dnum S0^T + dden z0^T)
      dKf  = dM^T Qf + w (V dS_N^T + 1 dz_N^T)
      dV   = A^T dnum + w (Kf dS_N)
      dS0  = Qf^T (s0 dnum) + gamma^N dS_N,   dz0 = Qf^T (s0 dden) + gamma^N dz_N
    and dq, dk from dQf, dKf through the feature map.
    Returns (dq, dk, dv, dS0, dz0) in float64, shaped like the inputs
    (dS0 [..., d', d], dz0 [..., d']).
    """
    shape = np.asarray(q).shape
    Q, K, V, dY = _bh(q), _bh(k), _bh(v), _bh(dy)
    G, N, _ = Q.shape
    dv = V.shape[-1]
    Qf = feature_map(Q, fmap, W)
    Kf = feature_map(K, fmap, W)
    dfeat = Qf.shape[-1]
    S, z = _state(S0, z0, G, dfeat, dv)
    dSN, dzN = _cot_state(dS_N, dz_N, G, dfeat, dv)
    gam = _gammas(decay, shape, G)
    if gam is not None and not causal:
        raise ValueError("decay is defined for the causal form only")
    lag = np.arange(N)[:, None] - np.arange(N)[None, :]
    dQf = np.empty_like(Qf)
    dKf = np.empty_like(Kf)
    dV = np.empty_like(V)
    dS0 = np.empty_like(S)
    dz0 = np.empty_like(z)
    for g in range(G):
        Gm = np.ones((N, N))
        s0 = np.ones(N)
        w = np.ones(N)
        carry = 1.0
        if causal:
            Gm = np.where(lag >= 0, 1.0, 0.0)
            if gam is not None:
                Gm = Gm * gam[g] ** np.maximum(lag, 0)
                s0 = gam[g] ** (np.arange(N) + 1.0)
                w = gam[g] ** (N - 1.0 - np.arange(N))
                carry = gam[g] ** N
        A = (Qf[g] @ Kf[g].T) * Gm
        num = A @ V[g] + s0[:, None] * (Qf[g] @ S[g])
        den = A.sum(axis=1) + s0 * (Qf[g] @ z[g])
        if normalize:
            Dn = np.maximum(den, EPS)
            dnum = dY[g] / Dn[:, None]
            dden = np.where(den >= EPS, -np.sum(dY[g] * num, axis=1) / Dn ** 2, 0.0)
        else:
            dnum = dY[g]
            dden = np.zeros(N)
        dM = (dnum @ V[g].T + dden[:, None]) * Gm
        dQf[g] = dM @ Kf[g] + s0[:, None] * (dnum @ S[g].T + dden[:, None] * z[g][None, :])
        dKf[g] = dM.T @ Qf[g] + w[:, None] * (V[g] @ dSN[g].T + dzN[g][None, :])
        dV[g] = A.T @ dnum + w[:, None] * (Kf[g] @ dSN[g])
        dS0[g] = Qf[g].T @ (s0[:, None] * dnum) + carry * dSN[g]
        dz0[g] = Qf[g].T @ (s0 * dden) + carry * dzN[g]
    dq = feature_map_vjp(Q, dQf, fmap, W)
    dk = feature_map_vjp(K, dKf, fmap, W)
    lead = shape[:-2]
    return (dq.reshape(shape), dk.reshape(shape), dV.reshape(lead + (N, dv)),
            dS0.reshape(lead + (dfeat, dv)), dz0.reshape(lead + (dfeat,)))


def recurrent_backward(q, k, v, dy, fmap="elu1", W=None, normalize=True,
                       S0=None, z0=None, dS_N=None, dz_N=None, decay=None):
    """Back-propagation through the recurrent form (causal), O(N d' d) per head.

    Forward sweep: S_t = gamma S_{t-1} + phi(k_t) v_t^T (z alike), the output
    cotangents dnum_t, dden_t as in `attention_backward`, and
    d phi(q_t) = S_t dnum_t + z_t dden_t. Reverse sweep with the adjoint
    states R = dL/dS_t, r = dL/dz_t, starting from (dS_N, dz_N):
      R += phi(q_t) dnum_t^T, r += phi(q_t) dden_t,
      d phi(k_t) = R v_t + r,  dv_t = R^T phi(k_t),
      then R, r <- gamma R, gamma r (on to S_{t-1}); finally dS0 = R, dz0 = r.
    Same return values as `attention_backward`.
    """
    shape = np.asarray(q).shape
    Q, K, V, dY = _bh(q), _bh(k), _bh(v), _bh(dy)
    G, N, _ = Q.shape
    dv = V.shape[-1]
    Qf = feature_map(Q, fmap, W)
    Kf = feature_map(K, fmap, W)
    dfeat = Qf.shape[-1]
    S, z = _state(S0, z0, G, dfeat, dv)
    R, r = _cot_state(dS_N, dz_N, G, dfeat, dv)
    R, r = R.copy(), r.copy()
    gam = _gammas(decay, shape, G)
    gm = np.ones(G) if gam is None else gam
    dQf = np.empty_like(Qf)
    dnum = np.empty_like(dY)
    dden = np.empty((G, N))
    for t in range(N):
        S = gm[:, None, None] * S + Kf[:, t, :, None] * V[:, t, None, :]
        z = gm[:, None] * z + Kf[:, t]
        num = np.einsum("gc,gce->ge", Qf[:, t], S)
        den = np.einsum("gc,gc->g", Qf[:, t], z)
        if normalize:
            Dn = np.maximum(den, EPS)
            dnum[:, t] = dY[:, t] / Dn[:, None]
            dden[:, t] = np.where(den >= EPS, -np.sum(dY[:, t] * num, axis=1) / Dn ** 2, 0.0)
        else:
            dnum[:, t] = dY[:, t]
            dden[:, t] = 0.0
        dQf[:, t] = np.einsum("gce,ge->gc", S, dnum[:, t]) + z * dden[:, t][:, None]
    dKf = np.empty_like(Kf)
    dV = np.empty_like(V)
    for t in range(N - 1, -1, -1):
        R = R + Qf[:, t, :, None] * dnum[:, t, None, :]
        r = r + Qf[:, t] * dden[:, t][:, None]
        dKf[:, t] = np.einsum("gce,ge->gc", R, V[:, t]) + r
        dV[:, t] = np.einsum("gce,gc->ge", R, Kf[:, t])
        R = gm[:, None, None] * R
        r = gm[:, None] * r
    dq = feature_map_vjp(Q, dQf, fmap, W)
    dk = feature_map_vjp(K, dKf, fmap, W)
    lead = shape[:-2]
    return (dq.reshape(shape), dk.reshape(shape), dV.reshape(lead + (N, dv)),
            R.reshape(lead + (dfeat, dv)), r.reshape(lead + (dfeat,)))


# ---------------------------------------------------------------------------
# Gated linear attention ([LA] "Variantes y extensiones", GLA item: the
# scalar decay replaced by a gate that depends on the data). Reading: a
# per-token, per-channel gate alpha_t in (0, 1]^d' on the feature dimension,
# S_t = diag(alpha_t) S_{t-1} + phi(k_t) v_t^T, the normalizer gated alike,
# z_t = alpha_t * z_{t-1} + phi(k_t), y_t = phi(q_t)^T S_t / phi(q_t).z_t.
# Gates are given as log-gates lg = log(alpha), an array [..., N, d'].
# Unrolled, token j enters output i through channel f with weight
# exp(L_if - L_jf), L_t = sum_{s<=t} lg_s; an initial state enters with
# exp(L_if). A constant gate equal over channels is the decay above.
# ---------------------------------------------------------------------------

def _lg(log_gates, G, N, dfeat):
    lg = np.asarray(log_gates, dtype=np.float64)
    return lg.reshape(G, N, dfeat)


def gated_attention(q, k, v, log_gates, fmap="elu1", W=None, normalize=True, S0=None, z0=None, rows=None):
    """Definition, causal: y_i = sum_{j<=i} sum_f phi(q_i)_f phi(k_j)_f exp(L_if - L_jf) v_j / (same without v_j).

    Each output row forms its weights over every earlier key explicitly
    (brute force); ``rows`` restricts the computation to sampled outputs.
    """
    shape = np.asarray(q).shape
    Q, K, V = _bh(q), _bh(k), _bh(v)
    G, N, _ = Q.shape
    dv = V.shape[-1]
    Qf = feature_map(Q, fmap, W)
    Kf = feature_map(K, fmap, W)
    dfeat = Qf.shape[-1]
    L = np.cumsum(_lg(log_gates, G, N, dfeat), axis=1)       # [G, N, d']
    S, z = _state(S0, z0, G, dfeat, dv)
    idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((G, idx.size, dv))
    for g in range(G):
        for n, i in enumerate(idx):
            wgt = np.exp(L[g, i][None, :] - L[g, :i + 1])       # [i+1, d'] per key and channel
            a = (Qf[g, i][None, :] * Kf[g, :i + 1] * wgt).sum(axis=1)
            s0 = np.exp(L[g, i])                                 # initial state, per channel
            num = a @ V[g, :i + 1] + (Qf[g, i] * s0) @ S[g]
            den = a.sum() + (Qf[g, i] * s0) @ z[g]
            out[g, n] = num / max(den, EPS) if normalize else num
    return out.reshape(shape[:-2] + (idx.size, dv))


def gated_final_state(k, v, log_gates, fmap="elu1", W=None, S0=None, z0=None):
    """S_N = diag(exp(L_N-1)) S0 + sum_j diag(exp(L_N-1 - L_j)) phi(k_j) v_j^T, z alike."""
    shape = np.asarray(k).shape
    K, V = _bh(k), _bh(v)
    G, N = K.shape[0], K.shape[1]
    Kf = feature_map(K, fmap, W)
    dfeat = Kf.shape[-1]
    L = np.cumsum(_lg(log_gates, G, N, dfeat), axis=1)
    S, z = _state(S0, z0, G, dfeat, V.shape[-1])
    if N > 0:
        last = L[:, -1]                                          # [G, d']
        wgt = np.exp(last[:, None, :] - L)                       # [G, N, d']
        S = np.exp(last)[:, :, None] * S + np.einsum("gnc,gnc,gne->gce", wgt, Kf, V)
        z = np.exp(last) * z + np.einsum("gnc,gnc->gc", wgt, Kf)
    lead = shape[:-2]
    return S.reshape(lead + S.shape[1:]), z.reshape(lead + z.shape[1:])


def gated_decode_step(S, z, q, k, v, log_gate, fmap="elu1", W=None, normalize=True):
    """One token per head: S = diag(alpha) S + phi(k) v^T, z = alpha z + phi(k), then the readout.

    log_gate: [..., d'] (log alpha of this token). Returns (y, S_new, z_new).
    """
    S = np.asarray(S, np.float64)
    z = np.asarray(z, np.float64)
    a = np.exp(np.asarray(log_gate, np.float64))
    qf = feature_map(np.asarray(q, np.float64), fmap, W)
    kf = feature_map(np.asarray(k, np.float64), fmap, W)
    v = np.asarray(v, np.float64)
    S_new = a[..., :, None] * S + kf[..., :, None] * v[..., None, :]
    z_new = a * z + kf
    num = np.einsum("...c,...ce->...e", qf, S_new)
    den = np.einsum("...c,...c->...", qf, z_new)
    return _finish(num, den, normalize), S_new, z_new


def gated_recurrent(q, k, v, log_gates, fmap="elu1", W=None, normalize=True, S0=None, z0=None):
    """Token-by-token loop of gated_decode_step. Returns (y, S_N, z_N)."""
    shape = np.asarray(q).shape
    Q, K, V = _bh(q), _bh(k), _bh(v)
    G, N, _ = Q.shape
    dv = V.shape[-1]
    dfeat = feature_dim(Q.shape[-1], fmap, W)
    lg = _lg(log_gates, G, N, dfeat)
    S, z = _state(S0, z0, G, dfeat, dv)
    y = np.empty((G, N, dv))
    for t in range(N):
        y[:, t], S, z = gated_decode_step(S, z, Q[:, t], K[:, t], V[:, t], lg[:, t], fmap, W, normalize)
    lead = shape[:-2]
    return (y.reshape(shape[:-1] + (dv,)), S.reshape(lead + S.shape[1:]),
            z.reshape(lead + z.shape[1:]))


def gated_chunked(q, k, v, log_gates, fmap="elu1", W=None, normalize=True, chunk=64, S0=None, z0=None):
    """Blockwise gated form ([LA] "Entrenamiento: forma paralela" applied to the
    gated recurrence): inside a block of L tokens with in-block cumulative
    log-gates lam (lam_r = sum of the block's log-gates up to row r), key j
    enters row i through channel f with weight exp(lam_if - lam_jf) (j <= i),
    the carried state with exp(lam_if), and the state moves on as
    S <- diag(exp(lam_last)) S + sum_j diag(exp(lam_last - lam_j)) phi(k_j) v_j^T.
    Returns (y, S_N, z_N)."""
    shape = np.asarray(q).shape
    Q, K, V = _bh(q), _bh(k), _bh(v)
    G, N, _ = Q.shape
    dv = V.shape[-1]
    Qf = feature_map(Q, fmap, W)
    Kf = feature_map(K, fmap, W)
    dfeat = Qf.shape[-1]
    lg = _lg(log_gates, G, N, dfeat)
    S, z = _state(S0, z0, G, dfeat, dv)
    y = np.empty((G, N, dv))
    for s in range(0, N, chunk):
        e = min(N, s + chunk)
        Lb = e - s
        qc, kc, vc = Qf[:, s:e], Kf[:, s:e], V[:, s:e]
        lam = np.cumsum(lg[:, s:e], axis=1)                      # [G, L, d']
        wgt = np.exp(lam[:, :, None, :] - lam[:, None, :, :])    # [G, L(i), L(j), d']
        A = np.einsum("gic,gjc,gijc->gij", qc, kc, wgt) * np.tril(np.ones((Lb, Lb)))[None]
        qs = qc * np.exp(lam)                                    # carried-state weight per channel
        num = np.einsum("gij,gje->gie", A, vc) + np.einsum("gic,gce->gie", qs, S)
        den = A.sum(axis=2) + np.einsum("gic,gc->gi", qs, z)
        y[:, s:e] = _finish(num, den, normalize)
        last = lam[:, -1]
        kw = kc * np.exp(last[:, None, :] - lam)
        S = np.exp(last)[:, :, None] * S + np.einsum("gjc,gje->gce", kw, vc)
        z = np.exp(last) * z + kw.sum(axis=1)
    lead = shape[:-2]
    return (y.reshape(shape[:-1] + (dv,)), S.reshape(lead + S.shape[1:]),
            z.reshape(lead + z.shape[1:]))
