"""The oracle pins catch plausible mistakes in the oracle.

Each case plants one mistake (a dropped term, a wrong sign, an off-by-one
index, a transposed operand, an exclusive instead of inclusive mask, ...) in
a copy of the oracle package, runs the pins (tests/test_oracle_pins.py, or
tests/test_oracle_backward_pins.py for the gradients) against that copy in a
fresh interpreter, and requires them to fail. Two controls
check the harness itself: an unaltered copy passes, and a copy that cannot
be imported fails.
"""

import os
import pathlib
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
SRC = (ROOT / "oracle" / "linattn_oracle.py").read_text()
INIT = (ROOT / "oracle" / "__init__.py").read_text()

# (text in the oracle, replacement, the mistake it stands for)
MUTANTS = [
    ("A = np.where(lag >= 0, A, 0.0)", "A = np.where(lag > 0, A, 0.0)",
     "definition: causal mask excludes the diagonal"),
    ("A = Qf[g] @ Kf[g].T", "A = Kf[g][:idx.size] @ Qf[g].T",
     "definition: similarity matrix transposed"),
    ("num = A @ V[g] + s0 * (Qf[g] @ S[g])", "num = A @ V[g]",
     "definition: initial state dropped from the numerator"),
    ("den = A.sum(axis=1) + s0[:, 0] * (Qf[g] @ z[g])", "den = A.sum(axis=1)",
     "definition: initial state dropped from the denominator"),
    ("return num / np.maximum(den, EPS)[..., None]", "return num / (den + EPS)[..., None]",
     "eps added to the denominator instead of a clamp"),
    ("np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))", "np.where(x > 0.0, x, np.exp(np.minimum(x, 0.0)))",
     "elu+1 without the +1"),
    ("np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))",
     "np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)) - 1.0)", "plain elu on the negative branch"),
    ("xt = x * d ** -0.25", "xt = x", "random features: input not scaled by d^(-1/4)"),
    ("xt = x * d ** -0.25", "xt = x * d ** -0.5", "random features: input scaled by d^(-1/2)"),
    ("return np.exp(u - 0.5 * sq) / np.sqrt(m)", "return np.exp(u - 0.5 * sq)",
     "random features: 1/sqrt(m) dropped"),
    ("return np.exp(u - 0.5 * sq) / np.sqrt(m)", "return np.exp(u + 0.5 * sq) / np.sqrt(m)",
     "random features: wrong sign of the norm term"),
    ("u = xt @ W.T", "u = xt @ W[:, ::-1].T", "random features: W columns reversed"),
    ("S = S + np.einsum(\"gnc,gne->gce\", Kf, V)", "S = S + np.einsum(\"gnc,gne->gce\", Kf[:, 1:], V[:, :-1])",
     "final state: keys and values misaligned by one"),
    ("z = z + Kf.sum(axis=1)", "z = z + Kf[:, 1:].sum(axis=1)", "final state: first key dropped from z"),
    ("den = np.einsum(\"gnc,gc->gn\", Qf, z)", "den = np.einsum(\"gnc,gc->gn\", Qf, z[:, ::-1])",
     "non-causal form: normalizer read with reversed feature index"),
    ("S_new = S + kf[..., :, None] * v[..., None, :]", "S_new = S + qf[..., :, None] * v[..., None, :]",
     "decode: state updated with phi(q)"),
    ("num = np.einsum(\"...c,...ce->...e\", qf, S_new)", "num = np.einsum(\"...c,...ce->...e\", qf, S)",
     "decode: numerator read before the update"),
    ("den = np.einsum(\"...c,...c->...\", qf, z_new)", "den = np.einsum(\"...c,...c->...\", qf, z)",
     "decode: denominator read before the update"),
    ("y[:, t], S, z = decode_step(S, z, Q[:, t], K[:, t], V[:, t], fmap, W, normalize, gam)",
     "y[:, t], S, z = decode_step(S, z, Q[:, t], K[:, t], V[:, max(t - 1, 0)], fmap, W, normalize, gam)",
     "recurrent loop: value of the previous token"),
    ("S = np.cumsum(kv, axis=1)", "S = np.cumsum(kv, axis=1) - kv", "cumulative form: exclusive prefix for S"),
    ("A = A * np.tril(np.ones((L, L)))[None]", "A = A * np.tril(np.ones((L, L)), -1)[None]",
     "blockwise form: strict mask inside the block"),
    ("+ sin[:, :, None] * np.einsum(\"gic,gce->gie\", qc, S)", "+ 0.0",
     "blockwise form: inter-block numerator dropped"),
    ("den = A.sum(axis=2) + sin * np.einsum(\"gic,gc->gi\", qc, z)", "den = A.sum(axis=2)",
     "blockwise form: inter-block denominator dropped"),
    ("z = carry[:, None] * z + np.einsum(\"gj,gjc->gc\", kw, kc)",
     "z = carry[:, None] * z + np.einsum(\"gj,gjc->gc\", kw[:, :-1], kc[:, :-1])",
     "blockwise form: last key of each block dropped from z"),
    ("A = A * np.where(lag >= 0, gam[g] ** np.maximum(lag, 0), 0.0)",
     "A = A * np.where(lag >= 0, gam[g] ** np.maximum(lag + 1, 0), 0.0)", "decay: exponent i-j+1"),
    ("s0 = (gam[g] ** (idx + 1.0))[:, None]", "s0 = (gam[g] ** idx)[:, None]",
     "decay: initial state weighted gamma^i instead of gamma^(i+1)"),
    ("        z = gam[:, None] ** N * z + np.einsum(\"gn,gnc->gc\", wgt, Kf)",
     "        z = z + np.einsum(\"gn,gnc->gc\", wgt, Kf)", "decay: initial normalizer not decayed"),
    ("        S = gam[..., None, None] * S\n", "        S = S\n", "decay: decode step without decay of S"),
    ("            sin = gam[:, None] ** (r[None, :] + 1.0)", "            sin = gam[:, None] ** r[None, :]",
     "decay: blockwise carried state weighted gamma^r"),
    ("            kw = gam[:, None] ** (L - 1.0 - r[None, :])", "            kw = gam[:, None] ** (L - r[None, :])",
     "decay: blockwise update weights off by one"),
]

# mistakes in the gradients, caught by tests/test_oracle_backward_pins.py
BACKWARD_MUTANTS = [
    ("dden = np.where(den >= EPS, -np.sum(dY[g] * num, axis=1) / Dn ** 2, 0.0)",
     "dden = np.where(den >= EPS, np.sum(dY[g] * num, axis=1) / Dn ** 2, 0.0)",
     "backward: wrong sign of the denominator cotangent"),
    ("dden = np.where(den >= EPS, -np.sum(dY[g] * num, axis=1) / Dn ** 2, 0.0)",
     "dden = np.where(den >= EPS, -np.sum(dY[g] * num, axis=1) / Dn, 0.0)",
     "backward: denominator cotangent divided by den once"),
    ("dM = (dnum @ V[g].T + dden[:, None]) * Gm", "dM = (dnum @ V[g].T) * Gm",
     "backward: denominator term dropped from the similarity cotangent"),
    ("dM = (dnum @ V[g].T + dden[:, None]) * Gm", "dM = dnum @ V[g].T + dden[:, None]",
     "backward: causal mask not applied to the similarity cotangent"),
    ("dKf[g] = dM.T @ Qf[g]", "dKf[g] = dM @ Qf[g]", "backward: key gradient with untransposed cotangent"),
    ("dV[g] = A.T @ dnum", "dV[g] = A @ dnum", "backward: value gradient with untransposed similarities"),
    ("dQf[g] = dM @ Kf[g] + s0[:, None] * (dnum @ S[g].T + dden[:, None] * z[g][None, :])",
     "dQf[g] = dM @ Kf[g] + s0[:, None] * (dnum @ S[g].T)",
     "backward: initial normalizer dropped from the query gradient"),
    ("dS0[g] = Qf[g].T @ (s0[:, None] * dnum) + carry * dSN[g]", "dS0[g] = Qf[g].T @ (s0[:, None] * dnum)",
     "backward: final-state cotangent not passed to the initial state"),
    ("dKf[g] = dM.T @ Qf[g] + w[:, None] * (V[g] @ dSN[g].T + dzN[g][None, :])",
     "dKf[g] = dM.T @ Qf[g] + w[:, None] * (V[g] @ dSN[g] + dzN[g][None, :])",
     "backward: final-state cotangent transposed in the key gradient"),
    ("                w = gam[g] ** (N - 1.0 - np.arange(N))", "                w = gam[g] ** (N - np.arange(N))",
     "backward: decay weights of the final state off by one"),
    ("return dphi * np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))", "return dphi",
     "backward: elu+1 derivative missing"),
    ("return dphi * np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))",
     "return dphi * np.where(x >= 0.0, 0.0, np.exp(np.minimum(x, 0.0))) + dphi * (x > 0.0)",
     "backward: elu+1 derivative, branch point moved"),
    ("return s * (t @ W - (x * s) * t.sum(axis=-1, keepdims=True))", "return s * (t @ W)",
     "backward: random-feature norm term dropped"),
    ("""        R = R + Qf[:, t, :, None] * dnum[:, t, None, :]
        r = r + Qf[:, t] * dden[:, t][:, None]
        dKf[:, t] = np.einsum("gce,ge->gc", R, V[:, t]) + r""",
     """        dKf[:, t] = np.einsum("gce,ge->gc", R, V[:, t]) + r
        R = R + Qf[:, t, :, None] * dnum[:, t, None, :]
        r = r + Qf[:, t] * dden[:, t][:, None]""",
     "recurrent backward: adjoint state exclusive of the current token"),
    ("        R = gm[:, None, None] * R\n", "        R = R\n", "recurrent backward: adjoint state not decayed"),
]

# mistakes in the gated forms, caught by tests/test_oracle_gated_pins.py
GATED_MUTANTS = [
    ("wgt = np.exp(L[g, i][None, :] - L[g, :i + 1])       # [i+1, d'] per key and channel",
     "wgt = np.exp(L[g, i][None, :] - L[g, :i + 1] + _lg(log_gates, G, N, dfeat)[g, :i + 1])",
     "gated definition: key weight includes its own gate"),
    ("s0 = np.exp(L[g, i])                                 # initial state, per channel",
     "s0 = np.exp(L[g, i] - _lg(log_gates, G, N, dfeat)[g, 0])",
     "gated definition: initial state skips the first gate"),
    ("num = a @ V[g, :i + 1] + (Qf[g, i] * s0) @ S[g]", "num = a @ V[g, :i + 1] + Qf[g, i] @ S[g]",
     "gated definition: initial state not gated"),
    ("wgt = np.exp(L[g, i][None, :] - L[g, :i + 1])       # [i+1, d'] per key and channel",
     "wgt = np.exp(L[g, i][None, :] - L[g, :i + 1])[:, ::-1]",
     "gated definition: channels of the gate reversed"),
    ("S_new = a[..., :, None] * S + kf[..., :, None] * v[..., None, :]",
     "S_new = a[..., None, :] * S + kf[..., :, None] * v[..., None, :]",
     "gated decode: gate applied to the value dimension"),
    ("z_new = a * z + kf", "z_new = z + kf", "gated decode: normalizer not gated"),
    ("wgt = np.exp(last[:, None, :] - L)                       # [G, N, d']",
     "wgt = np.exp(last[:, None, :] - L + _lg(log_gates, G, N, dfeat))",
     "gated final state: key weight off by one gate"),
    ("qs = qc * np.exp(lam)                                    # carried-state weight per channel",
     "qs = qc * np.exp(lam - lg[:, s:e])", "gated blockwise: carried state misses the row's own gate"),
    ("kw = kc * np.exp(last[:, None, :] - lam)", "kw = kc * np.exp(last[:, None, :] - lam + lg[:, s:e])",
     "gated blockwise: update weights off by one gate"),
]


POLY_MUTANTS = [
    ("one = np.ones(x.shape[:-1] + (1,))", "one = np.zeros(x.shape[:-1] + (1,))",
     "polynomial map: constant term dropped"),
    ("return np.concatenate([one, x, outer.reshape", "return np.concatenate([one, 0.5 * x, outer.reshape",
     "polynomial map: linear term scaled"),
    ("outer = x[..., :, None] * x[..., None, :]", "outer = x[..., :, None] * x[..., None, ::-1]",
     "polynomial map: second factor of x (x) x reversed"),
    ("outer = x[..., :, None] * x[..., None, :]", "outer = np.triu(x[..., :, None] * x[..., None, :])",
     "polynomial map: upper triangle of x (x) x only"),
    ("        return 1 + d + d * d", "        return d + d * d", "polynomial map: feature dimension without the 1"),
]


def _run_pins(tmp_path, src, init=INIT, pins="test_oracle_pins.py"):
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    (pkg / "linattn_oracle.py").write_text(src)
    (pkg / "__init__.py").write_text(init)
    env = dict(os.environ, LA_ORACLE_UNDER_TEST=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", str(ROOT / "tests" / pins), "-x", "-q",
                        "-p", "no:cacheprovider"], env=env, cwd=str(ROOT), capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.mark.parametrize("pins", ["test_oracle_pins.py", "test_oracle_backward_pins.py", "test_oracle_gated_pins.py",
                                  "test_oracle_poly_pins.py"])
def test_control_unaltered_copy_passes(tmp_path, pins):
    rc, out = _run_pins(tmp_path, SRC, pins=pins)
    assert rc == 0, out


def test_control_copy_is_the_one_imported(tmp_path):
    rc, _ = _run_pins(tmp_path, "raise ImportError('altered copy')\n")
    assert rc != 0


@pytest.mark.parametrize("old,new,what", MUTANTS, ids=[m[2] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, old, new, what):
    assert SRC.count(old) >= 1, f"mutation site not found: {old!r}"
    rc, out = _run_pins(tmp_path, SRC.replace(old, new, 1))
    assert rc != 0, f"the pins did not catch: {what}\n{out}"


@pytest.mark.parametrize("old,new,what", BACKWARD_MUTANTS, ids=[m[2] for m in BACKWARD_MUTANTS])
def test_backward_pins_catch_planted_mistake(tmp_path, old, new, what):
    assert SRC.count(old) >= 1, f"mutation site not found: {old!r}"
    rc, out = _run_pins(tmp_path, SRC.replace(old, new, 1), pins="test_oracle_backward_pins.py")
    assert rc != 0, f"the pins did not catch: {what}\n{out}"


@pytest.mark.parametrize("old,new,what", GATED_MUTANTS, ids=[m[2] for m in GATED_MUTANTS])
def test_gated_pins_catch_planted_mistake(tmp_path, old, new, what):
    assert SRC.count(old) >= 1, f"mutation site not found: {old!r}"
    rc, out = _run_pins(tmp_path, SRC.replace(old, new, 1), pins="test_oracle_gated_pins.py")
    assert rc != 0, f"the pins did not catch: {what}\n{out}"


@pytest.mark.parametrize("old,new,what", POLY_MUTANTS, ids=[m[2] for m in POLY_MUTANTS])
def test_poly_pins_catch_planted_mistake(tmp_path, old, new, what):
    assert SRC.count(old) >= 1, f"mutation site not found: {old!r}"
    rc, out = _run_pins(tmp_path, SRC.replace(old, new, 1), pins="test_oracle_poly_pins.py")
    assert rc != 0, f"the pins did not catch: {what}\n{out}"
