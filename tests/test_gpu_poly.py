"""GPU parity of the degree-2 polynomial feature map, phi(x) = (1, x, x (x) x)
("Linear Attention", marovi.ai, "Mapas de características", polynomial
bullet; d' = 1 + d + d^2), against the CPU oracle (whose map is pinned by
the kernel identity phi(q).phi(k) = 1 + q.k + (q.k)^2 and a brute force over
dot products). Tolerance as elsewhere: 2e-2 for bf16 inputs, 1e-4 for fp32.
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
from gpu_helpers import TOL, log, qkv, rel_err, to_dev, to_host  # noqa: E402


def _check(B, H, N, d, dt, seed, causal=True, normalize=True, scale=None, state=False):
    log(f"case poly2 forward B{B} H{H} N{N} d{d} {dt} causal={causal} norm={normalize} state={state}")
    q, k, v = qkv(B, H, N, d, seed, dt, 1.0 / np.sqrt(d) if scale is None else scale)
    kw, S0, z0 = {}, None, None
    if state:
        rng = np.random.default_rng(seed + 5)
        kk = la_inputs.gaussian(rng, (B, H, 40, d), 1.0 / np.sqrt(d), bf16=False)
        vv = la_inputs.gaussian(rng, (B, H, 40, d), bf16=False)
        S0, z0 = O.final_state(kk, vv, "poly2")
        kw = dict(S_in=torch.from_numpy(S0.astype(np.float32)).cuda(),
                  z_in=torch.from_numpy(z0.astype(np.float32)).cuda())
    y, S, z = la.la_forward(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), feature_map="poly2", causal=causal,
                            normalize=normalize, return_state=True, **kw)
    torch.cuda.synchronize()
    ref = O.attention(q, k, v, "poly2", causal=causal, normalize=normalize, S0=S0, z0=z0)
    Sr, zr = O.final_state(k, v, "poly2", S0=S0, z0=z0)
    e, eS = rel_err(to_host(y), ref), rel_err(to_host(S), Sr)
    ez = rel_err(to_host(z)[..., None], zr[..., None])
    log(f"  rel err y {e:.3e} S {eS:.3e} z {ez:.3e}")
    assert S.shape[-2] == 1 + d + d * d
    assert e <= TOL[dt] and eS <= TOL[dt] and ez <= TOL[dt], (e, eS, ez)


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_poly2_small(d, dt):
    for N in (1, 63, 64, 65, 200):
        _check(1, 2, N, d, dt, seed=600 + N + d)


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("normalize", [True, False])
def test_poly2_several_chunks(d, dt, causal, normalize):
    _check(2, 1, 64 * 9 - 21, d, dt, seed=650 + d + 2 * causal + normalize, causal=causal, normalize=normalize)


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_poly2_state_in_and_unit_scale_inputs(d, dt):
    _check(1, 2, 300, d, dt, seed=700 + d, state=True)
    _check(1, 2, 300, d, dt, seed=710 + d, causal=False, state=True)
    _check(1, 2, 150, d, dt, seed=720 + d, scale=1.0)   # q.k of size sqrt(d): the s^2 term dominates


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_poly2_decode_and_handoff(d, dt):
    log(f"case poly2 decode d{d} {dt}")
    B, H, N0, T = 2, 2, 70, 6
    q, k, v = qkv(B, H, N0 + T, d, 760 + d, dt, 1.0 / np.sqrt(d))
    tq, tk, tv = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    _, S, z = la.la_forward(tq[:, :, :N0].contiguous(), tk[:, :, :N0].contiguous(), tv[:, :, :N0].contiguous(),
                            feature_map="poly2", return_state=True)
    ref = O.attention(q, k, v, "poly2")
    for t in range(N0, N0 + T):
        y = la.la_decode_step(S, z, tq[:, :, t].contiguous(), tk[:, :, t].contiguous(), tv[:, :, t].contiguous(),
                              feature_map="poly2")
        torch.cuda.synchronize()
        e = rel_err(to_host(y)[:, :, None], ref[:, :, t:t + 1])
        assert e <= TOL[dt], (t, e)
    Sr, zr = O.final_state(k, v, "poly2")
    assert rel_err(to_host(S), Sr) <= TOL[dt]
    assert rel_err(to_host(z)[..., None], zr[..., None]) <= TOL[dt]


@pytest.mark.parametrize("din,dout", [("bf16", "f32"), ("f32", "f32"), ("bf16", "bf16")])
def test_feature_map_poly2(din, dout):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((37, 32)).astype(np.float32)
    if din == "bf16":
        x = la_inputs.bf16_round(x)
    y = to_host(la.la_feature_map_apply(to_dev(x, din), feature_map="poly2",
                                        out_dtype={"bf16": torch.bfloat16, "f32": torch.float32}[dout]))
    ref = O.phi_poly2(x)
    assert y.shape == (37, 1 + 32 + 32 * 32)
    if dout == "bf16":
        ref = la_inputs.bf16_round(ref.astype(np.float32)).astype(np.float64)
        np.testing.assert_array_equal(y, ref)
    else:
        np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)   # one fp32 product per feature


def test_poly2_empty_sequence_copies_state():
    d, H = 32, 2
    S0 = torch.randn(1, H, 1 + d + d * d, d, device="cuda")
    z0 = torch.rand(1, H, 1 + d + d * d, device="cuda")
    x = torch.zeros(1, H, 0, d, device="cuda", dtype=torch.bfloat16)
    _, S, z = la.la_forward(x, x.clone(), x.clone(), feature_map="poly2", S_in=S0, z_in=z0, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(z, z0)


def test_poly2_prefill_b4h8n2048d64_sampled_heads():
    """The prefill workload shape with the polynomial map, in one call; two
    whole heads against the oracle's recurrent form (token by token through
    the d' = 4161 state)."""
    W = la_inputs.WORKLOADS["prefill_b4h8n2048d64"]
    B, H, N, d = W["B"], W["H"], W["N"], W["d"]
    log(f"case poly2 prefill B{B} H{H} N{N} d{d} bf16 (two heads checked)")
    q, k, v = la_inputs.gaussian_qkv(B, H, N, d, seed=W["seed"], scale=W["scale"], bf16=True)
    y = la.la_forward(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), feature_map="poly2")
    torch.cuda.synchronize()
    got = to_host(y)
    for b, h in ((0, 0), (3, 7)):
        ref, _, _ = O.recurrent(q[b, h], k[b, h], v[b, h], "poly2")
        e = rel_err(got[b, h], ref)
        log(f"  head ({b}, {h}) rel err {e:.3e}")
        assert e <= TOL["bf16"], (b, h, e)
