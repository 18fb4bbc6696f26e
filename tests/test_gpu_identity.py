"""GPU parity of the identity feature map, phi(x) = x ("Linear Attention",
marovi.ai, "Mapas de características").

Without normalization the causal form is the masked product tril(Q K^T) V.
With normalization the denominator phi(q).sum(phi(k)) can be <= 0 for
signed inputs (both sides then clamp it to 1e-6); the normalized cases use
positive inputs so that it stays well away from the clamp.
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


def _positive(B, H, N, d, seed, dt):
    rng = np.random.default_rng(seed)
    x = [rng.uniform(0.05, 1.0, (B, H, N, d)).astype(np.float32) for _ in range(3)]
    if dt == "bf16":
        x = [la_inputs.bf16_round(t) for t in x]
    return x


@pytest.mark.parametrize("din,dout", [("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")])
def test_feature_map_identity(din, dout):
    log(f"case feature_map identity {din}->{dout}")
    rng = np.random.default_rng(4)
    x = rng.standard_normal((77, 64)).astype(np.float32)
    if din == "bf16":
        x = la_inputs.bf16_round(x)
    y = to_host(la.la_feature_map_apply(to_dev(x, din), feature_map="identity",
                                        out_dtype={"bf16": torch.bfloat16, "f32": torch.float32}[dout]))
    ref = O.phi_identity(x)
    if dout == "bf16":
        ref = la_inputs.bf16_round(ref.astype(np.float32)).astype(np.float64)
    np.testing.assert_array_equal(y, ref)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_identity_forward_unnormalized(d, dt):
    for N in (1, 65, 64 * 40 - 17):
        for causal in (True, False):
            log(f"case identity forward d{d} {dt} N{N} causal={causal} normalize=0")
            q, k, v = qkv(1, 2, N, d, 300 + N + d, dt, 1.0 / np.sqrt(d))
            y = la.la_forward(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), feature_map="identity", causal=causal,
                              normalize=False)
            torch.cuda.synchronize()
            ref = O.attention(q, k, v, "identity", causal=causal, normalize=False)
            err = rel_err(to_host(y), ref)
            log(f"  rel err {err:.3e}")
            assert err <= TOL[dt], err


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_identity_forward_normalized_positive(dt):
    for N in (200, 64 * 40 - 17):
        for causal in (True, False):
            log(f"case identity forward d64 {dt} N{N} causal={causal} normalize=1")
            q, k, v = _positive(1, 2, N, 64, 17 + N, dt)
            y, S, z = la.la_forward(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), feature_map="identity",
                                    causal=causal, return_state=True)
            torch.cuda.synchronize()
            assert rel_err(to_host(y), O.attention(q, k, v, "identity", causal=causal)) <= TOL[dt]
            Sr, zr = O.final_state(k, v, "identity")
            assert rel_err(to_host(S), Sr) <= TOL[dt]
            assert rel_err(to_host(z)[..., None], zr[..., None]) <= TOL[dt]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("normalize", [False, True])
def test_identity_decode(d, normalize):
    log(f"case identity decode d{d} normalize={normalize}")
    B, H, N0, T = 2, 3, 70, 4
    if normalize:
        q, k, v = _positive(B, H, N0 + T, d, 5 + d, "bf16")
    else:
        q, k, v = qkv(B, H, N0 + T, d, 5 + d, "bf16")
    S0, z0 = O.final_state(k[:, :, :N0], v[:, :, :N0], "identity")
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    Sr, zr = S0, z0
    for t in range(N0, N0 + T):
        y = la.la_decode_step(S, z, to_dev(q[:, :, t], "bf16"), to_dev(k[:, :, t], "bf16"), to_dev(v[:, :, t], "bf16"),
                              feature_map="identity", normalize=normalize)
        yr, Sr, zr = O.decode_step(Sr, zr, q[:, :, t], k[:, :, t], v[:, :, t], "identity", normalize=normalize)
        torch.cuda.synchronize()
        assert rel_err(to_host(y)[..., None, :], yr[..., None, :]) <= TOL["bf16"]
    assert rel_err(to_host(S), Sr) <= 1e-5
