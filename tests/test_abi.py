"""C-ABI checks that need no GPU: the library loads, exports every declared
function, and rejects bad arguments before enqueuing anything."""

import ctypes

import pytest

import causal_linear_attention_02_amd as la
from causal_linear_attention_02_amd import lib, la_feature_map

FAKE = 0x10000          # 16-byte aligned address that is never dereferenced
FAKE2 = 0x40000000
ELU = la_feature_map(la.LA_ELU1, 0, None)


def test_library_exports_every_declared_function():
    names = la.declared_functions()
    assert {"la_forward", "la_forward_ex", "la_decode_step", "la_feature_map_apply",
            "la_forward_workspace_size", "la_status_string", "la_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    for code in (la.LA_OK, la.LA_ERR_INVALID_ARG, la.LA_ERR_UNSUPPORTED, la.LA_ERR_WORKSPACE, la.LA_ERR_HIP, 7):
        s = la.la_status_string(code)
        assert isinstance(s, str) and s
    assert la.la_version() > 0


def _fwd(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, out=FAKE2, B=1, H=1, N=128, d=64, fm=ELU, causal=1,
         normalize=1, dtype=la.LA_BF16, S_in=None, z_in=None, S_out=None, z_out=None, ws=None, ws_bytes=0):
    return lib.la_forward(q, k, v, out, B, H, N, d, ctypes.byref(fm) if fm is not None else None, causal,
                          normalize, dtype, S_in, z_in, S_out, z_out, ws, ws_bytes, None)


def test_forward_rejects_bad_arguments():
    assert _fwd(B=-1) == la.LA_ERR_INVALID_ARG
    assert _fwd(N=-5) == la.LA_ERR_INVALID_ARG
    assert _fwd(causal=2) == la.LA_ERR_INVALID_ARG
    assert _fwd(normalize=-1) == la.LA_ERR_INVALID_ARG
    assert _fwd(dtype=5) == la.LA_ERR_INVALID_ARG
    assert _fwd(fm=None) == la.LA_ERR_INVALID_ARG
    assert _fwd(fm=la_feature_map(9, 0, None)) == la.LA_ERR_INVALID_ARG
    assert _fwd(d=48) == la.LA_ERR_UNSUPPORTED
    assert _fwd(d=256) == la.LA_ERR_UNSUPPORTED
    assert _fwd(q=None) == la.LA_ERR_INVALID_ARG
    assert _fwd(out=None) == la.LA_ERR_INVALID_ARG
    assert _fwd(q=FAKE + 2) == la.LA_ERR_INVALID_ARG               # misaligned
    assert _fwd(out=FAKE + 64) == la.LA_ERR_INVALID_ARG            # out overlaps q
    assert _fwd(S_in=FAKE2 + 0x100000) == la.LA_ERR_INVALID_ARG    # S_in without z_in
    assert _fwd(S_out=FAKE2 + 0x100000) == la.LA_ERR_INVALID_ARG   # S_out without z_out
    # S_out overlapping the output
    assert _fwd(S_out=FAKE2 + 256, z_out=FAKE2 + 0x200000) == la.LA_ERR_INVALID_ARG
    # performer map without W
    assert _fwd(fm=la_feature_map(la.LA_PERFORMER, 64, None)) == la.LA_ERR_INVALID_ARG


def test_identity_map_accepted_by_planning():
    ident = la_feature_map(la.LA_IDENTITY, 0, None)
    for d in (32, 64, 128):
        got = la.lib.la_forward_workspace_size(1, 2, 4096, d, ctypes.byref(ident), 1)
        want = la.lib.la_forward_workspace_size(1, 2, 4096, d, ctypes.byref(ELU), 1)
        assert got == want > 0   # same plan as elu+1 (d' = d, no mapped-feature buffers)
    assert _fwd(fm=ident, d=48) == la.LA_ERR_UNSUPPORTED


def test_forward_workspace_checks():
    # a long single sequence is split into segments and needs workspace
    need = lib.la_forward_workspace_size(1, 1, 65536, 128, ctypes.byref(ELU), 1)
    assert need > 0
    assert _fwd(N=65536, d=128) == la.LA_ERR_WORKSPACE
    assert _fwd(N=65536, d=128, ws=FAKE2 * 2, ws_bytes=need - 4) == la.LA_ERR_WORKSPACE
    assert _fwd(N=65536, d=128, ws=FAKE2 * 2 + 16, ws_bytes=need) == la.LA_ERR_INVALID_ARG  # not 256-aligned
    # workspace overlapping the output buffer
    assert _fwd(N=65536, d=128, ws=FAKE2, ws_bytes=need) == la.LA_ERR_INVALID_ARG


def test_empty_problems_are_noops():
    assert _fwd(B=0) == la.LA_OK
    assert _fwd(H=0, q=None, k=None, v=None, out=None) == la.LA_OK
    assert lib.la_decode_step(None, None, None, None, None, None, 0, 4, 64, ctypes.byref(ELU), 1, 1, None) == la.LA_OK
    assert lib.la_feature_map_apply(None, None, 0, 64, ctypes.byref(ELU), 1, 1, None) == la.LA_OK


def test_workspace_size_plan():
    ws = lambda B, H, N, d, c: lib.la_forward_workspace_size(B, H, N, d, ctypes.byref(ELU), c)
    st = lambda d: (d * d + d) * 4
    # one chunk per sequence: nothing to carry (causal), one total slot (non-causal)
    assert ws(4, 8, 64, 64, 1) == 0
    assert ws(4, 8, 64, 64, 0) == 32 * 2 * st(64)
    # many sequences: one segment each, no causal workspace
    assert ws(256, 32, 4096, 64, 1) == 0
    # invalid requests report 0
    assert ws(1, 1, 100, 48, 1) == 0
    assert ws(-1, 1, 100, 64, 1) == 0
    # long sequence: several segments, workspace grows with the state size
    a, b = ws(1, 16, 65536, 64, 1), ws(1, 16, 65536, 128, 1)
    assert a > 0 and b > 0 and b % st(128) == 0 and a % st(64) == 0
    assert b // st(128) == a // st(64)


def test_workspace_size_by_dtype():
    """Random features in bf16 project inside the chunked passes, causal or
    not, at every head dimension: their exact workspace is the segment states
    alone; fp32 also holds phi(q) and phi(k) ([B][H][N][m] fp32 each). The
    dtype-free size covers both element types."""
    B, H, N = 1, 2, 64 * 40 - 17
    for d, m in ((64, 256), (64, 64), (32, 128), (128, 64)):
        fm = la_feature_map(la.LA_PERFORMER, m, FAKE)
        for c in (1, 0):
            f32 = lib.la_forward_workspace_size_dt(B, H, N, d, ctypes.byref(fm), c, la.LA_F32)
            bf = lib.la_forward_workspace_size_dt(B, H, N, d, ctypes.byref(fm), c, la.LA_BF16)
            anyt = lib.la_forward_workspace_size(B, H, N, d, ctypes.byref(fm), c)
            phi = 2 * ((B * H * N * m * 4 + 255) // 256 * 256)
            assert anyt == max(f32, bf)
            assert f32 - bf == phi, (d, m, c)
            assert bf % ((m * d + m) * 4) == 0     # segment states only
    elu = lib.la_forward_workspace_size_dt(1, 16, 65536, 128, ctypes.byref(ELU), 1, la.LA_BF16)
    assert elu == lib.la_forward_workspace_size(1, 16, 65536, 128, ctypes.byref(ELU), 1) > 0
    assert lib.la_forward_workspace_size_dt(1, 16, 65536, 128, ctypes.byref(ELU), 1, 7) == 0


def test_decode_rejects_bad_arguments():
    dec = lambda **kw: lib.la_decode_step(kw.get("S", FAKE), kw.get("z", FAKE + 0x1000000),
                                          kw.get("q", FAKE + 0x2000000), kw.get("k", FAKE + 0x3000000),
                                          kw.get("v", FAKE + 0x4000000), kw.get("out", FAKE + 0x5000000),
                                          kw.get("B", 2), kw.get("H", 2), kw.get("d", 64),
                                          ctypes.byref(kw.get("fm", ELU)), kw.get("normalize", 1),
                                          kw.get("dtype", 1), None)
    assert dec(B=-1) == la.LA_ERR_INVALID_ARG
    assert dec(d=96) == la.LA_ERR_UNSUPPORTED
    assert dec(S=None) == la.LA_ERR_INVALID_ARG
    assert dec(out=FAKE + 0x2000000) == la.LA_ERR_INVALID_ARG   # out == q
    assert dec(z=FAKE + 64) == la.LA_ERR_INVALID_ARG             # z inside S
    assert dec(q=FAKE + 0x2000008) == la.LA_ERR_INVALID_ARG      # misaligned
    assert dec(normalize=3) == la.LA_ERR_INVALID_ARG
    assert dec(dtype=2) == la.LA_ERR_INVALID_ARG


def test_feature_map_apply_rejects_bad_arguments():
    fa = lambda **kw: lib.la_feature_map_apply(kw.get("x", FAKE), kw.get("phi", FAKE2), kw.get("rows", 10),
                                               kw.get("d", 64), ctypes.byref(kw.get("fm", ELU)),
                                               kw.get("i", 1), kw.get("o", 1), None)
    assert fa(rows=-1) == la.LA_ERR_INVALID_ARG
    assert fa(d=40) == la.LA_ERR_UNSUPPORTED
    assert fa(x=None) == la.LA_ERR_INVALID_ARG
    assert fa(phi=FAKE + 32) == la.LA_ERR_INVALID_ARG            # overlap
    assert fa(i=3) == la.LA_ERR_INVALID_ARG


def test_binding_maps_errors_to_exceptions():
    import torch
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):          # host tensors are refused, nothing is called
        la.la_forward(q, q.clone(), q.clone())
    with pytest.raises(NotImplementedError):
        la._check(la.LA_ERR_UNSUPPORTED, "x")
    with pytest.raises(ValueError):
        la._check(la.LA_ERR_WORKSPACE, "x")
    with pytest.raises(la.LinAttnError):
        la._check(la.LA_ERR_HIP, "x")
    la._check(la.LA_OK, "x")


def test_decay_entry_points_validate_before_launch():
    ident = ELU
    args = dict()
    # null gamma, non-causal is not reachable through la_forward_decay (always causal)
    st = lib.la_forward_decay(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, 1, 2, 64, 64,
                              ctypes.byref(ident), None, 1, la.LA_BF16, None, None, None, None, None, 0, None)
    assert st == la.LA_ERR_INVALID_ARG
    st = lib.la_forward_decay(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, 1, 2, 64, 64,
                              ctypes.byref(ident), FAKE2 + 2, 1, la.LA_BF16, None, None, None, None, None, 0, None)
    assert st == la.LA_ERR_INVALID_ARG          # misaligned gamma
    st = lib.la_decode_step_decay(FAKE, FAKE2, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                                  1, 2, 64, ctypes.byref(ident), None, 1, la.LA_BF16, None)
    assert st == la.LA_ERR_INVALID_ARG


def _bwd(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, dout=FAKE + 0x3000000, dq=FAKE2, dk=FAKE2 + 0x1000000,
         dv=FAKE2 + 0x2000000, B=1, H=1, N=128, d=64, fm=ELU, normalize=1, dtype=la.LA_BF16, S_in=None, z_in=None,
         dS_out=None, dz_out=None, dS_in=None, dz_in=None, ws=FAKE2 * 4, ws_bytes=1 << 30):
    return lib.la_backward(q, k, v, dout, dq, dk, dv, B, H, N, d, ctypes.byref(fm) if fm is not None else None,
                           normalize, dtype, S_in, z_in, dS_out, dz_out, dS_in, dz_in, ws, ws_bytes, None)


def test_backward_rejects_bad_arguments():
    assert _bwd(B=-1) == la.LA_ERR_INVALID_ARG
    assert _bwd(normalize=2) == la.LA_ERR_INVALID_ARG
    assert _bwd(dtype=3) == la.LA_ERR_INVALID_ARG
    assert _bwd(fm=None) == la.LA_ERR_INVALID_ARG
    assert _bwd(d=48) == la.LA_ERR_UNSUPPORTED
    W = FAKE2 * 8
    assert _bwd(fm=la_feature_map(la.LA_PERFORMER, 64, W)) == la.LA_ERR_UNSUPPORTED  # no random-feature gradients
    assert _bwd(dq=None) == la.LA_ERR_INVALID_ARG
    assert _bwd(dout=FAKE + 0x3000000 + 8) == la.LA_ERR_INVALID_ARG           # misaligned
    assert _bwd(dq=FAKE + 0x100) == la.LA_ERR_INVALID_ARG                      # dq overlaps q
    assert _bwd(dk=FAKE2 + 0x100) == la.LA_ERR_INVALID_ARG                     # dk overlaps dq
    assert _bwd(S_in=FAKE2 * 6) == la.LA_ERR_INVALID_ARG                       # S_in without z_in
    assert _bwd(dS_out=FAKE2 * 6) == la.LA_ERR_INVALID_ARG                     # dS_out without dz_out
    assert _bwd(dS_in=FAKE2 * 6) == la.LA_ERR_INVALID_ARG                      # dS_in without dz_in
    # dS_in overlapping dS_out
    assert _bwd(dS_out=FAKE2 * 6, dz_out=FAKE2 * 7, dS_in=FAKE2 * 6 + 256, dz_in=FAKE2 * 7 + 0x100000) \
        == la.LA_ERR_INVALID_ARG
    need = lib.la_backward_workspace_size(1, 1, 128, 64, ctypes.byref(ELU))
    assert need > 0
    assert _bwd(ws=None) == la.LA_ERR_WORKSPACE
    assert _bwd(ws_bytes=need - 1) == la.LA_ERR_WORKSPACE
    assert _bwd(ws=FAKE2 * 4 + 16) == la.LA_ERR_INVALID_ARG                    # not 256-aligned
    assert _bwd(ws=FAKE2, ws_bytes=need) == la.LA_ERR_INVALID_ARG              # workspace overlaps dq
    assert _bwd(B=0) == la.LA_OK and _bwd(N=0) == la.LA_OK                     # nothing to do


def _bwd_decay(gamma=FAKE2 * 9, **kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, dout=FAKE + 0x3000000, dq=FAKE2, dk=FAKE2 + 0x1000000,
             dv=FAKE2 + 0x2000000, B=1, H=1, N=128, d=64, fm=ELU, normalize=1, dtype=la.LA_BF16, S_in=None,
             z_in=None, dS_out=None, dz_out=None, dS_in=None, dz_in=None, ws=FAKE2 * 4, ws_bytes=1 << 30)
    a.update(kw)
    return lib.la_backward_decay(a["q"], a["k"], a["v"], a["dout"], a["dq"], a["dk"], a["dv"], a["B"], a["H"],
                                 a["N"], a["d"], ctypes.byref(a["fm"]) if a["fm"] is not None else None, gamma,
                                 a["normalize"], a["dtype"], a["S_in"], a["z_in"], a["dS_out"], a["dz_out"],
                                 a["dS_in"], a["dz_in"], a["ws"], a["ws_bytes"], None)


def test_backward_decay_rejects_bad_arguments():
    assert _bwd_decay(gamma=None) == la.LA_ERR_INVALID_ARG                   # gamma is required
    assert _bwd_decay(gamma=FAKE2 * 9 + 2) == la.LA_ERR_INVALID_ARG          # misaligned gamma
    assert _bwd_decay(gamma=FAKE2 + 0x40) == la.LA_ERR_INVALID_ARG           # gamma inside dq
    assert _bwd_decay(gamma=FAKE2 * 4 + 0x40) == la.LA_ERR_INVALID_ARG       # gamma inside the workspace
    assert _bwd_decay(B=-1) == la.LA_ERR_INVALID_ARG
    assert _bwd_decay(d=48) == la.LA_ERR_UNSUPPORTED
    assert _bwd_decay(fm=la_feature_map(la.LA_PERFORMER, 64, FAKE2 * 8)) == la.LA_ERR_UNSUPPORTED
    assert _bwd_decay(dq=FAKE + 0x100) == la.LA_ERR_INVALID_ARG
    assert _bwd_decay(ws=None) == la.LA_ERR_WORKSPACE
    assert _bwd_decay(N=0) == la.LA_OK


def test_backward_workspace_plan():
    ident = la_feature_map(la.LA_IDENTITY, 0, None)
    for d in (32, 64, 128):
        for N in (1, 64, 1000, 65536):
            a = lib.la_backward_workspace_size(2, 3, N, d, ctypes.byref(ELU))
            b = lib.la_backward_workspace_size(2, 3, N, d, ctypes.byref(ident))
            # at least the per-token statistics and one gradient state per sequence
            assert a == b >= 2 * 3 * (N * 8 + 2 * (d * d + d) * 4)
    assert lib.la_backward_workspace_size(1, 1, 0, 64, ctypes.byref(ELU)) == 0
    assert lib.la_backward_workspace_size(1, 1, 64, 48, ctypes.byref(ELU)) == 0
    assert lib.la_backward_workspace_size(1, 1, 64, 64, ctypes.byref(la_feature_map(la.LA_PERFORMER, 64, FAKE))) == 0


def test_gated_entry_points_validate_before_launch():
    ident = la_feature_map(la.LA_IDENTITY, 0, None)
    G = FAKE2 * 8

    def fg(lg=G, fm=ELU, d=64, N=128, ws=FAKE2 * 4, wsb=1 << 30, out=FAKE2):
        return lib.la_forward_gated(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, lg, out, 1, 1, N, d,
                                    ctypes.byref(fm), 1, la.LA_BF16, None, None, None, None, ws, wsb, None)
    assert fg(lg=None) == la.LA_ERR_INVALID_ARG
    assert fg(lg=G + 4) == la.LA_ERR_INVALID_ARG                          # misaligned gates
    assert fg(d=48) == la.LA_ERR_UNSUPPORTED
    assert fg(fm=la_feature_map(la.LA_PERFORMER, 64, FAKE2 * 9)) == la.LA_ERR_UNSUPPORTED
    assert fg(out=G) == la.LA_ERR_INVALID_ARG                             # out overlaps the gates
    assert fg(N=65536, ws=None) == la.LA_ERR_WORKSPACE
    assert fg(N=0) == la.LA_OK
    assert lib.la_forward_gated_workspace_size(1, 1, 65536, 128, ctypes.byref(ELU)) > 0
    assert lib.la_forward_gated_workspace_size(1, 1, 64, 48, ctypes.byref(ELU)) == 0
    assert lib.la_forward_gated_workspace_size(1, 2, 4096, 64, ctypes.byref(ident)) == \
        lib.la_forward_gated_workspace_size(1, 2, 4096, 64, ctypes.byref(ELU))
    st = lib.la_decode_step_gated(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000, None,
                                  FAKE + 0x500000, 1, 1, 64, ctypes.byref(ELU), 1, la.LA_BF16, None)
    assert st == la.LA_ERR_INVALID_ARG                                    # gate missing


def test_poly2_map_planning_and_limits():
    poly = la_feature_map(la.LA_POLY2, 0, None)
    B, H, N = 2, 3, 1000
    for d, slots, dslots in ((32, 2, 2), (64, 4, 4)):
        n = lib.la_forward_workspace_size(B, H, N, d, ctypes.byref(poly), 1)
        # partial numerators (fp32, [slots][B*H][N][d]) and partial denominators
        assert n >= slots * B * H * N * d * 4 + dslots * B * H * N * 4
        assert n == lib.la_forward_workspace_size(B, H, N, d, ctypes.byref(poly), 0)
    assert lib.la_forward_workspace_size(1, 1, 64, 128, ctypes.byref(poly), 1) == 0   # d' = 16513: not built
    assert lib.la_forward_workspace_size(1, 1, 0, 64, ctypes.byref(poly), 1) == 0
    need = lib.la_forward_workspace_size(1, 1, 128, 64, ctypes.byref(poly), 1)
    assert _fwd(fm=poly, d=128) == la.LA_ERR_UNSUPPORTED
    assert _fwd(fm=poly) == la.LA_ERR_WORKSPACE
    assert _fwd(fm=poly, ws=FAKE2 * 4, ws_bytes=need - 1) == la.LA_ERR_WORKSPACE
    assert _fwd(fm=poly, ws=FAKE2 * 4 + 16, ws_bytes=need) == la.LA_ERR_INVALID_ARG   # not 256-aligned
    assert _fwd(fm=poly, ws=FAKE2, ws_bytes=need) == la.LA_ERR_INVALID_ARG            # overlaps out
    assert _fwd(fm=poly, N=0) == la.LA_OK
    st = lib.la_forward_decay(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE2, 1, 1, 128, 64, ctypes.byref(poly),
                              FAKE2 * 9, 1, la.LA_BF16, None, None, None, None, FAKE2 * 4, need, None)
    assert st == la.LA_ERR_UNSUPPORTED                                    # no decay with this map
    assert _bwd(fm=poly) == la.LA_ERR_UNSUPPORTED                          # no gradients with this map
    st = lib.la_forward_gated(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE2 * 8, FAKE2, 1, 1, 128, 64,
                              ctypes.byref(poly), 1, la.LA_BF16, None, None, None, None, FAKE2 * 4, 1 << 30, None)
    assert st == la.LA_ERR_UNSUPPORTED
    st = lib.la_decode_step_gated(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                                  FAKE2 * 8, FAKE + 0x500000, 1, 1, 64, ctypes.byref(poly), 1, la.LA_BF16, None)
    assert st == la.LA_ERR_UNSUPPORTED
    assert la.feature_dim(64, "poly2") == 4161


def test_forward_rejects_state_and_decay_overlaps():
    """The segment workspace must overlap no state buffer (z_in, z_out
    included), and decay factors must overlap no output or the workspace;
    all of it is checked before any HIP call."""
    need = lib.la_forward_workspace_size(1, 1, 65536, 128, ctypes.byref(ELU), 1)
    ws = FAKE2 * 4
    base = dict(N=65536, d=128, ws=ws, ws_bytes=need)
    S_ok, z_ok = FAKE2 * 8, FAKE2 * 8 + 0x100000
    assert _fwd(S_out=S_ok, z_out=ws + 256, **base) == la.LA_ERR_INVALID_ARG      # z_out inside the workspace
    assert _fwd(S_in=S_ok, z_in=ws + 512, **base) == la.LA_ERR_INVALID_ARG        # z_in inside the workspace
    assert _fwd(S_out=ws + 1024, z_out=z_ok, **base) == la.LA_ERR_INVALID_ARG     # S_out inside the workspace

    def dec_fwd(gamma, out=FAKE2, S_out=None, z_out=None, ws_=ws):
        return lib.la_forward_decay(FAKE, FAKE + 0x10000000, FAKE + 0x20000000, out, 1, 1, 65536, 128,
                                    ctypes.byref(ELU), gamma, 1, la.LA_BF16, None, None, S_out, z_out, ws_, need,
                                    None)
    assert dec_fwd(FAKE2 + 64) == la.LA_ERR_INVALID_ARG                              # gamma inside out
    assert dec_fwd(ws + 4096) == la.LA_ERR_INVALID_ARG                               # gamma inside the workspace
    assert dec_fwd(z_ok + 8, S_out=S_ok, z_out=z_ok) == la.LA_ERR_INVALID_ARG        # gamma inside z_out
    assert dec_fwd(FAKE2 + 2) == la.LA_ERR_INVALID_ARG                               # misaligned gamma
    assert dec_fwd(None) == la.LA_ERR_INVALID_ARG


def test_decode_decay_rejects_gamma_overlaps():
    def dec(gamma):
        return lib.la_decode_step_decay(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000,
                                        FAKE + 0x4000000, FAKE + 0x5000000, 2, 2, 64, ctypes.byref(ELU), gamma, 1,
                                        la.LA_BF16, None)
    assert dec(FAKE + 0x5000000) == la.LA_ERR_INVALID_ARG    # gamma inside out
    assert dec(FAKE + 256) == la.LA_ERR_INVALID_ARG          # gamma inside S
    assert dec(FAKE + 0x1000000) == la.LA_ERR_INVALID_ARG    # gamma inside z
    assert dec(None) == la.LA_ERR_INVALID_ARG


def test_forward_static_validates_and_rejects_beyond_its_array():
    """la_forward_static validates like la_forward (before any HIP call) and
    refuses a request whose workspace would exceed its fixed array."""
    def st(q=FAKE, out=FAKE2, B=1, H=16, N=65536, d=64, fm=ELU, causal=1, dtype=la.LA_BF16):
        return lib.la_forward_static(q, FAKE + 0x10000000, FAKE + 0x20000000, out, B, H, N, d, ctypes.byref(fm),
                                     causal, 1, dtype, None, None, None, None, None)
    assert st(B=-1) == la.LA_ERR_INVALID_ARG
    assert st(out=FAKE + 64) == la.LA_ERR_INVALID_ARG      # out overlaps q
    assert st(d=96) == la.LA_ERR_UNSUPPORTED
    # random features through the two-stage path: phi(q), phi(k) would take 2 x 16 x 65536 x 256 x 4 bytes
    W = FAKE2 * 8
    perf = la_feature_map(la.LA_PERFORMER, 256, W)
    assert lib.la_forward_workspace_size(1, 16, 65536, 64, ctypes.byref(perf), 1) > la.LA_STATIC_SCRATCH_BYTES
    assert st(fm=perf, dtype=la.LA_F32) == la.LA_ERR_WORKSPACE
    # the long-context workload fits (16 heads x 16 segments x 66 KB)
    assert lib.la_forward_workspace_size(1, 16, 65536, 128, ctypes.byref(ELU), 1) <= la.LA_STATIC_SCRATCH_BYTES
