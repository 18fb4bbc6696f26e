#!/usr/bin/env python3
"""Benchmark of kernelized linear attention on one MI355X.

One step = one causal prefill of the long-context workload (B=1, H=16,
N=65536, d=128, bf16, elu+1, normalized), inputs resident in HBM. The decode
workload (256 sequences x 32 heads, d=64, fp32 state, 1000 single-token steps
after a 4096-token prefill) is timed in the same run and reported under
"decode". Prints one JSON line.

Roofline: per dominant kernel, algorithmic bytes per launch / average launch
duration (HIP events recorded on the launch stream) against 8 TB/s.
cpu_baseline: the CPU oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    # The GPU's clocks take some tens of milliseconds of sustained work to
    # settle (after 5 calls the long-context prefill took ~396 us/call, after
    # 200 calls ~338 us/call). Before the warm-up calls, the hot path runs
    # back to back for this long; the phase is reported in the JSON
    # ("settle") and lies outside the timed steps.
    p.add_argument("--settle-ms", type=float, default=300.0)
    # each further workload (gradients, gated, variants, short sequences,
    # random features, polynomial map) runs back to back this long before
    # its own warm-up and timed calls, reported as its "settle_ms"
    p.add_argument("--settle-ms-each", type=float, default=100.0)
    p.add_argument("--decode-steps", type=int, default=1000)
    p.add_argument("--decode-warmup", type=int, default=20)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--backward-steps", type=int, default=20)
    p.add_argument("--no-backward", action="store_true")
    p.add_argument("--gated-steps", type=int, default=20)
    p.add_argument("--no-gated", action="store_true")
    p.add_argument("--no-variants", action="store_true")
    p.add_argument("--poly-steps", type=int, default=50)
    p.add_argument("--no-poly", action="store_true")
    p.add_argument("--mid-steps", type=int, default=1000)
    p.add_argument("--no-mid", action="store_true")
    p.add_argument("--performer-steps", type=int, default=100)
    p.add_argument("--no-performer", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="time budget of the oracle's prefill sample (whole heads; the decode sample gets half)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="first run a plain device-to-device copy of this size three times (counter calibration)")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest(names):
    """sha256 over the kernel sources a counter summary was taken with."""
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "causal_linear_attention_02_amd", "csrc")
    for n in names:
        with open(os.path.join(base, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(summary, sources, bytes_per_launch):
    """HBM bytes per launch from a committed counter summary (key = value lines).

    Returns (traffic_bytes, note). traffic is None when the summary is missing
    or was taken with kernel sources other than the current ones."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", summary)
    try:
        with open(path) as f:
            kv = dict(line.split("=", 1) for line in f.read().splitlines() if "=" in line and not line.startswith("#"))
    except OSError:
        return None, "no counter summary"
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_digest") != kernel_source_digest(sources):
        return None, "kernel changed since the counters were taken"
    try:
        t = float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None, "summary without traffic"
    return t, f"{summary}: read {kv.get('read_bytes_per_launch')} + write {kv.get('write_bytes_per_launch')} B " \
              f"(calibrated FETCH_SIZE/WRITE_SIZE), {t / bytes_per_launch:.3f} x algorithmic"


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover
        return 1


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every sequence/head shards with no communication; see the design notes)", file=sys.stderr)
        return 2

    import torch
    import la_inputs
    import causal_linear_attention_02_amd as la

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib > 0:
        nb = args.copy_probe_mib << 20
        log(f"copy probe: 3 x {nb} bytes device-to-device")
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    W = la_inputs.WORKLOADS["prefill_b1h16n65536d128"]
    B, H, N, d = W["B"], W["H"], W["N"], W["d"]

    # ---------------- prefill ----------------
    log(f"prefill: generating inputs B{B} H{H} N{N} d{d}")
    q, k, v = la_inputs.gaussian_qkv(B, H, N, d, seed=W["seed"], scale=W["scale"], bf16=True)
    tq = torch.from_numpy(q).to(torch.bfloat16).to(dev)
    tk = torch.from_numpy(k).to(torch.bfloat16).to(dev)
    tv = torch.from_numpy(v).to(torch.bfloat16).to(dev)
    out = torch.empty_like(tq)
    ws_bytes = la.la_forward_workspace_size(B, H, N, d, causal=True)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    del q, k, v

    def fwd(events=None):
        la.la_forward_ex(tq, tk, tv, causal=True, normalize=True, out=out, workspace=ws, events=events)

    def settle_phase(fn, ms):
        # fn back to back for `ms` milliseconds, outside any timed region
        torch.cuda.synchronize()
        t_s = time.perf_counter()
        while time.perf_counter() - t_s < ms * 1e-3:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
        return round((time.perf_counter() - t_s) * 1e3, 1)

    log(f"prefill: settling the clocks for {args.settle_ms:.0f} ms")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t0 < args.settle_ms * 1e-3:
        for _ in range(20):
            fwd()
        n_settle += 20
        torch.cuda.synchronize()
    settle = {"calls": n_settle, "ms": round((time.perf_counter() - t0) * 1e3, 1),
              "why": "the hot path back to back until the clocks settle, before the warm-up and timed steps"}
    log(f"prefill: warmup {args.warmup}")
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    log(f"prefill: timing {args.steps} steps")
    # HIP events recorded on the launch stream at the pass boundaries of every
    # timed call give the per-pass durations of the same calls the wall clock
    # times
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:  # create the HIP events outside the timed region
        for x in e:
            x.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fwd(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    stage = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])  # ms
    ms_state, ms_scan, ms_out = stage.mean(axis=0)
    ms_dev = float(np.mean([e[0].elapsed_time(e[3]) for e in evs]))  # first to last marker of a call
    tokens = B * N
    value = tokens / (ms_step * 1e-3)
    head_tokens = B * H * N
    alg_bytes = head_tokens * 4 * d * 2                     # q, k, v read + out written, bf16
    out_gbs = alg_bytes / (ms_out * 1e-3) / 1e9
    whole_gbs = alg_bytes / (ms_step * 1e-3) / 1e9
    C = 64
    flops_useful = head_tokens * (4 * d * d + (C + 1) * 2 * d)  # chunked form, masked triangle
    log(f"prefill: {ms_step*1e3:.1f} us/step (state {ms_state*1e3:.1f}, scan {ms_scan*1e3:.1f}, "
        f"output {ms_out*1e3:.1f} us); output pass {out_gbs:.0f} GB/s")

    # ---------------- gradients (la_backward) on the same workload ----------------
    backward = None
    if not args.no_backward:
        gen = torch.Generator(device=dev)
        gen.manual_seed(W["seed"] + 7919)
        tdy = torch.randn((B, H, N, d), generator=gen, device=dev).to(torch.bfloat16)
        gq, gk, gv = torch.empty_like(tq), torch.empty_like(tq), torch.empty_like(tq)
        bws = torch.empty(la.la_backward_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev)

        def bwd():
            la.la_backward(tq, tk, tv, tdy, normalize=True, dq=gq, dk=gk, dv=gv, workspace=bws)

        b_settle = settle_phase(bwd, args.settle_ms_each)
        for _ in range(10):
            bwd()
        torch.cuda.synchronize()
        log(f"backward: timing {args.backward_steps} calls")
        t0 = time.perf_counter()
        for _ in range(args.backward_steps):
            bwd()
        torch.cuda.synchronize()
        bwall = (time.perf_counter() - t0) / args.backward_steps
        # least traffic any gradient pass needs: q, k, v, dout read and dq, dk, dv written once
        min_bytes = head_tokens * 7 * d * 2
        backward = {
            "metric": "causal linear-attn gradients (dq, dk, dv) head-tokens/s",
            "value": head_tokens / bwall, "unit": "head-tokens/s", "us_per_call": round(bwall * 1e6, 1),
            "steps": args.backward_steps, "settle_ms": b_settle, "forward_us_per_call": round(ms_step * 1e3, 1),
            "config": {"workload": "prefill_b1h16n65536d128", "batch": B, "heads": H, "seq_len": N, "d": d,
                       "feature_map": "elu1", "normalize": True, "dout": "N(0,1) bf16, seeded"},
            "min_traffic": {"bytes": min_bytes, "achieved_gbs": round(min_bytes / bwall / 1e9, 1),
                            "frac_hbm": round(min_bytes / bwall / 1e9 / HBM_PEAK_GBS, 4),
                            "note": "q, k, v, dout read once and dq, dk, dv written once, bf16"},
        }
        log(f"backward: {bwall*1e6:.1f} us/call ({bwall*1e3/ms_step:.2f}x the forward)")
        del tdy, gq, gk, gv, bws

    # ---------------- gated linear attention on the same workload ----------------
    gated = None
    if not args.no_gated:
        gen = torch.Generator(device=dev)
        gen.manual_seed(W["seed"] + 313)
        tlg = torch.log(torch.rand((B, H, N, d), generator=gen, device=dev) * 0.75 + 0.25)  # alpha ~ U(1/4, 1)
        gws = torch.empty(max(la.la_forward_gated_workspace_size(B, H, N, d), 256), dtype=torch.uint8, device=dev)

        def gfwd():
            la.la_forward_gated(tq, tk, tv, tlg, normalize=True, out=out, workspace=gws)

        g_settle = settle_phase(gfwd, args.settle_ms_each)
        for _ in range(10):
            gfwd()
        torch.cuda.synchronize()
        log(f"gated: timing {args.gated_steps} calls")
        t0 = time.perf_counter()
        for _ in range(args.gated_steps):
            gfwd()
        torch.cuda.synchronize()
        gwall = (time.perf_counter() - t0) / args.gated_steps
        g_bytes = head_tokens * (4 * d * 2 + d * 4)  # q, k, v read + out written (bf16), log-gates read (fp32)
        gated = {
            "metric": "causal gated linear-attn prefill tokens/s (per-channel gates)",
            "value": tokens / gwall, "unit": "tokens/s", "us_per_call": round(gwall * 1e6, 1),
            "steps": args.gated_steps, "settle_ms": g_settle,
            "config": {"workload": "prefill_b1h16n65536d128", "batch": B, "heads": H, "seq_len": N, "d": d,
                       "feature_map": "elu1", "normalize": True, "gates": "log U(1/4, 1), fp32, per token and channel"},
            "whole_op": {"bytes": g_bytes, "achieved_gbs": round(g_bytes / gwall / 1e9, 1),
                         "frac_hbm": round(g_bytes / gwall / 1e9 / HBM_PEAK_GBS, 4)},
        }
        log(f"gated: {gwall*1e6:.1f} us/call")
        del tlg, gws

    # ---------------- decay and identity-map forwards on the same workload ----------------
    variants = None
    if not args.no_variants:
        variants = {}
        gam = torch.linspace(0.9, 0.999, H, device=dev, dtype=torch.float32)  # one decay per head
        ws_nc = torch.empty(max(la.la_forward_workspace_size(B, H, N, d, causal=False), 256), dtype=torch.uint8,
                            device=dev)
        runs = {
            "decay": lambda: la.la_forward_decay(tq, tk, tv, gam, normalize=True, out=out, workspace=ws),
            "identity_map": lambda: la.la_forward(tq, tk, tv, feature_map="identity", normalize=False, out=out,
                                                  workspace=ws),
            # non-causal form: one state pass over every segment, the total by
            # the scan, then phi(Q) S / phi(Q) z; the same bytes as the causal form
            "non_causal": lambda: la.la_forward(tq, tk, tv, causal=False, normalize=True, out=out, workspace=ws_nc),
        }
        for name, fn in runs.items():
            v_settle = settle_phase(fn, args.settle_ms_each)
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
            vw = (time.perf_counter() - t0) / 20
            variants[name] = {"us_per_call": round(vw * 1e6, 1), "tokens_per_s": tokens / vw,
                              "settle_ms": v_settle,
                              "whole_op_frac_hbm": round(alg_bytes / vw / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"{name}: {vw*1e6:.1f} us/call")
        variants["note"] = ("same workload and bytes as the headline prefill; decay: gamma per head "
                            "0.9..0.999; identity map: numerator only; non_causal: sums over all tokens")
        del ws_nc

    del tq, tk, tv, out, ws
    torch.cuda.empty_cache()

    def time_calls(fn, warm, steps):
        # (seconds per call, settle phase in ms)
        st_ms = settle_phase(lambda: fn(0), args.settle_ms_each)
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps, st_ms

    # ---------------- elu+1 prefill at B=4 H=8 N=2048 d=64 ----------------
    # 33.6 MB per input set fits in the 256 MB last-level cache, so the calls
    # rotate over 8 input sets (268 MB) and every call reads from HBM
    mid = None
    if not args.no_mid:
        Wm = la_inputs.WORKLOADS["prefill_b4h8n2048d64"]
        Bm, Hm, Nm, dm = Wm["B"], Wm["H"], Wm["N"], Wm["d"]
        gen = torch.Generator(device=dev)
        gen.manual_seed(Wm["seed"])
        shp = (Bm, Hm, Nm, dm)
        sets = [[(torch.randn(shp, generator=gen, device=dev) * Wm["scale"]).to(torch.bfloat16) for _ in range(3)]
                + [torch.empty(shp, dtype=torch.bfloat16, device=dev)] for _ in range(8)]
        mws = torch.empty(max(la.la_forward_workspace_size(Bm, Hm, Nm, dm), 256), dtype=torch.uint8, device=dev)

        def mfwd(i):
            sq_, sk_, sv_, so_ = sets[i % 8]
            la.la_forward(sq_, sk_, sv_, causal=True, normalize=True, out=so_, workspace=mws)

        mwall, m_settle = time_calls(mfwd, 80, args.mid_steps)
        m_ht = Bm * Hm * Nm
        m_bytes = m_ht * 4 * dm * 2
        m_flops = m_ht * (4 * dm * dm + (C + 1) * 2 * dm)
        t_roof = max(m_bytes / (HBM_PEAK_GBS * 1e9), m_flops / (BF16_MFMA_PEAK_TFLOPS * 1e12))
        mid = {
            "metric": "causal linear-attn prefill tokens/s", "value": Bm * Nm / mwall, "unit": "tokens/s",
            "us_per_call": round(mwall * 1e6, 2), "steps": args.mid_steps, "settle_ms": m_settle,
            "config": {"workload": "prefill_b4h8n2048d64", "batch": Bm, "heads": Hm, "seq_len": Nm, "d": dm,
                       "feature_map": "elu1", "causal": True, "normalize": True, "input_sets": 8},
            "whole_op": {"bytes": m_bytes, "achieved_gbs": round(m_bytes / mwall / 1e9, 1),
                         "useful_tflops": round(m_flops / mwall / 1e12, 2), "roof_us": round(t_roof * 1e6, 2),
                         "bound": "hbm", "frac_roof": round(t_roof / mwall, 4)},
        }
        log(f"prefill b4h8n2048d64: {mwall*1e6:.1f} us/call ({t_roof / mwall:.1%} of the roof)")
        del sets, mws
        torch.cuda.empty_cache()

    # ---------------- random features, B=2 H=8 N=16384 d=64 m=256 ----------------
    perf = None
    if not args.no_performer:
        Wf = la_inputs.WORKLOADS["performer_b2h8n16384d64m256"]
        Bf, Hf, Nf, df, mf = Wf["B"], Wf["H"], Wf["N"], Wf["d"], Wf["m"]
        gen = torch.Generator(device=dev)
        gen.manual_seed(Wf["seed"])
        shp = (Bf, Hf, Nf, df)
        fq, fk, fv = (torch.randn(shp, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
        fW = torch.from_numpy(la_inputs.performer_W(mf, df, Wf["w_seed"])).to(dev)
        fout = torch.empty_like(fq)
        fws = torch.empty(max(la.la_forward_workspace_size(Bf, Hf, Nf, df, feature_map="performer", W=fW), 256),
                          dtype=torch.uint8, device=dev)

        def ffwd(i):
            la.la_forward(fq, fk, fv, feature_map="performer", W=fW, causal=True, normalize=True, out=fout,
                          workspace=fws)

        fwall, f_settle = time_calls(ffwd, 40, args.performer_steps)
        f_ht = Bf * Hf * Nf
        f_bytes = f_ht * 4 * df * 2
        # projections of q and k (2 m d each), read-out and state update
        # (2 m d each), in-chunk scores and products ((C + 1)(m + d))
        f_flops = f_ht * (4 * mf * df + 4 * mf * df + (C + 1) * (mf + df))
        t_roof = max(f_bytes / (HBM_PEAK_GBS * 1e9), f_flops / (BF16_MFMA_PEAK_TFLOPS * 1e12))
        perf = {
            "metric": "causal random-feature linear-attn prefill tokens/s", "value": Bf * Nf / fwall,
            "unit": "tokens/s", "us_per_call": round(fwall * 1e6, 2), "steps": args.performer_steps,
            "settle_ms": f_settle,
            "config": {"workload": "performer_b2h8n16384d64m256", "batch": Bf, "heads": Hf, "seq_len": Nf,
                       "d": df, "features": mf, "feature_map": "performer", "causal": True, "normalize": True},
            "whole_op": {"bytes": f_bytes, "flops": f_flops, "achieved_gbs": round(f_bytes / fwall / 1e9, 1),
                         "useful_tflops": round(f_flops / fwall / 1e12, 2),
                         "frac_bf16_mfma": round(f_flops / fwall / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                         "roof_us": round(t_roof * 1e6, 2), "frac_roof": round(t_roof / fwall, 4)},
        }
        log(f"performer: {fwall*1e6:.1f} us/call ({t_roof / fwall:.1%} of the roof)")
        # the non-causal form on the same inputs: the state pass over every
        # segment, the total by the scan, then the read-out phi(q).S / phi(q).z
        fws_nc = torch.empty(max(la.la_forward_workspace_size(Bf, Hf, Nf, df, feature_map="performer", W=fW,
                                                              causal=False, dtype=torch.bfloat16), 256),
                             dtype=torch.uint8, device=dev)

        def ffwd_nc(i):
            la.la_forward(fq, fk, fv, feature_map="performer", W=fW, causal=False, normalize=True, out=fout,
                          workspace=fws_nc)

        fwall_nc, _ = time_calls(ffwd_nc, 40, args.performer_steps)
        # k, v read for the sums, q read and out written for the read-out;
        # projections of k and q, state update and read-out (2 m d FLOP each)
        nc_flops = f_ht * 8 * mf * df
        nc_roof = max(f_bytes / (HBM_PEAK_GBS * 1e9), nc_flops / (BF16_MFMA_PEAK_TFLOPS * 1e12))
        perf["non_causal"] = {
            "us_per_call": round(fwall_nc * 1e6, 2), "value": Bf * Nf / fwall_nc, "unit": "tokens/s",
            "workspace_bytes": int(fws_nc.numel()),
            "whole_op": {"bytes": f_bytes, "flops": nc_flops, "achieved_gbs": round(f_bytes / fwall_nc / 1e9, 1),
                         "roof_us": round(nc_roof * 1e6, 2), "frac_roof": round(nc_roof / fwall_nc, 4)}}
        log(f"performer, non-causal: {fwall_nc*1e6:.1f} us/call ({nc_roof / fwall_nc:.1%} of the roof)")
        del fq, fk, fv, fW, fout, fws, fws_nc
        torch.cuda.empty_cache()

    # ---------------- degree-2 polynomial map (d' = 1 + d + d^2) ----------------
    poly = None
    if not args.no_poly:
        Wp = la_inputs.WORKLOADS["prefill_b4h8n2048d64"]
        Bp, Hp, Np, dp = Wp["B"], Wp["H"], Wp["N"], Wp["d"]
        gen = torch.Generator(device=dev)
        gen.manual_seed(Wp["seed"])
        shp = (Bp, Hp, Np, dp)
        pq, pk, pv = ((torch.randn(shp, generator=gen, device=dev) * s_).to(torch.bfloat16)
                      for s_ in (Wp["scale"], Wp["scale"], 1.0))
        pout = torch.empty_like(pq)
        pws = torch.empty(la.la_forward_workspace_size(Bp, Hp, Np, dp, feature_map="poly2"), dtype=torch.uint8,
                          device=dev)

        def pfwd():
            la.la_forward(pq, pk, pv, feature_map="poly2", normalize=True, out=pout, workspace=pws)

        p_settle = settle_phase(pfwd, args.settle_ms_each)
        for _ in range(20):
            pfwd()
        torch.cuda.synchronize()
        log(f"poly2: timing {args.poly_steps} calls")
        t0 = time.perf_counter()
        for _ in range(args.poly_steps):
            pfwd()
        torch.cuda.synchronize()
        pwall = (time.perf_counter() - t0) / args.poly_steps
        p_ht = Bp * Hp * Np
        # dense contractions per head-token: degree-2 read-out and update (2 d^3 each),
        # degree-1 and normalizer states (8 d^2), in-chunk scores and products (2 (C+1) d)
        p_flops = p_ht * (4 * dp ** 3 + 8 * dp * dp + 2 * (C + 1) * dp)
        p_tf = p_flops / pwall / 1e12
        poly = {
            "metric": "causal prefill tokens/s, degree-2 polynomial map (d' = 1 + d + d^2)",
            "value": Bp * Np / pwall, "unit": "tokens/s", "us_per_call": round(pwall * 1e6, 1),
            "steps": args.poly_steps, "settle_ms": p_settle,
            "config": {"workload": "prefill_b4h8n2048d64", "batch": Bp, "heads": Hp, "seq_len": Np, "d": dp,
                       "feature_dim": 1 + dp + dp * dp, "feature_map": "poly2", "normalize": True},
            "mfma": {"useful_tflops": round(p_tf, 2), "frac_bf16_mfma": round(p_tf / BF16_MFMA_PEAK_TFLOPS, 4),
                     "flops_per_head_token": 4 * dp ** 3 + 8 * dp * dp + 2 * (C + 1) * dp},
        }
        log(f"poly2: {pwall*1e6:.1f} us/call, {p_tf:.1f} TFLOP/s")
        del pq, pk, pv, pout, pws
        torch.cuda.empty_cache()
    prefill_sources = ["la_prefill.hip", "la_device.h", "la_kernels.h"]
    out_traffic, out_note = read_traffic("traffic_output_pass_prefill_b1h16n65536d128.txt", prefill_sources,
                                         alg_bytes)

    # ---------------- decode ----------------
    decode = None
    if not args.no_decode:
        Wd = la_inputs.WORKLOADS["decode_s256h32d64"]
        Bd, Hd, dd, N0 = Wd["B"], Wd["H"], Wd["d"], Wd["prefill"]
        T = args.decode_steps
        log(f"decode: prefill state from {N0} tokens x {Bd*Hd} heads")
        S = torch.empty((Bd, Hd, dd, dd), dtype=torch.float32, device=dev)
        z = torch.empty((Bd, Hd, dd), dtype=torch.float32, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(Wd["prefill_seed"])
        step_b = 32
        for b0 in range(0, Bd, step_b):
            shp = (step_b, Hd, N0, dd)
            pq = torch.randn(shp, generator=gen, device=dev).to(torch.bfloat16)
            pk = torch.randn(shp, generator=gen, device=dev).to(torch.bfloat16)
            pv = torch.randn(shp, generator=gen, device=dev).to(torch.bfloat16)
            _, s_, z_ = la.la_forward(pq, pk, pv, causal=True, return_state=True)
            S[b0:b0 + step_b].copy_(s_)
            z[b0:b0 + step_b].copy_(z_)
            del pq, pk, pv
        gen.manual_seed(Wd["step_seed"])
        nsteps = T + args.decode_warmup
        shp = (nsteps, Bd, Hd, dd)
        sq = torch.randn(shp, generator=gen, device=dev).to(torch.bfloat16)
        sk = torch.randn(shp, generator=gen, device=dev).to(torch.bfloat16)
        sv = torch.randn(shp, generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((Bd, Hd, dd), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for t in range(args.decode_warmup):
            la.la_decode_step(S, z, sq[t], sk[t], sv[t], out=y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        log(f"decode: timing {T} steps")
        t0 = time.perf_counter()
        e0.record()
        for t in range(T):
            la.la_decode_step(S, z, sq[args.decode_warmup + t], sk[args.decode_warmup + t],
                              sv[args.decode_warmup + t], out=y)
        e1.record()
        torch.cuda.synchronize()
        dwall = time.perf_counter() - t0
        # average launch duration: device time of the T back-to-back launches / T
        kern_ms = np.array([e0.elapsed_time(e1) / T])
        heads = Bd * Hd
        step_bytes = heads * (2 * 4 * (dd * dd + dd) + 3 * 2 * dd + 2 * dd)
        k_ms = float(kern_ms.mean())
        d_gbs = step_bytes / (k_ms * 1e-3) / 1e9
        dec_traffic, dec_note = read_traffic("traffic_decode_step_decode_s256h32d64.txt",
                                             ["la_decode.hip", "la_device.h", "la_kernels.h"], step_bytes)
        decode = {
            "metric": "decode steps/s",
            "value": T / dwall,
            "unit": "steps/s",
            "steps": T,
            "ms_per_step": dwall * 1e3 / T,
            "config": {"workload": "decode_s256h32d64", "sequences": Bd, "heads": Hd, "d": dd,
                       "prefill_tokens": N0, "state": "fp32", "inputs": "bf16"},
            "roofline": {"bound": "hbm", "kernel": "decode_step_kernel", "achieved": round(d_gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(d_gbs / HBM_PEAK_GBS, 4),
                         "traffic": dec_traffic, "traffic_note": dec_note, "bytes_per_launch": step_bytes,
                         "avg_launch_us": round(k_ms * 1e3, 2),
                         "rate": "effective: the 136 MB state stays in the 256 MB last-level cache (MALL) from "
                                 "step to step, and the calibrated FETCH_SIZE counts those hits too; "
                                 "beyond_mall gives the rate with a live state larger than that cache"},
        }
        log(f"decode: {dwall*1e6/T:.1f} us/step wall, kernel {k_ms*1e3:.1f} us, {d_gbs:.0f} GB/s")
        # the same T steps (next tokens, same state) captured once as a HIP graph and replayed
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            graph.capture_begin()
            for t in range(T):
                la.la_decode_step(S, z, sq[args.decode_warmup + t], sk[args.decode_warmup + t],
                                  sv[args.decode_warmup + t], out=y)
            graph.capture_end()
        torch.cuda.current_stream().wait_stream(cap)
        graph.replay()  # warm replay
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - t0
        decode["graph"] = {"value": T / gwall, "unit": "steps/s", "ms_per_step": gwall * 1e3 / T,
                           "how": f"{T} steps captured as one HIP graph, one replay timed"}
        log(f"decode: graph replay {gwall*1e6/T:.1f} us/step")
        del graph
        # the same kernel with three independent state sets (409 MB, more than
        # the 256 MB last-level cache) used in turn, so that every step reads
        # and writes a state that has left that cache since its last use
        nsets = 3
        extra = [(S.clone(), z.clone()) for _ in range(nsets - 1)]
        states = [(S, z)] + extra
        torch.cuda.synchronize()
        for t in range(3 * nsets):  # warm-up on the staged tokens, reused when there are fewer
            Sx, zx = states[t % nsets]
            tt = t % (args.decode_warmup + T)
            la.la_decode_step(Sx, zx, sq[tt], sk[tt], sv[tt], out=y)
        torch.cuda.synchronize()
        e0.record()
        for t in range(T):
            Sx, zx = states[t % nsets]
            la.la_decode_step(Sx, zx, sq[args.decode_warmup + t], sk[args.decode_warmup + t],
                              sv[args.decode_warmup + t], out=y)
        e1.record()
        torch.cuda.synchronize()
        mk = e0.elapsed_time(e1) / T
        m_gbs = step_bytes / (mk * 1e-3) / 1e9
        decode["beyond_mall"] = {"state_sets": nsets, "live_state_bytes": nsets * heads * 4 * (dd * dd + dd),
                                 "avg_launch_us": round(mk * 1e3, 2), "achieved": round(m_gbs, 1),
                                 "frac": round(m_gbs / HBM_PEAK_GBS, 4),
                                 "how": f"{T} steps, step t on state set t % {nsets} (sequences of each set "
                                        "advance every third step); bytes per step as above"}
        log(f"decode: {nsets} state sets (beyond the last-level cache) {mk*1e3:.1f} us/step, {m_gbs:.0f} GB/s")
        del extra, states, sq, sk, sv, S, z, y

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        log(f"cpu baseline: oracle blockwise form, whole heads of {N} tokens, budget {args.cpu_seconds:.0f} s")
        nh, tc = 0, 0.0
        while nh < H and tc < args.cpu_seconds:
            qc, kc, vc = la_inputs.gaussian_qkv(1, 1, N, d, seed=W["seed"] + 1 + nh, scale=W["scale"], bf16=True)
            t0 = time.perf_counter()
            O.chunked(qc, kc, vc, "elu1", causal=True, normalize=True, chunk=64)
            tc += time.perf_counter() - t0
            nh += 1
        cpu = {"value": (nh * N / H) / tc, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
               "sample": f"oracle.chunked (fp64, numpy) on {nh} of {H} heads x {N} tokens, d={d}; "
                         f"tokens/s = B*N*(heads timed/H)/time", "seconds": round(tc, 2)}
        if decode is not None:
            Wd = la_inputs.WORKLOADS["decode_s256h32d64"]
            heads = Wd["B"] * Wd["H"]
            rng = np.random.default_rng(0)
            Sd = rng.standard_normal((heads, Wd["d"], Wd["d"]))
            zd = np.abs(rng.standard_normal((heads, Wd["d"]))) * 100
            nt, td = 0, 0.0
            while nt < 1000 and td < args.cpu_seconds / 2:
                tq_, tk_, tv_ = la_inputs.decode_tokens(Wd["step_seed"], nt, (heads, Wd["d"]))
                t0 = time.perf_counter()
                _, Sd, zd = O.decode_step(Sd, zd, tq_, tk_, tv_, "elu1")
                td += time.perf_counter() - t0
                nt += 1
            cpu["decode"] = {"value": nt / td, "unit": "steps/s", "seconds": round(td, 2),
                             "sample": f"oracle.decode_step (fp64, numpy) over all {heads} heads, {nt} steps"}

    result = {
        "metric": "causal linear-attn prefill tokens/s (N=64K,d=128) + decode steps/s, % roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_b1h16n65536d128", "batch": B, "heads": H, "seq_len": N, "d": d,
                   "feature_map": "elu1", "causal": True, "normalize": True, "chunk": C, "accumulate": "fp32"},
        "roofline": {"bound": "hbm", "kernel": "output_pass_kernel", "achieved": round(out_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(out_gbs / HBM_PEAK_GBS, 4),
                     "traffic": out_traffic, "traffic_note": out_note, "bytes_per_launch": alg_bytes,
                     "avg_launch_us": round(ms_out * 1e3, 2),
                     # the whole timed call (every pass, wall clock) against the same bytes
                     "whole_op_achieved": round(whole_gbs, 1), "whole_op_frac": round(whole_gbs / HBM_PEAK_GBS, 4),
                     "whole_op_us": round(ms_step * 1e3, 2)},
        "settle": settle,
        "prefill_breakdown_us": {"state_pass": round(ms_state * 1e3, 2), "carry_scan": round(ms_scan * 1e3, 2),
                                 "output_pass": round(ms_out * 1e3, 2),
                                 "first_to_last_marker": round(ms_dev * 1e3, 2),
                                 "wall_per_call": round(ms_step * 1e3, 2)},
        "prefill_whole_op": {"achieved_gbs": round(whole_gbs, 1), "frac_hbm": round(whole_gbs / HBM_PEAK_GBS, 4),
                             "useful_tflops": round(flops_useful / (ms_step * 1e-3) / 1e12, 2),
                             "frac_bf16_mfma": round(flops_useful / (ms_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                                                     4),
                             "head_tokens_per_s": head_tokens / (ms_step * 1e-3)},
        "decode": decode,
        "backward": backward,
        "gated": gated,
        "variants": variants,
        "poly2": poly,
        "prefill_b4h8n2048d64": mid,
        "performer": perf,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
