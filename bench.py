#!/usr/bin/env python3
"""Benchmark of the mHC seam block on one MI355X.

A step is one seam of the hot path over one batch of T = 16384 tokens (n = 4
streams, hidden C = 5120, fused RMSNorm, 20 Sinkhorn iterations): the post
stage of seam k and the delayed pre stage of seam k+1, in one launch,
    mhc_post_pre_delayed(y, x, post_k, comb_k, pre_k) -> x', pre, post, comb, layer_input
(one post and one pre per token and step, as in a decoder's steady state; the
sublayer output y is synthetic, attention / MoE are not part of the seam).
The same seam as two launches (mhc_post, then mhc_pre_delayed on its output) is
timed beside it.  Inputs are synthetic, seeded, and resident in HBM before the
timed region.  Prints one JSON line.

Also reported: per-kernel durations from HIP events on the launch stream, the
roofline of the dominant kernel, a microseconds-per-call sweep at T = 1..128
(graph replay and eager), the model-entry seam, and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

T_SEAM = 16384
C = 5120
NS = 4
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "mHC seam tokens/s at T=16384 + µs/call T=1..128; HBM GB/s as % of peak"
SWEEP_T = (1, 2, 4, 6, 7, 8, 16, 32, 64, 128)
S_CPU = 2048          # tokens of the seam input the CPU oracle runs (a bounded sample)
NRMSE_T = (1, 8, 64, 1024)   # token counts of the fold-accuracy measurement (layer_input NRMSE vs fp64)


def pre_bytes(T, C=C, norm=True, delayed=True):
    """Algorithmic HBM bytes of one pre call: x, layer_input, gates, pre_in, weights."""
    K = NS * C
    per_tok = K * 2 + C * 2 + (16 + 16 + 64) + (16 if delayed else 0)
    fixed = K * 24 * 4 + 24 * 4 + 3 * 4 + (C * 2 if norm else 0)
    return T * per_tok + fixed


def post_bytes(T, C=C):
    """Algorithmic HBM bytes of one post call: y, x, out, post, comb."""
    return T * (C * 2 + 2 * NS * C * 2 + 16 + 64)


def fused_bytes(T, C=C, norm=True):
    """Algorithmic HBM bytes of one fused seam: y, x and the previous gates and pre-mix in;
    the next residual, layer_input and this seam's gates out; weights once."""
    K = NS * C
    per_tok = C * 2 + K * 2 + (16 + 64 + 16) + K * 2 + C * 2 + (16 + 16 + 64)
    fixed = K * 24 * 4 + 24 * 4 + 3 * 4 + (C * 2 if norm else 0)
    return T * per_tok + fixed


def entry_bytes(T, C=C, norm=True):
    return T * (C * 2 + NS * C * 2 + C * 2 + 96) + C * 24 * 4 + 108 + (C * 2 if norm else 0)


KERNEL_SOURCES = ("decode_mhc_pre_amd/csrc/mhc_kernels.hpp", "decode_mhc_pre_amd/csrc/mhc_persist.hpp",
                  "decode_mhc_pre_amd/csrc/mhc_device.hpp", "decode_mhc_pre_amd/csrc/mhc.hip")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "seam_T16384_hbm_counters.md")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary, or None
    when the kernels changed since the counters were taken (source hash differs)."""
    try:
        with open(COUNTERS_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    src = [ln.split(":", 1)[1].strip() for ln in lines if ln.startswith("source_hash:")]
    if not src or src[0] != kernel_source_hash():
        return None
    for ln in lines:
        if ln.startswith("traffic_bytes " + kernel_key + ":"):
            return int(ln.split(":", 1)[1].strip())
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # (a hundred untimed steps: the GPU's clock settles within a few tens of ms of
    # sustained work; with five the seam measured ~15% slower)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-sweep", action="store_true", help="skip the T=1..128 sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU oracle sample time")
    ap.add_argument("--sweep-only", default=None, metavar="T,...",
                    help="only the per-call latency sweep (eager and graph replay) at these token counts")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also run one plain 512 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: measures one GPU only (--gpus 1). The seam is per-token, so more GPUs "
              "would each run the same kernels on their own share of tokens with no exchange; "
              "no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_mhc_pre_amd as M
    import mhc_inputs as mi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    if args.sweep_only:
        # decode-size latency only (e.g. for a kernel trace of the small-T kernels)
        d = mi.pre_inputs(8, seed=2, delayed=True, norm=True)
        w = M.make_weights(f32(d["fn"]), f32(d["bias"]), f32(d["alpha"]))
        Ts = tuple(int(t) for t in args.sweep_only.split(","))
        print(json.dumps({"us_per_call_sweep": run_sweep(torch, M, mi, dev, bf, f32, w, bf(d["norm_weight"]), Ts),
                          "config": {"workload": "mhc seam ops at decode sizes, n=4, C=5120, fused RMSNorm, "
                                                 "20 Sinkhorn iters", "T": list(Ts)}}), flush=True)
        return

    # ---------------------------------------------------------------- seam inputs (HBM-resident)
    t0 = time.time()
    d = mi.pre_inputs(T_SEAM, seed=2, delayed=True, norm=True, outlier_frac=0.01)
    x = bf(d["x"])
    pre_in = f32(d["pre_in"])
    nw = bf(d["norm_weight"])
    w = M.make_weights(f32(d["fn"]), f32(d["bias"]), f32(d["alpha"]))
    x_host_sample = d["x"][:S_CPU].copy()
    fn_h, bias_h, alpha_h, nw_h = d["fn"], d["bias"], d["alpha"], d["norm_weight"]
    del d
    # seam k's sublayer output and gates: y ~ N(0,1) bf16, gates from the library's own
    # pre stage on the same residual (real gates: post in (0,2), comb column-stochastic)
    y_h = mi.post_inputs(T_SEAM, seed=3)["y"]
    y = bf(y_h)
    y_host_sample = y_h[:S_CPU].copy()
    del y_h
    pre_out, post, comb, li = M._pre_outputs(T_SEAM, C, dev)
    ws = M.workspace(dev, T_SEAM, C)
    pre_k, post_k, comb_k, _ = M.mhc_pre_delayed(x, pre_in, w, nw, 1e-6, 20, ws=ws)
    x_next = torch.empty_like(x)
    torch.cuda.synchronize()
    post_k_h, comb_k_h, pre_k_h = (post_k[:S_CPU].cpu().numpy(), comb_k[:S_CPU].cpu().numpy(),
                                   pre_k[:S_CPU].cpu().numpy())
    print("inputs ready in %.1f s" % (time.time() - t0), file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        # post of seam k and delayed pre of seam k+1, one launch
        if ev is not None:
            ev[0].record(stream)
        M.mhc_post_pre_delayed(y, x, post_k, comb_k, pre_k, w, nw, 1e-6, 20,
                               out=(x_next, pre_out, post, comb, li), ws=ws)
        if ev is not None:
            ev[1].record(stream)

    def step_two(ev=None):
        # the same seam as two launches
        if ev is not None:
            ev[0].record(stream)
        M.mhc_post(y, x, post_k, comb_k, out=x_next)
        if ev is not None:
            ev[1].record(stream)
        M.mhc_pre_delayed(x_next, pre_k, w, nw, 1e-6, 20, out=(pre_out, post, comb, li), ws=ws)
        if ev is not None:
            ev[2].record(stream)

    def timed(fn, nev):
        # nev == 0: one event pair brackets the K launches on the launch stream (a
        # timing event between back-to-back launches holds the next one back, ~8 us
        # here), and the average launch duration is the bracket / K, gaps included;
        # otherwise events bracket each launch, nev per step
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(max(nev, 2))]
               for _ in range(args.steps if nev else 1)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        if nev:
            for k in range(args.steps):
                fn(evs[k])
        else:
            evs[0][0].record(stream)
            for k in range(args.steps):
                fn()
            evs[0][1].record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t_start, evs

    t_total, evs = timed(step, 0)
    # a bounded wait that ran out would make the timed outputs unspecified: stop here
    M.check_workspace(ws, clear=False)
    fused_out_h = {"x_out": x_next[:S_CPU].view(torch.int16).cpu().numpy().view(np.uint16),
                   "pre_out": pre_out[:S_CPU].cpu().numpy(), "post": post[:S_CPU].cpu().numpy(),
                   "comb": comb[:S_CPU].cpu().numpy(),
                   "li": li[:S_CPU].view(torch.int16).cpu().numpy().view(np.uint16)}
    fused_ms = [evs[0][0].elapsed_time(evs[0][1]) / args.steps]
    ms_per_step = t_total * 1e3 / args.steps
    value = T_SEAM * args.steps / t_total
    # the two-call step: its rate from one bracket around the K steps (as the fused
    # step), its per-kernel times from events around each launch in a second pass
    t_two, _ = timed(step_two, 0)
    M.check_workspace(ws, clear=False)
    _, evs2 = timed(step_two, 3)
    M.check_workspace(ws, clear=False)
    post_ms = [e[0].elapsed_time(e[1]) for e in evs2]
    pre_ms = [e[1].elapsed_time(e[2]) for e in evs2]

    fused_avg = sum(fused_ms) / len(fused_ms)
    pre_avg = sum(pre_ms) / len(pre_ms)
    post_avg = sum(post_ms) / len(post_ms)
    fb, pb, qb = fused_bytes(T_SEAM), pre_bytes(T_SEAM), post_bytes(T_SEAM)

    def kentry(avg_ms, nbytes, key):
        return dict(avg_us=avg_ms * 1e3, alg_bytes=nbytes, gbs=nbytes / (avg_ms * 1e-3) / 1e9,
                    traffic=measured_traffic(key))

    kernels = {
        "mhc_persist_kernel<5120, true, false>": kentry(fused_avg, fb, "mhc_persist_kernel<5120, true, false>"),
        "mhc_persist_kernel<5120, false, false>": kentry(pre_avg, pb, "mhc_persist_kernel<5120, false, false>"),
        "mhc_post_kernel": kentry(post_avg, qb, "mhc_post_kernel"),
    }
    for v in kernels.values():
        v["frac"] = v["gbs"] / HBM_PEAK_GBS
    # the timed step is the fused kernel alone
    dom = "mhc_persist_kernel<5120, true, false>"
    traffic = kernels[dom]["traffic"]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(kernels[dom]["gbs"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kernels[dom]["frac"], 4),
                "traffic": traffic}
    seam_gbs = fb / (t_total / args.steps) / 1e9
    two_call = {"tokens_per_s": round(T_SEAM * args.steps / t_two, 1),
                "ms_per_step": round(t_two * 1e3 / args.steps, 4),
                "alg_GBps": round((pb + qb) / (t_two / args.steps) / 1e9, 1), "launches_per_seam": 2,
                "timing": "wall time of the K steps with no events between launches; per-kernel times "
                          "from a second pass with events around each launch"}

    if args.copy_ref:
        # a plain copy kernel of known size: reads and writes 512 MiB each
        src = torch.empty(256 << 20, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    copy = copy_ceiling(torch, dev)
    copy["fused_frac_of_copy"] = round(kernels[dom]["gbs"] / copy["copy_GBps"], 4)
    ceilings = memory_ceilings(torch, dev, x, y, x_next, li, fused_avg * 1e3, pre_avg * 1e3)

    # ---------------------------------------------------------------- T = 1..128 sweep
    sweep = None
    if not args.no_sweep:
        sweep = run_sweep(torch, M, mi, dev, bf, f32, w, nw)
    entry = None if args.no_sweep else run_entry(torch, M, mi, dev, bf, f32)
    collapse = None if args.no_sweep else run_collapse(torch, M, x, pre_in, nw)
    own = None if args.no_sweep else run_own(torch, M, x, w, ws)

    del x, x_next, li, y
    torch.cuda.empty_cache()
    chain = None if args.no_sweep else run_chain(torch, M, mi, dev, bf, f32)
    other = None if args.no_sweep else run_other_sizes(torch, M, mi, dev)

    M.check_default_workspaces(clear=False)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    accuracy = None
    if not args.no_cpu:
        cpu, o_fused = cpu_baseline(y_host_sample, x_host_sample, post_k_h, comb_k_h, pre_k_h, fn_h, bias_h,
                                    alpha_h, nw_h, args.cpu_seconds)
        accuracy = oracle_accuracy(torch, M, mi, dev, bf, f32, fused_out_h, o_fused)
        M.check_default_workspaces(clear=False)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 data, fp32 accumulate, projection weight bf16 hi+lo",
        "data": "synthetic",
        "config": {"workload": "mhc seam, one launch: post of seam k + delayed pre of seam k+1 with "
                               "fused RMSNorm, T=16384, n=4, C=5120, 20 Sinkhorn iters, 1% outlier rows x100",
                   "T": T_SEAM, "hc_mult": NS, "hidden": C, "sinkhorn_iters": 20,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "accuracy": accuracy,
        "copy_ceiling": copy,
        "memory_ceilings": ceilings,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "kernel_timing": "fused step: one HIP event pair on the launch stream around the timed launches "
                         "(average = bracket / steps, gaps between launches included); two-call step: "
                         "its rate from the wall time of K uninstrumented steps, the post and pre kernel "
                         "times from a second pass with events around each launch",
        "seam_alg_GBps": round(seam_gbs, 1),
        "launches_per_seam": 1,
        "two_call_seam": two_call,
        "us_per_call_sweep": sweep,
        "entry": entry,
        "collapse": collapse,
        "pre_own": own,
        "seam_chain": chain,
        "other_hidden_sizes": other,
    }
    print(json.dumps(line), flush=True)


def _median_us(fn, torch, reps=5, iters=200):
    """Median over `reps` of the mean time of `iters` back-to-back calls (HIP events)."""
    out = []
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn(iters)
        e.record()
        e.synchronize()
        out.append(s.elapsed_time(e) * 1e3 / iters)
    return statistics.median(out)


def run_sweep(torch, M, mi, dev, bf, f32, w, nw, Ts=SWEEP_T):
    res = {}
    for T in Ts:
        d = mi.pre_inputs(T, seed=50 + T, delayed=True)
        x = bf(d["x"])
        pin = f32(d["pre_in"])
        outs = M._pre_outputs(T, C, dev)
        xo = torch.empty_like(x)
        ws = M.workspace(dev, T, C)

        def pre_call():
            M.mhc_pre_delayed(x, pin, w, nw, 1e-6, 20, out=outs, ws=ws)

        outs_own = M._pre_outputs(T, C, dev)

        def own_call():
            # the non-delayed form (own pre-mix, no norm: configuration 0's op)
            M.mhc_pre(x, w, None, 1e-6, 20, out=outs_own, ws=ws)

        def post_call():
            M.mhc_post(outs[3], x, outs[1], outs[2], out=xo)

        def seam_call():
            pre_call()
            post_call()

        fo = (torch.empty_like(x),) + tuple(M._pre_outputs(T, C, dev))

        def fused_call():
            # post of the previous seam (gates: this seam's outputs above) and the delayed pre
            M.mhc_post_pre_delayed(outs[3], x, outs[1], outs[2], pin, w, nw, 1e-6, 20, out=fo, ws=ws)

        row = {}
        for name, fn in (("pre_delayed", pre_call), ("pre_own", own_call), ("post", post_call),
                         ("seam", seam_call), ("seam_fused", fused_call)):
            fn()
            torch.cuda.synchronize()
            # eager: host launch path included
            row[name + "_eager_us"] = round(_median_us(lambda n: [fn() for _ in range(n)], torch), 2)
            # graph replay: 20 calls captured once, replayed 10x per sample
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for _ in range(20):
                        fn()
            torch.cuda.current_stream().wait_stream(s)
            g.replay()
            torch.cuda.synchronize()
            row[name + "_graph_us"] = round(_median_us(lambda n: [g.replay() for _ in range(n // 20)],
                                                       torch), 2)
            del g
        res[str(T)] = row
    return res


def run_entry(torch, M, mi, dev, bf, f32):
    res = {}
    for T in (1, 128, T_SEAM):
        d = mi.entry_inputs(T, seed=999)
        h = bf(d["h"])
        we = M.make_weights(f32(d["fn"]), f32(d["bias"]), f32(d["alpha"]))
        nw = bf(d["norm_weight"])
        ws = M.workspace(dev, T, C)
        o = M.mhc_broadcast_entry(h, we, nw, 1e-6, 20, ws=ws)
        torch.cuda.synchronize()
        us = _median_us(lambda n: [M.mhc_broadcast_entry(h, we, nw, 1e-6, 20, out=o, ws=ws)
                                   for _ in range(n)], torch, reps=3, iters=20 if T > 1024 else 100)
        res[str(T)] = {"us": round(us, 2), "alg_GBps": round(entry_bytes(T) / (us * 1e-6) / 1e9, 1)}
        del o, h
    return res


def run_collapse(torch, M, x, pin, nw):
    """The standalone collapse (exact-order collapse + folded norm) on the seam's
    residual: one kernel, T x (40,960 + 16) bytes read, T x 10,240 written."""
    T = x.shape[0]
    out = M.mhc_collapse(x, pin, nw, 1e-6)
    torch.cuda.synchronize()
    us = _median_us(lambda n: [M.mhc_collapse(x, pin, nw, 1e-6, out=out) for _ in range(n)], torch,
                    reps=3, iters=20)
    nbytes = T * (NS * C * 2 + 16 + C * 2) + C * 2
    return {"T": T, "us": round(us, 2), "alg_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def run_own(torch, M, x, w, ws):
    """mhc_pre (own pre-mix, no norm) on the seam's residual at T = 16384: the
    gates-only persistent pass, then the collapse with those gates."""
    T = x.shape[0]
    outs = M._pre_outputs(T, C, x.device)
    M.mhc_pre(x, w, None, 1e-6, 20, out=outs, ws=ws)
    torch.cuda.synchronize()
    us = _median_us(lambda n: [M.mhc_pre(x, w, None, 1e-6, 20, out=outs, ws=ws) for _ in range(n)], torch,
                    reps=3, iters=20)
    nbytes = pre_bytes(T, norm=False, delayed=False)
    return {"T": T, "us": round(us, 2), "alg_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "launches": 2}


def run_other_sizes(torch, M, mi, dev, T=T_SEAM):
    """The fused seam and the delayed pre at the other hidden sizes with a persistent
    form (C = 4096 and 7168), T = 16384: inputs drawn on the device with torch's seeded
    generator (x, y ~ N(0,1) bf16; gates: post = 2 sigmoid(N(0,1)), comb rows
    normalised uniform, pre_in uniform), weights as the seam's; algorithmic GB/s and
    the fraction of 8 TB/s per kernel."""
    res = {}
    for Cx in (4096, 7168):
        g = torch.Generator(device=dev)
        g.manual_seed(Cx)
        x = torch.randn((T, NS, Cx), generator=g, device=dev).to(torch.bfloat16)
        y = torch.randn((T, Cx), generator=g, device=dev).to(torch.bfloat16)
        post_in = 2.0 * torch.sigmoid(torch.randn((T, NS), generator=g, device=dev))
        comb_in = torch.rand((T, NS, NS), generator=g, device=dev)
        comb_in = (comb_in / comb_in.sum(dim=-1, keepdim=True)).contiguous()
        pre_in = torch.rand((T, NS), generator=g, device=dev)
        fn, bias, alpha = mi.seam_weights(Cx, NS * Cx)
        w = M.make_weights(torch.from_numpy(fn).to(dev), torch.from_numpy(bias).to(dev),
                           torch.from_numpy(alpha).to(dev))
        nw = (1.0 + 0.1 * torch.randn((Cx,), generator=g, device=dev)).to(torch.bfloat16)
        ws = M.workspace(dev, T, Cx)
        xo = torch.empty_like(x)
        outs = M._pre_outputs(T, Cx, dev)
        M.mhc_post_pre_delayed(y, x, post_in, comb_in, pre_in, w, nw, 1e-6, 20, out=(xo, *outs), ws=ws)
        torch.cuda.synchronize()
        f_us = _median_us(lambda n: [M.mhc_post_pre_delayed(y, x, post_in, comb_in, pre_in, w, nw, 1e-6, 20,
                                                             out=(xo, *outs), ws=ws) for _ in range(n)],
                          torch, reps=3, iters=20)
        d_us = _median_us(lambda n: [M.mhc_pre_delayed(x, pre_in, w, nw, 1e-6, 20, out=outs, ws=ws)
                                     for _ in range(n)], torch, reps=3, iters=20)
        M.check_workspace(ws, clear=False)
        fb, pb = fused_bytes(T, Cx), pre_bytes(T, Cx)
        res[str(Cx)] = {
            "T": T,
            "fused": {"kernel": "mhc_persist_kernel<%d, true, false>" % Cx, "us": round(f_us, 2),
                      "alg_GBps": round(fb / (f_us * 1e-6) / 1e9, 1),
                      "frac": round(fb / (f_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
            "delayed": {"kernel": "mhc_persist_kernel<%d, false, false>" % Cx, "us": round(d_us, 2),
                        "alg_GBps": round(pb / (d_us * 1e-6) / 1e9, 1),
                        "frac": round(pb / (d_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        }
        del x, y, xo, outs
        torch.cuda.empty_cache()
    return res


def run_chain(torch, M, mi, dev, bf, f32, n_seams=80):
    """Configuration 4: the model-entry seam, then 80 seams with their own weights
    (seed 1000 + k, fused norm), the sublayer an identity stand-in (y = layer_input),
    each seam one mhc_post_pre_delayed launch, and the last post.  The whole chain
    is captured once in a HIP graph and replayed; reported per T: microseconds per
    seam (chain time / 80) and the chain's time."""
    ew = mi.entry_inputs(1, seed=999)
    we = M.make_weights(f32(ew["fn"]), f32(ew["bias"]), f32(ew["alpha"]))
    nw_e = bf(ew["norm_weight"])
    seams = []
    for k in range(n_seams):
        sw = mi.sweep_seam_weights(k, C=C)
        seams.append((M.make_weights(f32(sw["fn"]), f32(sw["bias"]), f32(sw["alpha"])), bf(sw["norm_weight"])))
    res = {}
    T = 1
    while T <= T_SEAM:
        h = bf(mi.entry_inputs(T, seed=999)["h"])
        ws = M.workspace(dev, T, C)
        sets = []
        for _ in range(2):
            sets.append((torch.empty((T, NS, C), dtype=torch.bfloat16, device=dev),) +
                        tuple(M._pre_outputs(T, C, dev)))
        x_fin = torch.empty((T, NS, C), dtype=torch.bfloat16, device=dev)

        def chain():
            a = sets[0]
            M.mhc_broadcast_entry(h, we, nw_e, 1e-6, 20, out=a, ws=ws)
            for k in range(n_seams):
                b = sets[(k + 1) % 2]
                # inputs: seam k's x, layer_input, gates and pre-mix; outputs: seam k+1's
                M.mhc_post_pre_delayed(a[4], a[0], a[2], a[3], a[1], seams[k][0], seams[k][1], 1e-6, 20,
                                       out=b, ws=ws)
                a = b
            M.mhc_post(a[4], a[0], a[2], a[3], out=x_fin)

        chain()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                chain()
        torch.cuda.current_stream().wait_stream(st)
        g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            s0 = torch.cuda.Event(enable_timing=True)
            e0 = torch.cuda.Event(enable_timing=True)
            s0.record()
            g.replay()
            e0.record()
            e0.synchronize()
            times.append(s0.elapsed_time(e0))
        ms = statistics.median(times)
        res[str(T)] = {"us_per_seam": round(ms * 1e3 / n_seams, 2), "chain_ms": round(ms, 3)}
        del g, sets, x_fin, h
        torch.cuda.empty_cache()
        T *= 2
    return res


def copy_ceiling(torch, dev, nbytes=1 << 30, reps=10):
    """A streaming-copy ceiling measured in the same run: the runtime's device-to-device
    copy of 1 GiB (read + write counted), averaged over `reps` copies."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    e0 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        dst.copy_(src)
    e0.record()
    e0.synchronize()
    ms = s0.elapsed_time(e0) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"kind": "torch copy_ of 1 GiB (read + write)", "copy_GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(2 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def memory_ceilings(torch, dev, x, y, xo, li, fused_us, delayed_us, reps=10):
    """What the memory system moves with no arithmetic, measured in the same run on
    the step's own buffers (bench_ceilings.hip; xo and li are overwritten): streams of
    16-byte non-temporal reads of x, writes of xo and a copy x -> xo; the floors they
    give the fused seam's and the delayed pre's bulk bytes (reads and writes adding
    up in time, R / read rate + W / write rate; and all bytes at the copy rate); and
    the traffic of the persistent pre kernels' own access pattern replayed with no
    arithmetic or exchange (same grid, tile walk, line loads and non-temporal
    stores)."""
    import ctypes
    path = os.path.join(ROOT, "bench_ceilings.so")
    if not os.path.exists(path):
        print("bench.py: bench_ceilings.so is not built (__graft_entry__.build() builds it); "
              "memory ceilings not measured", file=sys.stderr, flush=True)
        return {"skipped": "bench_ceilings.so not built"}
    L = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.ceil_stream.argtypes = [I, P, P, Z, P, P]
    L.ceil_pattern_run.argtypes = [I, P, P, P, P, I, I, P]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    nbytes = x.numel() * x.element_size()

    def run(fn, n):
        for _ in range(3):
            fn()
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(n):
            fn()
        e0.record(stream)
        e0.synchronize()
        return s0.elapsed_time(e0) * 1e3 / n   # us per call

    def stream_rate(kind):
        def fn():
            rc = L.ceil_stream(kind, x.data_ptr(), xo.data_ptr(), nbytes, sink.data_ptr(), sp)
            if rc != 0:
                raise RuntimeError("ceil_stream(%d) returned %d" % (kind, rc))
        moved = nbytes * (2 if kind == 2 else 1)
        return moved / (run(fn, reps) * 1e-6) / 1e9

    read_gbs, write_gbs, copy_gbs = stream_rate(0), stream_rate(1), stream_rate(2)
    T = x.shape[0]
    ng = max(1, min(16, torch.cuda.get_device_properties(dev).multi_processor_count // 16, (T + 63) // 64))

    def pattern(fused):
        def fn():
            rc = L.ceil_pattern_run(int(fused), x.data_ptr(), y.data_ptr(), xo.data_ptr(), li.data_ptr(), T, ng, sp)
            if rc != 0:
                raise RuntimeError("ceil_pattern_run returned %d" % rc)
        return run(fn, 20)

    fused_pat, delayed_pat = pattern(True), pattern(False)
    torch.cuda.synchronize()
    K = NS * C
    fr, fw = T * (C * 2 + K * 2), T * (K * 2 + C * 2)    # the fused seam's bulk reads / writes
    dr, dw = T * K * 2, T * C * 2                        # the delayed pre's
    floor_f = (fr / read_gbs + fw / write_gbs) / 1e3     # us
    floor_d = (dr / read_gbs + dw / write_gbs) / 1e3
    copy_f, copy_d = (fr + fw) / copy_gbs / 1e3, (dr + dw) / copy_gbs / 1e3
    return {"kind": "16-byte non-temporal accesses over the step's residual buffers (%d MB); the pre kernels' "
                    "access pattern replayed without arithmetic or exchange (T=%d, C=%d, %d groups of 16 "
                    "workgroups)" % (nbytes // 1000000, T, C, ng),
            "read_GBps": round(read_gbs, 1), "write_GBps": round(write_gbs, 1), "copy_GBps": round(copy_gbs, 1),
            "fused_seam": {"kernel_us": round(fused_us, 1), "additive_floor_us": round(floor_f, 1),
                           "copy_rate_floor_us": round(copy_f, 1), "pattern_probe_us": round(fused_pat, 1),
                           "kernel_over_pattern": round(fused_us / fused_pat, 3)},
            "delayed_pre": {"kernel_us": round(delayed_us, 1), "additive_floor_us": round(floor_d, 1),
                            "copy_rate_floor_us": round(copy_d, 1), "pattern_probe_us": round(delayed_pat, 1),
                            "kernel_over_pattern": round(delayed_us / delayed_pat, 3)}}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(y, x, post_k, comb_k, pre_k, fn, bias, alpha, nw, target_s):
    """The oracle as it stands (C, OpenMP over tokens) on a bounded sample of the
    same seam: the post stage of seam k, then the delayed pre with fused norm.
    Timed on all host threads (the reported value) and on one thread, plus its
    microseconds per call for the decode sizes T = 1..128.  Returns the baseline
    and the oracle's result on the sample (for the accuracy figures)."""
    import oracle
    oracle.lib()
    threads = oracle.max_threads()

    def run(S):
        t = time.perf_counter()
        r = oracle.mhc_post_pre_delayed(y[:S], x[:S], post_k[:S], comb_k[:S], pre_k[:S], fn, bias, alpha, 1e-6, 20,
                                        norm_weight=nw)
        return time.perf_counter() - t, r

    S = min(len(x), S_CPU)
    run(64)  # warm-up (page in, thread pool)
    reps, dt = 0, 0.0
    res = None
    while dt < target_s and reps < 1000:
        t, res = run(S)
        dt += t
        reps += 1
    # one thread, on a smaller share of the sample (same per-token work)
    oracle.set_threads(1)
    try:
        S1 = 64
        reps1, dt1 = 0, 0.0
        while dt1 < target_s / 4 and reps1 < 100:
            dt1 += run(S1)[0]
            reps1 += 1
    finally:
        oracle.set_threads(threads)
    # microseconds per call at the decode sizes (all threads; median of 5)
    us = {}
    for T in SWEEP_T:
        ts = sorted(run(T)[0] for _ in range(5))
        us[str(T)] = round(ts[2] * 1e6, 1)
    base = {"value": round(S * reps / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d tokens of the T=16384 seam input (post, then pre_delayed+norm) x %d passes, "
                      "%.1f s; %s" % (S, reps, dt, _cpu_model()),
            "one_thread_tokens_per_s": round(S1 * reps1 / dt1, 1),
            "us_per_call": us}
    return base, res


def oracle_accuracy(torch, M, mi, dev, bf, f32, fused_h, o_fused):
    """Accuracy against the oracle's float64 evaluation (the oracle leg):
    - the benchmark's own step at T = 16384, on the first S_CPU tokens: worst
      relative error of the gates, the next residual's bits, and layer_input NRMSE;
    - the fold-accuracy measurement of the wavefront-fix PR (Measurements): the
      delayed pre with the folded RMSNorm at T = 1/8/64/1024, layer_input NRMSE
      against the exact evaluation (NRMSE = RMS(gpu - ref) / RMS(ref), with ref the
      exact value rounded once to bf16 -- the page reports 0.0 at one token, which
      only a rounded reference gives -- and, beside it, the unrounded value)."""
    import oracle

    def rel(g, o):
        g = np.asarray(g, np.float64).reshape(len(g), -1)
        o = np.asarray(o, np.float64).reshape(len(o), -1)
        return float(np.max(np.abs(g - o) / np.abs(o)))

    def nrmse(bits, exact):
        g = oracle.bf16_to_f64(bits)
        return float(np.sqrt(np.mean((g - exact) ** 2)) / np.sqrt(np.mean(exact ** 2)))

    def nrmse_rounded(bits, exact_bits):
        # against the exact value rounded once to bf16: 0.0 when every output is the
        # correctly rounded one (the page's figure is 0.0 at one token)
        return nrmse(bits, oracle.bf16_to_f64(exact_bits))

    step = {"tokens": int(len(fused_h["pre_out"])),
            "gate_max_rel_err": max(rel(fused_h["pre_out"], o_fused["pre_out"]), rel(fused_h["post"], o_fused["post"]),
                                    rel(fused_h["comb"], o_fused["comb"])),
            "x_out_bits_equal_single_precision_post": bool(np.array_equal(fused_h["x_out"], o_fused["x_out"])),
            "layer_input_nrmse_vs_rounded_exact": nrmse_rounded(fused_h["li"], o_fused["li"]),
            "layer_input_nrmse_vs_exact": nrmse(fused_h["li"], o_fused["li_val"])}
    fold = {}
    for T in NRMSE_T:
        d = mi.pre_inputs(T, seed=77 + T, delayed=True, norm=True)
        w = M.make_weights(f32(d["fn"]), f32(d["bias"]), f32(d["alpha"]))
        pre_out, post, comb, li = M.mhc_pre_delayed(bf(d["x"]), f32(d["pre_in"]), w, bf(d["norm_weight"]), 1e-6, 20)
        torch.cuda.synchronize()
        o = oracle.mhc_pre_delayed(d["x"], d["pre_in"], d["fn"], d["bias"], d["alpha"], 1e-6, 20,
                                   norm_weight=d["norm_weight"])
        lb = li.view(torch.int16).cpu().numpy().view(np.uint16)
        fold[str(T)] = {"layer_input_nrmse_vs_rounded_exact": nrmse_rounded(lb, o["li"]),
                        "layer_input_nrmse_vs_exact": nrmse(lb, o["li_val"]),
                        "gate_max_rel_err": max(rel(pre_out.cpu().numpy(), o["pre_out"]),
                                                rel(post.cpu().numpy(), o["post"]),
                                                rel(comb.cpu().numpy(), o["comb"]))}
    return {"step_T16384_sample": step, "fold_delayed_norm": fold,
            "nrmse": "RMS(gpu - ref) / RMS(ref); ref = the float64 oracle's value rounded once to bf16 "
                     "(_vs_rounded_exact, the page's figure) or unrounded (_vs_exact, which includes the "
                     "output's own bf16 rounding)"}


if __name__ == "__main__":
    main()
