#!/usr/bin/env python3
"""Benchmark of the dequant-on-use MoE path on one MI355X.

Default workload ("layer64"): one full MoE block decoding 64 ragged tokens
(the GLM-5.2 MoE block: hidden 6144, 256 int4 experts of intermediate 2048,
top-8 sigmoid noaux_tc router with routed_scaling_factor 2.5, one int4 shared
expert).  A step is one coli_moe_layer call: router, device-side expert
grouping, fused gate/up + SwiGLU, down, shared expert and the weighted
combine.  Two copies of the expert bank live in HBM and steps alternate
between them, so no step finds its weights in the 256 MB last-level cache.

Other workloads: "decode16" (coli_moe_gemv, 16 tokens, given top-8 routing),
"qgemv" (int4 12288 x 6144, S = 1, over a rotation of weight copies),
"prefill2048" (2048 tokens, Zipf routing, bf16 matrix cores, router timed), "copy"
(a plain 1 GiB device copy, the yardstick for the HBM byte counters).

Prints ONE JSON line.  `value` is the step's algorithmic bytes (weights of
the experts actually used, scales, router, activations, outputs) divided by
the step time, in GB/s; tokens/s and the share of the 8 TB/s HBM peak are
reported beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 matrix peak
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 matrix peak (TOP/s)
METRIC = "int4 expert-GEMV HBM GB/s (% of peak) + MoE-layer decode tokens/s"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def expert_bytes(fmt, D, F, gs=0):
    """Bytes of one expert's gate+up and down matrices with their scales
    (one per row, or with gs > 0 one per gs elements of a row)."""
    from weight_streaming_gemv_qgemv_amd import synth
    rbD, rbF = synth.packed_row_bytes(fmt, D), synth.packed_row_bytes(fmt, F)
    sD, sF = (-(-D // gs), -(-F // gs)) if gs else (1, 1)
    gate_up = 2 * F * rbD + 2 * F * sD * 4
    down = D * rbF + D * sF * 4
    return gate_up, down


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bank_to_dev(bank, dev):
    out = dict(bank)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = to_dev(bank[k], dev)
    return out


def apply_layout(args, banks, shared=None, D=6144):
    """The expert banks (and shared experts) in the layout asked for: with
    --layout tiled each is repacked once on the device (coli_pack_tiled, a
    load-time step outside the timed region) and the row-major copy freed."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    if getattr(args, "layout", "rows") != "tiled":
        return banks, shared
    banks = [b.tile_mlps(bk) for bk in banks]
    if shared is not None:
        shared = [b.tile_mlps(sh, D) for sh in shared]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return banks, shared


def clone_bank(bd):
    out = dict(bd)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = bd[k].clone()
    return out


def source_hash(files):
    """sha256 over the named kernel sources (repository-relative), in order."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), f), "rb").read())
    return h.hexdigest()


def profile_record(fname, tag, workload):
    """The machine-readable line `tag: {json}` of a committed rocprofv3
    summary under profiles/, or None when the file or line is missing, it is
    for another workload, or the kernel sources it names have changed since
    the profile was taken (sha256 over them)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", fname)
    try:
        line = next(l for l in open(path) if l.startswith(tag + ": "))
        rec = json.loads(line[len(tag) + 2:])
        if rec.get("workload") != workload or source_hash(rec["sources"]) != rec.get("sha256"):
            return None
    except (OSError, StopIteration, ValueError, KeyError, TypeError):
        return None
    return rec


PROFILE_FILES = {"moe_layer_decode_64": ("moe_layer_decode64_kernels.md", "moe_layer_decode64_traffic.md"),
                 "moe_layer_prefill_2048_bf16": ("moe_layer_prefill2048_kernels.md",
                                                 "moe_layer_prefill2048_traffic.md")}


def recorded_traffic(workload, kernel_key):
    """HBM bytes per launch of one kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain
    copy), or None when there is none for this workload or the kernel sources
    have changed since the counters were taken."""
    if workload not in PROFILE_FILES:
        return None
    rec = profile_record(PROFILE_FILES[workload][1], "traffic-json", workload)
    k = rec.get("per_launch", {}).get(kernel_key) if rec else None
    return None if k is None else int(k["fetch_bytes"] + k["write_bytes"])


def recorded_trace_ms(workload, kernel_key):
    """Average duration (ms) of one kernel in the committed rocprofv3 kernel
    trace of this workload (the same bench command), or None as above."""
    if workload not in PROFILE_FILES:
        return None
    rec = profile_record(PROFILE_FILES[workload][0], "trace-json", workload)
    k = rec.get("avg_us", {}).get(kernel_key) if rec else None
    return None if k is None else k * 1e-3


def kernel_key(name, args):
    """rocprofv3's name of the int4 gate/up kernel (k_dec, k_pre) for the
    layout in use and its group-scale variant: 0, or the 32-element steps per
    group, 8 for every group of 256 or more."""
    tiled = 'true' if getattr(args, 'layout', 'rows') == 'tiled' else 'false'
    gs = getattr(args, "grouped", 0)
    return f"{name}<2, 2, {tiled}, {min(gs // 32, 8) if gs else 0}>"


def trace_roofline(dom, units_per_launch, peak):
    """The roofline fraction implied by the committed rocprofv3 trace's
    average duration of the dominant kernel (None when that trace is stale or
    missing), beside the live event-based one."""
    t = dom.get("trace_ms")
    if not t:
        return None
    ach = units_per_launch / (t * 1e-3)
    return {"ms_per_launch": round(t, 5), "achieved": round(ach, 2), "frac": round(ach / peak, 4),
            "event_over_trace": round(dom["ms_per_launch"] / t, 4) if dom["ms_per_launch"] else None}


REPS = 20


RAMP_S = 0.25


def clock_ramp(step, seconds):
    """Untimed steps, back to back, for `seconds` of wall time before the
    warm-up: after the host-side setup the GPU starts from a low clock, and
    the first tens of milliseconds of work run ~9% slower.  Returns the steps
    it ran."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_steps(step, steps, warmup, reps=REPS):
    """Warm up, then time exactly `steps` steps between two synchronisations
    (stage events off): the reported step time.  Then `reps` more blocks of
    `steps` steps, each between its own event pair, give the median and the
    minimum step time over repetitions.  A last pass of `steps` steps records
    a HIP event pair around every stage on the stream the kernels run on; it
    gives the per-kernel durations used for the roofline and the stage
    breakdown."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    ramp_steps = clock_ramp(step, RAMP_S)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    n = warmup + steps
    for r in range(reps):
        for i in range(steps):
            step(n)
            n += 1
        ev[r + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[r].elapsed_time(ev[r + 1]) / steps for r in range(reps))
    rep_stats = dict(reps=reps, steps_per_rep=steps, ms_per_step_median=float(np.median(per)),
                     ms_per_step_min=per[0], ms_per_step_max=per[-1],
                     clock_ramp_s=RAMP_S, clock_ramp_steps=ramp_steps)
    b.stage_times(reset=True)
    b.stage_timing(True)
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(steps):
        step(n + i)
    s1.record()
    torch.cuda.synchronize()
    b.stage_timing(False)
    stages = b.stage_times(reset=True)
    stages["_step_ms_with_stage_events"] = (s0.elapsed_time(s1), steps)
    stages["_reps"] = rep_stats
    return ms, wall, stages


def cpu_baseline_layer(bank, shared, Wr, bias, x, K, ntok, runs=1):
    """The oracle as it stands, on the first `ntok` tokens of the same input:
    the median wall time over `runs` runs (clock_gettime through
    time.perf_counter), and the routing it took."""
    from oracle import oracle
    xs = x[:ntok]
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        r = oracle.router(Wr, bias, xs, K, 1, 2.5)
        oracle.moe(bank, shared, xs, r["idx"], r["w"])
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), r["idx"]


def host_info():
    """Logical CPUs this process may use and the CPU model string."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def single_thread(fn):
    """Run fn() with the oracle on one host thread; returns (seconds, result)."""
    from oracle import oracle
    prev = oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        out = fn()
        return time.perf_counter() - t0, out
    finally:
        oracle.set_threads(prev)


def run_tail64(args, dev):
    """The 64-token decode layer as a layer tail: RMSNorm of the residual
    stream, the MoE block on the normalised rows, residual add
    (coli_moe_layer_tail)."""
    return run_layer64(args, dev, tail=True)


def run_layer64(args, dev, tail=False):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    from weight_streaming_gemv_qgemv_amd import synth
    S, K, E, D, F, fmt = 64, 8, 256, 6144, 2048, 2
    gs = args.grouped
    log("generating 256 int4 experts + shared expert (host)" + (f", one scale per {gs} elements" if gs else ""))
    bank = synth.expert_bank(4000, fmt, E, D, F, gs=gs)
    shared = synth.shared_mlp(4000, fmt, D, F, gs=gs)
    g = synth.rng(4001)
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    log("uploading")
    banks = [bank_to_dev(bank, dev)]
    banks.append(clone_bank(banks[0]))
    sd = [bank_to_dev(shared, dev)]
    sd.append(clone_bank(sd[0]))
    banks, sd = apply_layout(args, banks, sd, D)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    xd = to_dev(x, dev)
    out = torch.empty((S, D), dtype=torch.float32, device=dev)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    w_o = torch.empty((S, K), dtype=torch.float32, device=dev)
    ws = b.alloc_workspace(b.moe_workspace_bytes(S, K, E, D, F, F), dev)
    nw = to_dev(synth.rng(4002).uniform(0.5, 1.5, size=D).astype(np.float32), dev)

    def step(i):
        j = i & 1
        if tail:
            b.moe_layer_tail(rp, banks[j], sd[j], xd, nw, 1e-5, out=out, idx_out=idx_o, w_out=w_o, ws=ws)
        else:
            b.moe_layer(rp, banks[j], sd[j], xd, out=out, idx_out=idx_o, w_out=w_o, ws=ws)

    step(0)
    torch.cuda.synchronize()
    uniq = int(np.unique(idx_o.cpu().numpy()).size)
    gu, dn = expert_bytes(fmt, D, F, gs)
    step_bytes = (E * D * 4 + E * 4) + S * D * 4 + uniq * (gu + dn) + (gu + dn) + S * D * 4 + S * K * 8
    if tail:
        step_bytes += D * 4 + S * D * 4      # the norm weight, and x read again for the residual
    log(f"unique experts {uniq}; algorithmic bytes/step {step_bytes / 1e9:.4f} GB")
    ms, wall, stages = time_steps(step, args.steps, args.warmup)
    # dominant kernel: gate/up + SwiGLU (2/3 of the expert bytes), one launch per step
    gu_ms, gu_n = stages["gate_up"]
    gu_bytes = (uniq + 1) * gu + S * D * 4 + (S * K + S) * F * 4
    wl = ("moe_layer_tail_decode_64" if tail else "moe_layer_decode_64") + (f"_g{gs}" if gs else "")
    res = dict(workload=wl, ms=ms, wall=wall,
               step_bytes=step_bytes,
               tokens=S, stages=stages, uniq=uniq,
               dominant=dict(kernel="k_dec<I4,2> (grouped expert gate/up + SwiGLU, matrix cores)",
                             bytes_per_launch=gu_bytes, ms_per_launch=gu_ms / max(gu_n, 1),
                             launches=gu_n,
                             traffic=recorded_traffic(wl, kernel_key("k_dec", args)),
                             trace_ms=recorded_trace_ms(wl, kernel_key("k_dec", args))))
    if gs:
        res["weight_format"] = f"int4 grouped scales (one per {gs} elements)"
    if not args.no_cpu_baseline and not tail:
        ntok = args.cpu_tokens
        log(f"cpu baseline: oracle on {ntok} tokens")
        dt, sidx = cpu_baseline_layer(bank, shared, Wr, bias, x, K, ntok, runs=args.cpu_runs)
        su = int(np.unique(sidx).size)
        sb = (E * D * 4 + E * 4) + ntok * D * 4 + su * (gu + dn) + (gu + dn) + ntok * D * 4
        from oracle import oracle
        res["cpu"] = dict(value=sb / dt / 1e9, unit="GB/s", cores=oracle.num_threads(),
                          kind="oracle",
                          sample=f"router + MoE layer on the first {ntok} of the 64 tokens "
                                 f"({su} unique experts), median of {args.cpu_runs} runs, {dt:.2f} s each",
                          tokens_per_s=ntok / dt, seconds=dt)
        n1 = min(args.cpu_tokens_1t, ntok)
        if n1 > 0:
            log(f"cpu baseline: oracle on {n1} tokens, one thread")
            _, (dt1, idx1) = single_thread(lambda: cpu_baseline_layer(bank, shared, Wr, bias, x, K, n1,
                                                                      runs=3))
            u1 = int(np.unique(idx1).size)
            sb1 = (E * D * 4 + E * 4) + n1 * D * 4 + u1 * (gu + dn) + (gu + dn) + n1 * D * 4
            res["cpu"]["single_thread"] = dict(
                value=sb1 / dt1 / 1e9, tokens_per_s=n1 / dt1, seconds=dt1,
                sample=f"router + MoE layer on the first {n1} tokens ({u1} unique experts), median of 3 runs")
    return res


def per_expert_roofline_s(rows_per_expert, expert_bytes_total, D, F):
    """The prefill layer's bound: every expert (the shared one last) streams
    its weights once and multiplies them into its rows, so it takes at least
    max(bytes / HBM peak, flops / bf16 matrix peak); the layer at least the
    sum over experts (the router and the activations are left out)."""
    t = 0.0
    for r in rows_per_expert:
        if r <= 0:
            continue
        t += max(expert_bytes_total / (HBM_PEAK_GBS * 1e9), 2.0 * r * 3 * D * F / (BF16_PEAK_TFLOPS * 1e12))
    return t


def run_prefill2048(args, dev):
    """2048 tokens through the layer in bf16 precision: the router runs and
    is timed (coli_router), the experts take a fixed Zipf(1.1)-skewed
    routing through pre_idx / pre_w."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    from weight_streaming_gemv_qgemv_amd import synth
    S, K, E, D, F, fmt = 2048, 8, 256, 6144, 2048, 2
    gs = args.grouped
    log("generating 256 int4 experts + shared expert (host)" + (f", one scale per {gs} elements" if gs else ""))
    bank = synth.expert_bank(4000, fmt, E, D, F, gs=gs)
    shared = synth.shared_mlp(4000, fmt, D, F, gs=gs)
    g = synth.rng(4500)
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    bd, sd = bank_to_dev(bank, dev), bank_to_dev(shared, dev)
    (bd,), (sd,) = apply_layout(args, [bd], [sd], D)
    xd, idd, wd = to_dev(x, dev), to_dev(idx, dev), to_dev(w, dev)
    Wrd, bd_bias = to_dev(Wr, dev), to_dev(bias, dev)
    out = torch.empty((S, D), dtype=torch.float32, device=dev)
    rws = b.alloc_workspace(b.router_workspace_bytes(S, E, D), dev)
    prec = 2 if args.idot else 1
    ws = b.alloc_workspace(b.moe_workspace_bytes(S, K, E, D, F, F, prec), dev)

    def step(i):
        b.router(Wrd, bd_bias, xd, K, 1, 2.5, 0.0, ws=rws)
        b.moe_layer(None, bd, sd, xd, pre_idx=idd, pre_w=wd, out=out, prec=prec, ws=ws)

    uniq = int(np.unique(idx).size)
    gu, dn = expert_bytes(fmt, D, F, gs)
    step_bytes = (E * D * 4 + E * 4) + S * D * 4 + uniq * (gu + dn) + (gu + dn) + S * D * 4 + S * K * 8
    rows = S * K + S
    flops = 2 * rows * 3 * D * F            # gate, up, down on every routed and shared row
    t_star = per_expert_roofline_s(np.bincount(idx.ravel(), minlength=E).tolist() + [S], gu + dn, D, F)
    ms, wall, stages = time_steps(step, args.steps, args.warmup)
    gu_ms, gu_n = stages["gate_up"]
    gu_flops = 2 * rows * 2 * D * F
    if args.idot:
        # int8 activations on the int8 matrix cores: ops counted as the flops
        # of the same products, against the int8 dense peak
        return dict(workload="moe_layer_prefill_2048_idot", ms=ms, wall=wall, step_bytes=step_bytes,
                    tokens=S, stages=stages, uniq=uniq, flops=flops, t_star=t_star, idot=True,
                    dominant=dict(kernel="k_preid<I4,2> (grouped expert gate/up + SwiGLU, int8 matrix cores)",
                                  traffic=None, trace_ms=None,
                                  bytes_per_launch=(uniq + 1) * gu + S * D + rows * F * 4,
                                  flops_per_launch=gu_flops, ms_per_launch=gu_ms / max(gu_n, 1),
                                  launches=gu_n))
    if gs:
        return dict(workload=f"moe_layer_prefill_2048_g{gs}_bf16", ms=ms, wall=wall, step_bytes=step_bytes,
                    tokens=S, stages=stages, uniq=uniq, flops=flops, t_star=t_star,
                    weight_format=f"int4 grouped scales (one per {gs} elements)",
                    dominant=dict(kernel="k_pre<I4,2,SPG> (grouped-scale gate/up + SwiGLU, bf16 matrix cores)",
                                  traffic=None, trace_ms=None,
                                  bytes_per_launch=(uniq + 1) * gu + S * D * 4 + rows * F * 4,
                                  flops_per_launch=gu_flops, ms_per_launch=gu_ms / max(gu_n, 1),
                                  launches=gu_n))
    return dict(workload="moe_layer_prefill_2048_bf16", ms=ms, wall=wall, step_bytes=step_bytes,
                tokens=S, stages=stages, uniq=uniq, flops=flops, t_star=t_star,
                dominant=dict(kernel="k_pre<I4,2> (grouped expert gate/up + SwiGLU, bf16 matrix cores)",
                              traffic=recorded_traffic("moe_layer_prefill_2048_bf16", kernel_key("k_pre", args)),
                              trace_ms=recorded_trace_ms("moe_layer_prefill_2048_bf16", kernel_key("k_pre", args)),
                              bytes_per_launch=(uniq + 1) * gu + S * D * 4 + rows * F * 4,
                              flops_per_launch=gu_flops, ms_per_launch=gu_ms / max(gu_n, 1),
                              launches=gu_n))


def run_ep_slice(args, dev, prefill):
    """One GPU's share of the MoE block under expert parallelism over
    `args.ep_slice` GPUs (256 / N experts each): the router (replicated, so
    every GPU runs it), the local experts' grouped gate/up, SwiGLU and down
    on the rows routed to them, and the shared expert.  The slice timed is
    the one with the most routed rows, and it also holds the shared expert:
    the step time of the slowest GPU.  The all-gather of x before and the
    sum-reduction of the partial outputs after are not part of the step.
    Routing: the router's own output on the synthetic rows (decode, 64
    tokens) or the Zipf(1.1) routing of the prefill workload (2048 tokens,
    bf16 matrix cores), remapped to local ids, other slots -1 (empty)."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    from weight_streaming_gemv_qgemv_amd import synth
    N = args.ep_slice
    K, E, D, F, fmt = 8, 256, 6144, 2048, 2
    if E % N:
        raise SystemExit(f"--ep-slice {N}: 256 experts do not split evenly")
    El = E // N
    S = 2048 if prefill else 64
    g = synth.rng(4500 if prefill else 4001)
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    Wrd, biasd, xd = to_dev(Wr, dev), to_dev(bias, dev), to_dev(x, dev)
    rws = b.alloc_workspace(b.router_workspace_bytes(S, E, D), dev)
    if prefill:
        idx, w = synth.routing_zipf(g, S, K, E)
    else:
        r = b.router(Wrd, biasd, xd, K, 1, 2.5, 0.0, ws=rws)
        torch.cuda.synchronize()
        idx, w = r["idx"].cpu().numpy(), r["w"].cpu().numpy()
    rows_per_slice = np.bincount(idx.ravel() // El, minlength=N)
    gsl = int(np.argmax(rows_per_slice))
    lo = gsl * El
    local = (idx >= lo) & (idx < lo + El)
    idl = np.where(local, idx - lo, -1).astype(np.int32)
    wl = np.where(local, w, 0.0).astype(np.float32)
    log(f"slice {gsl} of {N}: experts {lo}..{lo + El - 1}, {int(local.sum())} routed rows "
        f"(per slice: {rows_per_slice.tolist()})")
    bank = synth.expert_bank(4000, fmt, E, D, F, experts=range(lo, lo + El))
    bank["E"] = El
    shared = synth.shared_mlp(4000, fmt, D, F)
    banks = [bank_to_dev(bank, dev)]
    banks.append(clone_bank(banks[0]))
    sd = [bank_to_dev(shared, dev)]
    sd.append(clone_bank(sd[0]))
    banks, sd = apply_layout(args, banks, sd, D)
    idd, wd = to_dev(idl, dev), to_dev(wl, dev)
    prec = 1 if prefill else 0
    out = torch.empty((S, D), dtype=torch.float32, device=dev)
    ws = b.alloc_workspace(b.moe_workspace_bytes(S, K, El, D, F, F, prec), dev)

    def step(i):
        j = i & 1
        b.router(Wrd, biasd, xd, K, 1, 2.5, 0.0, ws=rws)
        b.moe_layer(None, banks[j], sd[j], xd, pre_idx=idd, pre_w=wd, out=out, prec=prec, ws=ws)

    uniq = int(np.unique(idl[idl >= 0]).size)
    gu, dn = expert_bytes(fmt, D, F)
    nrows = int(local.sum())
    step_bytes = (E * D * 4 + E * 4) + S * D * 4 + uniq * (gu + dn) + (gu + dn) + S * D * 4 + S * K * 8
    ms, wall, stages = time_steps(step, args.steps, args.warmup)
    gu_ms, gu_n = stages["gate_up"]
    rows = nrows + S
    res = dict(workload=f"ep{N}_slice_{'prefill_2048_bf16' if prefill else 'decode_64'}", ms=ms,
               wall=wall, step_bytes=step_bytes, tokens=S, stages=stages, uniq=uniq,
               experts=El, ep=dict(gpus=N, slice=gsl, routed_rows=nrows,
                                   rows_per_slice=rows_per_slice.tolist(), shared_expert_here=True),
               dominant=dict(kernel=f"{'k_pre' if prefill else 'k_dec'}<I4,2> (grouped expert gate/up + SwiGLU)",
                             bytes_per_launch=(uniq + 1) * gu + S * D * 4 + rows * F * 4,
                             ms_per_launch=gu_ms / max(gu_n, 1), launches=gu_n))
    if prefill:
        res["flops"] = 2 * rows * 3 * D * F
        res["dominant"]["flops_per_launch"] = 2 * rows * 2 * D * F
        res["t_star"] = per_expert_roofline_s(np.bincount(idl[idl >= 0].ravel(), minlength=El).tolist() + [S],
                                              gu + dn, D, F)
    return res


def run_decode16(args, dev):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    from weight_streaming_gemv_qgemv_amd import synth
    S, K, E, D, F, fmt = 16, 8, 256, 6144, 2048, 2
    bank = synth.expert_bank(4100, fmt, E, D, F)
    g = synth.rng(4101)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_uniform(g, S, K, E)
    banks = [bank_to_dev(bank, dev)]
    banks.append(clone_bank(banks[0]))
    banks, _ = apply_layout(args, banks)
    xd, idd, wd = to_dev(x, dev), to_dev(idx, dev), to_dev(w, dev)
    out = torch.empty((S, D), dtype=torch.float32, device=dev)
    ws = b.alloc_workspace(b.moe_workspace_bytes(S, K, E, D, F), dev)

    def step(i):
        b.moe_gemv(banks[i & 1], xd, idd, wd, out=out, ws=ws)

    uniq = int(np.unique(idx).size)
    gu, dn = expert_bytes(fmt, D, F)
    step_bytes = S * D * 4 + uniq * (gu + dn) + S * D * 4 + S * K * 8
    ms, wall, stages = time_steps(step, args.steps, args.warmup)
    gu_ms, gu_n = stages["gate_up"]
    res = dict(workload="moe_expert_decode_16", ms=ms, wall=wall, step_bytes=step_bytes,
               tokens=S, stages=stages, uniq=uniq,
               dominant=dict(kernel="k_dec<I4,2> (grouped expert gate/up + SwiGLU, matrix cores)",
                             bytes_per_launch=uniq * gu + S * D * 4 + S * K * F * 4,
                             ms_per_launch=gu_ms / max(gu_n, 1), launches=gu_n))
    if not args.no_cpu_baseline:
        from oracle import oracle
        n = min(args.cpu_tokens, S)
        run = lambda m: oracle.moe(bank, None, x[:m], idx[:m], w[:m].astype(np.float64))
        t0 = time.perf_counter()
        run(n)
        dt = time.perf_counter() - t0
        su = int(np.unique(idx[:n]).size)
        res["cpu"] = dict(value=(n * D * 8 + su * (gu + dn)) / dt / 1e9, unit="GB/s",
                          cores=oracle.num_threads(), kind="oracle",
                          sample=f"routed experts for the first {n} of {S} tokens ({su} unique "
                                 f"experts), {dt:.2f} s", tokens_per_s=n / dt, seconds=dt)
        n1 = min(args.cpu_tokens_1t, n)
        if n1 > 0:
            dt1, _ = single_thread(lambda: run(n1))
            u1 = int(np.unique(idx[:n1]).size)
            res["cpu"]["single_thread"] = dict(
                value=(n1 * D * 8 + u1 * (gu + dn)) / dt1 / 1e9, tokens_per_s=n1 / dt1,
                seconds=dt1, sample=f"routed experts for the first {n1} tokens ({u1} unique experts)")
    return res


def run_qgemv(args, dev):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    from weight_streaming_gemv_qgemv_amd import synth
    fmt = {"f32": 0, "i8": 1, "i4": 2, "i2": 3}[args.fmt]
    O, I = (int(v) for v in getattr(args, "shape", "12288x6144").lower().split("x"))
    S = args.tokens
    g = synth.rng(4200, fmt)
    W = synth.weight_bytes(g, fmt, O, I)
    sc = synth.scales(g, O)
    x = synth.activations(g, S, I)
    Wd0 = to_dev(W, dev)
    ncopy = max(2, -(-(1 << 30) // W.nbytes))                  # a rotation of >= 1 GiB
    copies = [Wd0] + [Wd0.clone() for _ in range(ncopy - 1)]
    scd, xd = to_dev(sc, dev), to_dev(x, dev)
    y = torch.empty((S, O), dtype=torch.float32, device=dev)
    idot = getattr(args, "idot", False)
    gs = getattr(args, "grouped", 0)
    if gs:
        if fmt != 2 or idot:
            raise SystemExit("--grouped takes --fmt i4 (and not --idot)")
        sc = synth.scales(g, O * (-(-I // gs))).reshape(O, -1)
        scd = to_dev(sc, dev)
    if idot:
        if fmt not in (1, 2):
            raise SystemExit("--idot takes --fmt i8 or i4")
        wsq = b.alloc_workspace(b.qgemv_idot_workspace_bytes(S, I), dev)

    def step(i):
        if idot:
            b.qgemv_idot(fmt, copies[i % len(copies)], scd, xd, y, ws=wsq)
        elif gs:
            b.qgemv_grouped(copies[i % len(copies)], scd, gs, xd, y)
        else:
            b.qgemv(fmt, copies[i % len(copies)], scd, xd, y)

    step_bytes = O * W.shape[1] + sc.nbytes + S * I * 4 + S * O * 4
    ms, wall, stages = time_steps(step, args.steps, args.warmup)
    q_ms, q_n = stages["qgemv"]
    var = "_idot" if idot else f"_g{gs}" if gs else ""
    entry = "coli_qgemv_idot" if idot else "coli_qgemv_grouped" if gs else "coli_qgemv"
    name = f"qgemv{var}_{args.fmt}_{O}x{I}_s{S}"
    wf = {0: "fp32", 1: "int8 per-row scale", 2: "int4 per-row scale", 3: "int2 per-row scale"}[fmt]
    if idot:
        wf += ", int8 activations (integer dot)"
    if gs:
        wf = f"int4 one scale per {gs} elements"
    return dict(workload=name, ms=ms, wall=wall, step_bytes=step_bytes, weight_format=wf,
                tokens=S, stages=stages, uniq=None, O=O, I=I,
                dominant=dict(kernel=f"qgemv {args.fmt} ({entry})",
                              bytes_per_launch=step_bytes,
                              ms_per_launch=q_ms / max(q_n, 1), launches=q_n))


def run_copy(args, dev):
    """A plain 1 GiB device-to-device copy of known size: the yardstick that
    converts the FETCH_SIZE / WRITE_SIZE counters into bytes."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    c = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        c.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "copy_1GiB", "bytes_read_per_copy": n,
                      "bytes_written_per_copy": n, "copies": args.steps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="layer64",
                    choices=["layer64", "tail64", "decode16", "qgemv", "prefill2048", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fmt", default="i4", choices=["f32", "i8", "i4", "i2"], help="qgemv workload")
    ap.add_argument("--tokens", type=int, default=1, help="qgemv workload: S")
    ap.add_argument("--shape", default="12288x6144", metavar="OxI",
                    help="qgemv workload: output rows x input width (512x1024: the small, "
                         "L2-resident case, timed over a >= 1 GiB rotation of weight copies)")
    ap.add_argument("--idot", action="store_true",
                    help="qgemv and prefill2048 workloads: the integer-dot (int8 activation) variant")
    ap.add_argument("--grouped", type=int, default=0, metavar="GS",
                    help="qgemv, layer64, tail64 and prefill2048 workloads: grouped-scale int4, one "
                         "scale per GS elements (the MoE workloads: tiled layout)")
    ap.add_argument("--ep-slice", type=int, default=0, metavar="N",
                    help="layer64 / prefill2048: time one GPU's share under expert parallelism "
                         "over N GPUs (256/N local experts; the slice with the most routed rows, "
                         "with the shared expert)")
    ap.add_argument("--layout", default="tiled", choices=["rows", "tiled"],
                    help="expert weight layout: the tiled copy the library reads fastest "
                         "(coli_pack_tiled, made once at load time, outside the timed steps), "
                         "or the pages' row-major rows as given")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--cpu-tokens-1t", type=int, default=4,
                    help="tokens of the one-thread oracle timing (0 skips it)")
    ap.add_argument("--cpu-runs", type=int, default=5,
                    help="runs of the oracle timing; the median is reported")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build measures the per-GPU share of the "
              f"MoE block; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    from weight_streaming_gemv_qgemv_amd import binding as b
    b.lib()
    if args.idot and args.workload not in ("qgemv", "prefill2048"):
        raise SystemExit("--idot applies to the qgemv and prefill2048 workloads")
    if args.idot and args.workload == "prefill2048" and (args.layout != "tiled" or args.ep_slice):
        raise SystemExit("prefill2048 --idot runs on the tiled layout, without --ep-slice")
    if args.grouped and args.workload not in ("qgemv", "layer64", "tail64", "prefill2048"):
        raise SystemExit("--grouped applies to the qgemv, layer64, tail64 and prefill2048 workloads")
    if args.grouped and args.workload != "qgemv" and (args.layout != "tiled" or args.ep_slice or args.idot):
        raise SystemExit("grouped experts run on the tiled layout, without --ep-slice or --idot")
    if args.workload == "copy":
        run_copy(args, dev)
        return
    run = {"prefill2048": run_prefill2048, "layer64": run_layer64, "tail64": run_tail64,
           "decode16": run_decode16, "qgemv": run_qgemv}[args.workload]
    if args.ep_slice:
        if args.workload not in ("layer64", "prefill2048"):
            raise SystemExit("--ep-slice applies to the layer64 and prefill2048 workloads")
        r = run_ep_slice(args, dev, args.workload == "prefill2048")
    else:
        r = run(args, dev)
    ms = r["ms"]
    gbs = r["step_bytes"] / (ms * 1e-3) / 1e9
    dom = r["dominant"]
    ach = dom["bytes_per_launch"] / (dom["ms_per_launch"] * 1e-3) / 1e9 if dom["ms_per_launch"] else None
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp32 (vector ALUs, fp32 weights)" if r.get("weight_format") == "fp32" else
                  f"fp32 activations as bf16 hi+lo pairs on the bf16 matrix cores, fp32 accumulate "
                  f"({r.get('weight_format', 'int4').split()[0]} weights as exact bf16 codes)"),
        "data": "synthetic",
        "config": ({"workload": r["workload"], "tokens_per_step": r["tokens"],
                    "experts": r.get("experts", 256),
                    "unique_experts_per_step": r["uniq"], "hidden": 6144,
                    "moe_inter": 2048, "top_k": 8,
                    "weight_format": r.get("weight_format", "int4 per-row scale"),
                    "algorithmic_bytes_per_step": r["step_bytes"]} if r["uniq"] is not None else
                   {"workload": r["workload"], "tokens_per_step": r["tokens"],
                    "out_rows": r["O"], "in_width": r["I"],
                    "weight_format": r.get("weight_format", "int4 per-row scale"),
                    "algorithmic_bytes_per_step": r["step_bytes"]}),
        "tokens_per_s": round(r["tokens"] / (ms * 1e-3), 1),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "stage_ms_per_step": {k: round(v[0] / max(v[1], 1), 5) for k, v in r["stages"].items()
                              if not k.startswith("_reps") and v[1]},
        "timing": {k: (round(v, 5) if isinstance(v, float) else v) for k, v in r["stages"]["_reps"].items()},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2) if ach else None,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4) if ach else None,
                     "traffic": dom.get("traffic"), "kernel": dom["kernel"],
                     "algorithmic_bytes_per_launch": dom["bytes_per_launch"],
                     "ms_per_launch": round(dom["ms_per_launch"], 5),
                     "trace": trace_roofline(dom, dom["bytes_per_launch"] / 1e9, HBM_PEAK_GBS)},
        "context": {"pages_metal_moe_gemv_GBps": "358-389 (Apple-Silicon GPU, unified memory)"},
    }
    if "ep" in r:
        line["config"]["expert_parallel_share"] = r["ep"]
    if r["uniq"] is not None:
        line["config"]["weight_layout"] = args.layout
    if "flops" in r:
        # prefill: the matrix cores bound the dominant kernel
        tf = dom["flops_per_launch"] / (dom["ms_per_launch"] * 1e-3) / 1e12 if dom["ms_per_launch"] else None
        peak = INT8_PEAK_TOPS if r.get("idot") else BF16_PEAK_TFLOPS
        line["dtype"] = ("int8 activations (per-row absmax/127) x int4 weights, exact int32 dot, "
                         "fp32 epilogue" if r.get("idot") else
                         "bf16 (grouped-scale int4 weights, fp32 accumulate per group)" if "weight_format" in r else
                         "bf16 (int4 weights, fp32 accumulate)")
        line["roofline"] = {"bound": "mfma", "achieved": round(tf, 2) if tf else None,
                            "peak": peak, "unit": "TOP/s" if r.get("idot") else "TFLOP/s",
                            "frac": round(tf / peak, 4) if tf else None,
                            "traffic": dom.get("traffic"),
                            "kernel": dom["kernel"], "flops_per_launch": dom["flops_per_launch"],
                            "ms_per_launch": round(dom["ms_per_launch"], 5),
                            "trace": trace_roofline(dom, dom["flops_per_launch"] / 1e12, peak)}
        line["layer_mfma_utilisation"] = round(r["flops"] / (ms * 1e-3) / 1e12 / peak, 4)
        if "t_star" in r:
            line["per_expert_roofline"] = {"t_star_ms": round(r["t_star"] * 1e3, 5),
                                           "frac_of_step": round(r["t_star"] * 1e3 / ms, 4)}
    if "cpu" in r:
        c = r["cpu"]
        nproc, model = host_info()
        line["cpu_baseline"] = {"value": round(c["value"], 4), "unit": c["unit"], "cores": c["cores"],
                                "kind": c["kind"], "sample": c["sample"],
                                "tokens_per_s": round(c["tokens_per_s"], 3),
                                "nproc": nproc, "cpu_model": model}
        if "single_thread" in c:
            st = c["single_thread"]
            line["cpu_baseline"]["single_thread"] = {
                "value": round(st["value"], 4), "unit": c["unit"], "cores": 1,
                "tokens_per_s": round(st["tokens_per_s"], 3), "sample": st["sample"],
                "seconds": round(st["seconds"], 2)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
