#!/usr/bin/env python3
"""Benchmark of DualKV shared-prompt attention, forward + backward, on one MI355X.

One step is the whole hot path on one batch: Call 1 forward (dkv_ctx_fwd), Call 2
forward (dkv_fwd), Call 1 backward (dkv_ctx_bwd, clearing the shared fp32
accumulator) and Call 2 backward (dkv_bwd, adding the responses' terms and casting
dK_P/dV_P once).  Inputs are seeded synthetic tensors already resident in HBM.

Reported value: useful TFLOP/s = 14 * d * Hq * (visible pairs of both calls) / step
time (4*d per pair forward, 10*d backward; masked work is not counted).  Also
reported: the fraction of the bf16 MFMA peak, the speedup over the same library's
causal kernel run on the N-copy packing (eq. (1)/(2) of the DualKV paper), the
roofline of the dominant kernel (timed live with HIP events on its stream), and the
CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b")
    ap.add_argument("--no-ncopy", action="store_true", help="skip the N-copy comparator")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split", action="store_true",
                    help="sum the shared-prompt gradient through per-chunk slices and a "
                         "fixed-order reduction (DKV_ACC_SPLIT) instead of fp32 atomics")
    ap.add_argument("--dtype", choices=["bf16", "fp16"], default=None,
                    help="run a 16-bit workload in this element type instead of its own "
                         "(fp16: the precision of the paper's kernel benchmark)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--layout", action="store_true",
                    help="time the layout conversions (dkv_layout: N-copy <-> single-prompt "
                         "packing and first-token rows) on the workload's token layout "
                         "instead of the attention step")
    ap.add_argument("--hidden", type=int, default=4096,
                    help="elements per token row for --layout (Qwen3-8B hidden size)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (torch), the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    ap.add_argument("--graph", action="store_true",
                    help="also capture the step (both calls, forward and backward) into a "
                         "HIP graph once and time the same number of replays")
    ap.add_argument("--gemm-calibration", action="store_true",
                    help="also time a plain bf16 8192^3 matrix product (torch / hipBLASLt) "
                         "and report its TFLOP/s beside the published peak")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_algo_work(w, P, lens, pairs):
    """Algorithmic work per kernel class for one step: (amount, unit, bound).  P is the
    number of prompt rows (all groups' prompts)."""
    d, Hq, Hkv = w.d, w.Hq, w.Hkv
    T = P + sum(lens)                   # query rows over both calls
    eb = 4 if w.dtype == "fp32" else 2
    return {
        # forward: Q K^T and P V on every visible pair
        "attn_fwd": (4 * d * Hq * pairs, "flop", "mfma"),
        # dQ kernel: recomputes S and dP, then dS K
        "bwd_dq": (6 * d * Hq * pairs, "flop", "mfma"),
        # dK/dV kernel: recomputes S and dP, then P^T dO and dS^T Q
        "bwd_dkdv": (8 * d * Hq * pairs, "flop", "mfma"),
        # D = rowsum(dO * O): read O and dO, write one fp32 per row
        "bwd_pre": (T * Hq * (2 * d * eb + 4), "byte", "hbm"),
        # clear the two fp32 accumulators
        "acc_zero": (2 * P * Hkv * d * 4, "byte", "hbm"),
        # read the two fp32 accumulators, write dK_P, dV_P
        "acc_cast": (2 * P * Hkv * d * (4 + eb), "byte", "hbm"),
    }


def traffic_for(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec.get("sources", []):
        path = os.path.join(ROOT, f)
        if not os.path.exists(path):   # a source since renamed or removed: stale
            return None
        h.update(open(path, "rb").read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(args):
    """A plain copy of known size: 1 GiB read, 1 GiB written.  Under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE readings give the counters' scale factor."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(args, "copy calibration: %d bytes read, %d bytes written" % (4 << 28, 4 << 28))
    del src, dst


def gemm_calibration(args):
    """TFLOP/s of a plain bf16 8192^3 matrix product through torch (hipBLASLt): what a
    tuned dense contraction reaches on this GPU under sustained load, beside the
    published peak (context only; the roofline uses the published peak)."""
    import torch
    n = 8192
    g = torch.Generator(device="cuda:0").manual_seed(0)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
    log(args, "gemm calibration: bf16 %d^3 in %.3f ms = %.1f TFLOP/s" % (n, ms, tf))
    del a, b
    return round(tf, 1)


def layout_main(args):
    """One step = the five layout conversions of one micro-batch: UNPACK and PACK of a
    hidden-state tensor, UNPACK_BWD of its gradient, and the first-token GATHER and
    SCATTER, each on rows of --hidden bf16 elements.  Algorithmic bytes per op: every
    distinct input row read once plus every output row written once."""
    import torch
    import workloads
    from shared_prompt_exact_dkv_amd import _lib
    import shared_prompt_exact_dkv_amd as dkv

    dev = "cuda:0"
    w = workloads.WORKLOADS[args.workload]
    shapes = w.group_shapes()
    cu, ccu, scu = [0], [0], [0]
    for Pj, ls in shapes:
        ccu.append(ccu[-1] + Pj)
        scu.append(scu[-1] + len(ls))
        for r in ls:
            cu.append(cu[-1] + r)
    P, T, N = ccu[-1], cu[-1], len(cu) - 1
    gkw = dict(ctx_cu_host=ccu, group_seq_cu_host=scu) if w.groups > 1 else {}
    nrows = lambda op: dkv.layout_rows(op, cu, P, ccu if gkw else None, scu if gkw else None)
    H, eb = args.hidden, 2
    g = torch.Generator(device=dev).manual_seed(w.seed)
    ops = [dkv.DKV_UNPACK, dkv.DKV_PACK, dkv.DKV_UNPACK_BWD, dkv.DKV_FIRST_TOKEN_GATHER,
           dkv.DKV_FIRST_TOKEN_SCATTER]
    names = {dkv.DKV_UNPACK: "unpack", dkv.DKV_PACK: "pack", dkv.DKV_UNPACK_BWD: "unpack_bwd",
             dkv.DKV_FIRST_TOKEN_GATHER: "first_token_gather",
             dkv.DKV_FIRST_TOKEN_SCATTER: "first_token_scatter"}
    ncopy = nrows(dkv.DKV_UNPACK)[1]
    # distinct input rows read + output rows written, per op
    rows_moved = {dkv.DKV_UNPACK: (P + T) + ncopy, dkv.DKV_PACK: 2 * (P + T),
                  dkv.DKV_UNPACK_BWD: ncopy + (P + T), dkv.DKV_FIRST_TOKEN_GATHER: 2 * T,
                  dkv.DKV_FIRST_TOKEN_SCATTER: T + (P + T)}
    bufs = {}
    for op in ops:
        ri, ro = nrows(op)
        bufs[op] = (torch.randn((ri, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16),
                    torch.empty((ro, H), dtype=torch.bfloat16, device=dev))
    wsz = max(_lib.lib().dkv_layout_workspace_size(
        _lib.make_params(num_seqs=N, ctx_len=P, num_heads_q=1, num_heads_kv=1, head_dim=64,
                         cu_host=cu, **({"ctx_cu_host": ccu, "group_seq_cu_host": scu} if gkw else {}))[0], op)
        for op in ops)
    ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)

    def step():
        for op in ops:
            dkv.dkv_layout(op, bufs[op][0], cu, P, out=bufs[op][1], workspace=ws, **gkw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.lib().dkv_timing_reset()
    _lib.lib().dkv_timing_enable(1)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    _lib.lib().dkv_timing_enable(0)
    # per-op durations: one timed launch per op per step, in op order
    per_op = {}
    for op in ops:
        _lib.lib().dkv_timing_reset()
        _lib.lib().dkv_timing_enable(1)
        for _ in range(args.steps):
            dkv.dkv_layout(op, bufs[op][0], cu, P, out=bufs[op][1], workspace=ws, **gkw)
        _lib.lib().dkv_timing_enable(0)
        tot, n = _lib.timing_read()["layout"]
        per_op[op] = tot / n
    _lib.lib().dkv_timing_reset()
    if args.copy_calibration:
        copy_calibration(args)
    total_bytes = sum(rows_moved[op] * H * eb for op in ops)
    gbs = total_bytes / (ms * 1e-3) / 1e9
    dom = max(ops, key=lambda op: per_op[op])
    dom_gbs = rows_moved[dom] * H * eb / (per_op[dom] * 1e-3) / 1e9
    out = {
        "metric": "DualKV layout conversions GB/s (% HBM peak)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "P": P, "N": N, "T_R": T, "groups": len(shapes),
                   "row_elems": H, "ops": [names[op] for op in ops]},
        "pct_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "kernels": {names[op]: {"ms": round(per_op[op], 4),
                                "GB/s": round(rows_moved[op] * H * eb / (per_op[op] * 1e-3) / 1e9, 1)}
                    for op in ops},
        "roofline": {"kernel": "layout:" + names[dom], "bound": "hbm", "achieved": round(dom_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(dom_gbs / PEAK_HBM_GBS, 4),
                     "traffic": None, "avg_launch_ms": round(per_op[dom], 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from shared_prompt_exact_dkv_amd import accounting, _lib
    import shared_prompt_exact_dkv_amd as dkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.layout:
        return layout_main(args)
    dev = "cuda:0"
    w = workloads.WORKLOADS[args.workload]
    if args.dtype is not None:
        if w.dtype == "fp32":
            print("--dtype applies to the 16-bit workloads only", file=sys.stderr)
            sys.exit(2)
        import dataclasses
        w = dataclasses.replace(w, dtype=args.dtype)
    Hq, Hkv, d, wl = w.Hq, w.Hkv, w.d, w.window_left
    tdt = workloads.torch_dtype(w.dtype)
    log(args, "workload", w)

    # Prompt groups [(P_j, response lengths)]: one group unless the workload packs
    # several prompts into the micro-batch (then every call gets the group arrays).
    shapes = w.group_shapes()
    gkw = {}
    if w.groups > 1:
        _, x = workloads.make_group_inputs(shapes, Hq, Hkv, d, w.dtype, seed=w.seed,
                                           scaled=w.scaled, device=dev)
        cu_p_host = [int(c) for c in x.pop("ctx_cu")]
        gkw = dict(ctx_cu_host=cu_p_host, group_seq_cu_host=[int(c) for c in x.pop("seq_cu")])
    else:
        x = workloads.make_inputs(shapes[0][0], shapes[0][1], Hq, Hkv, d, w.dtype, seed=w.seed,
                                  scaled=w.scaled, device=dev)
        cu_p_host = [0, shapes[0][0]]
    lens = [r for _, ls in shapes for r in ls]
    N, P = len(lens), cu_p_host[-1]
    x = {k: (v.to(tdt).contiguous() if k != "cu" else v) for k, v in x.items()}
    cu_host = [int(c) for c in x["cu"]]
    cu = x["cu"].to(dev)
    cu_p = torch.tensor(cu_p_host, dtype=torch.int32, device=dev)
    T = cu_host[-1]

    # Preallocated outputs, accumulator and one workspace for every call.
    o_p = torch.empty_like(x["q_p"])
    o_r = torch.empty_like(x["q_r"])
    lse_p = torch.empty((Hq, P), dtype=torch.float32, device=dev)
    lse_r = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    dq_p = torch.empty_like(x["q_p"])
    dq_r = torch.empty_like(x["q_r"])
    dk_r = torch.empty_like(x["k_r"])
    dv_r = torch.empty_like(x["v_r"])
    dk_p = torch.empty_like(x["k_p"])
    dv_p = torch.empty_like(x["v_p"])
    acc = torch.empty((2, P, Hkv, d), dtype=torch.float32, device=dev)
    wsz = max(dkv.dkv_workspace_size(c, x["q_r"], x["k_r"], cu, cu_host=cu_host, ctx_len=P,
                                     window_left=wl, **gkw) for c in (1, 3, 4 if args.split else 3))
    wsz = max(wsz, max(dkv.dkv_workspace_size(c, x["q_p"], x["k_p"], cu_p, cu_host=cu_p_host,
                                              window_left=wl) for c in (0, 2)))
    ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)

    bwd_flags = dkv.DKV_ACC_FINALIZE | (dkv.DKV_ACC_SPLIT if args.split else 0)

    def dk_step():
        dkv.dkv_ctx_fwd(x["q_p"], x["k_p"], x["v_p"], cu_p, cu_host=cu_p_host, window_left=wl,
                        out=o_p, lse=lse_p, workspace=ws)
        dkv.dkv_fwd(x["q_r"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], cu, cu_host=cu_host,
                    window_left=wl, out=o_r, lse=lse_r, workspace=ws, **gkw)
        dkv.dkv_ctx_bwd(x["q_p"], x["k_p"], x["v_p"], o_p, lse_p, x["do_p"], cu_p,
                        cu_host=cu_p_host, window_left=wl, dq=dq_p, acc_dk=acc[0],
                        acc_dv=acc[1], acc_flags=dkv.DKV_ACC_ZERO, workspace=ws)
        dkv.dkv_bwd(x["q_r"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], o_r, lse_r, x["do_r"], cu,
                    acc_dk_p=acc[0], acc_dv_p=acc[1], acc_flags=bwd_flags,
                    cu_host=cu_host, window_left=wl, dq_r=dq_r, dk_r=dk_r, dv_r=dv_r,
                    dk_p=dk_p, dv_p=dv_p, workspace=ws, **gkw)

    def timed(step, k):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(k):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / k

    for _ in range(args.warmup):
        dk_step()
    torch.cuda.synchronize()
    _lib.lib().dkv_timing_reset()
    _lib.lib().dkv_timing_enable(1)
    ms = timed(dk_step, args.steps)
    _lib.lib().dkv_timing_enable(0)
    ktimes = _lib.timing_read()
    _lib.lib().dkv_timing_reset()
    log(args, "dualkv ms/step %.3f" % ms, ktimes)

    # The same step replayed from a HIP graph (no host work per step: the calls' work
    # lists and launches are captured once).
    graph_ms = None
    if args.graph:
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            dk_step()
        torch.cuda.synchronize()
        graph.replay()
        graph_ms = timed(graph.replay, args.steps)
        log(args, "graph replay ms/step %.3f" % graph_ms)
        del graph

    # Per-call breakdown, from a separate pass with events between the four calls (the
    # timed region above has none): the time of Call 1 and Call 2 against their own
    # visible pairs.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    call_names = ("ctx_fwd", "fwd", "ctx_bwd", "bwd")
    call_ms = dict.fromkeys(call_names, 0.0)
    n_call_steps = max(2, min(args.steps, 5))
    for _ in range(n_call_steps):
        ev[0].record()
        dkv.dkv_ctx_fwd(x["q_p"], x["k_p"], x["v_p"], cu_p, cu_host=cu_p_host, window_left=wl,
                        out=o_p, lse=lse_p, workspace=ws)
        ev[1].record()
        dkv.dkv_fwd(x["q_r"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], cu, cu_host=cu_host,
                    window_left=wl, out=o_r, lse=lse_r, workspace=ws, **gkw)
        ev[2].record()
        dkv.dkv_ctx_bwd(x["q_p"], x["k_p"], x["v_p"], o_p, lse_p, x["do_p"], cu_p,
                        cu_host=cu_p_host, window_left=wl, dq=dq_p, acc_dk=acc[0],
                        acc_dv=acc[1], acc_flags=dkv.DKV_ACC_ZERO, workspace=ws)
        ev[3].record()
        dkv.dkv_bwd(x["q_r"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], o_r, lse_r, x["do_r"], cu,
                    acc_dk_p=acc[0], acc_dv_p=acc[1], acc_flags=bwd_flags,
                    cu_host=cu_host, window_left=wl, dq_r=dq_r, dk_r=dk_r, dv_r=dv_r,
                    dk_p=dk_p, dv_p=dv_p, workspace=ws, **gkw)
        ev[4].record()
        torch.cuda.synchronize()
        for i, c in enumerate(call_names):
            call_ms[c] += ev[i].elapsed_time(ev[i + 1]) / n_call_steps
    pairs_c1 = sum(accounting.pairs_call1(Pj, wl) for Pj, _ in shapes)
    pairs_c2 = sum(accounting.pairs_call2(Pj, ls, wl) for Pj, ls in shapes)
    call_pairs = {"ctx_fwd": pairs_c1, "fwd": pairs_c2, "ctx_bwd": pairs_c1, "bwd": pairs_c2}
    calls = {}
    for c in call_names:
        fl = accounting.useful_flops(call_pairs[c], Hq, d, fwd=c.endswith("fwd"),
                                     bwd=c.endswith("bwd"))
        calls[c] = {"ms": round(call_ms[c], 4), "pairs_per_head": call_pairs[c],
                    # picoseconds per visible (row, key) pair of one q-head
                    "ps_per_pair": round(call_ms[c] * 1e9 / max(1, call_pairs[c] * Hq), 4),
                    "tflops": round(fl / max(call_ms[c], 1e-9) / 1e9, 2)}
    log(args, "calls", calls)

    pairs = sum(accounting.pairs_dualkv(Pj, ls, wl) for Pj, ls in shapes)
    pairs_nc = sum(accounting.pairs_ncopy(Pj, ls, wl) for Pj, ls in shapes)
    flops = accounting.useful_flops(pairs, Hq, d)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_FP32_TFLOPS if w.dtype == "fp32" else PEAK_BF16_TFLOPS   # fp16 = bf16 peak

    # Fwd/bwd split of the step (per call classes), from the live kernel times.
    fwd_ms = ktimes.get("attn_fwd", (0.0, 0))[0] / args.steps
    bwd_ms = sum(v[0] for k, v in ktimes.items() if k != "attn_fwd") / args.steps

    # Roofline of the dominant kernel class.
    algo = kernel_algo_work(w, P, lens, pairs)
    dom = max(ktimes, key=lambda k: ktimes[k][0]) if ktimes else None
    roof = None
    if dom is not None:
        tot_ms, launches = ktimes[dom]
        amount, unit, bound = algo[dom]
        per_launch = amount * args.steps / launches
        avg_s = tot_ms * 1e-3 / launches
        if unit == "flop":
            achieved = per_launch / avg_s / 1e12
            pk, un = peak, "TFLOP/s"
        else:
            achieved = per_launch / avg_s / 1e9
            pk, un = PEAK_HBM_GBS, "GB/s"
        roof = {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": pk,
                "unit": un, "frac": round(achieved / pk, 4),
                "traffic": traffic_for(dom, w.name), "avg_launch_ms": round(tot_ms / launches, 4),
                "launches_per_step": launches // args.steps}
    # Every kernel class's rate on its own algorithmic work (same live timings as the
    # roofline above), so the dQ and forward kernels' fractions sit beside the dominant one.
    kernels = {}
    for k, v in ktimes.items():
        rec = {"ms_per_step": round(v[0] / args.steps, 4), "launches_per_step": v[1] // args.steps}
        if k in algo and v[0] > 0:
            amount, unit, _ = algo[k]
            per_s = amount * args.steps / (v[0] * 1e-3)
            if unit == "flop":
                rec["tflops"] = round(per_s / 1e12, 2)
                rec["frac"] = round(per_s / 1e12 / peak, 4)
            else:
                rec["gbs"] = round(per_s / 1e9, 1)
                rec["frac"] = round(per_s / 1e9 / PEAK_HBM_GBS, 4)
        kernels[k] = rec

    # N-copy comparator: the same library's causal kernel over N sequences [P, R_i].
    ncopy_ms = None
    if not args.no_ncopy:
        # copy i: its group's prompt rows, then its own response rows
        grp = [j for j, (_, ls) in enumerate(shapes) for _ in ls]
        copy = lambda n, i: (x[n + "_p"][cu_p_host[grp[i]]:cu_p_host[grp[i] + 1]],
                             x[n + "_r"][cu_host[i]:cu_host[i + 1]])
        qn = torch.cat([t for i in range(N) for t in copy("q", i)])
        kn = torch.cat([t for i in range(N) for t in copy("k", i)])
        vn = torch.cat([t for i in range(N) for t in copy("v", i)])
        don = torch.cat([t for i in range(N) for t in copy("do", i)])
        cun_host = [0]
        for i, r in enumerate(lens):
            cun_host.append(cun_host[-1] + shapes[grp[i]][0] + r)
        cun = torch.tensor(cun_host, dtype=torch.int32, device=dev)
        on = torch.empty_like(qn)
        lsen = torch.empty((Hq, cun_host[-1]), dtype=torch.float32, device=dev)
        dqn = torch.empty_like(qn)
        dkn = torch.empty_like(kn)
        dvn = torch.empty_like(vn)
        wsn_sz = max(dkv.dkv_workspace_size(c, qn, kn, cun, cu_host=cun_host, window_left=wl)
                     for c in (0, 2))
        wsn = torch.empty(max(wsn_sz, 256), dtype=torch.uint8, device=dev)

        def nc_step():
            dkv.dkv_ctx_fwd(qn, kn, vn, cun, cu_host=cun_host, window_left=wl, out=on, lse=lsen,
                            workspace=wsn)
            dkv.dkv_ctx_bwd(qn, kn, vn, on, lsen, don, cun, cu_host=cun_host, window_left=wl,
                            dq=dqn, dk=dkn, dv=dvn, workspace=wsn)

        for _ in range(max(1, args.warmup // 2)):
            nc_step()
        ncopy_ms = timed(nc_step, max(2, args.steps // 2))
        log(args, "ncopy ms/step %.3f" % ncopy_ms)
        del qn, kn, vn, don, on, dqn, dkn, dvn, wsn
        torch.cuda.empty_cache()

    # CPU oracle on a bounded sample: the N-copy fwd+bwd of sequence 1 for two kv-head
    # groups (about 10-20 s on the host), extrapolated to the whole workload by
    # visible-pair count.  value: the metric's useful work (DualKV's visible pairs) over
    # the time the oracle takes to produce the same outputs (the full N-copy problem,
    # extrapolated); sample_tflops: the oracle's own rate on the work it did.
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        P0 = shapes[0][0]
        S0 = P0 + lens[0]
        G = Hq // Hkv
        ng = min(2, Hkv)
        xs = workloads.make_inputs(P0, [lens[0]], ng * G, ng, d, w.dtype, seed=w.seed + 100,
                                   scaled=w.scaled)
        q0, k0, v0 = oracle.copy_of(xs, 0)
        do0 = torch.cat([xs["do_p"], xs["do_r"]]).double().numpy()
        t0 = time.perf_counter()
        oracle.seq_fwd(q0, k0, v0, window_left=wl)
        t1 = time.perf_counter()
        oracle.seq_bwd(q0, k0, v0, do0, window_left=wl)
        t2 = time.perf_counter()
        fwd_s, bwd_s, cpu_s = t1 - t0, t2 - t1, t2 - t0
        sample_pairs = accounting.causal_pairs(S0, wl)
        scale_up = pairs_nc / sample_pairs * Hkv / ng
        full_s = cpu_s * scale_up
        sample_flops = accounting.useful_flops(sample_pairs, ng * G, d)
        cpu = {"value": round(flops / full_s / 1e12, 6), "unit": "TFLOP/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "affinity_cpus": len(os.sched_getaffinity(0)),
               "fwd_s": round(fwd_s, 3), "bwd_s": round(bwd_s, 3),
               "sample_tflops": round(sample_flops / cpu_s / 1e12, 6),
               "extrapolated_fwd_s": round(fwd_s * scale_up, 1),
               "extrapolated_bwd_s": round(bwd_s * scale_up, 1),
               "sample": "N-copy fwd+bwd (eq. 2, fp64) of sequence 1 (%d tokens) for %d of %d "
                         "kv-head groups (%d q-heads): fwd %.1f s + bwd %.1f s with %d OpenMP "
                         "threads (%d CPUs in the affinity mask); extrapolated by visible-pair "
                         "count to the full N-copy workload (%.0f s); value = the workload's "
                         "useful FLOPs over that time"
                         % (S0, ng, Hkv, ng * G, fwd_s, bwd_s, oracle.num_threads(),
                            len(os.sched_getaffinity(0)), full_s)}
        log(args, "cpu oracle sample %.2f s" % cpu_s)

    if args.copy_calibration:
        copy_calibration(args)
    gemm = gemm_calibration(args) if args.gemm_calibration else None

    speedup = (ncopy_ms / ms) if ncopy_ms else None
    out = {
        "metric": "DualKV fwd+bwd TFLOP/s (% MFMA peak); speedup vs N-copy causal attn",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name,
                   "P": P if w.groups == 1 else [Pj for Pj, _ in shapes], "N": N,
                   "groups": w.groups,
                   "R": w.R if w.R is not None else "U%s" % (list(w.R_range),),
                   "Hq": Hq, "Hkv": Hkv, "d": d, "window_left": wl,
                   "prompt_grad_sum": "split" if args.split else "atomic",
                   "parallelism": "single-gpu"},
        "pct_mfma_peak": round(100.0 * tflops / peak, 2),
        "speedup_vs_ncopy": round(speedup, 3) if speedup else None,
        "ideal_speedup": round(pairs_nc / pairs, 3),
        "ncopy_ms_per_step": round(ncopy_ms, 4) if ncopy_ms else None,
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "useful_tflop_per_step": round(flops / 1e12, 4),
        "kernels": kernels,
        "calls": calls,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if gemm is not None:
        out["gemm_calibration_tflops"] = gemm
    if graph_ms is not None:
        out["graph"] = {"ms_per_step": round(graph_ms, 4),
                        "tflops": round(flops / (graph_ms * 1e-3) / 1e12, 3)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
