"""Benchmark of the MoGA forward hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--path P] [--no-cpu-baseline]

A step is one pass of the whole path over one synthetic batch already resident
in HBM: route -> permute -> gated group attention (-> STGA sum for workloads
that have it).  --path picks how attention meets the permutation (default
fused_vtq: sort + K gather + V gathered transposed per head, attention reading
each query row through perm, with the gated unpermute in its epilogue;
fused_vt: the same with a gathered Q copy; fused_epilogue: as fused_vt with V
in row layout; gather_on_load: sort only, attention reads Q/K/V rows
through perm and writes the gated output in place; separate: gather,
attention, unpermute).
Prints ONE JSON line.

value = effective TFLOP/s of the whole step, counting only within-group
attention FLOPs 4*H*D*sum_g n_g^2 (plus the STGA windows when present);
tokens_per_s = N / step time.  The roofline object covers the dominant kernel
(the gated group attention), timed live with HIP events on the stream it runs
on.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "MoGA attn effective TFLOP/s + tokens/s per layer at N≈190k, %MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_group_attention_clip30s_122f.json")
ATTN_SOURCE = os.path.join(ROOT, "sparse_attention_long_router_amd", "csrc", "attention.hip")


def make_parser():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--path", default="fused_vtq",
                    choices=["fused_vtq", "fused_vt", "fused_epilogue", "gather_on_load", "separate"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--no-staged-backward", action="store_true",
                    help="time the attention backward with the minimum workspace only (dS not kept)")
    ap.add_argument("--cpu-rows", type=int, default=2000, help="sampled query rows per group for the oracle")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (reference for HBM byte counters)")
    return ap


def parse():
    return make_parser().parse_args()


def calibrate_copy(mib):
    """Plain device-to-device copies of a known size: the reference the
    FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)


def copy_rate_gbs(stream, mib=1024, reps=5):
    """Read + write bytes per second of a plain device-to-device copy (the
    practical ceiling of a streaming kernel), timed with HIP events."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    rate = 2.0 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return rate


def attn_flops(counts, H, D):
    return 4.0 * H * D * float(sum(int(c) ** 2 for c in counts))


def source_hash(path):
    """Hash of a C++ source with its comments and blank space removed, so that
    a change to comments alone does not disown counters taken on the same
    code (string literals in these kernels hold no comment markers)."""
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def traffic_entry(kernel, workload):
    """HBM bytes per attention launch from the committed counter summary, or
    None when it covers another kernel or workload, or the kernel source
    changed after the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel") != kernel or t.get("workload") != workload:
        return None
    if t.get("attention_source_sha256_16") != source_hash(ATTN_SOURCE):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp, wl, counts, rows_per_group):
    """The oracle, untuned, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    from workloads.gen import sample_rows, to_numpy_f32
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([int(i.get("num_threads", 1)) for i in info] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api', '?')} ({i.get('threading_layer', '?')})"
                                 for i in info if i.get("user_api") == "blas"})) or blas
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
    except (OSError, StopIteration):
        pass

    X, Wr, Q, K, V = (to_numpy_f32(inp[k]) for k in ("X", "Wr", "Q", "K", "V"))
    t0 = time.perf_counter()
    g, gate, _ = oracle.route(X, Wr)
    perm, cu, _ = oracle.permute(g, wl.M)
    t_route = time.perf_counter() - t0
    # sampled attention rows: first/last plus random rows of every group, all heads
    rows = sample_rows(g, wl.M, rows_per_group, seed=wl.seed)
    t1 = time.perf_counter()
    oracle.moga_output_rows(X, Wr, Q, K, V, wl.M, rows, routed=(g, gate))
    t_attn = time.perf_counter() - t1
    n = np.bincount(g, minlength=wl.M)
    sample_flops = 4.0 * wl.H * wl.D * float(sum(n[g[r]] for r in rows))
    total_flops = attn_flops(counts, wl.H, wl.D)
    t_full = t_route + t_attn * total_flops / sample_flops
    return {
        "value": total_flops / t_full / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"route + permute over all {wl.N} tokens ({t_route:.2f} s); attention of {rows.size} "
                   f"sampled query rows (first, last and {rows_per_group} random per group) x {wl.H} heads "
                   f"({t_attn:.2f} s, {sample_flops / 1e9:.1f} GFLOP), extrapolated by FLOPs to the full step "
                   f"({t_full:.1f} s; the sample is bounded so that the default run finishes in about a minute); "
                   f"float64 NumPy on {blas}, {threads} BLAS threads, "
                   f"{len(os.sched_getaffinity(0))} cores visible, {cpu}"),
    }


def backward_timing(moga, wl, X, Wr, Q, K, V, flops_fwd, steps, staged=True):
    """The training backward of the MoGA layer (unpermute, attention and
    router backward) on the same inputs, after a training forward.  The
    attention's algorithmic work is 2.5x the forward's (five n^2 D products
    per group and head: S, dP, dV, dQ, dK).  With `staged`, the attention
    backward gets a workspace that keeps dS (five products computed instead
    of seven) for every head, or for as many heads as free device memory
    holds with 8 GiB to spare; the minimum-workspace form is timed too and
    reported under "unstaged"."""
    import torch

    tr = moga.MogaTraining(wl.N, wl.d_model, wl.H, wl.D, wl.M, X.device)
    g = torch.Generator(device=X.device).manual_seed(wl.seed)
    dO = torch.randn(Q.shape, generator=g, device=X.device).bfloat16()
    tr.forward(X, Wr, Q, K, V)
    ws_min = tr.ws_bwd
    ws_staged, ds_bytes = None, moga.moga_attention_backward_staged_bytes(tr.cu_seqlens, wl.H)
    per_head = (ds_bytes - 4096) // wl.H
    room = torch.cuda.mem_get_info()[0] - (8 << 30) - 4096
    heads_fit = min(wl.H, max(room, 0) // max(per_head, 1))
    if staged and heads_fit >= 1:
        ws_staged = torch.empty(4096 + heads_fit * per_head, dtype=torch.uint8, device=X.device)
    stream = torch.cuda.current_stream()

    def run(ws):
        tr.ws_bwd = ws
        tr.backward(dO)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for e in evs:
            e[0].record(stream)
            moga.moga_unpermute_backward(dO, tr.Op, tr.perm, tr.gate, tr.dOp, tr.delta, tr.dgate)
            e[1].record(stream)
            moga.moga_group_attention_backward(tr.Qp, tr.Kp, tr.Vp, tr.dOp, tr.lse, tr.delta, tr.cu_seqlens, tr.perm,
                                               0.0, tr.dQ, tr.dK, tr.dV, ws)
            e[2].record(stream)
            moga.moga_route_backward(X, Wr, tr.group_id, tr.dgate, None, tr.dX, tr.dWr, tr.dbias, tr.ws_rbwd)
            e[3].record(stream)
        torch.cuda.synchronize()
        names = ["unpermute_backward", "group_attention_backward", "route_backward"]
        return {n: sum(e[k].elapsed_time(e[k + 1]) for e in evs) / steps for k, n in enumerate(names)}

    def frac(attn_ms):
        return 2.5 * flops_fwd / (attn_ms * 1e-3) / 1e12

    ms_min = run(ws_min)
    ms = ms_min
    used = 0
    if ws_staged is not None:
        ms = run(ws_staged)
        used = moga.moga_attention_backward_staged(ws_staged)
    total = sum(ms.values())
    attn = ms["group_attention_backward"]
    ws_staged_bytes = None if ws_staged is None else ws_staged.numel()
    del tr, ws_staged
    return {"ms": round(total, 4), "breakdown_ms": {k: round(v, 4) for k, v in ms.items()}, "steps": steps,
            "attention_tflops": round(frac(attn), 2),
            "attention_mfma_frac": round(frac(attn) / PEAK_BF16_TFLOPS, 4),
            "flops_per_launch": 2.5 * flops_fwd,
            "ds_staged_heads": used, "ds_bytes_all_heads": ds_bytes,
            "ds_workspace_bytes": 0 if ws_staged_bytes is None else ws_staged_bytes,
            "unstaged": {"group_attention_backward_ms": round(ms_min["group_attention_backward"], 4),
                         "attention_tflops": round(frac(ms_min["group_attention_backward"]), 2),
                         "attention_mfma_frac": round(frac(ms_min["group_attention_backward"]) / PEAK_BF16_TFLOPS,
                                                      4)},
            "unpermute_backward_gbs": round(wl.N * (6 * wl.H * wl.D + 4 * wl.H + 12) / (ms["unpermute_backward"] * 1e-3)
                                            / 1e9, 1)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "sharding the layer across GPUs (by head) is not implemented.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch

    import sparse_attention_long_router_amd as moga
    from workloads import get_workload, make_inputs
    from workloads.configs import BENCH_WORKLOAD

    wl = get_workload(args.workload or BENCH_WORKLOAD)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(wl, device=dev)
    X, Wr, Q, K, V = (inp[k] for k in ("X", "Wr", "Q", "K", "V"))
    fwd = moga.MogaForward(wl.N, wl.d_model, wl.H, wl.D, wl.M, dev, stga=wl.stga, path=args.path)
    stream = torch.cuda.current_stream()
    attn_kernel = {"gather_on_load": "attn_kernel (moga_group_attention_fused)",
                   "fused_epilogue": "attn_kernel (moga_group_attention_unpermute)",
                   "fused_vt": "attn_kernel (moga_group_attention_unpermute_vt)",
                   "fused_vtq": "attn_kernel (moga_group_attention_unpermute_vtq)",
                   "separate": "attn_kernel (moga_group_attention) + unpermute_kernel"}[args.path]

    def step(ev=None):
        # the library calls of MogaForward.__call__ for the chosen path, with
        # HIP events on the same stream between stages
        if ev is not None:
            ev[0].record(stream)
        moga.moga_route(X, Wr, None, fwd.group_id, fwd.gate)
        if ev is not None:
            ev[1].record(stream)
        if args.path == "gather_on_load":
            moga.moga_permute(fwd.group_id, wl.M, perm=fwd.perm, cu_seqlens=fwd.cu_seqlens,
                              max_seqlen=fwd.max_seqlen, ws=fwd.ws_perm)
        elif args.path == "fused_vt":
            moga.moga_permute_vt(fwd.group_id, wl.M, Q, K, V, fwd.Qp, fwd.Kp, fwd.Vt, fwd.perm, fwd.cu_seqlens,
                                 fwd.max_seqlen, fwd.ws_perm)
        elif args.path == "fused_vtq":
            moga.moga_permute_vt(fwd.group_id, wl.M, None, K, V, None, fwd.Kp, fwd.Vt, fwd.perm, fwd.cu_seqlens,
                                 fwd.max_seqlen, fwd.ws_perm)
        else:
            moga.moga_permute(fwd.group_id, wl.M, Q, K, V, fwd.Qp, fwd.Kp, fwd.Vp, fwd.perm, fwd.cu_seqlens,
                              fwd.max_seqlen, fwd.ws_perm)
        if ev is not None:
            ev[2].record(stream)
        if args.path == "gather_on_load":
            moga.moga_group_attention_fused(Q, K, V, fwd.cu_seqlens, fwd.perm, fwd.gate, 0.0, 0.0, fwd.O,
                                            fwd.ws_attn)
        elif args.path == "fused_epilogue":
            moga.moga_group_attention_unpermute(fwd.Qp, fwd.Kp, fwd.Vp, fwd.cu_seqlens, fwd.perm, fwd.gate, 0.0,
                                                0.0, fwd.O, fwd.ws_attn)
        elif args.path == "fused_vt":
            moga.moga_group_attention_unpermute_vt(fwd.Qp, fwd.Kp, fwd.Vt, fwd.cu_seqlens, fwd.perm, fwd.gate, 0.0,
                                                   0.0, fwd.O, fwd.ws_attn)
        elif args.path == "fused_vtq":
            moga.moga_group_attention_unpermute_vtq(Q, fwd.Kp, fwd.Vt, fwd.cu_seqlens, fwd.perm, fwd.gate, 0.0,
                                                    0.0, fwd.O, fwd.ws_attn)
        else:
            moga.moga_group_attention(fwd.Qp, fwd.Kp, fwd.Vp, fwd.cu_seqlens, 0.0, fwd.Op, fwd.ws_attn)
            moga.moga_unpermute(fwd.Op, fwd.perm, fwd.gate, 0.0, fwd.O)
        if ev is not None:
            ev[3].record(stream)
        if wl.stga is not None:
            s = wl.stga
            moga.moga_stga_attention(Q, K, V, s["T"], s["Hs"], s["Ws"], s["win_t"], s["tile_h"], s["tile_w"],
                                     0.0, 1.0, 1.0, fwd.O)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    stages = ["route", "permute", "group_attention", "stga"]
    per_step = {s: sorted(e[k].elapsed_time(e[k + 1]) for e in evs) for k, s in enumerate(stages)}
    if wl.stga is None:
        per_step.pop("stga")
    breakdown = {s: sum(v) / len(v) for s, v in per_step.items()}
    stage_stats = {s: {"median": round(v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2]), 4),
                       "min": round(v[0], 4)} for s, v in per_step.items()}

    counts = (fwd.cu_seqlens[1:] - fwd.cu_seqlens[:-1]).cpu().tolist()
    flops_moga = attn_flops(counts, wl.H, wl.D)
    flops_stga = 0.0
    if wl.stga is not None:
        s = wl.stga
        gsize = s["win_t"] * s["tile_h"] * s["tile_w"]
        flops_stga = 4.0 * wl.H * wl.D * gsize * gsize * (wl.N // gsize)
    step_flops = flops_moga + flops_stga
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    attn_ms = breakdown["group_attention"]
    achieved = flops_moga / (attn_ms * 1e-3) / 1e12

    traffic = traffic_entry(attn_kernel, wl.name)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": attn_kernel, "launch_ms": round(attn_ms, 4),
                "flops_per_launch": flops_moga}
    mean = wl.N / wl.M
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian-mixture tokens, random-init router and Q/K/V projections)",
        "config": {"workload": wl.name, "path": args.path, "N": wl.N, "d_model": wl.d_model, "H": wl.H, "D": wl.D,
                   "M": wl.M,
                   "group_sizes": {"min": int(min(counts)), "mean": round(mean, 1), "max": int(max(counts))},
                   "group_max_over_mean": round(max(counts) / mean, 3),
                   "skew_sum_n2_over_uniform": round(sum(c * c for c in counts) / (wl.N * mean), 3),
                   "stga": wl.stga},
        "tokens_per_s": round(wl.N / (ms_per_step * 1e-3), 1),
        "mfma_frac_step": round(value / PEAK_BF16_TFLOPS, 4),
        "breakdown_ms": {k: round(v, 4) for k, v in breakdown.items()},
        "stage_ms": stage_stats,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_backward:
        del fwd  # free the forward buffers before the training ones
        out["backward"] = backward_timing(moga, wl, X, Wr, Q, K, V, flops_moga, steps=max(2, args.steps // 4),
                                          staged=not args.no_staged_backward)
    hbm = {"route": wl.N * (2 * wl.d_model + 8) + 2 * wl.M * wl.d_model}  # algorithmic bytes per launch
    # sort + gather; the sort alone is latency-bound (reported in ms only)
    if args.path == "fused_vtq":  # K and V gathered, Q read through perm by the attention
        hbm["permute"] = wl.N * (8 * wl.H * wl.D + 16)
    elif args.path != "gather_on_load":
        hbm["permute"] = wl.N * (12 * wl.H * wl.D + 16)
    if wl.stga is not None:  # the STGA branch's own rate (a second MFMA-bound kernel of the step)
        stga_ms = breakdown["stga"]
        out["stga"] = {"kernel": "attn_kernel (moga_stga_attention)", "launch_ms": round(stga_ms, 4),
                       "flops_per_launch": flops_stga, "tflops": round(flops_stga / (stga_ms * 1e-3) / 1e12, 2),
                       "frac": round(flops_stga / (stga_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    out["hbm_gbs"] = {k: round(b / (breakdown[k] * 1e-3) / 1e9, 1) for k, b in hbm.items()}
    out["hbm_frac"] = {k: round(v / PEAK_HBM_GBS, 4) for k, v in out["hbm_gbs"].items()}
    copy_gbs = copy_rate_gbs(stream)
    out["hbm_copy_gbs"] = round(copy_gbs, 1)  # measured device-to-device copy, read + write bytes
    out["hbm_frac_of_copy"] = {k: round(v / copy_gbs, 4) for k, v in out["hbm_gbs"].items()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, wl, counts, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
