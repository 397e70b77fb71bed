"""Benchmark of the W4A16 INT4 MoE expert path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill|tp8|masked|tiny]
                    [--no-prefill] [--no-cpu-baseline] [--no-graph]

One step = one call of the whole path on one batch of seeded synthetic input
already resident in HBM: routing sort (align) -> gate/up GEMM with SiLU*gate in
its epilogue -> down GEMM -> top-k combine (for the masked and contiguous
workloads: the two GEMMs, then the combine).  With --combine fused the
combine runs in the down GEMM's epilogue.  W untimed warm-up steps, then exactly K timed steps
between two device synchronisations.  One JSON line is printed.

The headline workload (default) is the decode share of a Kimi-K2-like layer on
one GPU of an EP8 deployment (48 local experts, hidden 7168, intermediate 2048,
64 tokens x top-8, about 9-15 routed rows per local expert): a weight-streaming
problem, so its roofline is HBM bandwidth on the algorithmic weight bytes.
Unless --no-prefill is given, the same run then measures the EP8 prefill share
(8192 tokens over 384 experts, 48 local; MFMA-bound) and reports it in a
"prefill" sub-object with its own roofline (bf16 MFMA TFLOP/s) and CPU
baseline.  Two prepacked copies of the weights are used alternately so that no
call finds the previous call's weights in the 256 MB last-level cache.

Extra figures in the line: per-stage microseconds (HIP events on the stream the
kernels run on), the pages' unit (gate/up + down), the HIP-graph replay time of
the same step, the roofline object of the dominant kernel and the CPU oracle's
time on the host cores (all threads, and one thread).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

METRIC = "MoE layer µs/call; decode weight HBM GB/s and prefill TFLOP/s (% of peak)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "prefill", "tp8", "masked", "contiguous", "decode_mxfp4",
                            "decode_a8w4", "tiny"])
    p.add_argument("--copies", type=int, default=2, help="prepacked weight copies rotated per call")
    p.add_argument("--no-prefill", action="store_true",
                   help="do not add the prefill sub-object to the decode line")
    p.add_argument("--combine", choices=["separate", "fused"], default="separate",
                   help="indexed path: top-k combine as its own kernel or in the down GEMM's "
                        "epilogue (streaming kernel only)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=12.0,
                   help="target seconds of oracle work per CPU leg")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="run one plain device copy of this size before the warm-up (a known "
                        "byte count for scaling HBM counters)")
    return p.parse_args()


def kernel_source_hash() -> str:
    """Hash of the kernel sources and of the build script that holds their
    compiler flags (a profile taken on other code reads as stale)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a16_int4_mixture_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "w4a16_int4_mixture_amd", "build.py"), "rb") as fh:
        h.update(b"build.py" + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, src_hash: str):
    """HBM bytes per launch of the dominant kernel from committed PMC summaries
    (FETCH_SIZE and WRITE_SIZE runs scaled by a plain copy of known size), or
    None when no summary matches the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_gate_up_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def workload_name(name, wl):
    return {
        "decode": "EP8 decode share: 48 local experts, H7168 I2048, 64 tokens x top-8 (~10.7 rows/expert)",
        "prefill": "EP8 prefill share: 48 local experts, H7168 I2048, 8192 tokens x top-8 over 384",
        "tp8": "TP8 share: 384 experts, H7168 I256, 1024 tokens x top-8",
        "masked": "grouped masked EP32 share: 12 experts, 256 rows Zipf(1.2), expected_m 32",
        "contiguous": "grouped contiguous EP8 prefill share: 48 experts x 128 rows, H7168 I2048",
        "decode_mxfp4": "EP8 decode share with MXFP4 weights (E2M1 codes, E8M0 scales per 32): "
                        "48 local experts, H7168 I2048, 64 tokens x top-8",
        "decode_a8w4": "EP8 decode share in A8W4 (MXFP8 activations, MXFP4 weights, E8M0 scales "
                       "per 32): 48 local experts, H7168 I2048, 64 tokens x top-8",
        "tiny": "tiny: 8 experts, top-2, H256 I128, 16 tokens",
    }[name]


def run_workload(name, args, src_hash, cpu_legs=True):
    """Prepare one workload on the GPU, time `args.steps` calls of the path
    (after `args.warmup`), and return its figures as a dict."""
    import numpy as np
    import torch

    import synth
    import w4a16_int4_mixture_amd as m

    dev = torch.device("cuda", 0)

    def to_dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    t0 = time.time()
    a8 = name.endswith("_a8w4")
    mxfp4 = name.endswith("_mxfp4") or a8
    base = name.rsplit("_", 1)[0] if mxfp4 else name
    d = synth.make_workload(base, seed=0, weights=not mxfp4)
    wl = d["wl"]
    if mxfp4:
        d.update(synth.make_weights_mxfp4(wl.E_local, wl.H, wl.I, seed=0))
    mfma_bound = name in ("prefill", "contiguous")
    profile = m.PROFILE_PREFILL if mfma_bound else m.PROFILE_DECODE
    print(f"[bench] workload {name}: generated inputs in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)

    codes13, scales13 = to_dev(d["codes13"]), to_dev(d["scales13"])
    codes2, scales2 = to_dev(d["codes2"]), to_dev(d["scales2"])
    copies = []
    for _ in range(max(1, args.copies)):
        # W13 with gate/up interleave: SiLU*gate runs in the gate/up epilogue
        if mxfp4:
            fa8 = m.PACK_MXFP8_ACT if a8 else 0
            copies.append((m.prepare_weight_mxfp4(codes13, scales13,
                                                  m.PACK_GATE_UP_INTERLEAVE | fa8),
                           m.prepare_weight_mxfp4(codes2, scales2, fa8)))
        else:
            copies.append((m.prepare_weight(codes13, scales13, profile,
                                            m.PACK_GATE_UP_INTERLEAVE),
                           m.prepare_weight(codes2, scales2, profile)))
    del codes13, scales13, codes2, scales2
    torch.cuda.synchronize()

    X = to_dev(d["X"])
    ids = to_dev(d["topk_ids"])
    tw = to_dev(d["topk_weights"])
    em = None if d["expert_map"] is None else to_dev(d["expert_map"])
    masked = name == "masked"
    contig = name == "contiguous"

    # local routed rows and active experts (host-side knowledge of the draw)
    if masked:
        counts = d["masked_m"].astype(np.int64)
    elif contig:
        mi_h = d["m_indices"]
        counts = np.bincount(mi_h[mi_h >= 0], minlength=wl.E_local).astype(np.int64)
    else:
        flat = d["topk_ids"].ravel()
        loc = flat if d["expert_map"] is None else d["expert_map"][flat]
        loc = loc[(loc >= 0) & (loc < wl.E_local)]
        counts = np.bincount(loc, minlength=wl.E_local).astype(np.int64)
    rows = int(counts.sum())
    active = int((counts > 0).sum())
    H, I = wl.H, wl.I
    # codes (half a byte per weight) + one scale per 32 (bf16, or an E8M0 byte
    # for MXFP4)
    sb = 1 if mxfp4 else 2
    w13_bytes_per_expert = 2 * I * H // 2 + 2 * I * (H // 32) * sb
    w2_bytes_per_expert = H * I // 2 + H * (I // 32) * sb
    bytes13 = active * w13_bytes_per_expert
    bytes2 = active * w2_bytes_per_expert
    flops13 = 2.0 * rows * (2 * I) * H
    flops2 = 2.0 * rows * H * I

    if masked:
        max_m = d["max_m"]
        paths = [m.MaskedPath(w13, w2, max_m, wl.expected_m, wl.T, wl.top_k, device=dev)
                 for (w13, w2) in copies]
        a3 = to_dev(d["a3"].reshape(wl.E_local * max_m, H))
        mm = to_dev(d["masked_m"])
        row_of = to_dev(d["row_of"])

        def stages(p):
            ga, da = p.gate_up_args(a3, mm), p.down_args(mm)
            return [("gate_up", lambda: m._capi.w4a16_moe_w4a16_gemm(ga)),
                    ("down", lambda: m._capi.w4a16_moe_w4a16_gemm(da)),
                    ("combine", lambda: m._capi.w4a16_moe_combine(
                        p.Y2, p.Y2.shape[0], H, row_of, tw, wl.T, wl.top_k, p.out))]
    elif contig:
        a2 = to_dev(d["a2"])
        mi = to_dev(d["m_indices"])
        row_of = to_dev(d["row_of"])
        paths = [m.ContiguousPath(w13, w2, d["m_indices"].size, wl.T, wl.top_k, device=dev)
                 for (w13, w2) in copies]

        def stages(p):
            ga, da = p.gate_up_args(a2, mi), p.down_args(mi)
            return [("gate_up", lambda: m._capi.w4a16_moe_w4a16_gemm(ga)),
                    ("down", lambda: m._capi.w4a16_moe_w4a16_gemm(da)),
                    ("combine", lambda: m._capi.w4a16_moe_combine(
                        p.Y2, p.Y2.shape[0], H, row_of, tw, wl.T, wl.top_k, p.out))]
    else:
        fused = args.combine == "fused" and profile == m.PROFILE_DECODE
        paths = [m.IndexedPath(w13, w2, wl.T, wl.top_k, wl.E_global, rows_hint=rows, device=dev,
                               fuse_combine=fused)
                 for (w13, w2) in copies]

        def stages(p):
            ga, da = p.stage_args(X, tw)
            st = [("align", lambda: p.routing.align(ids, wl.E_global, em))]
            if p.a8:
                st.append(("quant_x", lambda: p.quant_x(X)))
            st.append(("gate_up", lambda: m._capi.w4a16_moe_w4a16_gemm(ga)))
            if p.separate_act:
                st.append(("act", lambda: p.act()))
            if p.a8:
                st.append(("quant_z", lambda: p.quant_z()))
            st.append(("down", lambda: m._capi.w4a16_moe_w4a16_gemm(da)))
            if not p.fuse_combine:
                st.append(("combine", lambda: p.combine(tw)))
            return st

    # pre-built argument structs (workspaces resolved once): the timed loop
    # only launches
    stage_lists = [stages(p) for p in paths]

    if args.calib_copy_mib > 0:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(i, events=None):
        st = stage_lists[i % len(stage_lists)]
        for j, (_, fn) in enumerate(st):
            if events is not None:
                events[j].record()
            fn()
        if events is not None:
            events[len(st)].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed steps: wall clock between synchronisations, nothing recorded
    # between the launches (a call as a caller makes it)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1000.0 / args.steps
    us_call = ms_per_step * 1000.0

    # the same steps again with HIP events between the stages (per-stage
    # times); every launch goes to torch's current stream, where the events
    # are recorded
    # (warm-up steps first, with no synchronisation before the events, so the
    # GPU runs without a pause into the measured steps)
    n_st = len(stage_lists[0])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_st + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    stage_us = {}
    for j, (sname, _) in enumerate(stage_lists[0]):
        vals = [ev[i][j].elapsed_time(ev[i][j + 1]) * 1000.0 for i in range(args.steps)]
        stage_us[sname] = float(np.median(vals))
    event_total = float(np.median([ev[i][0].elapsed_time(ev[i][n_st]) * 1000.0
                                   for i in range(args.steps)]))

    # HIP graph of one step per weight copy, replayed alternately
    graph_us = None
    if not args.no_graph:
        try:
            graphs = []
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for k in range(len(paths)):
                    step(k)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            for k in range(len(paths)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(k)
                graphs.append(g)
            for i in range(args.warmup):
                graphs[i % len(graphs)].replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for i in range(args.steps):
                graphs[i % len(graphs)].replay()
            torch.cuda.synchronize()
            graph_us = (time.perf_counter() - t1) * 1e6 / args.steps
        except Exception as exc:  # report, never hide
            print(f"[bench] graph capture failed: {exc}", file=sys.stderr)

    gu, dn = stage_us["gate_up"], stage_us["down"]
    # the dominant kernel is the gate/up GEMM; its algorithmic HBM bytes per
    # launch are the active experts' codes + scales, the activations read once
    # and the routed rows' outputs written once
    # (A8W4 reads the activations as E4M3 bytes plus one E8M0 byte per 32)
    x_rows = rows if masked or contig else wl.T
    x_bytes = x_rows * H + x_rows * (H // 32) if a8 else x_rows * H * 2
    out_bytes = rows * I * 2           # Z: SiLU*gate is applied in the epilogue
    alg_bytes13 = bytes13 + x_bytes + out_bytes
    if mfma_bound:
        bound, unit_rf = "mfma", "TFLOP/s"
        achieved = flops13 / (gu * 1e-6) / 1e12
        peak = BF16_PEAK_TFLOPS
    else:
        bound, unit_rf = "hbm", "GB/s"
        achieved = alg_bytes13 / (gu * 1e-6) / 1e9
        peak = HBM_PEAK_GBS
    plan13 = paths[0].plan if not masked else None
    kname = {"prefill": "k_gemm_large (gate/up GEMM of the PREFILL profile, SiLU*gate in its "
                        "epilogue: one launch per call)",
             "contiguous": "k_gemm_large (gate/up GEMM, grouped contiguous layout, SiLU*gate in "
                           "its epilogue: one launch per call)",
             "decode_a8w4": "k_gemm_mx (A8W4 gate/up GEMM on the block-scaled MFMA, MXFP8 "
                            "activations x MXFP4 weights, SiLU*gate in its epilogue: one launch "
                            "per call)"}.get(
        name, "k_gemm_small (gate/up GEMM with SiLU*gate epilogue and in-kernel split-K fix-up: "
              "one launch per call)")
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit_rf,
                "frac": round(achieved / peak, 4),
                "traffic": traffic_from_profiles(name, src_hash),
                "kernel": kname,
                "algorithmic_per_launch": alg_bytes13 if bound == "hbm" else flops13,
                "launch_us": round(gu, 2)}

    del paths, stage_lists, copies
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    cpu = None
    if cpu_legs and not args.no_cpu_baseline:
        cpu = cpu_baseline(d, wl, name, args.cpu_budget_s)

    weight_bytes = bytes13 + bytes2
    return {
        "wl": wl, "rows": rows, "active": active, "us_call": us_call, "ms_per_step": ms_per_step,
        "stage_us": stage_us, "event_total": event_total, "graph_us": graph_us,
        "gu": gu, "dn": dn, "roofline": roofline, "cpu": cpu, "plan13": plan13,
        "weight_bytes": weight_bytes, "flops": flops13 + flops2, "copies": args.copies,
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path runs on one GPU; multi-GPU sharding (EP all-to-all, TP "
              "reduce-scatter) is described in DESIGN.md but not built. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    src_hash = kernel_source_hash()

    r = run_workload(args.workload, args, src_hash)
    wl = r["wl"]
    plan13 = r["plan13"]
    gu, dn, us_call = r["gu"], r["dn"], r["us_call"]
    span = gu + dn
    line = {
        "metric": METRIC,
        "value": round(us_call, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations x int4 weights (fp32 accumulate)",
        "data": "synthetic (seeded, random-init weights)",
        "config": {"workload": workload_name(args.workload, wl), "tokens": wl.T,
                   "top_k": wl.top_k, "local_experts": wl.E_local, "hidden": wl.H,
                   "intermediate": wl.I, "routed_rows": r["rows"],
                   "active_experts": r["active"], "weight_copies": r["copies"],
                   "gate_up_tile_m": None if plan13 is None else plan13.tile_m,
                   "gate_up_split_k": None if plan13 is None else plan13.split_k},
        "stages_us": {k: round(v, 2) for k, v in r["stage_us"].items()},
        "event_total_us": round(r["event_total"], 2),
        "gate_up_plus_down_us": round(span, 2),
        "graph_us_per_call": None if r["graph_us"] is None else round(r["graph_us"], 2),
        "weight_GBps_path": round(r["weight_bytes"] / (us_call * 1e-6) / 1e9, 1),
        "weight_GBps_gate_up_plus_down": round(r["weight_bytes"] / (span * 1e-6) / 1e9, 1),
        "frac_hbm_gate_up_plus_down": round(r["weight_bytes"] / (span * 1e-6) / 1e9
                                            / HBM_PEAK_GBS, 4),
        "tflops_gate_up_plus_down": round(r["flops"] / (span * 1e-6) / 1e12, 2),
        "roofline": r["roofline"],
        "cpu_baseline": r["cpu"],
        "kernel_source_hash": src_hash,
    }

    if args.workload == "decode" and not args.no_prefill:
        p = run_workload("prefill", args, src_hash)
        pg, pd, pu = p["gu"], p["dn"], p["us_call"]
        ps = pg + pd
        line["prefill"] = {
            "workload": workload_name("prefill", p["wl"]),
            "routed_rows": p["rows"],
            "us_per_call": round(pu, 2),
            "stages_us": {k: round(v, 2) for k, v in p["stage_us"].items()},
            "gate_up_plus_down_us": round(ps, 2),
            "tflops_gate_up_plus_down": round(p["flops"] / (ps * 1e-6) / 1e12, 2),
            "frac_mfma_gate_up_plus_down": round(p["flops"] / (ps * 1e-6) / 1e12
                                                 / BF16_PEAK_TFLOPS, 4),
            "tflops_path": round(p["flops"] / (pu * 1e-6) / 1e12, 2),
            "graph_us_per_call": None if p["graph_us"] is None else round(p["graph_us"], 2),
            "gate_up_tile_m": p["plan13"].tile_m,
            "roofline": p["roofline"],
            "cpu_baseline": p["cpu"],
        }
    print(json.dumps(line), flush=True)


def _oracle_call(oracle, d, wl, workload, tokens):
    """The oracle's whole path on the first `tokens` tokens (or, masked, the
    whole workload)."""
    if workload == "masked":
        G, max_m = wl.E_local, d["max_m"]
        a3 = d["a3"].reshape(G * max_m, wl.H)
        Z = oracle.silu_mul(oracle.masked_gemm(a3, d["masked_m"], d["codes13"], d["scales13"]))
        Y2 = oracle.masked_gemm(Z, d["masked_m"], d["codes2"], d["scales2"])
        oracle.combine(Y2, d["row_of"], d["topk_weights"])
        return
    # the PREFILL profile's kernel rounds each dequantised weight to bf16 once:
    # its oracle is the one with bf16-rounded weights (same cost); the
    # contiguous workload computes the same rows as the indexed path
    wmode = 1 if workload in ("prefill", "contiguous") else 0
    n = tokens
    fwd = (oracle.moe_forward_a8w4 if workload.endswith("_a8w4") else
           oracle.moe_forward_mx if workload.endswith("_mxfp4") else oracle.moe_forward)
    kw = {} if workload.endswith(("_mxfp4", "_a8w4")) else {"wmode": wmode}
    fwd(d["X"][:n], d["topk_ids"][:n], d["topk_weights"][:n], wl.E_global, d["expert_map"],
        d["codes13"], d["scales13"], d["codes2"], d["scales2"], **kw)


def _timed_leg(oracle, d, wl, workload, budget_s):
    """Oracle seconds for as many tokens as fit in about budget_s (the whole
    call when it fits), scaled to one call."""
    T = wl.T
    if workload == "masked":
        t0 = time.perf_counter()
        _oracle_call(oracle, d, wl, workload, T)
        dt = time.perf_counter() - t0
        return dt * 1e6, "the full masked workload, one call", dt
    # grow the sample until it takes about the budget (or covers the call):
    # a short probe overestimates the time per token (fixed costs)
    n = max(1, min(T, 4))
    while True:
        t0 = time.perf_counter()
        _oracle_call(oracle, d, wl, workload, n)
        dt = time.perf_counter() - t0
        if n >= T or dt >= 0.5 * budget_s:
            break
        n = int(min(T, max(n + 1, n * budget_s / max(dt, 1e-6))))
    return dt * 1e6 * T / n, f"first {n} of {T} tokens of the same workload (time scaled to the full call)", dt


def cpu_baseline(d, wl, workload, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    once on all the threads OpenMP gives it, once on one thread."""
    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads()
    try:
        host_cpus = len(os.sched_getaffinity(0))
    except AttributeError:
        host_cpus = os.cpu_count()
    value, sample, dt = _timed_leg(oracle, d, wl, workload, budget_s)
    oracle.set_num_threads(1)
    try:
        value1, sample1, dt1 = _timed_leg(oracle, d, wl, workload, budget_s / 3)
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(value, 1), "unit": "us/call", "cores": threads, "kind": "oracle",
            "sample": sample, "measured_s": round(dt, 2), "cpu_model": cpu_model(),
            "host_cpus": host_cpus,
            "single_thread": {"value": round(value1, 1), "unit": "us/call", "cores": 1,
                              "sample": sample1, "measured_s": round(dt1, 2)}}


if __name__ == "__main__":
    main()
