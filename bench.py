"""Throughput of the causal grouped-query flash attention hot path on one MI355X.

A step is one pass of the whole path over one synthetic batch: attn_fwd, then
attn_bwd_dq, then attn_bwd_dkv, all through the C-ABI, with inputs resident in HBM.
The workload is B=16, T=1024, Hq=6, Hkv=2, d=64 (bf16 N(0,1) inputs, seeded).

Flop convention (causal pairs only, pairs = B*Hq*T*(T+1)/2; diagonal-tile waste and
the backward's recomputation are not credited):
  forward  = 4*d per pair (S = Q K^T and P V),
  backward = 10*d per pair (five contractions: S, dP, dQ, dK, dV),
  step     = 14*d per pair.
Per kernel, for the roofline line: attn_fwd 4*d, attn_bwd_dq 6*d (S, dP, dQ),
attn_bwd_dkv 8*d (S, dP, dV, dK) per pair.

Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 dense bf16/fp16 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
WORKLOAD = "B16_T1024_Hq6_Hkv2_d64"
KERNEL_SOURCES = ["causal_gqa_flash_amd/csrc/attn_fwd.hip", "causal_gqa_flash_amd/csrc/attn_fwd_par.hip",
                  "causal_gqa_flash_amd/csrc/attn_bwd.hip",
                  "causal_gqa_flash_amd/csrc/cgqa_device.hpp", "causal_gqa_flash_amd/csrc/cgqa_launch.hpp",
                  "causal_gqa_flash_amd/csrc/api.hip", "causal_gqa_flash_amd/build.py"]
# Device kernels behind each entry point (the one a launch uses depends on d and the shape).
KERNEL_NAMES = {"attn_fwd": ("attn_fwd_kernel", "attn_fwd_par_kernel"),
                "attn_bwd_dq": ("attn_bwd_dq_kernel", "attn_bwd_dq_pipe_kernel"),
                "attn_bwd_dkv": ("attn_bwd_dkv_kernel",)}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_B16_T1024_Hq6_Hkv2_d64.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the kernels as they are now; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


COPY_BYTES = 256 << 20   # calibration copy: 256 MiB read and 256 MiB written


def pmc_workload(args):
    """A short run for rocprofv3 --pmc: each kernel a few times, then a plain device copy
    of COPY_BYTES (torch's copy kernel) whose FETCH_SIZE / WRITE_SIZE calibrate the
    counters to bytes."""
    import numpy as np
    import torch
    import causal_gqa_flash_amd as cg
    import synthetic_inputs as si
    w = si.WORKLOAD_BY_NAME[WORKLOAD]
    x = si.make_workload_inputs(w, seed=3)
    dev = {n: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for n, a in x.items()}
    for _ in range(args.steps):
        o, lse = cg.attn_fwd(dev["q"], dev["k"], dev["v"], scale=w.scale)
        delta, dq = cg.attn_bwd_dq(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=w.scale)
        cg.attn_bwd_dkv(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, scale=w.scale)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_workload": w.name, "steps": args.steps, "copy_bytes": COPY_BYTES}), flush=True)


def pmc_summarize(fetch_dir, write_dir, out_path):
    """Per-launch HBM bytes of each kernel from two rocprofv3 --pmc runs of
    pmc_workload (FETCH_SIZE, then WRITE_SIZE), scaled by what the same counters read
    for the calibration copy (COPY_BYTES each way)."""
    import csv
    import glob

    def read(d, counter):
        path = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
        per = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        return per

    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = read(d, counter)
        copy = [v for (i, name), v in per.items() if "copy" in name.lower() or "elementwise" in name.lower()]
        if not copy:
            raise SystemExit(f"no copy kernel found in {d}")
        factor = COPY_BYTES / (max(copy) * 1024.0)     # counter is in KiB
        for kern, names in KERNEL_NAMES.items():
            vals = [v for (i, name), v in per.items() if any(n + "<" in name for n in names)]
            if vals:
                kb = sum(vals) / len(vals)
                res.setdefault(kern, {})[counter] = {"kib_per_dispatch": round(kb, 1), "calibration": round(factor, 4),
                                                     "bytes": kb * 1024.0 * factor}
    out = {"workload": WORKLOAD, "kernel_source_hash": kernel_source_hash(), "copy_bytes": COPY_BYTES,
           "kernels": {k: {"bytes_per_launch": round(v["FETCH_SIZE"]["bytes"] + v["WRITE_SIZE"]["bytes"]),
                           "fetch": v["FETCH_SIZE"], "write": v["WRITE_SIZE"]} for k, v in res.items()}}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def pmc_counters(dirs):
    """Per-dispatch averages of the SQ/GRBM counters of rocprofv3 --pmc runs of the
    profiling workload (one folder per pass) for each attention kernel, with ratios that
    need no clock: executed matrix-core instructions against the credited ones (S, dP,
    dV, dK and O per 32x32x16 instruction), LDS bank-conflict cycles per LDS-active cycle,
    and each wave's cycles spent waiting, issuing VALU or issuing LDS."""
    import csv
    import glob
    import synthetic_inputs as si
    w = si.WORKLOAD_BY_NAME[WORKLOAD]
    per = {}
    for d in dirs:
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        for r in csv.DictReader(open(path)):
            for kern, names in KERNEL_NAMES.items():
                if any(n + "<" in r["Kernel_Name"] for n in names):
                    c = per.setdefault(kern, {}).setdefault(r["Counter_Name"], {})
                    c[r["Dispatch_Id"]] = c.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    credited = {"attn_fwd": 4, "attn_bwd_dq": 6, "attn_bwd_dkv": 8}   # flops per pair / d
    out = {"workload": WORKLOAD, "kernel_source_hash": kernel_source_hash(), "kernels": {}}
    for kern, cs in per.items():
        avg = {n: sum(v.values()) / len(v) for n, v in cs.items()}
        e = {"counters_per_dispatch": {n: round(x, 1) for n, x in sorted(avg.items())}}
        if "SQ_INSTS_MFMA" in avg:
            cred = credited[kern] * w.d * w.causal_pairs / (2 * 32 * 32 * 16)
            e["mfma_insts_executed_per_credited"] = round(avg["SQ_INSTS_MFMA"] / cred, 4)
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
            e["lds_bank_conflict_per_active_cycle"] = round(avg["SQ_LDS_BANK_CONFLICT"] / avg["SQ_LDS_IDX_ACTIVE"], 4)
        if avg.get("SQ_WAVE_CYCLES"):
            for n in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                      "SQ_ACTIVE_INST_ANY"):
                if n in avg:
                    e[n.lower() + "_per_wave_cycle"] = round(avg[n] / avg["SQ_WAVE_CYCLES"], 4)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg.get("SQ_INSTS_MFMA"):
            e["mfma_busy_cycles_per_inst"] = round(avg["SQ_VALU_MFMA_BUSY_CYCLES"] / avg["SQ_INSTS_MFMA"], 2)
        out["kernels"][kern] = e
    print(json.dumps(out, indent=1), flush=True)


def trace_summary(trace_dir):
    """From a rocprofv3 --kernel-trace folder of a bench run, for the bench workload's
    launches (each kernel's most frequent grid, the one of the step loops): every launch's
    average duration; every forward, dQ, dK/dV triple that ran back to back (the step
    loops) with each kernel's duration inside those steps, the gaps between consecutive
    kernels, and the span from one step's forward to the next (microseconds)."""
    import csv
    import glob
    import statistics as st
    path = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))

    def kind(name):
        for kern, names in KERNEL_NAMES.items():
            if any(n + "<" in name for n in names):
                return kern
        return None
    grid = lambda r: (r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"], r["Kernel_Name"])
    counts = {}
    for r in rows:
        if kind(r["Kernel_Name"]):
            counts[(kind(r["Kernel_Name"]), grid(r))] = counts.get((kind(r["Kernel_Name"]), grid(r)), 0) + 1
    main_grid = {}
    for (k, g), c in counts.items():
        if c > counts.get((k, main_grid.get(k)), 0):
            main_grid[k] = g
    rows = [r for r in rows if kind(r["Kernel_Name"]) and grid(r) == main_grid[kind(r["Kernel_Name"])]]
    seq = [(kind(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    order = ["attn_fwd", "attn_bwd_dq", "attn_bwd_dkv"]
    starts = [i for i in range(len(seq) - 2) if [x[0] for x in seq[i:i + 3]] == order]
    dur = {k: [] for k in order}
    gap = {"fwd->dq": [], "dq->dkv": [], "dkv->next fwd": []}
    span = []
    for i in starts:
        for j, k in enumerate(order):
            dur[k].append((seq[i + j][2] - seq[i + j][1]) / 1e3)
        gap["fwd->dq"].append((seq[i + 1][1] - seq[i][2]) / 1e3)
        gap["dq->dkv"].append((seq[i + 2][1] - seq[i + 1][2]) / 1e3)
        if i + 3 < len(seq) and seq[i + 3][0] == "attn_fwd":
            gap["dkv->next fwd"].append((seq[i + 3][1] - seq[i + 2][2]) / 1e3)
            span.append((seq[i + 3][1] - seq[i][1]) / 1e3)
    f = lambda v: {"median": round(st.median(v), 2), "mean": round(st.mean(v), 2), "n": len(v)} if v else None
    every = {k: [(e - b) / 1e3 for kk, b, e in seq if kk == k] for k in order}
    out = {"trace": path, "kernels": {k: main_grid[k][3] + " grid " + "x".join(main_grid[k][:3]) for k in order},
           "all_launches_us": {k: f(v) for k, v in every.items()},
           "steps": len(starts), "kernel_us": {k: f(v) for k, v in dur.items()},
           "gap_us": {k: f(v) for k, v in gap.items()}, "step_span_us": f(span),
           "kernel_sum_median_us": round(sum(st.median(v) for v in dur.values()), 2) if starts else None}
    print(json.dumps(out, indent=1), flush=True)


def gemm_bench(w, graph_timed):
    """The projections around attention for the workload's B*T tokens (model width Hq*d,
    fused QKV width (Hq + 2 Hkv) d): forward QKV and WO (+ residual), and the QKV
    projection's dX and dW, each timed through cgqa_gemm, with torch.matmul (hipBLASLt)
    on the same bf16 operands beside it for reference. Both sides are timed as replays of
    a captured HIP graph of back-to-back calls (their host dispatch exceeds these short
    kernels) on the current stream."""
    import torch
    import causal_gqa_flash_amd as cg
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    Mt, D, Q = w.B * w.T, w.Hq * w.d, (w.Hq + 2 * w.Hkv) * w.d
    rnd = lambda *s: (torch.randn(*s, generator=g, device="cuda") * 0.05).to(torch.bfloat16)
    x, wqkv, wo, dqkv = rnd(Mt, D), rnd(Q, D), rnd(D, D), rnd(Mt, Q)
    resid = torch.randn(Mt, D, generator=g, device="cuda")
    c_qkv = torch.empty(Mt, Q, dtype=torch.bfloat16, device="cuda")
    c_f32 = torch.empty(Mt, D, device="cuda")
    c_dw = torch.empty(Q, D, device="cuda")
    ws_dw = torch.empty((max(cg.gemm_workspace_bytes(Q, D, Mt), 4) // 4,), device="cuda")
    cases = {
        "qkv": (Mt, Q, D, lambda: cg.gemm(x, wqkv, c=c_qkv),
                lambda: torch.matmul(x, wqkv.t())),
        "wo_residual": (Mt, D, D, lambda: cg.gemm(x, wo, r=resid, c=c_f32),
                        lambda: torch.matmul(x, wo.t())),
        "dx_qkv": (Mt, D, Q, lambda: cg.gemm(dqkv, wqkv, c=c_f32, b_kn=True),
                   lambda: torch.matmul(dqkv, wqkv)),
        "dw_qkv": (Q, D, Mt, lambda: cg.gemm(dqkv, x, c=c_dw, a_km=True, b_kn=True, workspace=ws_dw),
                   lambda: torch.matmul(dqkv.t(), x)),
    }
    res, best = {}, None
    for name, (M, N, K, ours, lib) in cases.items():
        ours(); lib()
        torch.cuda.synchronize()
        ms, ms_lib = graph_timed(ours, 20), graph_timed(lib, 20)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        res[name] = {"M": M, "N": N, "K": K, "ms": round(ms, 5), "tflops": round(tf, 1),
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "torch_matmul_ms": round(ms_lib, 5)}
        if best is None or tf > best[1]:
            best = (name, tf)
    return {"shapes": res, "roofline": {"bound": "mfma", "kernel": "gemm_bf16_kernel (" + best[0] + ")",
                                        "achieved": round(best[1], 1), "peak": PEAK_BF16_TFLOPS,
                                        "unit": "TFLOP/s", "frac": round(best[1] / PEAK_BF16_TFLOPS, 4)},
            "note": "ms: one call's share of a replayed HIP graph of 20 back-to-back calls "
                    "(HIP events, median of repeats); torch_matmul_ms: the same for torch.matmul "
                    "(hipBLASLt) on the same bf16 operands (bf16 output, no residual)"}


def cpu_baseline(w, x, budget_s):
    """The fp64 CPU oracle (as it is) on whole (batch, kv head) slices of the workload,
    forward and backward, until about budget_s seconds have passed."""
    import numpy as np
    import oracle
    import synthetic_inputs as si
    threads = oracle.default_threads()
    slices = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    done, t0 = 0, time.perf_counter()
    for b, g in slices:
        xs = si.slice_group(x, w.Hq, w.Hkv, b, g)
        f = {n: oracle.bf16_to_f64(a) for n, a in xs.items()}
        oracle.attn_bwd(f["q"], f["k"], f["v"], f["do"], w.scale, threads=threads)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    secs = time.perf_counter() - t0
    pairs = done * w.G * w.T * (w.T + 1) // 2
    tflops = 14 * w.d * pairs / secs / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(secs, 3),
            "sample": f"{done} of {len(slices)} (batch, kv head) slices of {w.name}, forward and "
                      f"backward in fp64, {threads} threads; same 14*d flop/pair convention"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--repeats", type=int, default=5, help="timed repeats; the median is reported")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warmup steps, run steps for this long so the GPU clocks "
                         "leave their idle state (the first tens of ms run 5-11%% slower)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-naive", action="store_true", help="skip timing the naive reference mode")
    ap.add_argument("--no-gemm", action="store_true", help="skip timing the projection matmuls")
    ap.add_argument("--no-rope", action="store_true", help="skip timing the rotary embedding")
    ap.add_argument("--no-configs", action="store_true", help="skip timing the other workloads")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="run the short workload that rocprofv3 --pmc profiles (see profiles/)")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders into the traffic summary")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="summarise the step loops of a rocprofv3 --kernel-trace folder of a bench run")
    ap.add_argument("--pmc-counters", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc folders (SQ counters) of the profiling workload")
    args = ap.parse_args()
    if args.pmc_summarize:
        pmc_summarize(args.pmc_summarize[0], args.pmc_summarize[1], TRAFFIC_FILE)
        return
    if args.pmc_counters:
        pmc_counters(args.pmc_counters)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    if args.pmc_workload:
        pmc_workload(args)
        return

    import numpy as np
    import torch
    import causal_gqa_flash_amd as cg
    import synthetic_inputs as si

    w = si.WORKLOAD_BY_NAME[WORKLOAD]
    x = si.make_workload_inputs(w, seed=3)
    dev = {n: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for n, a in x.items()}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.T), dtype=torch.float32, device="cuda")
    delta = cg.bwd_delta(w.B, w.Hq, w.T, device="cuda")
    dq = torch.empty((w.B, w.T, w.Hq, w.d), dtype=torch.float32, device="cuda")
    dk = torch.empty((w.B, w.T, w.Hkv, w.d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    stream = torch.cuda.current_stream()

    # The calls launch on the current stream: `stream` in the timed loops, the capture
    # stream while a HIP graph of them is captured.
    def fwd():
        cg.attn_fwd(q, k, v, scale=w.scale, o=o, lse=lse)

    def bwd_dq():
        cg.attn_bwd_dq(q, k, v, o, do, lse, scale=w.scale, delta=delta, dq=dq)

    def bwd_dkv():
        cg.attn_bwd_dkv(q, k, v, do, lse, delta, scale=w.scale, dk=dk, dv=dv)

    def step():
        fwd()
        bwd_dq()
        bwd_dkv()

    def timed(fn, n):
        """Median over repeats of the mean ms per call of n back-to-back calls, timed
        with HIP events on the stream the kernels run on."""
        per = []
        for _ in range(args.repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / n)
        return float(np.median(per))

    graph_failures = []

    def graph_timed(fn, n):
        """As timed, for kernels shorter than their host dispatch: the n calls are captured
        once in a HIP graph (fn launches on the current stream) and the graph is replayed.
        If the capture fails, falls back to timed and records the failure."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):   # warm-up off the default stream, as capture wants
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        try:
            with torch.cuda.graph(graph):
                for _ in range(n):
                    fn()
        except RuntimeError as e:
            print(f"graph capture failed: {e}", file=sys.stderr, flush=True)
            graph_failures.append(getattr(fn, "__name__", "call"))
            torch.cuda.synchronize()
            return timed(fn, n)
        torch.cuda.synchronize()
        graph.replay()
        cur = torch.cuda.current_stream()
        per = []
        for _ in range(args.repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(cur)
            graph.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / n)
        del graph
        return float(np.median(per))

    # Clock settle: untimed steps until settle_ms of wall time has passed, then the W
    # warmup steps. Both run the full step; neither is inside the timed region.
    settle_steps = 0
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        settle_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Whole-step timing: exactly `steps` steps between synchronisations.
    ms_step = timed(step, args.steps)
    # Each kernel's average launch duration: a captured HIP graph of `steps` back-to-back
    # launches of it, replayed (no host dispatch in the timed region; a short kernel timed
    # in a Python loop is bounded by the host's dispatch of each call instead). The
    # graph-replayed step is timed the same way.
    ms_k = {"attn_fwd": graph_timed(fwd, args.steps), "attn_bwd_dq": graph_timed(bwd_dq, args.steps),
            "attn_bwd_dkv": graph_timed(bwd_dkv, args.steps)}
    ms_step_graph = graph_timed(step, args.steps)
    # Each kernel's share of the step as the step runs it: a replayed graph of `steps`
    # steps less a replayed graph of `steps` steps without that kernel (the others keep
    # their order). A kernel alone back to back runs differently from the step (the
    # forward about 15% longer); events between the calls would add their own time.
    pair_ms = {"attn_fwd": graph_timed(lambda: (bwd_dq(), bwd_dkv()), args.steps),
               "attn_bwd_dq": graph_timed(lambda: (fwd(), bwd_dkv()), args.steps),
               "attn_bwd_dkv": graph_timed(lambda: (fwd(), bwd_dq()), args.steps)}
    ms_in_step = {k: ms_step_graph - v for k, v in pair_ms.items()}

    pairs = w.causal_pairs
    fl = {"attn_fwd": 4 * w.d * pairs, "attn_bwd_dq": 6 * w.d * pairs, "attn_bwd_dkv": 8 * w.d * pairs}
    step_flops = 14 * w.d * pairs
    value = step_flops / (ms_step * 1e-3) / 1e12
    fwd_tflops = fl["attn_fwd"] / (ms_k["attn_fwd"] * 1e-3) / 1e12
    bwd_ms = ms_k["attn_bwd_dq"] + ms_k["attn_bwd_dkv"]
    bwd_tflops = 10 * w.d * pairs / (bwd_ms * 1e-3) / 1e12
    dom = max(ms_k, key=ms_k.get)
    achieved = fl[dom] / (ms_k[dom] * 1e-3) / 1e12
    traffic = measured_traffic(dom)
    kernels = {}
    for name in ms_k:
        a = fl[name] / (ms_k[name] * 1e-3) / 1e12
        a_in = fl[name] / (ms_in_step[name] * 1e-3) / 1e12 if ms_in_step[name] > 0 else None
        kernels[name] = {"ms": round(ms_k[name], 5), "tflops": round(a, 2),
                         "frac": round(a / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(name),
                         "ms_in_step": round(ms_in_step[name], 5),
                         "frac_in_step": round(a_in / PEAK_BF16_TFLOPS, 4) if a_in else None}

    out = {
        "metric": "causal attention TFLOP/s fwd and fwd+bwd, % of bf16 MFMA peak, 1xMI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_graph": round(ms_step_graph, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 fwd, fp16 bwd",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                   "pass": "fwd+bwd", "inputs": "bf16 N(0,1), seed 3"},
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_pct_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_pct_peak_in_step": (round(100 * fl["attn_fwd"] / (ms_in_step["attn_fwd"] * 1e-3) / 1e12
                                       / PEAK_BF16_TFLOPS, 2) if ms_in_step["attn_fwd"] > 0 else None),
        "bwd_tflops": round(bwd_tflops, 2),
        "fwdbwd_pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "compute": "fwd bf16 matrix core; bwd fp16 matrix core (dO and dS scaled by powers of two); "
                   "fp32 accumulation and softmax",
        "kernel_timing": "kernels.ms: HIP events around a replayed HIP graph of `steps` back-to-back "
                         "launches of each; kernels.ms_in_step: a replayed graph of `steps` steps "
                         "less one of `steps` steps without the kernel; ms_per_step: the plain loop "
                         "of `steps` steps; ms_per_step_graph: a replayed graph of `steps` steps",
        "kernels": kernels,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": None,
    }
    if not args.no_naive:
        # The naive reference mode on the same inputs (outside the timed step): every
        # T x T probability goes through an fp32 workspace in HBM.
        ws = torch.empty((cg.attn_naive_workspace_bytes(w.B, w.T, w.Hq) // 4,), dtype=torch.float32,
                         device="cuda")
        def naive_fwd():
            cg.attn_naive_fwd(q, k, v, scale=w.scale, workspace=ws, stream=stream)
        def naive_bwd():
            cg.attn_naive_bwd(q, k, v, do, scale=w.scale, workspace=ws, stream=stream)
        naive_fwd(); naive_bwd()
        torch.cuda.synchronize()
        nf, nb = timed(naive_fwd, 3), timed(naive_bwd, 3)
        out["naive"] = {"fwd_ms": round(nf, 4), "bwd_ms": round(nb, 4),
                        "workspace_bytes": int(ws.numel() * 4),
                        "flash_speedup_fwd": round(nf / ms_k["attn_fwd"], 1),
                        "flash_speedup_bwd": round(nb / bwd_ms, 1)}
        del ws
    if not args.no_gemm:
        out["gemm"] = gemm_bench(w, graph_timed)
    if not args.no_rope:
        # Rotary embedding: the rotation pass of Q and K (HBM-bound: each element read and
        # written once, plus the tables), and the backward with dQ, dK turned back inside.
        c_np, s_np = si.rope_tables(w.T, w.d)
        rc, rs = torch.from_numpy(c_np).cuda(), torch.from_numpy(s_np).cuda()
        q_rot = torch.empty_like(q)
        k_rot = torch.empty_like(k)
        def rope_pass():
            cg.rope_qk(q, k, rc, rs, q_out=q_rot, k_out=k_rot)
        def bwd_rope():
            cg.attn_bwd_dq(q, k, v, o, do, lse, scale=w.scale, delta=delta, dq=dq, stream=stream, rope=(rc, rs))
            cg.attn_bwd_dkv(q, k, v, do, lse, delta, scale=w.scale, dk=dk, dv=dv, stream=stream, rope=(rc, rs))
        # The forward with Q and K turned as they are loaded (d = 64), against the pass
        # followed by the plain forward.
        fused = w.d == 64
        o_f, lse_f = torch.empty_like(o), torch.empty_like(lse)
        def fwd_rope():
            cg.attn_fwd(q, k, v, scale=w.scale, o=o_f, lse=lse_f, rope=(rc, rs))
        def pass_then_fwd():
            rope_pass()
            cg.attn_fwd(q_rot, k_rot, v, scale=w.scale, o=o_f, lse=lse_f)
        rope_pass(); bwd_rope()
        if fused:
            fwd_rope(); pass_then_fwd()
        torch.cuda.synchronize()
        ms_rope, ms_bwd_rope = graph_timed(rope_pass, args.steps), timed(bwd_rope, args.steps)
        fused_ms = {}
        if fused:
            fused_ms = {"fused_fwd_ms": round(graph_timed(fwd_rope, args.steps), 5),
                        "pass_then_fwd_ms": round(graph_timed(pass_then_fwd, args.steps), 5)}
        rope_bytes = 2 * 2 * w.B * w.T * (w.Hq + w.Hkv) * w.d + 2 * 4 * w.T * (w.d // 2)
        gbs = rope_bytes / (ms_rope * 1e-3) / 1e9
        out["rope"] = {"pass_ms": round(ms_rope, 5), "bytes": rope_bytes,
                       "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)},
                       "bwd_ms": round(ms_bwd_rope, 5), "bwd_plain_ms": round(bwd_ms, 5), **fused_ms}
    # The measured matrix-core peak (calibration kernel, the way the pages measure theirs):
    # one wave of workgroups (2 per CU, 8 waves per CU), every wave 4 independent chains of
    # 32x32x16 bf16 products on registers; HIP events around one launch; the kernel's own
    # shader-clock / 100 MHz counter ratio gives the clock the matrix cores ran at.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cb, ci = 2 * cus, 8192
    c_sink = torch.empty(cb * 256, dtype=torch.float32, device="cuda")
    c_clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    def calib():
        return cg.calib_mfma(cb, ci, stream=stream, sink=c_sink, clocks=c_clk)[2]
    for _ in range(3):
        calib_flops = calib()
    ms_calib = timed(calib, 4)
    assert bool((c_sink == ci / 64.0).all()), "calibration products are off"
    clk = c_clk.cpu().tolist()
    peak_meas = calib_flops / (ms_calib * 1e-3) / 1e12
    out["mfma_measured_peak"] = {
        "tflops": round(peak_meas, 1), "frac_of_spec": round(peak_meas / PEAK_BF16_TFLOPS, 4),
        "clock_ghz": round(clk[0] / (clk[1] * 1e-8) / 1e9, 3) if clk[1] else None,
        "method": f"cgqa_calib_mfma: {cb} workgroups x 4 waves (one wave of workgroups on {cus} CUs), "
                  f"4 independent chains of {ci} v_mfma_f32_32x32x16_bf16 per wave, no memory traffic; "
                  f"HIP events around one launch, median of {args.repeats}"}
    for name in kernels:
        kernels[name]["frac_measured_peak"] = round(kernels[name]["tflops"] / peak_meas, 4)
    out["roofline"]["frac_measured_peak"] = round(achieved / peak_meas, 4)
    out["fwdbwd_pct_measured_peak"] = round(100 * value / peak_meas, 2)
    del c_sink, c_clk

    if not args.no_configs:
        # Every workload: each kernel's share of a step as above, but from replays of captured
        # HIP graphs (the small workloads' kernels are shorter than their host dispatch);
        # credited flops per causal pair as above, against the spec and the measured peak.
        cfgs = {}
        for wi, wk in enumerate(si.WORKLOADS):
            xw = si.make_workload_inputs(wk, seed=wi + 1)
            dw = {n: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for n, a in xw.items()}
            del xw
            ow = torch.empty_like(dw["q"])
            lw = torch.empty((wk.B, wk.Hq, wk.T), dtype=torch.float32, device="cuda")
            dlw = cg.bwd_delta(wk.B, wk.Hq, wk.T, device="cuda")
            dqw = torch.empty((wk.B, wk.T, wk.Hq, wk.d), dtype=torch.float32, device="cuda")
            dkw = torch.empty((wk.B, wk.T, wk.Hkv, wk.d), dtype=torch.float32, device="cuda")
            dvw = torch.empty_like(dkw)
            # (launched on the current stream, which graph capture switches)
            fns = (lambda: cg.attn_fwd(dw["q"], dw["k"], dw["v"], scale=wk.scale, o=ow, lse=lw),
                   lambda: cg.attn_bwd_dq(dw["q"], dw["k"], dw["v"], ow, dw["do"], lw, scale=wk.scale,
                                          delta=dlw, dq=dqw),
                   lambda: cg.attn_bwd_dkv(dw["q"], dw["k"], dw["v"], dw["do"], lw, dlw, scale=wk.scale,
                                           dk=dkw, dv=dvw))
            n = 10 if wk.d * wk.causal_pairs > 5e10 else args.steps
            for _ in range(3):
                for fn in fns:
                    fn()
            torch.cuda.synchronize()
            ms3 = [graph_timed(fn, n) for fn in fns]
            st_ms = graph_timed(lambda: [fn() for fn in fns], n)
            entry = {"steps": n}
            for name, ms_, per_pair in zip(("attn_fwd", "attn_bwd_dq", "attn_bwd_dkv"), ms3, (4, 6, 8)):
                tf = per_pair * wk.d * wk.causal_pairs / (ms_ * 1e-3) / 1e12
                entry[name] = {"ms": round(ms_, 5), "tflops": round(tf, 1),
                               "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                               "pct_measured_peak": round(100 * tf / peak_meas, 2)}
            st_tf = 14 * wk.d * wk.causal_pairs / (st_ms * 1e-3) / 1e12
            entry["step"] = {"ms": round(st_ms, 5), "tflops": round(st_tf, 1),
                             "pct_peak": round(100 * st_tf / PEAK_BF16_TFLOPS, 2)}
            cfgs[wk.name] = entry
            del dw, ow, lw, dlw, dqw, dkw, dvw, fns
            torch.cuda.empty_cache()
        out["configs"] = cfgs

    if graph_failures:
        out["graph_capture_failed"] = graph_failures   # these were timed call by call instead
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
