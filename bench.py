#!/usr/bin/env python3
"""Benchmark of FourTune's W4A4G4 triple-branch linear on one MI355X.

One step = forward + backward of the FLUX fused-QKV linear (4608 tokens,
3072 -> 9216, stabilizer rank 32, LoRA rank 16) through the C ABI:
  fwd: quantize X + down-projection U  |  MXFP4 GEMM + U V epilogue -> Y
  bwd: quantize dY + down-projection P |  MXFP4 dgrad GEMM + P D^T -> dX
       | dA = X^T P_lora | dB = U_lora^T dY
Four independent input sets (X, dY, W_res, ...) are rotated across steps so
that no step finds the previous step's operands in the 256 MB last-level
cache.  The weight quantization (32x32 tiles) happens once per layer
before training and is not part of a step; it is timed separately on the
quantizer stress shapes together with the dual-layout activation quantizer.

Prints ONE JSON line.  `value` = algorithmic FLOP of the step / measured
step time.  The roofline entry is for the kernel with the largest share of
the step, timed with HIP events on the stream it runs on.  Beside the
headline the line carries: the oracle's CPU rate on the same layer
(cpu_baseline), the FLUX MLP pair with its GELU glue (mlp_pair), the fused
against the unfused low-rank branches (fusion_breakdown), all linears of a
DiT block (dit_block), the four precision settings of the precision
ablation (precision_settings), tiles against group-wise weights
(weight_block), the step at larger ranks (rank_variants) and the quantizers
at the stress shapes (quantizer_stress).

    python bench.py [--steps 50] [--warmup 10] [--gpus 1] [--only PART]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_FP4_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
METRIC = "W4A4G4 linear fwd+bwd TFLOP/s at FLUX shapes; % MXFP4 MFMA peak; quantizer GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--cpu-rows", type=int, default=4608,
                    help="tokens of the QKV layer the CPU oracle baseline runs")
    ap.add_argument("--cpu-reps", type=int, default=3,
                    help="timed repetitions of the CPU oracle step (the rate is their mean)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stress", action="store_true")
    ap.add_argument("--no-mlp", action="store_true")
    ap.add_argument("--no-fusion", action="store_true")
    ap.add_argument("--no-block", action="store_true")
    ap.add_argument("--no-precision", action="store_true")
    ap.add_argument("--no-wblock", action="store_true")
    ap.add_argument("--no-ranks", action="store_true")
    ap.add_argument("--graph-replay", action="store_true",
                    help="also time the step replayed from HIP graphs (reported beside the "
                         "direct launches)")
    ap.add_argument("--only", choices=["step", "stress", "mlp", "fusion", "block", "precision",
                                       "wblock", "ranks"],
                    default=None,
                    help="run only one part (for profiler runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain bf16 elementwise copy of known size (the reference "
                         "kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE to bytes)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print per-launch means of the counters of a rocprofv3 --pmc run of "
                         "this script (JSON), with derived matrix-core busy and wait fractions")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print per-launch HBM traffic (JSON) from two rocprofv3 --pmc runs of "
                         "this script with --copy-probe (FETCH_SIZE, then WRITE_SIZE) and exit")
    ap.add_argument("--summarize-pmc-kernels", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="as --summarize-pmc, but per kernel name (any section, e.g. --only "
                         "stress), printed as a markdown table, and exit")
    return ap.parse_args()


def layer_work(M, K, N, rs, rl):
    """Algorithmic FLOP and HBM bytes of each kernel of one fwd+bwd step.

    For adapter ranks up to 64 the dB product runs inside the backward
    quantize kernel (which reads dY anyway), so it is counted there and the
    adapter-gradient kernel reads only X for dA."""
    R = rs + rl
    db_fused = 0 < rl <= 64
    w = {
        "fwd_quant_down": {"flop": 2 * M * K * R,
                           "bytes": 2 * M * K + M * K // 2 + M * K // 32 + 2 * M * R + 2 * K * R,
                           "bound": "hbm"},
        "fwd_gemm": {"flop": 2 * M * N * K + 2 * M * R * N,
                     "mfma_flop": 2 * M * N * K,
                     "bytes": M * K // 2 + M * K // 32 + N * K // 2 + N * K // 1024 + 2 * M * R
                     + 2 * R * N + 2 * M * N,
                     "bound": "mfma"},
        "bwd_quant_down": {"flop": 2 * M * N * R + (2 * M * N * rl if db_fused else 0),
                           "bytes": 2 * M * N + M * N // 2 + M * N // 32 + 2 * M * R + 2 * N * R
                           + (2 * M * rl if db_fused else 0),
                           "bound": "hbm"},
        "bwd_gemm_dgrad": {"flop": 2 * M * N * K + 2 * M * R * K,
                           "mfma_flop": 2 * M * N * K,
                           "bytes": M * N // 2 + M * N // 32 + N * K // 2 + N * K // 1024
                           + 2 * M * R + 2 * R * K + 2 * M * K,
                           "bound": "mfma"},
        "bwd_lora_grads": {"flop": 2 * M * K * rl + (0 if db_fused else 2 * M * N * rl),
                           "bytes": 2 * M * K + 2 * M * rl + 2 * (K + N) * rl
                           + (0 if db_fused else 2 * M * N + 2 * M * rl),
                           "bound": "hbm"},
    }
    return w


def source_sha():
    h = hashlib.sha256()
    d = os.path.join(HERE, "bit_quantized_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, sha):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources."""
    p = os.path.join(HERE, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(kernel)
    if not e or e.get("source_sha") != sha:
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(rows, reps=1):
    """The oracle as it stands, on the first `rows` tokens of the same layer,
    run `reps` times back to back."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from bit_quantized_amd import synth
    from oracle import linear as OL
    from oracle import mxfp4 as OQ
    c = synth.qkv_case()
    rows = min(rows, c.M)
    wc, ws = OQ.quantize_tile32(c.W_res)   # offline weight prep, not timed
    X, dY = c.X[:rows], c.dY[:rows]
    t0 = time.perf_counter()
    for _ in range(reps):
        f = OL.linear_fwd(X, wc, ws, c.L1, c.L2, c.A, c.B)
        OL.linear_bwd(dY, X, f["U"], wc, ws, c.L1, c.L2, c.A, c.B)
    dt = (time.perf_counter() - t0) / reps
    flop = sum(v["flop"] for v in layer_work(rows, c.K, c.N, c.r_s, c.r_l).values())
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas_vendor = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in blas})) or None
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas_vendor,
            "seconds_per_step": round(dt, 3), "reps": reps,
            "sample": f"float64 numpy oracle, {reps} x forward+backward of the same QKV linear on "
                      f"its first {rows} of {c.M} tokens (X and dY quantization, both 4-bit products, "
                      f"low-rank branches, adapter gradients); the oracle's 32x32 weight "
                      f"quantization runs before the timer as offline preparation",
            "host_cpus": len(os.sched_getaffinity(0))}


# ------------------------------------------------------------ rocprofv3 summaries
def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name):
    """Kernel name without its argument list."""
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def summarize_trace(d):
    """Markdown table of a `rocprofv3 --kernel-trace --stats` run."""
    rows = _csv_rows(d, "kernel_stats.csv")
    out = ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% |")
    return "\n".join(out)


COPY_PROBE_ELEMS = 1 << 27      # bf16 elements of the reference copy (256 MiB each way)


def _step_kernel(kname, state):
    """Name of the step kernel a dispatch belongs to (None if it is not one).

    Dispatches are taken in order: each quantize + down-projection opens a
    new phase (forward, then backward), and the reduction kernel after it
    belongs to the same launch, as the adapter-gradient reduce belongs to
    the adapter-gradient launch.  Returns (name, opens_launch)."""
    if "k_quant_down" in kname:
        state["fwd"] = not state.get("fwd", False)
        return ("fwd_quant_down" if state["fwd"] else "bwd_quant_down"), True
    if "k_rank_reduce" in kname:
        return ("fwd_quant_down" if state.get("fwd") else "bwd_quant_down"), False
    if "k_gemm" in kname:
        return ("fwd_gemm" if state.get("fwd") else "bwd_gemm_dgrad"), True
    if "k_lora_reduce" in kname:
        return "bwd_lora_grads", False
    if "k_lora" in kname:
        return "bwd_lora_grads", True
    return None, False


def summarize_trace_by_step_kernel(d):
    """Mean duration per launch of each step kernel from a kernel trace
    (the quantize + down-projection launch is its two kernels together)."""
    rows = sorted(_csv_rows(d, "kernel_trace.csv"), key=lambda r: int(r["Dispatch_Id"]))
    tot, n, state = {}, {}, {}
    for r in rows:
        name, opens = _step_kernel(r["Kernel_Name"], state)
        if name is None:
            continue
        tot[name] = tot.get(name, 0.0) + (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        n[name] = n.get(name, 0) + int(opens)
    return {k: (round(tot[k] / n[k], 2), n[k]) for k in tot if n.get(k)}


def _pmc_per_step_kernel(d, counter):
    """Mean counter value per launch of each step kernel, and of the reference copy."""
    rows = sorted(_csv_rows(d, "counter_collection.csv"), key=lambda r: int(r["Dispatch_Id"]))
    acc, n_launch, state = {}, {}, {}
    copy = []
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        k, v = r["Kernel_Name"], float(r["Counter_Value"])
        if "neg_kernel" in k:
            copy.append(v)
            continue
        name, opens = _step_kernel(k, state)
        if name is None:
            continue
        acc[name] = acc.get(name, 0.0) + v
        n_launch[name] = n_launch.get(name, 0) + int(opens)
    per = {k: acc[k] / n_launch[k] for k in acc if n_launch.get(k)}
    return per, (sum(copy) / len(copy) if copy else None)


def summarize_counters(d):
    """Per step kernel, the mean of every counter of a `rocprofv3 --pmc` run
    per launch, with two derived fractions: matrix-core busy =
    SQ_VALU_MFMA_BUSY_CYCLES over the SIMD cycles of the launch (GRBM_GUI_ACTIVE,
    which counts each of the 8 XCDs, over 8, times 256 CUs x 4 SIMDs), and
    waiting = SQ_WAIT_ANY over SQ_WAVE_CYCLES."""
    rows = sorted(_csv_rows(d, "counter_collection.csv"), key=lambda r: int(r["Dispatch_Id"]))
    names = sorted({r["Counter_Name"] for r in rows})
    per = {}
    for c in names:
        vals, _ = _pmc_per_step_kernel(d, c)
        for k, v in vals.items():
            per.setdefault(k, {})[c] = v
    for k, cs in per.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" in cs and cs.get("GRBM_GUI_ACTIVE"):
            cs["mfma_busy_frac"] = cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (cs["GRBM_GUI_ACTIVE"] / 8 * 1024)
        if "SQ_WAIT_ANY" in cs and cs.get("SQ_WAVE_CYCLES"):
            cs["wait_frac"] = cs["SQ_WAIT_ANY"] / cs["SQ_WAVE_CYCLES"]
    return {k: {c: round(v, 4) for c, v in cs.items()} for k, cs in per.items()}


def summarize_pmc(fetch_dir, write_dir):
    """HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of each
    kernel, each divided by the same counter's reading per byte of a plain
    bf16 copy of COPY_PROBE_ELEMS elements."""
    fr, fc = _pmc_per_step_kernel(fetch_dir, "FETCH_SIZE")
    wr, wc = _pmc_per_step_kernel(write_dir, "WRITE_SIZE")
    if fc is None or wc is None:
        raise SystemExit("no reference copy in the counter runs (run them with --copy-probe)")
    nbytes = 2 * COPY_PROBE_ELEMS
    f_fac = fc * 1024 / nbytes
    w_fac = wc * 1024 / nbytes
    sha = source_sha()
    out = {"_scaling": {"copy_bytes_each_way": nbytes, "fetch_KiB_per_copy": fc,
                        "write_KiB_per_copy": wc, "fetch_factor": round(f_fac, 4),
                        "write_factor": round(w_fac, 4)}}
    for k in fr:
        fb = fr[k] * 1024 / f_fac
        wb = wr.get(k, 0.0) * 1024 / w_fac
        out[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                  "hbm_bytes_per_launch": round(fb + wb), "source_sha": sha}
    return out


def _pmc_per_kernel(d, counter):
    """Mean counter value per dispatch of each kernel name, and of the reference copy."""
    acc, n, copy = {}, {}, []
    for r in _csv_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        k, v = r["Kernel_Name"], float(r["Counter_Value"])
        if "neg_kernel" in k:
            copy.append(v)
            continue
        acc[k] = acc.get(k, 0.0) + v
        n[k] = n.get(k, 0) + 1
    return {k: acc[k] / n[k] for k in acc}, (sum(copy) / len(copy) if copy else None)


def summarize_pmc_kernels(fetch_dir, write_dir):
    """HBM bytes per dispatch of every library kernel (ft::), FETCH_SIZE and
    WRITE_SIZE scaled by the plain copy's reading, as a markdown table."""
    fr, fc = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    wr, wc = _pmc_per_kernel(write_dir, "WRITE_SIZE")
    if fc is None or wc is None:
        raise SystemExit("no reference copy in the counter runs (run them with --copy-probe)")
    nbytes = 2 * COPY_PROBE_ELEMS
    f_fac, w_fac = fc * 1024 / nbytes, wc * 1024 / nbytes
    lines = [f"copy probe: {nbytes} bytes each way; fetch factor {f_fac:.4f}, write factor {w_fac:.4f}; "
             f"kernel sources `source_sha` {source_sha()}", "",
             "| kernel | fetch MB | write MB | total MB |", "|---|---|---|---|"]
    for k in sorted(fr, key=lambda x: -fr[x]):
        name = k.replace("(anonymous namespace)::", "").split("(")[0].removeprefix("void ")
        if not name.startswith("ft::"):
            continue
        fb, wb = fr[k] * 1024 / f_fac / 1e6, wr.get(k, 0.0) * 1024 / w_fac / 1e6
        lines.append(f"| `{name}` | {fb:.1f} | {wb:.1f} | {fb + wb:.1f} |")
    return "\n".join(lines)


def copy_probe(dev, stream):
    import torch
    src = torch.ones(COPY_PROBE_ELEMS, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def time_graph_replay(step, sets, stream, e0, e1, a):
    """Mean step time (ms) of the layer step replayed from HIP graphs, one
    graph per input set, captured after a warm-up on a side stream."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(len(sets)):
            step(i, None)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(len(sets)):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step(i, None)
        graphs.append(gr)
    torch.cuda.synchronize()
    for i in range(a.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        graphs[i % len(graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    print(f"bench: graph replay {ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    return ms


def main():
    a = parse()
    if a.summarize_trace:
        print(summarize_trace(a.summarize_trace))
        print("\nPer step kernel (the quantize + down-projection launch is its two kernels):\n")
        print("| step kernel | launches | avg us |\n|---|---|---|")
        for k, (us, cnt) in summarize_trace_by_step_kernel(a.summarize_trace).items():
            print(f"| {k} | {cnt} | {us} |")
        return
    if a.summarize_pmc:
        print(json.dumps(summarize_pmc(*a.summarize_pmc), indent=1))
        return
    if a.summarize_pmc_kernels:
        print(summarize_pmc_kernels(*a.summarize_pmc_kernels))
        return
    if a.summarize_counters:
        print(json.dumps(summarize_counters(a.summarize_counters), indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: a step is one GPU's "
                                   "share of the layer, and no multi-GPU run is made",
                          "n_gpus": a.gpus}))
        sys.exit(2)

    import numpy as np
    import torch
    from bit_quantized_amd import ops, synth
    from bit_quantized_amd.layer import QuantizedLinear, bf16_tensor

    dev = torch.device("cuda:0")
    ops.lib()
    out = {"metric": METRIC}
    stream = torch.cuda.current_stream()

    def log(*x):
        print(*x, file=sys.stderr, flush=True)

    if a.copy_probe:
        copy_probe(dev, stream)

    # ------------------------------------------------------------ layer step
    c = synth.qkv_case()
    M, K, N, rs, rl = c.M, c.K, c.N, c.r_s, c.r_l
    work = layer_work(M, K, N, rs, rl)
    step_flop = sum(v["flop"] for v in work.values())
    if a.only in (None, "step"):
        log(f"bench: QKV linear M={M} K={K} N={N} r_s={rs} r_l={rl}, {a.sets} input sets")
        X0, dY0, W0 = (bf16_tensor(x, dev) for x in (c.X, c.dY, c.W_res))
        L1, L2, A, B = (bf16_tensor(x, dev) for x in (c.L1, c.L2, c.A, c.B))
        sets = []
        for s in range(a.sets):
            # distinct memory per set with the same values, rolled along tokens / rows
            X = torch.roll(X0, 97 * s, 0).contiguous()
            dY = torch.roll(dY0, 97 * s, 0).contiguous()
            W = torch.roll(W0, 32 * s, 0).contiguous()
            lay = QuantizedLinear.from_factors(W, L1.clone(), L2.clone(), A.clone(), B.clone())
            del W
            U = torch.empty((M, rs + rl), dtype=torch.bfloat16, device=dev)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
            dA = torch.empty((rl, K), dtype=torch.bfloat16, device=dev)   # dA^T, like A^T
            dB = torch.empty((rl, N), dtype=torch.bfloat16, device=dev)
            wsf = lay.workspace(M, False)
            wsb = lay.workspace(M, True)
            sets.append((lay, X, dY, U, Y, dX, dA, dB, wsf, wsb))
        del X0, dY0, W0
        torch.cuda.synchronize()

        def step(i, st=stream):
            lay, X, dY, U, Y, dX, dA, dB, wsf, wsb = sets[i % len(sets)]
            d = lay.desc(M)
            ops.fourtune_linear_fwd(d, X, Y, U, None, None, wsf, wsf.numel(), st)
            ops.fourtune_linear_bwd(d, dY, X, U, None, dX, dA, dB, ops.FT_BF16, None, None, None, wsb,
                                    wsb.numel(), st)

        for i in range(a.warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(a.steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / a.steps
        log(f"bench: {ms * 1e3:.1f} us/step, {step_flop / (ms * 1e-3) / 1e12:.1f} TFLOP/s")

        # Optionally, the same steps replayed from HIP graphs, one per input set
        # (the library records no memset, so a step is six kernel nodes).
        # Measured no faster than launching them one by one on this stack, so
        # the headline stays with the direct launches.
        ms_graph = None
        if a.graph_replay:
            ms_graph = time_graph_replay(step, sets, stream, e0, e1, a)

        # same steps again with every launch bracketed by HIP events
        ops.fourtune_timing_reset()
        ops.fourtune_timing_enable(True)
        e0.record(stream)
        for i in range(a.steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ops.fourtune_timing_enable(False)
        ms_instr = e0.elapsed_time(e1) / a.steps
        tm = ops.fourtune_timing_read()
        sha = source_sha()
        kernels = {}
        for name, (tot, cnt) in tm.items():
            if name not in work or cnt == 0:
                continue
            us = tot / cnt * 1e3
            wk = work[name]
            if wk["bound"] == "mfma":
                ach = wk["mfma_flop"] / (us * 1e-6) / 1e12
                kernels[name] = {"avg_us": round(us, 2), "launches": cnt, "bound": "mfma",
                                 "achieved": round(ach, 1), "peak": PEAK_FP4_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(ach / PEAK_FP4_TFLOPS, 4)}
            else:
                ach = wk["bytes"] / (us * 1e-6) / 1e9
                kernels[name] = {"avg_us": round(us, 2), "launches": cnt, "bound": "hbm",
                                 "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": round(ach / PEAK_HBM_GBS, 4)}
        if "bwd_lora_grads" not in kernels and "bwd_gemm_dgrad" in kernels:
            # the adapter gradients were made by the dgrad's launch on the
            # CUs its tiles leave free: no launch of their own
            kernels["bwd_lora_grads"] = {"avg_us": 0.0, "launches": 0, "bound": "hbm",
                                         "beside_dgrad": True,
                                         "note": "dA and dB made inside bwd_gemm_dgrad's launch on "
                                                 "the CUs its tiles leave free"}
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
        dk = kernels[dom]
        traffic = load_traffic(dom, sha)
        # the whole step against the sum of its kernels' roofline times: a
        # GEMM at the MXFP4 peak for its 4-bit FLOP plus the bf16 peak for its
        # fused low-rank FLOP, every other kernel at the HBM peak for its bytes
        roof_us = {}
        for name, wk in work.items():
            if wk["bound"] == "mfma":
                t = wk["mfma_flop"] / (PEAK_FP4_TFLOPS * 1e6) + \
                    (wk["flop"] - wk["mfma_flop"]) / (PEAK_BF16_TFLOPS * 1e6)
            else:
                t = wk["bytes"] / (PEAK_HBM_GBS * 1e3)
            roof_us[name] = round(t, 2)
        layer_roof = {"sum_roofline_us": round(sum(roof_us.values()), 2),
                      "step_us": round(ms * 1e3, 2),
                      "frac": round(sum(roof_us.values()) / (ms * 1e3), 4),
                      "per_kernel_roofline_us": roof_us}
        out.update({
            "value": round(step_flop / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4",
            "data": "synthetic",
            "config": {"workload": "flux_qkv_linear_fwd_bwd", "M": M, "K": K, "N": N,
                       "r_stab": rs, "r_lora": rl, "input_sets": a.sets,
                       "step_flop": step_flop},
            "roofline": {"kernel": dom, "bound": dk["bound"], "achieved": dk["achieved"],
                         "peak": dk["peak"], "unit": dk["unit"], "frac": dk["frac"],
                         "traffic": traffic},
            "kernels": kernels,
            "ms_per_step_graph_replay": None if ms_graph is None else round(ms_graph, 5),
            "ms_per_step_with_kernel_events": round(ms_instr, 5),
            "sum_kernel_us": round(sum(v["avg_us"] for v in kernels.values()), 2),
            "layer_roofline": layer_roof,
            "source_sha": sha,
        })
        del sets
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ MLP pair with GELU
    if not a.no_mlp and a.only in (None, "mlp"):
        Mm, Km, Fm, rsm, rlm = 4608, 3072, 12288, 32, 32
        log(f"bench: MLP pair M={Mm} {Km}->{Fm}->GELU->{Km}, ranks {rsm}/{rlm}")
        c1 = synth.flux_linear_case("mlp_fc1", Mm, Km, Fm, rsm, rlm, seed=2)
        c2 = synth.flux_linear_case("mlp_fc2", Mm, Fm, Km, rsm, rlm, seed=3)
        up = lambda x: bf16_tensor(x, dev)
        msets = []
        for s_ in range(2):
            fc1 = QuantizedLinear.from_factors(torch.roll(up(c1.W_res), 32 * s_, 0).contiguous(),
                                               up(c1.L1), up(c1.L2), up(c1.A), up(c1.B),
                                               act_out=ops.FT_ACT_GELU_TANH)
            fc2 = QuantizedLinear.from_factors(torch.roll(up(c2.W_res), 32 * s_, 0).contiguous(),
                                               up(c2.L1), up(c2.L2), up(c2.A), up(c2.B),
                                               act_in=ops.FT_ACT_GELU_TANH)
            X1 = torch.roll(up(c1.X), 97 * s_, 0).contiguous()
            dY2 = torch.roll(up(c2.dY), 97 * s_, 0).contiguous()
            bt = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device=dev)
            bufs = dict(h=bt(Mm, Fm), U1=bt(Mm, rsm + rlm), Y2=bt(Mm, Km), U2=bt(Mm, rsm + rlm),
                        dX2=bt(Mm, Fm), dA2=bt(rlm, Fm), dB2=bt(rlm, Km), dX1=bt(Mm, Km),
                        dA1=bt(rlm, Km), dB1=bt(rlm, Fm))
            ws = {k: (lay.workspace(Mm, False), lay.workspace(Mm, True)) for k, lay in (("1", fc1), ("2", fc2))}
            nmlp = ops.fourtune_mlp_workspace_bytes(fc1.desc(Mm), fc2.desc(Mm))
            ws["mlp"] = torch.empty(nmlp, dtype=torch.uint8, device=dev)
            nmlpb = ops.fourtune_mlp_bwd_workspace_bytes(fc1.desc(Mm), fc2.desc(Mm))
            ws["mlp_bwd"] = torch.empty(nmlpb, dtype=torch.uint8, device=dev)
            msets.append((fc1, fc2, X1, dY2, bufs, ws))
        del c1, c2
        torch.cuda.synchronize()

        # variants: 0 the two linears one after the other; 1 the MLP fusion of
        # the pages (fourtune_mlp_fwd: FC1's GEMM epilogue makes FC2's quantized
        # input and down-projection sums); 2 that and its mirror in the backward
        # (fourtune_mlp_bwd: FC2's dgrad epilogue makes FC1's incoming gradient,
        # its quantization and its down-projection sums)
        def mlp_step(i, var=0):
            fc1, fc2, X1, dY2, b, ws = msets[i % len(msets)]
            d1, d2 = fc1.desc(Mm), fc2.desc(Mm)
            (w1f, w1b), (w2f, w2b) = ws["1"], ws["2"]
            if var:
                wm = ws["mlp"]
                ops.fourtune_mlp_fwd(d1, d2, X1, b["h"], b["Y2"], b["U1"], b["U2"], None, None, wm,
                                     wm.numel(), stream)
            else:
                ops.fourtune_linear_fwd(d1, X1, b["h"], b["U1"], None, None, w1f, w1f.numel(), stream)
                ops.fourtune_linear_fwd(d2, b["h"], b["Y2"], b["U2"], None, None, w2f, w2f.numel(),
                                        stream)
            if var == 2:
                wmb = ws["mlp_bwd"]
                ops.fourtune_mlp_bwd(d1, d2, dY2, X1, b["h"], b["U1"], b["U2"], b["dX1"], b["dA1"],
                                     b["dB1"], b["dA2"], b["dB2"], ops.FT_BF16, wmb, wmb.numel(),
                                     stream)
            else:
                ops.fourtune_linear_bwd(d2, dY2, b["h"], b["U2"], None, b["dX2"], b["dA2"], b["dB2"],
                                        ops.FT_BF16, None, None, None, w2b, w2b.numel(), stream)
                ops.fourtune_linear_bwd(d1, b["dX2"], X1, b["U1"], b["h"], b["dX1"], b["dA1"],
                                        b["dB1"], ops.FT_BF16, None, None, None, w1b, w1b.numel(),
                                        stream)

        nst = max(5, a.steps // 5)
        for i in range(3):
            for var in range(3):
                mlp_step(i, var)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # the variants in rotating order over rounds (median per variant), so
        # that clock drift favours none
        t_var = {0: [], 1: [], 2: []}
        for rnd in range(6):
            for k in range(3):
                var = (rnd + k) % 3
                e0.record(stream)
                for i in range(nst):
                    mlp_step(i, var)
                e1.record(stream)
                torch.cuda.synchronize()
                t_var[var].append(e0.elapsed_time(e1) / nst)
        mms = statistics.median(t_var[0])
        mms_fused = statistics.median(t_var[1])
        mms_both = statistics.median(t_var[2])
        w1 = layer_work(Mm, Km, Fm, rsm, rlm)
        w2 = layer_work(Mm, Fm, Km, rsm, rlm)
        mflop = sum(v["flop"] for v in w1.values()) + sum(v["flop"] for v in w2.values())
        per_var = {}
        for var in range(3):
            ops.fourtune_timing_reset()
            ops.fourtune_timing_enable(True)
            for i in range(nst):
                mlp_step(i, var)
            torch.cuda.synchronize()
            ops.fourtune_timing_enable(False)
            per_var[var] = {k: round(tot / cnt * 1e3, 2)
                            for k, (tot, cnt) in ops.fourtune_timing_read().items() if cnt}
        out["mlp_pair"] = {
            "workload": f"FLUX MLP pair fwd+bwd: {Mm} tokens, {Km}->{Fm} -> tanh-GELU -> {Fm}->{Km}, "
                        f"r_stab={rsm}, r_lora={rlm}; GELU applied inside the quantizers and the "
                        f"adapter-gradient kernel",
            "us_per_step": round(mms * 1e3, 1), "TFLOP/s": round(mflop / (mms * 1e-3) / 1e12, 1),
            "step_flop": mflop, "steps": nst,
            "mlp_fused_us_per_step": round(mms_fused * 1e3, 1),
            "mlp_fusion_speedup": round(mms / mms_fused, 3),
            "mlp_fused_fwd_bwd_us_per_step": round(mms_both * 1e3, 1),
            "mlp_fused_fwd_bwd_speedup": round(mms / mms_both, 3),
            "kernel_avg_us_both_linears": per_var[0],
            "kernel_avg_us_both_linears_mlp_fused": per_var[1],
            "kernel_avg_us_both_linears_mlp_fused_fwd_bwd": per_var[2]}
        log("bench: mlp", json.dumps(out["mlp_pair"]))
        del msets
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ fusion breakdown
    # The same QKV step with the low-rank branches unfused: the library's
    # 4-bit path without ranks (quantize + 4-bit GEMM, forward and dgrad) and
    # each low-rank product as a separate bf16 matrix product, each branch sum
    # as a separate elementwise add.  Against the fused step this is the
    # "LoRA fusion" factor of the pages' fusion breakdown (section 4, Fig. 9).
    if not a.no_fusion and a.only in (None, "fusion"):
        c = synth.qkv_case()
        M, K, N, rs, rl = c.M, c.K, c.N, c.r_s, c.r_l
        log(f"bench: fusion breakdown, QKV linear M={M} K={K} N={N} r_s={rs} r_l={rl}")
        up = lambda x: bf16_tensor(x, dev)
        bt = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device=dev)
        fsets = []
        for s_ in range(2):
            X = torch.roll(up(c.X), 97 * s_, 0).contiguous()
            dY = torch.roll(up(c.dY), 97 * s_, 0).contiguous()
            W = torch.roll(up(c.W_res), 32 * s_, 0).contiguous()
            L1, L2, A, B = up(c.L1), up(c.L2), up(c.A), up(c.B)
            fused = QuantizedLinear.from_factors(W, L1, L2, A, B)
            plain = QuantizedLinear.from_factors(W, None, None, None, None)
            del W
            D = torch.cat([L1, A], 1).contiguous()          # [K, R]
            V = torch.cat([L2, B], 0).contiguous()          # [R, N]
            b = dict(X=X, dY=dY, D=D, V=V, Dt=D.t().contiguous(), Vt=V.t().contiguous(),
                     U=bt(M, rs + rl), Y=bt(M, N), T=bt(M, N), dX=bt(M, K), T2=bt(M, K),
                     P=bt(M, rs + rl), dA=bt(rl, K), dB=bt(rl, N), dAk=bt(K, rl))
            ws = (fused.workspace(M, False), fused.workspace(M, True),
                  plain.workspace(M, False), plain.workspace(M, True))
            fsets.append((fused, plain, b, ws))
        torch.cuda.synchronize()

        def fused_step(i):
            fused, _, b, (wf, wb, _, _) = fsets[i % 2]
            d = fused.desc(M)
            ops.fourtune_linear_fwd(d, b["X"], b["Y"], b["U"], None, None, wf, wf.numel(), stream)
            ops.fourtune_linear_bwd(d, b["dY"], b["X"], b["U"], None, b["dX"], b["dA"], b["dB"],
                                    ops.FT_BF16, None, None, None, wb, wb.numel(), stream)

        def unfused_step(i):
            _, plain, b, (_, _, pf, pb) = fsets[i % 2]
            d = plain.desc(M)
            ops.fourtune_linear_fwd(d, b["X"], b["Y"], None, None, None, pf, pf.numel(), stream)
            torch.matmul(b["X"], b["D"], out=b["U"])                       # U = X [L1|A]
            torch.matmul(b["U"], b["V"], out=b["T"])                       # U [L2;B]
            b["Y"].add_(b["T"])
            ops.fourtune_linear_bwd(d, b["dY"], b["X"], None, None, b["dX"], None, None,
                                    ops.FT_BF16, None, None, None, pb, pb.numel(), stream)
            torch.matmul(b["dY"], b["Vt"], out=b["P"])                     # P = dY [L2;B]^T
            torch.matmul(b["P"], b["Dt"], out=b["T2"])                     # P [L1|A]^T
            b["dX"].add_(b["T2"])
            torch.matmul(b["X"].t(), b["P"][:, rs:], out=b["dAk"])         # dA = X^T (dY B^T)
            torch.matmul(b["U"][:, rs:].t(), b["dY"], out=b["dB"])         # dB = (X A)^T dY

        res = {}
        nst = max(5, a.steps // 5)
        for name, fn in (("fused_us", fused_step), ("unfused_us", unfused_step)):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(nst):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = round(e0.elapsed_time(e1) / nst * 1e3, 1)
        out["fusion_breakdown"] = {
            "workload": f"QKV linear fwd+bwd, {M} tokens, {K}->{N}, r_stab={rs}, r_lora={rl}",
            "unfused": "library 4-bit quantize + GEMM without ranks; low-rank products as separate "
                       "bf16 matrix products (torch / hipBLASLt) and separate elementwise adds",
            **res, "lora_fusion_speedup": round(res["unfused_us"] / res["fused_us"], 3), "steps": nst}
        log("bench: fusion", json.dumps(out["fusion_breakdown"]))
        del fsets
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ DiT block
    # Every linear of one double-stream DiT block at batch 2: per stream QKV,
    # out-projection and the MLP pair (GELU glue), plus the modulation linear
    # at M = 2; forward of all, then backward of all.  Inputs are drawn on the
    # device (the kernels' timing does not depend on the values).
    if not a.no_block and a.only in (None, "block"):
        rs_, rl_ = 32, 16
        g = torch.Generator(device=dev)
        g.manual_seed(6)
        rnd = lambda *sh, sc=1.0: (torch.randn(sh, generator=g, device=dev) * sc).to(torch.bfloat16)
        bt = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device=dev)
        blk, bflop = [], 0
        for name, Mb, Kb, Nb in synth.dit_block_linears():
            act_in = ops.FT_ACT_GELU_TANH if name.endswith("fc2") else ops.FT_ACT_NONE
            act_out = ops.FT_ACT_GELU_TANH if name.endswith("fc1") else ops.FT_ACT_NONE
            Wb, L1b, L2b, Ab, Bb = (rnd(Nb, Kb, sc=0.02), rnd(Kb, rs_, sc=0.1), rnd(rs_, Nb, sc=0.1),
                                    rnd(Kb, rl_, sc=0.01), rnd(rl_, Nb, sc=0.01))
            lay = QuantizedLinear.from_factors(Wb, L1b, L2b, Ab, Bb, act_in=act_in, act_out=act_out)
            # the same layer without ranks, for the unfused variant below
            plain = QuantizedLinear.from_factors(Wb, None, None, None, None, act_in=act_in,
                                                 act_out=act_out)
            Db = torch.cat([L1b, Ab], 1).contiguous()
            Vb = torch.cat([L2b, Bb], 0).contiguous()
            del Wb
            blk.append(dict(name=name, M=Mb, lay=lay, X=rnd(Mb, Kb), dY=rnd(Mb, Nb, sc=1e-3),
                            Y=bt(Mb, Nb), U=bt(Mb, rs_ + rl_), dX=bt(Mb, Kb), dA=bt(rl_, Kb),
                            dB=bt(rl_, Nb), wf=lay.workspace(Mb, False), wb=lay.workspace(Mb, True),
                            plain=plain, D=Db, V=Vb, Dt=Db.t().contiguous(), Vt=Vb.t().contiguous(),
                            pf=plain.workspace(Mb, False), pb=plain.workspace(Mb, True),
                            act_in=act_in != ops.FT_ACT_NONE, act_out=act_out != ops.FT_ACT_NONE))
            bflop += sum(v["flop"] for v in layer_work(Mb, Kb, Nb, rs_, rl_).values())
        by = {e["name"]: e for e in blk}
        for st_ in ("img", "txt"):          # fc2 reads fc1's output h; fc1's gradient is fc2's dX
            by[st_ + "_fc2"]["X"] = by[st_ + "_fc1"]["Y"]
            by[st_ + "_fc1"]["dY"] = by[st_ + "_fc2"]["dX"]
        torch.cuda.synchronize()

        mlp_ws, mlp_wsb = {}, {}
        for st_ in ("img", "txt"):
            f1, f2 = by[st_ + "_fc1"], by[st_ + "_fc2"]
            dd1, dd2 = f1["lay"].desc(f1["M"]), f2["lay"].desc(f2["M"])
            n_ = ops.fourtune_mlp_workspace_bytes(dd1, dd2)
            mlp_ws[st_] = torch.empty(n_, dtype=torch.uint8, device=dev)
            n_ = ops.fourtune_mlp_bwd_workspace_bytes(dd1, dd2)
            mlp_wsb[st_] = torch.empty(n_, dtype=torch.uint8, device=dev)

        # mlp_fused: 1 the forward MLP fusion, 2 also its mirror in the backward
        def block_step(mlp_fused=0):
            for e in blk:
                nm = e["name"]
                if mlp_fused and nm.endswith("fc2"):
                    continue                      # made together with its fc1 below
                if mlp_fused and nm.endswith("fc1"):
                    e2 = by[nm[:4] + "fc2"]
                    w_ = mlp_ws[nm[:3]]
                    ops.fourtune_mlp_fwd(e["lay"].desc(e["M"]), e2["lay"].desc(e2["M"]), e["X"], e["Y"],
                                         e2["Y"], e["U"], e2["U"], None, None, w_, w_.numel(), stream)
                    continue
                d = e["lay"].desc(e["M"])
                ops.fourtune_linear_fwd(d, e["X"], e["Y"], e["U"], None, None, e["wf"], e["wf"].numel(),
                                        stream)
            for e in reversed(blk):
                nm = e["name"]
                if mlp_fused == 2 and nm.endswith("fc1"):
                    continue                      # made together with its fc2 below
                if mlp_fused == 2 and nm.endswith("fc2"):
                    e1 = by[nm[:4] + "fc1"]
                    w_ = mlp_wsb[nm[:3]]
                    ops.fourtune_mlp_bwd(e1["lay"].desc(e1["M"]), e["lay"].desc(e["M"]), e["dY"],
                                         e1["X"], e1["Y"], e1["U"], e["U"], e1["dX"], e1["dA"],
                                         e1["dB"], e["dA"], e["dB"], ops.FT_BF16, w_, w_.numel(),
                                         stream)
                    continue
                d = e["lay"].desc(e["M"])
                H = by[nm[:4] + "fc1"]["Y"] if nm.endswith("fc1") else None
                ops.fourtune_linear_bwd(d, e["dY"], e["X"], e["U"], H, e["dX"], e["dA"], e["dB"],
                                        ops.FT_BF16, None, None, None, e["wb"], e["wb"].numel(), stream)

        for _ in range(2):
            for v_ in range(3):
                block_step(mlp_fused=v_)
        torch.cuda.synchronize()
        nst = max(3, a.steps // 10)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_blk = {0: [], 1: [], 2: []}
        for rnd in range(4):
            for k_ in range(3):
                v_ = (rnd + k_) % 3
                e0.record(stream)
                for _ in range(nst):
                    block_step(mlp_fused=v_)
                e1.record(stream)
                torch.cuda.synchronize()
                t_blk[v_].append(e0.elapsed_time(e1) / nst)
        bms = statistics.median(t_blk[0])
        bms_all = statistics.median(t_blk[1])
        bms_all2 = statistics.median(t_blk[2])
        # each linear on its own: fwd and bwd, event-timed over the same
        # number of repetitions (the modulation linears run the split GEMMs)
        per_lin = {}
        for e in blk:
            d = e["lay"].desc(e["M"])
            H = by[e["name"][:4] + "fc1"]["Y"] if e["name"].endswith("fc1") else None

            def lf(e=e, d=d):
                ops.fourtune_linear_fwd(d, e["X"], e["Y"], e["U"], None, None, e["wf"], e["wf"].numel(),
                                        stream)

            def lb(e=e, d=d, H=H):
                ops.fourtune_linear_bwd(d, e["dY"], e["X"], e["U"], H, e["dX"], e["dA"], e["dB"],
                                        ops.FT_BF16, None, None, None, e["wb"], e["wb"].numel(), stream)
            ent = {}
            for kind, fn in (("fwd", lf), ("bwd", lb)):
                fn()
                e0.record(stream)
                for _ in range(nst):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ent[kind + "_us"] = round(e0.elapsed_time(e1) / nst * 1e3, 1)
            per_lin[e["name"]] = ent
        # The block with the low-rank branches unfused (the pages' fusion
        # breakdown, section 4, Fig. 9, at block level): per linear the
        # library's 4-bit path without ranks (quantize + GEMM; GELU still
        # inside its quantizers) and every low-rank product, GELU of the
        # branch input and branch sum as separate torch operations.
        def unfused_block():
            for e in blk:
                d = e["plain"].desc(e["M"])
                ops.fourtune_linear_fwd(d, e["X"], e["Y"], None, None, None, e["pf"], e["pf"].numel(),
                                        stream)
                xa = torch.nn.functional.gelu(e["X"], approximate="tanh") if e["act_in"] else e["X"]
                torch.matmul(xa, e["D"], out=e["U"])
                e["Y"].add_(torch.matmul(e["U"], e["V"]))
            for e in reversed(blk):
                d = e["plain"].desc(e["M"])
                H = by[e["name"][:4] + "fc1"]["Y"] if e["name"].endswith("fc1") else None
                ops.fourtune_linear_bwd(d, e["dY"], e["X"], None, H, e["dX"], None, None, ops.FT_BF16,
                                        None, None, None, e["pb"], e["pb"].numel(), stream)
                gr = (torch.ops.aten.gelu_backward(e["dY"], H, approximate="tanh") if e["act_out"]
                      else e["dY"])
                xa = torch.nn.functional.gelu(e["X"], approximate="tanh") if e["act_in"] else e["X"]
                P = torch.matmul(gr, e["Vt"])
                e["dX"].add_(torch.matmul(P, e["Dt"]))
                e["dA"].copy_(torch.matmul(xa.t(), P[:, rs_:].contiguous()).t())
                torch.matmul(e["U"][:, rs_:].t(), gr, out=e["dB"])

        for _ in range(2):
            unfused_block()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(nst):
            unfused_block()
        e1.record(stream)
        torch.cuda.synchronize()
        ums = e0.elapsed_time(e1) / nst
        out["fusion_breakdown_block"] = {
            "workload": "the DiT block above (every linear, fwd+bwd)",
            "unfused_us": round(ums * 1e3, 1),
            "lora_fused_us": round(bms * 1e3, 1),
            "all_fused_us": round(bms_all * 1e3, 1),
            "all_fused_with_mirrored_backward_us": round(bms_all2 * 1e3, 1),
            "lora_fusion_speedup": round(ums / bms, 3),
            "mlp_fusion_speedup": round(bms / bms_all, 3),
            "all_fusion_speedup": round(ums / bms_all, 3)}
        log("bench: block fusion", json.dumps(out["fusion_breakdown_block"]))
        out["dit_block"] = {
            "workload": "all linears of one double-stream DiT block at batch 2, fwd+bwd: per stream "
                        "(image 8192 tokens, text 1024) QKV 3072->9216, out-projection 3072->3072, "
                        "MLP 3072->12288->GELU->3072, and the modulation linear 3072->18432 at M=2; "
                        "r_stab=32, r_lora=16",
            "us_per_step": round(bms * 1e3, 1), "TFLOP/s": round(bflop / (bms * 1e-3) / 1e12, 1),
            "step_flop": bflop, "steps": nst, "per_linear": per_lin}
        log("bench: block", json.dumps(out["dit_block"]))
        del blk, by
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ layer variants
    # The QKV step (fwd+bwd) with the layer built in several ways, timed in
    # interleaved rounds (median over rounds) so that clock drift during the
    # run does not favour one variant: two rotated input sets per variant.
    # A variant's "ranks": (r_stab, r_lora) other than the QKV case's 32/16,
    # with factors drawn the same way (the inputs and the weight are the same).
    def qkv_variants(kws, rounds=3):
        c = synth.qkv_case()
        M, K, N, rs, rl = c.M, c.K, c.N, c.r_s, c.r_l
        X0, dY0, W0 = (bf16_tensor(x, dev) for x in (c.X, c.dY, c.W_res))
        factors = {(rs, rl): tuple(bf16_tensor(x, dev) for x in (c.L1, c.L2, c.A, c.B))}
        bt = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device=dev)
        sets = {}
        for name, kw in kws.items():
            kw = dict(kw)
            vrs, vrl = kw.pop("ranks", (rs, rl))
            if (vrs, vrl) not in factors:
                vc = synth.flux_linear_case(f"qkv_r{vrs}_{vrl}", 8, K, N, vrs, vrl, seed=1)
                factors[(vrs, vrl)] = tuple(bf16_tensor(x, dev) for x in (vc.L1, vc.L2, vc.A, vc.B))
            L1, L2, A, B = factors[(vrs, vrl)]
            sets[name] = []
            for s_ in range(2):
                lay = QuantizedLinear.from_factors(torch.roll(W0, 32 * s_, 0).contiguous(), L1, L2, A, B, **kw)
                sets[name].append((lay, torch.roll(X0, 97 * s_, 0).contiguous(),
                                   torch.roll(dY0, 97 * s_, 0).contiguous(), bt(M, vrs + vrl), bt(M, N),
                                   bt(M, K), bt(vrl, K), bt(vrl, N), lay.workspace(M, False),
                                   lay.workspace(M, True)))
        torch.cuda.synchronize()

        def vstep(name, i):
            lay, X, dY, U, Y, dX, dA, dB, wsf, wsb = sets[name][i % 2]
            d = lay.desc(M)
            ops.fourtune_linear_fwd(d, X, Y, U, None, None, wsf, wsf.numel(), stream)
            ops.fourtune_linear_bwd(d, dY, X, U, None, dX, dA, dB, ops.FT_BF16, None, None, None,
                                    wsb, wsb.numel(), stream)

        nst = max(5, a.steps // 5)
        times = {name: [] for name in kws}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for name in kws:
            for i in range(3):
                vstep(name, i)
        torch.cuda.synchronize()
        for _ in range(rounds):
            for name in kws:
                e0.record(stream)
                for i in range(nst):
                    vstep(name, i)
                e1.record(stream)
                torch.cuda.synchronize()
                times[name].append(e0.elapsed_time(e1) / nst * 1e3)
        res = {}
        for name in kws:
            ops.fourtune_timing_reset()
            ops.fourtune_timing_enable(True)
            for i in range(nst):
                vstep(name, i)
            torch.cuda.synchronize()
            ops.fourtune_timing_enable(False)
            per = {k: round(tot / cnt * 1e3, 2) for k, (tot, cnt) in ops.fourtune_timing_read().items()
                   if cnt}
            res[name] = {"us_per_step": round(float(np.median(times[name])), 1),
                         "us_per_step_rounds": [round(t, 1) for t in times[name]],
                         "kernel_avg_us": per}
        extra = (sets, W0, (M, K, N, rs, rl))
        return res, extra

    # ------------------------------------------------------------ precision settings
    # The four precision settings of the pages' precision ablation (section
    # 4.3, Table 4).  A 16-bit side multiplies bf16 by the weight tiles
    # dequantized to bf16 in each call (as QLoRA-style training does), on the
    # bf16 matrix cores.
    if not a.no_precision and a.only in (None, "precision"):
        names = ("W4A4G4", "W4A16G4", "W4A4G16", "W4A16G16")
        res, (sets_, W0, (M, K, N, rs, rl)) = qkv_variants({n: {"precision": n} for n in names})
        wk = layer_work(M, K, N, rs, rl)
        pflop = sum(v["flop"] for v in wk.values())
        for pname, ent in res.items():
            ent["TFLOP/s"] = round(pflop / (ent["us_per_step"] * 1e-6) / 1e12, 1)
            per = ent["kernel_avg_us"]
            # a 16-bit product runs on the bf16 matrix cores: its own peak
            for kname, on in (("fwd_gemm", "A16" in pname), ("bwd_gemm_dgrad", "G16" in pname)):
                if on and kname in per:
                    ach = wk[kname]["mfma_flop"] / (per[kname] * 1e-6) / 1e12
                    ent[kname + "_bf16"] = {"achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                                            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
            log("bench: precision", pname, json.dumps(ent))
        base = res["W4A4G4"]["us_per_step"]
        out["precision_settings"] = {
            "workload": f"QKV linear fwd+bwd (M={M}, K={K}, N={N}, r_stab={rs}, r_lora={rl}) in the "
                        "precision settings of the precision ablation; 16-bit sides read the weight "
                        "tiles dequantized to bf16 by each call; interleaved rounds, median",
            **res,
            "time_vs_W4A4G4": {k: round(v["us_per_step"] / base, 3) for k, v in res.items()}}
        del sets_, W0
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ weight layout
    # The QKV step with the residual weight stored three ways: the method's
    # 32x32 tiles stored once, the dgrad reading the same bytes transposed
    # (section 3.2); the same tiles plus a stored transposed layout copy that
    # the dgrad reads row-wise (twice the resident 4-bit bytes); and the
    # group-wise 1x32 blocks of the block-shape ablation (section 4.3,
    # "Impact of Quantization Granularity", Table 5), which need W and W^T
    # quantized separately.  weight_bytes: resident codes and scales.
    if not a.no_wblock and a.only in (None, "wblock"):
        variants = ("tile32", "tile32_t", "row32")
        res, (sets_, W0, (M, K, N, rs, rl)) = qkv_variants({w: {"w_block": w} for w in variants})
        pflop = sum(v["flop"] for v in layer_work(M, K, N, rs, rl).values())
        nst = max(5, a.steps // 5)
        for wbk, ent in res.items():
            ent["TFLOP/s"] = round(pflop / (ent["us_per_step"] * 1e-6) / 1e12, 1)
            lay = sets_[wbk][0][0]
            mode = ops.FT_Q_ROW32_T if wbk == "row32" else ops.FT_Q_TILE32
            qname = "quant_row32_t" if wbk == "row32" else "quant_tile32"
            ops.fourtune_timing_reset()
            ops.fourtune_timing_enable(True)
            for _ in range(nst):
                ops.fourtune_quantize(mode, W0, N, K, K, lay.w_codes, lay.w_scales, lay.wt_codes,
                                      lay.wt_scales, stream=stream)
            torch.cuda.synchronize()
            ops.fourtune_timing_enable(False)
            tot, cnt = ops.fourtune_timing_read()[qname]
            ent["weight_prep_us"] = round(tot / cnt * 1e3, 2)
            ent["weight_bytes"] = lay.weight_bytes()
            ent["dgrad_us"] = ent["kernel_avg_us"].get("bwd_gemm_dgrad")
            log("bench: wblock", wbk, json.dumps(ent))
        out["weight_block"] = {
            "workload": f"QKV linear fwd+bwd (M={M}, K={K}, N={N}, r_stab={rs}, r_lora={rl}) with the "
                        "residual weight as 32x32 tiles stored once (the method: the dgrad reads them "
                        "transposed), the tiles plus a stored transposed copy (tile32_t), or 1x32 "
                        "groups along each product's reduction (row32, both orientations stored); "
                        f"weight_prep_us quantizes the bf16 weight [{N}, {K}] into the stored "
                        "layouts; interleaved rounds, median",
            **res,
            "step_time_vs_tile32": {w: round(res[w]["us_per_step"] / res["tile32"]["us_per_step"], 3)
                                    for w in variants}}
        del sets_, W0
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ ranks
    # The QKV step at larger stabilizer and adapter ranks: above R = 64 the
    # GEMMs take four 32-rank steps per tile instead of two and the fused
    # quantizer 5 to 8 rank groups.
    if not a.no_ranks and a.only in (None, "ranks"):
        variants = {"r32_16": (32, 16), "r32_32": (32, 32), "r32_64": (32, 64), "r64_64": (64, 64)}
        res, (sets_, W0, (M, K, N, rs, rl)) = qkv_variants({k: {"ranks": v} for k, v in variants.items()})
        for name, (vrs, vrl) in variants.items():
            ent = res[name]
            pflop = sum(v["flop"] for v in layer_work(M, K, N, vrs, vrl).values())
            ent["r_stab"], ent["r_lora"] = vrs, vrl
            ent["TFLOP/s"] = round(pflop / (ent["us_per_step"] * 1e-6) / 1e12, 1)
            log("bench: ranks", name, json.dumps(ent))
        out["rank_variants"] = {
            "workload": f"QKV linear fwd+bwd (M={M}, K={K}, N={N}) at stabilizer/adapter ranks "
                        "32/16 (the benchmark's), 32/32, 32/64 and 64/64; TFLOP/s counts each "
                        "variant's own rank work; interleaved rounds, median",
            **res,
            "step_time_vs_r32_16": {k: round(res[k]["us_per_step"] / res["r32_16"]["us_per_step"], 3)
                                    for k in variants}}
        del sets_, W0
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ quantizer stress
    if not a.no_stress and a.only in (None, "stress"):
        rows, cols, wn = 16384, 12288, 12288
        g = torch.Generator(device=dev)
        g.manual_seed(4)
        log("bench: quantizer stress shapes")
        T = torch.randn((rows, cols), generator=g, device=dev)
        chi = sum(torch.randn((rows, cols), generator=g, device=dev) ** 2 for _ in range(3)) / 3.0
        T = T / chi.sqrt() * 1e-3
        del chi
        T = torch.where(torch.rand((rows, cols), generator=g, device=dev) < 1e-3, T * 1e3, T)
        zt = (torch.rand((rows // 32, 1, cols // 32, 1), generator=g, device=dev) < 0.01)
        T = T.view(rows // 32, 32, cols // 32, 32).masked_fill(zt, 0.0).view(rows, cols)
        T = T.to(torch.bfloat16).contiguous()
        W = (torch.randn((wn, wn), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        u8 = torch.uint8
        c1 = torch.empty((rows, cols // 2), dtype=u8, device=dev)
        s1 = torch.empty((rows, cols // 32), dtype=u8, device=dev)
        c2 = torch.empty((cols, rows // 2), dtype=u8, device=dev)
        s2 = torch.empty((cols, rows // 32), dtype=u8, device=dev)
        cw = torch.empty((wn, wn // 2), dtype=u8, device=dev)
        sw = torch.empty((wn // 32, wn // 32), dtype=u8, device=dev)
        flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)   # 1 GiB

        def timed(fn, iters=10):
            ts = []
            for _ in range(iters):
                flush.fill_(1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            return float(np.median(ts)), float(np.min(ts))

        q_t = lambda: ops.fourtune_quantize(ops.FT_Q_ROW32_T, T, rows, cols, cols, c1, s1, c2, s2,
                                            stream)
        q_w = lambda: ops.fourtune_quantize(ops.FT_Q_TILE32, W, wn, wn, wn, cw, sw, None, None,
                                            stream)
        cwt = torch.empty((wn, wn // 2), dtype=u8, device=dev)
        swt = torch.empty((wn // 32, wn // 32), dtype=u8, device=dev)
        q_w2 = lambda: ops.fourtune_quantize(ops.FT_Q_TILE32, W, wn, wn, wn, cw, sw, cwt, swt,
                                             stream)
        q_r = lambda: ops.fourtune_quantize(ops.FT_Q_ROW32, T, rows, cols, cols, c1, s1, None,
                                            None, stream)
        q_t(); q_w(); q_w2(); q_r()
        torch.cuda.synchronize()
        res = {}
        for name, fn, nbytes in (
                ("quant_row32_t", q_t, rows * cols * (2 + 2 * (0.5 + 1 / 32))),
                ("quant_tile32", q_w, wn * wn * (2 + 0.5 + 1 / 1024)),
                ("quant_tile32_both_layouts", q_w2, wn * wn * (2 + 2 * (0.5 + 1 / 1024))),
                ("quant_row32", q_r, rows * cols * (2 + 0.5 + 1 / 32))):
            med, mn = timed(fn)
            res[name] = {"median_us": round(med, 2), "min_us": round(mn, 2),
                         "GB/s": round(nbytes / (med * 1e-6) / 1e9, 1),
                         "frac_hbm": round(nbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": int(nbytes)}
        res["shapes"] = {"activation": [rows, cols], "weight": [wn, wn]}
        out["quantizer_stress"] = res
        log("bench: stress", json.dumps(res))
        del T, W, flush

    # ------------------------------------------------------------ CPU oracle
    if not a.no_cpu_baseline and a.only is None:
        log(f"bench: CPU oracle baseline on {a.cpu_rows} tokens")
        out["cpu_baseline"] = cpu_baseline(a.cpu_rows, a.cpu_reps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
