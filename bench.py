"""Benchmark of the attention hot path on one MI355X.

One step = one attn_decode_paged call (split kernel + LSE merge, every row of
the path) on the Qwen3-14B-shaped paged decode: batch 64, one query token,
40 query / 8 KV heads, head_dim 128, page_size 128, seq_lens uniform on
[256, 8192], bf16. Inputs are resident in HBM before timing starts.

Beside the average over the timed steps (ms_per_step, value), the line holds
the per-step median and p10-p90 range with warm caches and with L2 and the
MALL evicted before each step (a 512 MB read), the split kernel's
roofline, the secondary workloads (prefill, MLA decode, FP8 prefill, the
prologue kernels; each timed once the GPU's clocks have settled under it, as
the median of five event windows), ceilings measured on the GPU, a
sha256 of the input bytes, and the oracle timed on the host.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0         # MI355X dense FP8 MFMA, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(names: list[str]) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "softmax_attention_paged_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Workloads whose HBM traffic is measured with rocprofv3 counters: the kernel
# the roofline names (a substring of its symbol) and the sources it is built
# from. A record under profiles/ is used only while those sources hash the
# same as when the counters were taken.
TRAFFIC_KERNELS = {
    "qwen3_14b_decode": ("decode_gqa_wave_kernel<128, false>",
                         ["decode_gqa.hip", "device_common.h", "attn_internal.h"]),
    "dense_causal_prefill_d128": ("prefill_pp8_kernel<128, 0>",
                                  ["prefill.hip", "prefill_unit.h", "device_common.h", "attn_internal.h"]),
    "dense_causal_prefill_d256": ("prefill_pipe_kernel<256, 0>",
                                  ["prefill.hip", "prefill_unit.h", "device_common.h", "attn_internal.h"]),
    "ragged_paged_prefill_80k": ("prefill_pp8_kernel<128, 1>",
                                 ["prefill.hip", "prefill_unit.h", "device_common.h", "attn_internal.h"]),
    "single_chunk_prefill_80k": ("prefill_pp8_kernel<128, 1>",
                                 ["prefill.hip", "prefill_unit.h", "device_common.h", "attn_internal.h"]),
    "mla_decode_80k_bf16": ("decode_mla_kernel<false, false, false>",
                            ["decode_mla.hip", "device_common.h", "attn_internal.h"]),
    "mla_decode_80k_fp8_e4m3": ("decode_mla_kernel<true, false, false>",
                                ["decode_mla.hip", "device_common.h", "attn_internal.h"]),
    "mla_decode_80k_fp8_q": ("decode_mla_kernel<true, true, false>",
                             ["decode_mla.hip", "device_common.h", "attn_internal.h"]),
    "fp8_mla_prefill_8k": ("prefill_fp8_kernel",
                           ["prefill_fp8.hip", "prefill_unit.h", "device_common.h", "attn_internal.h"]),
}


def load_traffic(workload: str, plan: dict | None = None) -> dict | None:
    """HBM bytes per launch of the workload's roofline kernel, measured with
    rocprofv3 counters (FETCH_SIZE, WRITE_SIZE, each scaled by what the same
    counter reads for a plain copy of known size), stored under profiles/ by
    --traffic-summary; None once the kernel's sources (or, for a split
    decode, its split plan) differ from those the counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(TRAFFIC_KERNELS[workload][1]):
        return None
    if plan is not None and (rec.get("num_splits"), rec.get("split_tokens"), rec.get("key_ranges")) != (
            plan["num_splits"], plan["split_tokens"], plan["key_ranges"]):
        return None
    return rec


def _counter_means(run_dir: str, kernel: str, counter: str) -> tuple[str, float, int]:
    """Mean over the dispatches of the kernel whose symbol contains `kernel`
    of one counter in a rocprofv3 --pmc CSV (summed over the counter's
    instances within a dispatch); returns (symbol, mean, dispatches)."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = {}
    name = None
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if kernel not in row["Kernel_Name"] or row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                key = (fn, row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for a kernel matching {kernel!r} under {run_dir}")
    return name, sum(per.values()) / len(per), len(per)


def traffic_summary(workload: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                    copy_bytes: int) -> dict:
    """Write profiles/traffic_<workload>.json from four rocprofv3 --pmc runs
    (the workload with FETCH_SIZE, then WRITE_SIZE; a copy of copy_bytes
    with each): the counters in KiB per dispatch, scaled so that the copy
    reads and writes copy_bytes."""
    kernel, sources = TRAFFIC_KERNELS[workload]
    name, fetch, n_f = _counter_means(fetch_dir, kernel, "FETCH_SIZE")
    _, write, n_w = _counter_means(write_dir, kernel, "WRITE_SIZE")
    _, cfetch, _ = _counter_means(copy_fetch_dir, "copy", "FETCH_SIZE")
    _, cwrite, _ = _counter_means(copy_write_dir, "copy", "WRITE_SIZE")
    fs, ws = copy_bytes / 1024.0 / cfetch, copy_bytes / 1024.0 / cwrite
    only = "--only " + workload if workload != "qwen3_14b_decode" else "--only qwen3_14b_decode"
    rec = {
        "workload": workload,
        "kernel": name,
        "source_hash": kernel_source_hash(sources),
        "fetch_kib_per_dispatch": round(fetch, 3),
        "write_kib_per_dispatch": round(write, 3),
        "dispatches": [n_f, n_w],
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib": round(cfetch, 3), "write_kib": round(cwrite, 3),
                             "fetch_scale": round(fs, 6), "write_scale": round(ws, 6)},
        "bytes_per_launch": int(round((fetch * fs + write * ws) * 1024)),
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- python3 bench.py {only} --steps 3",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- python3 bench.py {only} --steps 3",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {copy_fetch_dir} -o run -- python3 bench.py "
            f"--copy-calibration {copy_bytes}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {copy_write_dir} -o run -- python3 bench.py "
            f"--copy-calibration {copy_bytes}",
            f"python3 bench.py --traffic-summary {workload} {fetch_dir} {write_dir} {copy_fetch_dir} "
            f"{copy_write_dir} {copy_bytes}",
        ],
    }
    if workload == "qwen3_14b_decode":
        from softmax_attention_paged_amd import inputs
        import softmax_attention_paged_amd as sap
        case = inputs.qwen3_14b_decode()
        p = sap.decode_params(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                              max_seq_len=case.max_seq_len, softmax_scale=case.scale,
                              total_kv_tokens=int(case.seq_lens.sum()))
        plan = sap.decode_plan(p)
        rec["num_splits"], rec["split_tokens"] = plan["num_splits"], plan["split_tokens"]
        rec["key_ranges"] = plan["key_ranges"]
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def trace_summary(workload: str, trace_dir: str, steps: int) -> str:
    """Write profiles/kernel_trace_<workload>.md from a rocprofv3
    --kernel-trace --stats run of `bench.py --only <workload>`."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_stats.csv under {trace_dir}")
    rows = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda r: -r[5])
    lines = [f"# Kernel trace: {workload}", "",
             "Command (repository root, MI355X, rocprofv3 from ROCm 7.2):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o run -- "
             f"python3 bench.py --only {workload} --steps {steps}",
             f"python3 bench.py --trace-summary {workload} {trace_dir} {steps}", "```", "",
             "Every dispatch of the run: the workload's untimed settling calls, then its timed windows "
             "(attention kernels), and torch's input staging and fills.", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in rows:
        short = name if len(name) <= 90 else name[:87] + "..."
        lines.append(f"| `{short}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f}% |")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.md"), "w") as f:
        f.write(text)
    return text


COUNTER_PASSES = [
    "MfmaUtil",
    "VALUBusy",
    "SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_LDS SQ_INSTS_LDS "
    "SQ_INSTS_VALU SQ_WAIT_ANY",
    "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS_LOAD_BANDWIDTH GRBM_GUI_ACTIVE",
]


def counter_summary(workload: str, run_dir: str) -> str:
    """Write profiles/counters_<workload>.md from the four rocprofv3 --pmc
    passes (run_dir/p1 .. p4, one counter block each) of `bench.py --only
    <workload> --steps 3`: means over the dispatches of the workload's
    roofline kernel."""
    import csv
    import glob
    kernel = TRAFFIC_KERNELS[workload][0]
    agg: dict[str, list[float]] = {}
    name = None
    for i in range(1, len(COUNTER_PASSES) + 1):
        files = glob.glob(os.path.join(run_dir, f"p{i}", "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise FileNotFoundError(f"no counter_collection.csv under {run_dir}/p{i}")
        per: dict[tuple[str, str], float] = {}
        with open(files[0]) as f:
            for r in csv.DictReader(f):
                if kernel not in r["Kernel_Name"]:
                    continue
                name = r["Kernel_Name"]
                key = (r.get("Dispatch_Id", r.get("Correlation_Id", "")), r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (_, c), v in per.items():
            agg.setdefault(c, []).append(v)
    m = {c: sum(v) / len(v) for c, v in agg.items()}
    n = len(agg.get("SQ_INSTS_MFMA", []))
    mf = m["SQ_INSTS_MFMA"]
    row = (f"| {workload} | `{name.split('(attn')[0].replace('void ', '').split('::')[-1]}` | {n} | "
           f"{m['MfmaUtil']:.1f} | {m['VALUBusy']:.1f} | {mf:.3g} | {m['SQ_VALU_MFMA_BUSY_CYCLES'] / mf:.1f} | "
           f"{m['SQ_INSTS_VALU'] / mf:.2f} | {m['SQ_INSTS_LDS'] / mf:.2f} | "
           f"{100 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.0f}% | "
           f"{100 * m['SQ_LDS_BANK_CONFLICT'] / max(m['SQ_LDS_IDX_ACTIVE'], 1):.1f}% |")
    lines = [f"# MFMA, VALU and LDS counters: {workload}", "", "Commands (repository root, MI355X, rocprofv3 "
             "from ROCm 7.2; one counter block per run, as rocprofv3 collects no counters over several passes):",
             "", "```"]
    for i, c in enumerate(COUNTER_PASSES, 1):
        lines.append(f"rocprofv3 --pmc {c} --output-format csv -d {run_dir}/p{i} -o run -- "
                     f"python3 bench.py --only {workload} --steps 3")
    lines += [f"python3 bench.py --counter-summary {workload} {run_dir}", "```", "",
              "Means over the dispatches of the kernel in the run (settling calls, warm-up and timed calls). "
              "MfmaUtil and VALUBusy are rocprofv3's derived metrics (percent of active cycles); per-MFMA columns "
              "divide by SQ_INSTS_MFMA; waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES; conflicts = SQ_LDS_BANK_CONFLICT / "
              "SQ_LDS_IDX_ACTIVE.", "",
              "| workload | kernel | dispatches | MfmaUtil % | VALUBusy % | MFMA instr./dispatch | busy cycles/MFMA | "
              "vector instr./MFMA | LDS instr./MFMA | wave cycles waiting | LDS bank conflicts |",
              "|---|---|---|---|---|---|---|---|---|---|---|", row]
    text = "\n".join(lines) + "\n"
    with open(os.path.join(ROOT, "profiles", f"counters_{workload}.md"), "w") as f:
        f.write(text)
    return text


def time_events(fn, steps: int, stream) -> float:
    """Average milliseconds per call of fn, HIP events on `stream`."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_each(fn, steps: int, stream, before=None) -> list[float]:
    """Milliseconds of each of `steps` calls of fn, one HIP event pair per
    call on `stream`; `before` (untimed) runs ahead of each call."""
    import torch
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in pairs:
        if before is not None:
            before()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def spread(ms: list[float]) -> dict:
    q = np.percentile(np.asarray(ms), [10, 50, 90])
    return {"median_ms": round(float(q[1]), 5), "p10_ms": round(float(q[0]), 5), "p90_ms": round(float(q[2]), 5),
            "n": len(ms)}


def ceilings_lib():
    """The ceiling kernels (softmax_attention_paged_amd/ceilings), built
    beside the attention library."""
    import ctypes
    path = os.path.join(ROOT, "softmax_attention_paged_amd", "libattn_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build first (python -m softmax_attention_paged_amd.build)")
    lib = ctypes.CDLL(path)
    lib.ceil_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.ceil_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.ceil_mfma_bf16_varied.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.ceil_mfma_fma_overlap.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    lib.ceil_lds_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


class Evictor:
    """Reads a 512 MB buffer with the streaming-read kernel: evicts the
    inputs from L2 and the 256 MB MALL without leaving dirty lines whose
    write-back would load the next timed step."""

    def __init__(self, dev):
        import torch
        self.lib = ceilings_lib()
        self.buf = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(4096, dtype=torch.int32, device=dev)
        self.stream = torch.cuda.current_stream(dev)

    def __call__(self):
        rc = self.lib.ceil_stream_read(self.buf.data_ptr(), self.buf.numel(), self.sink.data_ptr(), 4096,
                                       self.stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"ceil_stream_read failed: {rc}")


def measured_peaks() -> dict:
    """Ceilings measured on this GPU, as secondary denominators: a 1 GiB
    streaming read and a bf16 32x32x16 MFMA loop (the ceiling kernels; the
    loop once with fixed operands and once with operands that change every
    instruction, as a real contraction's do; LDS reads of 16 bytes per lane,
    plain and transposing), and
    for context a 1 GiB torch copy (bytes read + written) and a bf16 8192^3
    GEMM through torch.matmul (hipBLASLt)."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    lib = ceilings_lib()
    x = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.float32, device=dev)

    def read():
        if lib.ceil_stream_read(x.data_ptr(), x.numel(), sink.data_ptr(), 4096, stream.cuda_stream) != 0:
            raise RuntimeError("ceil_stream_read failed")

    iters, blocks = 4096, 2048            # 2048 workgroups of 4 waves: 8 per SIMD

    def mfma():
        if lib.ceil_mfma_bf16(sink.data_ptr(), iters, blocks, stream.cuda_stream) != 0:
            raise RuntimeError("ceil_mfma_bf16 failed")

    def mfma_varied():
        if lib.ceil_mfma_bf16_varied(sink.data_ptr(), iters, blocks, stream.cuda_stream) != 0:
            raise RuntimeError("ceil_mfma_bf16_varied failed")

    lds_iters, lds_blocks = 4096, 2048     # two 64 KB workgroups per CU
    lds_sink = torch.zeros(lds_blocks * 256, dtype=torch.int32, device=dev)

    def lds(kind):
        if lib.ceil_lds_read(lds_sink.data_ptr(), kind, lds_iters, lds_blocks, stream.cuda_stream) != 0:
            raise RuntimeError("ceil_lds_read failed")

    for f in (read, mfma, mfma_varied, lambda: lds(0), lambda: lds(1)):
        f()
    read_ms = time_events(read, 10, stream)
    mfma_ms = time_events(mfma, 5, stream)
    varied_ms = time_events(mfma_varied, 5, stream)
    lds_ms = [time_events(lambda: lds(k), 5, stream) for k in (0, 1)]
    lds_bytes = lds_blocks * 256 * 16 * lds_iters
    y = torch.empty_like(x)
    y.copy_(x)
    copy_ms = time_events(lambda: y.copy_(x), 10, stream)
    del x, y
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    gemm_ms = time_events(lambda: torch.matmul(a, b, out=c), 10, stream)
    del a, b, c, sink
    torch.cuda.empty_cache()
    mfma_flops = blocks * 4 * iters * 4 * 32768
    return {"stream_read_GBs": round((1 << 30) / (read_ms * 1e-3) / 1e9, 1),
            "mfma_bf16_loop_TFLOPs": round(mfma_flops / (mfma_ms * 1e-3) / 1e12, 1),
            "mfma_bf16_loop_varied_operands_TFLOPs": round(mfma_flops / (varied_ms * 1e-3) / 1e12, 1),
            "lds_read_b128_TBs": round(lds_bytes / (lds_ms[0] * 1e-3) / 1e12, 1),
            "lds_read_b64_tr_b16_TBs": round(lds_bytes / (lds_ms[1] * 1e-3) / 1e12, 1),
            "torch_copy_GBs": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
            "hipblaslt_bf16_gemm_8192_TFLOPs": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1)}


def overlap_probe() -> dict:
    """How far MFMA and FMA work of two waves sharing a SIMD overlap: one
    wave per SIMD of back-to-back bf16 MFMAs (32x32x16, or 16x16x32 for the
    same flops), one of eight independent FMA chains, each alone and both
    together; best of three launches of 256 workgroups, in ms."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    lib = ceilings_lib()
    blocks = 256
    sink = torch.zeros(blocks * 512, dtype=torch.float32, device=dev)
    res = {}
    for kind, name in ((0, "32x32x16"), (1, "16x16x32")):
        for mode, what in ((1, "mfma"), (2, "fma"), (3, "both")):
            def launch():
                if lib.ceil_mfma_fma_overlap(sink.data_ptr(), kind, mode, 4096, 8192, blocks, stream.cuda_stream) != 0:
                    raise RuntimeError("ceil_mfma_fma_overlap failed")
            launch()
            res[f"{name}_{what}_ms"] = round(min(time_events(launch, 1, stream) for _ in range(3)), 4)
        alone = max(res[f"{name}_mfma_ms"], res[f"{name}_fma_ms"])
        res[f"{name}_fma_time_exposed"] = round((res[f"{name}_both_ms"] - alone) / res[f"{name}_fma_ms"], 3)
    return res


def input_sha256(tensors) -> str:
    """sha256 over the bytes of the workload's host-side input tensors."""
    import torch
    h = hashlib.sha256()
    for t in tensors:
        h.update(memoryview(t.contiguous().view(-1).view(torch.uint8).numpy()))
    return h.hexdigest()


def settle(fn, seconds: float = 0.3) -> None:
    """Run fn untimed for about `seconds`: the GPU's clocks ramp up over the
    first tens of milliseconds of sustained work (an 80K MLA decode runs
    0.46-0.55 ms per call in its first 20 calls and 0.41 ms after), so a
    short workload is timed only once they have settled."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_settled(fn, steps: int, stream, windows: int = 5) -> float:
    """Median over `windows` HIP-event windows of `steps` calls each, after
    the clocks have settled."""
    settle(fn)
    return float(np.median([time_events(fn, steps, stream) for _ in range(windows)]))


def time_graph(fn, steps: int) -> float:
    """Average milliseconds per call of fn, with the calls captured in one HIP
    graph and the replay timed by HIP events: for kernels shorter than the
    host's per-call launch cost, so the host does not set the pace. (The
    entry points allocate and synchronise nothing, so they capture.)"""
    import torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fn()                                  # warm the launch path outside the capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    start.record(cur)
    graph.replay()
    end.record(cur)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def cpu_baseline(case, budget_s: float = 10.0) -> dict:
    """The fp64 oracle on the host cores, over whole requests of the same
    workload, cycling through the batch until about budget_s of work (at
    least one request)."""
    import numpy as np
    import oracle
    import torch
    from threadpoolctl import threadpool_info

    q = case.q.view(torch.int16).numpy().view(np.uint16)
    kc = case.k_cache.view(torch.int16).numpy().view(np.uint16)
    vc = case.v_cache.view(torch.int16).numpy().view(np.uint16)
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    b_n, q_len, hq, _ = case.q.shape
    row_bytes = 2 * case.k_cache.shape[2] * case.k_cache.shape[3] * 2
    t0 = time.perf_counter()
    done_bytes, done_req = 0, 0
    while time.perf_counter() - t0 < budget_s:
        b = done_req % b_n
        rows = [(b, t, h) for t in range(q_len) for h in range(hq)]
        oracle.decode_paged_rows(q, kc, vc, bt, sl, case.page_size, case.scale, case.causal,
                                 case.head_dim_v, rows, "bf16", 1.0, "bf16")
        done_bytes += int(sl[b]) * row_bytes
        done_req += 1
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpus_allowed": len(os.sched_getaffinity(0)), "cpu_model": model,
            "sample": f"{done_req} requests, cycling through the {b_n} of the workload ({done_bytes / 1e6:.1f} MB "
                      f"of KV), {dt:.1f} s, fp64 numpy, BLAS pool of {threads} threads (the cores it used)"}


def causal_pairs(cu_q: list[int], kv_lens: list[int], causal: bool) -> int:
    """Unmasked (query, key) pairs of a ragged batch (bottom-right causal)."""
    tot = 0
    for b, lk in enumerate(kv_lens):
        lq = cu_q[b + 1] - cu_q[b]
        if not causal:
            tot += lq * lk
            continue
        for i in range(lq):
            tot += min(lk, max(0, lk - lq + i + 1))
    return tot


def secondary_prefill(key: str, name_fn, steps: int, kv_splits: int = 0) -> dict:
    import torch
    import softmax_attention_paged_amd as sap
    case = name_fn()
    c = case.to("cuda:0")
    tq, hq, d = case.q.shape
    flops = causal_pairs(case.cu_seqlens_q.tolist(), case.seq_lens_kv.tolist(), case.causal) * hq * 2 * (d + d)
    # Q read, O and LSE written once; K and V of each (request, KV head) read once
    hkv = case.k.shape[-2]
    alg_bytes = tq * hq * (2 * d + 2 * d + 4) + int(case.seq_lens_kv.sum()) * hkv * 2 * d * 2
    out = torch.empty_like(c.q)
    kw = dict(max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, causal=c.causal, kv_splits=kv_splits)
    kv = dict(seq_lens_kv=c.seq_lens_kv, block_table=c.block_table) if c.paged else dict(cu_seqlens_kv=c.cu_seqlens_kv)
    # key-split partials: one workspace, allocated before the timed region
    ws_bytes = sap.prefill_workspace_size(c.q, c.k, c.v, c.cu_seqlens_q, **kv, **kw)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=c.q.device)
    splits = ws_bytes // (tq * hq * (d + 1) * 4) if ws_bytes else 1
    fn = lambda: sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, softmax_scale=c.scale, out=out, workspace=ws, **kv, **kw)
    ms = time_settled(fn, steps, torch.cuda.current_stream())
    tf = flops / (ms * 1e-3) / 1e12
    kernel = (f"{'prefill_pp8_kernel' if d == 128 else 'prefill_pipe_kernel'}<{d}, {1 if c.paged else 0}>" +
              (" + merge" if splits > 1 else ""))
    traffic = load_traffic(key)
    return {"workload": case.name, "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "kv_splits": splits,
            "roofline": {"bound": "mfma", "kernel": kernel,
                         "achieved": round(tf, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": None if traffic is None else traffic["bytes_per_launch"],
                         "algorithmic_bytes_per_launch": alg_bytes}}


def secondary_mla(kv_dtype: str, steps: int, q_dtype: str = "bf16") -> dict:
    """The 80K MLA-shaped decode. bf16 q runs both products on the bf16
    MFMA; with fp8 q (and fp8 KV) QK runs on the FP8 MFMA and P.V on bf16,
    so the roof is the two peaks blended by each part's flops."""
    import torch
    import softmax_attention_paged_amd as sap
    from softmax_attention_paged_amd import inputs
    case = inputs.mla_decode(kv_dtype=kv_dtype, q_dtype=q_dtype)
    c = case.to("cuda:0")
    b_n, q_len, hq, dqk = case.q.shape
    kw = dict(max_seq_len=c.max_seq_len, softmax_scale=c.scale, causal=c.causal, head_dim_v=512,
              kv_dtype=None if kv_dtype == "bf16" else kv_dtype, k_scale=c.kv_scale, v_scale=c.kv_scale,
              q_scale=None if q_dtype == "bf16" else c.q_scale)
    plan = sap.decode_plan(sap.decode_params(c.q, c.k_cache, None, c.block_table, c.seq_lens, **kw))
    ws = torch.empty(plan["workspace_bytes"] + 16, dtype=torch.uint8, device=c.q.device)
    out = torch.empty((b_n, q_len, hq, 512), dtype=torch.bfloat16, device=c.q.device)
    fn = lambda: sap.decode_paged(c.q, c.k_cache, None, c.block_table, c.seq_lens, workspace=ws, out=out, **kw)
    ms = time_settled(fn, steps, torch.cuda.current_stream())
    lens = case.seq_lens.tolist()
    pairs = hq * sum(min(lk, max(0, lk - q_len + t + 1)) if case.causal else lk for lk in lens for t in range(q_len))
    qk, pv = pairs * 2 * dqk, pairs * 2 * 512
    flops = qk + pv
    tf = flops / (ms * 1e-3) / 1e12
    if q_dtype == "bf16":
        peak = BF16_PEAK_TFLOPS   # bf16 MFMA for both products (fp8 KV is widened to bf16)
    else:
        peak = flops / (qk / FP8_PEAK_TFLOPS + pv / BF16_PEAK_TFLOPS)
    traffic = load_traffic(f"mla_decode_80k_{kv_dtype}" if q_dtype == "bf16" else "mla_decode_80k_fp8_q")
    return {"workload": case.name, "ms": round(ms, 4), "TFLOP/s": round(tf, 1),
            "kv_GB/s": round(case.kv_read_bytes() / (ms * 1e-3) / 1e9, 1), "num_splits": plan["num_splits"],
            "roofline": {"bound": "mfma", "kernel": "decode_mla_kernel + merge", "achieved": round(tf, 1),
                         "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                         "traffic": None if traffic is None else traffic["bytes_per_launch"],
                         "algorithmic_bytes_per_launch": case.kv_read_bytes() +
                         case.q.numel() * case.q.element_size() + b_n * q_len * hq * (512 * 2 + 4)}}


def secondary_prefill_fp8(steps: int) -> dict:
    """FP8 MLA-shaped prefill (8K x 8K causal, 128 heads, q/k 192, v 128).
    QK runs on FP8 MFMA and P.V on bf16 MFMA, so the roof is the blend of the
    two published peaks weighted by each part's flops."""
    import torch
    import softmax_attention_paged_amd as sap
    from softmax_attention_paged_amd import inputs
    case = inputs.fp8_mla_prefill()
    c = case.to("cuda:0")
    f8 = lambda t: t.view(torch.float8_e4m3fn)
    tq, hq, dqk = case.q.shape
    dv = case.v.shape[2]
    out = torch.empty((tq, hq, dv), dtype=torch.bfloat16, device="cuda:0")
    fn = lambda: sap.prefill(f8(c.q), f8(c.k), f8(c.v), c.cu_seqlens_q, cu_seqlens_kv=c.cu_seqlens_kv,
                             max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, softmax_scale=c.scale,
                             causal=True, out=out, q_scale=c.q_scale, k_scale=c.k_scale, v_scale=c.v_scale)
    ms = time_settled(fn, steps, torch.cuda.current_stream())
    pairs = causal_pairs(case.cu_seqlens_q.tolist(), case.cu_seqlens_kv.diff().tolist(), True) * hq
    qk, pv = pairs * 2 * dqk, pairs * 2 * dv
    tf = (qk + pv) / (ms * 1e-3) / 1e12
    peak = (qk + pv) / (qk / FP8_PEAK_TFLOPS + pv / BF16_PEAK_TFLOPS)
    traffic = load_traffic("fp8_mla_prefill_8k")
    alg_bytes = tq * hq * (dqk + 2 * dv + 4) + case.k.numel() + case.v.numel()
    return {"workload": case.name, "ms": round(ms, 4), "TFLOP/s": round(tf, 1),
            "roofline": {"bound": "mfma", "kernel": "prefill_fp8_kernel", "achieved": round(tf, 1),
                         "peak": round(peak, 1), "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                         "peak_note": "QK flops at the FP8 peak, P.V flops at the bf16 peak",
                         "traffic": None if traffic is None else traffic["bytes_per_launch"],
                         "algorithmic_bytes_per_launch": alg_bytes}}


def secondary_mla_pack(steps: int) -> dict:
    """MLA K/V pack + FP8 quantise at the TokenSpeed-MLA prefill shape (8K
    tokens, 128 heads, K = 128 nope + 64 rope, V = 128): HBM-bound."""
    import torch
    import softmax_attention_paged_amd as sap
    from softmax_attention_paged_amd import inputs
    case = inputs.pack_case(num_tokens=8192, heads=128, seed=7, strided=True)
    c = case.to("cuda:0")
    t, h, dn = case.k_nope.shape
    dr, dv = case.k_rope.shape[1], case.v.shape[2]
    k_out = torch.empty((t, h, dn + dr), dtype=torch.float8_e4m3fn, device="cuda:0")
    v_out = torch.empty((t, h, dv), dtype=torch.float8_e4m3fn, device="cuda:0")
    fn = lambda: sap.mla_kv_pack_fp8(c.k_nope, c.k_rope, c.v, k_scale=c.k_scale, v_scale=c.v_scale,
                                     k_out=k_out, v_out=v_out)
    ms = time_settled(fn, steps, torch.cuda.current_stream())
    alg = t * h * (dn + dv) * 2 + t * dr * 2 + t * h * (dn + dr + dv)    # bf16 in (rope once), E4M3 out
    gbs = alg / (ms * 1e-3) / 1e9
    return {"workload": f"mla_kv_pack_fp8_t{t}_h{h}_d{dn}+{dr}_v{dv}", "ms": round(ms, 4), "GB/s": round(gbs, 1),
            "roofline": {"bound": "hbm", "kernel": "mla_kv_pack_kernel", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": alg}}


def secondary_append(steps: int) -> dict:
    """K/V cache append of an 8K-token prefill chunk (8 KV heads of 128, as
    in the Qwen3-14B-shaped decode) into a 128-row-page bf16 cache."""
    import torch
    import softmax_attention_paged_amd as sap
    from softmax_attention_paged_amd import inputs
    case = inputs.append_case(num_tokens=8192, hkv=8, dk=128, dv=128, page_size=128, pages_per_layer=1024,
                              layers=1, layer=0, seed=8)
    c = case.to("cuda:0")
    fn = lambda: sap.cache_append(c.k_new, c.v_new, c.k_cache, c.v_cache, c.slot_mapping,
                                  layer_base_rows=c.layer_base_rows)
    settle(fn)
    ms = float(np.median([time_graph(fn, max(steps, 20)) for _ in range(5)]))   # a 14 us kernel: replayed from a graph
    n, hkv, dk = case.k_new.shape
    alg = 2 * (n * hkv * dk * 2) * 2 + n * 8                            # K and V read and written, slots
    gbs = alg / (ms * 1e-3) / 1e9
    return {"workload": f"cache_append_bf16_n{n}_hkv{hkv}_d{dk}_ps128", "ms": round(ms, 4), "GB/s": round(gbs, 1),
            "roofline": {"bound": "hbm", "kernel": "cache_append_kernel<false>", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": alg}}


def secondary_tiny_decode(steps: int) -> dict:
    """The tiny paged GQA decode (2 requests of 37 and 100 keys, 8/2 heads,
    D 64, 16-row pages): launch-bound, so timed as graph replays; reported as
    latency per call under the planner's own plan (requests this short run as
    one unsplit launch), with no roofline."""
    import torch
    import softmax_attention_paged_amd as sap
    from softmax_attention_paged_amd import inputs
    case = inputs.gqa_decode_tiny()
    c = case.to("cuda:0")
    kw = dict(max_seq_len=c.max_seq_len, softmax_scale=c.scale)
    plan = sap.decode_plan(sap.decode_params(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, **kw))
    ws = torch.empty(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device=c.q.device)
    out = torch.empty((2, 1, 8, 64), dtype=torch.bfloat16, device=c.q.device)
    fn = lambda: sap.decode_paged(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, workspace=ws, out=out, **kw)
    settle(fn, 0.1)
    ms = float(np.median([time_graph(fn, max(steps, 20)) for _ in range(5)]))
    eager = time_settled(fn, max(steps, 20), torch.cuda.current_stream())
    return {"workload": case.name, "us_per_call_graph": round(ms * 1e3, 2), "us_per_call_eager": round(eager * 1e3, 2),
            "num_splits": plan["num_splits"], "key_ranges": plan["key_ranges"],
            "note": "launch-bound: " + ("one kernel per call" if plan["workspace_bytes"] == 0
                                        else "two kernels (split + merge) per call")}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--num-splits", type=int, default=0, help="override the planner's KV split count")
    ap.add_argument("--prefill-kv-splits", type=int, default=0,
                    help="override the prefill planner's key split count (1: unsplit)")
    ap.add_argument("--no-secondary", action="store_true", help="time only the main workload")
    ap.add_argument("--only", default="", metavar="WORKLOAD",
                    help="time one workload alone (for profiling): qwen3_14b_decode (the main line), "
                         "dense_causal_prefill_d128, "
                         "dense_causal_prefill_d256, ragged_paged_prefill_80k, single_chunk_prefill_80k, mla_decode_80k_bf16, "
                         "mla_decode_80k_fp8_e4m3, mla_decode_80k_fp8_q")
    ap.add_argument("--counter-summary", nargs=2, metavar=("WORKLOAD", "RUN_DIR"),
                    help="write profiles/counters_<workload>.md from four rocprofv3 --pmc passes under RUN_DIR")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 3 device-to-device copies of BYTES (reference for HBM counters)")
    ap.add_argument("--traffic-summary", nargs=6, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                           "COPY_WRITE_DIR", "COPY_BYTES"),
                    help="write profiles/traffic_<WORKLOAD>.json from rocprofv3 FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--overlap-probe", action="store_true",
                    help="time matrix and vector waves alone and together on each SIMD (the ceilings library)")
    ap.add_argument("--trace-summary", nargs=3, metavar=("WORKLOAD", "TRACE_DIR", "STEPS"),
                    help="write profiles/kernel_trace_<WORKLOAD>.md from a rocprofv3 --kernel-trace --stats run")
    args = ap.parse_args()
    if args.traffic_summary:
        w, fd, wd, cfd, cwd, cb = args.traffic_summary
        print(json.dumps(traffic_summary(w, fd, wd, cfd, cwd, int(cb))))
        return 0
    if args.trace_summary:
        print(trace_summary(args.trace_summary[0], args.trace_summary[1], int(args.trace_summary[2])))
        return 0
    if args.counter_summary:
        print(counter_summary(args.counter_summary[0], args.counter_summary[1]))
        return 0
    if args.overlap_probe:
        print(json.dumps(overlap_probe()))
        return 0
    if args.copy_calibration:
        import torch
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration}))
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "this path runs on one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        return 2

    import torch
    import softmax_attention_paged_amd as sap
    from softmax_attention_paged_amd import inputs

    secondaries = {
        "dense_causal_prefill_d128": lambda steps: secondary_prefill(
            "dense_causal_prefill_d128", lambda: inputs.dense_causal_prefill(d=128), steps, args.prefill_kv_splits),
        "dense_causal_prefill_d256": lambda steps: secondary_prefill(
            "dense_causal_prefill_d256", lambda: inputs.dense_causal_prefill(d=256), steps, args.prefill_kv_splits),
        "ragged_paged_prefill_80k": lambda steps: secondary_prefill(
            "ragged_paged_prefill_80k", inputs.ragged_paged_prefill, steps, args.prefill_kv_splits),
        "single_chunk_prefill_80k": lambda steps: secondary_prefill(
            "single_chunk_prefill_80k", inputs.single_chunk_prefill, steps, args.prefill_kv_splits),
        "mla_decode_80k_bf16": lambda steps: secondary_mla("bf16", steps),
        "mla_decode_80k_fp8_e4m3": lambda steps: secondary_mla("fp8_e4m3", steps),
        "mla_decode_80k_fp8_q": lambda steps: secondary_mla("fp8_e4m3", steps, "fp8_e4m3"),
        "fp8_mla_prefill_8k": secondary_prefill_fp8,
        "mla_kv_pack_fp8_8k": secondary_mla_pack,
        "cache_append_8k": secondary_append,
        "tiny_gqa_decode": secondary_tiny_decode,
    }
    if args.only and args.only != "qwen3_14b_decode":
        print(json.dumps({args.only: secondaries[args.only](args.steps)}), flush=True)
        return 0
    if args.only:                       # the main decode alone: no secondaries, no host baseline
        args.no_secondary = args.no_cpu_baseline = True

    log("generating inputs ...")
    case = inputs.qwen3_14b_decode(seed=args.seed)
    dev = torch.device("cuda:0")
    c = case.to(dev)
    b_n, q_len, hq, d = case.q.shape
    tokens = int(case.seq_lens.sum())
    kv_bytes = case.kv_read_bytes()
    alg_bytes = kv_bytes + case.q.numel() * 2 + b_n * q_len * hq * (case.head_dim_v * 2 + 4)
    flops = tokens * q_len * hq * 2 * (d + case.head_dim_v)

    # the host knows the batch's total of keys (a serving scheduler does): the
    # planner uses it to keep every split unit resident at once
    params = sap.decode_params(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                               max_seq_len=c.max_seq_len, softmax_scale=c.scale, num_splits=args.num_splits,
                               total_kv_tokens=tokens)
    plan = sap.decode_plan(params)
    ws = torch.empty(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device=dev)
    out = torch.empty((b_n, q_len, hq, case.head_dim_v), dtype=torch.bfloat16, device=dev)
    log(f"plan {plan}")

    # The call's parameters are marshalled once; each step is one C-ABI call
    # (so the host's per-call cost stays well below the kernels' time, also
    # for the merge phase alone).
    import ctypes
    from softmax_attention_paged_amd import _ffi
    stream = torch.cuda.current_stream(dev)
    lib = _ffi.load()
    cparams = sap.decode_params(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, max_seq_len=c.max_seq_len,
                                softmax_scale=c.scale, num_splits=args.num_splits, workspace=ws, out=out,
                                total_kv_tokens=tokens)
    pref, sh = ctypes.byref(cparams), ctypes.c_void_p(stream.cuda_stream)

    def entry(name):
        fn = getattr(lib, name)
        _ffi.check(fn(pref, sh), name)
        return lambda: fn(pref, sh)

    step = entry("attn_decode_paged")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms = time_events(step, args.steps, stream)
    # Per-step spread, warm (inputs as the previous step left the caches) and
    # cold (a 512 MB read ahead of each step evicts L2 and the MALL).
    warm = spread(time_each(step, args.steps, stream))
    evict = Evictor(dev)
    cold = spread(time_each(step, args.steps, stream, before=evict))
    del evict
    cold["GBs_at_median"] = round(kv_bytes / (cold["median_ms"] * 1e-3) / 1e9, 2)
    # The call's two kernels timed apart (attn_decode_paged_split, then
    # attn_decode_paged_merge on the partials the split phase left).
    split_step, merge_step = entry("attn_decode_paged_split"), entry("attn_decode_paged_merge")
    for _ in range(3):
        split_step()
    split_ms = time_events(split_step, args.steps, stream)
    merge_ms = 0.0
    if plan["workspace_bytes"] > 0:
        for _ in range(3):
            merge_step()
        merge_ms = time_events(merge_step, args.steps, stream)
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    achieved = alg_bytes / (split_ms * 1e-3) / 1e9
    traffic = load_traffic("qwen3_14b_decode", plan)
    line = {
        "metric": "prefill attn TFLOP/s (% MFMA peak); decode KV-read GB/s (% HBM peak)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, "batch": b_n, "q_len": q_len, "num_q_heads": hq,
                   "num_kv_heads": case.k_cache.shape[2], "head_dim": d, "page_size": case.page_size,
                   "total_kv_tokens": tokens, "kv_bytes": kv_bytes, "seed": args.seed,
                   "num_splits": plan["num_splits"], "split_tokens": plan["split_tokens"],
                   "key_ranges": plan["key_ranges"],
                   "input_sha256": input_sha256([case.q, case.k_cache, case.v_cache, case.block_table,
                                                 case.seq_lens]),
                   "parallelism": "single GPU"},
        "step_spread": {"warm": warm, "cold": cold},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": "decode_gqa_wave_kernel<128, false>", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "algorithmic_bytes_per_launch": alg_bytes, "avg_launch_ms": round(split_ms, 5),
                     "merge_avg_launch_ms": round(merge_ms, 5),
                     "timing": "kernel averages from HIP events on the launch stream over back-to-back "
                               "calls of each phase alone"},
        "decode_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
    }
    if not args.no_secondary:
        del c, ws, out
        torch.cuda.empty_cache()
        line["measured_peaks"] = measured_peaks()
        torch.cuda.empty_cache()
        sec = {}
        for key, fn in secondaries.items():
            log(f"secondary {key} ...")
            sec[key] = fn(max(3, args.steps // 5))
            torch.cuda.empty_cache()
        line["secondary"] = sec
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        line["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
