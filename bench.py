"""Benchmark of the 4-bit block-dequant decode matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-secondary]
                    [--kernel kmajor|canonical]   (or W4_KERNEL=...)
    python bench.py --probes      (launch cost and streaming-read rates only)

The step is one decode body pass of the 3.8B-dense-shaped model at M = 1:
32 layers x 4 W4 matmuls (3072x9216 QKV, 3072x3072 out, 3072x16384
gate+up, 8192x3072 down), 2.32 GB of packed weights, i.e. 128 launches of
the fused dequant-GEMV on one stream, captured once in a HIP graph and
replayed.  The weights are quantized on the GPU into the canonical layout
and prepacked once (K-major copy of the same bytes) before timing; the
timed GEMV reads the prepacked copy (`--kernel canonical` times the
canonical-layout GEMV instead, for A/B).  The weights are far larger than
the 256 MB Infinity Cache, so every pass streams them from HBM.  `value` is
the pass's algorithmic bytes (packed weights, scales, zero points, x and y,
each counted once) divided by the measured time per pass.

Also reported on the same JSON line:
  * roofline: the GEMV kernel's algorithmic bytes per launch over its
    average launch duration (the timed pass over its 128 launches, all of
    them this kernel), against the 8 TB/s HBM peak and against the launch
    floor: the same 128-launch graph with a plain streaming-read kernel
    (w4_read_bytes) reading each matrix's packed bytes; per-shape times from
    graphs of one shape's 32 launches; the committed rocprofv3 figures for
    the same kernel beside the live ones;
  * cpu_baseline: the CPU oracle (dequantize, then fp64 matmul) at 1, 4 and
    all host threads, median of 3, on a bounded sample of every workload;
  * parity: GPU outputs of the first layers against the oracle, per output;
  * secondary: the GPT-2-small-shaped decode pass (48 matmuls with bias),
    the int8 head [768, 50257], the GPT-2 prefill pass at M = 58 plus the
    last-row head, the 3.8B pass at M = 4 and M = 16, each against its own
    roofline.
Inputs are seeded synthetic data of the workloads' shapes and distributions
(see synth.py); nothing is read from disk.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

METRIC = "W4 decode GEMV achieved HBM GB/s (% of peak) + body-pass tokens/s, 1 GPU"
HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0
FLOOR_LOADS = (4, 8, 16)       # streaming-read reference: 16-byte loads per lane
ROOT = os.path.dirname(os.path.abspath(__file__))

# The dominant kernel of the timed pass, the sources that define it, and the
# committed counter summary that bench.py reads `roofline.traffic` from.  The
# summary records a digest of these sources; once they change, traffic is
# reported as null until the counters are taken again.
GEMV_KERNEL = "k_gemv_kmajor"
GEMV_SOURCES = ("w4_block_dequant_amd/csrc/kmajor.hip", "w4_block_dequant_amd/csrc/common.h")
PROFILE_DIR = "profiles"
TRACE_SUMMARY = "k_gemv_kmajor_dense38_m1_kernel_trace.md"
TRAFFIC_SUMMARY = "k_gemv_kmajor_dense38_m1_traffic.md"
SECONDARY_SUMMARY = "secondary_workloads_kernel_trace.md"
MFMA_SUMMARY = "k_mm_x3_matrix_core_utilisation.md"
COPY_FLOATS = 1 << 26          # calibration copy: 256 MiB read, 256 MiB written
PROFILE_COMMANDS = (
    "cd <repo root>; export TMPDIR=/tmp",
    "rocprofv3 --kernel-trace --stats --output-format csv -d /tmp/w4prof/trace -o run "
    "-- python bench.py --steps 10 --warmup 2 --skip-secondary --skip-cpu "
    "--json-out /tmp/w4prof/trace_bench.json",
    "timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE --output-format csv -d /tmp/w4prof/fetch "
    "-o run -- python bench.py --profile-run --steps 2",
    "timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE --output-format csv -d /tmp/w4prof/write "
    "-o run -- python bench.py --profile-run --steps 2",
    "timeout -s KILL 300 rocprofv3 --pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_BUBBLE_sum "
    "TCC_EA0_RDREQ_DRAM_sum --output-format csv -d /tmp/w4prof/rdreq -o run "
    "-- python bench.py --profile-run --steps 2",
    "python bench.py --json-out /tmp/w4prof/bench.json",
    "rocprofv3 --kernel-trace --stats --output-format csv -d /tmp/w4prof/trace_all -o run "
    "-- python bench.py --steps 10 --warmup 2 --skip-cpu "
    "--json-out /tmp/w4prof/trace_all_bench.json",
    "timeout -s KILL 300 rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 "
    "SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_F32 --output-format csv "
    "-d /tmp/w4prof/mfma -o run "
    "-- python bench.py --profile-run-mfma --steps 2",
    "timeout -s KILL 300 rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU "
    "SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT --output-format csv "
    "-d /tmp/w4prof/sq -o run -- python bench.py --profile-run-mfma --steps 2",
    "timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE --output-format csv -d /tmp/w4prof/fetch4 "
    "-o run -- python bench.py --profile-run --profile-rows 4 --steps 2",
    "timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE --output-format csv -d /tmp/w4prof/write4 "
    "-o run -- python bench.py --profile-run --profile-rows 4 --steps 2",
    "python bench.py --summarize-profiles /tmp/w4prof --out profiles",
)


def gemv_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMV_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_summary_fields(path: str) -> dict:
    """`key: value` lines of a committed profile summary (one per line, after a dash)."""
    out = {}
    if not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                out[k.strip("`")] = v.strip().strip("`")
    return out


def committed_traffic():
    """HBM bytes per GEMV launch from the committed counter summary, if still current."""
    f = read_summary_fields(os.path.join(ROOT, PROFILE_DIR, TRAFFIC_SUMMARY))
    if not f or f.get("gemv_source_sha256") != gemv_digest():
        return None, None
    try:
        fetch = float(f["fetch_bytes_per_launch"])
        write = float(f["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None, None
    return fetch + write, {"fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
                           "fetch_factor": float(f.get("fetch_factor", "nan")),
                           "write_factor": float(f.get("write_factor", "nan")),
                           "source": f"{PROFILE_DIR}/{TRAFFIC_SUMMARY}"}


def committed_trace(avg_bytes: float, launches: int):
    """The GEMV's rocprofv3 kernel-trace average from the committed summary, as
    a roofline figure beside the live one (null once the sources changed)."""
    f = read_summary_fields(os.path.join(ROOT, PROFILE_DIR, TRACE_SUMMARY))
    if not f or f.get("gemv_source_sha256") != gemv_digest():
        return None
    try:
        us = float(f["gemv_avg_us_rocprof"])
    except (KeyError, ValueError):
        return None
    gbs = avg_bytes / (us * 1e-6) / 1e9
    out = {"avg_launch_us_rocprof": us, "achieved_GB_s_rocprof": round(gbs, 1),
           "frac_rocprof": round(gbs / HBM_PEAK_GBS, 4),
           "source": f"{PROFILE_DIR}/{TRACE_SUMMARY}"}
    for k in ("gemv_avg_us_bench_untraced", "tracer_overhead"):
        if k in f:
            out[k] = f[k]
    return out


def cpu_baseline(orc, pass_bytes: int, log):
    """The CPU oracle (dequantize, then fp64 matmul; the head: dequantize the
    int8 table, then the fp64 product) on a bounded sample of every workload,
    at 1 and 4 threads (the page's thread counts) and on every host core,
    median of 3 runs each.  GB/s of algorithmic bytes; equivalent tokens/s =
    rows / time for the whole workload at that rate.  Results do not depend
    on the thread count (each output's sum runs in order)."""
    import platform
    import statistics

    import synth

    nproc = os.cpu_count() or 1
    threads = sorted({1, 4, nproc})
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass

    def w4_case(shapes, M, cfg, with_bias):
        items = []
        for slot, (K, N) in shapes:
            W = synth.weights(K, N, cfg, 0, slot)
            packed = orc.quantize_pack(W)
            x = synth.activations(M, K, cfg, 0, slot)
            b = synth.bias(N, cfg, 0, slot) if with_bias else None
            nb = K * N // 2 + (K // 32) * N * 4 + (K // 32) * N // 2
            items.append((x, packed, b, nb + 4 * M * K + 4 * M * N + (4 * N if with_bias else 0)))
        return (lambda: [orc.w4_matmul(x, *pk, b) for x, pk, b, _ in items],
                sum(it[3] for it in items))

    cases = []
    f1, b1 = w4_case([(0, (768, 768))], 1, synth.CFG_SINGLE, False)
    cases.append(("config1_768x768_m1", f1, b1, b1, 1, "the whole matmul"))
    f2, b2 = w4_case(list(enumerate(synth.GPT2_SHAPES)), 1, synth.CFG_GPT2_DECODE, True)
    cases.append(("config2_gpt2_decode_pass_m1", f2, b2, b2 * synth.GPT2_LAYERS, 1,
                  "layer 0 of 12 (4 matmuls with bias)"))
    E = synth.head_table()
    Q, hs = orc.i8_quantize_head(E)
    del E
    xl = synth.activations(1, synth.GPT2_HIDDEN, synth.CFG_HEAD)[0]
    bh = synth.GPT2_HIDDEN * synth.GPT2_VOCAB + 8 * synth.GPT2_VOCAB + 4 * synth.GPT2_HIDDEN
    cases.append(("config3_int8_head_768x50257", lambda: orc.i8_head_logits(xl, Q, hs), bh, bh, 1,
                  "the whole head (last row)"))
    f4, b4 = w4_case([(1, (768, 768))], synth.GPT2_PROMPT, synth.CFG_GPT2_PREFILL, True)
    full4 = sum(K * N // 2 + (K // 32) * N * 4 + (K // 32) * N // 2
                + 4 * synth.GPT2_PROMPT * (K + N) + 4 * N
                for K, N in synth.GPT2_SHAPES) * synth.GPT2_LAYERS
    cases.append(("config4_gpt2_prefill_m58_body", f4, b4, full4, synth.GPT2_PROMPT,
                  "the 768x768 out-projection of layer 0 at M=58 (the body's 48 matmuls "
                  "scaled by bytes; the head is config 3)"))
    f5, b5 = w4_case(list(enumerate(synth.DENSE38_SHAPES)), 1, synth.CFG_DENSE38, False)
    cases.append(("config5_dense38_pass_m1", f5, b5, pass_bytes, 1,
                  "layer 0 of 32 (4 matmuls)"))
    before = orc.threads()
    out = {}
    try:
        for name, fn, sample_bytes, full_bytes, rows, sample in cases:
            res = {}
            for t in threads:
                orc.set_threads(t)
                times = []
                for _ in range(3):
                    t0 = time.perf_counter()
                    fn()
                    times.append(time.perf_counter() - t0)
                med = statistics.median(times)
                gbs = sample_bytes / med / 1e9
                res[str(t)] = {"s": round(med, 4), "GB_s": round(gbs, 4),
                               "tokens_per_s_equiv": round(rows * gbs * 1e9 / full_bytes, 4)}
            out[name] = {"sample": sample, "sample_bytes": sample_bytes, "threads": res}
            log(f"CPU oracle {name}: {res}")
    finally:
        orc.set_threads(before)
    main = out["config5_dense38_pass_m1"]["threads"][str(nproc)]
    return {"value": main["GB_s"], "unit": "GB/s", "cores": nproc, "kind": "oracle",
            "sample": "layer 0 of the 3.8B-dense M=1 pass (4 matmuls, "
                      f"{b5 / 1e6:.1f} MB), dequantize then fp64 matmul, median of 3, "
                      f"{nproc} threads; every workload at 1, 4 and {nproc} threads below",
            "tokens_per_s_equiv": main["tokens_per_s_equiv"], "cpu_model": model,
            "threads": threads, "configs": out}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--skip-secondary", action="store_true")
    p.add_argument("--kernel", choices=("kmajor", "canonical"),
                   default=os.environ.get("W4_KERNEL", "kmajor"),
                   help="GEMV timed in the step (A/B switch; also W4_KERNEL)")
    p.add_argument("--skip-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU-oracle time budget for the baseline sample")
    p.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    p.add_argument("--profile-run", action="store_true",
                   help="short eager run for hardware counters: `--steps` M=1 passes, then "
                        "a plain copy of known size for calibration")
    p.add_argument("--profile-rows", type=int, default=1,
                   help="with --profile-run: rows of x in the profiled passes (4: the "
                        "matrix-core kernels' traffic)")
    p.add_argument("--profile-run-mfma", action="store_true",
                   help="short eager run for matrix-core counters: `--steps` passes of the "
                        "3.8B body at M=4 (prepacked) and M=16 (both layouts) and of the "
                        "GPT-2 prefill at M=58")
    p.add_argument("--summarize-profiles", metavar="DIR", default=None,
                   help="turn rocprofv3 CSV output under DIR into the profile summaries")
    p.add_argument("--out", default=PROFILE_DIR, help="where --summarize-profiles writes")
    p.add_argument("--probes", action="store_true",
                   help="only the machine probes behind the launch-cost and streaming-rate "
                        "figures: near-empty launches in a graph, and one streaming-read "
                        "launch per buffer at 6 MiB to 1 GiB (one JSON line)")
    return p.parse_args()


PROBE_MIB = (6, 16, 32, 64, 256, 1024)
PROBE_POOL_BYTES = 2 << 30     # buffers rotated per size: 8x the 256 MB Infinity Cache


def probes(w4, torch, dev, capture, time_graph, log, args):
    """Launch cost and single-launch streaming rate, with the library's own
    streaming-read kernel (w4_read_bytes), so that the figures the design
    notes quote can be measured again from committed code."""
    words = max(w4._lib.w4_read_bytes_words(n << 20, L) for n in PROBE_MIB for L in FLOOR_LOADS)
    out = torch.empty(words, dtype=torch.int32, device=dev)
    steps = max(5, args.steps // 2)

    # a launch that reads 16 bytes (one workgroup): the fixed cost of a graph node
    tiny = torch.zeros(16, dtype=torch.uint8, device=dev)
    launch = {}
    for n in (1, 32, 128):
        g = capture(lambda n=n: [w4.w4_read_bytes(tiny, 4, out=out) for _ in range(n)])
        ms, _ = time_graph(g, steps, 2)
        del g
        launch[str(n)] = round(1e3 * ms / n, 3)
    log(f"near-empty launch, us per node by graph length: {launch}")

    stream = {}
    for mib in PROBE_MIB:
        nbytes = mib << 20
        nbuf = max(2, PROBE_POOL_BYTES // nbytes)
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        best = None
        for L in FLOOR_LOADS:
            g = capture(lambda L=L: [w4.w4_read_bytes(b, L, out=out) for b in bufs])
            ms, _ = time_graph(g, steps, 2)
            del g
            us = 1e3 * ms / nbuf
            if best is None or us < best[0]:
                best = (us, L)
        del bufs
        torch.cuda.empty_cache()
        us, L = best
        stream[f"{mib}MiB"] = {"us_per_launch": round(us, 3), "loads_per_lane": L,
                               "TB_s": round(nbytes / (us * 1e-6) / 1e12, 3),
                               "buffers_rotated": nbuf}
        log(f"streaming read {mib} MiB: {stream[f'{mib}MiB']}")
    line = {"probes": "w4_read_bytes", "device": torch.cuda.get_device_name(dev),
            "graph_replays": steps,
            "near_empty_launch_us_per_node": launch,
            "streaming_read_one_launch": stream}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.out)
        return
    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU sharding or collectives).", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import w4_block_dequant_amd as w4

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ------------------------------------------------------------------ setup
    pool = cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4))

    class Mat:
        __slots__ = ("layer", "slot", "K", "N", "Wq", "s", "z", "P", "b", "x", "y", "bytes",
                     "wbytes", "flops")

    def build_body(name, cfg, M, with_bias, outliers, f16=False, g64=False):
        shapes = synth.body(name)
        ahead = 16                  # bounded look-ahead: at most 16 fp32 matrices on the host
        futs = {}
        mats = []
        for i, (l, s, K, N) in enumerate(shapes):
            if i % 32 == 0:
                log(f"  {name}: matrix {i} of {len(shapes)}")
            for j in range(i, min(i + ahead, len(shapes))):
                if j not in futs:
                    lj, sj, Kj, Nj = shapes[j]
                    futs[j] = pool.submit(synth.weights, Kj, Nj, cfg, lj, sj)
            W = torch.from_numpy(futs.pop(i).result()).to(dev)
            m = Mat()
            m.layer, m.slot, m.K, m.N = l, s, K, N
            if f16:  # fp16-scale variant: binary16 scales, K-major copy only
                Wq, s16, z = w4.w4h_quantize_pack(W)
                m.P = w4.w4h_prepack_kmajor(Wq, s16, z)
                m.Wq = m.s = m.z = None
                del Wq, s16, z
            elif g64:  # group-64 affine variant: K-major copy only
                Wq, sg, mg = w4.w4g_quantize_pack(W)
                m.P = w4.w4g_prepack_kmajor(Wq, sg, mg)
                m.Wq = m.s = m.z = None
                del Wq, sg, mg
            else:
                m.Wq, m.s, m.z = w4.w4_quantize_pack(W)
                m.P = w4.w4_prepack_kmajor(m.Wq, m.s, m.z) if K % 64 == 0 else None
            del W
            m.b = torch.from_numpy(synth.bias(N, cfg, l, s)).to(dev) if with_bias else None
            m.x = torch.from_numpy(synth.activations(M, K, cfg, l, s, outliers=outliers)).to(dev)
            m.y = torch.empty((M, N), dtype=torch.float32, device=dev)
            if g64:  # codes + fp32 scale and minimum per 64 rows
                wbytes = K * N // 2 + 2 * 4 * (K // 64) * N
            else:
                wbytes = K * N // 2 + (K // 32) * N * (2 if f16 else 4) + (K // 32) * N // 2
            m.wbytes = wbytes
            m.bytes = wbytes + 4 * M * K + 4 * M * N + (4 * N if with_bias else 0)
            m.flops = 2 * M * K * N
            mats.append(m)
        torch.cuda.synchronize()
        return mats

    def with_x(mats, cfg, M, outliers):
        out = []
        for m in mats:
            n = Mat()
            for a in Mat.__slots__:
                setattr(n, a, getattr(m, a))
            n.x = torch.from_numpy(synth.activations(M, m.K, cfg, m.layer, m.slot,
                                                     outliers=outliers)).to(dev)
            n.y = torch.empty((M, m.N), dtype=torch.float32, device=dev)
            wbytes = m.K * m.N // 2 + (m.K // 32) * m.N * 4 + (m.K // 32) * m.N // 2
            n.bytes = wbytes + 4 * M * m.K + 4 * M * m.N + (4 * m.N if m.b is not None else 0)
            n.flops = 2 * M * m.K * m.N
            out.append(n)
        return out

    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)

    def matmul(m, layout):
        if layout == "kmajor":
            w4.w4_matmul_kmajor(m.x, *m.P, bias=m.b, out=m.y)
        else:
            w4.w4_matmul(m.x, m.Wq, m.s, m.z, m.b, out=m.y, workspace=ws)

    def run_pass(mats, head=None, layout="kmajor"):
        for m in mats:
            matmul(m, layout)
        if head is not None:
            head()

    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time_graph(g, steps, warmup):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall

    if args.probes:
        probes(w4, torch, dev, capture, time_graph, log, args)
        return

    log("building the 3.8B-dense-shaped body (2.32 GB packed) ...")
    t = time.perf_counter()
    dense = build_body("dense38", synth.CFG_DENSE38, 1, with_bias=False, outliers=False)
    log(f"  built in {time.perf_counter() - t:.1f} s")

    if args.profile_run:
        # eager passes (one dispatch per matmul), then the calibration copy
        mats = dense if args.profile_rows == 1 else with_x(dense, synth.CFG_DENSE38,
                                                           args.profile_rows, outliers=True)
        for _ in range(args.warmup):
            run_pass(mats)
        torch.cuda.synchronize()
        for i in range(args.steps):
            run_pass(mats)
            torch.cuda.synchronize()
            log(f"profile pass {i + 1} of {args.steps} done")
        src = torch.randn(COPY_FLOATS, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)      # reads and writes COPY_FLOATS * 4 bytes
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": True, "passes": args.steps, "launches_per_pass": len(dense),
                          "rows": args.profile_rows,
                          "bytes_per_pass": sum(m.bytes for m in mats),
                          "copy_bytes": COPY_FLOATS * 4}), flush=True)
        return

    if args.profile_run_mfma:
        # eager passes on the matrix-core paths: 3.8B body at M = 16 (prepacked:
        # the bf16 kernel; canonical: fp32 MFMA), GPT-2 body at M = 58
        # (prepacked: the bf16 kernel)
        d16 = with_x(dense, synth.CFG_DENSE38, 16, outliers=True)
        d4 = with_x(dense, synth.CFG_DENSE38, 4, outliers=True)
        gpt2 = build_body("gpt2", synth.CFG_GPT2_DECODE, 1, with_bias=True, outliers=False)
        pre = with_x(gpt2, synth.CFG_GPT2_PREFILL, synth.GPT2_PROMPT, outliers=False)
        for mats, layout, what in ((d4, "kmajor", "3.8B M=4 prepacked"),
                                   (d16, "kmajor", "3.8B M=16 prepacked"),
                                   (d16, "canonical", "3.8B M=16 canonical"),
                                   (pre, "kmajor", "GPT-2 M=58 prepacked")):
            run_pass(mats, layout=layout)
            torch.cuda.synchronize()
            for i in range(args.steps):
                run_pass(mats, layout=layout)
                torch.cuda.synchronize()
            log(f"profile passes done: {what}")
        print(json.dumps({"profile_run_mfma": True, "passes": args.steps}), flush=True)
        return

    # ------------------------------------------------------------ timed steps
    graph = capture(lambda: run_pass(dense, layout=args.kernel))
    ms, wall = time_graph(graph, args.steps, args.warmup)
    pass_bytes = sum(m.bytes for m in dense)
    pass_flops = sum(m.flops for m in dense)
    value = pass_bytes / (ms * 1e-3) / 1e9
    log(f"dense38 M=1 pass ({args.kernel}): {ms:.4f} ms, {value:.1f} GB/s, {1e3 / ms:.1f} tok/s")

    # ------------------------------------------------------ per-kernel roofline
    # Every launch of the timed pass is the GEMV kernel, so its average launch
    # duration is the timed pass time (HIP events on the launch stream around
    # the graph replays) over the launches; the small gaps between graph nodes
    # are included, which makes it a slight overestimate.
    launches = len(dense)
    avg_bytes = pass_bytes / launches
    avg_ms = ms / launches
    achieved = avg_bytes / (avg_ms * 1e-3) / 1e9
    per_shape = {}
    for slot, (K, N) in enumerate(synth.DENSE38_SHAPES):
        sub = [m for m in dense if m.slot == slot]
        gs = capture(lambda: run_pass(sub, layout=args.kernel))
        mss, _ = time_graph(gs, max(5, args.steps // 2), 2)
        del gs
        us = 1e3 * mss / len(sub)
        # the same matrix replayed as often, so that it sits in the Infinity
        # Cache: how much of a launch is its bytes, and how much fixed cost
        gw = capture(lambda: run_pass([sub[0]] * len(sub), layout=args.kernel))
        msw, _ = time_graph(gw, max(5, args.steps // 2), 2)
        del gw
        usw = 1e3 * msw / len(sub)
        per_shape[f"{K}x{N}"] = {"us": round(us, 3),
                                 "GB_s": round(sub[0].bytes / (us * 1e-6) / 1e9, 1),
                                 "us_cache_warm": round(usw, 3),
                                 "cold_over_warm": round(us / usw, 3)}
    log(f"GEMV per launch: {1e3 * avg_ms:.2f} us avg, {achieved:.1f} GB/s; {per_shape}")
    traffic, traffic_detail = committed_traffic()
    profile = committed_trace(avg_bytes, launches)

    # the launch floor: the same 128 launches reading each matrix's packed bytes
    # with the streaming-read reference and nothing else
    wb = [m.wbytes for m in dense]
    floor_bufs = [torch.empty(n, dtype=torch.uint8, device=dev) for n in wb]
    floor_out = torch.empty(1 << 20, dtype=torch.int32, device=dev)
    floor = {}
    for L in FLOOR_LOADS:
        gf = capture(lambda L=L: [w4.w4_read_bytes(buf, L, out=floor_out) for buf in floor_bufs])
        msf, _ = time_graph(gf, max(5, args.steps // 2), 2)
        del gf
        floor[L] = msf
    floor_L = min(floor, key=floor.get)
    floor_ms = floor[floor_L]
    # per shape, as for the GEMV: graphs of one shape's 32 launches
    floor_shape = {}
    for K, N in synth.DENSE38_SHAPES:
        bufs = [b for b, m in zip(floor_bufs, dense) if (m.K, m.N) == (K, N)]
        gf = capture(lambda bufs=bufs: [w4.w4_read_bytes(b, floor_L, out=floor_out) for b in bufs])
        msf, _ = time_graph(gf, max(5, args.steps // 2), 2)
        del gf
        us = 1e3 * msf / len(bufs)
        floor_shape[f"{K}x{N}"] = {"us": round(us, 3),
                                   "gemv_over_floor": round(per_shape[f"{K}x{N}"]["us"] / us, 3)}
    floor_line = {"ms": round(floor_ms, 5), "us_per_launch": round(1e3 * floor_ms / launches, 3),
                  "GB_s": round(pass_bytes / (floor_ms * 1e-3) / 1e9, 1),
                  "frac_hbm_peak": round(pass_bytes / (floor_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "loads_per_lane": floor_L,
                  "ms_by_loads_per_lane": {str(k): round(v, 5) for k, v in floor.items()},
                  "per_shape": floor_shape,
                  "kernel": "w4_read_bytes (streaming read of each matrix's packed bytes, "
                            "one launch per matrix, same graph)"}
    del floor_bufs
    torch.cuda.empty_cache()
    log(f"launch floor: {floor_line}")

    # the same pass on the other layout, for comparison
    other = "canonical" if args.kernel == "kmajor" else "kmajor"
    gcan = capture(lambda: run_pass(dense, layout=other))
    ms_can, _ = time_graph(gcan, max(3, args.steps // 4), 2)
    del gcan
    other_pass = {"layout": other, "ms": round(ms_can, 4),
                  "GB_s": round(pass_bytes / (ms_can * 1e-3) / 1e9, 1),
                  "tokens_per_s": round(1e3 / ms_can, 1),
                  "vs_timed_pass": round(ms_can / ms, 4)}
    log(f"{other}-layout pass: {other_pass}")
    # restore the timed layout's outputs for the parity check below
    run_pass(dense, layout=args.kernel)

    # ------------------------------------------------ parity + CPU baseline
    import oracle
    orc = oracle.default()
    parity = {"checked_outputs": 0, "max_err_over_bound": 0.0, "ok": True}
    torch.cuda.synchronize()
    for m in dense[:8]:   # the first two layers: every shape twice
        W = synth.weights(m.K, m.N, synth.CFG_DENSE38, m.layer, m.slot)
        Wq, s, z = orc.quantize_pack(W)
        y_ref, bound = orc.w4_matmul(m.x.cpu().numpy(), Wq, s, z)
        y = m.y.cpu().numpy()
        r = float(np.max(np.abs(y.astype(np.float64) - y_ref) / bound))
        parity["checked_outputs"] += y.size
        parity["max_err_over_bound"] = max(parity["max_err_over_bound"], r)
        parity["ok"] &= bool(r <= 1.0)
    log(f"parity: {parity}")
    cpu = None
    if not args.skip_cpu:
        cpu = cpu_baseline(orc, pass_bytes, log)

    # ------------------------------------------------------------- secondary
    secondary = {}
    if not args.skip_secondary:
        # The same M=1 pass with the fused epilogues of a decode layer: SwiGLU
        # on the gate+up matmul (columns read as interleaved gate/up pairs,
        # 8192 outputs), the residual add on the out- and down-projections
        # (in place on one residual-stream row); QKV plain.
        resid = torch.zeros((1, synth.DENSE38_SHAPES[1][1]), device=dev)
        glu = torch.empty((1, synth.DENSE38_SHAPES[2][1] // 2), device=dev)

        def run_pass_ep(mats):
            for m in mats:
                if m.slot == 2:
                    w4.w4_matmul_kmajor(m.x, *m.P, act="swiglu", out=glu)
                elif m.slot in (1, 3):
                    w4.w4_matmul_kmajor(m.x, *m.P, residual=resid, out=resid)
                else:
                    w4.w4_matmul_kmajor(m.x, *m.P, bias=m.b, out=m.y)

        gep = capture(lambda: run_pass_ep(dense))
        msep, _ = time_graph(gep, max(5, args.steps // 2), 2)
        del gep
        secondary["dense38_m1_pass_fused_epilogues"] = {
            "ms": round(msep, 4), "tokens_per_s": round(1e3 / msep, 1),
            "vs_plain_pass": round(msep / ms, 4),
            "note": "SwiGLU fused into gate+up, residual add fused into out- and "
                    "down-projections; same weight bytes"}
        log(f"fused-epilogue pass: {secondary['dense38_m1_pass_fused_epilogues']}")

        # 3.8B body at M = 4 and M = 16 (batched decode), same weights.  From 3
        # rows on the K-major path runs the bf16 matrix cores on exact
        # three-part activations (one 16-row tile up to 16 rows): 3 bf16 MFMAs
        # per fp32 product on 16 rows however many are used.  That work at the
        # bf16 peak (348 GFLOP, 139 us) is below the HBM time of the 2.42 GB
        # (303 us at M = 16), so each line's own roofline is HBM.
        def own_roofline(mats, msv, mfma_rows):
            b = sum(m.bytes for m in mats)
            mf = sum(3 * 2 * mfma_rows * m.K * m.N for m in mats)
            t_hbm = b / (HBM_PEAK_GBS * 1e9)
            t_mfma = mf / (BF16_MFMA_PEAK_TFLOPS * 1e12)
            bound = "hbm" if t_hbm >= t_mfma else "bf16 mfma"
            return {"bound": bound, "bound_ms": round(1e3 * max(t_hbm, t_mfma), 4),
                    "frac": round(max(t_hbm, t_mfma) / (msv * 1e-3), 4),
                    "GB_s": round(b / (msv * 1e-3) / 1e9, 1),
                    "bf16_mfma_TFLOP_s_issued": round(mf / (msv * 1e-3) / 1e12, 1)}

        for Mb in (4, 16):
            dm = with_x(dense, synth.CFG_DENSE38, Mb, outliers=True)
            flm = sum(m.flops for m in dm)
            for layout in ("kmajor", "canonical"):
                gm = capture(lambda: run_pass(dm, layout=layout))
                msm, _ = time_graph(gm, 3, 1)
                del gm
                line_m = {"ms": round(msm, 4), "tokens_per_s": round(Mb * 1e3 / msm, 1),
                          "TFLOP_s": round(flm / (msm * 1e-3) / 1e12, 3)}
                if layout == "kmajor":
                    line_m["roofline"] = own_roofline(dm, msm, 16)
                    line_m["kernel"] = ("k_mm_x3k (whole-K, one launch per matmul; "
                                        if Mb <= 16 else "k_mm_x3 (split-K + reduce; ") + \
                        "bf16 x3 matrix cores, exact operands)"
                else:
                    line_m["frac_fp32_mfma_peak"] = round(
                        flm / (msm * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4)
                    line_m["kernel"] = "k_mm_mfma (fp32 matrix cores)"
                secondary[f"dense38_m{Mb}_pass_{layout}"] = line_m
                log(f"M={Mb} {layout} pass: {line_m}")
            del dm
        del graph
        dense.clear()
        torch.cuda.empty_cache()

        # the fp16-scale variant of the same body (0.578125 B/weight), M = 1
        log("building the fp16-scale body ...")
        dh = build_body("dense38", synth.CFG_DENSE38, 1, with_bias=False, outliers=False, f16=True)
        gh = capture(lambda: run_pass(dh))
        msh, _ = time_graph(gh, max(5, args.steps // 2), 2)
        hbytes = sum(m.bytes for m in dh)
        secondary["dense38_m1_pass_fp16_scales"] = {
            "ms": round(msh, 4), "tokens_per_s": round(1e3 / msh, 1),
            "GB_s": round(hbytes / (msh * 1e-3) / 1e9, 1),
            "algorithmic_bytes_per_step": hbytes}
        del gh
        dh.clear()
        torch.cuda.empty_cache()

        # the group-64 affine variant of the same body (0.625 B/weight), M = 1
        log("building the group-64 affine body ...")
        dg = build_body("dense38", synth.CFG_DENSE38, 1, with_bias=False, outliers=False,
                        g64=True)
        gg64 = capture(lambda: [w4.w4g_matmul_kmajor(m.x, *m.P, out=m.y) for m in dg])
        msg64, _ = time_graph(gg64, max(5, args.steps // 2), 2)
        del gg64
        g64_bytes = sum(m.bytes for m in dg)
        secondary["dense38_m1_pass_group64_affine"] = {
            "ms": round(msg64, 4), "tokens_per_s": round(1e3 / msg64, 1),
            "GB_s": round(g64_bytes / (msg64 * 1e-3) / 1e9, 1),
            "algorithmic_bytes_per_step": g64_bytes}
        log(f"group-64 affine pass: {secondary['dense38_m1_pass_group64_affine']}")
        dg.clear()
        torch.cuda.empty_cache()

        gpt2 = build_body("gpt2", synth.CFG_GPT2_DECODE, 1, with_bias=True, outliers=False)
        gb = sum(m.bytes for m in gpt2)
        for layout in ("kmajor", "canonical"):
            gg = capture(lambda: run_pass(gpt2, layout=layout))
            msg, _ = time_graph(gg, 200, 20)
            secondary[f"gpt2_decode_pass_{layout}"] = {
                "ms": round(msg, 5), "tokens_per_s": round(1e3 / msg, 1),
                "GB_s": round(gb / (msg * 1e-3) / 1e9, 1),
                "note": "55 MB body: resident in the 256 MB Infinity Cache across passes"}
            del gg

        # the same pass cold: 20 copies of the prepacked body (1.1 GB, over
        # four times the Infinity Cache) read in turn, one pass per copy
        copies = [[tuple(t.clone() for t in m.P) for m in gpt2] for _ in range(20)]

        def run_cold():
            for cp in copies:
                for m, P in zip(gpt2, cp):
                    w4.w4_matmul_kmajor(m.x, *P, bias=m.b, out=m.y)

        gc = capture(run_cold)
        msc, _ = time_graph(gc, 5, 1)
        del gc, copies
        msc /= 20
        secondary["gpt2_decode_pass_kmajor_cold"] = {
            "ms": round(msc, 5), "tokens_per_s": round(1e3 / msc, 1),
            "GB_s": round(gb / (msc * 1e-3) / 1e9, 1),
            "note": "20 copies of the 55 MB body read in turn: weights from HBM"}
        # one 768 x 768 matmul cold: 2,800 copies (1.06 GB) in turn
        m0 = gpt2[1]
        assert (m0.K, m0.N) == (768, 768)
        one = [tuple(t.clone() for t in m0.P) for _ in range(2800)]
        g1 = capture(lambda: [w4.w4_matmul_kmajor(m0.x, *P, bias=m0.b, out=m0.y) for P in one])
        ms1, _ = time_graph(g1, 3, 1)
        del g1, one
        us1 = 1e3 * ms1 / 2800
        secondary["gpt2_768x768_cold"] = {
            "us": round(us1, 3), "GB_s": round(m0.bytes / (us1 * 1e-6) / 1e9, 1),
            "note": "2,800 copies read in turn; latency-bound (384 KB per launch)"}
        log(f"GPT-2 cold: {secondary['gpt2_decode_pass_kmajor_cold']}, "
            f"{secondary['gpt2_768x768_cold']}")
        torch.cuda.empty_cache()

        # int8 head [768, 50257]: 8 copies of each table (> the 256 MB Infinity
        # Cache) are read in turn, 24 launches per graph replay, so every launch
        # streams its table from HBM and graph launch costs are amortized
        E = torch.from_numpy(synth.head_table()).to(dev)
        xl = torch.from_numpy(synth.activations(1, synth.GPT2_HIDDEN, synth.CFG_HEAD)).to(dev)[0]
        heads = {}
        hb_lane = 4 * synth.GPT2_VOCAB * 2 + 4 * synth.GPT2_HIDDEN
        for ldq in (synth.GPT2_VOCAB, 50272):
            Q, hs = w4.i8_quantize_head(E, ldq=ldq)
            heads[str(ldq)] = {"Q": Q, "hs": hs}
        del E
        Qk = w4.i8_prepack_head(heads["50272"]["Q"], synth.GPT2_VOCAB)
        hsk = heads["50272"]["hs"]
        outh = torch.empty(synth.GPT2_VOCAB, device=dev)
        variants = {
            "50257": (heads["50257"]["Q"], lambda T: w4.i8_head_logits(
                xl, T, heads["50257"]["hs"], out=outh, workspace=ws),
                synth.GPT2_HIDDEN * synth.GPT2_VOCAB),
            "50272": (heads["50272"]["Q"], lambda T: w4.i8_head_logits(
                xl, T, hsk, out=outh, workspace=ws), synth.GPT2_HIDDEN * 50272),
            "token_major": (Qk, lambda T: w4.i8_head_logits_kmajor(
                xl, T, hsk, synth.GPT2_HIDDEN, out=outh), synth.GPT2_HIDDEN * synth.GPT2_VOCAB),
        }
        head_times = {}
        for name, (T0, call, tbytes) in variants.items():
            tabs = [T0.clone() for _ in range(8)]
            gh = capture(lambda: [call(tabs[i % 8]) for i in range(24)])
            msh, _ = time_graph(gh, 20, 3)
            del gh, tabs
            us = 1e3 * msh / 24
            head_times[name] = {"us": round(us, 3),
                                "GB_s": round((tbytes + hb_lane) / (us * 1e-6) / 1e9, 1)}
        secondary["i8_head_768x50257"] = head_times

        # full-sequence logits [58 x 50257] (the export before the last-position
        # slice): one pass over the token-major table for all rows; 8 table
        # copies in turn
        xs = torch.from_numpy(synth.activations(synth.GPT2_PROMPT, synth.GPT2_HIDDEN,
                                                synth.CFG_HEAD)).to(dev)
        outs = torch.empty((synth.GPT2_PROMPT, synth.GPT2_VOCAB), device=dev)
        tabs = [Qk.clone() for _ in range(8)]
        gs = capture(lambda: [w4.i8_head_logits_rows(xs, tabs[i % 8], hsk, out=outs)
                              for i in range(16)])
        mss, _ = time_graph(gs, 10, 2)
        del gs, tabs
        us = 1e3 * mss / 16
        fb = (synth.GPT2_HIDDEN * synth.GPT2_VOCAB + 4 * synth.GPT2_VOCAB
              + 4 * synth.GPT2_PROMPT * (synth.GPT2_HIDDEN + synth.GPT2_VOCAB))
        ff = 2 * synth.GPT2_PROMPT * synth.GPT2_HIDDEN * synth.GPT2_VOCAB
        secondary["i8_head_full_sequence_58x768x50257"] = {
            "us": round(us, 3), "GB_s": round(fb / (us * 1e-6) / 1e9, 1),
            "TOP_s_equiv": round(ff / (us * 1e-6) / 1e12, 2)}

        pre = with_x(gpt2, synth.CFG_GPT2_PREFILL, synth.GPT2_PROMPT, outliers=False)
        last = pre[-1]
        lg = torch.empty(synth.GPT2_VOCAB, device=dev)

        def head_last():
            # the head reads the last prompt row of the body's output (768 wide)
            w4.i8_head_logits_kmajor(last.y[-1], Qk, hsk, synth.GPT2_HIDDEN, out=lg)

        fp = sum(m.flops for m in pre) + 2 * synth.GPT2_HIDDEN * synth.GPT2_VOCAB
        # own roofline: the body's bytes plus the head table at 8 TB/s, or the
        # bf16 MFMA work of the body (4 row tiles of 16, 3 parts) at 2.5 PFLOP/s
        pre_bytes = sum(m.bytes for m in pre) + hb_lane + synth.GPT2_HIDDEN * synth.GPT2_VOCAB
        pre_mfma = sum(3 * 2 * 64 * m.K * m.N for m in pre)
        t_pre = max(pre_bytes / (HBM_PEAK_GBS * 1e9), pre_mfma / (BF16_MFMA_PEAK_TFLOPS * 1e12))
        for layout, name in (("kmajor", "gpt2_prefill_m58_pass_plus_head"),
                             ("canonical", "gpt2_prefill_m58_pass_plus_head_canonical_mfma")):
            gp = capture(lambda: run_pass(pre, head_last, layout=layout))
            msp, _ = time_graph(gp, 20, 3)
            del gp
            secondary[name] = {
                "ms": round(msp, 4), "tokens_per_s": round(synth.GPT2_PROMPT * 1e3 / msp, 1),
                "TFLOP_s": round(fp / (msp * 1e-3) / 1e12, 3),
                "frac_own_roofline": round(t_pre / (msp * 1e-3), 4),
                "own_roofline_ms": round(1e3 * t_pre, 4)}
            if layout == "kmajor":
                # the same 48 dependent launches plus the head at one row (the
                # decode pass above and the token-major head): what launches
                # alone cost here, against a roofline that ignores them
                m1 = secondary["gpt2_decode_pass_kmajor"]["ms"] + head_times["token_major"]["us"] / 1e3
                secondary[name]["same_launches_at_m1_ms"] = round(m1, 4)
                secondary[name]["vs_same_launches_at_m1"] = round(msp / m1, 3)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; weights N(0,0.02) quantized on the GPU, x N(0,1))",
        "config": {
            "workload": "3.8B-dense-shaped decode body pass, M=1: 32 layers x (3072x9216, "
                        "3072x3072, 3072x16384, 8192x3072) W4 matmuls, uint4 block-32 "
                        "asymmetric, fp32 scales, packed uint4 zeros",
            "kernel_switch": args.kernel,
            "launches_per_step": launches,
            "algorithmic_bytes_per_step": pass_bytes,
            "flops_per_step": pass_flops,
        },
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "body_pass_tokens_per_s": round(1e3 / ms, 2),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "traffic_detail": traffic_detail,
                     "kernel": GEMV_KERNEL if args.kernel == "kmajor" else "k_gemv_fast",
                     "avg_launch_us": round(1e3 * avg_ms, 3),
                     "avg_bytes_per_launch": round(avg_bytes), "per_shape": per_shape,
                     "launch_floor": floor_line,
                     "frac_of_launch_floor": round(floor_ms / ms, 4),
                     "profile": profile},
        "other_layout_pass": other_pass,
        "cpu_baseline": cpu,
        "parity": parity,
        "secondary": secondary,
    }
    text = json.dumps(line)
    print(text, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(text + "\n")


def _csvs(root: str, suffix: str):
    out = []
    for d, _, files in os.walk(root):
        out += [os.path.join(d, f) for f in files if f.endswith(suffix)]
    return sorted(out)


def _pct(v, q):
    """Percentile q (0-100) of the values v, nearest-rank."""
    w = sorted(v)
    return w[min(len(w) - 1, max(0, int(round(q / 100.0 * (len(w) - 1)))))]


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    name = name.split("(")[0]
    return name if len(name) <= 90 else name[:87] + "..."


def summarize_profiles(src: str, out_dir: str):
    """Write the kernel-trace and traffic summaries from rocprofv3 CSV output.

    src/trace: `--kernel-trace --stats` of the timed bench command (plus the
    bench's own JSON line in src/trace_bench.json); src/fetch and src/write:
    `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` of `--profile-run`.  The counters
    are scaled by what they read for the calibration copy (COPY_FLOATS * 4
    bytes each way), so the traffic figures are in bytes.
    """
    import csv
    import statistics

    os.makedirs(out_dir, exist_ok=True)
    cmds = "\n".join(f"    {c}" for c in PROFILE_COMMANDS)

    # ---- kernel trace
    rows = []
    for f in _csvs(os.path.join(src, "trace"), "kernel_trace.csv"):
        rows += list(csv.DictReader(open(f)))
    durs = {}
    for r in rows:
        durs.setdefault(r["Kernel_Name"], []).append(
            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    gemv = [d for k, v in durs.items() if GEMV_KERNEL in k for d in v]
    def last_json(path):
        if not os.path.exists(path):
            return {}
        return json.loads(open(path).read().strip().splitlines()[-1])

    bench = last_json(os.path.join(src, "trace_bench.json"))   # the traced run
    plain = last_json(os.path.join(src, "bench.json"))         # the same bench, untraced
    lines = [f"# {GEMV_KERNEL}: kernel trace of the M=1 3.8B-dense-shaped body pass", "",
             "Made by:", "", cmds, "",
             "Every dispatch of the traced run: the timed graph replays, the per-shape "
             "graphs and the canonical-layout comparison pass.  The GEMV average below "
             "is over all K-major GEMV dispatches; the untraced bench's figure is the "
             "timed pass over its launches (`python bench.py --json-out <dir>/bench.json`).",
             ""]
    lines += ["| kernel | calls | avg us | p10 us | median us | p90 us | min us | max us |",
              "|---|---|---|---|---|---|---|---|"]
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1]))[:12]:
        lines.append(f"| `{_short(k)}` | {len(v)} | {statistics.mean(v) / 1e3:.3f} | "
                     f"{_pct(v, 10) / 1e3:.3f} | {_pct(v, 50) / 1e3:.3f} | {_pct(v, 90) / 1e3:.3f} | "
                     f"{min(v) / 1e3:.3f} | {max(v) / 1e3:.3f} |")
    avg_gemv_us = statistics.mean(gemv) / 1e3 if gemv else float("nan")
    lines += ["", f"- gemv_dispatches: {len(gemv)}",
              f"- gemv_avg_us_rocprof: {avg_gemv_us:.3f}"]
    if bench:
        rl = bench.get("roofline", {})
        lines += [f"- gemv_avg_us_bench_traced_run: {rl.get('avg_launch_us')}"]
    if plain:
        rl = plain.get("roofline", {})
        lines += [f"- gemv_avg_us_bench_untraced: {rl.get('avg_launch_us')}",
                  f"- bench_value_GB_s: {plain.get('value')}",
                  f"- bench_ms_per_step: {plain.get('ms_per_step')}",
                  f"- roofline_achieved_GB_s: {rl.get('achieved')}",
                  f"- roofline_frac: {rl.get('frac')}"]
        if bench and rl.get("avg_launch_us"):
            traced = bench.get("roofline", {}).get("avg_launch_us")
            if traced:
                # the same bench clock (HIP events around the graph) with and
                # without the tracer: what tracing adds per launch
                lines.append(f"- tracer_overhead: {traced / rl['avg_launch_us']:.4f}")
    # per launch shape: the trace's dispatches grouped by grid and workgroup size
    groups = {}
    for r in rows:
        if GEMV_KERNEL in r["Kernel_Name"]:
            key = (int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if groups:
        lines += ["", "GEMV dispatches by launch shape (grid threads, workgroup threads; the "
                  "3.8B shapes are 147456/192 for 3072x9216, 98304/192 for 3072x3072, "
                  "196608/192 for 3072x16384 and 131072/256 for 8192x3072):", "",
                  "| grid | workgroup | calls | avg us | median us |", "|---|---|---|---|---|"]
        for (gx, wx), v in sorted(groups.items()):
            lines.append(f"| {gx} | {wx} | {len(v)} | {statistics.mean(v) / 1e3:.3f} | "
                         f"{_pct(v, 50) / 1e3:.3f} |")
        if plain:
            lines += ["", "Untraced per-shape launch times of the same bench (graphs of one "
                      "shape's 32 launches, HIP events, gaps included): "
                      + json.dumps(plain.get("roofline", {}).get("per_shape", {}))]
    lines.append(f"- gemv_source_sha256: {gemv_digest()}")
    with open(os.path.join(out_dir, TRACE_SUMMARY), "w") as f:
        f.write("\n".join(lines) + "\n")

    # ---- counters
    def per_dispatch(sub, counter):
        vals = {}
        for f in _csvs(os.path.join(src, sub), "counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = (f, r["Dispatch_Id"])
                name, v = r["Kernel_Name"], float(r["Counter_Value"])
                vals[key] = (name, vals.get(key, (name, 0.0))[1] + v)
        return list(vals.values())

    copy_bytes = COPY_FLOATS * 4
    res = {}
    for sub, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        d = per_dispatch(sub, counter)
        copy = [v for k, v in d if "neg_kernel" in k]
        g = [v for k, v in d if GEMV_KERNEL in k]
        if not copy or not g:
            raise SystemExit(f"no {counter} rows for the copy or the GEMV under {src}/{sub}")
        factor = statistics.median(copy) * 1024.0 / copy_bytes
        res[sub] = {"factor": factor, "per_launch": statistics.mean(g) * 1024.0 / factor,
                    "n": len(g), "copy_kib": statistics.median(copy), "gemv_kib": statistics.mean(g)}
    alg = None
    if bench:
        alg = bench.get("roofline", {}).get("avg_bytes_per_launch")
    lines = [f"# {GEMV_KERNEL}: HBM traffic per launch, M=1 3.8B-dense-shaped body pass", "",
             "Made by:", "", cmds, "",
             "FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  Each is scaled by "
             "what it reads for a plain copy kernel (`torch.neg`, "
             f"{copy_bytes} bytes read and {copy_bytes} bytes written) so that the figures "
             "below are bytes.", "",
             f"- fetch_copy_kib: {res['fetch']['copy_kib']:.1f}",
             f"- write_copy_kib: {res['write']['copy_kib']:.1f}",
             f"- fetch_factor: {res['fetch']['factor']:.5f}",
             f"- write_factor: {res['write']['factor']:.5f}",
             f"- gemv_dispatches_counted: {res['fetch']['n']}",
             f"- fetch_kib_per_launch_raw: {res['fetch']['gemv_kib']:.1f}",
             f"- write_kib_per_launch_raw: {res['write']['gemv_kib']:.1f}",
             f"- fetch_bytes_per_launch: {res['fetch']['per_launch']:.0f}",
             f"- write_bytes_per_launch: {res['write']['per_launch']:.0f}"]
    if alg:
        tot = res["fetch"]["per_launch"] + res["write"]["per_launch"]
        lines += [f"- algorithmic_bytes_per_launch: {alg}",
                  f"- traffic_over_algorithmic: {tot / alg:.4f}"]
    # cross-check: the raw read requests at the memory interface (32-byte,
    # 64-byte and 128-byte ones) counted separately, for the copy and the GEMV
    rq = {c: per_dispatch("rdreq", c) for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum",
                                               "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_DRAM_sum")}
    if all(rq.values()):
        def req_bytes(sel):
            tot = {}
            for c, d in rq.items():
                v = [x for k, x in d if sel(k)]
                tot[c] = statistics.median(v) if v else float("nan")
            r, r32, bub = tot["TCC_EA0_RDREQ_sum"], tot["TCC_EA0_RDREQ_32B_sum"], tot["TCC_BUBBLE_sum"]
            return 128 * bub + 64 * (r - bub - r32) + 32 * r32, tot
        cb, ct = req_bytes(lambda k: "neg_kernel" in k)
        gb, gt = req_bytes(lambda k: GEMV_KERNEL in k)
        lines += ["", "Raw read requests at the memory interface (median per dispatch): "
                  "128-byte (TCC_BUBBLE), 32-byte (TCC_EA0_RDREQ_32B) and the rest 64-byte "
                  "(of TCC_EA0_RDREQ); DRAM requests (TCC_EA0_RDREQ_DRAM) beside them.", "",
                  f"- rdreq_copy_requests: {ct['TCC_EA0_RDREQ_sum']:.0f}",
                  f"- rdreq_copy_bytes_from_requests: {cb:.0f}",
                  f"- rdreq_copy_fraction_of_true_bytes: {cb / copy_bytes:.5f}",
                  f"- rdreq_gemv_requests: {gt['TCC_EA0_RDREQ_sum']:.0f}",
                  f"- rdreq_gemv_32B_requests: {gt['TCC_EA0_RDREQ_32B_sum']:.0f}",
                  f"- rdreq_gemv_128B_requests: {gt['TCC_BUBBLE_sum']:.0f}",
                  f"- rdreq_gemv_dram_requests: {gt['TCC_EA0_RDREQ_DRAM_sum']:.0f}",
                  f"- rdreq_gemv_bytes_from_requests: {gb:.0f}",
                  f"- rdreq_gemv_bytes_scaled_by_copy: {gb * copy_bytes / cb:.0f}"]
    lines.append(f"- gemv_source_sha256: {gemv_digest()}")
    with open(os.path.join(out_dir, TRAFFIC_SUMMARY), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(os.path.join(out_dir, TRACE_SUMMARY)).read())
    print(open(os.path.join(out_dir, TRAFFIC_SUMMARY)).read())

    # ---- kernel trace of the whole bench, secondary workloads included
    rows = []
    for f in _csvs(os.path.join(src, "trace_all"), "kernel_trace.csv"):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        return
    durs = {}
    for r in rows:
        durs.setdefault(r["Kernel_Name"], []).append(
            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = ["# Kernel trace of the whole bench: the timed pass and every secondary workload",
             "", "Made by:", "", cmds, "",
             "Every dispatch of the traced run of the full bench (the secondary lines "
             "included), by total time.  Template arguments name the instantiation: "
             "`k_gemv_kmajor<rows, passes, ragged, lane mode, fp16 scales, epilogue, affine, "
             "whole-run x>` the K-major GEMV (lane mode 2: 32-lane halves summed in "
             "registers), `k_mm_x3<MT, NT, QPW, DQ, fp16 scales>` the bf16 matrix-core "
             "matmul for M >= 3 with MT tiles of 16 rows (split-K), `k_mm_x3k<row block, "
             "column tiles per wave, waves, quads ahead, fp16 scales, three parts in one MFMA, "
             "quads per wave if fixed>` its whole-K form, `k_gemv_fast` + `k_splitk_reduce` the "
             "canonical-layout GEMV, `k_mm_mfma` the canonical fp32 matrix-core matmul, "
             "`k_head_fp32` the token-major last-row head, `k_head_whole<rows per lane, "
             "16-byte rows, lanes per row, waves>` the last-row head on the [K, ldq] table, "
             "`k_head_rows_x3` the full-sequence head, "
             "`k_read_bytes` the launch floor's streaming read.", "",
             "| kernel | calls | avg us | p10 us | median us | p90 us | min us | max us | total ms |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1]))[:40]:
        lines.append(f"| `{_short(k)}` | {len(v)} | {statistics.mean(v) / 1e3:.3f} | "
                     f"{_pct(v, 10) / 1e3:.3f} | {_pct(v, 50) / 1e3:.3f} | {_pct(v, 90) / 1e3:.3f} | "
                     f"{min(v) / 1e3:.3f} | {max(v) / 1e3:.3f} | {sum(v) / 1e6:.3f} |")
    if plain:  # tracing inflates graph replays: the untraced bench's lines
        lines += ["", "Secondary lines of the untraced bench (`python bench.py --json-out "
                  "<dir>/bench.json`, HIP events around graph replays):", ""]
        for k, v in plain.get("secondary", {}).items():
            lines.append(f"- {k}: {json.dumps(v)}")
    with open(os.path.join(out_dir, SECONDARY_SUMMARY), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(os.path.join(out_dir, SECONDARY_SUMMARY)).read())

    # ---- matrix-core utilisation of the M > 1 kernels
    per = {}  # (file, dispatch) -> {kernel, counters, duration}
    for f in _csvs(os.path.join(src, "mfma"), "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            d = per.setdefault((f, r["Dispatch_Id"]), {
                "k": r["Kernel_Name"], "c": {},
                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        return
    kern = {}
    for d in per.values():
        if "MfmaUtil" not in d["c"]:
            continue
        kern.setdefault(d["k"], []).append(d)
    lines = ["# Matrix-core utilisation of the M > 1 kernels", "", "Made by:", "", cmds, "",
             "Counters per dispatch of `--profile-run-mfma` (eager passes: the 3.8B body at "
             "M = 4 prepacked, at M = 16 on the prepacked and the canonical layout, the "
             "GPT-2 body at M = 58 prepacked).  `MfmaUtil` is rocprofv3's derived metric: "
             "MFMA-busy cycles over active cycles times SIMDs, in percent.  MFMA FLOP/s "
             "count the matrix-core operations the kernel issued (MOPS x 512 over the "
             "dispatch's duration under counter collection): `k_mm_x3` (split-K) and "
             "`k_mm_x3k` (whole-K, up to 16 rows; row groups of 16 up to 128 rows on small "
             "matrices) issue three bf16 MFMAs per fp32 product "
             "(exact three-part splits of each activation) on whole 16-row tiles, so their "
             "useful fp32 rate is at most a third of the bf16 rate, and at M = 4 a quarter "
             "of that again; `k_mm_mfma` runs fp32 MFMA.  Peaks: bf16 2.5 PFLOP/s, fp32 "
             "157.3 TFLOP/s (dense).", "",
             "| kernel | dispatches | MfmaUtil % (mean) | fp16 MFMA TFLOP/s | "
             "bf16 MFMA TFLOP/s | fp32 MFMA TFLOP/s | avg us |",
             "|---|---|---|---|---|---|---|"]
    for k, ds in sorted(kern.items(), key=lambda kv: -sum(d["ns"] for d in kv[1])):
        util = statistics.mean(d["c"]["MfmaUtil"] for d in ds)
        ns = sum(d["ns"] for d in ds)
        h16 = sum(d["c"].get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) for d in ds) * 512
        bf = sum(d["c"].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for d in ds) * 512
        f32 = sum(d["c"].get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) for d in ds) * 512
        if h16 == 0 and bf == 0 and f32 == 0:
            continue
        lines.append(f"| `{_short(k)}` | {len(ds)} | {util:.1f} | {h16 / ns / 1e3:.1f} | "
                     f"{bf / ns / 1e3:.1f} | {f32 / ns / 1e3:.1f} | {ns / len(ds) / 1e3:.2f} |")
    # issue and wait counters of the same passes (a run of their own)
    sq = {}
    for f in _csvs(os.path.join(src, "sq"), "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            d = sq.setdefault((f, r["Dispatch_Id"]), {
                "k": r["Kernel_Name"], "c": {},
                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    sqk = {}
    for d in sq.values():
        if d["c"].get("SQ_WAVES", 0.0) > 0 and ("x3" in d["k"] or "mfma" in d["k"]):
            sqk.setdefault(d["k"], []).append(d)
    if sqk:
        lines += ["", "Issue and wait counters (`--pmc SQ_WAVES SQ_WAVE_CYCLES SQ_INSTS_VALU "
                  "SQ_ACTIVE_INST_VALU SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_INSTS_LDS "
                  "SQ_LDS_BANK_CONFLICT`, same passes, summed over each kernel's "
                  "dispatches).  VALU busy: SQ_ACTIVE_INST_VALU (one quad-cycle, 4 clocks, "
                  "per wave64 instruction) over the 1024 SIMDs x 2.4 GHz x the dispatch "
                  "durations.  Waiting to issue: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (the wave "
                  "holds an instruction it cannot issue yet); at a wait count: SQ_WAIT_ANY / "
                  "SQ_WAVE_CYCLES.", "",
                  "| kernel | dispatches | VALU instr per wave | VALU busy % | waiting to "
                  "issue % | at a wait count % | LDS bank-conflict cycles per LDS instr | "
                  "avg us |",
                  "|---|---|---|---|---|---|---|---|"]
        for k, ds in sorted(sqk.items(), key=lambda kv: -sum(d["ns"] for d in kv[1])):
            c = {n: sum(d["c"].get(n, 0.0) for d in ds) for n in (
                "SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
                "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT")}
            ns = sum(d["ns"] for d in ds)
            busy = 100.0 * c["SQ_ACTIVE_INST_VALU"] * 4 / (1024 * 2.4 * ns)
            wc = max(c["SQ_WAVE_CYCLES"], 1.0)
            lines.append(
                f"| `{_short(k)}` | {len(ds)} | {c['SQ_INSTS_VALU'] / c['SQ_WAVES']:.0f} | "
                f"{busy:.0f} | {100 * c['SQ_WAIT_INST_ANY'] / wc:.0f} | "
                f"{100 * c['SQ_WAIT_ANY'] / wc:.0f} | "
                f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_INSTS_LDS'], 1.0):.2f} | "
                f"{ns / len(ds) / 1e3:.2f} |")
    # HBM traffic of the matrix-core kernels: the 3.8B pass at M = 4
    # (`--profile-run --profile-rows 4`), FETCH_SIZE and WRITE_SIZE per
    # dispatch scaled by the same run's copy kernel, against the pass's
    # algorithmic bytes (weights once, x and y once) per launch
    import synth
    tr = {}
    for sub, counter in (("fetch4", "FETCH_SIZE"), ("write4", "WRITE_SIZE")):
        d = per_dispatch(sub, counter)
        copy = [v for k, v in d if "neg_kernel" in k]
        mm = [v for k, v in d if "k_mm_x3" in k]
        if copy and mm:
            factor = statistics.median(copy) * 1024.0 / copy_bytes
            tr[sub] = (statistics.mean(mm) * 1024.0 / factor, len(mm), factor)
    if len(tr) == 2:
        shapes = synth.DENSE38_SHAPES
        M4 = 4
        alg = sum(K * N // 2 + (K // 32) * N * 4 + (K // 32) * N // 2 + 4 * M4 * K + 4 * M4 * N
                  for K, N in shapes) / len(shapes)
        fb, nf, ff = tr["fetch4"]
        wb, _, wf = tr["write4"]
        lines += ["", "HBM traffic of the matrix-core kernels, 3.8B pass at M = 4 "
                  "(`--profile-run --profile-rows 4`: FETCH_SIZE, then WRITE_SIZE, per "
                  "dispatch of `k_mm_x3k`, each scaled by the same run's copy kernel):", "",
                  f"- dispatches_counted: {nf}",
                  f"- fetch_factor: {ff:.5f}",
                  f"- write_factor: {wf:.5f}",
                  f"- fetch_bytes_per_launch: {fb:.0f}",
                  f"- write_bytes_per_launch: {wb:.0f}",
                  f"- algorithmic_bytes_per_launch: {alg:.0f}",
                  f"- traffic_over_algorithmic: {(fb + wb) / alg:.4f}"]
    with open(os.path.join(out_dir, MFMA_SUMMARY), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(os.path.join(out_dir, MFMA_SUMMARY)).read())


if __name__ == "__main__":
    main()
