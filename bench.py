"""Throughput of the affine group-quantized matmul on one MI355X.

Headline workload (the decode GEMV at hidden size 5120): one step is one 4-bit
qmv with K = 5120 for each of the two projection widths N = 5120 and N = 13824,
M = 1, bf16 out. ``value`` is the algorithmic bytes of the step (codes, scales,
biases, activations, outputs, each moved once) divided by the measured step time,
in GB/s.

Inputs sit in HBM before timing starts. Each step reads a different copy of all
tensors (copies rotate through more than 1 GiB), so the 256 MB Infinity Cache and
the 4 MB L2s cannot serve them: every step streams its weights from HBM, as a
decode step does when every layer has its own weights.

Timing: after W eager warm-up steps, the K timed steps are captured into one HIP
graph, replayed once to upload it and once more untimed, then replayed R times
(``--repeats``), each replay between two HIP events on the stream the kernels run
on, so host-side launch cost is excluded. Every reported time is the median of
the R replays; ``spread_pct`` is (max - min) / median and ``reps_us`` lists them
all, the first (coldest) included. ``roofline`` is for the dominant kernel (the
N = 13824 GEMV), timed the same way on its own.

Also reported:
  ``suite``: every other workload of the hot path, timed the same way, each with a
      ``roofline`` object against its own bound (HBM, or the matrix cores for the
      600-token prefill GEMMs); the 8-bit vs 4-bit bytes-against-time ratios;
      counter figures and the traced-vs-untraced reconciliation from the committed
      rocprofv3 summaries under ``profiles/`` when they were taken on these kernel
      sources.
  ``measured_ceilings``: a plain streaming read of 8, 16, 40 and 160 MiB and 1 GiB in
      the decode GEMV's access shape, timed by graph replay like the workloads, and a loop of independent bf16 matrix-core
      instructions (``libbitmm_probe.so``): what this chip reaches, beside the
      published peaks.
  ``cpu_baseline``: the CPU oracle on the host cores, whole headline steps for about
      ``--cpu-seconds``; ``per_config`` times one bounded sample of every workload on
      all cores and, for the tiny, hidden-5120 and 8-bit GEMVs, on one core.

Profiling helpers (no GPU needed for the second):
  ``--only NAMES``: run only the suite workloads whose names contain one of the
      comma-separated strings (no headline, no CPU legs): one workload per process
      for rocprofv3 counter passes.
  ``--markers``: wrap each workload's timed replays in a ROCTx range named
      ``bitmm:<workload>`` (for ``rocprofv3 --marker-trace``).
  ``--summarize DIR``: read the rocprofv3 CSV output under DIR and print the summary
      text kept under ``profiles/`` (kernel statistics, per-workload kernel time per
      launch from the markers, counter figures per kernel). ``--bench-json`` names the
      untraced bench line of the same session, ``--workload`` takes the algorithmic
      bytes of one of its workloads for the traffic ratio, ``--title`` and ``--command``
      head the text. Every file under ``profiles/`` is this output, redirected.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats R] [--no-suite]
                       [--no-cpu] [--no-ceilings] [--calibrate-copy] [--only NAMES]
                       [--markers] [--summarize DIR [--bench-json FILE] [--workload NAME]
                                                    [--title TEXT] [--command CMD]]
"""

from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
ROTATE_BYTES = 1 << 30
CU_NUM, SIMD_NUM = 256, 1024    # MI355X compute units and SIMDs (counter normalisation)
XCD_NUM = 8                     # GRBM_GUI_ACTIVE comes summed over the 8 XCDs' counters

HEADLINE = ("qmv_M1_K5120_N5120_b4", "qmv_M1_K5120_N13824_b4")
TRACE_SUMMARY = "hot_path_kernel_trace"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_matmul_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def read_summary(name: str, src_hash: str):
    """key: value lines of a committed summary (profiles/<name>.txt), or None when it is
    missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256_16") != src_hash:
        return None
    return kv


def num(kv, key):
    try:
        return float(kv[key])
    except (KeyError, TypeError, ValueError):
        return None


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def suite_specs(I):
    """(kind, factory, bound): every workload of the hot path besides the headline. The
    600-token prefill GEMMs are bound by the matrix cores, everything else by HBM
    (the MoE prefill gathers at 103.8 flop/B, below the ridge of 2.5 PFLOP/s over
    8 TB/s = 312.5)."""
    return [
        ("qmv", lambda: I.hidden5120(1, 5120, 8), "hbm"),
        ("qmv", lambda: I.hidden5120(1, 13824, 8), "hbm"),
        ("qmm", lambda: I.hidden5120(600, 13824, 4), "mfma"),
        ("qmm", lambda: I.hidden5120(3, 13824, 4), "hbm"),
        ("qmm", lambda: I.hidden5120(600, 13824, 8), "mfma"),
        ("qmm", lambda: I.hidden5120(3, 13824, 8), "hbm"),
        ("gather", lambda: I.moe_gather("up"), "hbm"),
        ("gather", lambda: I.moe_gather("down"), "hbm"),
        ("gather_indexed", lambda: I.moe_prefill_indexed("up"), "hbm"),
        ("gather_indexed", lambda: I.moe_prefill_indexed("down"), "hbm"),
        ("gather_qmv", lambda: I.moe_decode("up", 1), "hbm"),
        ("gather_qmv", lambda: I.moe_decode("down", 1), "hbm"),
        ("gather_qmv", lambda: I.moe_decode("up", 4), "hbm"),
        ("gather_qmv", lambda: I.moe_decode("down", 4), "hbm"),
        ("gather_indexed", lambda: I.moe_prefill_indexed("up", tokens=46), "hbm"),
        ("gather_indexed", lambda: I.moe_prefill_indexed("down", tokens=46), "hbm"),
        ("gather_mm", lambda: I.moe_gather_mm("up"), "hbm"),
        ("gather_mm", lambda: I.moe_gather_mm("down"), "hbm"),
        ("gather_mm", lambda: I.moe_gather_mm("up", layout="kn"), "hbm"),
        ("qmv", lambda: I.random_dense(1, 13824, 5120, 2, seed=1), "hbm"),
        # 13952 rows rather than 13824: a grid of its own in kernel traces
        ("qmv", lambda: I.random_dense(1, 13952, 5120, 4, seed=1, group=128), "hbm"),
        ("qmm", lambda: I.random_dense(600, 13824, 5120, 4, seed=1, group=32), "mfma"),
    ]


def suite_names():
    """Workload names of the suite, in order (for --only), without building inputs."""
    return ["qmv_M1_K5120_N5120_b8", "qmv_M1_K5120_N13824_b8", "qmm_M600_K5120_N13824_b4",
            "qmm_M3_K5120_N13824_b4", "qmm_M600_K5120_N13824_b8", "qmm_M3_K5120_N13824_b8",
            "gather_up_B4584_E128_K2816_N704_b4", "gather_down_B4584_E128_K704_N2816_b4",
            "gather_indexed_up_B4584_E128_K2816_N704_b4", "gather_indexed_down_B4584_E128_K704_N2816_b4",
            "moe_decode_up_T1_B8_E128_K2816_N704_b4", "moe_decode_down_T1_B8_E128_K704_N2816_b4",
            "moe_decode_up_T4_B32_E128_K2816_N704_b4", "moe_decode_down_T4_B32_E128_K704_N2816_b4",
            "gather_indexed_up_B368_E128_K2816_N704_b4", "gather_indexed_down_B368_E128_K704_N2816_b4",
            "gather_mm_up_B4584_E128_K2816_N704_bf16_nk", "gather_mm_down_B4584_E128_K704_N2816_bf16_nk",
            "gather_mm_up_B4584_E128_K2816_N704_bf16_kn", "dense_M1_K5120_N13824_b2",
            "dense_M1_K5120_N13952_b4_g128", "dense_M600_K5120_N13824_b4_g32"]


class Case:
    """One workload on the device with rotating copies of every tensor."""

    def __init__(self, torch, problem, kind, out_dtype, copies=None):
        import bit_matmul_amd as bm
        self.torch, self.p, self.kind = torch, problem, kind
        dev = torch.device("cuda:0")

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev)

        self.ids = None
        if kind == "gather_mm":
            def half(a):
                t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
                return t.view(torch.bfloat16 if problem.dtype == "bf16" else torch.float16).to(dev)
            base = [half(problem.x), half(problem.w)]
        else:
            base = [bf16(problem.x), i32(problem.w), bf16(problem.scales), bf16(problem.biases)]
        if kind == "gather":
            base.append(i32(problem.expert_idx))
            rows = problem.B
        elif kind in ("gather_qmv", "gather_indexed", "gather_mm"):
            # the ids stay put: each step's rows read a different copy of every tensor
            self.ids = (None if problem.token_idx is None else i32(problem.token_idx),
                        i32(problem.expert_idx))
            rows = problem.B
        else:
            rows = problem.M
        out_shape = (rows, problem.N)
        self.bytes = problem.algorithmic_bytes(2 if out_dtype == torch.bfloat16 else 4)
        self.flops = problem.flops()
        per = sum(t.numel() * t.element_size() for t in base) + rows * problem.N * 2
        self.copies = copies or max(2, -(-ROTATE_BYTES // per))
        self.sets = []
        for i in range(self.copies):
            ts = [t.clone() for t in base]
            y = torch.empty(out_shape, dtype=out_dtype, device=dev)
            ws = None
            if kind == "gather":
                ws = torch.empty(bm.bitmm_gather_qmm_workspace_bytes(problem.B, problem.N, problem.E),
                                 dtype=torch.uint8, device=dev)
            elif kind == "gather_indexed":
                ws = torch.empty(bm.bitmm_gather_qmm_indexed_workspace_bytes(problem.B, problem.N, problem.E),
                                 dtype=torch.uint8, device=dev)
            elif kind == "gather_mm":
                ws = torch.empty(bm.bitmm_gather_mm_workspace_bytes(problem.B, problem.N, problem.E),
                                 dtype=torch.uint8, device=dev)
            self.sets.append((ts, y, ws))
        self.bm = bm
        self.i = 0

    def launch(self):
        ts, y, ws = self.sets[self.i % self.copies]
        self.i += 1
        bm, p = self.bm, self.p
        gs = getattr(p, "group", 64)
        if self.kind == "qmv":
            bm.bitmm_qmv(*ts, y, p.bits, group_size=gs)
        elif self.kind == "qmm":
            bm.bitmm_qmm(*ts, y, p.bits, group_size=gs)
        elif self.kind == "gather_qmv":
            bm.bitmm_gather_qmv(*ts, *self.ids, y, p.bits, group_size=gs)
        elif self.kind == "gather_indexed":
            bm.bitmm_gather_qmm_indexed(*ts, *self.ids, y, ws, p.bits, group_size=gs)
        elif self.kind == "gather_mm":
            bm.bitmm_gather_mm(*ts, *self.ids, y, ws, p.layout)
        else:
            bm.bitmm_gather_qmm(*ts, y, ws, p.bits, group_size=gs)


class Markers:
    """ROCTx ranges around timed regions (rocprofv3 --marker-trace); a no-op unless
    enabled."""

    def __init__(self, enabled: bool):
        self.lib = None
        if enabled:
            for name in ("librocprofiler-sdk-roctx.so", "/opt/rocm/lib/librocprofiler-sdk-roctx.so",
                         "libroctx64.so"):
                try:
                    self.lib = ctypes.CDLL(name)
                    break
                except OSError:
                    continue
            if self.lib is None:
                raise RuntimeError("--markers: no ROCTx library found")
            self.lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
            self.lib.roctxRangePushA.restype = ctypes.c_int
            self.lib.roctxRangePop.argtypes = []
            self.lib.roctxRangePop.restype = ctypes.c_int

    def push(self, name: str):
        if self.lib is not None:
            self.lib.roctxRangePushA(("bitmm:" + name).encode())

    def pop(self):
        if self.lib is not None:
            self.lib.roctxRangePop()


def time_steps(torch, cases, steps, warmup, repeats=1, markers=None, label=""):
    """Time `steps` steps (each launches every case once, in order) after `warmup` eager
    steps. The timed launches are captured into one HIP graph; it is replayed once to
    upload it and once untimed, then `repeats` times, each replay between two events on
    the stream it runs on, so the host's per-launch cost (Python argument marshalling)
    is not part of the measurement. Returns the seconds of each timed replay."""
    for _ in range(warmup):
        for c in cases:
            c.launch()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(steps):
            for c in cases:
                c.launch()
    torch.cuda.synchronize()
    graph.replay()                      # first replay uploads the graph
    graph.replay()                      # and one more brings the clocks up
    torch.cuda.synchronize()
    out = []
    if markers is not None:
        markers.push(label)
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / 1e3)
    if markers is not None:
        markers.pop()
    del graph
    return out


def stats(reps_s, per):
    """Median, spread and all repetitions, in microseconds per launch."""
    us = [r / per * 1e6 for r in reps_s]
    med = float(np.median(us))
    return med, {"reps_us": [round(u, 3) for u in us],
                 "spread_pct": round((max(us) - min(us)) / med * 100.0, 2) if med > 0 else None}


def roofline_obj(bound, nbytes, flops, secs, ceilings=None):
    if bound == "mfma":
        achieved = flops / secs / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
        if ceilings and ceilings.get("mfma_bf16_TFLOP_s"):
            r["frac_of_measured"] = round(achieved / ceilings["mfma_bf16_TFLOP_s"], 4)
    else:
        achieved = nbytes / secs / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(achieved / HBM_PEAK_GBS, 4)}
        if ceilings and ceilings.get("read_GB_s"):
            # the measured streaming read of the size closest to this workload's bytes
            sizes = ceilings["read_GB_s"]
            best = min(sizes, key=lambda k: abs(math.log(int(k) / max(nbytes, 1))))
            r["measured_read_GB_s_at"] = {"bytes": int(best), "GB_s": sizes[best]}
            r["frac_of_measured"] = round(achieved / sizes[best], 4)
    return r


def summarize(case, secs, name, bound, extra, ceilings):
    t = secs
    s = {"workload": name, "us_per_launch": round(t * 1e6, 3),
         "GB_s": round(case.bytes / t / 1e9, 1),
         "hbm_frac": round(case.bytes / t / 1e9 / HBM_PEAK_GBS, 4),
         "TFLOP_s": round(case.flops / t / 1e12, 2),
         "mfma_frac": round(case.flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
         "bytes": case.bytes, "flops": case.flops, "copies": case.copies}
    s.update(extra)
    s["roofline"] = roofline_obj(bound, case.bytes, case.flops, t, ceilings)
    return s


def attach_profiles(entry, src_hash):
    """Counter figures and the traced-vs-untraced reconciliation of one workload, from
    the committed summaries when they match these kernel sources."""
    name = entry["workload"]
    tr = read_summary(TRACE_SUMMARY, src_hash)
    if tr is not None:
        ksum = num(tr, f"wl.{name}.kernel_us_per_launch")
        if ksum:
            entry["reconciliation"] = {
                "traced_kernel_sum_us": ksum,
                "untraced_events_us": entry["us_per_launch"],
                "kernel_share_pct": round(100.0 * ksum / entry["us_per_launch"], 1)}
    pm = read_summary(f"counters_{name}", src_hash)
    if pm is not None:
        c = {}
        for key in ("traffic_bytes_per_launch", "traffic_over_algorithmic", "MfmaUtil_pct", "VALUBusy_pct",
                    "OccupancyPercent", "TA_BUSY_avr_pct", "LDSBankConflict_pct"):
            v = num(pm, key)
            if v is not None:
                c[key] = v
        if c:
            entry["counters"] = c
            if "traffic_bytes_per_launch" in c:
                entry["roofline"]["traffic"] = int(c["traffic_bytes_per_launch"])


# ---------------------------------------------------------------------------
# measured ceilings
# ---------------------------------------------------------------------------

def measured_ceilings(torch):
    path = os.path.join(ROOT, "bit_matmul_amd", "libbitmm_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build with `python -m bit_matmul_amd.build`")
    L = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.bitmm_probe_stream_read_sink_words.argtypes = [I64, I]
    L.bitmm_probe_stream_read_sink_words.restype = I64
    L.bitmm_probe_stream_read.argtypes = [P, I64, I, P, P]
    L.bitmm_probe_stream_read.restype = I
    L.bitmm_probe_mfma.argtypes = [P, I, I, P]
    L.bitmm_probe_mfma.restype = I
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    out = {"read_GB_s": {}, "read_unroll": {}}

    class _Read:
        """One probe read per launch, rotating through the buffers (on the stream current at
        launch time, so that it can be captured)."""

        def __init__(self, bufs, size, unroll, sink):
            self.bufs, self.size, self.unroll, self.sink, self.i = bufs, size, unroll, sink, 0

        def launch(self):
            b = self.bufs[self.i % len(self.bufs)]
            self.i += 1
            rc = L.bitmm_probe_stream_read(b.data_ptr(), self.size, self.unroll, self.sink.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"stream read probe failed ({rc})")

    # Sizes around every workload's bytes (the MoE decode's 9 MB, the N = 5120 GEMV's 15 MB,
    # the headline's 40 MB, the grouped GEMMs' 175 MB, the dense grouped product's 0.5 GB).
    for size in (8 << 20, 16 << 20, 40 << 20, 160 << 20, 1 << 30):
        copies = max(2, -(-ROTATE_BYTES // size)) if size < ROTATE_BYTES else 2
        bufs = [torch.ones(size, dtype=torch.uint8, device=dev) for _ in range(copies)]
        best = None
        for unroll in (4, 8, 16):
            sink = torch.empty(int(L.bitmm_probe_stream_read_sink_words(size, unroll)), dtype=torch.int32,
                               device=dev)
            steps = max(copies, 20) if size < (1 << 30) else 6
            # timed like the workloads: the reads captured into one graph, replayed
            secs = time_steps(torch, [_Read(bufs, size, unroll, sink)], steps, copies, repeats=3)
            gbs = size * steps / sorted(secs)[1] / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, unroll)
        out["read_GB_s"][str(size)] = round(best[0], 1)
        out["read_unroll"][str(size)] = best[1]
        log(f"ceiling: streaming read of {size >> 20} MiB: {best[0]:.1f} GB/s (unroll {best[1]})")
        del bufs
        torch.cuda.empty_cache()
    waves, iters = 2048, 20000
    sink = torch.empty(waves, dtype=torch.float32, device=dev)
    if L.bitmm_probe_mfma(sink.data_ptr(), waves, 200, stream) != 0:
        raise RuntimeError("mfma probe failed")
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    L.bitmm_probe_mfma(sink.data_ptr(), waves, iters, stream)
    e1.record()
    torch.cuda.synchronize()
    tflops = waves * iters * 8 * 32768 / (e0.elapsed_time(e1) / 1e3) / 1e12
    out["mfma_bf16_TFLOP_s"] = round(tflops, 1)
    out["mfma_probe"] = f"{waves} waves x {iters} x 8 independent v_mfma_f32_32x32x16_bf16"
    out["read_probe"] = ("one pass over the buffer, each wave instruction 1 KB contiguous, all loads of a wave "
                         "issued before use; best of 4, 8, 16 KB per wave; copies rotate through >= 1 GiB; "
                         "timed by graph replay like the workloads, middle of 3 replays")
    log(f"ceiling: bf16 matrix cores {tflops:.1f} TFLOP/s")
    return out


# ---------------------------------------------------------------------------
# CPU oracle
# ---------------------------------------------------------------------------

def cpu_baseline(problems, budget_s=10.0):
    """The oracle (as it is) on the host cores, repeating whole steps for about
    budget_s seconds; GB/s of algorithmic bytes."""
    import oracle
    threads = oracle.default_threads()
    nbytes = sum(p.algorithmic_bytes(2) for p in problems)
    t0 = time.perf_counter()
    steps = 0
    while True:
        for p in problems:
            oracle.qmm(p.x, p.w, p.scales, p.biases, p.bits, threads=threads)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 1000:
            break
    return {"value": round(steps * nbytes / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} full step(s) of the headline workload (qmv K=5120, N=5120 and "
                      f"N=13824, 4-bit, M=1) in {el:.1f} s, f64, {threads} threads"}


def oracle_sample(p, kind, macs_budget):
    """A prefix of the workload's output rows that the oracle computes in about
    macs_budget multiply-adds: (callable, rows taken, rows in full)."""
    import oracle
    if kind in ("qmv", "qmm"):
        full = p.M
        m = max(1, min(full, int(macs_budget // (p.N * p.K))))
        return (lambda th: oracle.qmm(p.x[:m], p.w, p.scales, p.biases, p.bits, group=p.group, threads=th)), m, full
    if kind == "gather":
        full = p.B
        m = max(1, min(full, int(macs_budget // (p.N * p.K))))
        return (lambda th: oracle.gather_qmm(p.x[:m], p.w, p.scales, p.biases, p.expert_idx[:m], p.bits,
                                             group=p.group, threads=th)), m, full
    if kind in ("gather_indexed", "gather_qmv"):
        full = p.B
        m = max(1, min(full, int(macs_budget // (p.N * p.K))))
        tok = None if p.token_idx is None else p.token_idx[:m]
        x = p.x if p.token_idx is not None else p.x[:m]
        return (lambda th: oracle.gather_qmm_indexed(x, p.w, p.scales, p.biases, tok, p.expert_idx[:m], p.bits,
                                                     group=p.group, threads=th)), m, full
    if kind == "gather_mm":
        full = p.B
        m = max(1, min(full, int(macs_budget // (p.N * p.K))))
        tok = None if p.token_idx is None else p.token_idx[:m]
        x = p.x if p.token_idx is not None else p.x[:m]
        return (lambda th: oracle.gather_mm(x, p.w, tok, p.expert_idx[:m], dtype=p.dtype, layout=p.layout,
                                            threads=th)), m, full
    raise ValueError(kind)


def oracle_per_config(entries, threads_all):
    """One bounded oracle sample per workload (about a second of work each) on all
    cores, and on one core for the tiny, hidden-5120 and 8-bit decode GEMVs; projected
    to the full workload by its multiply-add count, beside the GPU time."""
    out = []
    single = {"qmv_K512_N256_b4", "qmv_M1_K5120_N5120_b4", "qmv_M1_K5120_N13824_b4",
              "qmv_M1_K5120_N5120_b8", "qmv_M1_K5120_N13824_b8"}
    for name, p, kind, gpu_s in entries:
        for th in ((threads_all, 1) if name in single else (threads_all,)):
            fn, m, full = oracle_sample(p, kind, 8e7 * th)
            t0 = time.perf_counter()
            fn(th)
            el = time.perf_counter() - t0
            macs = m * p.N * p.K
            proj = el * full / m
            r = {"workload": name, "threads": th,
                 "sample": f"output rows 0..{m - 1} of {full}" if m < full else "whole workload",
                 "seconds": round(el, 4), "mac_per_s": round(macs / el, 1),
                 "projected_full_s": round(proj, 4)}
            if gpu_s:
                r["gpu_us"] = round(gpu_s * 1e6, 3)
                r["gpu_speedup"] = round(proj / gpu_s, 1)
            out.append(r)
            log(f"oracle {name} T={th}: {r['sample']} in {el:.3f} s -> {proj:.3f} s projected")
    return out


# ---------------------------------------------------------------------------
# rocprofv3 output summary
# ---------------------------------------------------------------------------

def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row and row[n] not in (None, ""):
            return row[n]
    low = {k.lower(): k for k in row}
    for n in names:
        k = low.get(n.lower())
        if k is not None and row[k] not in (None, ""):
            return row[k]
    return None


def _short(name: str, width: int = 150) -> str:
    name = " ".join(name.split())
    return name if len(name) <= width else name[:width - 3] + "..."


def _pct(v, q):
    return float(np.percentile(np.asarray(v, dtype=np.float64), q))


COPY_KERNEL = "__amd_rocclr_copyBuffer"
CALIB_BYTES = 256 << 20   # --calibrate-copy: the first CALIB_COPIES device copies of the run
CALIB_COPIES = 5


def summarize_counters(files, algorithmic_bytes=None):
    """Counter values per dispatch, averaged over the dispatches of each kernel of the
    library; derived utilisations (GRBM_GUI_ACTIVE, reported as the sum over the XCDs,
    divided by XCD_NUM is the kernel's cycle count); HBM traffic per call from FETCH_SIZE
    and WRITE_SIZE, each scaled by what the counter reads for the calibration copies of
    CALIB_BYTES (the first CALIB_COPIES device copies of each run: bench.py makes them
    before anything else)."""
    out = []
    vals = {}
    copies = {}
    for fi, c in enumerate(files):
        for r in _rows(c):
            name = _col(r, "Kernel_Name")
            cn = _col(r, "Counter_Name")
            cv = _col(r, "Counter_Value")
            did = _col(r, "Dispatch_Id", "Correlation_Id")
            grid = _col(r, "Grid_Size")
            if name is None or cn is None or cv is None:
                continue
            if COPY_KERNEL in name:
                copies.setdefault(cn, {}).setdefault(fi, {}).setdefault(int(did or 0), 0.0)
                copies[cn][fi][int(did or 0)] += float(cv)
                continue
            if "bitmm" not in name:
                continue
            key = (name, grid)
            vals.setdefault(key, {}).setdefault(cn, {}).setdefault((fi, did), 0.0)
            vals[key][cn][(fi, did)] += float(cv)
    scale = {}
    if copies:
        out.append(f"# calibration: the first {CALIB_COPIES} device copies of each run ({CALIB_BYTES >> 10} KiB each)")
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            if cn not in copies:
                continue
            first = []
            for fi, byd in copies[cn].items():
                first += [byd[d] for d in sorted(byd)[:CALIB_COPIES]]
            raw = float(np.mean(first))
            spread = (max(first) - min(first)) / raw if raw > 0 else float("inf")
            out.append(f"copy_{cn.lower()}_kib: {raw:.1f}")
            out.append(f"# spread over the calibration copies: {100 * spread:.2f} %")
            if raw > 0 and spread < 0.05:
                scale[cn] = CALIB_BYTES / 1024 / raw
                out.append(f"{cn.lower().replace('_size', '')}_scale: {scale[cn]:.5f}")
    out.append("# counters per dispatch, averaged over the dispatches of each kernel (grid in work-items)")
    main, main_g = None, -1.0
    traffic = 0.0
    have_traffic = {"FETCH_SIZE": False, "WRITE_SIZE": False}
    for (name, grid), cs in sorted(vals.items()):
        out.append(f"# kernel: {_short(name)} grid {grid}")
        avg = {cn: float(np.mean(list(v.values()))) for cn, v in cs.items()}
        out.append(f"# dispatches: {max(len(v) for v in cs.values())}")
        for cn, v in sorted(avg.items()):
            out.append(f"#   {cn}: {v:.1f}")
        g = avg.get("GRBM_GUI_ACTIVE")
        g = g / XCD_NUM if g else g
        derived = {}
        if g:
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                derived["MfmaUtil_pct"] = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * SIMD_NUM)
            if "SQ_ACTIVE_INST_VALU" in avg:
                derived["VALUBusy_pct"] = 100.0 * avg["SQ_ACTIVE_INST_VALU"] / CU_NUM / g
            if "SQ_WAVE_CYCLES" in avg:
                derived["OccupancyPercent"] = 400.0 * avg["SQ_WAVE_CYCLES"] / g / CU_NUM / 32
            if "SQ_LDS_BANK_CONFLICT" in avg:
                derived["LDSBankConflict_pct"] = 100.0 * avg["SQ_LDS_BANK_CONFLICT"] / g / CU_NUM
            if "TA_BUSY_avr" in avg:
                derived["TA_BUSY_avr_pct"] = 100.0 * avg["TA_BUSY_avr"] / g
        for k, v in derived.items():
            out.append(f"#   {k}: {v:.1f}")
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            if cn in avg and cn in scale:
                traffic += avg[cn] * scale[cn] * 1024
                have_traffic[cn] = True
        if g is not None and g > main_g:
            main, main_g = (name, derived), g
    if main is not None:
        out.append(f"# the longest kernel: {_short(main[0], 120)}")
        for k, v in main[1].items():
            out.append(f"{k}: {v:.1f}")
    if all(have_traffic.values()):
        out.append(f"traffic_bytes_per_launch: {traffic:.0f}")
        if algorithmic_bytes:
            out.append(f"algorithmic_bytes_per_launch: {algorithmic_bytes}")
            out.append(f"traffic_over_algorithmic: {traffic / algorithmic_bytes:.4f}")
    return out


def workload_bytes(bench_json: str, workload: str) -> int:
    """Algorithmic bytes per launch of `workload` in an untraced bench line."""
    with open(bench_json) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                j = json.loads(line)
                for e in j.get("suite", []) + j.get("per_kernel", []):
                    if e["workload"] == workload:
                        return int(e["bytes"])
    raise SystemExit(f"{workload}: not in {bench_json}")


def summarize_profile(d: str, bench_json: str | None, command: str | None,
                      algorithmic_bytes: int | None = None, title: str | None = None,
                      argv: list | None = None) -> str:
    """Text summary of the rocprofv3 CSV output under d (searched recursively)."""
    out = []
    src_hash = kernel_sources_hash()
    if title:
        out.append(f"# {title}")
    if argv:
        # how this text was made (the rocprofv3 command is the line below)
        shown, skip = [], False
        for a in argv:
            if skip:
                shown.append("CMD")
                skip = False
                continue
            shown.append(a if (a.replace("/", "").replace("_", "").replace("-", "").replace(".", "").isalnum())
                         else json.dumps(a))
            skip = a == "--command"
        out.append("# summarised by: python3 bench.py " + " ".join(shown))
    if command:
        out.append("# command (from the repository root on the MI355X host; cd /tmp && export TMPDIR=/tmp first):")
        out.append(f"#   {command}")
    out.append(f"kernel_sources_sha256_16: {src_hash}")
    traces = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    markers = sorted(glob.glob(os.path.join(d, "**", "*marker_api_trace.csv"), recursive=True))
    counters = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    disp = []
    for t in traces:
        for r in _rows(t):
            s, e = _col(r, "Start_Timestamp"), _col(r, "End_Timestamp")
            name = _col(r, "Kernel_Name")
            if s is None or e is None or name is None:
                continue
            grid = _col(r, "Grid_Size", "Grid_Size_X")
            disp.append((int(s), int(e), name, int(grid) if grid else 0))
    if disp:
        by = {}
        for s, e, name, grid in disp:
            by.setdefault(name, []).append(e - s)
        tot = sum(sum(v) for v in by.values())
        out.append("# kernels: calls, median ns, p10 ns, p90 ns, mean ns, share of GPU time, kernel")
        for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"# {len(v):6d} {np.median(v):11.1f} {_pct(v, 10):10.1f} {_pct(v, 90):10.1f} "
                       f"{np.mean(v):11.1f} {100.0 * sum(v) / tot:6.2f}%  {_short(name)}")
    ranges = []
    for m in markers:
        for r in _rows(m):
            msg = _col(r, "Message", "Function", "Name", "Marker_Message") or ""
            s, e = _col(r, "Start_Timestamp"), _col(r, "End_Timestamp")
            if "bitmm:" in msg and s is not None and e is not None:
                ranges.append((msg[msg.index("bitmm:") + 6:].strip(), int(s), int(e)))
    untraced = {}
    if bench_json and os.path.exists(bench_json):
        with open(bench_json) as f:
            for line in f:
                line = line.strip()
                if line.startswith("{"):
                    j = json.loads(line)
                    for e in j.get("suite", []) + j.get("per_kernel", []):
                        untraced[e["workload"]] = e["us_per_launch"]
    if ranges:
        out.append("# per workload (ROCTx range over its timed replays): kernel time per launch, "
                   "summed over the kernels of one call, against the bench's event time")
        if bench_json:
            out.append(f"# untraced event times from: {os.path.basename(bench_json)}")
        for wl, s0, e0 in ranges:
            ks = [(s, e, n) for s, e, n, _ in disp if s >= s0 and e <= e0 and "bitmm" in n]
            if not ks:
                continue
            names = {}
            for s, e, n in ks:
                names.setdefault(n, []).append(e - s)
            launches = max(len(v) for v in names.values())
            total = sum(e - s for s, e, _ in ks)
            per = total / launches / 1e3
            out.append(f"wl.{wl}.launches: {launches}")
            out.append(f"wl.{wl}.kernel_us_per_launch: {per:.3f}")
            for n, v in names.items():
                out.append(f"wl.{wl}.kernel: {_short(n, 110)} | median {np.median(v) / 1e3:.3f} us, "
                           f"p10 {_pct(v, 10) / 1e3:.3f}, p90 {_pct(v, 90) / 1e3:.3f}")
            if wl in untraced:
                out.append(f"wl.{wl}.untraced_events_us: {untraced[wl]}")
                out.append(f"wl.{wl}.kernel_share_of_untraced_pct: {100.0 * per / untraced[wl]:.1f}")
    if counters:
        out.extend(summarize_counters(counters, algorithmic_bytes))
    return "\n".join(out) + "\n"


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=3)
    ap.add_argument("--no-suite", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", default=None)
    ap.add_argument("--markers", action="store_true")
    ap.add_argument("--summarize", default=None, metavar="DIR")
    ap.add_argument("--bench-json", default=None)
    ap.add_argument("--command", default=None)
    ap.add_argument("--algorithmic-bytes", type=int, default=None)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--title", default=None)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device-to-device copy 5 times: the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.summarize:
        nbytes = args.algorithmic_bytes
        if args.workload:
            if not args.bench_json:
                raise SystemExit("--workload needs --bench-json")
            nbytes = workload_bytes(args.bench_json, args.workload)
        sys.stdout.write(summarize_profile(args.summarize, args.bench_json, args.command, nbytes,
                                           args.title, sys.argv[1:]))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_matmul_amd as bm
    from bit_matmul_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bm.lib()
    log(f"device: {torch.cuda.get_device_name(0)}")
    markers = Markers(args.markers)
    R = max(1, args.repeats)
    src_hash = kernel_sources_hash()
    only = [s for s in args.only.split(",") if s] if args.only else None

    result = {}
    if args.calibrate_copy:
        # first of all, so that these are the run's first device copies
        src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(CALIB_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = CALIB_BYTES
        del src, dst
        torch.cuda.empty_cache()
    ceilings = None
    pa = pb = None
    gpu_time = {}
    if only is None:
        if not args.no_ceilings:
            ceilings = measured_ceilings(torch)
        # ---- headline: decode GEMV at hidden 5120 ---------------------------
        t0 = time.perf_counter()
        pa = I.hidden5120(1, 5120, 4)
        pb = I.hidden5120(1, 13824, 4)
        log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
        ca = Case(torch, pa, "qmv", torch.bfloat16)
        cb = Case(torch, pb, "qmv", torch.bfloat16)
        reps = time_steps(torch, [ca, cb], args.steps, args.warmup, R)
        total, spread = stats(reps, 1)
        total /= 1e6
        step_bytes = ca.bytes + cb.bytes
        value = step_bytes * args.steps / total / 1e9
        log(f"headline: {args.steps} steps in {total * 1e3:.3f} ms (median of {R}) -> {value:.1f} GB/s")
        # Each kernel alone, same launch configuration, for the per-kernel roofline.
        ta, sa = stats(time_steps(torch, [ca], args.steps, args.warmup, R, markers, pa.name), args.steps)
        tb, sb = stats(time_steps(torch, [cb], args.steps, args.warmup, R, markers, pb.name), args.steps)
        kb = bm.bitmm_last_launches()
        ta, tb = ta / 1e6, tb / 1e6
        gpu_time[pa.name], gpu_time[pb.name] = ta, tb
        roofline = roofline_obj("hbm", cb.bytes, cb.flops, tb, ceilings)
        tr = read_summary("counters_qmv_M1_K5120_N13824_b4", src_hash)
        roofline.update({"traffic": int(num(tr, "traffic_bytes_per_launch")) if tr and num(tr, "traffic_bytes_per_launch") else None,
                         "kernel": "qmv_dma_kernel<4, 64, 3, 2> (K=5120, N=13824, 4-bit, M=1: two steps of "
                                   "1 row x 64 lanes x 3 chunks per wave)",
                         "algorithmic_bytes_per_launch": cb.bytes,
                         "avg_launch_us": round(tb * 1e6, 3), "spread_pct": sb["spread_pct"],
                         "launch": kb})
        result = {
            "metric": "qmv HBM GB/s (% of peak); qmm & MoE gather_qmm TFLOPS (% of MFMA peak)",
            "value": round(value, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(total / args.steps * 1e3, 6),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "decode qmv, hidden 5120: M=1, K=5120, N in {5120, 13824}, "
                                   "4-bit affine group 64, bf16 x/y, f32 accumulate",
                       "step": "one qmv at N=5120 + one at N=13824",
                       "hbm_frac": round(value / HBM_PEAK_GBS, 4),
                       "rotating_copies": ca.copies,
                       "repeats": R, "step_spread_pct": spread["spread_pct"],
                       "kernel_sources_sha256_16": src_hash},
            "roofline": roofline,
            "per_kernel": [summarize(ca, ta, pa.name, "hbm", sa, ceilings),
                           summarize(cb, tb, pb.name, "hbm", sb, ceilings)],
        }
        if ceilings:
            result["measured_ceilings"] = ceilings
        for e in result["per_kernel"]:
            attach_profiles(e, src_hash)
        del ca, cb
        torch.cuda.empty_cache()

    # ---- the rest of the hot path ------------------------------------------
    oracle_entries = []
    if not args.no_suite:
        suite = []
        names = suite_names()
        specs = suite_specs(I)
        if only is not None:
            # the headline's two GEMVs can be profiled on their own too
            names = list(HEADLINE) + names
            specs = [("qmv", lambda: I.hidden5120(1, 5120, 4), "hbm"),
                     ("qmv", lambda: I.hidden5120(1, 13824, 4), "hbm")] + specs
        for (kind, make, bound), name in zip(specs, names):
            if only is not None and not any(s in name for s in only):
                continue
            p = make()
            assert p.name == name, (p.name, name)
            c = Case(torch, p, kind, torch.bfloat16)
            steps = max(20, args.steps // 2)
            t1, sp = stats(time_steps(torch, [c], steps, max(5, args.warmup // 2), R, markers, p.name), steps)
            t1 /= 1e6
            gpu_time[p.name] = t1
            sp["kernels"] = bm.bitmm_last_launches()  # what the library enqueued for one call
            s = summarize(c, t1, p.name, bound, sp, ceilings)
            attach_profiles(s, src_hash)
            log(f"suite {p.name}: {s['us_per_launch']} us (spread {sp['spread_pct']} %), {s['GB_s']} GB/s, "
                f"{s['TFLOP_s']} TFLOP/s")
            suite.append(s)
            if only is None and not args.no_cpu:
                oracle_entries.append((p.name, p, kind, t1))
            del c
            torch.cuda.empty_cache()
        result["suite"] = suite
        # The 8-bit vs 4-bit controlled pair: 1.89x the bytes, and the time it takes.
        by = {e["workload"]: e for e in suite + result.get("per_kernel", [])}
        pairs = []
        for a4, a8 in (("qmv_M1_K5120_N5120_b4", "qmv_M1_K5120_N5120_b8"),
                       ("qmv_M1_K5120_N13824_b4", "qmv_M1_K5120_N13824_b8"),
                       ("qmm_M600_K5120_N13824_b4", "qmm_M600_K5120_N13824_b8"),
                       ("qmm_M3_K5120_N13824_b4", "qmm_M3_K5120_N13824_b8")):
            if a4 in by and a8 in by:
                pairs.append({"pair": f"{a8} vs {a4}",
                              "bytes_ratio": round(by[a8]["bytes"] / by[a4]["bytes"], 3),
                              "time_ratio": round(by[a8]["us_per_launch"] / by[a4]["us_per_launch"], 3)})
        if pairs:
            result["bits_8_vs_4"] = pairs

    if only is None and not args.no_cpu:
        import oracle
        threads = oracle.default_threads()
        result["cpu_baseline"] = cpu_baseline([pa, pb], args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']}")
        head = [("qmv_K512_N256_b4", I.tiny_qmv(), "qmv", None),
                (pa.name, pa, "qmv", gpu_time.get(pa.name)), (pb.name, pb, "qmv", gpu_time.get(pb.name))]
        result["cpu_baseline"]["per_config"] = oracle_per_config(head + oracle_entries, threads)
    elif only is None:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
