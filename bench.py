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

Timing: after W eager warm-up steps, the K timed steps are captured into one
HIP graph and replayed between two HIP events on the stream the kernels run on
(torch's current stream), so host-side launch cost is excluded. ``roofline`` is
for the dominant kernel (the N = 13824 GEMV), timed the same way on its own.

Also reported: ``cpu_baseline``, the CPU oracle timed on the host cores on a
bounded sample of the same workload, and ``suite``, every other workload of the
hot path (the 8-bit GEMV, the prefill GEMM at M = 600 and M = 3, 4- and 8-bit,
the MoE expert-gathered GEMM in both orientations, sorted and in routing order through
the indexed entry point, also at a 46-token prompt below the grouped path's gate, the
MoE decode step's gathered GEMV at 1 and 4 tokens in both orientations, and the dense
grouped product of a non-quantized MoE layer, bf16, both orientations and both weight
layouts, and the format variants: the decode GEMV with 2-bit codes and with groups of
128, the prefill GEMM with groups of 32), timed the same way.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-suite] [--no-cpu]
                       [--calibrate-copy]
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
ROTATE_BYTES = 1 << 30


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


def read_traffic(name: str, src_hash: str):
    """HBM bytes per launch from a committed counter summary (profiles/<name>.txt),
    valid only while the kernel sources are the ones it was measured on."""
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
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


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


def time_steps(torch, cases, steps, warmup):
    """Time `steps` steps (each launches every case once, in order) after `warmup`
    eager steps. The timed launches are captured into one HIP graph and replayed
    between two events on the stream they run on, so the host's per-launch cost
    (Python argument marshalling) is not part of the measurement. Returns seconds."""
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
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / 1e3


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


def summarize(case, secs_per_launch, name):
    t = secs_per_launch
    return {"workload": name, "us_per_launch": round(t * 1e6, 3),
            "GB_s": round(case.bytes / t / 1e9, 1),
            "hbm_frac": round(case.bytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOP_s": round(case.flops / t / 1e12, 2),
            "mfma_frac": round(case.flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "bytes": case.bytes, "flops": case.flops, "copies": case.copies}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-suite", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device-to-device copy 5 times: the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
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

    # ---- headline: decode GEMV at hidden 5120 -------------------------------
    t0 = time.perf_counter()
    pa = I.hidden5120(1, 5120, 4)
    pb = I.hidden5120(1, 13824, 4)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    ca = Case(torch, pa, "qmv", torch.bfloat16)
    cb = Case(torch, pb, "qmv", torch.bfloat16)
    total = time_steps(torch, [ca, cb], args.steps, args.warmup)
    step_bytes = ca.bytes + cb.bytes
    value = step_bytes * args.steps / total / 1e9
    log(f"headline: {args.steps} steps in {total * 1e3:.3f} ms -> {value:.1f} GB/s")
    # Each kernel alone, same launch configuration, for the per-kernel roofline.
    ta = time_steps(torch, [ca], args.steps, args.warmup) / args.steps
    tb = time_steps(torch, [cb], args.steps, args.warmup) / args.steps

    src_hash = kernel_sources_hash()
    achieved = cb.bytes / tb / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic("qmv_K5120_N13824_b4_traffic", src_hash),
                "kernel": "qmv_dma_kernel<4, 64, 3, 1> (K=5120, N=13824, 4-bit, M=1: one step of "
                          "1 row x 64 lanes x 3 chunks per wave)",
                "algorithmic_bytes_per_launch": cb.bytes,
                "avg_launch_us": round(tb * 1e6, 3)}

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
                   "kernel_sources_sha256_16": src_hash},
        "roofline": roofline,
        "per_kernel": [summarize(ca, ta, pa.name), summarize(cb, tb, pb.name)],
    }
    del ca, cb
    torch.cuda.empty_cache()

    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = n
        del src, dst
        torch.cuda.empty_cache()

    # ---- the rest of the hot path ------------------------------------------
    if not args.no_suite:
        suite = []
        specs = [("qmv", lambda: I.hidden5120(1, 5120, 8)), ("qmv", lambda: I.hidden5120(1, 13824, 8)),
                 ("qmm", lambda: I.hidden5120(600, 13824, 4)), ("qmm", lambda: I.hidden5120(3, 13824, 4)),
                 ("qmm", lambda: I.hidden5120(600, 13824, 8)), ("qmm", lambda: I.hidden5120(3, 13824, 8)),
                 ("gather", lambda: I.moe_gather("up")), ("gather", lambda: I.moe_gather("down")),
                 ("gather_indexed", lambda: I.moe_prefill_indexed("up")),
                 ("gather_indexed", lambda: I.moe_prefill_indexed("down")),
                 ("gather_qmv", lambda: I.moe_decode("up", 1)), ("gather_qmv", lambda: I.moe_decode("down", 1)),
                 ("gather_qmv", lambda: I.moe_decode("up", 4)), ("gather_qmv", lambda: I.moe_decode("down", 4)),
                 ("gather_indexed", lambda: I.moe_prefill_indexed("up", tokens=46)),
                 ("gather_indexed", lambda: I.moe_prefill_indexed("down", tokens=46)),
                 ("gather_mm", lambda: I.moe_gather_mm("up")), ("gather_mm", lambda: I.moe_gather_mm("down")),
                 ("gather_mm", lambda: I.moe_gather_mm("up", layout="kn")),
                 ("qmv", lambda: I.random_dense(1, 13824, 5120, 2, seed=1)),
                 # 13952 rows rather than 13824: a grid of its own in kernel traces
                 ("qmv", lambda: I.random_dense(1, 13952, 5120, 4, seed=1, group=128)),
                 ("qmm", lambda: I.random_dense(600, 13824, 5120, 4, seed=1, group=32))]
        for kind, make in specs:
            p = make()
            c = Case(torch, p, kind, torch.bfloat16)
            steps = max(20, args.steps // 2)
            t1 = time_steps(torch, [c], steps, max(5, args.warmup // 2)) / steps
            s = summarize(c, t1, p.name)
            log(f"suite {p.name}: {s['us_per_launch']} us, {s['GB_s']} GB/s, {s['TFLOP_s']} TFLOP/s")
            suite.append(s)
            del c
            torch.cuda.empty_cache()
        result["suite"] = suite

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline([pa, pb], args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']}")
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
