"""Benchmark of the NVFP4 matrix-vector path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass over a workload's whole weight set (default: the decode
GEMV, 64 distinct 4096x4096 NVFP4 matrices rotated, N=1), replayed as one HIP
graph, with weights and activations resident in HBM before timing starts.
Prints one JSON line: whole-job throughput in GB/s of algorithmic traffic
(compressed weights + activations + outputs), the roofline of the dominant
kernel from per-launch HIP events, and the fp64 CPU oracle timed on a bounded
sample of the same workload (which also re-checks those GPU outputs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import block_scaled_bit_nvfp4_amd as nv                       # noqa: E402
from block_scaled_bit_nvfp4_amd import workloads as wl        # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
DEV = "cuda:0"


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


# ------------------------------------------------------------------ set-up --

class Matrix:
    """A repacked NVFP4 (or MXFP4) matrix resident in HBM (quantised and
    repacked by the library from seeded fp32 weights; set-up, not timed)."""

    def __init__(self, workload, m, copy):
        W = wl.weights(m.rows, m.cols, seed=wl.seed_of(workload.name, m.name, copy),
                       outliers=workload.outliers, device=DEV)
        self.fmt = workload.fmt
        codes = torch.empty(m.rows, m.cols // 2, dtype=torch.uint8, device=DEV)
        if self.fmt == "mxfp4":
            scales = torch.empty(m.rows, m.cols // 32, dtype=torch.uint8, device=DEV)
            nv.mxfp4_quantize(W, m.rows, m.cols, workload.tscale, codes, scales)
            self.wq, self.ws = nv.alloc_mx_repacked(m.rows, m.cols, DEV)
            nv.mxfp4_repack(codes, scales, m.rows, m.cols, self.wq, self.ws)
        else:
            scales = torch.empty(m.rows, m.cols // 16, dtype=torch.uint8, device=DEV)
            nv.nvfp4_quantize(W, m.rows, m.cols, workload.tscale, codes, scales)
            self.wq, self.ws = nv.alloc_repacked(m.rows, m.cols, DEV)
            nv.nvfp4_repack(codes, scales, m.rows, m.cols, self.wq, self.ws)
        self.rows, self.cols, self.name, self.copy = m.rows, m.cols, m.name, copy
        self.tscale = workload.tscale

    def weight_bytes(self):
        return weight_bytes(self.rows, self.cols, self.fmt)

    def gemv(self, x, n, y):
        f = nv.mxfp4_gemv if self.fmt == "mxfp4" else nv.nvfp4_gemv
        f(self.wq, self.ws, self.tscale, self.rows, self.cols, x, n, y)


def weight_bytes(rows, cols, fmt="nvfp4"):
    """Code and scale bytes: 0.5625 B per element for NVFP4 (a scale per 16),
    0.53125 for MXFP4 (a scale per 32)."""
    return rows * cols * 17 // 32 if fmt == "mxfp4" else rows * cols * 9 // 16


def gemv_bytes(rows, cols, n, fmt="nvfp4"):
    """Algorithmic bytes of one product: weights + X + Y."""
    return weight_bytes(rows, cols, fmt) + n * cols * 2 + n * rows * 4


class Step:
    """The launches of one pass over a workload, with their algorithmic bytes."""

    def __init__(self, name, fused_mlp=True):
        self.w = wl.WORKLOADS[name]
        w = self.w
        self.n = w.n
        self.launches = []          # (callable, bytes, flops, kernel tag)
        t0 = time.time()
        if name == "decode_4096x4096":
            m = w.matrices[0]
            self.x = wl.activations(1, m.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.mats = [Matrix(w, m, c) for c in range(w.copies)]
            self.ys = [torch.empty(1, m.rows, dtype=torch.float32, device=DEV) for _ in range(2)]
            for i, M in enumerate(self.mats):
                y = self.ys[i % 2]
                self.launches.append((self._gemv(M, self.x, 1, y), gemv_bytes(M.rows, M.cols, 1),
                                      2 * M.rows * M.cols, "gemv"))
        elif name == "mlp_27b_decode":
            gu_m, dn_m = w.matrices
            self.x = wl.activations(1, gu_m.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.layers = [(Matrix(w, gu_m, c), Matrix(w, dn_m, c)) for c in range(w.copies)]
            F, Dh = dn_m.cols, gu_m.cols
            self.gu = torch.empty(1, gu_m.rows, dtype=torch.float32, device=DEV)
            self.h = torch.empty(1, F, dtype=torch.bfloat16, device=DEV)
            self.y = torch.empty(1, dn_m.rows, dtype=torch.float32, device=DEV)
            for G_, D in self.layers:
                if fused_mlp:
                    # gate||up with SwiGLU in the epilogue (writes h), then down
                    nbytes = G_.weight_bytes() + 2 * Dh + 2 * F
                    self.launches.append((self._gemv_swiglu(G_, Dh, F), nbytes, 2 * G_.rows * G_.cols, "gemv"))
                else:
                    self.launches.append((self._gemv(G_, self.x, 1, self.gu), gemv_bytes(G_.rows, G_.cols, 1),
                                          2 * G_.rows * G_.cols, "gemv"))
                    self.launches.append((self._swiglu(F), 1 * 2 * F * 4 + F * 2, 4 * F, "swiglu"))
                self.launches.append((self._gemv(D, self.h, 1, self.y), gemv_bytes(D.rows, D.cols, 1),
                                      2 * D.rows * D.cols, "gemv"))
        elif name in ("verify_vocab_n4", "verify_vocab_n8"):
            mw, head = w.matrices
            n = w.n
            self.x = wl.activations(n, mw.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.M1, self.M2 = Matrix(w, mw, 0), Matrix(w, head, 0)
            self.y1 = torch.empty(n, mw.rows, dtype=torch.float32, device=DEV)
            self.logits = torch.empty(n, head.rows, dtype=torch.float32, device=DEV)
            self.am = torch.empty(n, dtype=torch.int32, device=DEV)
            self.wsp = torch.empty(nv.nvfp4_gemv_argmax_workspace_bytes(head.rows, head.cols, n), dtype=torch.uint8,
                                   device=DEV)
            self.launches.append((self._gemv(self.M1, self.x, n, self.y1), gemv_bytes(mw.rows, mw.cols, n),
                                  2 * n * mw.rows * mw.cols, "gemv"))
            self.launches.append((self._argmax(), gemv_bytes(head.rows, head.cols, n) + 4 * n,
                                  2 * n * head.rows * head.cols, "gemv"))
        elif name == "draft_head_8192x4096":
            m = w.matrices[0]
            self.x = wl.activations(1, m.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.mats = [Matrix(w, m, c) for c in range(w.copies)]
            self.logits2 = [torch.empty(1, m.rows, dtype=torch.float32, device=DEV) for _ in range(2)]
            self.am2 = [torch.empty(1, dtype=torch.int32, device=DEV) for _ in range(2)]
            self.wsp = torch.empty(nv.nvfp4_gemv_argmax_workspace_bytes(m.rows, m.cols, 1), dtype=torch.uint8,
                                   device=DEV)
            for i, M in enumerate(self.mats):
                self.launches.append((self._argmax_of(M, self.logits2[i % 2], self.am2[i % 2]),
                                      gemv_bytes(M.rows, M.cols, 1) + 4, 2 * M.rows * M.cols, "gemv"))
        elif name == "mxfp4_gemv_17408x5120":
            m = w.matrices[0]
            self.x = wl.activations(1, m.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.mats = [Matrix(w, m, c) for c in range(w.copies)]
            self.ys = [torch.empty(1, m.rows, dtype=torch.float32, device=DEV) for _ in range(2)]
            for i, M in enumerate(self.mats):
                self.launches.append((self._gemv(M, self.x, 1, self.ys[i % 2]), gemv_bytes(M.rows, M.cols, 1, "mxfp4"),
                                      2 * M.rows * M.cols, "gemv"))
        elif name in ("prefill_n512", "mxfp4_prefill_n512"):
            m = w.matrices[0]
            self.x = wl.activations(512, m.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.mats = [Matrix(w, m, c) for c in range(w.copies)]
            self.M = self.mats[0]
            self.ys = [torch.empty(512, m.rows, dtype=torch.float32, device=DEV) for _ in range(2)]
            for i, M in enumerate(self.mats):
                self.launches.append((self._gemv(M, self.x, 512, self.ys[i % 2]),
                                      gemv_bytes(m.rows, m.cols, 512, w.fmt), 2 * 512 * m.rows * m.cols, "gemm"))
        else:
            raise SystemExit("unknown workload %r (choose from %s)" % (name, ", ".join(wl.WORKLOADS)))
        torch.cuda.synchronize()
        log("set-up of %s took %.1f s" % (name, time.time() - t0))
        self.bytes = sum(b for _, b, _, _ in self.launches)
        self.flops = sum(f for _, _, f, _ in self.launches)

    @staticmethod
    def _gemv(M, x, n, y):
        def f():
            M.gemv(x, n, y)
        return f

    def _gemv_swiglu(self, G_, Dh, F):
        def f():
            nv.nvfp4_gemv_swiglu(G_.wq, G_.ws, G_.tscale, Dh, F, self.x, 1, None, self.h)
        return f

    def _swiglu(self, F):
        def f():
            nv.nvfp4_swiglu(self.gu, F, 1, self.h)
        return f

    def _argmax(self):
        M = self.M2

        def f():
            nv.nvfp4_gemv_argmax(M.wq, M.ws, M.tscale, M.rows, M.cols, self.x, self.n, self.logits, self.am,
                                 self.wsp)
        return f

    def _argmax_of(self, M, logits, am):
        def f():
            nv.nvfp4_gemv_argmax(M.wq, M.ws, M.tscale, M.rows, M.cols, self.x, 1, logits, am, self.wsp)
        return f

    def run(self):
        for f, _, _, _ in self.launches:
            f()


# ------------------------------------------------------------------ timing --

def time_graph(step, steps, warmup):
    """Capture one step as a HIP graph, replay it `warmup` times, then time
    `steps` replays: host wall clock between two device synchronisations, and
    a HIP event pair on the replay stream around the same replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            step.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = e0.elapsed_time(e1) * 1e-3 / steps
    return wall, ev, g


# ------------------------------------------------------------ cpu baseline --

def cpu_baseline(step, budget_s=12.0, min_s=10.0):
    """The fp64 CPU oracle on a bounded sample of the workload's products,
    timed on this host; the same oracle outputs re-check the GPU outputs of
    the sample (computed here, eagerly, by the library).  Items are quantised
    by the oracle once (not timed); the oracle's products are timed, and the
    sample is passed over again until about min_s seconds of product time
    have run, so that small workloads are timed over a stable interval."""
    import oracle
    w = step.w
    sample = []
    if w.name == "decode_4096x4096":
        for M in step.mats:
            sample.append((M, step.x, None))
    elif w.name == "mlp_27b_decode":
        for G_, D in step.layers:
            sample.append((G_, step.x, None))
    elif w.name in ("verify_vocab_n4", "verify_vocab_n8"):
        sample.append((step.M1, step.x, None))
        sample.append((step.M2, step.x, np.arange(0, step.M2.rows, 8)))
    elif w.name in ("prefill_n512", "mxfp4_prefill_n512"):
        sample.append((step.M, step.x, np.arange(0, step.M.rows, 256)))
    elif w.name == "mxfp4_gemv_17408x5120":
        for M in step.mats:
            sample.append((M, step.x, None))
    elif w.name == "draft_head_8192x4096":
        for M in step.mats:
            sample.append((M, step.x, None))
    gemv = oracle.mx_gemv if w.fmt == "mxfp4" else oracle.gemv
    xb_cache, prepared = {}, []
    t_total, bytes_done, checked, worst, outputs = 0.0, 0, 0, 0.0, 0
    for M, x, rows in sample:
        if t_total >= budget_s:
            break
        Wf = wl.weights(M.rows, M.cols, seed=wl.seed_of(w.name, M.name, M.copy), outliers=w.outliers, device=DEV)
        rsel = np.arange(M.rows) if rows is None else rows
        Wh = Wf[torch.as_tensor(rsel, device=DEV)].cpu().numpy()
        del Wf
        quantize = oracle.mx_quantize if w.fmt == "mxfp4" else oracle.quantize
        codes, scales = quantize(Wh, w.tscale)
        del Wh
        key = id(x)
        if key not in xb_cache:
            xb_cache[key] = wl.bf16_bits(x)
        xb = xb_cache[key]
        n = x.shape[0]
        t0 = time.perf_counter()
        Y_ref, S = gemv(codes, scales, w.tscale, xb)
        t_total += time.perf_counter() - t0
        nbytes = gemv_bytes(len(rsel), M.cols, n, w.fmt)
        bytes_done += nbytes
        outputs += Y_ref.size
        y = torch.empty(n, M.rows, dtype=torch.float32, device=DEV)
        M.gemv(x, n, y)
        yg = y.cpu().numpy()[:, rsel].astype(np.float64)
        err = np.abs(yg - Y_ref) / (1e-5 * S + 1e-6)
        worst = max(worst, float(err.max()))
        checked += err.size
        prepared.append((codes, scales, xb, nbytes, Y_ref.size))
    passes, first_outputs = 1, outputs
    while t_total < min_s and prepared:
        for codes, scales, xb, nbytes, nout in prepared:
            t0 = time.perf_counter()
            gemv(codes, scales, w.tscale, xb)
            t_total += time.perf_counter() - t0
            bytes_done += nbytes
            outputs += nout
            if t_total >= budget_s:
                break
        passes += 1
    value = bytes_done / t_total / 1e9
    return {
        "value": round(value, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
        "sample": "%d outputs of %s (%d per pass over the sample, %d passes; %.1f MB of algorithmic "
                  "traffic) in %.2f s of oracle products" % (outputs, w.name, first_outputs, passes,
                                                              bytes_done / 1e6, t_total),
        "parity": {"outputs": checked, "max_err_over_tolerance": worst, "pass": bool(worst <= 1.0)},
    }


# ---------------------------------------------------------------- traffic --

def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_bit_nvfp4_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, variant=None):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if absent, taken on different kernel sources, or taken
    on another variant of the step (the counters were collected on the
    default one)."""
    if variant:
        return None
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


# ------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_4096x4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mlp-three-launches", action="store_true",
                    help="run the decode MLP as gate||up matvec, SwiGLU and down matvec (three launches "
                         "per layer) instead of gate||up with SwiGLU fused, then down (two launches)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (read + write), e.g. to "
                         "calibrate HBM traffic counters against a known byte count")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the NVFP4 matvec path runs on a single MI355X "
              "(row sharding across GPUs is a design note, not built); rerun with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=DEV)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes, "launches": 5}))
        return
    nv.load()
    step = Step(args.workload, fused_mlp=not args.mlp_three_launches)
    step.run()
    torch.cuda.synchronize()

    step_s, step_ev_s, graph = time_graph(step, args.steps, args.warmup)
    # Dominant kernel: the products.  Where a step holds only product launches
    # (the decode rotation, the prefill contraction) the event time per step
    # divided by the launches is the average launch duration; otherwise the
    # figure covers the whole step and says so.
    tags = {t for _, _, _, t in step.launches}
    kernel = "gemm" if args.workload in ("prefill_n512", "mxfp4_prefill_n512") else "gemv"
    n_launch = sum(1 for _, _, _, t in step.launches if t == kernel)
    per_launch_s = step_ev_s / n_launch
    if args.workload == "draft_head_8192x4096":
        scope = ("average call: the product with per-workgroup argmax keys plus the one-workgroup argmax "
                 "finish (HIP events around %d graph replays of %d calls)" % (args.steps, n_launch))
    elif tags == {kernel}:
        scope = "average launch of the %s kernel (HIP events around %d graph replays of %d launches)" % (
            kernel, args.steps, n_launch)
    else:
        scope = "whole step, %s launches plus %s (HIP events around %d graph replays)" % (
            kernel, "/".join(sorted(tags - {kernel})) or "-", args.steps)
    per_launch_bytes = step.bytes / n_launch
    if kernel == "gemm":
        achieved = step.flops / n_launch / per_launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(args.workload)}
    else:
        achieved = per_launch_bytes / per_launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(args.workload, "three launches" if args.mlp_three_launches else None)}
    roof["kernel_avg_us"] = round(per_launch_s * 1e6, 3)
    roof["scope"] = scope

    value = step.bytes / step_s / 1e9
    w = step.w
    result = {
        "metric": "NVFP4 GEMV achieved HBM GB/s (% of peak) at N=1 and N=4; layer-tokens/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights with 0.1% 8-sigma outliers, bf16 N(0,1) activations)",
        "config": {
            "workload": w.name, "description": w.description, "n": w.n,
            "matrices": ["%dx%d" % (m.rows, m.cols) for m in w.matrices], "copies": w.copies,
            "bytes_per_step": step.bytes, "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "layer_tokens_per_s": round(w.copies * w.n / step_s, 1),
            "timing": "one HIP graph replay per step",
            "mlp": ("three launches per layer" if args.mlp_three_launches else
                    "two launches per layer (gate||up with SwiGLU fused, down)")
            if args.workload == "mlp_27b_decode" else None,
        },
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(step)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
