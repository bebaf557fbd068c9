"""Benchmark of the NVFP4 matrix-vector path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|NAME] [--no-cpu-baseline]

By default every configuration the metric is quoted on is measured, in one
process:

    C1 gemv_256x512         single 256x512 matvec, N=1 (latency-bound; parity case)
    C2 decode_4096x4096     decode GEMV, 64 distinct 4096x4096 matrices rotated, N=1
    C3 mlp_27b_decode       gate||up 34816x5120 + SwiGLU, down 5120x17408, 8 layers rotated, N=1
    C4 verify_vocab_n4      17408x5120 and a 151936x5120 vocabulary head with argmax in one
                            launch (nvfp4_gemv_batch), N=4
    C5 prefill_n512         17408x5120 at N=512 on MFMA, 4 layer copies rotated

A step is one pass over a configuration's whole weight set, replayed as one
HIP graph, with weights and activations resident in HBM before timing
starts.  The JSON line's top-level `value` is C2's whole-step throughput in
GB/s of algorithmic traffic (compressed weights + activations + outputs);
`configs` holds each configuration's step time, throughput, layer-tokens/s,
per-kernel times, its dominant kernel's roofline, the plain-read (or bare
MFMA) wall measured in the same process at the same byte counts and launch
counts, with, for the matvec configurations, a read-then-store-the-outputs
wall beside it, and the fp64 CPU oracle timed on a bounded sample of the same
workload on this host (which also re-checks those GPU outputs).
"""
from __future__ import annotations

import argparse
import ctypes
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
METRIC = "NVFP4 GEMV achieved HBM GB/s (% of peak) at N=1 and N=4; layer-tokens/s"

# The configurations the metric is quoted on, in order; C2 carries `value`.
CONFIGS = [("C1", "gemv_256x512"), ("C2", "decode_4096x4096"), ("C3", "mlp_27b_decode"),
           ("C4", "verify_vocab_n4"), ("C5", "prefill_n512")]
HEADLINE = "decode_4096x4096"
MFMA_WORKLOADS = ("prefill_n512", "mxfp4_prefill_n512")


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


class Launch:
    """One call of the step: the callable, its algorithmic bytes and FLOPs,
    the kernel it is timed as, the distinct weight set it reads, and how many
    of its bytes are outputs it writes."""

    def __init__(self, fn, nbytes, flops, kernel, weight_key, out_bytes=0):
        self.fn, self.bytes, self.flops, self.kernel, self.weight_key = fn, nbytes, flops, kernel, weight_key
        self.out_bytes = out_bytes


class Step:
    """The launches of one pass over a workload."""

    def __init__(self, name, fused_mlp=True):
        if name not in wl.WORKLOADS:
            raise SystemExit("unknown workload %r (choose from all, %s)" % (name, ", ".join(wl.WORKLOADS)))
        self.w = w = wl.WORKLOADS[name]
        self.n = w.n
        self.launches = []
        t0 = time.time()
        if name in ("gemv_256x512", "decode_4096x4096", "mxfp4_gemv_17408x5120"):
            m = w.matrices[0]
            self.x = wl.activations(1, m.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.mats = [Matrix(w, m, c) for c in range(w.copies)]
            self.ys = [torch.empty(1, m.rows, dtype=torch.float32, device=DEV) for _ in range(2)]
            for i, M in enumerate(self.mats):
                self.launches.append(Launch(self._gemv(M, self.x, 1, self.ys[i % 2]),
                                            gemv_bytes(M.rows, M.cols, 1, w.fmt), 2 * M.rows * M.cols,
                                            "matvec %dx%d" % (M.rows, M.cols), (M.name, i), 4 * M.rows))
        elif name == "mlp_27b_decode":
            gu_m, dn_m = w.matrices
            self.x = wl.activations(1, gu_m.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.layers = [(Matrix(w, gu_m, c), Matrix(w, dn_m, c)) for c in range(w.copies)]
            F, Dh = dn_m.cols, gu_m.cols
            self.gu = torch.empty(1, gu_m.rows, dtype=torch.float32, device=DEV)
            self.h = torch.empty(1, F, dtype=torch.bfloat16, device=DEV)
            self.y = torch.empty(1, dn_m.rows, dtype=torch.float32, device=DEV)
            for i, (G_, D) in enumerate(self.layers):
                if fused_mlp:
                    # gate||up with SwiGLU in the epilogue (writes h), then down
                    self.launches.append(Launch(self._gemv_swiglu(G_, Dh, F), G_.weight_bytes() + 2 * Dh + 2 * F,
                                                2 * G_.rows * G_.cols, "gate||up+SwiGLU %dx%d" % (G_.rows, G_.cols),
                                                ("gate_up", i), 2 * F))
                else:
                    self.launches.append(Launch(self._gemv(G_, self.x, 1, self.gu), gemv_bytes(G_.rows, G_.cols, 1),
                                                2 * G_.rows * G_.cols, "gate||up %dx%d" % (G_.rows, G_.cols),
                                                ("gate_up", i), 4 * G_.rows))
                    self.launches.append(Launch(self._swiglu(F), 2 * F * 4 + F * 2, 4 * F, "SwiGLU", None))
                self.launches.append(Launch(self._gemv(D, self.h, 1, self.y), gemv_bytes(D.rows, D.cols, 1),
                                            2 * D.rows * D.cols, "down %dx%d" % (D.rows, D.cols), ("down", i),
                                            4 * D.rows))
        elif name in ("verify_vocab_n4", "verify_vocab_n8"):
            mw, head = w.matrices
            n = w.n
            self.x = wl.activations(n, mw.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.M1, self.M2 = Matrix(w, mw, 0), Matrix(w, head, 0)
            self.y1 = torch.empty(n, mw.rows, dtype=torch.float32, device=DEV)
            self.logits = torch.empty(n, head.rows, dtype=torch.float32, device=DEV)
            self.am = torch.empty(n, dtype=torch.int32, device=DEV)
            # both products in one launch of the matvec, then the head's
            # argmax finish (nvfp4_gemv_batch)
            self.prods = [dict(wq=self.M2.wq, ws=self.M2.ws, tscale=self.M2.tscale, rows=head.rows, y=self.logits,
                               argmax=self.am),
                          dict(wq=self.M1.wq, ws=self.M1.ws, tscale=self.M1.tscale, rows=mw.rows, y=self.y1)]
            self.wsp = torch.empty(max(8, nv.nvfp4_gemv_batch_workspace_bytes(self.prods, mw.cols, n)),
                                   dtype=torch.uint8, device=DEV)
            self.launches.append(Launch(self._verify_batch(mw.cols),
                                        gemv_bytes(mw.rows, mw.cols, n) + gemv_bytes(head.rows, head.cols, n)
                                        - n * mw.cols * 2 + 4 * n,
                                        2 * n * (mw.rows + head.rows) * mw.cols,
                                        "matvec+argmax batch %dx%d, %dx%d" % (head.rows, head.cols, mw.rows, mw.cols),
                                        ("w+lm_head", 0), 4 * n * (mw.rows + head.rows) + 4 * n))
        elif name == "draft_head_8192x4096":
            m = w.matrices[0]
            self.x = wl.activations(1, m.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.mats = [Matrix(w, m, c) for c in range(w.copies)]
            self.logits2 = [torch.empty(1, m.rows, dtype=torch.float32, device=DEV) for _ in range(2)]
            self.am2 = [torch.empty(1, dtype=torch.int32, device=DEV) for _ in range(2)]
            self.wsp = torch.empty(nv.nvfp4_gemv_argmax_workspace_bytes(m.rows, m.cols, 1), dtype=torch.uint8,
                                   device=DEV)
            for i, M in enumerate(self.mats):
                self.launches.append(Launch(self._argmax(M, self.logits2[i % 2], self.am2[i % 2]),
                                            gemv_bytes(M.rows, M.cols, 1) + 4, 2 * M.rows * M.cols,
                                            "matvec+argmax %dx%d" % (M.rows, M.cols), (M.name, i), 4 * M.rows + 4))
        elif name in MFMA_WORKLOADS:
            m = w.matrices[0]
            self.x = wl.activations(512, m.cols, seed=wl.seed_of(name, "x"), device=DEV)
            self.mats = [Matrix(w, m, c) for c in range(w.copies)]
            self.M = self.mats[0]
            self.ys = [torch.empty(512, m.rows, dtype=torch.float32, device=DEV) for _ in range(2)]
            for i, M in enumerate(self.mats):
                self.launches.append(Launch(self._gemv(M, self.x, 512, self.ys[i % 2]),
                                            gemv_bytes(m.rows, m.cols, 512, w.fmt), 2 * 512 * m.rows * m.cols,
                                            "wide %dx%d n=512" % (m.rows, m.cols), (M.name, i), 4 * 512 * m.rows))
        else:
            raise SystemExit("workload %r has no bench step" % name)
        torch.cuda.synchronize()
        log("set-up of %s took %.1f s" % (name, time.time() - t0))
        self.bytes = sum(L.bytes for L in self.launches)
        self.flops = sum(L.flops for L in self.launches)

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

    def _argmax(self, M, logits, am):
        def f():
            nv.nvfp4_gemv_argmax(M.wq, M.ws, M.tscale, M.rows, M.cols, self.x, self.n, logits, am, self.wsp)
        return f

    def _verify_batch(self, cols):
        def f():
            nv.nvfp4_gemv_batch(self.prods, cols, self.x, self.n, self.wsp)
        return f

    def run(self, kernels=None):
        for L in self.launches:
            if kernels is None or L.kernel in kernels:
                L.fn()


# ------------------------------------------------------------------ timing --

def time_graph(run, steps, warmup, per_graph=1):
    """Capture `per_graph` calls of run() (consecutive steps) as one HIP
    graph, replay it for `warmup` steps, then time `steps` steps
    (steps / per_graph replays): host wall clock between two device
    synchronisations, and a HIP event pair recorded on the replay stream
    around the same replays.  Returns (wall s, event s) per step."""
    assert steps % per_graph == 0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            run()
    for _ in range(max(1, warmup // per_graph)):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps // per_graph):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = e0.elapsed_time(e1) * 1e-3 / steps
    del g
    return wall, ev


# Steps per graph replay.  A replay costs about 10 us of launch before its
# first kernel (the 256 x 512 case measures it), which a whole-model decode
# graph pays once per token over hundreds of launches.  Steps of only a few
# launches therefore go several to a replay, which charges that cost to all
# of them; this repeats no cached work: the 256 x 512 case is
# cache-resident anyway, and every verify step streams the 440 MB
# vocabulary head, which evicts the previous step's bytes from the 256 MB
# Infinity Cache.  The other workloads have 4 to 64 launches per step.
STEP_BATCH = {"gemv_256x512": 16, "verify_vocab_n4": 4, "verify_vocab_n8": 4}
INFINITY_CACHE = 256 << 20


def steps_per_graph(name, steps):
    cap = STEP_BATCH.get(name, 1)
    return max(d for d in range(1, cap + 1) if steps % d == 0)


def kernel_times(step, steps, warmup, per_graph):
    """Per kernel of the step: a graph of only that kernel's launches (in step
    order), timed like the step; us per launch (per call for the argmax,
    whose call is the product plus its finish launch).  Several steps go to a
    replay as for the step itself, except where the kernel's own weights
    would fit the Infinity Cache and a repeat would read them from there."""
    out = []
    for k in dict.fromkeys(L.kernel for L in step.launches):
        ls = [L for L in step.launches if L.kernel == k]
        distinct = sum({L.weight_key: L.bytes for L in ls if L.weight_key is not None}.values())
        pg = per_graph if (distinct > INFINITY_CACHE or step.w.name == "gemv_256x512") else 1
        _, ev = time_graph(lambda: step.run({k}), steps, warmup, pg)
        per = ev / len(ls)
        e = {"kernel": k, "launches_per_step": len(ls), "us_per_launch": round(per * 1e6, 3),
             "steps_per_replay": pg}
        nb, fl = ls[0].bytes, ls[0].flops
        if step.w.name in MFMA_WORKLOADS:
            e["tflops"] = round(fl / per / 1e12, 2)
            e["pct_of_bf16_peak"] = round(100 * fl / per / 1e12 / BF16_PEAK_TFLOPS, 2)
        else:
            e["gbs"] = round(nb / per / 1e9, 1)
            e["pct_of_hbm_peak"] = round(100 * nb / per / 1e9 / HBM_PEAK_GBS, 2)
        out.append(e)
    return out


# ------------------------------------------------------------ measured walls --

class Probe:
    """libnvfp4_probe: the plain streaming read and the bare MFMA loop that
    give the measured walls (a measurement aid beside the product library)."""

    def __init__(self):
        path = os.path.join(ROOT, "block_scaled_bit_nvfp4_amd", "libnvfp4_probe.so")
        if not os.path.exists(path):
            raise RuntimeError("libnvfp4_probe.so is not built; run `python -m block_scaled_bit_nvfp4_amd.build`")
        lib = ctypes.CDLL(path)
        lib.nvfp4_probe_stream_read.restype = ctypes.c_int
        lib.nvfp4_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                                ctypes.c_void_p]
        lib.nvfp4_probe_stream_read_store.restype = ctypes.c_int
        lib.nvfp4_probe_stream_read_store.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                      ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
        lib.nvfp4_probe_mfma_bf16.restype = ctypes.c_int
        lib.nvfp4_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                              ctypes.c_void_p]
        self.lib = lib
        self.sink = torch.zeros(64, dtype=torch.int32, device=DEV)

    def read(self, buf, nbytes, groups):
        st = self.lib.nvfp4_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, groups,
                                              ctypes.c_void_p(self.sink.data_ptr()),
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st:
            raise RuntimeError("stream-read probe failed: %s" % nv.nvfp4_strerror(st))

    def read_store(self, buf, rbytes, out, obytes, groups):
        st = self.lib.nvfp4_probe_stream_read_store(ctypes.c_void_p(buf.data_ptr()), rbytes,
                                                    ctypes.c_void_p(out.data_ptr()), obytes, groups,
                                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st:
            raise RuntimeError("stream-read-store probe failed: %s" % nv.nvfp4_strerror(st))

    def mfma(self, groups, waves, iters):
        st = self.lib.nvfp4_probe_mfma_bf16(groups, waves, iters, ctypes.c_void_p(self.sink.data_ptr()),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st:
            raise RuntimeError("MFMA probe failed: %s" % nv.nvfp4_strerror(st))


READ_GROUPS = (256, 512, 1024, 2048, 4096, 8192)


def read_wall(probe, step, steps, warmup, per_graph):
    """The plain-read wall of a step: one streaming read per product launch,
    of that launch's algorithmic bytes, each distinct weight set with its own
    buffer (so the working set matches), in step order in one HIP graph.
    The read's grid is swept per launch size and the fastest kept.  Beside
    it, the read-and-store wall: each launch reads its input bytes and then
    writes its output bytes (rounded up to 16) from every workgroup after
    its reads, as a product writes its outputs after its sums."""
    reads = [L for L in step.launches if L.weight_key is not None]
    bufs = {}
    for L in reads:
        if L.weight_key not in bufs:
            bufs[L.weight_key] = torch.empty(L.bytes, dtype=torch.uint8, device=DEV).fill_(0x5A)
    obytes = {id(L): (L.out_bytes + 15) // 16 * 16 for L in reads}
    outs = [torch.empty(max(16, max(obytes.values())), dtype=torch.uint8, device=DEV) for _ in range(2)]

    def sweep(one):
        best = {}
        for size in sorted({L.bytes for L in reads}):
            same = [L for L in reads if L.bytes == size]
            t = {}
            for g in READ_GROUPS:
                _, t[g] = time_graph(lambda: [one(L, i, g) for i, L in enumerate(same)], 10, 2)
            best[size] = min(t, key=t.get)
        return best

    def plain(L, i, g):
        probe.read(bufs[L.weight_key], L.bytes, g)

    def with_store(L, i, g):
        probe.read_store(bufs[L.weight_key], L.bytes - L.out_bytes, outs[i % 2], obytes[id(L)], g)

    best = sweep(plain)
    _, ev = time_graph(lambda: [plain(L, i, best[L.bytes]) for i, L in enumerate(reads)],
                       steps, warmup, per_graph)
    best_s = sweep(with_store)
    _, ev_s = time_graph(lambda: [with_store(L, i, best_s[L.bytes]) for i, L in enumerate(reads)],
                         steps, warmup, per_graph)
    nbytes = sum(L.bytes for L in reads)
    del bufs, outs
    return {"kind": "plain read", "us_per_step": round(ev * 1e6, 3), "gbs": round(nbytes / ev / 1e9, 1),
            "launches_per_step": len(reads), "bytes_per_step": nbytes, "steps_per_replay": per_graph,
            "groups": {str(s): g for s, g in best.items()},
            "how": "one nontemporal 128-bit streaming read per product launch, of that launch's algorithmic "
                   "bytes, the grid (256-thread workgroups) swept per size, in one HIP graph",
            "read_store": {"us_per_step": round(ev_s * 1e6, 3), "gbs": round(nbytes / ev_s / 1e9, 1),
                           "groups": {str(s): g for s, g in best_s.items()},
                           "how": "the same launches reading their input bytes, then each workgroup storing "
                                  "its share of the launch's output bytes with 128-bit stores after its reads"}}


def mfma_wall(probe):
    """The bare bf16 MFMA loop's best rate over a few launch shapes."""
    best = 0.0
    for groups, waves in ((256, 4), (256, 8), (512, 8), (256, 16)):
        iters = 400
        fl = groups * waves * iters * 8 * 16384
        _, ev = time_graph(lambda: probe.mfma(groups, waves, iters), 5, 1)
        best = max(best, fl / ev / 1e12)
    return {"kind": "bare MFMA loop", "tflops": round(best, 1),
            "how": "v_mfma_f32_16x16x32_bf16, eight independent chains per wave, best of four launch shapes"}


# ------------------------------------------------------------ cpu baseline --

def host_facts():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_baseline(step, budget_s=12.0, min_s=8.0):
    """The fp64 CPU oracle on a bounded sample of the workload's products,
    timed on this host; the same oracle outputs re-check the GPU outputs of
    the sample (computed here, eagerly, by the library).  Items are quantised
    by the oracle once (not timed); the oracle's products are timed, and the
    sample is passed over again until about min_s seconds of product time
    have run, so that small workloads are timed over a stable interval."""
    import oracle
    w = step.w
    sample = []
    if w.name in ("gemv_256x512", "decode_4096x4096", "mxfp4_gemv_17408x5120", "draft_head_8192x4096"):
        for M in step.mats:
            sample.append((M, step.x, None, None))
    elif w.name == "mlp_27b_decode":
        for G_, D in step.layers:
            sample.append((G_, step.x, None, None))
    elif w.name in ("verify_vocab_n4", "verify_vocab_n8"):
        # the step's own outputs (both products of its one batched launch)
        step.run()
        torch.cuda.synchronize()
        sample.append((step.M1, step.x, None, step.y1.cpu().numpy()))
        sample.append((step.M2, step.x, np.arange(0, step.M2.rows, 8), step.logits.cpu().numpy()))
    elif w.name in MFMA_WORKLOADS:
        sample.append((step.M, step.x, np.arange(0, step.M.rows, 256), None))
    gemv = oracle.mx_gemv if w.fmt == "mxfp4" else oracle.gemv
    xb_cache, prepared = {}, []
    t_total, bytes_done, flops_done, checked, worst, outputs = 0.0, 0, 0, 0, 0.0, 0
    for M, x, rows, out in sample:
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
        flops_done += 2 * n * len(rsel) * M.cols
        outputs += Y_ref.size
        if out is None:
            y = torch.empty(n, M.rows, dtype=torch.float32, device=DEV)
            M.gemv(x, n, y)
            out = y.cpu().numpy()
        yg = out[:, rsel].astype(np.float64)
        err = np.abs(yg - Y_ref) / (1e-5 * S + 1e-6)
        worst = max(worst, float(err.max()))
        checked += err.size
        prepared.append((codes, scales, xb, nbytes, 2 * n * len(rsel) * M.cols, Y_ref.size))
    passes, first_outputs = 1, outputs
    while t_total < min_s and prepared:
        for codes, scales, xb, nbytes, fl, nout in prepared:
            t0 = time.perf_counter()
            gemv(codes, scales, w.tscale, xb)
            t_total += time.perf_counter() - t0
            bytes_done += nbytes
            flops_done += fl
            outputs += nout
            if t_total >= budget_s:
                break
        passes += 1
    gbs = bytes_done / t_total / 1e9
    out = {
        "value": round(gbs, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
        "sample": "%d outputs of %s (%d per pass over the sample, %d passes; %.1f MB of algorithmic "
                  "traffic) in %.2f s of oracle products" % (outputs, w.name, first_outputs, passes,
                                                              bytes_done / 1e6, t_total),
        # the workload's layer-tokens at the oracle's rate over its own bytes
        "layer_tokens_per_s": round(gbs * 1e9 / step.bytes * w.copies * w.n, 2),
        "parity": {"outputs": checked, "max_err_over_tolerance": worst, "pass": bool(worst <= 1.0)},
    }
    if w.name in MFMA_WORKLOADS:
        out["gflops"] = round(flops_done / t_total / 1e9, 2)
    return out, prepared


def oracle_one_thread(prepared, w, reps_s=2.0):
    """The oracle's fp64 product on one thread, over the first prepared item
    of the sample (repeated for about reps_s seconds)."""
    import oracle
    gemv = oracle.mx_gemv if w.fmt == "mxfp4" else oracle.gemv
    codes, scales, xb, nbytes, _, _ = prepared[0]
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        t, reps = 0.0, 0
        while t < reps_s or reps < 2:
            t0 = time.perf_counter()
            gemv(codes, scales, w.tscale, xb)
            t += time.perf_counter() - t0
            reps += 1
    finally:
        oracle.set_num_threads(threads)
    per = t / reps
    return {"ms_per_product": round(per * 1e3, 3), "gbs": round(nbytes / per / 1e9, 4), "repetitions": reps,
            "product": "%dx%d, N=%d" % (codes.shape[0], codes.shape[1] * 2, xb.shape[0])}


# ---------------------------------------------------------------- traffic --

def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_bit_nvfp4_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, variant=None):
    """HBM bytes of one dominant call (its product kernel, plus the argmax
    finish where the call has one) from the committed counter summary, or
    None if absent, taken on different kernel sources, or taken on another
    variant of the step (the counters were collected on the default one)."""
    if variant:
        return None
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("dominant_bytes_per_launch")


# ------------------------------------------------------------- one config --

def measure(name, args, probe, mfma_peak=None):
    """Every figure of one workload; returns (the entry, the step's wall-clock
    seconds per step, the step)."""
    step = Step(name, fused_mlp=not args.mlp_three_launches)
    step.run()
    torch.cuda.synchronize()
    w = step.w
    per_graph = steps_per_graph(name, args.steps)
    step_s, step_ev_s = time_graph(step.run, args.steps, args.warmup, per_graph)
    kernels = kernel_times(step, args.steps, args.warmup, per_graph)
    # Dominant kernel: the one moving the most bytes per step (the wide
    # kernel for the N = 512 workloads).
    dom = max(kernels, key=lambda e: e["launches_per_step"] * next(
        L.bytes for L in step.launches if L.kernel == e["kernel"]))
    dl = next(L for L in step.launches if L.kernel == dom["kernel"])
    per_s = dom["us_per_launch"] * 1e-6
    variant = "three launches" if args.mlp_three_launches and name == "mlp_27b_decode" else None
    if name in MFMA_WORKLOADS:
        achieved = dl.flops / per_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(name)}
    else:
        achieved = dl.bytes / per_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name, variant)}
    roof["kernel"] = dom["kernel"]
    roof["kernel_avg_us"] = dom["us_per_launch"]
    roof["scope"] = ("average %s of %s: HIP events on the replay stream around %d steps of a graph of its "
                     "%d launches per step, %d step(s) per replay" % (
                         "call (product + argmax finish)" if "argmax" in dom["kernel"] else "launch",
                         dom["kernel"], args.steps, dom["launches_per_step"], dom["steps_per_replay"]))
    value = step.bytes / step_s / 1e9
    e = {
        "workload": name, "description": w.description, "n": w.n,
        "matrices": ["%dx%d" % (m.rows, m.cols) for m in w.matrices], "copies": w.copies,
        "bytes_per_step": step.bytes, "us_per_step": round(step_s * 1e6, 3),
        "us_per_step_events": round(step_ev_s * 1e6, 3), "steps_per_replay": per_graph,
        "gbs": round(value, 1), "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "layer_tokens_per_s": round(w.copies * w.n / step_s, 1),
        "kernels": kernels, "roofline": roof,
    }
    if name in MFMA_WORKLOADS:
        tf = step.flops / step_s / 1e12
        e["tflops"] = round(tf, 2)
        e["pct_of_bf16_peak"] = round(100 * tf / BF16_PEAK_TFLOPS, 2)
        if mfma_peak is not None:
            e["measured_wall"] = mfma_peak
            e["pct_of_measured_wall"] = round(100 * tf / mfma_peak["tflops"], 2)
    elif probe is not None:
        wall = read_wall(probe, step, args.steps, args.warmup, per_graph)
        e["measured_wall"] = wall
        # the same bytes: the wall's time over the step's
        e["pct_of_measured_wall"] = round(100 * wall["us_per_step"] / (step_s * 1e6), 2)
        e["pct_of_read_store_wall"] = round(100 * wall["read_store"]["us_per_step"] / (step_s * 1e6), 2)
    if name == "mlp_27b_decode":
        e["mlp"] = ("three launches per layer" if args.mlp_three_launches else
                    "two launches per layer (gate||up with SwiGLU fused, down)")
    if name == "gemv_256x512":
        e["note"] = "latency-bound parity case (75.8 KB per call): no bandwidth claim"
    if not args.no_cpu_baseline:
        cb, prepared = cpu_baseline(step)
        if name in ("gemv_256x512", HEADLINE) and prepared:
            cb["one_thread"] = oracle_one_thread(prepared, w)
        e["cpu_baseline"] = cb
    return e, step_s, step


# ------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all",
                    help="all (the five configurations; C2 carries value) or one workload name")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-wall", action="store_true", help="skip the measured-wall probes")
    ap.add_argument("--mlp-three-launches", action="store_true",
                    help="run the decode MLP as gate||up matvec, SwiGLU and down matvec (three launches "
                         "per layer) instead of gate||up with SwiGLU fused, then down (two launches)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (read + write), e.g. to "
                         "calibrate HBM traffic counters against a known byte count")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the NVFP4 matvec path runs on a single MI355X (sharding "
              "the rows across GPUs is described, not built); rerun with --gpus 1", file=sys.stderr)
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
    probe = None if args.no_wall else Probe()
    names = [c for _, c in CONFIGS] if args.workload == "all" else [args.workload]
    mfma_peak = mfma_wall(probe) if probe is not None and any(n in MFMA_WORKLOADS for n in names) else None
    entries, head = {}, None
    for cid, name in ([(c, n) for c, n in CONFIGS] if args.workload == "all" else [(None, args.workload)]):
        log("measuring %s" % name)
        e, step_s, step = measure(name, args, probe, mfma_peak)
        if cid:
            e["config"] = cid
        entries[name] = e
        if name == (HEADLINE if args.workload == "all" else args.workload):
            head = (e, step_s, step.w)
        del step
        torch.cuda.empty_cache()
    e, step_s, w = head
    result = {
        "metric": METRIC,
        "value": e["gbs"],
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
        "config": {k: e[k] for k in ("workload", "description", "n", "matrices", "copies", "bytes_per_step",
                                     "pct_of_hbm_peak", "layer_tokens_per_s") if k in e},
        "roofline": e["roofline"],
    }
    result["config"]["timing"] = "HIP graph replays, %d step(s) per replay" % e["steps_per_replay"]
    for k in ("pct_of_measured_wall", "pct_of_read_store_wall"):
        if k in e:
            result["config"][k] = e[k]
    if "cpu_baseline" in e:
        result["cpu_baseline"] = e["cpu_baseline"]
    result["host"] = host_facts()
    if args.workload == "all":
        result["configs"] = entries
    else:
        result["detail"] = e
    print(json.dumps(result))


if __name__ == "__main__":
    main()
