"""Seeded synthetic inputs for the NVFP4 matrix-vector path.

This module holds no NVFP4 arithmetic: it only draws the fp32 weights and the
bf16 activations that both the HIP library and the CPU oracle consume (each
side quantises and multiplies on its own).  Shapes stand in for the pages'
workloads: single-stream decode of a 27B-class dense model (5120 hidden,
17408 MLP width, a 151936-entry vocabulary), the K+1 = 4 column speculative
verify, a 512-token prefill chunk, and the trimmed-vocabulary draft head of
speculative decoding (bw24 README and wiki, performance and feature
sections, the FR-Spec draft trims; qwentin README, "Performance" and "How it
works").

Weights: fp32 N(0, 0.02); where a workload has outliers, every element is
independently an outlier with probability 0.001 and is then replaced by
+-0.16 (8 sigma) with a fair sign.  Activations: fp32 N(0, 1) rounded to
bf16.  Every draw comes from a ``torch.Generator`` on the device the tensor
is made on, seeded by (workload, tensor, copy), so a run is reproducible on
one device type; the CPU and GPU streams differ, and tests always hand the
same tensor to both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SIGMA = 0.02
OUTLIER_P = 0.001
OUTLIER_SIGMAS = 8.0


@dataclass(frozen=True)
class Matrix:
    name: str
    rows: int
    cols: int


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    n: int                     # activation columns per call
    matrices: tuple            # one layer / pass, in call order
    copies: int = 1            # distinct weight sets rotated over
    outliers: bool = True
    tscale: float = 1.0
    argmax: tuple = field(default_factory=tuple)   # names of matrices with an argmax
    fmt: str = "nvfp4"         # weight format: "nvfp4" or "mxfp4"


WORKLOADS = {
    "gemv_256x512": Workload(
        "gemv_256x512", "single NVFP4 matvec 256x512, N=1, seed 0, no outliers",
        1, (Matrix("w", 256, 512),), copies=1, outliers=False),
    "decode_4096x4096": Workload(
        "decode_4096x4096", "decode GEMV 4096x4096, N=1, 64 distinct matrices rotated",
        1, (Matrix("w", 4096, 4096),), copies=64),
    "mlp_27b_decode": Workload(
        "mlp_27b_decode", "27B-class MLP decode, N=1: gate||up 34816x5120, SwiGLU, "
        "down 5120x17408; 8 layer copies rotated",
        1, (Matrix("gate_up", 34816, 5120), Matrix("down", 5120, 17408)), copies=8),
    "verify_vocab_n4": Workload(
        "verify_vocab_n4", "speculative verify N=4: 17408x5120 and lm_head 151936x5120 "
        "with per-column argmax",
        4, (Matrix("w", 17408, 5120), Matrix("lm_head", 151936, 5120)), copies=1,
        argmax=("lm_head",)),
    # The widest verify the matvec takes: seven drafted tokens plus one.
    "verify_vocab_n8": Workload(
        "verify_vocab_n8", "speculative verify N=8: 17408x5120 and lm_head 151936x5120 "
        "with per-column argmax",
        8, (Matrix("w", 17408, 5120), Matrix("lm_head", 151936, 5120)), copies=1,
        argmax=("lm_head",)),
    # The N = 512 contraction runs over four layer copies per step, so that a
    # step's launches run back to back as a prefill's layers would.
    "prefill_n512": Workload(
        "prefill_n512", "prefill-width contraction N=512: 17408x5120, 4 layer copies rotated",
        512, (Matrix("w", 17408, 5120),), copies=4),
    # A trimmed-vocabulary draft head (an 8192-row subset of a vocabulary at a
    # 4096 hidden size: 18.9 MB at NVFP4) drafting one token per call;
    # 16 copies (302 MB) rotate past the 256 MB Infinity Cache.
    "draft_head_8192x4096": Workload(
        "draft_head_8192x4096", "trimmed-vocabulary draft head 8192x4096 with argmax, N=1; "
        "16 distinct heads rotated",
        1, (Matrix("draft_head", 8192, 4096),), copies=16, argmax=("draft_head",)),
    # The second block-scaled format (E2M1 with one E8M0 scale per 32
    # elements) on the 17408 x 5120 matrix: N = 1 over 8 rotated copies
    # (379 MB, past the Infinity Cache), and the N = 512 contraction.
    "mxfp4_gemv_17408x5120": Workload(
        "mxfp4_gemv_17408x5120", "MXFP4 matvec 17408x5120, N=1, 8 distinct matrices rotated",
        1, (Matrix("w", 17408, 5120),), copies=8, fmt="mxfp4"),
    "mxfp4_prefill_n512": Workload(
        "mxfp4_prefill_n512", "MXFP4 prefill-width contraction N=512: 17408x5120, 4 layer copies rotated",
        512, (Matrix("w", 17408, 5120),), copies=4, fmt="mxfp4"),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def seed_of(workload: str, tensor: str, copy: int = 0) -> int:
    """Stable 63-bit seed from (workload, tensor, copy); the small workload
    keeps the literal seed 0 for its weights."""
    if workload == "gemv_256x512" and tensor == "w" and copy == 0:
        return 0
    h = 1469598103934665603
    for ch in ("%s/%s/%d" % (workload, tensor, copy)).encode():
        h = ((h ^ ch) * 1099511628211) & ((1 << 63) - 1)
    return h


def weights(rows: int, cols: int, seed: int, outliers: bool = True,
            device="cpu") -> torch.Tensor:
    """fp32 [rows][cols]: N(0, 0.02) with optional 0.1% outliers at +-8 sigma."""
    g = _gen(device, seed)
    w = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    w.mul_(SIGMA)
    if outliers:
        u = torch.rand(rows, cols, generator=g, device=device, dtype=torch.float32)
        mask = u < OUTLIER_P
        del u
        sign = torch.rand(rows, cols, generator=g, device=device) < 0.5
        val = torch.where(sign, -OUTLIER_SIGMAS * SIGMA, OUTLIER_SIGMAS * SIGMA)
        w = torch.where(mask, val.to(torch.float32), w)
    return w


def activations(n: int, cols: int, seed: int, device="cpu") -> torch.Tensor:
    """bf16 [n][cols]: fp32 N(0, 1) rounded to nearest-even bf16."""
    g = _gen(device, seed)
    x = torch.randn(n, cols, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def bf16_bits(x: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return x.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
