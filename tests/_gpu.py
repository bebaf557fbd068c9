"""Helpers for the GPU parity tests: run the HIP library through its C ABI on
seeded inputs and fetch what the oracle needs.  No NVFP4 arithmetic here."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_scaled_bit_nvfp4_amd as nv
from block_scaled_bit_nvfp4_amd import workloads as wl

DEV = "cuda:0"


def note(msg: str):
    """Name the case before a GPU step, flushed, so a fault is attributable."""
    sys.stdout.write("[gpu] %s\n" % msg)
    sys.stdout.flush()


def u8_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").numpy()


def bits_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (host) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def quantize_gpu(W: torch.Tensor, tscale: float = 1.0):
    R, K = W.shape
    codes = torch.empty(R, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(R, K // 16, dtype=torch.uint8, device=DEV)
    nv.nvfp4_quantize(W, R, K, tscale, codes, scales)
    return codes, scales


def repack_gpu(codes: torch.Tensor, scales: torch.Tensor, R: int, K: int):
    wq, ws = nv.alloc_repacked(R, K, DEV)
    wq.fill_(0xA5)     # every byte must be overwritten
    ws.fill_(0x5A)
    nv.nvfp4_repack(codes, scales, R, K, wq, ws)
    return wq, ws


def canonical_to_dev(codes: np.ndarray, scales: np.ndarray):
    return (torch.from_numpy(np.ascontiguousarray(codes)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(scales)).to(DEV))


def gemv_gpu(wq, ws, tscale, R, K, X: torch.Tensor) -> torch.Tensor:
    n = X.shape[0]
    Y = torch.full((n, R), float("nan"), dtype=torch.float32, device=DEV)
    nv.nvfp4_gemv(wq, ws, tscale, R, K, X, n, Y)
    return Y


def gemv_argmax_gpu(wq, ws, tscale, R, K, X: torch.Tensor, with_logits=True, workspace=None):
    n = X.shape[0]
    logits = torch.full((n, R), float("nan"), dtype=torch.float32, device=DEV) if with_logits else None
    am = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    if workspace is None:      # any contents: the call overwrites the workspace
        workspace = torch.full((nv.nvfp4_gemv_argmax_workspace_bytes(R, K, n),), 0xA5, dtype=torch.uint8,
                               device=DEV)
    wsp = workspace
    nv.nvfp4_gemv_argmax(wq, ws, tscale, R, K, X, n, logits, am, wsp)
    return logits, am


def seeded_matrix(R: int, K: int, seed: int, outliers=True, device=DEV):
    return wl.weights(R, K, seed=seed, outliers=outliers, device=device)


def seeded_x(n: int, K: int, seed: int, device=DEV):
    return wl.activations(n, K, seed=seed, device=device)


def assert_within_tolerance(Y_gpu: np.ndarray, Y_ref: np.ndarray, S: np.ndarray, what: str):
    """|y_gpu - y_ref| <= 1e-5 * sum|w*x| + 1e-6, elementwise."""
    Y_gpu = np.asarray(Y_gpu, np.float64)
    err = np.abs(Y_gpu - Y_ref)
    bound = 1e-5 * S + 1e-6
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d outputs out of tolerance, e.g. %s" % (
            what, int(bad.sum()), bad.size,
            [(tuple(i), float(Y_gpu[tuple(i)]), float(Y_ref[tuple(i)]), float(bound[tuple(i)])) for i in idx]))
    return float((err / bound).max()) if err.size else 0.0
