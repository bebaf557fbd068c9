"""The seeded input generators: shapes, dtypes, determinism and the
outlier recipe (0.1% of elements at +-8 sigma)."""
import torch

from block_scaled_bit_nvfp4_amd import workloads as wl


def test_workload_table():
    assert set(wl.WORKLOADS) == {"gemv_256x512", "decode_4096x4096", "mlp_27b_decode",
                                 "verify_vocab_n4", "verify_vocab_n8", "prefill_n512", "draft_head_8192x4096",
                                 "mxfp4_gemv_17408x5120", "mxfp4_prefill_n512"}
    assert wl.WORKLOADS["mxfp4_prefill_n512"].fmt == "mxfp4"
    assert wl.WORKLOADS["prefill_n512"].fmt == "nvfp4"
    d = wl.WORKLOADS["draft_head_8192x4096"]
    assert (d.matrices[0].rows, d.matrices[0].cols, d.n, d.copies) == (8192, 4096, 1, 16)
    assert d.argmax == ("draft_head",)
    m = wl.WORKLOADS["mlp_27b_decode"].matrices
    assert (m[0].rows, m[0].cols, m[1].rows, m[1].cols) == (34816, 5120, 5120, 17408)
    assert wl.WORKLOADS["verify_vocab_n4"].n == 4
    assert wl.WORKLOADS["verify_vocab_n8"].n == 8
    assert wl.WORKLOADS["verify_vocab_n8"].matrices == wl.WORKLOADS["verify_vocab_n4"].matrices
    assert wl.WORKLOADS["prefill_n512"].n == 512
    assert wl.seed_of("gemv_256x512", "w") == 0
    assert wl.seed_of("decode_4096x4096", "w", 1) != wl.seed_of("decode_4096x4096", "w", 2)


def test_weights_deterministic_and_distributed():
    a = wl.weights(256, 1024, seed=5)
    b = wl.weights(256, 1024, seed=5)
    assert a.dtype == torch.float32 and a.shape == (256, 1024)
    assert torch.equal(a, b)
    out = (a.abs() == 0.16).float().mean().item()
    assert 0.0005 < out < 0.002
    body = a[a.abs() != 0.16]
    assert abs(body.std().item() - 0.02) < 0.001
    c = wl.weights(64, 512, seed=0, outliers=False)
    assert (c.abs() == 0.16).sum().item() == 0


def test_activations_bf16():
    x = wl.activations(4, 5120, seed=3)
    assert x.dtype == torch.bfloat16 and x.shape == (4, 5120)
    assert abs(x.float().std().item() - 1.0) < 0.05
    bits = wl.bf16_bits(x)
    assert bits.dtype.name == "uint16" and bits.shape == (4, 5120)
