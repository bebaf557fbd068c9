"""Host logic of bench.py that needs no GPU: the one-GPU refusal, the
algorithmic byte counts its rooflines divide by, the steps per graph replay,
and the rule that a committed HBM-traffic figure is used only on the kernel
sources it was taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench                                   # noqa: E402
import block_scaled_bit_nvfp4_amd as nv        # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, env=env, timeout=300)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      (["--gpus", "1"], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(args, env):
    r = _run_bench(args, env)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line for a run that measured nothing


def test_algorithmic_bytes_of_the_workloads():
    # 4096 x 4096 NVFP4 at one column: 8 MiB of codes, 1 MiB of scales,
    # 8 KiB of bf16 activations, 16 KiB of fp32 outputs
    assert bench.weight_bytes(4096, 4096) == 4096 * 4096 // 2 + 4096 * 4096 // 16
    assert bench.gemv_bytes(4096, 4096, 1) == 9461760
    # MXFP4: one scale byte per 32 elements
    assert bench.weight_bytes(17408, 5120, "mxfp4") == 17408 * 5120 // 2 + 17408 * 5120 // 32
    # N = 512 prefill: X and Y grow with the columns
    assert bench.gemv_bytes(17408, 5120, 512) == 17408 * 5120 * 9 // 16 + 512 * 5120 * 2 + 512 * 17408 * 4


@pytest.mark.parametrize("rows,cols", [(4096, 4096), (34816, 5120), (5120, 17408), (151936, 5120), (256, 512)])
def test_weight_bytes_equal_the_repacked_planes_where_nothing_is_padded(rows, cols):
    """For rows a multiple of 64 and cols a multiple of 128 elements the
    repacked planes hold no padding, so the bytes the products stream are
    exactly the algorithmic weight bytes (both formats)."""
    nv.load()
    assert nv.nvfp4_repacked_code_bytes(rows, cols) + nv.nvfp4_repacked_scale_bytes(rows, cols) == \
        bench.weight_bytes(rows, cols)
    assert nv.mxfp4_repacked_code_bytes(rows, cols) + nv.mxfp4_repacked_scale_bytes(rows, cols) == \
        bench.weight_bytes(rows, cols, "mxfp4")


def test_steps_per_graph_divides_the_steps():
    assert bench.steps_per_graph("decode_4096x4096", 50) == 1
    assert bench.steps_per_graph("mlp_27b_decode", 50) == 1
    assert bench.steps_per_graph("gemv_256x512", 48) == 16
    assert bench.steps_per_graph("gemv_256x512", 50) == 10
    assert bench.steps_per_graph("verify_vocab_n4", 50) == 2
    for name in ("gemv_256x512", "verify_vocab_n4", "verify_vocab_n8", "prefill_n512"):
        for steps in (1, 7, 20, 50, 64):
            assert steps % bench.steps_per_graph(name, steps) == 0


def test_traffic_is_used_only_on_the_sources_it_was_taken_on(monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_decode_4096x4096.json")
    with open(path) as f:
        d = json.load(f)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: d["kernel_source_hash"])
    assert bench.measured_traffic("decode_4096x4096") == d["dominant_bytes_per_launch"]
    assert bench.measured_traffic("decode_4096x4096", variant="three launches") is None
    assert bench.measured_traffic("no_such_workload") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic("decode_4096x4096") is None


def test_kernel_source_hash_covers_every_kernel_source(tmp_path, monkeypatch):
    """A change anywhere in the kernel sources' bytes, a comment included, or
    a new source file changes the hash (so a traffic figure is never carried
    over to edited kernels)."""
    csrc = tmp_path / "block_scaled_bit_nvfp4_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("// one\n")
    (csrc / "b.h").write_text("int x;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "b.h").write_text("int x; // a comment\n")
    h1 = bench.kernel_source_hash()
    (csrc / "c.hip").write_text("__global__ void k() {}\n")
    h2 = bench.kernel_source_hash()
    assert len({h0, h1, h2}) == 3
