"""nvfp4_gemv_argmax_noalloc, the argmax product for callers that cannot
allocate: its keys live in the library's static per-GPU array instead of a
caller's workspace.  It must give nvfp4_gemv_argmax's logits and indices bit
for bit, call after call, whatever an earlier call left in the array, and
reject shapes whose keys would not fit before anything is launched."""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_bit_nvfp4_amd as nv
from tests import _gpu as G

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 1 << 20        # NVFP4_ARGMAX_SCRATCH_BYTES


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()
    yield
    torch.cuda.synchronize()


def _weights(R, K, seed):
    W = G.seeded_matrix(R, K, seed)
    codes, scales = G.quantize_gpu(W)
    wq, ws = G.repack_gpu(codes, scales, R, K)
    return W, wq, ws


def _noalloc(wq, ws, R, K, X):
    n = X.shape[0]
    logits = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV)
    am = torch.full((n,), -7, dtype=torch.int32, device=G.DEV)
    nv.nvfp4_gemv_argmax_noalloc(wq, ws, 1.0, R, K, X, n, logits, am)
    return logits, am


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    """A larger call, then a smaller one on other inputs: each equals the
    workspace entry point's result, and the argmax equals the oracle's."""
    for i, (R, K, n) in enumerate([(65620, 528, 5), (2000, 1024, 8)]):
        W, wq, ws = _weights(R, K, 300 + i)
        X = G.seeded_x(n, K, seed=310 + i)
        G.note("noalloc call %d: %dx%d n=%d" % (i, R, K, n))
        logits, am = _noalloc(wq, ws, R, K, X)
        ref_logits, ref_am = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, X)
        assert torch.equal(logits.view(torch.int32), ref_logits.view(torch.int32)), i
        assert torch.equal(am, ref_am), i
        c_ref, s_ref = oracle.quantize(W.cpu().numpy())
        Y_ref, _ = oracle.gemv(c_ref, s_ref, 1.0, G.wl.bf16_bits(X))
        assert list(am.cpu().numpy()) == list(oracle.argmax_first(Y_ref)), i
        # without logits: the same rows
        am2 = torch.full((n,), -7, dtype=torch.int32, device=G.DEV)
        nv.nvfp4_gemv_argmax_noalloc(wq, ws, 1.0, R, K, X, n, None, am2)
        assert torch.equal(am2, ref_am), i


def test_noalloc_largest_shape_and_the_first_rejected():
    """1047424 rows at n = 8 use all of the array (the finish's 1152-byte
    header, then one key per 64-row workgroup and column); one row more
    needs a workgroup past it and is rejected on the host, before any
    launch."""
    R, K, n = 1047424, 16, 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(R, K, n) == SCRATCH_BYTES
    assert nv.nvfp4_gemv_argmax_workspace_bytes(R + 1, K, n) > SCRATCH_BYTES
    _, wq, ws = _weights(R, K, 320)
    X = G.seeded_x(n, K, seed=321)
    G.note("noalloc largest %dx%d n=%d" % (R, K, n))
    logits, am = _noalloc(wq, ws, R, K, X)
    ref_logits, ref_am = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, X)
    assert torch.equal(logits.view(torch.int32), ref_logits.view(torch.int32))
    assert torch.equal(am, ref_am)
    wq1, ws1 = nv.alloc_repacked(R + 1, K, G.DEV)
    with pytest.raises(nv.NVFP4Error) as err:
        _noalloc(wq1, ws1, R + 1, K, X)
    assert err.value.status == -4
