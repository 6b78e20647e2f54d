"""w4_matmul_noalloc (the allocation-free entry point) against w4_matmul.

Through the C ABI, on the same seeded inputs: two calls in a row, the second
with a smaller input, each bit-identical to w4_matmul with its own workspace
(same kernels, fixed summation order) and within the oracle's bound; a shape
whose split-K partials exceed the library's scratch is refused.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4_block_dequant_amd as w4

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _case(M, K, N, cfg):
    orc = oracle.default()
    W = synth.weights(K, N, cfg=cfg)
    x = synth.activations(M, K, cfg=cfg, outliers=True)
    b = synth.bias(N, cfg=cfg)
    Wq, s, z = orc.quantize_pack(W)
    y_ref, bound = orc.w4_matmul(x, Wq, s, z, b)
    return [_dev(a) for a in (x, Wq, s, z, b)], y_ref, bound


def _noalloc(x, Wq, s, z, b, M, K, N):
    y = torch.full((M, N), float("nan"), device=DEV)
    st = w4.library().w4_matmul_noalloc(x.data_ptr(), M, K, Wq.data_ptr(), s.data_ptr(),
                                        z.data_ptr(), N, b.data_ptr(), y.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
    assert st == w4.W4_OK, w4.w4_strerror(st)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_noalloc_matches_w4_matmul_twice_then_smaller():
    # first: split-K over many workgroups (about 22 MB of partial sums);
    # second: a smaller shape that reuses the start of the same scratch
    for M, K, N, cfg in ((58, 3072, 3072, 271), (1, 768, 768, 272)):
        need = w4.w4_matmul_workspace_bytes(M, K, N)
        print(f"noalloc M={M} K={K} N={N} partial bytes {need}", flush=True)
        assert need <= w4.NOALLOC_SCRATCH_BYTES
        (x, Wq, s, z, b), y_ref, bound = _case(M, K, N, cfg)
        got = _noalloc(x, Wq, s, z, b, M, K, N)
        ws = torch.full((max(need, 256),), 0x5A, dtype=torch.uint8, device=DEV)
        want = w4.w4_matmul(x, Wq, s, z, b, workspace=ws).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"M={M}: differs"
        err = np.abs(got.astype(np.float64) - y_ref)
        assert np.all(np.isfinite(got)) and np.all(err <= bound), f"M={M}: out of bound"
    assert w4.w4_matmul_workspace_bytes(58, 3072, 3072) > w4.w4_matmul_workspace_bytes(1, 768, 768)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    M, K, N = 64, 8192, 3072
    assert w4.w4_matmul_workspace_bytes(M, K, N) > w4.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), device=DEV)
    Wq = torch.zeros((K, N // 2), dtype=torch.uint8, device=DEV)
    s = torch.zeros((K // 32, N), device=DEV)
    z = torch.zeros((K // 32, N // 2), dtype=torch.uint8, device=DEV)
    y = torch.zeros((M, N), device=DEV)
    st = w4.library().w4_matmul_noalloc(x.data_ptr(), M, K, Wq.data_ptr(), s.data_ptr(),
                                        z.data_ptr(), N, None, y.data_ptr(), None)
    assert st == w4.W4_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not y.any()  # nothing was enqueued
