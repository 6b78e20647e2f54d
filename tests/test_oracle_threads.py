"""The oracle's results do not depend on its OpenMP thread count (it shares
independent output columns and rows among threads; each output's own sum runs
in order), so the CPU baseline may be timed at any thread count."""
import os

import numpy as np

import oracle
import synth


def test_results_identical_across_thread_counts():
    orc = oracle.default()
    before = orc.threads()
    K, N, M = 768, 1000, 3
    W = synth.weights(K, N, cfg=91)
    x = synth.activations(M, K, cfg=91, outliers=True)
    b = synth.bias(N, cfg=91)
    Wq, s, z = orc.quantize_pack(W)
    Q, hs = orc.i8_quantize_head(synth.head_table(K, 700, cfg=92), ldq=703)
    outs = []
    try:
        for t in sorted({1, 4, os.cpu_count() or 1}):
            orc.set_threads(t)
            assert orc.threads() == t
            y, bound = orc.w4_matmul(x, Wq, s, z, b)
            lg, lb = orc.i8_head_logits(x[-1], Q, hs)
            outs.append((y, bound, lg, lb))
    finally:
        orc.set_threads(before)
    for o in outs[1:]:
        for a, ref in zip(o, outs[0]):
            assert np.array_equal(a.view(np.uint8), ref.view(np.uint8))
