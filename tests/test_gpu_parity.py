"""HIP path against the CPU oracle on the same seeded inputs (needs a gfx950 GPU).

Bars:
  * packing, unpacking, dequantization, the head table and its scales, and
    the token lookup: bit-exact;
  * every fp32 output of a matmul or the head: |y_gpu - y_ref| <= bound, the
    oracle's per-output 1e-5 * (sum_k |x w_hat| + |bias|) + 1e-6.
Every call goes through the C ABI (via the thin binding).  Shapes span
several tiles and split-K workgroups with ragged tails; the full-size
3.8B-dense shapes are checked on sampled columns that the oracle computes
on its own (quantization is per column, so a column subset quantizes to the
same codes).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4_block_dequant_amd as w4

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ORC = oracle.default()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def note(msg):
    print(msg, flush=True)


def assert_bits(a, b, label):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    assert a.shape == b.shape, (label, a.shape, b.shape)
    av = a.view(np.uint32) if a.dtype == np.float32 else a
    bv = b.view(np.uint32) if b.dtype == np.float32 else b
    bad = np.count_nonzero(av != bv)
    note(f"{label}: {a.size - bad}/{a.size} bit-exact")
    assert bad == 0


def assert_bound(y, y_ref, bound, label):
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    ratio = float(np.max(err / bound)) if err.size else 0.0
    note(f"{label}: max |err|/bound = {ratio:.3e} over {err.size} outputs")
    assert np.all(np.isfinite(y))
    assert np.all(err <= bound), f"{label}: {np.count_nonzero(err > bound)} outputs out of bound"


# --------------------------------------------------------------------------
# weights with every kind of block the format meets
# --------------------------------------------------------------------------
def mixed_weights(K, N, cfg):
    W = synth.weights(K, N, cfg=cfg)
    g = np.random.default_rng([cfg, K, N])
    if N >= 8:
        W[:, 0] = 0.0                                       # all-zero blocks
        W[:, 1] = 0.5                                       # constant positive
        W[:, 2] = -0.25                                     # constant negative
        W[:, 3] = np.abs(W[:, 3]) + np.float32(0.3)         # same sign
        W[:, 4] = (g.standard_normal(K) * 1e-41).astype(np.float32)  # subnormal
        W[:, 5] = g.standard_t(2, size=K).astype(np.float32)          # heavy tail
    return W


PACK_SHAPES = [(32, 2), (64, 34), (96, 530), (768, 2304), (3072, 768), (160, 1024)]


@pytest.mark.parametrize("K,N", PACK_SHAPES)
def test_quantize_pack_bit_exact(K, N):
    note(f"quantize_pack K={K} N={N}")
    W = mixed_weights(K, N, cfg=200)
    ref = ORC.quantize_pack(W)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = w4.w4_quantize_pack(dev(W), d_status=st)
    for name, a, b in zip(("Wq", "scales", "zeros"), got, ref):
        assert_bits(host(a), b, f"{name} {K}x{N}")
    assert host(st)[0] == 0


def test_quantize_pack_on_grid_and_ties():
    from oracle_pins import _on_grid
    W, q, z, s = _on_grid(256, 34, 4)
    ref = ORC.quantize_pack(W)
    got = w4.w4_quantize_pack(dev(W))
    for name, a, b in zip(("Wq", "scales", "zeros"), got, ref):
        assert_bits(host(a), b, f"on-grid {name}")
    # halfway weights: (c - z + 1/2) * 2^e
    g = np.random.default_rng(31)
    K, N = 64, 16
    Wt = np.zeros((K, N), np.float32)
    for b in range(K // 32):
        for n in range(N):
            s_ = np.float32(2.0 ** int(g.integers(-9, -4)))
            zz = int(g.integers(1, 15))
            rows = g.permutation(32)
            for i, r in enumerate(rows):
                c = 0 if i == 0 else 15 if i == 1 else int(g.integers(0, 15))
                off = 0.0 if i < 2 else 0.5
                Wt[b * 32 + r, n] = np.float32(c - zz + off) * s_
    ref = ORC.quantize_pack(Wt)
    got = w4.w4_quantize_pack(dev(Wt))
    for name, a, b in zip(("Wq", "scales", "zeros"), got, ref):
        assert_bits(host(a), b, f"ties {name}")


@pytest.mark.parametrize("K,N", [(64, 34), (768, 768), (96, 530)])
def test_unpack_and_dequantize_bit_exact(K, N):
    note(f"unpack/dequantize K={K} N={N}")
    W = mixed_weights(K, N, cfg=201)
    Wq, s, z = ORC.quantize_pack(W)
    q_ref, z_ref = ORC.unpack(Wq, z, K, N)
    q, zz = w4.w4_unpack(dev(Wq), dev(z), K, N)
    assert_bits(host(q), q_ref, "q")
    assert_bits(host(zz), z_ref, "z")
    What = w4.w4_dequantize(dev(Wq), dev(s), dev(z))
    assert_bits(host(What), ORC.dequantize(Wq, s, z, K, N), "W_hat")


def test_quantize_nonfinite_sets_status():
    W = synth.weights(64, 32, cfg=202)
    W[40, 7] = np.nan
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    w4.w4_quantize_pack(dev(W), d_status=st)
    assert host(st)[0] == w4.W4_ERR_NONFINITE
    W[40, 7] = 1.0
    W[3, 3], W[4, 3] = 3e38, -3e38
    st.zero_()
    w4.w4_quantize_pack(dev(W), d_status=st)
    assert host(st)[0] == w4.W4_ERR_NONFINITE


# --------------------------------------------------------------------------
# matmul
# --------------------------------------------------------------------------
def run_matmul_case(M, K, N, cfg, bias=True, outliers=False, weights=None):
    W = mixed_weights(K, N, cfg) if weights is None else weights
    x = synth.activations(M, K, cfg=cfg, outliers=outliers)
    b = synth.bias(N, cfg=cfg) if bias else None
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z, b)
    y = w4.w4_matmul(dev(x), dev(Wq), dev(s), dev(z), None if b is None else dev(b))
    return host(y), y_ref, bound


GEMV_SHAPES = [
    (32, 16), (64, 256), (96, 272), (768, 768), (768, 2304), (3072, 768), (768, 3072),
    (1024, 1008), (8192, 512), (256, 40), (128, 2), (4096, 4112),
]


@pytest.mark.parametrize("K,N", GEMV_SHAPES)
@pytest.mark.parametrize("bias", [True, False])
def test_gemv_m1(K, N, bias):
    note(f"gemv M=1 K={K} N={N} bias={bias}")
    y, y_ref, bound = run_matmul_case(1, K, N, cfg=210, bias=bias, outliers=(K % 64 == 0))
    assert_bound(y, y_ref, bound, f"gemv {K}x{N}")


@pytest.mark.parametrize("M", [2, 3, 16, 58, 64, 65])
@pytest.mark.parametrize("K,N", [(768, 768), (96, 272), (256, 40)])
def test_small_m(M, K, N):
    note(f"small-M M={M} K={K} N={N}")
    y, y_ref, bound = run_matmul_case(M, K, N, cfg=211, outliers=True)
    assert_bound(y, y_ref, bound, f"M={M} {K}x{N}")


@pytest.mark.parametrize("M", [1, 58])
@pytest.mark.parametrize("slot", range(4))
def test_gpt2_body_shapes(M, slot):
    K, N = synth.GPT2_SHAPES[slot]
    note(f"gpt2 slot {slot} M={M} K={K} N={N}")
    W = synth.weights(K, N, cfg=synth.CFG_GPT2_PREFILL, slot=slot)
    y, y_ref, bound = run_matmul_case(M, K, N, cfg=synth.CFG_GPT2_PREFILL, weights=W)
    assert_bound(y, y_ref, bound, f"gpt2 M={M} {K}x{N}")


def sample_pairs(N, count, seed):
    g = np.random.default_rng(seed)
    pairs = np.sort(g.choice(N // 2, size=count, replace=False))
    pairs[0], pairs[-1] = 0, N // 2 - 1
    return np.unique(pairs)


@pytest.mark.parametrize("slot", range(4))
@pytest.mark.parametrize("M", [1, 4, 16])
def test_dense38_full_size_sampled(slot, M):
    """Full-size 3.8B-dense shapes in the benchmark's launch configuration."""
    K, N = synth.DENSE38_SHAPES[slot]
    note(f"dense38 slot {slot} M={M} K={K} N={N} (sampled columns)")
    W = synth.weights(K, N, cfg=synth.CFG_DENSE38, layer=0, slot=slot)
    x = synth.activations(M, K, cfg=synth.CFG_DENSE38, layer=0, slot=slot, outliers=True)
    Wq_d, s_d, z_d = w4.w4_quantize_pack(dev(W))
    y = host(w4.w4_matmul(dev(x), Wq_d, s_d, z_d))
    pairs = sample_pairs(N, 48, seed=slot)
    cols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
    Wq, s, z = ORC.quantize_pack(W[:, cols])
    # packing of the sampled column pairs is bit-exact
    assert_bits(host(Wq_d)[:, pairs], Wq, "sampled Wq")
    assert_bits(host(s_d)[:, cols], s, "sampled scales")
    assert_bits(host(z_d)[:, pairs], z, "sampled zeros")
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
    assert_bound(y[:, cols], y_ref, bound, f"dense38 {K}x{N} M={M}")


# The canonical layout indexes in 64 bits: a matrix past 2^31 weights
# (K = 8192, N = 262160, a ragged last 256-column tile), drawn on the device
# from a seeded torch generator (8.6 GB of fp32), checked on sampled column
# pairs (the last pair included): packed bytes bit-exact, outputs within the
# bound, through the decode GEMV (M = 1) and the fp32 matrix cores (M = 4).
@pytest.mark.parametrize("M", [1, 4])
def test_canonical_past_2_31_sampled(M):
    K, N = 8192, 262160
    assert K * N > 2 ** 31
    note(f"canonical past 2^31 M={M} K={K} N={N} (sampled columns)")
    g = torch.Generator(device=DEV)
    g.manual_seed(3_000_017)
    W_d = torch.randn((K, N), generator=g, device=DEV, dtype=torch.float32).mul_(0.02)
    Wq_d, s_d, z_d = w4.w4_quantize_pack(W_d)
    pairs = sample_pairs(N, 48, seed=70)
    cols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
    pairs_t = torch.from_numpy(pairs).to(DEV)
    cols_t = torch.from_numpy(cols).to(DEV)
    W = host(W_d[:, cols_t])
    del W_d
    Wq, s, z = ORC.quantize_pack(W)
    assert_bits(host(Wq_d[:, pairs_t]), Wq, "sampled Wq past 2^31")
    assert_bits(host(s_d[:, cols_t]), s, "sampled scales past 2^31")
    assert_bits(host(z_d[:, pairs_t]), z, "sampled zeros past 2^31")
    x = synth.activations(M, K, cfg=synth.CFG_DENSE38, layer=3, slot=M, outliers=True)
    y = host(w4.w4_matmul(dev(x), Wq_d, s_d, z_d))
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
    assert_bound(y[:, cols], y_ref, bound, f"canonical past 2^31 M={M}")


def test_matmul_empty_and_bias_only():
    K, N = 64, 32
    W = synth.weights(K, N, cfg=212)
    Wq, s, z = (dev(a) for a in ORC.quantize_pack(W))
    b = synth.bias(N, cfg=212)
    y = w4.w4_matmul(torch.zeros((0, K), device=DEV), Wq, s, z, dev(b))
    assert y.shape == (0, N)
    # K == 0: the output is the bias
    e = torch.zeros((0, N // 2), dtype=torch.uint8, device=DEV)
    y = w4.w4_matmul(torch.zeros((3, 0), device=DEV), e,
                     torch.zeros((0, N), device=DEV), e, dev(b))
    assert_bits(host(y), np.stack([b, b, b]), "K=0 bias")
    y = w4.w4_matmul(torch.zeros((1, 0), device=DEV), e, torch.zeros((0, N), device=DEV), e)
    assert not host(y).any()


def test_matmul_one_hot_rows_are_dequantized_rows():
    K, N = 256, 512
    W = synth.weights(K, N, cfg=213)
    Wq, s, z = ORC.quantize_pack(W)
    What = ORC.dequantize(Wq, s, z, K, N)
    Wd = [dev(a) for a in (Wq, s, z)]
    for k in (0, 31, 32, 200, K - 1):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y = host(w4.w4_matmul(dev(x), *Wd))
        assert_bits(y[0], What[k], f"one-hot row {k}")


def test_matmul_deterministic_with_dirty_workspace():
    """Repeated calls give identical bits; the workspace needs no initial contents."""
    K, N = 3072, 9216
    W = synth.weights(K, N, cfg=214)
    x = dev(synth.activations(1, K, cfg=214))
    Wd = w4.w4_quantize_pack(dev(W))
    need = w4.w4_matmul_workspace_bytes(1, K, N)
    assert need > 0
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)   # garbage: NaN-ish floats
    y1 = host(w4.w4_matmul(x, *Wd, workspace=ws))
    y2 = host(w4.w4_matmul(x, *Wd, workspace=ws))
    assert_bits(y1, y2, "repeat")
    Wq, s, z = (host(t) for t in Wd)
    y_ref, bound = ORC.w4_matmul(host(x), Wq, s, z)
    assert_bound(y1, y_ref, bound, "dirty workspace")


def test_matmul_rejects_bad_device_pointers():
    K, N = 64, 32
    Wq, s, z = (dev(a) for a in ORC.quantize_pack(synth.weights(K, N, cfg=215)))
    x = torch.zeros((1, K + 4), device=DEV)[:, 1:K + 1]     # 4-byte offset view
    lib = w4.library()
    st = lib.w4_matmul(x.data_ptr(), 1, K, Wq.data_ptr(), s.data_ptr(), z.data_ptr(), N, None,
                       torch.empty(N, device=DEV).data_ptr(), None, 0, None)
    assert st == w4.W4_ERR_MISALIGNED


# --------------------------------------------------------------------------
# int8 head and token lookup
# --------------------------------------------------------------------------
@pytest.mark.parametrize("K,N,ldq", [(768, 50257, 50257), (768, 50257, 50272), (100, 37, 37),
                                     (100, 37, 48), (64, 300, 301), (33, 1000, 1003),
                                     # the whole-K kernel: K = 64 L, L = 4, 8, 12, 16; a
                                     # ragged last workgroup, chunks wholly past N, odd ldq;
                                     # 128-column workgroups below N = 32768, 256 above
                                     (256, 16400, 16401), (512, 16384, 16384),
                                     (768, 16385, 16387), (1024, 20000, 20016),
                                     (1024, 16513, 16513), (256, 32769, 32771),
                                     (512, 33000, 33008), (1024, 40000, 40000),
                                     (768, 32999, 32999)])
def test_head(K, N, ldq):
    note(f"head K={K} N={N} ldq={ldq}")
    cfg = synth.CFG_HEAD if (K, N) == (768, 50257) else 220
    E = synth.head_table(K, N, cfg=cfg)
    if N > 10:
        E[:, 5] = 0.0
    Q_ref, hs_ref = ORC.i8_quantize_head(E, ldq=ldq)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    Q, hs = w4.i8_quantize_head(dev(E), ldq=ldq, d_status=st)
    assert_bits(host(Q), Q_ref, f"head Q {K}x{N}/{ldq}")
    assert_bits(host(hs), hs_ref, f"head hs {K}x{N}/{ldq}")
    assert host(st)[0] == 0
    x = synth.activations(58, K, cfg=cfg, outliers=True)
    x_last = dev(x)[-1]                       # the last position only
    logits = host(w4.i8_head_logits(x_last, dev(Q_ref), dev(hs_ref)))
    ref, bound = ORC.i8_head_logits(x[-1], Q_ref, hs_ref)
    assert_bound(logits, ref, bound, f"head logits {K}x{N}/{ldq}")


def test_embed():
    K, N, ldq = 768, 50257, 50257
    E = synth.head_table(K, N)
    Q, hs = ORC.i8_quantize_head(E, ldq=ldq)
    toks = synth.tokens(58, N, cfg=synth.CFG_HEAD)
    toks[0], toks[-1] = 0, N - 1
    out = w4.i8_embed(dev(toks), dev(Q), dev(hs))
    assert_bits(host(out), ORC.i8_embed(toks, Q, hs), "embedding rows")
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    bad = np.array([3, N, -1], np.int64)
    out = host(w4.i8_embed(dev(bad), dev(Q), dev(hs), d_status=st))
    assert host(st)[0] == w4.W4_ERR_BAD_SHAPE
    assert not out[1:].any()
    assert_bits(out[0], ORC.i8_embed(bad[:1], Q, hs)[0], "valid row beside bad ids")


# --------------------------------------------------------------------------
# int8 head on the token-major table (integer MFMA)
# --------------------------------------------------------------------------
def token_major(Q, N, ldt):
    """The oracle's table [K, ldq] as rows per token, zero-padded to ldt."""
    K = Q.shape[0]
    Qt = np.zeros((N, ldt), np.int8)
    Qt[:, :K] = Q[:, :N].T
    return Qt


@pytest.mark.parametrize("K,N,ldq,ldt", [(768, 50257, 50272, 768), (64, 300, 301, 64),
                                         (100, 37, 48, 112), (33, 1000, 1003, 48)])
def test_head_prepack_bit_exact(K, N, ldq, ldt):
    note(f"head prepack K={K} N={N} ldq={ldq} ldt={ldt}")
    cfg = synth.CFG_HEAD if (K, N) == (768, 50257) else 221
    Q, hs = ORC.i8_quantize_head(synth.head_table(K, N, cfg=cfg), ldq=ldq)
    Qt = w4.i8_prepack_head(dev(Q), N, ldt=ldt)
    assert_bits(host(Qt), token_major(Q, N, ldt), f"head token-major {K}x{N}")


# The int8 head at its largest token count: the token-major table Qt [N, 768]
# one row short of 2^31 bytes (N = 2^31 / 768 - 1), and the [K, ldq] table
# past 2^31 bytes (64-bit offsets; ldq odd or a multiple of 16).  The fp32
# table (8.6 GB) is drawn on the device from a seeded torch generator; the
# quantizer's sampled bytes and scales are bit-exact, both heads' sampled
# logits within the bound (the last 20 tokens always among the samples).
@pytest.mark.parametrize("pad", [16, 23])
def test_head_index_limit_sampled(pad):
    K, N = 768, 2 ** 31 // 768 - 1
    ldq = N + pad
    assert N * K < 2 ** 31 and K * ldq > 2 ** 31
    note(f"head index limit K={K} N={N} ldq={ldq} (sampled tokens)")
    g = torch.Generator(device=DEV)
    g.manual_seed(2_000_003 + pad)
    E_d = torch.randn((K, N), generator=g, device=DEV, dtype=torch.float32).mul_(0.02)
    Q_d, hs_d = w4.i8_quantize_head(E_d, ldq=ldq)
    rng = np.random.default_rng(60 + pad)
    idx = np.unique(np.concatenate([rng.choice(N, 76, replace=False),
                                    np.arange(N - 20, N), [0]])).astype(np.int64)
    idx_t = torch.from_numpy(idx).to(DEV)
    E = host(E_d[:, idx_t])
    del E_d
    Q, hs = ORC.i8_quantize_head(E, ldq=len(idx))
    assert_bits(host(Q_d[:, idx_t]), Q, "sampled head codes at the index limit")
    assert_bits(host(hs_d[idx_t]), hs, "sampled head scales at the index limit")
    x = synth.activations(58, K, cfg=synth.CFG_HEAD, outliers=True)[-1]
    ref, bound = ORC.i8_head_logits(x, Q, hs)
    logits = host(w4.i8_head_logits(dev(x), Q_d, hs_d))
    assert_bound(logits[idx], ref, bound, f"[K, ldq] head at the index limit, ldq={ldq}")
    Qt = w4.i8_prepack_head(Q_d, N, ldt=K)
    del Q_d
    assert_bits(host(Qt[idx_t]), np.ascontiguousarray(Q.T), "sampled token-major rows")
    logits_t = host(w4.i8_head_logits_kmajor(dev(x), Qt, hs_d, K))
    assert_bound(logits_t[idx], ref, bound, "token-major head at the index limit")


def head_kmajor_case(K, N, ldt, x, label):
    cfg = synth.CFG_HEAD if (K, N) == (768, 50257) else 222
    E = synth.head_table(K, N, cfg=cfg)
    if N > 10:
        E[:, 5] = 0.0
    Q, hs = ORC.i8_quantize_head(E, ldq=N)
    Qt = dev(token_major(Q, N, ldt))
    logits = host(w4.i8_head_logits_kmajor(dev(x), Qt, dev(hs), K))
    ref, bound = ORC.i8_head_logits(x, Q, hs)
    assert_bound(logits, ref, bound, label)


@pytest.mark.parametrize("K,N,ldt", [(768, 50257, 768), (768, 50257, 784), (64, 300, 64),
                                     (128, 37, 144), (256, 1000, 256), (512, 77, 512),
                                     (1024, 515, 1024), (2048, 130, 2048), (8192, 70, 8192),
                                     (48, 100, 48), (784, 333, 800), (1040, 65, 1040)])
def test_head_kmajor(K, N, ldt):
    note(f"head kmajor K={K} N={N} ldt={ldt}")
    cfg = synth.CFG_HEAD if (K, N) == (768, 50257) else 223
    x = synth.activations(58, K, cfg=cfg, outliers=True)[-1]
    head_kmajor_case(K, N, ldt, x, f"head kmajor {K}x{N}/{ldt}")


def test_head_kmajor_special_inputs():
    K, N = 768, 3000
    cases = {
        "one-hot": np.eye(1, K, 17, dtype=np.float32)[0],
        "zeros": np.zeros(K, np.float32),
        "tiny": synth.activations(1, K, cfg=224)[0] * np.float32(1e-30),
        "huge": synth.activations(1, K, cfg=225)[0] * np.float32(1e30),
        "negative max": -np.abs(synth.activations(1, K, cfg=226)[0]),
    }
    spread = synth.activations(1, K, cfg=227)[0]
    spread[::7] *= np.float32(1000.0)          # three decades between entries
    spread[3::7] *= np.float32(1e-3)
    cases["spread"] = spread
    for name, x in cases.items():
        note(f"head kmajor x={name}")
        head_kmajor_case(K, N, K, x.astype(np.float32), f"head kmajor x={name}")


@pytest.mark.parametrize("factor", [1e5, 1e7, 1e12])
def test_head_kmajor_isolated_outlier(factor):
    """One activation far above the rest of its 64-value segment, on a code
    row that is zero for many tokens: the rest keeps its own precision."""
    K, N = 768, 3000
    E = synth.head_table(K, N, cfg=231)
    E[100, : N // 2] = 0.0
    Q, hs = ORC.i8_quantize_head(E, ldq=N)
    x = synth.activations(1, K, cfg=231)[0]
    x[100] *= np.float32(factor)
    logits = host(w4.i8_head_logits_kmajor(dev(x), dev(token_major(Q, N, K)), dev(hs), K))
    ref, bound = ORC.i8_head_logits(x, Q, hs)
    assert_bound(logits, ref, bound, f"head kmajor outlier x{factor:g}")
    xs = synth.activations(5, K, cfg=232)
    xs[:, 100] *= np.float32(factor)
    got = host(w4.i8_head_logits_rows(dev(xs), dev(token_major(Q, N, K)), dev(hs)))
    for m in range(5):
        ref, bound = ORC.i8_head_logits(xs[m], Q, hs)
        assert_bound(got[m], ref, bound, f"head rows outlier x{factor:g} row {m}")


@pytest.mark.parametrize("ldq", [32771, 32784])
def test_head_whole_special_inputs(ldq):
    """The [K, ldq] table's one-launch kernel (K = 768, 256-column workgroups)
    on special activations: exact zeros, tiny and huge magnitudes, decades of
    spread, and one entry 1e12 above the rest on a code row that is zero for
    half the tokens."""
    K, N = 768, 32769
    E = synth.head_table(K, N, cfg=233)
    E[100, : N // 2] = 0.0
    Q, hs = ORC.i8_quantize_head(E, ldq=ldq)
    base = synth.activations(1, K, cfg=234)[0]
    spread = base.copy()
    spread[::7] *= np.float32(1000.0)
    spread[3::7] *= np.float32(1e-3)
    outlier = base.copy()
    outlier[100] *= np.float32(1e12)
    cases = {"zeros": np.zeros(K, np.float32), "tiny": base * np.float32(1e-30),
             "huge": base * np.float32(1e30), "spread": spread, "isolated outlier": outlier,
             "one-hot": np.eye(1, K, 17, dtype=np.float32)[0]}
    Qd, hsd = dev(Q), dev(hs)
    for name, x in cases.items():
        note(f"head whole ldq={ldq} x={name}")
        logits = host(w4.i8_head_logits(dev(x.astype(np.float32)), Qd, hsd))
        ref, bound = ORC.i8_head_logits(x.astype(np.float32), Q, hs)
        assert_bound(logits, ref, bound, f"head whole ldq={ldq} x={name}")


def test_head_kmajor_nonfinite_gives_nan():
    K, N = 128, 50
    Q, hs = ORC.i8_quantize_head(synth.head_table(K, N, cfg=228), ldq=N)
    x = synth.activations(1, K, cfg=228)[0]
    x[9] = np.inf
    logits = host(w4.i8_head_logits_kmajor(dev(x), dev(token_major(Q, N, K)), dev(hs), K))
    assert np.isnan(logits).all()


@pytest.mark.parametrize("M,K,N,ldt", [(58, 768, 50257, 768), (1, 768, 50257, 784), (3, 768, 4099, 768),
                                       (5, 64, 300, 64), (9, 128, 37, 144), (6, 2048, 130, 2048),
                                       (17, 512, 1000, 512), (4, 1024, 515, 1024),
                                       (130, 64, 500, 64), (65, 64, 300, 64), (33, 48, 70, 48),
                                       (3, 4096, 90, 4096)])
def test_head_rows(M, K, N, ldt):
    """Full-sequence logits: every row of x against the oracle's head."""
    note(f"head rows M={M} K={K} N={N} ldt={ldt}")
    cfg = synth.CFG_HEAD if (K, N) == (768, 50257) else 229
    E = synth.head_table(K, N, cfg=cfg)
    if N > 10:
        E[:, 5] = 0.0
    Q, hs = ORC.i8_quantize_head(E, ldq=N)
    x = synth.activations(M, K, cfg=cfg, outliers=True)
    got = host(w4.i8_head_logits_rows(dev(x), dev(token_major(Q, N, ldt)), dev(hs)))
    refs = [ORC.i8_head_logits(x[m], Q, hs) for m in range(M)]
    ref = np.stack([r[0] for r in refs])
    bound = np.stack([r[1] for r in refs])
    assert_bound(got, ref, bound, f"head rows {M}x{K}x{N}")


# A long prefill through the full-sequence head: 1024 rows (and a ragged
# 1000) of the GPT-2 head, checked against the oracle on sampled tokens (the
# last 20 among them) for every row.
@pytest.mark.parametrize("M", [1024, 1000])
def test_head_rows_long_sequence_sampled(M):
    K, N = 768, 50257
    note(f"head rows long sequence M={M} K={K} N={N} (sampled tokens)")
    Q, hs = ORC.i8_quantize_head(synth.head_table(K, N, cfg=synth.CFG_HEAD), ldq=N)
    x = synth.activations(M, K, cfg=291, outliers=True)
    got = host(w4.i8_head_logits_rows(dev(x), dev(token_major(Q, N, K)), dev(hs)))
    assert got.shape == (M, N)
    rng = np.random.default_rng(291)
    idx = np.unique(np.concatenate([rng.choice(N, 60, replace=False), np.arange(N - 20, N), [0]]))
    Qs, hss = np.ascontiguousarray(Q[:, idx]), np.ascontiguousarray(hs[idx])
    for m in range(M):
        ref, bound = ORC.i8_head_logits(x[m], Qs, hss)
        assert_bound(got[m, idx], ref, bound, f"head rows long sequence row {m}")


def test_head_rows_special_rows():
    K, N, M = 768, 2000, 6
    Q, hs = ORC.i8_quantize_head(synth.head_table(K, N, cfg=230), ldq=N)
    x = synth.activations(M, K, cfg=230)
    x[1] = 0.0                                   # all-zero row
    x[2] *= np.float32(1e-30)                    # tiny row beside normal ones
    x[3, 11] = np.inf                            # non-finite row: NaN logits, others unaffected
    x[4] *= np.float32(1e30)
    got = host(w4.i8_head_logits_rows(dev(x), dev(token_major(Q, N, K)), dev(hs)))
    assert np.isnan(got[3]).all()
    for m in (0, 1, 2, 4, 5):
        ref, bound = ORC.i8_head_logits(x[m], Q, hs)
        assert_bound(got[m], ref, bound, f"head rows special row {m}")


def test_embed_kmajor():
    K, N = 768, 50257
    E = synth.head_table(K, N)
    Q, hs = ORC.i8_quantize_head(E, ldq=N)
    Qt = dev(token_major(Q, N, 768))
    toks = synth.tokens(58, N, cfg=synth.CFG_HEAD)
    toks[0], toks[-1] = 0, N - 1
    out = w4.i8_embed_kmajor(dev(toks), Qt, dev(hs), K)
    assert_bits(host(out), ORC.i8_embed(toks, Q, hs), "token-major embedding rows")
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    bad = np.array([3, N, -1], np.int64)
    out = host(w4.i8_embed_kmajor(dev(bad), Qt, dev(hs), K, d_status=st))
    assert host(st)[0] == w4.W4_ERR_BAD_SHAPE
    assert not out[1:].any()


# --------------------------------------------------------------------------
# K-major (prepacked) layout and its GEMV
# --------------------------------------------------------------------------
@pytest.mark.parametrize("K,N", [(64, 34), (768, 2304), (3072, 768), (192, 530)])
def test_prepack_kmajor_bit_exact(K, N):
    note(f"prepack_kmajor K={K} N={N}")
    W = mixed_weights(K, N, cfg=230)
    Wq, s, z = ORC.quantize_pack(W)
    ref = ORC.prepack_kmajor(Wq, s, z, K, N)
    got = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    for name, a, b in zip(("Pq", "Ps", "Pz"), got, ref):
        assert_bits(host(a), b, f"{name} {K}x{N}")


# (3072, 3080): every lane owns one block and the matrix fills the chip, so
# M = 1 and 2 take the whole-run activation loads, with a ragged last
# workgroup (3080 is not a multiple of the 12 columns per workgroup)
KMAJOR_SHAPES = [(64, 16), (768, 768), (768, 2304), (768, 3072), (3072, 768), (1024, 1008),
                 (192, 530), (8192, 512), (128, 2), (4096, 4112), (320, 96), (3072, 3080)]


@pytest.mark.parametrize("K,N", KMAJOR_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16])
def test_kmajor_matmul(M, K, N):
    note(f"kmajor M={M} K={K} N={N}")
    W = mixed_weights(K, N, cfg=231)
    x = synth.activations(M, K, cfg=231, slot=M, outliers=True)
    b = synth.bias(N, cfg=231)
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z, b)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b)))
    assert_bound(y, y_ref, bound, f"kmajor M={M} {K}x{N}")


X3_SHAPES = [(128, 16), (768, 768), (768, 2304), (768, 3072), (3072, 768), (1024, 1008),
             (256, 530), (8192, 512), (128, 2), (640, 4112), (384, 96), (3072, 3072)]


@pytest.mark.parametrize("K,N", X3_SHAPES)
@pytest.mark.parametrize("M", [3, 4, 5, 16, 17, 58, 64, 65, 130])
def test_kmajor_matrix_cores(M, K, N):
    """M >= 3 on the bf16 matrix cores (split-K, ragged N, partial m-tiles)."""
    note(f"kmajor x3 M={M} K={K} N={N} ws={w4.w4_matmul_kmajor_workspace_bytes(M, K, N)}")
    W = mixed_weights(K, N, cfg=232)
    x = synth.activations(M, K, cfg=232, slot=M, outliers=True)
    b = synth.bias(N, cfg=232)
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z, b)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b)))
    assert_bound(y, y_ref, bound, f"kmajor x3 M={M} {K}x{N}")


# seeded draws over the K-major plan's corners: K a multiple of 64 (the GEMV,
# whole-run activation loads or not, one or several blocks per lane) or of
# 128 (the matrix cores: the fp16 kernel up to 16 rows, bf16 beyond, with and
# without split-K), N even and ragged, M from 1 to 70
def _random_kmajor_cases(n, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        K = int(g.choice([64, 128, 192, 256, 384, 640, 768, 1024, 1536, 2048, 3072, 4096]))
        N = 2 * int(g.integers(1, 2600))
        M = int(g.choice([1, 1, 2, 2, 3, 4, 5, 8, 12, 16, 17, 33, 70]))
        out.append((M, K, N))
    return out


@pytest.mark.parametrize("M,K,N", _random_kmajor_cases(24))
def test_kmajor_random_shapes(M, K, N):
    note(f"kmajor random M={M} K={K} N={N}")
    W = mixed_weights(K, N, cfg=236)
    x = synth.activations(M, K, cfg=236, slot=M, outliers=True)
    b = synth.bias(N, cfg=236)
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z, b)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b)))
    assert_bound(y, y_ref, bound, f"kmajor random M={M} {K}x{N}")


def _random_epilogue_cases(n, seed=777):
    acts = ("none", "gelu", "swiglu")
    return [(M, K, N, acts[i % 3], (i // 3) % 2 == 1)
            for i, (M, K, N) in enumerate(_random_kmajor_cases(n, seed=seed))]


@pytest.mark.parametrize("M,K,N,act,res", _random_epilogue_cases(48))
def test_kmajor_random_shapes_epilogue(M, K, N, act, res):
    note(f"kmajor random epilogue M={M} K={K} N={N} act={act} residual={res}")
    W = mixed_weights(K, N, cfg=237)
    x = synth.activations(M, K, cfg=237, slot=M, outliers=True)
    b = synth.bias(N, cfg=237)
    nout = N // 2 if act == "swiglu" else N
    r = synth.activations(M, nout, cfg=238, slot=M) if res else None
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul_ep(x, Wq, s, z, b, r, act=act)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b), act=act,
                                 residual=None if r is None else dev(r)))
    assert y.shape == (M, nout)
    assert_bound(y, y_ref, bound, f"kmajor random epilogue {act} M={M} {K}x{N}")


def test_kmajor_matrix_cores_special_inputs():
    K, N, M = 768, 2304, 16
    W = mixed_weights(K, N, cfg=233)
    Wq, s, z = ORC.quantize_pack(W)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    base = synth.activations(M, K, cfg=233)
    cases = {"zeros": np.zeros((M, K), np.float32),
             "one-hot rows": np.eye(M, K, 5, dtype=np.float32),
             "tiny": base * np.float32(1e-30),
             "huge": base * np.float32(1e30),
             "spread": base * np.where(np.arange(K) % 3 == 0, 1e3, 1e-3).astype(np.float32),
             # rows 10^-30 .. 10^30 apart in one 16-row tile: each row keeps
             # its own scale on the M <= 16 path
             "row magnitudes": base * np.logspace(-30, 30, M, dtype=np.float64)
                                        .astype(np.float32)[:, None]}
    for name, x in cases.items():
        y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
        y = host(w4.w4_matmul_kmajor(dev(x), *P))
        assert_bound(y, y_ref, bound, f"kmajor x3 x={name}")


@pytest.mark.parametrize("M", [3, 4, 16, 17, 58])
@pytest.mark.parametrize("factor", [1e5, 1e7, 1e12])
def test_kmajor_matrix_cores_isolated_outlier(M, factor):
    """One activation far above the rest of its 512-wide K range, sitting on
    a row of zero weights (q = z, so it adds nothing to the bound): every
    other product must keep its own precision."""
    K, N = 1024, 768
    note(f"kmajor outlier M={M} factor={factor:g}")
    W = mixed_weights(K, N, cfg=239)
    W[300, :] = 0.0
    W[700, 5:] = 0.0
    x = synth.activations(M, K, cfg=239, slot=M)
    x[:, 300] *= np.float32(factor)
    x[M // 2, 700] = np.float32(factor)
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y = host(w4.w4_matmul_kmajor(dev(x), *P))
    assert_bound(y, y_ref, bound, f"kmajor outlier x{factor:g} M={M}")


@pytest.mark.parametrize("M", [1, 2, 4, 16, 58])
def test_large_scales_do_not_overflow(M):
    """Weights near 1e33 (block scales above 2^104) on every matmul path."""
    K, N = 768, 512
    note(f"large scales M={M}")
    W = synth.weights(K, N, cfg=240) * np.float32(5e34)
    assert np.all(np.isfinite(W))
    x = synth.activations(M, K, cfg=240, slot=M)
    Wq, s, z = ORC.quantize_pack(W)
    assert float(np.max(s)) > 2.0 ** 104
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
    assert np.all(np.isfinite(y_ref))
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    assert_bound(host(w4.w4_matmul_kmajor(dev(x), *P)), y_ref, bound, f"large scales kmajor M={M}")
    assert_bound(host(w4.w4_matmul(dev(x), dev(Wq), dev(s), dev(z))), y_ref, bound,
                 f"large scales canonical M={M}")


def test_kmajor_matrix_cores_deterministic_with_dirty_workspace():
    K, N, M = 3072, 256, 16   # 16 column tiles: the split-K kernel
    W = mixed_weights(K, N, cfg=234)
    P = w4.w4_prepack_kmajor(*w4.w4_quantize_pack(dev(W)))
    x = dev(synth.activations(M, K, cfg=234))
    need = w4.w4_matmul_kmajor_workspace_bytes(M, K, N)
    assert need > 0
    ws = torch.full((need + 256,), 0x7F, dtype=torch.uint8, device=DEV)
    y1 = host(w4.w4_matmul_kmajor(x, *P, workspace=ws))
    ws.fill_(0xFF)
    y2 = host(w4.w4_matmul_kmajor(x, *P, workspace=ws))
    assert_bits(y1, y2, "x3 repeat")


# The whole-K matrix-core kernel (3 <= M <= 16 rows, N >= 497: one
# workgroup per 16 columns, or 32 from 5 rows where N >= 16353, over all of
# K, no workspace).  K = 128 and 256 leave waves of a workgroup with no
# quads; 2050, 3080, 2344 and 16400 are ragged N (16400: two column tiles per
# wave, a half-empty last workgroup); 8192 gives 8 quads per wave; M = 3,
# 5..8 and 12 exercise the row padding of the 4-, 8- and 16-row images.
WHOLE_K_SHAPES = [(128, 2048), (256, 2050), (384, 2344), (3072, 3080), (8192, 2064),
                  (128, 16400)]


@pytest.mark.parametrize("K,N", WHOLE_K_SHAPES)
@pytest.mark.parametrize("M", [3, 4, 5, 6, 8, 12, 16])
def test_kmajor_whole_k_kernel(M, K, N):
    assert w4.w4_matmul_kmajor_workspace_bytes(M, K, N) == 0
    note(f"kmajor whole-K M={M} K={K} N={N}")
    W = mixed_weights(K, N, cfg=242)
    x = synth.activations(M, K, cfg=242, slot=M, outliers=True)
    b = synth.bias(N, cfg=242)
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z, b)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y1 = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b)))
    assert_bound(y1, y_ref, bound, f"kmajor whole-K M={M} {K}x{N}")
    y2 = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b)))
    assert_bits(y1, y2, "whole-K repeat")


@pytest.mark.parametrize("act,res", [("gelu", False), ("swiglu", True), ("none", True)])
@pytest.mark.parametrize("M,K,N", [(4, 384, 2344), (7, 384, 2344), (12, 128, 16400),
                                   (4, 3072, 2064), (3, 8192, 2048)])
def test_kmajor_whole_k_epilogue(M, K, N, act, res):
    note(f"kmajor whole-K epilogue M={M} act={act} residual={res}")
    W = mixed_weights(K, N, cfg=243)
    x = synth.activations(M, K, cfg=243, slot=M, outliers=True)
    b = synth.bias(N, cfg=243)
    nout = N // 2 if act == "swiglu" else N
    r = synth.activations(M, nout, cfg=244, slot=M) if res else None
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul_ep(x, Wq, s, z, b, r, act=act)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b), act=act,
                                 residual=None if r is None else dev(r)))
    assert_bound(y, y_ref, bound, f"kmajor whole-K epilogue {act} M={M}")


@pytest.mark.parametrize("M,K", [(3, 768), (8, 768), (4, 3072)])
def test_kmajor_whole_k_special_inputs(M, K):
    N = 2304
    W = mixed_weights(K, N, cfg=245)
    W[300, :] = 0.0
    Wq, s, z = ORC.quantize_pack(W)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    base = synth.activations(M, K, cfg=245)
    outlier = base.copy()
    outlier[:, 300] *= np.float32(1e12)   # on a row of zero weights
    cases = {"zeros": np.zeros((M, K), np.float32),
             "tiny": base * np.float32(1e-30),
             "huge": base * np.float32(1e30),
             "subnormal": base * np.float32(1e-40),
             "spread": base * np.where(np.arange(K) % 3 == 0, 1e3, 1e-3).astype(np.float32),
             "row magnitudes": base * np.logspace(-30, 30, M, dtype=np.float64)
                                        .astype(np.float32)[:, None],
             "isolated outlier": outlier}
    for name, x in cases.items():
        y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
        y = host(w4.w4_matmul_kmajor(dev(x), *P))
        assert_bound(y, y_ref, bound, f"kmajor whole-K x={name} M={M}")


def test_kmajor_whole_k_large_scales_and_f16():
    K, N, M = 768, 2048, 4
    W = synth.weights(K, N, cfg=246) * np.float32(5e34)
    x = synth.activations(M, K, cfg=246, slot=M)
    Wq, s, z = ORC.quantize_pack(W)
    assert float(np.max(s)) > 2.0 ** 104
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    assert_bound(host(w4.w4_matmul_kmajor(dev(x), *P)), y_ref, bound, "whole-K large scales")
    W = mixed_weights_f16(K, N, cfg=247)
    b = synth.bias(N, cfg=247)
    Wq, s16, z = ORC.quantize_pack_f16(W)
    y_ref, bound = ORC.w4h_matmul(x, Wq, s16, z, b)
    s_dev = torch.from_numpy(s16.view(np.float16)).to(DEV)
    P = w4.w4h_prepack_kmajor(dev(Wq), s_dev, dev(z))
    assert_bound(host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b))), y_ref, bound,
                 "whole-K binary16 scales")


@pytest.mark.parametrize("slot", range(4))
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_dense38_kmajor_full_size_sampled(slot, M):
    """Full-size 3.8B-dense shapes on the K-major path the benchmark times
    (M = 1, 4 and 16), and at 2 rows (the two-row GEMV) and 8 (the whole-K
    kernel's 8-row blocks)."""
    K, N = synth.DENSE38_SHAPES[slot]
    note(f"dense38 kmajor slot {slot} M={M} K={K} N={N} (sampled columns)")
    W = synth.weights(K, N, cfg=synth.CFG_DENSE38, layer=0, slot=slot)
    x = synth.activations(M, K, cfg=synth.CFG_DENSE38, layer=0, slot=slot, outliers=True)
    P = w4.w4_prepack_kmajor(*w4.w4_quantize_pack(dev(W)))
    y = host(w4.w4_matmul_kmajor(dev(x), *P))
    pairs = sample_pairs(N, 48, seed=10 + slot)
    cols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
    Wq, s, z = ORC.quantize_pack(W[:, cols])
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
    assert_bound(y[:, cols], y_ref, bound, f"dense38 kmajor {K}x{N} M={M}")


@pytest.mark.parametrize("slot", range(4))
@pytest.mark.parametrize("M", [1, 4])
def test_f16_dense38_full_size_sampled(slot, M):
    """The fp16-scale format at the full 3.8B-dense shapes the benchmark times:
    the GPU quantizer's sampled bytes bit-exact, the matmul within the bound."""
    K, N = synth.DENSE38_SHAPES[slot]
    note(f"f16 dense38 slot {slot} M={M} K={K} N={N} (sampled columns)")
    W = synth.weights(K, N, cfg=synth.CFG_DENSE38, layer=0, slot=slot)
    x = synth.activations(M, K, cfg=synth.CFG_DENSE38, layer=0, slot=slot, outliers=True)
    Wq_d, s_d, z_d = w4.w4h_quantize_pack(dev(W))
    y = host(w4.w4_matmul_kmajor(dev(x), *w4.w4h_prepack_kmajor(Wq_d, s_d, z_d)))
    pairs = sample_pairs(N, 48, seed=30 + slot)
    cols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
    Wq, s16, z = ORC.quantize_pack_f16(W[:, cols])
    assert_bits(host(Wq_d)[:, pairs], Wq, "sampled Wq (fp16 scales)")
    assert_bits(f16_bits(s_d)[:, cols], s16, "sampled fp16 scales")
    assert_bits(host(z_d)[:, pairs], z, "sampled zeros (fp16 scales)")
    y_ref, bound = ORC.w4h_matmul(x, Wq, s16, z)
    assert_bound(y[:, cols], y_ref, bound, f"f16 dense38 {K}x{N} M={M}")


# The benchmark's fused-epilogue pass at full size: SwiGLU on the gate+up
# matrix (interleaved gate/up columns, half as many outputs), the residual
# added in place on the out- and down-projections.
@pytest.mark.parametrize("slot,act,res", [(2, "swiglu", False), (1, "none", True),
                                          (3, "none", True)])
def test_ep_dense38_full_size_sampled(slot, act, res):
    K, N = synth.DENSE38_SHAPES[slot]
    note(f"epilogue dense38 slot {slot} act={act} residual={res} K={K} N={N} (sampled columns)")
    W = synth.weights(K, N, cfg=synth.CFG_DENSE38, layer=0, slot=slot)
    x = synth.activations(1, K, cfg=synth.CFG_DENSE38, layer=0, slot=slot, outliers=True)
    P = w4.w4_prepack_kmajor(*w4.w4_quantize_pack(dev(W)))
    pairs = sample_pairs(N, 48, seed=40 + slot)
    cols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
    if act == "swiglu":
        y = host(w4.w4_matmul_kmajor(dev(x), *P, act="swiglu"))
        assert y.shape == (1, N // 2)
        r_s, y_s = None, y[:, pairs]
    else:
        r = synth.activations(1, N, cfg=synth.CFG_DENSE38, layer=1, slot=slot)
        yr = dev(r)
        w4.w4_matmul_kmajor(dev(x), *P, residual=yr, out=yr)
        r_s, y_s = r[:, cols], host(yr)[:, cols]
    Wq, s, z = ORC.quantize_pack(W[:, cols])
    y_ref, bound = ORC.w4_matmul_ep(x, Wq, s, z, None, r_s, act=act)
    assert_bound(y_s, y_ref, bound, f"epilogue dense38 {act} {K}x{N}")


# At the 32-bit indexing limit of the K-major kernels: K N = 2^31 - 131072
# (K = 8192, N = 262128).  The weights (8.6 GB of fp32) are drawn on the
# device from a seeded torch generator, quantized and prepacked on the GPU,
# and checked on sampled column pairs, the last pair included: the sampled
# bytes bit-exact, the outputs within the bound.
@pytest.mark.parametrize("M", [1, 4, 16])
def test_kmajor_index_limit_sampled(M):
    K, N = 8192, 262128
    assert K * N < 2 ** 31 and K * (N + 16) >= 2 ** 31 - 2 ** 16
    note(f"kmajor index limit M={M} K={K} N={N} (sampled columns)")
    g = torch.Generator(device=DEV)
    g.manual_seed(1_000_003)
    W_d = torch.randn((K, N), generator=g, device=DEV, dtype=torch.float32).mul_(0.02)
    Wq_d, s_d, z_d = w4.w4_quantize_pack(W_d)
    pairs = sample_pairs(N, 48, seed=50)
    cols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
    pairs_t = torch.from_numpy(pairs).to(DEV)
    cols_t = torch.from_numpy(cols).to(DEV)
    W = host(W_d[:, cols_t])
    del W_d
    Wq, s, z = ORC.quantize_pack(W)
    assert_bits(host(Wq_d[:, pairs_t]), Wq, "sampled Wq at the index limit")
    assert_bits(host(s_d[:, cols_t]), s, "sampled scales at the index limit")
    assert_bits(host(z_d[:, pairs_t]), z, "sampled zeros at the index limit")
    P = w4.w4_prepack_kmajor(Wq_d, s_d, z_d)
    del Wq_d, s_d, z_d
    x = synth.activations(M, K, cfg=synth.CFG_DENSE38, layer=2, slot=M, outliers=True)
    y = host(w4.w4_matmul_kmajor(dev(x), *P))
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
    assert_bound(y[:, cols], y_ref, bound, f"kmajor index limit M={M}")


# The fp16-scale and group-64 affine formats at the same indexing limit
# (M = 1, the decode GEMV's instantiations for those formats).
@pytest.mark.parametrize("fmt", ["fp16 scales", "group-64 affine"])
def test_formats_index_limit_sampled(fmt):
    K, N = 8192, 262128
    note(f"{fmt} index limit K={K} N={N} (sampled columns)")
    g = torch.Generator(device=DEV)
    g.manual_seed(4_000_037)
    W_d = torch.randn((K, N), generator=g, device=DEV, dtype=torch.float32).mul_(0.02)
    pairs = sample_pairs(N, 48, seed=80)
    cols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
    W = host(W_d[:, torch.from_numpy(cols).to(DEV)])
    x = synth.activations(1, K, cfg=synth.CFG_DENSE38, layer=4, slot=0, outliers=True)
    if fmt == "fp16 scales":
        P = w4.w4h_prepack_kmajor(*w4.w4h_quantize_pack(W_d))
        del W_d
        y = host(w4.w4_matmul_kmajor(dev(x), *P))
        Wq, s16, z = ORC.quantize_pack_f16(W)
        y_ref, bound = ORC.w4h_matmul(x, Wq, s16, z)
    else:
        P = w4.w4g_prepack_kmajor(*w4.w4g_quantize_pack(W_d))
        del W_d
        y = host(w4.w4g_matmul_kmajor(dev(x), *P))
        Wq, sg, mg = ORC.quantize_pack_g64(W)
        y_ref, bound = ORC.w4g_matmul(x, Wq, sg, mg)
    assert_bound(y[:, cols], y_ref, bound, f"{fmt} at the index limit")


# A long prefill on the K-major matrix cores: 1024 rows (and a ragged 1000)
# of the 3.8B QKV shape, sampled columns checked for every row.
@pytest.mark.parametrize("M", [1024, 1000])
def test_kmajor_long_prefill_sampled(M):
    K, N = synth.DENSE38_SHAPES[0]
    note(f"kmajor long prefill M={M} K={K} N={N} ws={w4.w4_matmul_kmajor_workspace_bytes(M, K, N)}")
    W = synth.weights(K, N, cfg=synth.CFG_DENSE38, layer=5, slot=0)
    x = synth.activations(M, K, cfg=synth.CFG_DENSE38, layer=5, slot=0, outliers=True)
    P = w4.w4_prepack_kmajor(*w4.w4_quantize_pack(dev(W)))
    y = host(w4.w4_matmul_kmajor(dev(x), *P))
    pairs = sample_pairs(N, 32, seed=90)
    cols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
    Wq, s, z = ORC.quantize_pack(W[:, cols])
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z)
    assert_bound(y[:, cols], y_ref, bound, f"kmajor long prefill M={M}")


def test_kmajor_rejects_bad_shapes():
    lib = w4.library()
    A = torch.zeros(64, dtype=torch.uint8, device=DEV).data_ptr()
    assert lib.w4_matmul_kmajor(A, 1, 96, A, A, A, 16, None, A, None, 0, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.w4_prepack_kmajor(A, A, A, 96, 16, A, A, A, None) == w4.W4_ERR_BAD_SHAPE


# --------------------------------------------------------------------------
# fp16-scale variant
# --------------------------------------------------------------------------
def f16_bits(t):
    return host(t).view(np.uint16)


def mixed_weights_f16(K, N, cfg):
    W = mixed_weights(K, N, cfg)
    g = np.random.default_rng(cfg)
    if N >= 12:
        W[:32, 8] = (g.standard_normal(32) * 1e-8).astype(np.float32)   # scale rounds to 0
        W[:32, 9] = (g.standard_normal(32) * 3e-5).astype(np.float32)   # subnormal binary16 scale
        W[:32, 10] = (g.standard_normal(32) * 9e4).astype(np.float32)   # scale near the top
    return W


@pytest.mark.parametrize("K,N", [(64, 16), (768, 2304), (3072, 768), (192, 530)])
def test_f16_quantize_pack_bit_exact(K, N):
    note(f"f16 quantize K={K} N={N}")
    W = mixed_weights_f16(K, N, cfg=240)
    Wq_r, s_r, z_r = ORC.quantize_pack_f16(W)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    Wq, s, z = w4.w4h_quantize_pack(dev(W), d_status=st)
    assert_bits(host(Wq), Wq_r, f"f16 Wq {K}x{N}")
    assert_bits(f16_bits(s), s_r, f"f16 scales {K}x{N}")
    assert_bits(host(z), z_r, f"f16 zeros {K}x{N}")
    assert host(st)[0] == 0
    W_hat = host(w4.w4h_dequantize(Wq, s, z))
    assert_bits(W_hat, ORC.dequantize(Wq_r, ORC.f16_to_f32(s_r), z_r, K, N), f"f16 W_hat {K}x{N}")
    P = w4.w4h_prepack_kmajor(Wq, s, z)
    if K % 64 == 0:
        Pq_r, Ps_r, Pz_r = ORC.prepack_kmajor_f16(Wq_r, s_r, z_r, K, N)
        assert_bits(host(P[0]), Pq_r, "f16 Pq")
        assert_bits(f16_bits(P[1]), Ps_r, "f16 Ps")
        assert_bits(host(P[2]), Pz_r, "f16 Pz")


def test_f16_scale_overflow_sets_status():
    W = np.zeros((32, 4), np.float32)
    W[0, 1] = 1e6                       # (hi - lo) / 15 > 65504
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    w4.w4h_quantize_pack(dev(W), d_status=st)
    assert host(st)[0] == w4.W4_ERR_NONFINITE


@pytest.mark.parametrize("K,N", [(768, 2304), (3072, 768), (128, 530), (8192, 512), (640, 96)])
@pytest.mark.parametrize("M", [1, 2, 4, 16, 58])
def test_f16_matmul_kmajor(M, K, N):
    note(f"f16 kmajor M={M} K={K} N={N}")
    W = mixed_weights_f16(K, N, cfg=241)
    x = synth.activations(M, K, cfg=241, slot=M, outliers=True)
    b = synth.bias(N, cfg=241)
    Wq, s16, z = ORC.quantize_pack_f16(W)
    y_ref, bound = ORC.w4h_matmul(x, Wq, s16, z, b)
    s_dev = torch.from_numpy(s16.view(np.float16)).to(DEV)
    P = w4.w4h_prepack_kmajor(dev(Wq), s_dev, dev(z))
    y = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b)))
    assert_bound(y, y_ref, bound, f"f16 kmajor M={M} {K}x{N}")


# K = 3072 and N >= 3072 at M = 1 and 2: two column slots per workgroup read
# the activations once and share them through LDS.  At M = 1 4096 columns
# take 4 passes (512 workgroups, no ragged tail), 3078 and 3080 take 3 (3080
# with a ragged last workgroup); at M = 2 4096 take 4 passes and 3078 and
# 3080 take 2 (3078 ragged).  K = 8192 keeps one column slot per workgroup.
# Every scale format and epilogue goes through these modes here.
@pytest.mark.parametrize("K,N", [(3072, 3078), (3072, 3080), (3072, 4096), (8192, 3080)])
@pytest.mark.parametrize("variant", ["plain", "f16", "g64", "gelu", "swiglu+res"])
@pytest.mark.parametrize("M", [1, 2])
def test_kmajor_shared_activations(M, variant, K, N):
    note(f"shared activations {variant} M={M} K={K} N={N}")
    W = mixed_weights_f16(K, N, cfg=271) if variant == "f16" else mixed_weights(K, N, cfg=271)
    x = synth.activations(M, K, cfg=271, slot=M, outliers=True)
    b = synth.bias(N, cfg=271)
    if variant == "f16":
        Wq, s16, z = ORC.quantize_pack_f16(W)
        y_ref, bound = ORC.w4h_matmul(x, Wq, s16, z, b)
        s_dev = torch.from_numpy(s16.view(np.float16)).to(DEV)
        y = host(w4.w4_matmul_kmajor(dev(x), *w4.w4h_prepack_kmajor(dev(Wq), s_dev, dev(z)),
                                     bias=dev(b)))
    elif variant == "g64":
        Wq, s, m = ORC.quantize_pack_g64(W)
        y_ref, bound = ORC.w4g_matmul(x, Wq, s, m, b)
        y = host(w4.w4g_matmul_kmajor(dev(x), *w4.w4g_prepack_kmajor(dev(Wq), dev(s), dev(m)),
                                      bias=dev(b)))
    else:
        act = "gelu" if variant == "gelu" else ("swiglu" if variant.startswith("swiglu") else "none")
        r = synth.activations(M, N // 2, cfg=272, slot=M) if variant.endswith("+res") else None
        Wq, s, z = ORC.quantize_pack(W)
        y_ref, bound = ORC.w4_matmul_ep(x, Wq, s, z, b, r, act=act)
        P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
        y = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b), act=act,
                                     residual=None if r is None else dev(r)))
    assert_bound(y, y_ref, bound, f"shared activations {variant} {K}x{N}")


# 17 to 128 rows on small matrices: the whole-K matrix-core kernel in row
# groups of 16 (grid.y) when the 48 column groups times the row groups reach
# 128 workgroups (from 33 rows); 128 rows is the largest, 40 and 100 leave a
# ragged last group, 3072 x 768 has 24 quads per column.  SwiGLU with the
# residual updated in place, and the plain store with bias.
@pytest.mark.parametrize("M", [40, 100, 128])
@pytest.mark.parametrize("K,N", [(768, 768), (3072, 768)])
@pytest.mark.parametrize("act", ["none", "swiglu"])
def test_kmajor_whole_k_row_groups(M, K, N, act):
    assert w4.w4_matmul_kmajor_workspace_bytes(M, K, N) == 0
    note(f"row groups act={act} M={M} K={K} N={N}")
    W = mixed_weights(K, N, cfg=281)
    x = synth.activations(M, K, cfg=281, slot=M, outliers=True)
    b = synth.bias(N, cfg=281)
    nout = N // 2 if act == "swiglu" else N
    r = synth.activations(M, nout, cfg=282, slot=M)
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul_ep(x, Wq, s, z, b, r, act=act)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y = dev(r)  # the residual stream, updated in place
    w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b), act=act, residual=y, out=y)
    assert_bound(host(y), y_ref, bound, f"row groups {act} M={M} {K}x{N}")


# Around the whole-K kernel's grid threshold (32 workgroups of 16 columns per
# row group): 31 column tiles take the split-K kernel and its workspace, 32 the
# whole-K kernel (with 8 or 16 waves on these narrow grids); M = 20 forms two
# row groups of 16.
@pytest.mark.parametrize("M,K,N,whole", [(4, 768, 496, False), (4, 768, 498, True),
                                         (16, 3072, 496, False), (16, 3072, 528, True),
                                         (20, 768, 240, False), (20, 768, 256, True),
                                         (3, 8192, 512, True)])
def test_kmajor_grid_threshold(M, K, N, whole):
    ws = w4.w4_matmul_kmajor_workspace_bytes(M, K, N)
    assert (ws == 0) == whole, f"workspace {ws} for M={M} K={K} N={N}"
    note(f"grid threshold M={M} K={K} N={N} whole={whole}")
    W = mixed_weights(K, N, cfg=283)
    x = synth.activations(M, K, cfg=283, slot=M, outliers=True)
    b = synth.bias(N, cfg=283)
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul(x, Wq, s, z, b)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b)))
    assert_bound(y, y_ref, bound, f"grid threshold M={M} {K}x{N}")


# --------------------------------------------------------------------------
# fused epilogues (GELU, SwiGLU on interleaved gate/up columns, residual add)
# --------------------------------------------------------------------------
EP_CASES = [("none", True), ("gelu", False), ("gelu", True), ("swiglu", False), ("swiglu", True)]
# (M, K, N): the decode GEMV (M <= 2, and M = 3 with K % 128 != 0), its row
# loop (M > 4 with K % 128 != 0), the matrix cores from M = 3 with one split
# and with split-K, a ragged N, and K = 2048 (one column slot per workgroup:
# an odd column count is made even for SwiGLU)
EP_SHAPES = [(1, 768, 2304), (1, 3072, 768), (3, 192, 530), (4, 2048, 768), (1, 2048, 768),
             (2, 3072, 768), (7, 64, 96), (16, 768, 2304), (58, 768, 768), (16, 3072, 3072),
             (65, 256, 530)]


@pytest.mark.parametrize("M,K,N", EP_SHAPES)
@pytest.mark.parametrize("act,res", EP_CASES)
def test_kmajor_epilogue(M, K, N, act, res):
    note(f"epilogue act={act} residual={res} M={M} K={K} N={N} "
         f"ws={w4.w4_matmul_kmajor_workspace_bytes(M, K, N)}")
    W = mixed_weights(K, N, cfg=241)
    x = synth.activations(M, K, cfg=241, slot=M, outliers=True)
    b = synth.bias(N, cfg=241)
    nout = N // 2 if act == "swiglu" else N
    r = synth.activations(M, nout, cfg=242, slot=M) if res else None
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul_ep(x, Wq, s, z, b, r, act=act)
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    y = host(w4.w4_matmul_kmajor(dev(x), *P, bias=dev(b), act=act,
                                 residual=None if r is None else dev(r)))
    assert y.shape == (M, nout)
    assert_bound(y, y_ref, bound, f"epilogue {act}{'+res' if res else ''} M={M} {K}x{N}")


@pytest.mark.parametrize("M", [1, 16])
def test_kmajor_epilogue_in_place_residual(M):
    """residual == y: the residual stream updated in place (out-proj / down-proj)."""
    K, N = 3072, 768
    W = mixed_weights(K, N, cfg=243)
    x = synth.activations(M, K, cfg=243, slot=M)
    r = synth.activations(M, N, cfg=244, slot=M)
    Wq, s, z = ORC.quantize_pack(W)
    y_ref, bound = ORC.w4_matmul_ep(x, Wq, s, z, None, r, act="none")
    P = w4.w4_prepack_kmajor(dev(Wq), dev(s), dev(z))
    h = dev(r)
    w4.w4_matmul_kmajor(dev(x), *P, act="none", residual=h, out=h)
    assert_bound(host(h), y_ref, bound, f"in-place residual M={M}")


def test_kmajor_epilogue_bias_only_and_plain_path_unchanged():
    K, N, M = 0, 64, 3
    b = synth.bias(N, cfg=245)
    r = synth.activations(M, N // 2, cfg=245)
    Wq = np.zeros((0, N // 2), np.uint8)
    s = np.zeros((0, N), np.float32)
    zp = np.zeros((0, N // 2), np.uint8)
    x = np.zeros((M, 0), np.float32)
    y_ref, bound = ORC.w4_matmul_ep(x, Wq, s, zp, b, r, act="swiglu")
    P = (torch.zeros((N, 0), dtype=torch.uint8, device=DEV),
         torch.zeros((N, 0), dtype=torch.float32, device=DEV),
         torch.zeros((N, 0), dtype=torch.uint8, device=DEV))
    y = host(w4.w4_matmul_kmajor(torch.zeros((M, 0), device=DEV), *P, bias=dev(b),
                                 act="swiglu", residual=dev(r)))
    assert_bound(y, y_ref, bound, "K=0 swiglu epilogue")
    # act "none" without a residual takes the plain entry point: bit-identical
    K, N, M = 768, 2304, 16
    W = mixed_weights(K, N, cfg=246)
    P = w4.w4_prepack_kmajor(*w4.w4_quantize_pack(dev(W)))
    x = dev(synth.activations(M, K, cfg=246))
    bb = dev(synth.bias(N, cfg=246))
    y0 = host(w4.w4_matmul_kmajor(x, *P, bias=bb))
    zero = torch.zeros((M, N), device=DEV)
    y1 = host(w4.w4_matmul_kmajor(x, *P, bias=bb, residual=zero))
    assert_bits(y1, y0 + 0.0, "epilogue with a zero residual")


# --------------------------------------------------------------------------
# group-64 affine variant
# --------------------------------------------------------------------------
G64_SHAPES = [(64, 2), (128, 34), (192, 530), (768, 2304), (3072, 768), (8192, 512)]


@pytest.mark.parametrize("K,N", G64_SHAPES)
def test_g64_quantize_dequantize_prepack_bit_exact(K, N):
    note(f"g64 quantize/dequantize/prepack K={K} N={N}")
    W = mixed_weights(K, N, cfg=251)
    Wq_r, s_r, m_r = ORC.quantize_pack_g64(W)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    Wq, s, m = w4.w4g_quantize_pack(dev(W), d_status=st)
    assert int(host(st)[0]) == 0
    assert_bits(host(Wq), Wq_r, f"g64 Wq {K}x{N}")
    assert_bits(host(s), s_r, f"g64 scales {K}x{N}")
    assert_bits(host(m), m_r, f"g64 mins {K}x{N}")
    assert_bits(host(w4.w4g_dequantize(Wq, s, m)), ORC.dequantize_g64(Wq_r, s_r, m_r, K, N),
                f"g64 W_hat {K}x{N}")
    for name, a, b in zip(("Pq", "Ps", "Pm"), w4.w4g_prepack_kmajor(Wq, s, m),
                          ORC.prepack_kmajor_g64(Wq_r, s_r, m_r, K, N)):
        assert_bits(host(a), b, f"g64 {name} {K}x{N}")


def test_g64_nonfinite_sets_status():
    W = synth.weights(128, 8, cfg=252)
    W[70, 3] = np.nan
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    w4.w4g_quantize_pack(dev(W), d_status=st)
    assert int(host(st)[0]) == w4.W4_ERR_NONFINITE


@pytest.mark.parametrize("K,N", [(64, 16), (768, 2304), (3072, 768), (192, 530), (8192, 512),
                                 (1024, 1008)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16, 58])
def test_g64_matmul_kmajor(M, K, N):
    note(f"g64 matmul M={M} K={K} N={N}")
    W = mixed_weights(K, N, cfg=253)
    x = synth.activations(M, K, cfg=253, slot=M, outliers=True)
    b = synth.bias(N, cfg=253)
    Wq, s, m = ORC.quantize_pack_g64(W)
    y_ref, bound = ORC.w4g_matmul(x, Wq, s, m, b)
    P = w4.w4g_prepack_kmajor(dev(Wq), dev(s), dev(m))
    y = host(w4.w4g_matmul_kmajor(dev(x), *P, bias=dev(b)))
    assert_bound(y, y_ref, bound, f"g64 M={M} {K}x{N}")


@pytest.mark.parametrize("slot", range(4))
def test_g64_dense38_full_size_sampled(slot):
    K, N = synth.DENSE38_SHAPES[slot]
    note(f"g64 dense38 slot {slot} K={K} N={N} (sampled columns)")
    W = synth.weights(K, N, cfg=synth.CFG_DENSE38, layer=0, slot=slot)
    x = synth.activations(1, K, cfg=synth.CFG_DENSE38, layer=0, slot=slot, outliers=True)
    P = w4.w4g_prepack_kmajor(*w4.w4g_quantize_pack(dev(W)))
    y = host(w4.w4g_matmul_kmajor(dev(x), *P))
    pairs = sample_pairs(N, 48, seed=20 + slot)
    cols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
    Wq, s, m = ORC.quantize_pack_g64(W[:, cols])
    y_ref, bound = ORC.w4g_matmul(x, Wq, s, m)
    assert_bound(y[:, cols], y_ref, bound, f"g64 dense38 {K}x{N}")


def test_g64_special_inputs():
    K, N, M = 768, 2304, 4
    W = mixed_weights(K, N, cfg=254)
    Wq, s, m = ORC.quantize_pack_g64(W)
    P = w4.w4g_prepack_kmajor(dev(Wq), dev(s), dev(m))
    base = synth.activations(M, K, cfg=254)
    cases = {"zeros": np.zeros((M, K), np.float32),
             "one-hot rows": np.eye(M, K, 7, dtype=np.float32),
             "tiny": base * np.float32(1e-30),
             "huge": base * np.float32(1e30),
             "spread": base * np.where(np.arange(K) % 3 == 0, 1e3, 1e-3).astype(np.float32)}
    for name, x in cases.items():
        y_ref, bound = ORC.w4g_matmul(x, Wq, s, m)
        y = host(w4.w4g_matmul_kmajor(dev(x), *P))
        assert_bound(y, y_ref, bound, f"g64 x={name}")


def test_shared_workspace_growth_keeps_captured_graphs_valid():
    """A graph captured with the shared scratch must stay correct after a later
    call grows the scratch (the old buffer is kept, not freed and reused)."""
    K, N = 3072, 768
    W = mixed_weights(K, N, cfg=261)
    Wq, s, z = w4.w4_quantize_pack(dev(W))
    x = dev(synth.activations(1, K, cfg=261))
    y = torch.empty((1, N), device=DEV)
    need_small = w4.w4_matmul_workspace_bytes(1, K, N)
    assert need_small > 0
    ref = host(w4.w4_matmul(x, Wq, s, z))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w4.w4_matmul(x, Wq, s, z, out=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.w4_matmul(x, Wq, s, z, out=y)
    # a call needing far more scratch grows the pool
    M2, K2, N2 = 64, 4096, 4096
    assert w4.w4_matmul_workspace_bytes(M2, K2, N2) > 2 * need_small
    W2 = synth.weights(K2, N2, cfg=262)
    P2 = w4.w4_quantize_pack(dev(W2))
    x2 = dev(synth.activations(M2, K2, cfg=262))
    junk = [torch.full((1 << 22,), 7.0, device=DEV) for _ in range(4)]  # reuse pressure
    w4.w4_matmul(x2, *P2)
    del junk
    for _ in range(3):
        y.zero_()
        g.replay()
        assert_bits(host(y), ref, "graph replay after the scratch grew")


@pytest.mark.parametrize("nbytes,loads", [(1 << 20, 8), (4096 * 16 + 48, 4), (18186240, 16),
                                          (16, 6), (300000 * 16, 12)])
def test_read_bytes_xor_words(nbytes, loads):
    """The streaming-read reference: wave w's word is the XOR of the 32-bit
    words it read (lane t of workgroup g reads pieces g*256 + t + j*256*G)."""
    g = np.random.default_rng(nbytes)
    data = g.integers(0, 256, size=nbytes, dtype=np.uint8)
    out = host(w4.w4_read_bytes(dev(data), loads))
    words = w4.library().w4_read_bytes_words(nbytes, loads)
    lanes = words * 64
    pieces = data.view(np.uint32).reshape(-1, 4)
    n16 = pieces.shape[0]
    grp = (np.arange(n16) % lanes) // 64
    want = np.zeros(words, np.uint32)
    np.bitwise_xor.at(want, grp, np.bitwise_xor.reduce(pieces, axis=1))
    assert np.array_equal(out[:words].view(np.uint32), want)


def test_empty_inputs_on_every_entry_point():
    """Zero rows, columns, K or tokens: every entry point returns empty (or
    bias-only) results of the right shape and enqueues no failing work."""
    K, N = 128, 64
    W = synth.weights(K, N, cfg=290)
    # the quantizer and the K-major prepack on no rows and on no columns
    Wq0, s0, z0 = w4.w4_quantize_pack(torch.zeros((0, N), device=DEV))
    assert (Wq0.shape, s0.shape, z0.shape) == ((0, N // 2), (0, N), (0, N // 2))
    WqN, sN, zN = w4.w4_quantize_pack(torch.zeros((K, 0), device=DEV))
    assert (WqN.shape, sN.shape, zN.shape) == ((K, 0), (K // 32, 0), (K // 32, 0))
    P0 = w4.w4_prepack_kmajor(WqN, sN, zN)
    assert tuple(p.shape[0] for p in P0) == (0, 0, 0)
    # the K-major matmul on no rows and on no columns
    P = w4.w4_prepack_kmajor(*w4.w4_quantize_pack(dev(W)))
    assert w4.w4_matmul_kmajor(torch.zeros((0, K), device=DEV), *P).shape == (0, N)
    assert w4.w4_matmul_kmajor(torch.zeros((16, K), device=DEV), *P0).shape == (16, 0)
    assert w4.w4_matmul(torch.zeros((2, K), device=DEV), WqN, sN, zN).shape == (2, 0)
    # the int8 head: no tokens in the table, no rows, no tokens to look up
    E = synth.head_table(K, 40, cfg=290)
    Q, hs = w4.i8_quantize_head(dev(E))
    Qz, hz = w4.i8_quantize_head(torch.zeros((K, 0), device=DEV))
    assert Qz.shape == (K, 0) and hz.shape == (0,)
    x = dev(synth.activations(1, K, cfg=290)[0])
    assert w4.i8_head_logits(x, Qz, hz).shape == (0,)
    Qt = w4.i8_prepack_head(Q, 40)
    assert w4.i8_head_logits_rows(torch.zeros((0, K), device=DEV), Qt, hs).shape == (0, 40)
    tok = torch.zeros(0, dtype=torch.int64, device=DEV)
    assert w4.i8_embed(tok, Q, hs).shape == (0, K)
    assert w4.i8_embed_kmajor(tok, Qt, hs, K).shape == (0, K)
    torch.cuda.synchronize()
