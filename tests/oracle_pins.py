"""Pins for the CPU oracle: checks against what the method and mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
on a violation.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` runs them on copies of the oracle with planted
mistakes and requires every mutant to fail at least one pin.

None of these recomputes the oracle's formula and compares: each check is a
different route to the same fact.
  * packing: the low-nibble-first convention's worked examples and an
    exhaustive round trip over all 256 bytes (the page's "raw packed UINT4",
    low nibble first, pairs along N);
  * quantizer: exact reproduction of weights that lie on a power-of-two grid;
    the round-trip bound |w - w_hat| <= s/2 (plus fp32 rounding slack) for
    every weight; brute-force nearest code in exact rational arithmetic;
    degenerate blocks in closed form;
  * dequantization: every (q, z) pair against the exactly rounded rational
    product;
  * matmul: exact rational sums on tiny shapes, one-hot rows, constant-0.5
    weights (every output half the sum of its row of x), zero activations;
  * head: one-hot rows, sign symmetry, full use of [-127, 127], the
    round-trip bound, exact rational logits;
  * embedding lookup: rows of the dequantized table;
  * byte budget: the GPT-2 small q4 file size the page prints;
  * group-64 affine variant: on-grid groups reproduced exactly, the byte
    count, brute-force nearest codes in exact rationals, the minimum kept
    exactly, constant groups, every code through the single-rounding
    dequantization, exact rational matmuls;
  * fused epilogues: GELU against the exact (erf) GELU within the tanh form's
    known 5e-4 gap, SiLU against its tanh form, the odd-part identity
    f(v) - f(-v) = v of both, and one-hot rows through the epilogue (exact
    pre-activation values, gate/up pairing, a closed gate).
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as oracle_mod
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BLOCK = 32


# --------------------------------------------------------------------------
# exact-arithmetic helpers
# --------------------------------------------------------------------------
def F(v) -> Fraction:
    """Exact rational value of a float32/float64 scalar."""
    return Fraction(float(v))


def f32_round(fr: Fraction) -> np.float32:
    """The fp32 value nearest to the rational ``fr`` (ties to even significand)."""
    if fr == 0:
        return np.float32(0.0)
    c = np.float32(float(fr))
    cands = {float(c)}
    for d in (np.inf, -np.inf):
        n = np.nextafter(c, np.float32(d))
        if np.isfinite(n):
            cands.add(float(n))
    best = None
    for v in cands:
        err = abs(Fraction(v) - fr)
        key = (err, int(np.float32(v).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(best[1])


def ulp32(v) -> float:
    return float(np.spacing(np.float32(abs(v))))


# --------------------------------------------------------------------------
# packing
# --------------------------------------------------------------------------
def pin_pack_worked_examples(orc):
    # low nibble first: element 0 sits in bits 0..3, element 1 in bits 4..7
    assert orc.pack_u4([3, 10]).tolist() == [0xA3]
    assert orc.pack_u4([1, 2, 3, 4]).tolist() == [0x21, 0x43]
    assert orc.pack_u4([15, 0, 0, 15]).tolist() == [0x0F, 0xF0]
    assert orc.unpack_u4([0xA3]).tolist() == [3, 10]
    assert orc.unpack_u4([0x21, 0x43]).tolist() == [1, 2, 3, 4]


def pin_pack_exhaustive(orc):
    every_byte = np.arange(256, dtype=np.uint8)
    v = orc.unpack_u4(every_byte)
    assert v.max() <= 15
    assert np.array_equal(orc.pack_u4(v), every_byte)
    # all 16 x 16 (even, odd) pairs, in every position of a row
    pairs = np.array([(a, b) for a in range(16) for b in range(16)], np.uint8).reshape(-1)
    packed = orc.pack_u4(pairs)
    assert np.array_equal(orc.unpack_u4(packed), pairs)
    # a byte's value identifies the pair: 16 * odd + even
    assert np.array_equal(packed, (pairs[1::2].astype(int) * 16 + pairs[0::2]).astype(np.uint8))


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------
def _on_grid(K, N, seed):
    """Weights w = (q - z) * 2**e per block, with code 0 and 15 both present."""
    g = np.random.default_rng(seed)
    nb = K // BLOCK
    e = g.integers(-10, -3, size=(nb, N))
    z = g.integers(0, 16, size=(nb, N)).astype(np.uint8)
    q = g.integers(0, 16, size=(K, N)).astype(np.uint8)
    for b in range(nb):
        for n in range(N):
            r0, r1 = g.choice(BLOCK, size=2, replace=False)
            q[b * BLOCK + r0, n] = 0
            q[b * BLOCK + r1, n] = 15
    s = np.ldexp(np.float32(1.0), e).astype(np.float32)
    srow = np.repeat(s, BLOCK, axis=0)
    zrow = np.repeat(z, BLOCK, axis=0)
    W = ((q.astype(np.float32) - zrow.astype(np.float32)) * srow).astype(np.float32)
    return W, q, z, s


def pin_quantize_on_grid(orc):
    for K, N, seed in ((32, 2, 1), (64, 6, 2), (96, 10, 3), (256, 34, 4)):
        W, q, z, s = _on_grid(K, N, seed)
        Wq, sc, zp = orc.quantize_pack(W)
        assert Wq.shape == (K, N // 2) and sc.shape == (K // BLOCK, N)
        assert zp.shape == (K // BLOCK, N // 2)
        assert np.array_equal(sc, s), "scale of an on-grid block must be its exact 2**e"
        q2, z2 = orc.unpack(Wq, zp, K, N)
        assert np.array_equal(z2, z), "zero points of on-grid blocks must be exact"
        assert np.array_equal(q2, q), "codes of on-grid weights must be exact"
        # the bytes themselves follow the packing convention, row-major over [K, N]
        assert np.array_equal(Wq.reshape(-1), orc.pack_u4(q.reshape(-1)))
        assert np.array_equal(zp.reshape(-1), orc.pack_u4(z.reshape(-1)))
        assert np.array_equal(orc.dequantize(Wq, sc, zp, K, N), W), "on-grid w_hat == w"


def pin_quantize_ties_half_even(orc):
    """Weights exactly halfway between two codes take the even multiple of s.

    The page does not state a tie rule.  The format is ONNX's blocked
    QuantizeLinear/DequantizeLinear pair, whose rounding is to nearest with
    ties to even (also IEEE's default mode and numpy's ``round``); this pin
    fixes that reading.
    """
    g = np.random.default_rng(13)
    K, N = 64, 8
    nb = K // BLOCK
    W = np.zeros((K, N), np.float32)
    want = np.zeros((K, N), np.uint8)
    for b in range(nb):
        for n in range(N):
            e = int(g.integers(-9, -4))
            s = np.float32(2.0 ** e)
            z = int(g.integers(1, 15))
            rows = g.permutation(BLOCK)
            for i, r in enumerate(rows):
                k = b * BLOCK + r
                if i == 0:
                    c = 0
                elif i == 1:
                    c = 15
                else:
                    c = int(g.integers(0, 15))
                    t = (c - z) + 0.5                 # w / s, exactly halfway
                    W[k, n] = np.float32(t) * s
                    lo_int = c - z                    # the two neighbours of t
                    even = lo_int if lo_int % 2 == 0 else lo_int + 1
                    want[k, n] = even + z
                    continue
                W[k, n] = np.float32(c - z) * s
                want[k, n] = c
    Wq, sc, zp = orc.quantize_pack(W)
    q, _ = orc.unpack(Wq, zp, K, N)
    assert np.array_equal(q, want), "ties must round to the even multiple"


def _test_weights():
    """A spread of block contents: normal, heavy-tailed, same-sign, tiny, huge."""
    out = []
    g = np.random.default_rng(7)
    out.append(synth.weights(128, 64, cfg=100))
    t = g.standard_t(2, size=(64, 32)).astype(np.float32) * np.float32(0.02)
    out.append(t)
    out.append(np.abs(g.standard_normal((64, 16))).astype(np.float32) + np.float32(0.3))
    out.append(-np.abs(g.standard_normal((64, 16))).astype(np.float32) - np.float32(0.3))
    out.append((g.standard_normal((32, 8)) * 1e-30).astype(np.float32))
    out.append((g.standard_normal((32, 8)) * 1e30).astype(np.float32))
    sub = (g.standard_normal((32, 8)) * 1e-41).astype(np.float32)  # subnormal fp32
    out.append(sub)
    return out


def pin_round_trip_bound(orc):
    for W in _test_weights():
        K, N = W.shape
        Wq, s, zp = orc.quantize_pack(W)
        What = orc.dequantize(Wq, s, zp, K, N)
        q, z = orc.unpack(Wq, zp, K, N)
        assert q.max() <= 15 and z.max() <= 15
        srow = np.repeat(s, BLOCK, axis=0).astype(np.float64)
        err = np.abs(W.astype(np.float64) - What.astype(np.float64))
        # s/2 from rounding to the nearest code, plus the fp32 roundings of
        # w / s and of (q - z) * s (each at most 15 * 2**-24 * s); in the
        # subnormal range the absolute spacing 2**-149 replaces the relative one
        lim = srow * (0.5 + 2.0 ** -19) + 2.0 ** -148
        assert np.all(err <= lim), f"round-trip error {np.max(err / np.maximum(srow, 1e-300))} s"


def pin_nearest_code_bruteforce(orc):
    g = np.random.default_rng(11)
    cases = [synth.weights(32, 4, cfg=101),
             (g.standard_normal((32, 4)) * 0.3 + 0.1).astype(np.float32),
             np.abs(g.standard_normal((32, 2))).astype(np.float32)]
    for W in cases:
        K, N = W.shape
        Wq, s, zp = orc.quantize_pack(W)
        q, z = orc.unpack(Wq, zp, K, N)
        for n in range(N):
            sn = F(s[0, n])
            assert sn > 0
            zn = int(z[0, n])
            for k in range(K):
                w = F(W[k, n])
                t = w / sn
                frac = t - (t.numerator // t.denominator)
                if abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 20):
                    continue  # tie zone: decided by the rounding convention
                errs = [abs(w - (qq - zn) * sn) for qq in range(16)]
                best = min(errs)
                assert errs[int(q[k, n])] == best, (k, n, int(q[k, n]), errs.index(best))
            # codes 0 and 15 sit within s/2 of the ends of the 0-inclusive range
            lo = min(min(F(v) for v in W[:, n]), Fraction(0))
            hi = max(max(F(v) for v in W[:, n]), Fraction(0))
            slack = sn * Fraction(1, 2 ** 18)
            assert abs(lo - (0 - zn) * sn) <= sn / 2 + slack
            assert abs(hi - (15 - zn) * sn) <= sn / 2 + slack
            # the block's minimum maps to code 0 when it is negative
            if lo < 0:
                kmin = int(np.argmin(W[:, n]))
                assert int(q[kmin, n]) == 0


def pin_degenerate_blocks(orc):
    K, N = 32, 8
    W = np.zeros((K, N), np.float32)
    W[:, 1] = 0.5                     # constant positive block
    W[:, 2] = -0.25                   # constant negative block
    W[7, 3] = 3.0                     # one nonzero weight
    W[:, 4] = -0.0                    # negative zeros
    W[:, 5] = np.float32(1e-45)       # smallest subnormal
    Wq, s, zp = orc.quantize_pack(W)
    q, z = orc.unpack(Wq, zp, K, N)
    What = orc.dequantize(Wq, s, zp, K, N)
    # all-zero block: everything 0
    for n in (0, 4, 6, 7):
        assert s[0, n] == 0 and z[0, n] == 0 and not q[:, n].any() and not What[:, n].any()
    # constant c > 0: range [0, c], zero point 0, every code 15
    assert z[0, 1] == 0 and np.all(q[:, 1] == 15)
    assert s[0, 1] == f32_round(Fraction(1, 2) / 15)
    assert np.all(What[:, 1] == np.float32(0.5)), "15 * fl32(0.5/15) rounds back to 0.5"
    # constant c < 0: range [c, 0], zero point 15, every code 0
    assert z[0, 2] == 15 and np.all(q[:, 2] == 0)
    assert np.all(What[:, 2] == f32_round(-15 * F(s[0, 2])))
    # one nonzero weight: it takes code 15, the zeros code z = 0
    assert z[0, 3] == 0 and q[7, 3] == 15 and np.count_nonzero(q[:, 3]) == 1
    assert What[7, 3] == np.float32(3.0)
    # a range of one subnormal ulp: s = fl32(2**-149 / 15) rounds to 0
    assert s[0, 5] == 0 and not q[:, 5].any()


def pin_shape_and_value_errors(orc):
    for shape in ((31, 4), (32, 3), (33, 2)):
        try:
            orc.quantize_pack(np.zeros(shape, np.float32))
        except oracle_mod.OracleError as e:
            assert e.status == oracle_mod.BAD_SHAPE
        else:
            raise AssertionError(f"shape {shape} accepted")
    for bad in (np.nan, np.inf, -np.inf):
        W = np.zeros((32, 2), np.float32)
        W[5, 1] = bad
        try:
            orc.quantize_pack(W)
        except oracle_mod.OracleError as e:
            assert e.status == oracle_mod.NONFINITE
        else:
            raise AssertionError(f"{bad} accepted")
    W = np.zeros((32, 2), np.float32)
    W[0, 0], W[1, 0] = 3e38, -3e38      # hi - lo overflows fp32
    try:
        orc.quantize_pack(W)
    except oracle_mod.OracleError as e:
        assert e.status == oracle_mod.NONFINITE
    else:
        raise AssertionError("overflowing range accepted")


# --------------------------------------------------------------------------
# dequantization
# --------------------------------------------------------------------------
def pin_dequant_all_pairs(orc):
    # 16 blocks x 16 columns: block b, column n has zero point (b + n) % 16 and
    # its 32 rows hold codes 0..15 twice, so all 256 (q, z) pairs occur
    nb, N = 16, 16
    K = nb * BLOCK
    z = np.array([[(b + n) % 16 for n in range(N)] for b in range(nb)], np.uint8)
    q = np.array([[(k % 16) for _ in range(N)] for k in range(K)], np.uint8)
    g = np.random.default_rng(5)
    s = np.abs(g.standard_normal((nb, N))).astype(np.float32) * np.float32(0.01)
    s[0, :4] = [np.float32(1e-40), np.float32(3e-39), np.float32(1e30), np.float32(2.0 ** 100)]
    Wq = orc.pack_u4(q.reshape(-1)).reshape(K, N // 2)
    zp = orc.pack_u4(z.reshape(-1)).reshape(nb, N // 2)
    What = orc.dequantize(Wq, s, zp, K, N)
    seen = set()
    for k in range(K):
        for n in range(N):
            b = k // BLOCK
            qq, zz = int(q[k, n]), int(z[b, n])
            seen.add((qq, zz))
            want = f32_round((qq - zz) * F(s[b, n]))
            got = What[k, n]
            assert got == want or (want == 0 and got == 0), (k, n, got, want)
    assert len(seen) == 256


def pin_prepack_kmajor(orc):
    """The K-major relayout is the transpose of the unpacked codes, packed
    low-nibble-first along K; scales and zero points transpose the same way."""
    for K, N in ((64, 2), (128, 6), (192, 34)):
        W = synth.weights(K, N, cfg=108, slot=K)
        Wq, s, z = orc.quantize_pack(W)
        q, zz = orc.unpack(Wq, z, K, N)
        Pq, Ps, Pz = orc.prepack_kmajor(Wq, s, z, K, N)
        assert Pq.shape == (N, K // 2) and Ps.shape == (N, K // 32) and Pz.shape == (N, K // 64)
        assert np.array_equal(orc.unpack_u4(Pq).reshape(N, K), np.ascontiguousarray(q.T))
        assert np.array_equal(orc.unpack_u4(Pz).reshape(N, K // 32), np.ascontiguousarray(zz.T))
        assert np.array_equal(Ps, np.ascontiguousarray(s.T))
        # spot check of the low-nibble-first pairing along K on one element
        k, n = K - 3, N - 1
        byte = int(Pq[n, k // 2])
        assert (byte >> (4 * (k % 2))) & 15 == int(q[k, n])
    try:
        orc.prepack_kmajor(*orc.quantize_pack(synth.weights(32, 4, cfg=108)), 32, 4)
    except oracle_mod.OracleError as e:
        assert e.status == oracle_mod.BAD_SHAPE
    else:
        raise AssertionError("K % 64 != 0 accepted")


# --------------------------------------------------------------------------
# matmul
# --------------------------------------------------------------------------
def _exact_check(y, bound, x, What, bias):
    M, K = x.shape
    N = What.shape[1]
    for m in range(M):
        for n in range(N):
            terms = [F(x[m, k]) * F(What[k, n]) for k in range(K)]
            exact = sum(terms, Fraction(0))
            mag = sum((abs(t) for t in terms), Fraction(0))
            if bias is not None:
                exact += F(bias[n])
                mag += abs(F(bias[n]))
            # fp64 accumulation error plus one fp32 rounding
            tol = Fraction(ulp32(float(exact))) / 2 + (K + 2) * Fraction(1, 2 ** 53) * mag
            assert abs(F(y[m, n]) - exact) <= tol, (m, n, float(y[m, n]), float(exact))
            want_bound = float(Fraction(1, 10 ** 5) * mag + Fraction(1, 10 ** 6))
            assert abs(bound[m, n] - want_bound) <= 1e-12 * want_bound, (bound[m, n], want_bound)


def pin_matmul_exact_small(orc):
    for M, K, N, outl in ((1, 32, 2, False), (3, 64, 6, True), (2, 96, 4, False)):
        W = synth.weights(K, N, cfg=102, slot=M)
        x = synth.activations(M, K, cfg=102, slot=M, outliers=outl)
        b = synth.bias(N, cfg=102, slot=M)
        Wq, s, zp = orc.quantize_pack(W)
        What = orc.dequantize(Wq, s, zp, K, N)
        for bias in (None, b):
            y, bound = orc.w4_matmul(x, Wq, s, zp, bias)
            _exact_check(y, bound, x, What, bias)
            y2, bound2 = orc.matmul_f64(x, What, bias)
            assert np.array_equal(y, y2) and np.array_equal(bound, bound2)


def pin_matmul_special_cases(orc):
    K, N = 64, 10
    W = synth.weights(K, N, cfg=103)
    b = synth.bias(N, cfg=103)
    Wq, s, zp = orc.quantize_pack(W)
    What = orc.dequantize(Wq, s, zp, K, N)
    # one-hot rows pick out rows of W_hat; with a bias, one fp32 addition
    x = np.eye(K, dtype=np.float32)
    y, _ = orc.w4_matmul(x, Wq, s, zp)
    assert np.array_equal(y, What)
    y, _ = orc.w4_matmul(x, Wq, s, zp, b)
    assert np.array_equal(y, What + b[None, :])
    # zero activations give the bias exactly
    y, _ = orc.w4_matmul(np.zeros((2, K), np.float32), Wq, s, zp, b)
    assert np.array_equal(y, np.stack([b, b]))
    # constant 0.5 weights quantize losslessly; y = half the row sums
    Wc = np.full((K, N), 0.5, np.float32)
    Wq2, s2, zp2 = orc.quantize_pack(Wc)
    xi = np.random.default_rng(9).integers(-20, 21, size=(3, K)).astype(np.float32)
    y, _ = orc.w4_matmul(xi, Wq2, s2, zp2)
    half = (xi.sum(axis=1, dtype=np.float64) * 0.5).astype(np.float32)
    assert np.array_equal(y, np.repeat(half[:, None], N, axis=1))
    # empty reductions and empty outputs
    y, bound = orc.w4_matmul(np.zeros((2, 0), np.float32), np.zeros((0, N // 2), np.uint8),
                             np.zeros((0, N), np.float32), np.zeros((0, N // 2), np.uint8), b)
    assert np.array_equal(y, np.stack([b, b]))
    y, _ = orc.w4_matmul(np.zeros((0, K), np.float32), Wq, s, zp, b)
    assert y.shape == (0, N)


# --------------------------------------------------------------------------
# int8 head and embedding
# --------------------------------------------------------------------------
def pin_head_quantizer(orc):
    K, N = 96, 40
    E = synth.head_table(K, N, cfg=104)
    E[:, 3] = 0.0                                  # zero column
    E[:, 4] = -E[:, 5]                             # mirrored column
    Q, hs = orc.i8_quantize_head(E, ldq=48)
    assert Q.shape == (K, 48) and not Q[:, N:].any(), "padding columns are 0"
    assert Q[:, :N].min() >= -127
    assert hs[3] == 0 and not Q[:, 3].any()
    assert hs[4] == hs[5] and np.array_equal(Q[:, 4], -Q[:, 5]), "Q(-E) = -Q(E)"
    Qn, hsn = orc.i8_quantize_head(-E)
    assert np.array_equal(hsn, hs) and np.array_equal(Qn, -Q[:, :N])
    for n in range(N):
        if n == 3:
            continue
        assert np.max(np.abs(Q[:, n].astype(int))) == 127, "the largest entry uses 127"
        # the column maximum lies on the grid: max|E| = 127 * hs up to one rounding
        amax = F(np.max(np.abs(E[:, n])))
        assert abs(127 * F(hs[n]) - amax) <= 127 * Fraction(ulp32(hs[n])) / 2
        err = np.abs(E[:, n].astype(np.float64) - Q[:, n].astype(np.float64) * float(hs[n]))
        assert np.all(err <= float(hs[n]) * (0.5 + 2.0 ** -17))
    # nearest-code check in exact arithmetic on one column
    n = 7
    for k in range(K):
        e = F(E[k, n])
        t = e / F(hs[n])
        if abs(abs(t - (t.numerator // t.denominator)) - Fraction(1, 2)) < Fraction(1, 2 ** 20):
            continue
        errs = {c: abs(e - c * F(hs[n])) for c in range(-127, 128)}
        assert errs[int(Q[k, n])] == min(errs.values())
    # zero point is 0: the dequantized table is odd in Q
    Eh = orc.i8_dequantize_head(Q, hs)
    assert np.all(Eh[:, 3] == 0)


def pin_head_logits(orc):
    K, N = 64, 12
    E = synth.head_table(K, N, cfg=105)
    Q, hs = orc.i8_quantize_head(E, ldq=16)
    Eh = orc.i8_dequantize_head(Q, hs)
    for n in range(N):
        for k in range(K):
            assert Eh[k, n] == f32_round(int(Q[k, n]) * F(hs[n]))
    # one-hot rows
    for k in (0, 17, K - 1):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        logits, _ = orc.i8_head_logits(x, Q, hs)
        assert np.array_equal(logits, Eh[k])
    # exact rational logits
    x = synth.activations(1, K, cfg=105, outliers=True)[0]
    logits, bound = orc.i8_head_logits(x, Q, hs)
    _exact_check(logits[None, :], bound[None, :], x[None, :], Eh, None)


def pin_embedding(orc):
    K, N = 48, 30
    E = synth.head_table(K, N, cfg=106)
    Q, hs = orc.i8_quantize_head(E, ldq=32)
    Eh = orc.i8_dequantize_head(Q, hs)
    toks = np.array([0, 5, 29, 5, 17], np.int64)
    out = orc.i8_embed(toks, Q, hs)
    assert out.shape == (5, K)
    for t, tok in enumerate(toks):
        assert np.array_equal(out[t], Eh[:, tok])
    # the lookup is the head's transpose: the logits of one-hot e_k, read at
    # the looked-up tokens, equal column k of the looked-up rows
    logits, _ = orc.i8_head_logits(np.eye(K, dtype=np.float32)[3], Q, hs)
    assert np.array_equal(logits[toks], out[:, 3])
    for bad in (-1, N):
        try:
            orc.i8_embed(np.array([bad], np.int64), Q, hs)
        except oracle_mod.OracleError as e:
            assert e.status == oracle_mod.BAD_SHAPE
        else:
            raise AssertionError("token out of range accepted")


# --------------------------------------------------------------------------
# byte budget against the page's printed file size
# --------------------------------------------------------------------------
def pin_file_size(orc):
    with open(os.path.join(GOLDEN, "gpt2_small_q4_file_size.json")) as f:
        g = json.load(f)
    body = 0
    for K, N in synth.GPT2_SHAPES:
        Wq, s, zp = orc.quantize_pack(synth.weights(K, N, cfg=107))
        body += synth.GPT2_LAYERS * (Wq.nbytes + s.nbytes + zp.nbytes)
    Q, hs = orc.i8_quantize_head(np.zeros((synth.GPT2_HIDDEN, synth.GPT2_VOCAB), np.float32))
    rest = g["fp32_position_table_bytes"] + g["fp32_bias_and_norm_bytes"]
    total = body + Q.nbytes + hs.nbytes + rest
    assert abs(total / 1e6 - g["q4_shipped_MB"]) < 0.5, total
    # the fp32 model of the same architecture
    params = sum(synth.GPT2_LAYERS * K * N for K, N in synth.GPT2_SHAPES)
    fp32 = 4 * (params + synth.GPT2_HIDDEN * synth.GPT2_VOCAB) + rest
    assert abs(fp32 / 1e6 - g["fp32_MB"]) < 0.5, fp32


# --------------------------------------------------------------------------
# fp16-scale variant (the measurements table's "fp16 scales" file)
# --------------------------------------------------------------------------
def pin_f16_conversion(orc):
    """binary16 rounding against numpy's IEEE conversion (a library routine)."""
    g = np.random.default_rng(21)
    edges = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
             3 * 2.0 ** -25, 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1 + 2.0 ** -11,
             1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -20, 2047.5, 2049.0, 4095.0,
             6.1e-5, 5.96e-8, 1e-8, float("inf"), float("-inf")]
    vals = [np.float32(v) for v in edges]
    vals += list((g.standard_normal(4000) * np.exp(g.uniform(-25, 12, 4000))).astype(np.float32))
    vals += list(g.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32).view(np.float32))
    v = np.array([x for x in vals if not np.isnan(x)], np.float32)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = orc.f32_to_f16(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(ref[i])) for i in bad[:5]]
    nan = orc.f32_to_f16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0
    # every binary16 pattern back to fp32, exactly
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    back = orc.f16_to_f32(h)
    ref32 = h.view(np.float16).astype(np.float32)
    same = (back.view(np.uint32) == ref32.view(np.uint32)) | (np.isnan(back) & np.isnan(ref32))
    assert same.all()


def pin_f16_quantizer(orc):
    """Stored scale = binary16((hi - lo) / 15); codes are the nearest ones to w
    against that stored scale (exact rationals); the ends of the range are
    reproduced within half a scale plus the scale's own rounding."""
    g = np.random.default_rng(22)
    cases = [synth.weights(64, 6, cfg=102),
             (g.standard_normal((32, 4)) * 0.3 + 0.1).astype(np.float32),
             (g.standard_normal((32, 4)) * 3e-5).astype(np.float32),      # subnormal scales
             (g.standard_normal((32, 2)) * 9e4).astype(np.float32)]       # scales near the top
    for W in cases:
        K, N = W.shape
        Wq, s16, zp = orc.quantize_pack_f16(W)
        q, z = orc.unpack(Wq, zp, K, N)
        for b in range(K // 32):
            blk = W[32 * b:32 * b + 32]
            for n in range(N):
                col = blk[:, n]
                lo = min(np.float32(0), col.min())
                hi = max(np.float32(0), col.max())
                s32 = np.float32(np.float32(hi - lo) / np.float32(15))
                assert int(s16[b, n]) == int(np.array([s32]).astype(np.float16).view(np.uint16)[0])
                sn = F(np.float16(s32).astype(np.float32))
                if sn == 0:
                    assert z[b, n] == 0 and not q[32 * b:32 * b + 32, n].any()
                    continue
                zn = int(z[b, n])
                assert zn == min(15, max(0, int(np.rint(np.float32(-lo) / np.float32(sn)))))
                for k in range(32):
                    w = F(col[k])
                    t = w / sn
                    frac = t - (t.numerator // t.denominator)
                    if abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 20):
                        continue
                    errs = [abs(w - (qq - zn) * sn) for qq in range(16)]
                    assert errs[int(q[32 * b + k, n])] == min(errs)
                # the ends: within s/2 plus 15 times the scale's rounding error
                srel = abs(sn - F(s32))
                slack = sn * Fraction(1, 2 ** 18) + 16 * srel
                assert abs(F(lo) - (0 - zn) * sn) <= sn / 2 + slack
                assert abs(F(hi) - (15 - zn) * sn) <= sn / 2 + slack


def pin_f16_degenerate_and_errors(orc):
    W = np.zeros((32, 6), np.float32)
    W[:, 1] = 1e-8                    # scale below binary16's smallest: all zero codes
    W[3, 2] = 1.0                     # one weight: s = fp16(1/15)
    W[:, 3] = -0.5
    W[:, 4] = 65504.0 * 15.0 * 0.5    # scale 32752: representable
    Wq, s16, zp = orc.quantize_pack_f16(W)
    q, z = orc.unpack(Wq, zp, 32, 6)
    assert s16[0, 0] == 0 and s16[0, 1] == 0 and z[0, 1] == 0 and not q[:, 1].any()
    assert s16[0, 2] == np.array([np.float32(1) / np.float32(15)]).astype(np.float16).view(np.uint16)[0]
    assert q[3, 2] == 15 and z[0, 2] == 0
    assert z[0, 3] == 15 and not q[:, 3].any()
    assert not np.isinf(orc.f16_to_f32(s16[0, 4]))
    big = np.zeros((32, 2), np.float32)
    big[0, 0] = 1e6                   # (hi - lo) / 15 > 65504: the scale overflows
    with pytest.raises(oracle_mod.OracleError):
        orc.quantize_pack_f16(big)
    nan = np.zeros((32, 2), np.float32)
    nan[1, 1] = np.nan
    with pytest.raises(oracle_mod.OracleError):
        orc.quantize_pack_f16(nan)
    # the fp16-scale matmul is the fp32 matmul on the scales' exact values
    x = synth.activations(3, 64, cfg=103)
    W = synth.weights(64, 4, cfg=103)
    Wq, s16, zp = orc.quantize_pack_f16(W)
    y, bound = orc.w4h_matmul(x, Wq, s16, zp)
    What = orc.dequantize(Wq, orc.f16_to_f32(s16), zp, 64, 4)
    for m in range(3):
        for n in range(4):
            exact = sum(F(x[m, k]) * F(What[k, n]) for k in range(64))
            assert abs(F(y[m, n]) - exact) <= F(ulp32(y[m, n]))


# --------------------------------------------------------------------------
# fused epilogues
# --------------------------------------------------------------------------
def pin_activations(orc):
    import math
    v = np.concatenate([np.linspace(-8.0, 8.0, 161), [-30.0, -1e-3, 1e-3, 30.0]])
    g = orc.gelu(v)
    si = orc.silu(v)
    assert orc.gelu([0.0])[0] == 0.0 and orc.silu([0.0])[0] == 0.0
    for a, ga, sa in zip(v, g, si):
        # both are v times a sigmoid-like gate: f(v) - f(-v) = v
        assert abs((ga - orc.gelu([-a])[0]) - a) <= 1e-14 * (1 + abs(a))
        assert abs((sa - orc.silu([-a])[0]) - a) <= 1e-14 * (1 + abs(a))
        # the tanh form stays within 5e-4 of the exact (erf) GELU
        assert abs(ga - 0.5 * a * (1.0 + math.erf(a / math.sqrt(2.0)))) <= 5e-4
        # silu through tanh instead of exp: v/2 (1 + tanh(v/2))
        assert abs(sa - 0.5 * a * (1.0 + math.tanh(0.5 * a))) <= 1e-14 * (1 + abs(a))
    # far tails: the identity and the zero gate
    assert abs(orc.gelu([12.0])[0] - 12.0) < 1e-12 and abs(orc.gelu([-12.0])[0]) < 1e-12
    assert abs(orc.silu([-40.0])[0]) < 1e-15


def pin_epilogue_matmul(orc):
    K, N = 64, 8
    W, q, z, s = _on_grid(K, N, seed=11)
    Wq, sc, zp = orc.quantize_pack(W)
    What = orc.dequantize(Wq, sc, zp, K, N)
    assert np.array_equal(What, W)  # on-grid weights come back exactly
    b = (np.arange(N, dtype=np.float32) - 3.0) * np.float32(0.25)
    # one-hot rows: t = row k of W + bias, exact in fp64
    x = np.eye(K, dtype=np.float32)[[0, 5, 33, 63]]
    t = What[[0, 5, 33, 63]].astype(np.float64) + b[None, :]
    r4 = np.linspace(-1.0, 1.0, 4 * N, dtype=np.float32).reshape(4, N)
    # no activation: fl32(t + r)
    y, bound = orc.w4_matmul_ep(x, Wq, sc, zp, b, r4, act="none")
    for m in range(4):
        for n in range(N):
            assert y[m, n] == f32_round(F(t[m, n]) + F(r4[m, n]))
    y0, b0 = orc.w4_matmul(x, Wq, sc, zp, b)
    yn, bn = orc.w4_matmul_ep(x, Wq, sc, zp, b, None, act="none")
    assert np.array_equal(yn, y0)
    assert np.allclose(bn, b0 + np.ldexp(np.abs(y0.astype(np.float64)), -23), rtol=1e-12, atol=0)
    # GELU on t, then the residual
    y, bound = orc.w4_matmul_ep(x, Wq, sc, zp, b, r4, act="gelu")
    want = (orc.gelu(t) + r4).astype(np.float32)
    assert np.array_equal(y, want)
    assert (bound >= 1.13e-6).all() and np.isfinite(bound).all()
    # SwiGLU: columns 2i (gate) and 2i+1 (up) of t
    r2 = r4[:, : N // 2]
    y, bound = orc.w4_matmul_ep(x, Wq, sc, zp, b, r2, act="swiglu")
    assert y.shape == (4, N // 2)
    for m in range(4):
        for i in range(N // 2):
            gt, up = t[m, 2 * i], t[m, 2 * i + 1]
            gate = 0.5 * gt * (1.0 + np.tanh(0.5 * gt))  # silu(g) through tanh
            want = gate * up + float(r2[m, i])
            assert abs(float(y[m, i]) - want) <= ulp32(want) + 1e-15 * abs(gate * up), (m, i)
    # a zero gate closes its output: W's gate column 0 is zero -> y = r
    Wz = W.copy()
    Wz[:, 0] = 0.0
    Wq2, sc2, zp2 = orc.quantize_pack(Wz)
    y, _ = orc.w4_matmul_ep(x, Wq2, sc2, zp2, None, r2, act="swiglu")
    assert np.array_equal(y[:, 0], r2[:, 0])
    # an unknown activation code is a shape error
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod._check("orc_w4_matmul_ep", orc._l.orc_w4_matmul_ep(
            None, 0, K, None, None, None, N, None, None, 7, None, None))


def _gelu64(v: float) -> float:
    import math
    return 0.5 * v * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v ** 3)))


def _silu64(v: float) -> float:
    import math
    return v / (1.0 + math.exp(-v))


def _slope_max(f, lo, hi, step=1e-4):
    """Largest |f'| on [lo, hi], from central differences on a fine grid."""
    v = np.arange(lo, hi, step)
    h = 1e-6
    return max(abs(f(a + h) - f(a - h)) / (2 * h) for a in v)


def _targeted_epilogue_case(orc, targets, seed):
    """x, W_hat and exact pre-activations t[m, n] = sum_k x W_hat + b, with t
    steered close to targets[m, n] and sum_k |x W_hat| large (so the matmul
    bound dominates the activation's own rounding allowance).  Column n of W
    is nonzero on rows 8n .. 8n + 7 only, so each column's activations can be
    chosen on their own."""
    g = np.random.default_rng(seed)
    M, N = targets.shape
    K = (8 * N + 31) // 32 * 32
    W = np.zeros((K, N), np.float32)
    for n in range(N):
        W[8 * n:8 * n + 8, n] = g.standard_normal(8).astype(np.float32)
    Wq, sc, zp = orc.quantize_pack(W)
    What = orc.dequantize(Wq, sc, zp, K, N)
    assert np.all(np.isfinite(What)) and all(np.any(What[8 * n:8 * n + 8, n]) for n in range(N))
    b = (g.standard_normal(N) * 0.5).astype(np.float32)
    x = (g.standard_normal((M, K)) * 60.0).astype(np.float32)
    for m in range(M):
        for n in range(N):
            w = What[8 * n:8 * n + 8, n].astype(np.float64)
            j = int(np.argmax(np.abs(w)))
            rest = sum(float(x[m, 8 * n + i]) * w[i] for i in range(8) if i != j)
            x[m, 8 * n + j] = np.float32((targets[m, n] - float(b[n]) - rest) / w[j])
    assert np.all(np.isfinite(x))
    t = np.empty((M, N))
    tb = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            tt = sum((F(x[m, k]) * F(What[k, n]) for k in range(K)), F(b[n]))
            ab = sum((abs(F(x[m, k]) * F(What[k, n])) for k in range(K)), abs(F(b[n])))
            t[m, n] = float(tt)
            tb[m, n] = 1e-5 * float(ab) + 1e-6    # the matmul's stated tolerance
    return x, Wq, sc, zp, b, t, tb


def pin_epilogue_bound(orc):
    """The fused epilogue's tolerance, checked against the activations
    themselves: every pre-activation value the matmul bound admits must map
    inside the bound (sufficiency), and where the activation is steepest the
    bound may not exceed the worst such deviation by more than 5% (tightness).
    t is exact (rationals); the activations are evaluated in fp64 here, from
    their formulas, at many points of the admitted interval."""
    eval_allow = lambda *a: 2.0 ** -21 * sum(abs(v) for v in a)   # fp32 evaluation slack
    # slopes measured, not assumed: GELU (tanh form) and SiLU
    sg = _slope_max(_gelu64, -8.0, 8.0)
    ss = _slope_max(_silu64, -12.0, 12.0)
    assert 1.12 < sg < 1.13 and 1.09 < ss < 1.1, (sg, ss)
    v_steep = max(np.arange(0.0, 4.0, 1e-3), key=lambda a: abs(_gelu64(a + 1e-6) - _gelu64(a - 1e-6)))
    # ---- GELU: rows steered to the steepest point and across [-6, 6]
    M, N = 12, 6
    targets = np.empty((M, N))
    targets[:4] = v_steep
    targets[4:] = np.linspace(-6.0, 6.0, 8 * N).reshape(8, N)
    x, Wq, sc, zp, b, t, tb = _targeted_epilogue_case(orc, targets, seed=71)
    y, bound = orc.w4_matmul_ep(x, Wq, sc, zp, b, None, act="gelu")
    tight = 0
    for m in range(M):
        for n in range(N):
            o = _gelu64(t[m, n])
            dev_max = max(abs(_gelu64(tp) - o) for tp in np.linspace(t[m, n] - tb[m, n],
                                                                     t[m, n] + tb[m, n], 41))
            need = dev_max + eval_allow(t[m, n], o)
            assert bound[m, n] >= need, ("gelu bound too small", m, n, bound[m, n], need)
            if m < 4 and tb[m, n] > 2.0 ** -13 * (abs(t[m, n]) + abs(o)):
                assert bound[m, n] <= 1.05 * dev_max + 2.0 ** -17 * (abs(t[m, n]) + abs(o)), \
                    ("gelu bound too loose", m, n, bound[m, n], dev_max)
                tight += 1
    assert tight >= 12  # the steep-point rows were reached
    # ---- SwiGLU: gate near SiLU's steepest point, large up values; and spread
    v_ss = max(np.arange(0.0, 6.0, 1e-3), key=lambda a: abs(_silu64(a + 1e-6) - _silu64(a - 1e-6)))
    M, N = 12, 8
    targets = np.empty((M, N))
    targets[:, 0::2] = v_ss
    targets[:, 1::2] = np.where(np.arange(M)[:, None] % 2 == 0, 12.0, -9.0)
    targets[6:, 0::2] = np.linspace(-8.0, 8.0, 6 * (N // 2)).reshape(6, N // 2)
    x, Wq, sc, zp, b, t, tb = _targeted_epilogue_case(orc, targets, seed=72)
    y, bound = orc.w4_matmul_ep(x, Wq, sc, zp, b, None, act="swiglu")
    tight = 0
    for m in range(M):
        for i in range(N // 2):
            gt, ut, gb, ub = t[m, 2 * i], t[m, 2 * i + 1], tb[m, 2 * i], tb[m, 2 * i + 1]
            o = _silu64(gt) * ut
            dev_max = max(abs(_silu64(gp) * up - o)
                          for gp in np.linspace(gt - gb, gt + gb, 17)
                          for up in np.linspace(ut - ub, ut + ub, 9))
            need = dev_max + eval_allow(gt * ut, o)
            assert bound[m, i] >= need, ("swiglu bound too small", m, i, bound[m, i], need)
            if m < 6 and gb * abs(ut) > 2.0 ** -13 * (abs(gt * ut) + abs(o)):
                assert bound[m, i] <= 1.05 * dev_max + 2.0 ** -17 * (abs(gt * ut) + abs(o)), \
                    ("swiglu bound too loose", m, i, bound[m, i], dev_max)
                tight += 1
    assert tight >= 12


# --------------------------------------------------------------------------
# group-64 affine variant
# --------------------------------------------------------------------------
GROUP = 64


def _on_grid_g64(K, N, seed):
    """w = q * 2**e + m per group, with m a multiple of 2**e and codes 0 and 15
    both present, so that s = 2**e and the minimum m are exact."""
    g = np.random.default_rng(seed)
    ng = K // GROUP
    e = g.integers(-10, -3, size=(ng, N))
    mz = g.integers(-40, 20, size=(ng, N))
    q = g.integers(0, 16, size=(K, N)).astype(np.uint8)
    for b in range(ng):
        for n in range(N):
            r0, r1 = g.choice(GROUP, size=2, replace=False)
            q[b * GROUP + r0, n] = 0
            q[b * GROUP + r1, n] = 15
    s = np.ldexp(np.float32(1.0), e).astype(np.float32)
    m = (mz * s).astype(np.float32)
    W = (q.astype(np.float32) * np.repeat(s, GROUP, axis=0) +
         np.repeat(m, GROUP, axis=0)).astype(np.float32)
    return W, q, s, m


def pin_g64_on_grid_and_layout(orc):
    K, N = 192, 6
    W, q, s, m = _on_grid_g64(K, N, seed=21)
    Wq, sc, mn = orc.quantize_pack_g64(W)
    assert np.array_equal(sc, s) and np.array_equal(mn, m)
    assert np.array_equal(orc.unpack_u4(Wq).reshape(K, N), q)
    assert np.array_equal(orc.dequantize_g64(Wq, sc, mn, K, N), W)
    # bytes per weight: 4-bit codes plus two fp32 per 64 weights
    assert Wq.nbytes + sc.nbytes + mn.nbytes == K * N * 5 // 8
    # K-major copy: transposed codes packed along K, scales and mins transposed
    Pq, Ps, Pm = orc.prepack_kmajor_g64(Wq, sc, mn, K, N)
    assert np.array_equal(orc.unpack_u4(Pq).reshape(N, K), np.ascontiguousarray(q.T))
    assert np.array_equal(Ps, np.ascontiguousarray(s.T)) and np.array_equal(Pm, np.ascontiguousarray(m.T))
    for bad in ((32, 4), (64, 3)):
        with pytest.raises(oracle_mod.OracleError):
            orc.quantize_pack_g64(np.zeros(bad, np.float32))


def pin_g64_nearest_code_and_bounds(orc):
    g = np.random.default_rng(22)
    cases = [synth.weights(64, 4, cfg=121),
             (g.standard_normal((64, 4)) * 0.3 + 0.1).astype(np.float32),
             np.abs(g.standard_normal((128, 2))).astype(np.float32) + np.float32(5.0)]
    for W in cases:
        K, N = W.shape
        Wq, sc, mn = orc.quantize_pack_g64(W)
        q = orc.unpack_u4(Wq).reshape(K, N)
        What = orc.dequantize_g64(Wq, sc, mn, K, N)
        for b in range(K // GROUP):
            for n in range(N):
                col = W[b * GROUP:(b + 1) * GROUP, n]
                lo, hi = F(col.min()), F(col.max())
                sn, mm = F(sc[b, n]), F(mn[b, n])
                assert mm == lo                             # the offset is the minimum
                assert abs(sn - (hi - lo) / 15) <= F(ulp32(float(sn)))
                for r in range(GROUP):
                    k = b * GROUP + r
                    w = F(W[k, n])
                    t = (w - mm) / sn
                    frac = t - (t.numerator // t.denominator)
                    if abs(frac - Fraction(1, 2)) >= Fraction(1, 2 ** 20):
                        errs = [abs(w - (qq * sn + mm)) for qq in range(16)]
                        assert errs[int(q[k, n])] == min(errs), (k, n)
                    # round trip: half a step plus the roundings of w - lo, of
                    # the quotient and of W_hat
                    assert abs(F(What[k, n]) - w) <= sn / 2 + sn * Fraction(1, 2 ** 18) + \
                        F(ulp32(float(W[k, n])))
                kmin = b * GROUP + int(np.argmin(col))
                assert int(q[kmin, n]) == 0 and What[kmin, n] == col.min()
    # a constant group: s = 0, every code 0, W_hat = the constant exactly
    Wc = np.full((64, 2), np.float32(-0.3), np.float32)
    Wc[:, 1] = np.float32(7.25)
    Wq, sc, mn = orc.quantize_pack_g64(Wc)
    assert (sc == 0).all() and not orc.unpack_u4(Wq).any()
    assert np.array_equal(orc.dequantize_g64(Wq, sc, mn, 64, 2), Wc)
    bad = np.zeros((64, 2), np.float32)
    bad[3, 1] = np.inf
    with pytest.raises(oracle_mod.OracleError):
        orc.quantize_pack_g64(bad)


def pin_g64_dequant_and_matmul(orc):
    # every code with sampled scales and offsets: W_hat = q s + m rounded once
    ng, N = 4, 16
    K = ng * GROUP
    q = np.array([[(k + n) % 16 for n in range(N)] for k in range(K)], np.uint8)
    g = np.random.default_rng(23)
    s = (np.abs(g.standard_normal((ng, N))) * 0.01).astype(np.float32)
    m = (g.standard_normal((ng, N)) * 0.05).astype(np.float32)
    s[0, :3] = [np.float32(1e-40), np.float32(1.0) / np.float32(3.0), np.float32(2.0 ** 60)]
    m[0, :3] = [np.float32(0.0), np.float32(-5.0), np.float32(-(2.0 ** 63))]
    Wq = orc.pack_u4(q.reshape(-1)).reshape(K, N // 2)
    What = orc.dequantize_g64(Wq, s, m, K, N)
    for k in range(K):
        for n in range(N):
            b = k // GROUP
            want = f32_round(int(q[k, n]) * F(s[b, n]) + F(m[b, n]))
            assert What[k, n] == want, (k, n, What[k, n], want)
    # the matmul is the plain fp64 matmul on W_hat, exact on tiny shapes
    for M, K, N in ((1, 64, 2), (3, 128, 6)):
        W = synth.weights(K, N, cfg=124, slot=M)
        x = synth.activations(M, K, cfg=124, slot=M, outliers=True)
        b = synth.bias(N, cfg=124, slot=M)
        Wq, sc, mn = orc.quantize_pack_g64(W)
        What = orc.dequantize_g64(Wq, sc, mn, K, N)
        for bias in (None, b):
            y, bound = orc.w4g_matmul(x, Wq, sc, mn, bias)
            _exact_check(y, bound, x, What, bias)


ALL_PINS = [
    pin_g64_on_grid_and_layout,
    pin_g64_nearest_code_and_bounds,
    pin_g64_dequant_and_matmul,
    pin_activations,
    pin_epilogue_matmul,
    pin_epilogue_bound,
    pin_f16_conversion,
    pin_f16_quantizer,
    pin_f16_degenerate_and_errors,
    pin_pack_worked_examples,
    pin_pack_exhaustive,
    pin_quantize_on_grid,
    pin_quantize_ties_half_even,
    pin_round_trip_bound,
    pin_nearest_code_bruteforce,
    pin_degenerate_blocks,
    pin_shape_and_value_errors,
    pin_dequant_all_pairs,
    pin_prepack_kmajor,
    pin_matmul_exact_small,
    pin_matmul_special_cases,
    pin_head_quantizer,
    pin_head_logits,
    pin_embedding,
    pin_file_size,
]
