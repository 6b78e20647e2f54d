"""CPU oracle for the 4-bit block-dequant matmul and the int8 tied head.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package.
Only the tests, the smoke check and the benchmark's CPU-baseline leg call it.
It shares no code with the HIP library (``w4_block_dequant_amd``) and does not
import it; the two meet only in the tests, which feed both the same seeded
inputs from the separate ``synth`` module.

The arithmetic lives in plain C (``oracle.c``, built with gcc, no fast-math,
no FMA contraction); this file only builds the shared object and marshals
numpy arrays.  What each function computes, and the passage of the page
"ONNX export, quantization and the browser runtime" it follows, is stated in
``oracle.h``.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, exhaustive enumeration, exact rational arithmetic and special
cases (see that file's header).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
          "-shared", "-Wall", "-Wextra"]

OK, BAD_SHAPE, NONFINITE, NO_MEMORY = 0, 1, 2, 3
BLOCK = 32
GROUP = 64


class OracleError(RuntimeError):
    """A nonzero status from the C oracle."""

    def __init__(self, fn: str, status: int):
        names = {BAD_SHAPE: "BAD_SHAPE", NONFINITE: "NONFINITE", NO_MEMORY: "NO_MEMORY"}
        super().__init__(f"{fn}: status {status} ({names.get(status, '?')})")
        self.status = status


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``src`` into the shared object ``out`` with gcc (about a second)."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64

_SIGS = {
    "orc_set_threads": (None, [ctypes.c_int]),
    "orc_get_threads": (ctypes.c_int, []),
    "orc_pack_u4": (None, [_P, _I64, _P]),
    "orc_unpack_u4": (None, [_P, _I64, _P]),
    "orc_w4_quantize_pack": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "orc_w4_unpack": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "orc_w4_dequantize": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "orc_w4_prepack_kmajor": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P, _P]),
    "orc_matmul_f64": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, _P]),
    "orc_w4_matmul": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P]),
    "orc_i8_quantize_head": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P]),
    "orc_i8_dequantize_head": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _P]),
    "orc_i8_head_logits": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, _P, _P]),
    "orc_i8_embed": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, _I64, _P]),
    "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
    "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
    "orc_f16_array_to_f32": (None, [_P, _I64, _P]),
    "orc_w4h_quantize_pack": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "orc_w4g_quantize_pack": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "orc_w4g_dequantize": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "orc_w4g_prepack_kmajor": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P, _P]),
    "orc_w4g_matmul": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P]),
    "orc_gelu": (ctypes.c_double, [ctypes.c_double]),
    "orc_silu": (ctypes.c_double, [ctypes.c_double]),
    "orc_w4_matmul_ep": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, ctypes.c_int,
                                         _P, _P]),
}


def load_library(path: str):
    """Load a compiled oracle (the default one, or a variant a test built)."""
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _stale() -> bool:
    if not os.path.exists(_LIB):
        return True
    t = os.path.getmtime(_LIB)
    return any(os.path.getmtime(p) > t for p in (_SRC, _HDR))


def lib():
    """The default oracle library, built on first use if missing or stale."""
    global _lib
    with _lock:
        if _lib is None:
            if _stale():
                build()
            _lib = load_library(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(fn: str, st: int):
    if st != OK:
        raise OracleError(fn, st)


class Oracle:
    """numpy front end over one compiled oracle library."""

    def __init__(self, clib=None):
        self._l = clib if clib is not None else lib()

    # -- threads (results do not depend on them) ----------------------------
    def set_threads(self, n: int):
        self._l.orc_set_threads(int(n))

    def threads(self) -> int:
        return int(self._l.orc_get_threads())

    # -- nibble packing -------------------------------------------------------
    def pack_u4(self, v):
        v = _c(v, np.uint8).reshape(-1)
        assert v.size % 2 == 0
        out = np.empty(v.size // 2, np.uint8)
        self._l.orc_pack_u4(_ptr(v), v.size, _ptr(out))
        return out

    def unpack_u4(self, packed):
        p = _c(packed, np.uint8).reshape(-1)
        v = np.empty(p.size * 2, np.uint8)
        self._l.orc_unpack_u4(_ptr(p), v.size, _ptr(v))
        return v

    # -- 4-bit block format -----------------------------------------------------
    def quantize_pack(self, W):
        """W fp32 [K, N] -> (Wq uint8 [K, N/2], scales fp32 [K/32, N], zeros uint8 [K/32, N/2])."""
        W = _c(W, np.float32)
        K, N = W.shape
        Wq = np.zeros((K, N // 2), np.uint8)
        s = np.zeros((K // BLOCK, N), np.float32)
        z = np.zeros((K // BLOCK, N // 2), np.uint8)
        _check("orc_w4_quantize_pack",
               self._l.orc_w4_quantize_pack(_ptr(W), K, N, _ptr(Wq), _ptr(s), _ptr(z)))
        return Wq, s, z

    def unpack(self, Wq, zeros, K, N):
        """-> (q uint8 [K, N], z uint8 [K/32, N])."""
        q = np.zeros((K, N), np.uint8)
        z = np.zeros((K // BLOCK, N), np.uint8)
        _check("orc_w4_unpack", self._l.orc_w4_unpack(_ptr(_c(Wq, np.uint8)),
                                                      _ptr(_c(zeros, np.uint8)), K, N,
                                                      _ptr(q), _ptr(z)))
        return q, z

    def dequantize(self, Wq, scales, zeros, K, N):
        """-> W_hat fp32 [K, N]."""
        out = np.zeros((K, N), np.float32)
        _check("orc_w4_dequantize",
               self._l.orc_w4_dequantize(_ptr(_c(Wq, np.uint8)), _ptr(_c(scales, np.float32)),
                                         _ptr(_c(zeros, np.uint8)), K, N, _ptr(out)))
        return out

    def prepack_kmajor(self, Wq, scales, zeros, K, N):
        """-> (Pq uint8 [N, K/2], Ps fp32 [N, K/32], Pz uint8 [N, K/64])."""
        Pq = np.zeros((N, K // 2), np.uint8)
        Ps = np.zeros((N, K // BLOCK), np.float32)
        Pz = np.zeros((N, K // 64), np.uint8)
        _check("orc_w4_prepack_kmajor",
               self._l.orc_w4_prepack_kmajor(_ptr(_c(Wq, np.uint8)), _ptr(_c(scales, np.float32)),
                                             _ptr(_c(zeros, np.uint8)), K, N, _ptr(Pq), _ptr(Ps),
                                             _ptr(Pz)))
        return Pq, Ps, Pz

    def matmul_f64(self, x, W, bias=None):
        """x fp32 [M, K], W fp32 [K, N] -> (y fp32 [M, N], bound fp64 [M, N])."""
        x = _c(x, np.float32)
        W = _c(W, np.float32)
        M, K = x.shape
        K2, N = W.shape
        assert K == K2
        b = None if bias is None else _c(bias, np.float32)
        y = np.zeros((M, N), np.float32)
        bound = np.zeros((M, N), np.float64)
        _check("orc_matmul_f64", self._l.orc_matmul_f64(_ptr(x), M, K, _ptr(W), N, _ptr(b),
                                                        _ptr(y), _ptr(bound)))
        return y, bound

    def w4_matmul(self, x, Wq, scales, zeros, bias=None):
        """y = x . dequantize(Wq, scales, zeros) (+ bias) -> (y [M, N], bound [M, N])."""
        x = _c(x, np.float32)
        M, K = x.shape
        N = _c(scales, np.float32).shape[1]
        b = None if bias is None else _c(bias, np.float32)
        y = np.zeros((M, N), np.float32)
        bound = np.zeros((M, N), np.float64)
        _check("orc_w4_matmul",
               self._l.orc_w4_matmul(_ptr(x), M, K, _ptr(_c(Wq, np.uint8)),
                                     _ptr(_c(scales, np.float32)), _ptr(_c(zeros, np.uint8)),
                                     N, _ptr(b), _ptr(y), _ptr(bound)))
        return y, bound

    # -- group-64 affine variant ---------------------------------------------------
    def quantize_pack_g64(self, W):
        """W fp32 [K, N] -> (Wq uint8 [K, N/2], scales fp32 [K/64, N], mins fp32 [K/64, N])."""
        W = _c(W, np.float32)
        K, N = W.shape
        Wq = np.zeros((K, N // 2), np.uint8)
        s = np.zeros((K // GROUP, N), np.float32)
        m = np.zeros((K // GROUP, N), np.float32)
        _check("orc_w4g_quantize_pack", self._l.orc_w4g_quantize_pack(
            _ptr(W), K, N, _ptr(Wq), _ptr(s), _ptr(m)))
        return Wq, s, m

    def dequantize_g64(self, Wq, scales, mins, K, N):
        out = np.zeros((K, N), np.float32)
        _check("orc_w4g_dequantize", self._l.orc_w4g_dequantize(
            _ptr(_c(Wq, np.uint8)), _ptr(_c(scales, np.float32)), _ptr(_c(mins, np.float32)),
            K, N, _ptr(out)))
        return out

    def prepack_kmajor_g64(self, Wq, scales, mins, K, N):
        """-> (Pq uint8 [N, K/2], Ps fp32 [N, K/64], Pm fp32 [N, K/64])."""
        Pq = np.zeros((N, K // 2), np.uint8)
        Ps = np.zeros((N, K // GROUP), np.float32)
        Pm = np.zeros((N, K // GROUP), np.float32)
        _check("orc_w4g_prepack_kmajor", self._l.orc_w4g_prepack_kmajor(
            _ptr(_c(Wq, np.uint8)), _ptr(_c(scales, np.float32)), _ptr(_c(mins, np.float32)),
            K, N, _ptr(Pq), _ptr(Ps), _ptr(Pm)))
        return Pq, Ps, Pm

    def w4g_matmul(self, x, Wq, scales, mins, bias=None):
        """y = x . dequantize_g64(W) (+ bias) -> (y [M, N], bound [M, N])."""
        x = _c(x, np.float32)
        M, K = x.shape
        N = _c(scales, np.float32).shape[1]
        b = None if bias is None else _c(bias, np.float32)
        y = np.zeros((M, N), np.float32)
        bound = np.zeros((M, N), np.float64)
        _check("orc_w4g_matmul", self._l.orc_w4g_matmul(
            _ptr(x), M, K, _ptr(_c(Wq, np.uint8)), _ptr(_c(scales, np.float32)),
            _ptr(_c(mins, np.float32)), N, _ptr(b), _ptr(y), _ptr(bound)))
        return y, bound

    # -- fused epilogues -----------------------------------------------------------
    ACTS = {"none": 0, "gelu": 1, "swiglu": 2}

    def gelu(self, v):
        """gelu (tanh form) of each element, fp64."""
        f = self._l.orc_gelu
        return np.array([f(float(a)) for a in np.asarray(v, np.float64).reshape(-1)]).reshape(
            np.shape(v))

    def silu(self, v):
        """silu of each element, fp64."""
        f = self._l.orc_silu
        return np.array([f(float(a)) for a in np.asarray(v, np.float64).reshape(-1)]).reshape(
            np.shape(v))

    def w4_matmul_ep(self, x, Wq, scales, zeros, bias=None, residual=None, act="none"):
        """act(x . dequantize(W) + bias) (+ residual) -> (y [M, N_out], bound [M, N_out])."""
        x = _c(x, np.float32)
        M, K = x.shape
        N = _c(scales, np.float32).shape[1]
        a = self.ACTS[act]
        nout = N // 2 if act == "swiglu" else N
        b = None if bias is None else _c(bias, np.float32)
        r = None if residual is None else _c(residual, np.float32)
        y = np.zeros((M, nout), np.float32)
        bound = np.zeros((M, nout), np.float64)
        _check("orc_w4_matmul_ep",
               self._l.orc_w4_matmul_ep(_ptr(x), M, K, _ptr(_c(Wq, np.uint8)),
                                        _ptr(_c(scales, np.float32)), _ptr(_c(zeros, np.uint8)),
                                        N, _ptr(b), _ptr(r), a, _ptr(y), _ptr(bound)))
        return y, bound

    # -- fp16-scale variant ------------------------------------------------------
    def f32_to_f16(self, v):
        """fp32 array -> binary16 bit patterns (uint16), one oracle call per element."""
        v = _c(v, np.float32).reshape(-1)
        out = np.empty(v.size, np.uint16)
        for i in range(v.size):
            out[i] = self._l.orc_f32_to_f16(float(v[i]))
        return out

    def f16_to_f32(self, h):
        """binary16 bit patterns -> fp32."""
        h = _c(h, np.uint16)
        out = np.empty(h.shape, np.float32)
        self._l.orc_f16_array_to_f32(_ptr(h), h.size, _ptr(out))
        return out

    def quantize_pack_f16(self, W):
        """W fp32 [K, N] -> (Wq uint8 [K, N/2], scales uint16 [K/32, N] (binary16), zeros)."""
        W = _c(W, np.float32)
        K, N = W.shape
        Wq = np.zeros((K, N // 2), np.uint8)
        s = np.zeros((K // BLOCK, N), np.uint16)
        z = np.zeros((K // BLOCK, N // 2), np.uint8)
        _check("orc_w4h_quantize_pack",
               self._l.orc_w4h_quantize_pack(_ptr(W), K, N, _ptr(Wq), _ptr(s), _ptr(z)))
        return Wq, s, z

    def w4h_matmul(self, x, Wq, scales16, zeros, bias=None):
        """The fp16-scale format's matmul: the scales' fp32 values, then w4_matmul."""
        return self.w4_matmul(x, Wq, self.f16_to_f32(scales16), zeros, bias)

    def prepack_kmajor_f16(self, Wq, scales16, zeros, K, N):
        """K-major copy with binary16 scales: (Pq, Ps uint16 [N, K/32], Pz)."""
        Pq, Ps, Pz = self.prepack_kmajor(Wq, self.f16_to_f32(scales16), zeros, K, N)
        back = self.f32_to_f16(Ps).reshape(Ps.shape)  # exact: every value came from binary16
        return Pq, back, Pz

    # -- int8 head -------------------------------------------------------------
    def i8_quantize_head(self, E, ldq=None):
        """E fp32 [K, N] -> (Q int8 [K, ldq], hs fp32 [N])."""
        E = _c(E, np.float32)
        K, N = E.shape
        ldq = N if ldq is None else ldq
        Q = np.zeros((K, ldq), np.int8)
        hs = np.zeros(N, np.float32)
        _check("orc_i8_quantize_head",
               self._l.orc_i8_quantize_head(_ptr(E), K, N, ldq, _ptr(Q), _ptr(hs)))
        return Q, hs

    def i8_dequantize_head(self, Q, hs):
        Q = _c(Q, np.int8)
        hs = _c(hs, np.float32)
        K, ldq = Q.shape
        N = hs.size
        out = np.zeros((K, N), np.float32)
        _check("orc_i8_dequantize_head",
               self._l.orc_i8_dequantize_head(_ptr(Q), ldq, _ptr(hs), K, N, _ptr(out)))
        return out

    def i8_head_logits(self, x_last, Q, hs):
        """x_last fp32 [K] -> (logits fp32 [N], bound fp64 [N])."""
        x = _c(x_last, np.float32).reshape(-1)
        Q = _c(Q, np.int8)
        hs = _c(hs, np.float32)
        K, ldq = Q.shape
        assert x.size == K
        N = hs.size
        out = np.zeros(N, np.float32)
        bound = np.zeros(N, np.float64)
        _check("orc_i8_head_logits",
               self._l.orc_i8_head_logits(_ptr(x), K, _ptr(Q), ldq, _ptr(hs), N, _ptr(out),
                                          _ptr(bound)))
        return out, bound

    def i8_embed(self, tokens, Q, hs):
        """tokens int64 [T] -> fp32 [T, K] rows of the dequantized table."""
        t = _c(tokens, np.int64).reshape(-1)
        Q = _c(Q, np.int8)
        hs = _c(hs, np.float32)
        K, ldq = Q.shape
        N = hs.size
        out = np.zeros((t.size, K), np.float32)
        _check("orc_i8_embed", self._l.orc_i8_embed(_ptr(t), t.size, _ptr(Q), ldq, _ptr(hs),
                                                    K, N, _ptr(out)))
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
