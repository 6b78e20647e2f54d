"""Python binding of libw4.so, the gfx950 4-bit block-dequant matmul library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/w4.h``.  PyTorch supplies device
memory and the current stream; nothing here computes on the host.  The
functions carry the C names:

    w4_quantize_pack(W)                    -> (Wq, scales, zeros)
    w4_unpack(Wq, zeros, K, N)             -> (q, z)
    w4_dequantize(Wq, scales, zeros)       -> W_hat
    w4_matmul(x, Wq, scales, zeros, bias)  -> y
    w4_prepack_kmajor(Wq, scales, zeros)   -> (Pq, Ps, Pz)  K-major copy
    w4_matmul_kmajor(x, Pq, Ps, Pz, bias)  -> y             decode GEMV on it
    i8_quantize_head(E, ldq)               -> (Q, hs)
    i8_head_logits(x_last, Q, hs)          -> logits
    i8_embed(tokens, Q, hs)                -> rows of the dequantized table

If the library has not been built this module raises ImportError: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # loaded first: libw4.so then binds to the HIP runtime torch loaded

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python w4_block_dequant_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

_P, _I64, _SZ, _INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
_SIGS = {
    "w4_abi_version": (_INT, []),
    "w4_strerror": (ctypes.c_char_p, [_INT]),
    "w4_quantize_pack": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "w4_unpack": (_INT, [_P, _P, _I64, _I64, _P, _P, _P]),
    "w4_dequantize": (_INT, [_P, _P, _P, _I64, _I64, _P, _P]),
    "w4_matmul_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "w4_matmul": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _SZ, _P]),
    "w4_check_matmul_args": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _SZ]),
    "w4_matmul_noalloc": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P]),
    "w4_read_bytes_words": (_SZ, [_I64, _INT]),
    "w4_read_bytes": (_INT, [_P, _I64, _INT, _P, _P]),
    "w4_prepack_kmajor": (_INT, [_P, _P, _P, _I64, _I64, _P, _P, _P, _P]),
    "w4_matmul_kmajor_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "w4_matmul_kmajor": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _SZ, _P]),
    "w4_check_matmul_kmajor_args": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _SZ]),
    "i8_quantize_head": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "i8_head_workspace_bytes": (_SZ, [_I64, _I64]),
    "i8_head_logits": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _SZ, _P]),
    "i8_embed": (_INT, [_P, _I64, _P, _I64, _P, _I64, _I64, _P, _P, _P]),
    "i8_prepack_head": (_INT, [_P, _I64, _I64, _I64, _P, _I64, _P]),
    "i8_check_head_logits_kmajor_args": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P]),
    "i8_head_logits_kmajor": (_INT, [_P, _I64, _P, _I64, _P, _I64, _P, _P]),
    "i8_embed_kmajor": (_INT, [_P, _I64, _P, _I64, _P, _I64, _I64, _P, _P, _P]),
    "w4h_quantize_pack": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "w4h_dequantize": (_INT, [_P, _P, _P, _I64, _I64, _P, _P]),
    "w4h_prepack_kmajor": (_INT, [_P, _P, _P, _I64, _I64, _P, _P, _P, _P]),
    "w4h_check_matmul_kmajor_args": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _SZ]),
    "w4h_matmul_kmajor": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _SZ, _P]),
    "i8_head_rows_workspace_bytes": (_SZ, [_I64, _I64]),
    "w4g_quantize_pack": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "w4g_dequantize": (_INT, [_P, _P, _P, _I64, _I64, _P, _P]),
    "w4g_prepack_kmajor": (_INT, [_P, _P, _P, _I64, _I64, _P, _P, _P, _P]),
    "w4g_check_matmul_kmajor_args": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P]),
    "w4g_matmul_kmajor": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P]),
    "w4_check_matmul_kmajor_ep_args": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _INT, _P,
                                              _P, _SZ]),
    "w4_matmul_kmajor_ep": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _INT, _P, _P, _SZ,
                                   _P]),
    "i8_check_head_logits_rows_args": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _SZ]),
    "i8_head_logits_rows": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _SZ, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

W4_OK, W4_ERR_NULL_PTR, W4_ERR_BAD_SHAPE, W4_ERR_MISALIGNED = 0, 1, 2, 3
W4_ERR_WORKSPACE, W4_ERR_DEVICE, W4_ERR_LAUNCH, W4_ERR_NONFINITE = 4, 5, 6, 7
BLOCK = 32


class W4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {w4_strerror(status)} (status {status})")
        self.status = status


def library():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def w4_abi_version() -> int:
    return _lib.w4_abi_version()


def w4_strerror(status: int) -> str:
    return _lib.w4_strerror(status).decode()


def _check(fn: str, st: int):
    if st != W4_OK:
        raise W4Error(fn, st)


def _dev(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a tensor on a HIP device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Workspace:
    """Device scratch for split-K partial sums, grown on demand.

    One buffer per (device, stream): calls on one stream run in order, so
    they can share it, and a call on another stream gets a buffer of its own
    (two streams sharing one buffer would race on the partial sums).  A
    buffer that is outgrown is kept alive, not freed: a HIP graph captured
    with it still names its address, and freeing it would let the caching
    allocator hand that memory to another tensor under the graph.
    """

    def __init__(self):
        self._buf = {}
        self._retired = []
        self._lock = threading.Lock()

    def get(self, device, nbytes: int):
        if nbytes == 0:
            return None, 0
        key = (torch.device(device).index, _stream(device))
        with self._lock:
            buf = self._buf.get(key)
            if buf is None or buf.numel() < nbytes:
                if buf is not None:
                    self._retired.append(buf)
                size = max(nbytes, 1 << 20, 2 * (buf.numel() if buf is not None else 0))
                buf = torch.empty(size, dtype=torch.uint8, device=device)
                self._buf[key] = buf
        return buf, buf.numel()


_workspace = Workspace()


def w4_quantize_pack(W: torch.Tensor, d_status: torch.Tensor | None = None):
    """W fp32 [K, N] -> (Wq uint8 [K, N/2], scales fp32 [K/32, N], zeros uint8 [K/32, N/2])."""
    _dev(W, torch.float32, "W")
    K, N = W.shape
    Wq = torch.empty((K, N // 2), dtype=torch.uint8, device=W.device)
    s = torch.empty((K // BLOCK, N), dtype=torch.float32, device=W.device)
    z = torch.empty((K // BLOCK, N // 2), dtype=torch.uint8, device=W.device)
    if d_status is not None:
        _dev(d_status, torch.int32, "d_status")
    _check("w4_quantize_pack", _lib.w4_quantize_pack(
        _ptr(W), K, N, _ptr(Wq), _ptr(s), _ptr(z), _ptr(d_status), _stream(W.device)))
    return Wq, s, z


def w4_unpack(Wq: torch.Tensor, zeros: torch.Tensor, K: int, N: int):
    """-> (q uint8 [K, N], z uint8 [K/32, N])."""
    _dev(Wq, torch.uint8, "Wq")
    _dev(zeros, torch.uint8, "zeros")
    q = torch.empty((K, N), dtype=torch.uint8, device=Wq.device)
    z = torch.empty((K // BLOCK, N), dtype=torch.uint8, device=Wq.device)
    _check("w4_unpack", _lib.w4_unpack(_ptr(Wq), _ptr(zeros), K, N, _ptr(q), _ptr(z),
                                       _stream(Wq.device)))
    return q, z


def w4_dequantize(Wq: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor):
    """-> W_hat fp32 [K, N]."""
    _dev(Wq, torch.uint8, "Wq")
    _dev(scales, torch.float32, "scales")
    _dev(zeros, torch.uint8, "zeros")
    K, N = Wq.shape[0], scales.shape[1]
    out = torch.empty((K, N), dtype=torch.float32, device=Wq.device)
    _check("w4_dequantize", _lib.w4_dequantize(_ptr(Wq), _ptr(scales), _ptr(zeros), K, N,
                                               _ptr(out), _stream(Wq.device)))
    return out


def w4_matmul_workspace_bytes(M: int, K: int, N: int) -> int:
    return _lib.w4_matmul_workspace_bytes(M, K, N)


def w4_matmul(x: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
              bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None):
    """y fp32 [M, N] = x [M, K] . dequantize(Wq, scales, zeros) (+ bias)."""
    _dev(x, torch.float32, "x")
    _dev(Wq, torch.uint8, "Wq")
    _dev(scales, torch.float32, "scales")
    _dev(zeros, torch.uint8, "zeros")
    if bias is not None:
        _dev(bias, torch.float32, "bias")
    M, K = x.shape
    N = scales.shape[1]
    if Wq.shape != (K, N // 2):
        raise ValueError(f"Wq shape {tuple(Wq.shape)} does not match K={K}, N={N}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    else:
        _dev(out, torch.float32, "out")
    need = _lib.w4_matmul_workspace_bytes(M, K, N)
    if workspace is None:
        ws, wsb = _workspace.get(x.device, need)
    else:
        _dev(workspace, torch.uint8, "workspace")
        ws, wsb = workspace, workspace.numel()
    _check("w4_matmul", _lib.w4_matmul(_ptr(x), M, K, _ptr(Wq), _ptr(scales), _ptr(zeros), N,
                                       _ptr(bias), _ptr(out), _ptr(ws), wsb,
                                       _stream(x.device)))
    return out


def w4_read_bytes(src: torch.Tensor, loads_per_lane: int = 8, out: torch.Tensor | None = None):
    """Streaming-read reference over a contiguous uint8 tensor (the benchmark's
    launch floor); returns the per-workgroup XOR words."""
    _dev(src, torch.uint8, "src")
    n = src.numel()
    words = _lib.w4_read_bytes_words(n, loads_per_lane)
    if out is None:
        out = torch.empty(max(words, 1), dtype=torch.int32, device=src.device)
    _check("w4_read_bytes", _lib.w4_read_bytes(_ptr(src), n, loads_per_lane, _ptr(out),
                                               _stream(src.device)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def w4_matmul_noalloc(x: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor,
                      zeros: torch.Tensor, bias: torch.Tensor | None = None,
                      out: torch.Tensor | None = None):
    """w4_matmul through the allocation-free entry point (the library's own
    per-GPU scratch; calls on one GPU must not overlap)."""
    _dev(x, torch.float32, "x")
    _dev(Wq, torch.uint8, "Wq")
    _dev(scales, torch.float32, "scales")
    _dev(zeros, torch.uint8, "zeros")
    if bias is not None:
        _dev(bias, torch.float32, "bias")
    M, K = x.shape
    N = scales.shape[1]
    if Wq.shape != (K, N // 2):
        raise ValueError(f"Wq shape {tuple(Wq.shape)} does not match K={K}, N={N}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    else:
        _dev(out, torch.float32, "out")
    _check("w4_matmul_noalloc", _lib.w4_matmul_noalloc(
        _ptr(x), M, K, _ptr(Wq), _ptr(scales), _ptr(zeros), N, _ptr(bias), _ptr(out),
        _stream(x.device)))
    return out


def w4_prepack_kmajor(Wq: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor):
    """Canonical layout -> K-major copy (Pq uint8 [N, K/2], Ps fp32 [N, K/32], Pz uint8 [N, K/64])."""
    _dev(Wq, torch.uint8, "Wq")
    _dev(scales, torch.float32, "scales")
    _dev(zeros, torch.uint8, "zeros")
    K, N = Wq.shape[0], scales.shape[1]
    Pq = torch.empty((N, K // 2), dtype=torch.uint8, device=Wq.device)
    Ps = torch.empty((N, K // BLOCK), dtype=torch.float32, device=Wq.device)
    Pz = torch.empty((N, K // 64), dtype=torch.uint8, device=Wq.device)
    _check("w4_prepack_kmajor", _lib.w4_prepack_kmajor(
        _ptr(Wq), _ptr(scales), _ptr(zeros), K, N, _ptr(Pq), _ptr(Ps), _ptr(Pz),
        _stream(Wq.device)))
    return Pq, Ps, Pz


def w4_matmul_kmajor_workspace_bytes(M: int, K: int, N: int) -> int:
    return _lib.w4_matmul_kmajor_workspace_bytes(M, K, N)


ACTS = {"none": 0, "gelu": 1, "swiglu": 2}  # W4_ACT_NONE, W4_ACT_GELU, W4_ACT_SWIGLU


def w4_matmul_kmajor(x: torch.Tensor, Pq: torch.Tensor, Ps: torch.Tensor, Pz: torch.Tensor,
                     bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, act: str = "none",
                     residual: torch.Tensor | None = None):
    """y fp32 = act(x [M, K] . dequantize(K-major weights) (+ bias)) (+ residual).

    Ps fp32 is the base format; Ps float16 (binary16 scales) the fp16-scale
    variant (w4h_matmul_kmajor, no epilogue).  act: "none" (y [M, N]), "gelu"
    (y [M, N]) or "swiglu" (gate/up columns interleaved, y [M, N/2]); an
    epilogue or a residual goes through w4_matmul_kmajor_ep."""
    _dev(x, torch.float32, "x")
    _dev(Pq, torch.uint8, "Pq")
    f16 = Ps.dtype == torch.float16  # binary16 scales: the fp16-scale variant
    _dev(Ps, torch.float16 if f16 else torch.float32, "Ps")
    _dev(Pz, torch.uint8, "Pz")
    if bias is not None:
        _dev(bias, torch.float32, "bias")
    if act not in ACTS:
        raise ValueError(f"unknown activation {act!r}")
    ep = act != "none" or residual is not None
    if ep and f16:
        raise ValueError("the fused epilogue takes fp32 scales")
    M, K = x.shape
    N = Pq.shape[0]
    if Pq.shape != (N, K // 2) or Ps.shape != (N, K // BLOCK):
        raise ValueError("K-major weights do not match x")
    nout = N // 2 if act == "swiglu" else N
    if residual is not None:
        _dev(residual, torch.float32, "residual")
        if residual.shape != (M, nout):
            raise ValueError("residual must be [M, N_out]")
    if out is None:
        out = torch.empty((M, nout), dtype=torch.float32, device=x.device)
    else:
        _dev(out, torch.float32, "out")
    need = _lib.w4_matmul_kmajor_workspace_bytes(M, K, N)
    if workspace is None:
        ws, wsb = _workspace.get(x.device, need) if need else (None, 0)
    else:
        _dev(workspace, torch.uint8, "workspace")
        ws, wsb = workspace, workspace.numel()
    if ep:
        _check("w4_matmul_kmajor_ep", _lib.w4_matmul_kmajor_ep(
            _ptr(x), M, K, _ptr(Pq), _ptr(Ps), _ptr(Pz), N, _ptr(bias), _ptr(residual),
            ACTS[act], _ptr(out), _ptr(ws), wsb, _stream(x.device)))
        return out
    fn = "w4h_matmul_kmajor" if f16 else "w4_matmul_kmajor"
    _check(fn, getattr(_lib, fn)(
        _ptr(x), M, K, _ptr(Pq), _ptr(Ps), _ptr(Pz), N, _ptr(bias), _ptr(out),
        _ptr(ws), wsb, _stream(x.device)))
    return out


def i8_quantize_head(E: torch.Tensor, ldq: int | None = None,
                     d_status: torch.Tensor | None = None):
    """E fp32 [K, N] -> (Q int8 [K, ldq], hs fp32 [N])."""
    _dev(E, torch.float32, "E")
    K, N = E.shape
    ldq = N if ldq is None else ldq
    Q = torch.empty((K, ldq), dtype=torch.int8, device=E.device)
    hs = torch.empty(N, dtype=torch.float32, device=E.device)
    if d_status is not None:
        _dev(d_status, torch.int32, "d_status")
    _check("i8_quantize_head", _lib.i8_quantize_head(_ptr(E), K, N, ldq, _ptr(Q), _ptr(hs),
                                                     _ptr(d_status), _stream(E.device)))
    return Q, hs


def i8_head_workspace_bytes(K: int, N: int) -> int:
    return _lib.i8_head_workspace_bytes(K, N)


def i8_head_logits(x_last: torch.Tensor, Q: torch.Tensor, hs: torch.Tensor,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """x_last fp32 [K] (the last row) -> logits fp32 [N]."""
    _dev(x_last, torch.float32, "x_last")
    _dev(Q, torch.int8, "Q")
    _dev(hs, torch.float32, "hs")
    K, ldq = Q.shape
    N = hs.numel()
    if x_last.numel() != K:
        raise ValueError("x_last must have K elements")
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=Q.device)
    need = _lib.i8_head_workspace_bytes(K, N)
    if workspace is None:
        ws, wsb = _workspace.get(Q.device, need)
    else:
        _dev(workspace, torch.uint8, "workspace")
        ws, wsb = workspace, workspace.numel()
    _check("i8_head_logits", _lib.i8_head_logits(_ptr(x_last), K, _ptr(Q), ldq, _ptr(hs), N,
                                                 _ptr(out), _ptr(ws), wsb, _stream(Q.device)))
    return out


def i8_embed(tokens: torch.Tensor, Q: torch.Tensor, hs: torch.Tensor,
             d_status: torch.Tensor | None = None):
    """tokens int64 [T] -> fp32 [T, K] (columns of the dequantized table)."""
    _dev(tokens, torch.int64, "tokens")
    _dev(Q, torch.int8, "Q")
    _dev(hs, torch.float32, "hs")
    K, ldq = Q.shape
    N = hs.numel()
    T = tokens.numel()
    out = torch.empty((T, K), dtype=torch.float32, device=Q.device)
    if d_status is not None:
        _dev(d_status, torch.int32, "d_status")
    _check("i8_embed", _lib.i8_embed(_ptr(tokens), T, _ptr(Q), ldq, _ptr(hs), K, N, _ptr(out),
                                     _ptr(d_status), _stream(Q.device)))
    return out


def i8_prepack_head(Q: torch.Tensor, N: int, ldt: int | None = None) -> torch.Tensor:
    """Q int8 [K, ldq] (N used columns) -> token-major copy Qt int8 [N, ldt]."""
    _dev(Q, torch.int8, "Q")
    K, ldq = Q.shape
    if ldt is None:
        ldt = (K + 15) // 16 * 16
    Qt = torch.empty((N, ldt), dtype=torch.int8, device=Q.device)
    _check("i8_prepack_head", _lib.i8_prepack_head(_ptr(Q), K, N, ldq, _ptr(Qt), ldt,
                                                   _stream(Q.device)))
    return Qt


def i8_head_logits_kmajor(x_last: torch.Tensor, Qt: torch.Tensor, hs: torch.Tensor, K: int,
                          out: torch.Tensor | None = None):
    """x_last fp32 [K] -> logits fp32 [N] from the token-major table Qt [N, ldt]."""
    _dev(x_last, torch.float32, "x_last")
    _dev(Qt, torch.int8, "Qt")
    _dev(hs, torch.float32, "hs")
    N, ldt = Qt.shape
    if x_last.numel() != K or hs.numel() != N:
        raise ValueError("x_last must have K elements and hs N")
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=Qt.device)
    _check("i8_head_logits_kmajor",
           _lib.i8_head_logits_kmajor(_ptr(x_last), K, _ptr(Qt), ldt, _ptr(hs), N, _ptr(out),
                                      _stream(Qt.device)))
    return out


def i8_embed_kmajor(tokens: torch.Tensor, Qt: torch.Tensor, hs: torch.Tensor, K: int,
                    d_status: torch.Tensor | None = None):
    """tokens int64 [T] -> fp32 [T, K] (rows of the dequantized token-major table)."""
    _dev(tokens, torch.int64, "tokens")
    _dev(Qt, torch.int8, "Qt")
    _dev(hs, torch.float32, "hs")
    N, ldt = Qt.shape
    T = tokens.numel()
    out = torch.empty((T, K), dtype=torch.float32, device=Qt.device)
    if d_status is not None:
        _dev(d_status, torch.int32, "d_status")
    _check("i8_embed_kmajor", _lib.i8_embed_kmajor(_ptr(tokens), T, _ptr(Qt), ldt, _ptr(hs), K, N,
                                                   _ptr(out), _ptr(d_status), _stream(Qt.device)))
    return out


def i8_head_logits_rows(x: torch.Tensor, Qt: torch.Tensor, hs: torch.Tensor,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """x fp32 [M, K] -> logits fp32 [M, N] for every row (token-major table Qt [N, ldt]).

    `workspace`: optional uint8 tensor (the head needs none:
    i8_head_rows_workspace_bytes returns 0)."""
    _dev(x, torch.float32, "x")
    _dev(Qt, torch.int8, "Qt")
    _dev(hs, torch.float32, "hs")
    M, K = x.shape
    N, ldt = Qt.shape
    if hs.numel() != N:
        raise ValueError("hs must have N elements")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=Qt.device)
    need = _lib.i8_head_rows_workspace_bytes(M, K)
    if workspace is None:
        ws, wsb = _workspace.get(Qt.device, need)
    else:
        _dev(workspace, torch.uint8, "workspace")
        ws, wsb = workspace, workspace.numel()
    _check("i8_head_logits_rows", _lib.i8_head_logits_rows(
        _ptr(x), M, K, _ptr(Qt), ldt, _ptr(hs), N, _ptr(out), _ptr(ws), wsb,
        _stream(Qt.device)))
    return out


# -- fp16-scale variant: scales are float16 tensors (IEEE binary16) -------------
def w4h_quantize_pack(W: torch.Tensor, d_status: torch.Tensor | None = None):
    """W fp32 [K, N] -> (Wq uint8 [K, N/2], scales float16 [K/32, N], zeros uint8 [K/32, N/2])."""
    _dev(W, torch.float32, "W")
    K, N = W.shape
    Wq = torch.empty((K, N // 2), dtype=torch.uint8, device=W.device)
    s = torch.empty((K // BLOCK, N), dtype=torch.float16, device=W.device)
    z = torch.empty((K // BLOCK, N // 2), dtype=torch.uint8, device=W.device)
    if d_status is not None:
        _dev(d_status, torch.int32, "d_status")
    _check("w4h_quantize_pack", _lib.w4h_quantize_pack(
        _ptr(W), K, N, _ptr(Wq), _ptr(s), _ptr(z), _ptr(d_status), _stream(W.device)))
    return Wq, s, z


def w4h_dequantize(Wq: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor):
    """-> W_hat fp32 [K, N] (scales float16)."""
    _dev(Wq, torch.uint8, "Wq")
    _dev(scales, torch.float16, "scales")
    _dev(zeros, torch.uint8, "zeros")
    K, N = Wq.shape[0], scales.shape[1]
    out = torch.empty((K, N), dtype=torch.float32, device=Wq.device)
    _check("w4h_dequantize", _lib.w4h_dequantize(_ptr(Wq), _ptr(scales), _ptr(zeros), K, N,
                                                 _ptr(out), _stream(Wq.device)))
    return out


def w4h_prepack_kmajor(Wq: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor):
    """-> K-major copy (Pq uint8 [N, K/2], Ps float16 [N, K/32], Pz uint8 [N, K/64])."""
    _dev(Wq, torch.uint8, "Wq")
    _dev(scales, torch.float16, "scales")
    _dev(zeros, torch.uint8, "zeros")
    K, N = Wq.shape[0], scales.shape[1]
    Pq = torch.empty((N, K // 2), dtype=torch.uint8, device=Wq.device)
    Ps = torch.empty((N, K // BLOCK), dtype=torch.float16, device=Wq.device)
    Pz = torch.empty((N, K // 64), dtype=torch.uint8, device=Wq.device)
    _check("w4h_prepack_kmajor", _lib.w4h_prepack_kmajor(
        _ptr(Wq), _ptr(scales), _ptr(zeros), K, N, _ptr(Pq), _ptr(Ps), _ptr(Pz),
        _stream(Wq.device)))
    return Pq, Ps, Pz


# -- group-64 affine variant: fp32 scales and minima per 64 rows ----------------
GROUP = 64


def w4g_quantize_pack(W: torch.Tensor, d_status: torch.Tensor | None = None):
    """W fp32 [K, N] -> (Wq uint8 [K, N/2], scales fp32 [K/64, N], mins fp32 [K/64, N])."""
    _dev(W, torch.float32, "W")
    K, N = W.shape
    Wq = torch.empty((K, N // 2), dtype=torch.uint8, device=W.device)
    s = torch.empty((K // GROUP, N), dtype=torch.float32, device=W.device)
    m = torch.empty((K // GROUP, N), dtype=torch.float32, device=W.device)
    if d_status is not None:
        _dev(d_status, torch.int32, "d_status")
    _check("w4g_quantize_pack", _lib.w4g_quantize_pack(_ptr(W), K, N, _ptr(Wq), _ptr(s), _ptr(m),
                                                       _ptr(d_status), _stream(W.device)))
    return Wq, s, m


def w4g_dequantize(Wq: torch.Tensor, scales: torch.Tensor, mins: torch.Tensor):
    """-> W_hat fp32 [K, N] = q * s + m (one rounding)."""
    _dev(Wq, torch.uint8, "Wq")
    _dev(scales, torch.float32, "scales")
    _dev(mins, torch.float32, "mins")
    K, N = Wq.shape[0], scales.shape[1]
    out = torch.empty((K, N), dtype=torch.float32, device=Wq.device)
    _check("w4g_dequantize", _lib.w4g_dequantize(_ptr(Wq), _ptr(scales), _ptr(mins), K, N,
                                                 _ptr(out), _stream(Wq.device)))
    return out


def w4g_prepack_kmajor(Wq: torch.Tensor, scales: torch.Tensor, mins: torch.Tensor):
    """-> (Pq uint8 [N, K/2], Ps fp32 [N, K/64], Pm fp32 [N, K/64])."""
    _dev(Wq, torch.uint8, "Wq")
    _dev(scales, torch.float32, "scales")
    _dev(mins, torch.float32, "mins")
    K, N = Wq.shape[0], scales.shape[1]
    Pq = torch.empty((N, K // 2), dtype=torch.uint8, device=Wq.device)
    Ps = torch.empty((N, K // GROUP), dtype=torch.float32, device=Wq.device)
    Pm = torch.empty((N, K // GROUP), dtype=torch.float32, device=Wq.device)
    _check("w4g_prepack_kmajor", _lib.w4g_prepack_kmajor(
        _ptr(Wq), _ptr(scales), _ptr(mins), K, N, _ptr(Pq), _ptr(Ps), _ptr(Pm),
        _stream(Wq.device)))
    return Pq, Ps, Pm


def w4g_matmul_kmajor(x: torch.Tensor, Pq: torch.Tensor, Ps: torch.Tensor, Pm: torch.Tensor,
                      bias: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """y fp32 [M, N] = x [M, K] . W_hat (+ bias) on the group-64 affine K-major copy."""
    _dev(x, torch.float32, "x")
    _dev(Pq, torch.uint8, "Pq")
    _dev(Ps, torch.float32, "Ps")
    _dev(Pm, torch.float32, "Pm")
    if bias is not None:
        _dev(bias, torch.float32, "bias")
    M, K = x.shape
    N = Pq.shape[0]
    if Pq.shape != (N, K // 2) or Ps.shape != (N, K // GROUP) or Pm.shape != Ps.shape:
        raise ValueError("K-major weights do not match x")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    else:
        _dev(out, torch.float32, "out")
    _check("w4g_matmul_kmajor", _lib.w4g_matmul_kmajor(
        _ptr(x), M, K, _ptr(Pq), _ptr(Ps), _ptr(Pm), N, _ptr(bias), _ptr(out),
        _stream(x.device)))
    return out
