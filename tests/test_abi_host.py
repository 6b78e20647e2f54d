"""The C-ABI library on a machine without a GPU: exports, host-side checks, plans.

No compute call is made here.  Every entry point validates its arguments on
the host before touching HIP, so each error code below is produced without a
device; a well-formed call reaches the device check and reports
W4_ERR_DEVICE when no gfx950 is present.
"""
import ctypes
import os
import re

import pytest
import torch

import w4_block_dequant_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")

NO_GPU = not torch.cuda.is_available()
A = 1 << 12  # a fake, 4 KiB-aligned "device address": never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for must in ("w4_quantize_pack", "w4_matmul", "i8_head_logits", "w4_unpack", "w4_dequantize",
                 "w4_prepack_kmajor", "w4_matmul_kmajor", "w4_check_matmul_kmajor_args",
                 "i8_quantize_head", "i8_embed", "w4_matmul_workspace_bytes",
                 "i8_head_workspace_bytes", "w4_check_matmul_args", "w4_strerror",
                 "w4_abi_version", "i8_prepack_head", "i8_head_logits_kmajor",
                 "i8_check_head_logits_kmajor_args", "i8_embed_kmajor",
                 "i8_head_logits_rows", "i8_check_head_logits_rows_args",
                 "i8_head_rows_workspace_bytes", "w4_matmul_kmajor_ep",
                 "w4g_quantize_pack", "w4g_dequantize", "w4g_prepack_kmajor",
                 "w4g_check_matmul_kmajor_args", "w4g_matmul_kmajor",
                 "w4_check_matmul_kmajor_ep_args",
                 "w4h_quantize_pack", "w4h_dequantize", "w4h_prepack_kmajor",
                 "w4h_matmul_kmajor", "w4h_check_matmul_kmajor_args", "w4_matmul_noalloc",
                 "w4_read_bytes", "w4_read_bytes_words"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(w4.LIB_PATH)
    missing = [n for n in header_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_strings():
    assert w4.w4_abi_version() == 1
    for code in range(8):
        assert w4.w4_strerror(code)
    assert w4.w4_strerror(99) == "unknown status"


def check(M, K, N, x=A, Wq=A, s=A, z=A, bias=None, y=A, ws=A, wsb=None):
    if wsb is None:
        wsb = w4.w4_matmul_workspace_bytes(M, K, N)
    return w4.library().w4_check_matmul_args(x, M, K, Wq, s, z, N, bias, y, ws, wsb)


def test_matmul_shape_checks():
    assert check(1, 768, 768) == w4.W4_OK
    assert check(-1, 768, 768) == w4.W4_ERR_BAD_SHAPE
    assert check(1, 100, 768) == w4.W4_ERR_BAD_SHAPE       # K % 32 != 0
    assert check(1, 768, 767) == w4.W4_ERR_BAD_SHAPE       # N odd
    assert check(1, -32, 768) == w4.W4_ERR_BAD_SHAPE
    assert check(1, 1 << 30, 1 << 30) == w4.W4_ERR_BAD_SHAPE  # beyond the index range
    # empty problems need no pointers at all
    assert check(0, 768, 768, x=None, Wq=None, s=None, z=None, y=None) == w4.W4_OK
    assert check(4, 768, 0, x=None, Wq=None, s=None, z=None, y=None) == w4.W4_OK
    assert check(1, 0, 768, x=None, Wq=None, s=None, z=None) == w4.W4_OK


def test_matmul_pointer_checks():
    assert check(1, 768, 768, x=None) == w4.W4_ERR_NULL_PTR
    assert check(1, 768, 768, Wq=None) == w4.W4_ERR_NULL_PTR
    assert check(1, 768, 768, y=None) == w4.W4_ERR_NULL_PTR
    assert check(1, 768, 768, Wq=A + 8) == w4.W4_ERR_MISALIGNED
    assert check(1, 768, 768, s=A + 4) == w4.W4_ERR_MISALIGNED
    assert check(1, 768, 768, x=A + 4) == w4.W4_ERR_MISALIGNED
    assert check(1, 768, 768, y=A + 2) == w4.W4_ERR_MISALIGNED
    assert check(1, 768, 768, bias=A + 1) == w4.W4_ERR_MISALIGNED
    assert check(1, 768, 768, bias=A + 4) == w4.W4_OK


def test_workspace_rules():
    K, N = 3072, 9216
    need = w4.w4_matmul_workspace_bytes(1, K, N)
    assert need > 0                      # this shape splits K across workgroups
    assert check(1, K, N, ws=None, wsb=0) == w4.W4_ERR_WORKSPACE
    assert check(1, K, N, ws=A, wsb=need - 1) == w4.W4_ERR_WORKSPACE
    assert check(1, K, N, ws=A, wsb=need) == w4.W4_OK
    assert check(1, K, N, ws=A + 16, wsb=need) == w4.W4_ERR_MISALIGNED
    assert w4.w4_matmul_workspace_bytes(1, 100, N) == 0   # invalid shape
    # split-K workspace: whole fp32 partial planes of the padded row
    tiles = (N + 255) // 256
    assert need % (256 * tiles * 4) == 0


def test_every_body_shape_is_planned():
    import synth
    for K, N in synth.GPT2_SHAPES + synth.DENSE38_SHAPES:
        assert check(1, K, N, ws=A, wsb=w4.w4_matmul_workspace_bytes(1, K, N)) == w4.W4_OK
    # the GPT-2 head (K = 768) runs the one-launch whole-K kernel: no
    # workspace; K off the whole-K sizes takes the split-K kernel and its planes
    assert w4.i8_head_workspace_bytes(768, 50257) == 0
    assert w4.i8_head_workspace_bytes(800, 50257) > 0


@pytest.mark.skipif(not NO_GPU, reason="needs a machine without a GPU")
def test_valid_calls_report_no_device():
    lib = w4.library()
    need = w4.w4_matmul_workspace_bytes(1, 768, 768)
    st = lib.w4_matmul(A, 1, 768, A, A, A, 768, None, A, A if need else None, need, None)
    assert st == w4.W4_ERR_DEVICE
    assert lib.w4_quantize_pack(A, 64, 64, A, A, A, None, None) == w4.W4_ERR_DEVICE


def test_entry_points_reject_before_any_hip_call():
    lib = w4.library()
    assert lib.w4_quantize_pack(A, 33, 64, A, A, A, None, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.w4_quantize_pack(None, 32, 64, A, A, A, None, None) == w4.W4_ERR_NULL_PTR
    assert lib.w4_quantize_pack(A + 4, 32, 64, A, A, A, None, None) == w4.W4_ERR_MISALIGNED
    assert lib.w4_unpack(A, A, 32, 63, A, A, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.w4_dequantize(A, A, None, 32, 64, A, None) == w4.W4_ERR_NULL_PTR
    assert lib.w4_matmul(A, 1, 768, A, A, A, 767, None, A, None, 0, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.i8_quantize_head(A, 768, 100, 99, A, A, None, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.i8_quantize_head(A, 768, 100, 100, A + 1, A, None, None) == w4.W4_ERR_MISALIGNED
    assert lib.i8_head_logits(A, 768, A, 50256, A, 50257, A, None, 0, None) == w4.W4_ERR_BAD_SHAPE
    need = w4.i8_head_workspace_bytes(800, 50257)   # K = 800: the split-K head
    assert lib.i8_head_logits(A, 800, A, 50257, A, 50257, A, None, 0, None) == w4.W4_ERR_WORKSPACE
    assert lib.i8_head_logits(A, 800, A, 50257, A, 50257, A, A, need - 4, None) == w4.W4_ERR_WORKSPACE
    assert lib.i8_embed(A, 4, A, 50257, A, 768, 50258, A, None, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.i8_embed(A + 4, 4, A, 50257, A, 768, 50257, A, None, None) == w4.W4_ERR_MISALIGNED
    km = lib.w4_check_matmul_kmajor_args
    assert km(A, 1, 96, A, A, A, 16, None, A, None, 0) == w4.W4_ERR_BAD_SHAPE
    assert km(A, 1, 128, A, A, A, 16, None, A, None, 0) == w4.W4_OK
    assert km(A, 1, 128, A + 8, A, A, 16, None, A, None, 0) == w4.W4_ERR_MISALIGNED
    assert km(None, 1, 128, A, A, A, 16, None, A, None, 0) == w4.W4_ERR_NULL_PTR
    # M >= 3 on the matrix-core path: split-K needs a workspace for narrow N
    assert w4.w4_matmul_kmajor_workspace_bytes(2, 3072, 3072) == 0      # M = 2: the GEMV
    assert w4.w4_matmul_kmajor_workspace_bytes(3, 3072, 3072) == 0      # M = 3: whole-K matrix cores
    assert w4.w4_matmul_kmajor_workspace_bytes(16, 3072, 3072) == 0     # up to 16 rows
    assert w4.w4_matmul_kmajor_workspace_bytes(3, 3072, 768) == 0       # 48 workgroups: still whole-K
    assert w4.w4_matmul_kmajor_workspace_bytes(3, 3072, 256) > 0        # too few columns: split-K
    assert w4.w4_matmul_kmajor_workspace_bytes(17, 3072, 3072) > 0      # 17 rows: split-K
    # past 16 rows, small matrices (at most 2^22 weights): whole-K row groups
    assert w4.w4_matmul_kmajor_workspace_bytes(58, 768, 2304) == 0
    assert w4.w4_matmul_kmajor_workspace_bytes(58, 768, 768) == 0
    assert w4.w4_matmul_kmajor_workspace_bytes(128, 3072, 768) == 0
    assert w4.w4_matmul_kmajor_workspace_bytes(129, 768, 768) > 0     # past 128 rows: split-K
    assert w4.w4_matmul_kmajor_workspace_bytes(58, 768, 16) > 0       # too few workgroups
    need = w4.w4_matmul_kmajor_workspace_bytes(16, 3072, 256)
    assert need > 0
    assert w4.w4_matmul_kmajor_workspace_bytes(1, 3072, 3072) == 0
    assert w4.w4_matmul_kmajor_workspace_bytes(16, 3008, 3072) == 0   # K % 128 != 0: GEMV path
    assert km(A, 16, 3072, A, A, A, 256, None, A, None, 0) == w4.W4_ERR_WORKSPACE
    assert km(A, 16, 3072, A, A, A, 256, None, A, A, need - 1) == w4.W4_ERR_WORKSPACE
    assert km(A, 16, 3072, A, A, A, 256, None, A, A + 64, need) == w4.W4_ERR_MISALIGNED
    assert km(A, 16, 3072, A, A, A, 256, None, A, A, need) == w4.W4_OK
    assert lib.w4_prepack_kmajor(A, A, A, 96, 16, A, A, A, None) == w4.W4_ERR_BAD_SHAPE
    # empty work succeeds without a device
    assert lib.w4_matmul(None, 0, 768, None, None, None, 768, None, None, None, 0, None) == w4.W4_OK
    assert lib.i8_embed(None, 0, None, 10, None, 768, 10, None, None, None) == w4.W4_OK


def test_read_bytes_host_checks():
    lib = w4.library()
    assert lib.w4_read_bytes_words(1 << 20, 8) == 4 * (1 << 20) // (256 * 16 * 8)
    assert lib.w4_read_bytes_words(1 << 20, 5) == 0
    assert lib.w4_read_bytes_words(100, 8) == 0
    assert lib.w4_read_bytes(A, 100, 8, A, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.w4_read_bytes(A, 4096, 7, A, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.w4_read_bytes(A + 8, 4096, 8, A, None) == w4.W4_ERR_MISALIGNED
    assert lib.w4_read_bytes(None, 4096, 8, A, None) == w4.W4_ERR_NULL_PTR
    assert lib.w4_read_bytes(None, 0, 8, None, None) == w4.W4_OK
    if NO_GPU:
        assert lib.w4_read_bytes(A, 4096, 8, A, None) == w4.W4_ERR_DEVICE


def test_noalloc_host_checks():
    lib = w4.library()
    f = lib.w4_matmul_noalloc
    # a shape whose split-K partials exceed the library's scratch: refused on the host
    assert w4.w4_matmul_workspace_bytes(64, 8192, 3072) > w4.NOALLOC_SCRATCH_BYTES
    assert f(A, 64, 8192, A, A, A, 3072, None, A, None) == w4.W4_ERR_WORKSPACE
    assert f(A, 1, 100, A, A, A, 64, None, A, None) == w4.W4_ERR_BAD_SHAPE
    assert f(A + 4, 1, 768, A, A, A, 768, None, A, None) == w4.W4_ERR_MISALIGNED
    assert f(None, 1, 768, A, A, A, 768, None, A, None) == w4.W4_ERR_NULL_PTR
    assert f(None, 0, 768, None, None, None, 768, None, None, None) == w4.W4_OK
    if NO_GPU:
        assert f(A, 58, 3072, A, A, A, 3072, None, A, None) == w4.W4_ERR_DEVICE


def check_headk(K, N, ldt=None, x=A, Qt=A, hs=A, out=A):
    if ldt is None:
        ldt = K
    return w4.library().i8_check_head_logits_kmajor_args(x, K, Qt, ldt, hs, N, out)


def test_head_kmajor_checks():
    assert check_headk(768, 50257) == w4.W4_OK
    assert check_headk(768, 50257, ldt=784) == w4.W4_OK
    assert check_headk(8192, 1000) == w4.W4_OK
    assert check_headk(808, 10) == w4.W4_ERR_BAD_SHAPE          # K % 16 != 0
    assert check_headk(800, 10, ldt=800) == w4.W4_OK            # K % 16 == 0 is enough
    assert check_headk(0, 10) == w4.W4_ERR_BAD_SHAPE
    assert check_headk(8256, 10) == w4.W4_ERR_BAD_SHAPE         # K > 8192
    assert check_headk(768, 10, ldt=776) == w4.W4_ERR_BAD_SHAPE  # ldt % 16 != 0
    assert check_headk(768, 10, ldt=704) == w4.W4_ERR_BAD_SHAPE  # ldt < K
    assert check_headk(768, 1 << 22) == w4.W4_ERR_BAD_SHAPE     # N * ldt >= 2^31
    assert check_headk(768, 0, x=None, Qt=None, hs=None, out=None) == w4.W4_OK
    assert check_headk(768, 10, Qt=None) == w4.W4_ERR_NULL_PTR
    assert check_headk(768, 10, x=A + 4) == w4.W4_ERR_MISALIGNED
    assert check_headk(768, 10, Qt=A + 8) == w4.W4_ERR_MISALIGNED
    assert check_headk(768, 10, out=A + 2) == w4.W4_ERR_MISALIGNED
    lib = w4.library()
    assert lib.i8_prepack_head(A, 768, 10, 10, A, 776, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.i8_prepack_head(A, 768, 10, 9, A, 768, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.i8_prepack_head(A + 4, 768, 10, 10, A, 768, None) == w4.W4_ERR_MISALIGNED
    assert lib.i8_embed_kmajor(A, 4, A, 776, A, 768, 10, A, None, None) == w4.W4_ERR_BAD_SHAPE
    if NO_GPU:
        assert lib.i8_head_logits_kmajor(A, 768, A, 768, A, 10, A, None) == w4.W4_ERR_DEVICE
        assert lib.i8_prepack_head(A, 768, 10, 16, A, 768, None) == w4.W4_ERR_DEVICE


def test_head_rows_checks():
    lib = w4.library()
    chk = lib.i8_check_head_logits_rows_args
    # the full-sequence head needs no workspace
    assert lib.i8_head_rows_workspace_bytes(58, 768) == 0
    assert lib.i8_head_rows_workspace_bytes(0, 768) == 0
    assert chk(A, 58, 768, A, 768, A, 50257, A, None, 0) == w4.W4_OK
    assert chk(A, 58, 768, A, 768, A, 50257, A, A, 12345) == w4.W4_OK  # a workspace is ignored
    assert chk(A, 58, 8192, A, 8192, A, 100, A, None, 0) == w4.W4_OK
    assert chk(A, 58, 8208, A, 8208, A, 100, A, None, 0) == w4.W4_ERR_BAD_SHAPE  # K > 8192
    assert chk(A, 58, 808, A, 816, A, 100, A, None, 0) == w4.W4_ERR_BAD_SHAPE    # K % 16 != 0
    assert chk(A, -1, 768, A, 768, A, 100, A, None, 0) == w4.W4_ERR_BAD_SHAPE
    assert chk(None, 0, 768, None, 768, None, 100, None, None, 0) == w4.W4_OK
    assert chk(A, 2, 768, None, 768, A, 100, A, None, 0) == w4.W4_ERR_NULL_PTR
    assert chk(A + 4, 2, 768, A, 768, A, 100, A, None, 0) == w4.W4_ERR_MISALIGNED  # x 16-byte
    assert chk(A, 2, 768, A + 8, 768, A, 100, A, None, 0) == w4.W4_ERR_MISALIGNED
    if NO_GPU:
        assert lib.i8_head_logits_rows(A, 2, 768, A, 768, A, 100, A, None, 0, None) == \
            w4.W4_ERR_DEVICE


def test_f16_variant_checks():
    lib = w4.library()
    km = lib.w4h_check_matmul_kmajor_args
    assert km(A, 1, 3072, A, A, A, 3072, None, A, None, 0) == w4.W4_OK
    assert km(A, 1, 96, A, A, A, 16, None, A, None, 0) == w4.W4_ERR_BAD_SHAPE
    assert km(A, 1, 128, A, A + 8, A, 16, None, A, None, 0) == w4.W4_ERR_MISALIGNED
    need = w4.w4_matmul_kmajor_workspace_bytes(16, 3072, 256)
    assert need > 0
    assert km(A, 16, 3072, A, A, A, 256, None, A, None, 0) == w4.W4_ERR_WORKSPACE
    assert km(A, 16, 3072, A, A, A, 256, None, A, A, need) == w4.W4_OK
    assert km(A, 16, 3072, A, A, A, 3072, None, A, None, 0) == w4.W4_OK   # whole-K: none
    assert lib.w4h_quantize_pack(A, 100, 64, A, A, A, None, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.w4h_quantize_pack(A, 64, 64, A, A + 2, A, None, None) == w4.W4_ERR_MISALIGNED
    assert lib.w4h_prepack_kmajor(A, A, A, 96, 16, A, A, A, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.w4h_dequantize(A, None, A, 32, 64, A, None) == w4.W4_ERR_NULL_PTR
    if NO_GPU:
        assert lib.w4h_quantize_pack(A, 64, 64, A, A, A, None, None) == w4.W4_ERR_DEVICE


def test_kmajor_epilogue_checks():
    chk = w4.library().w4_check_matmul_kmajor_ep_args
    M, K, N = 1, 768, 2304
    for act in (0, 1, 2):
        assert chk(A, M, K, A, A, A, N, A, A, act, A, None, 0) == w4.W4_OK
    assert chk(A, M, K, A, A, A, N, A, A, 3, A, None, 0) == w4.W4_ERR_BAD_SHAPE
    assert chk(A, M, K, A, A, A, N, A, A, -1, A, None, 0) == w4.W4_ERR_BAD_SHAPE
    assert chk(A, M, K, A, A, A, N, A, A + 2, 1, A, None, 0) == w4.W4_ERR_MISALIGNED
    assert chk(A, M, K, A, A, A, N, None, None, 2, A, None, 0) == w4.W4_OK
    ws = w4.w4_matmul_kmajor_workspace_bytes(16, 3072, 3072)
    assert chk(A, 16, 3072, A, A, A, 3072, None, A, 2, A, None, 0) == \
        (w4.W4_ERR_WORKSPACE if ws else w4.W4_OK)
    if NO_GPU:
        assert w4.library().w4_matmul_kmajor_ep(A, M, K, A, A, A, N, A, A, 1, A, None, 0,
                                                None) == w4.W4_ERR_DEVICE


def test_g64_checks():
    lib = w4.library()
    chk = lib.w4g_check_matmul_kmajor_args
    assert chk(A, 1, 3072, A, A, A, 9216, None, A) == w4.W4_OK
    assert chk(A, 1, 3072 + 32, A, A, A, 9216, None, A) == w4.W4_ERR_BAD_SHAPE   # K % 64
    assert chk(A, 1, 3072, A, A, A, 9215, None, A) == w4.W4_ERR_BAD_SHAPE       # N odd
    assert chk(A, 4 * 65536, 64, A, A, A, 8, None, A) == w4.W4_ERR_BAD_SHAPE    # grid rows
    assert chk(A, 1, 3072, A, A + 8, A, 9216, None, A) == w4.W4_ERR_MISALIGNED
    assert chk(A, 1, 3072, A, A, None, 9216, None, A) == w4.W4_ERR_NULL_PTR
    assert chk(None, 0, 3072, None, None, None, 9216, None, None) == w4.W4_OK
    if NO_GPU:
        assert lib.w4g_quantize_pack(A, 64, 8, A, A, A, None, None) == w4.W4_ERR_DEVICE
        assert lib.w4g_matmul_kmajor(A, 1, 64, A, A, A, 8, None, A, None) == w4.W4_ERR_DEVICE
    assert lib.w4g_quantize_pack(A, 96, 8, A, A, A, None, None) == w4.W4_ERR_BAD_SHAPE
    assert lib.w4g_dequantize(A, A, A, 64, 8, A + 4, None) == w4.W4_ERR_MISALIGNED


def test_kmajor_index_limit():
    """The K-major path indexes in 32 bits: K * N, M * K and M * N below 2^31
    are accepted and 2^31 is refused, before any HIP call."""
    km = w4.library().w4_check_matmul_kmajor_args
    K = 8192
    assert km(A, 1, K, A, A, A, 262128, None, A, None, 0) == w4.W4_OK      # K N = 2^31 - 131072
    assert km(A, 4, K, A, A, A, 262128, None, A, None, 0) == w4.W4_OK      # whole-K: no workspace
    assert km(A, 1, K, A, A, A, 262144, None, A, None, 0) == w4.W4_ERR_BAD_SHAPE  # K N = 2^31
    assert km(A, 262144, K, A, A, A, 16, None, A, None, 0) == w4.W4_ERR_BAD_SHAPE  # M K = 2^31
