"""The C-ABI library loads and exports every symbol include/mgemm.h declares,
and its host-side checks reject bad arguments before touching a device (CPU).

No call here reaches the device: every call either fails validation or is a
no-op (M == 0), which the ABI returns from before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mgemm.h")

from moe_grouped_gemm_bf16_amd import _lib  # noqa: E402

L = _lib.LIB
OK, NUL, SHAPE, ALIGN, DEV, LAUNCH, OFFS = range(7)
A = 0x10000          # a 16-byte-aligned fake address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "defined"})


def test_header_declares_expected_api():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert L.mg_abi_version() == 1


def test_status_strings():
    for s in range(7):
        assert _lib.status_str(s).startswith("MG_")
    assert "unknown" in _lib.status_str(99)


def _host_check(off, E, M):
    arr = np.ascontiguousarray(off, dtype=np.int32)
    return L.mg_check_offsets_host(arr.ctypes.data, E, M)


def test_host_offsets_check():
    assert _host_check([0, 200, 200, 384, 512], 4, 512) == OK
    assert _host_check([0, 200, 200, 384, 500], 4, 512) == OK      # trailing rows
    assert _host_check([1, 200, 200, 384, 512], 4, 512) == OFFS    # no leading zero
    assert _host_check([0, 200, 100, 384, 512], 4, 512) == OFFS    # decreasing
    assert _host_check([0, 200, 200, 384, 513], 4, 512) == OFFS    # past M
    assert _host_check([0, 0], 1, 0) == OK
    assert L.mg_check_offsets_host(None, 4, 512) == NUL
    assert _host_check([0], 0, 0) == SHAPE
    assert _host_check([0] * 1026, 1025, 0) == SHAPE


@pytest.mark.parametrize("fn", ["mgemm_fwd", "mgemm_dgrad"])
def test_mgrouped_argument_errors(fn):
    f = getattr(L, fn)
    # (x, w, offsets, out, M, N, K, E, max_m_per_e, stream)
    assert f(A, A, A, A, 512, 128, 256, 0, 0, None) == SHAPE            # E < 1
    assert f(A, A, A, A, 512, 128, 256, 1025, 0, None) == SHAPE         # E too large
    assert f(A, A, A, A, -1, 128, 256, 4, 0, None) == SHAPE             # M < 0
    assert f(A, A, A, A, 512, 100, 256, 4, 0, None) == SHAPE            # N % 8
    assert f(A, A, A, A, 512, 128, 252, 4, 0, None) == SHAPE            # K % 8
    assert f(A, A, A, A, 512, 128, 1 << 23, 4, 0, None) == SHAPE        # K too large
    assert f(A, A, A, A, 512, 128, 256, 4, -1, None) == SHAPE           # bad hint
    assert f(None, A, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, None, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, None, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, None, 512, 128, 256, 4, 0, None) == NUL
    assert f(A + 8, A, A, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A, A + 2, A, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A, A, A + 2, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A, A, A, A + 4, 512, 128, 256, 4, 0, None) == ALIGN
    # no rows: a valid no-op that never touches the (NULL) buffers or device
    assert f(None, None, None, None, 0, 128, 256, 4, 0, None) == OK


@pytest.mark.parametrize("fn", ["kgemm_wgrad", "kgemm_wgrad_noalloc"])
def test_wgrad_argument_errors(fn):
    f = getattr(L, fn)
    # (dy, x, offsets, dw, M, N, K, E, accumulate, stream)
    assert f(A, A, A, A, 512, 128, 256, 0, 0, None) == SHAPE
    assert f(A, A, A, A, 512, 120, 252, 4, 0, None) == SHAPE
    assert f(A, A, None, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, None, 512, 128, 256, 4, 0, None) == NUL
    assert f(None, A, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, A + 8, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A + 8, A, A, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(None, None, None, None, 0, 0, 256, 4, 0, None) == OK       # empty dw


def test_mx_argument_errors():
    f = L.mgemm_fwd_mx
    # (x, x_scale, w, w_scale, offsets, y, M, N, K, E, max_m_per_e, stream)
    assert f(A, A, A, A, A, A, 512, 128, 256, 0, 0, None) == SHAPE        # E < 1
    assert f(A, A, A, A, A, A, 512, 128, 48, 4, 0, None) == SHAPE         # K % 32
    assert f(A, A, A, A, A, A, 512, 100, 256, 4, 0, None) == SHAPE        # N % 8
    assert f(A, A, A, A, A, A, 512, 128, 256, 4, -1, None) == SHAPE       # bad hint
    assert f(A, A, A, A, A, A, 1 << 30, 128, 4096, 4, 0, None) == SHAPE   # scale offsets > 2^31
    assert f(None, A, A, A, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, None, A, A, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, None, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, A, None, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A + 8, A, A, A, A, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A, A + 2, A, A, A, A, 512, 128, 256, 4, 0, None) == ALIGN     # scales 4-byte aligned
    assert f(A, A + 4, A, A, A, A + 8, 512, 128, 256, 4, 0, None) == ALIGN  # y 16-byte aligned
    assert f(None, None, None, None, None, None, 0, 128, 256, 4, 0, None) == OK
    g = L.mg_mx_scales_blocked
    # (scales, blocked, rows, K, batch, stream)
    assert g(A, A, 10, 48, 1, None) == SHAPE                             # K % 32
    assert g(A, A, -1, 64, 1, None) == SHAPE
    assert g(A, A, 10, 64, -1, None) == SHAPE
    assert g(None, A, 10, 64, 1, None) == NUL
    assert g(A, A + 2, 10, 64, 1, None) == ALIGN
    assert g(None, None, 0, 64, 1, None) == OK                           # nothing to convert


def test_wgrad_mx_argument_errors():
    f = L.kgemm_wgrad_mx
    # (dyt, dyt_scale, xt, xt_scale, offsets, dw, M, N, K, E, accumulate, stream)
    assert f(A, A, A, A, A, A, 512, 128, 256, 0, 0, None) == SHAPE        # E < 1
    assert f(A, A, A, A, A, A, 500, 128, 256, 4, 0, None) == SHAPE        # M % 128
    assert f(A, A, A, A, A, A, 512, 100, 256, 4, 0, None) == SHAPE        # N % 8
    assert f(A, A, A, A, A, A, 1 << 24, 128, 256, 4, 0, None) == SHAPE    # 256 M >= 2^32
    assert f(None, A, A, A, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, None, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, A, None, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, A, A, None, 512, 128, 256, 4, 0, None) == NUL
    assert f(A + 8, A, A, A, A, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A, A + 2, A, A, A, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A, A, A, A, A, A + 8, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(None, None, None, None, None, None, 512, 0, 256, 4, 0, None) == OK   # empty dw


def test_wgrad_mx_tm_argument_errors():
    f = L.kgemm_wgrad_mx_tm
    # (dy8, dy_scale, x8, x_scale, offsets, dw, M, N, K, E, accumulate, stream)
    assert f(A, A, A, A, A, A, 512, 128, 256, 0, 0, None) == SHAPE        # E < 1
    assert f(A, A, A, A, A, A, 500, 128, 256, 4, 0, None) == SHAPE        # M % 128
    assert f(A, A, A, A, A, A, 512, 136, 256, 4, 0, None) == SHAPE        # N % 16
    assert f(A, A, A, A, A, A, 512, 128, 264, 4, 0, None) == SHAPE        # K % 16
    assert f(A, A, A, A, A, A, 1 << 31, 128, 256, 4, 0, None) == SHAPE    # M too large
    assert f(None, A, A, A, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, None, A, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, A, None, A, 512, 128, 256, 4, 0, None) == NUL
    assert f(A, A, A, A, A, None, 512, 128, 256, 4, 0, None) == NUL
    assert f(A + 8, A, A, A, A, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A, A, A + 8, A, A, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A, A + 2, A, A, A, A, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(A, A, A, A, A, A + 8, 512, 128, 256, 4, 0, None) == ALIGN
    assert f(None, None, None, None, None, None, 512, 0, 256, 4, 0, None) == OK   # empty dw


def test_swiglu_backward_and_saving_forward_argument_errors():
    f = L.mgemm_dgrad_swiglu
    # (dy, w2, gu, offsets, dgu, M, N, I, E, max_m_per_e, stream)
    assert f(A, A, A, A, A, 512, 256, 128, 0, 0, None) == SHAPE          # E < 1
    assert f(A, A, A, A, A, 512, 250, 128, 4, 0, None) == SHAPE          # N % 8
    assert f(A, A, A, A, A, 512, 256, 100, 4, 0, None) == SHAPE          # I % 8
    assert f(A, A, A, A, A, 512, 256, 128, 4, -1, None) == SHAPE         # bad hint
    assert f(A, A, None, A, A, 512, 256, 128, 4, 0, None) == NUL          # gu
    assert f(A, A, A, A, None, 512, 256, 128, 4, 0, None) == NUL          # dgu
    assert f(A, A, A + 8, A, A, 512, 256, 128, 4, 0, None) == ALIGN
    assert f(A, A, A, A, A + 8, 512, 256, 128, 4, 0, None) == ALIGN
    assert f(None, None, None, None, None, 0, 256, 128, 4, 0, None) == OK
    g = L.mgemm_fwd_swiglu_gu
    # (x, gather, w13, offsets, h, gu, M, T, I, K, E, max_m_per_e, stream)
    assert g(A, None, A, A, A, A, 512, 0, 100, 256, 4, 0, None) == SHAPE   # I % 8
    assert g(A, None, A, A, A, A + 8, 512, 0, 128, 256, 4, 0, None) == ALIGN
    assert g(A, None, A, A, A, None, 0, 0, 128, 256, 4, 0, None) == OK


def test_moe_combine_argument_errors():
    f = L.mg_moe_combine
    # (rows, token_rows, weights, out, M, T, k, D, stream)
    assert f(A, A, None, A, 100, 10, 0, 64, None) == SHAPE          # k < 1
    assert f(A, A, None, A, 100, 10, 65, 64, None) == SHAPE         # k > 64
    assert f(A, A, None, A, 100, 10, 4, 60, None) == SHAPE          # D % 8
    assert f(A, A, None, A, -1, 10, 4, 64, None) == SHAPE
    assert f(A, None, None, A, 100, 10, 4, 64, None) == NUL
    assert f(A, A, None, None, 100, 10, 4, 64, None) == NUL
    assert f(A + 8, A, None, A, 100, 10, 4, 64, None) == ALIGN
    assert f(A, A + 2, None, A, 100, 10, 4, 64, None) == ALIGN
    assert f(A, A, A + 2, A, 100, 10, 4, 64, None) == ALIGN
    assert f(None, None, None, None, 100, 0, 4, 64, None) == OK      # no tokens


def test_python_binding_rejects_bad_tensors_on_host():
    torch = pytest.importorskip("torch")
    import moe_grouped_gemm_bf16_amd as mg
    x = torch.zeros(8, 16, dtype=torch.bfloat16)
    w = torch.zeros(2, 8, 16, dtype=torch.bfloat16)
    off = torch.tensor([0, 4, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        mg.fwd(x, w, off)
    with pytest.raises(TypeError):
        mg.fwd(x.float(), w, off)
    with pytest.raises(ValueError):
        mg.fwd(x, w[:, :, :8].contiguous(), off)
    with pytest.raises(ValueError):
        mg.Kgemm(x, x, off, descriptor="gw9")


def test_host_list_check():
    """mg_check_list_host enforces the mg_gemm_desc rules (no device use)."""
    import ctypes
    from moe_grouped_gemm_bf16_amd._lib import GemmDesc
    P = 0x10000                                   # any 16-byte aligned address
    def chk(*descs):
        arr = (GemmDesc * len(descs))(*descs)
        return _lib.LIB.mg_check_list_host(arr, len(descs))
    ok = GemmDesc(P, P, P, 5, 16, 24, 24, 32, 16)
    assert chk(ok) == _lib.MG_OK
    assert chk(ok, GemmDesc(0, 0, 0, 0, 8, 8, 8, 8, 8)) == _lib.MG_OK       # empty group
    assert chk(GemmDesc(0, 0, P, 3, 8, 0, 0, 0, 8)) == _lib.MG_OK          # k == 0
    assert chk(GemmDesc(P, P, P, -1, 8, 8, 8, 8, 8)) == _lib.MG_ERR_SHAPE
    assert chk(GemmDesc(P, P, P, 2, 12, 8, 8, 8, 16)) == _lib.MG_ERR_SHAPE  # n % 8
    assert chk(GemmDesc(P, P, P, 2, 8, 16, 8, 16, 8)) == _lib.MG_ERR_SHAPE  # lda < k
    assert chk(GemmDesc(P, P, P, 2, 16, 8, 8, 8, 8)) == _lib.MG_ERR_SHAPE   # ldd < n
    assert chk(GemmDesc(P, 0, P, 2, 8, 8, 8, 8, 8)) == _lib.MG_ERR_NULL
    assert chk(GemmDesc(P + 8, P, P, 2, 8, 8, 8, 8, 8)) == _lib.MG_ERR_ALIGN
    assert _lib.LIB.mg_check_list_host(None, 1) == _lib.MG_ERR_NULL
    arr = (GemmDesc * 1)(ok)
    assert _lib.LIB.mg_check_list_host(arr, 0) == _lib.MG_ERR_SHAPE
    assert _lib.LIB.mgemm_list(None, 1, None) == _lib.MG_ERR_NULL
    assert _lib.LIB.mgemm_list(ctypes.addressof(arr), 2000, None) == _lib.MG_ERR_SHAPE


def test_probe_library_exports_its_header_and_rejects_bad_arguments():
    """libmgemm_probe.so (the matrix-core ceiling probe bench.py --ceiling
    runs) exports what include/mgemm_probe.h declares; bad arguments return
    1 before any device call."""
    probe_h = os.path.join(ROOT, "include", "mgemm_probe.h")
    text = re.sub(r"/\*.*?\*/", "", open(probe_h).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "defined"})
    assert names == ["mg_probe_mfma_bf16", "mg_probe_mfma_bf16_flops"]
    lib = ctypes.CDLL(os.path.join(ROOT, "moe_grouped_gemm_bf16_amd", "libmgemm_probe.so"))
    for n in names:
        assert hasattr(lib, n), n
    lib.mg_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.mg_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.mg_probe_mfma_bf16_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    assert lib.mg_probe_mfma_bf16(0, 1, A, None) == 1
    assert lib.mg_probe_mfma_bf16(1, 0, A, None) == 1
    assert lib.mg_probe_mfma_bf16(1, 1, None, None) == 1
    assert lib.mg_probe_mfma_bf16_flops(256, 16384) == 256 * 16384 * 64 * 32768.0
