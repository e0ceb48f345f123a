"""MoE grouped GEMM for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of libmgemm.so (include/mgemm.h): argument
checks and marshalling only.  Every step of the computation runs in the HIP
kernels; PyTorch provides device memory and the current stream.

  fwd(x, w, offsets)      Y[i] = x[i] W[e]^T          M-grouped forward
  dgrad(dy, w, offsets)   dX[i] = dy[i] W[e]          M-grouped input gradient
  wgrad(dy, x, offsets)   dW[e] = sum_i dy[i]^T x[i]  K-grouped fp32 weight gradient
  fwd_swiglu(x, w13, offsets, gather)                  gate-up forward, SwiGLU fused,
      h[i] = silu(x[r] w1[e]^T) * (x[r] w3[e]^T), r = gather[i]   rows gathered by index
  grouped_list([(A_g, B_g), ...])   D_g = A_g B_g^T    independent GEMMs, per-group shapes

Page-shaped aliases follow the RapidGEMM README ("Kernels"):
  Mgemm(x, w, cnt, max_M_per_E, transpose_B) and Kgemm(grad, X, cnt, descriptor).
"""
from __future__ import annotations

import torch

from ._lib import LIB, GemmDesc, MgemmError, check, status_str  # noqa: F401

__all__ = ["fwd", "dgrad", "wgrad", "wgrad_noalloc", "fwd_swiglu", "dgrad_swiglu",
           "moe_combine", "grouped_list", "list_descriptors", "grouped_list_desc",
           "mx_scales_blocked", "fwd_mx", "wgrad_mx", "wgrad_mx_tm", "Mgemm", "Kgemm",
           "MgemmError", "status_str", "LIB"]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(dev, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the data on {dev}")


def _offsets(offsets: torch.Tensor, E: int, dev) -> torch.Tensor:
    _need(offsets, "offsets", torch.int32, 1)
    if offsets.numel() != E + 1:
        raise ValueError(f"offsets must have E+1 = {E + 1} entries, got {offsets.numel()}")
    if offsets.device != dev:
        raise ValueError("offsets must be on the same device as the data")
    return offsets


def fwd(x: torch.Tensor, w: torch.Tensor, offsets: torch.Tensor, max_m_per_e: int = 0,
        out: torch.Tensor | None = None) -> torch.Tensor:
    """M-grouped forward: out[i] = x[i] @ w[e].T for offsets[e] <= i < offsets[e+1].

    x bf16 [M, K], w bf16 [E, N, K], offsets int32 [E+1] (device).  Rows past
    offsets[E] of `out` are left untouched (uninitialised when `out` is None)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 3)
    M, K = x.shape
    E, N, K2 = w.shape
    if K2 != K:
        raise ValueError(f"x is [M, {K}] but w is [E, N, {K2}]")
    _offsets(offsets, E, x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, "out", torch.bfloat16, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be [{M}, {N}]")
    _same_device(x.device, w=w, out=out)
    with torch.cuda.device(x.device):
        st = LIB.mgemm_fwd(x.data_ptr(), w.data_ptr(), offsets.data_ptr(), out.data_ptr(),
                           M, N, K, E, int(max_m_per_e), _stream(x))
    check(st, "mgemm_fwd")
    return out


def dgrad(dy: torch.Tensor, w: torch.Tensor, offsets: torch.Tensor, max_m_per_e: int = 0,
          out: torch.Tensor | None = None) -> torch.Tensor:
    """M-grouped input gradient: out[i] = dy[i] @ w[e] for the rows of expert e.

    dy bf16 [M, N], w bf16 [E, N, K]; returns bf16 [M, K]."""
    _need(dy, "dy", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 3)
    M, N = dy.shape
    E, N2, K = w.shape
    if N2 != N:
        raise ValueError(f"dy is [M, {N}] but w is [E, {N2}, K]")
    _offsets(offsets, E, dy.device)
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device)
    else:
        _need(out, "out", torch.bfloat16, 2)
        if tuple(out.shape) != (M, K):
            raise ValueError(f"out must be [{M}, {K}]")
    _same_device(dy.device, w=w, out=out)
    with torch.cuda.device(dy.device):
        st = LIB.mgemm_dgrad(dy.data_ptr(), w.data_ptr(), offsets.data_ptr(), out.data_ptr(),
                             M, N, K, E, int(max_m_per_e), _stream(dy))
    check(st, "mgemm_dgrad")
    return out


def wgrad(dy: torch.Tensor, x: torch.Tensor, offsets: torch.Tensor, E: int | None = None,
          out: torch.Tensor | None = None, accumulate: bool = False) -> torch.Tensor:
    """K-grouped fp32 weight gradient: out[e] (=|+=) dy[rows_e].T @ x[rows_e].

    dy bf16 [M, N], x bf16 [M, K]; returns fp32 [E, N, K].  E defaults to
    offsets.numel() - 1.  With accumulate=True the sum is added into `out`."""
    return _wgrad("kgemm_wgrad", dy, x, offsets, E, out, accumulate)


def wgrad_noalloc(dy: torch.Tensor, x: torch.Tensor, offsets: torch.Tensor, out: torch.Tensor,
                  E: int | None = None, accumulate: bool = False) -> torch.Tensor:
    """wgrad through kgemm_wgrad_noalloc: the library allocates nothing (its
    token-split workspace is a static device array shared by every call on
    the GPU, so calls that can overlap race).  `out` (fp32 [E, N, K]) is
    required: the binding allocates nothing either."""
    if out is None:
        raise ValueError("wgrad_noalloc needs `out`")
    return _wgrad("kgemm_wgrad_noalloc", dy, x, offsets, E, out, accumulate)


def _wgrad(fn: str, dy, x, offsets, E, out, accumulate):
    _need(dy, "dy", torch.bfloat16, 2)
    _need(x, "x", torch.bfloat16, 2)
    M, N = dy.shape
    M2, K = x.shape
    if M2 != M:
        raise ValueError(f"dy has {M} rows but x has {M2}")
    if E is None:
        E = offsets.numel() - 1
    _offsets(offsets, E, dy.device)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs `out`")
        out = torch.empty((E, N, K), dtype=torch.float32, device=dy.device)
    else:
        _need(out, "out", torch.float32, 3)
        if tuple(out.shape) != (E, N, K):
            raise ValueError(f"out must be [{E}, {N}, {K}]")
    _same_device(dy.device, x=x, out=out)
    with torch.cuda.device(dy.device):
        st = getattr(LIB, fn)(dy.data_ptr(), x.data_ptr(), offsets.data_ptr(), out.data_ptr(),
                              M, N, K, E, 1 if accumulate else 0, _stream(dy))
    check(st, fn)
    return out


def fwd_swiglu(x: torch.Tensor, w13: torch.Tensor, offsets: torch.Tensor,
               gather: torch.Tensor | None = None, max_m_per_e: int = 0,
               out: torch.Tensor | None = None, gu_out: torch.Tensor | None = None
               ) -> torch.Tensor:
    """Gate-up forward with SwiGLU fused, on rows gathered through an index.

    w13 bf16 [E, 2I, K] stacks each expert's gate (rows 0..I-1) and up
    (rows I..2I-1) weights.  With `gather` (int32 [M], device), row i of the
    expert-grouped problem is x[gather[i]] of the token-major x bf16 [T, K];
    without it x is bf16 [M, K], already grouped.  Returns h bf16 [M, I]:
    h[i, j] = silu(g) * u, g = x[r] . w13[e, j], u = x[r] . w13[e, I + j].
    With `gu_out` (bf16 [M, 2I]) the pre-activation g | u is written too, for
    dgrad_swiglu.  Rows past offsets[E] of `out` are left untouched."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w13, "w13", torch.bfloat16, 3)
    T, K = x.shape
    E, N2, K2 = w13.shape
    if K2 != K:
        raise ValueError(f"x is [T, {K}] but w13 is [E, 2I, {K2}]")
    if N2 % 2:
        raise ValueError(f"w13 must stack two halves (2I rows), got {N2}")
    I = N2 // 2
    if gather is None:
        M = T
        gptr = 0
    else:
        _need(gather, "gather", torch.int32, 1)
        if gather.device != x.device:
            raise ValueError("gather must be on the same device as the data")
        M = gather.numel()
        gptr = gather.data_ptr()
    _offsets(offsets, E, x.device)
    if out is None:
        out = torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, "out", torch.bfloat16, 2)
        if tuple(out.shape) != (M, I):
            raise ValueError(f"out must be [{M}, {I}]")
    guptr = 0
    if gu_out is not None:
        _need(gu_out, "gu_out", torch.bfloat16, 2)
        if tuple(gu_out.shape) != (M, 2 * I):
            raise ValueError(f"gu_out must be [{M}, {2 * I}]")
        guptr = gu_out.data_ptr()
    _same_device(x.device, w13=w13, out=out, gu_out=gu_out)
    with torch.cuda.device(x.device):
        st = LIB.mgemm_fwd_swiglu_gu(x.data_ptr(), gptr, w13.data_ptr(), offsets.data_ptr(),
                                     out.data_ptr(), guptr, M, T, I, K, E, int(max_m_per_e),
                                     _stream(x))
    check(st, "mgemm_fwd_swiglu_gu")
    return out


def dgrad_swiglu(dy: torch.Tensor, w2: torch.Tensor, gu: torch.Tensor, offsets: torch.Tensor,
                 max_m_per_e: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """Down-projection input gradient fused with the SwiGLU backward.

    dy bf16 [M, N], w2 bf16 [E, N, I] (the down weights), gu bf16 [M, 2I] (the
    saved pre-activation g | u).  Returns dgu bf16 [M, 2I]: with
    dh = dy[i] @ w2[e], dgu[i, j] = dh u silu'(g), dgu[i, I + j] = dh silu(g)."""
    _need(dy, "dy", torch.bfloat16, 2)
    _need(w2, "w2", torch.bfloat16, 3)
    _need(gu, "gu", torch.bfloat16, 2)
    M, N = dy.shape
    E, N2, I = w2.shape
    if N2 != N:
        raise ValueError(f"dy is [M, {N}] but w2 is [E, {N2}, I]")
    if tuple(gu.shape) != (M, 2 * I):
        raise ValueError(f"gu must be [{M}, {2 * I}]")
    _offsets(offsets, E, dy.device)
    if out is None:
        out = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dy.device)
    else:
        _need(out, "out", torch.bfloat16, 2)
        if tuple(out.shape) != (M, 2 * I):
            raise ValueError(f"out must be [{M}, {2 * I}]")
    _same_device(dy.device, w2=w2, gu=gu, out=out)
    with torch.cuda.device(dy.device):
        st = LIB.mgemm_dgrad_swiglu(dy.data_ptr(), w2.data_ptr(), gu.data_ptr(),
                                    offsets.data_ptr(), out.data_ptr(), M, N, I, E,
                                    int(max_m_per_e), _stream(dy))
    check(st, "mgemm_dgrad_swiglu")
    return out


def _matrix(t: torch.Tensor, name: str) -> int:
    """Row stride of a bf16 matrix view whose rows are contiguous; the row
    length where no stride is needed (one row, or rows of no elements, whose
    stride torch reports as 1)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D bfloat16 tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows")
    return int(t.stride(0)) if t.shape[0] > 1 and t.shape[1] > 0 else int(t.shape[1])


def list_descriptors(groups, outs) -> torch.Tensor:
    """Device array of mg_gemm_desc for groups [(A [m, k], B [n, k]), ...] and
    outputs [D [m, n], ...] (row-strided views are fine).  The copy to the
    device is synchronous, so the host staging buffer outlives it."""
    descs = (GemmDesc * len(groups))()
    dev = None
    for g, ((a, b), d) in enumerate(zip(groups, outs)):
        lda, ldb, ldd = _matrix(a, f"A[{g}]"), _matrix(b, f"B[{g}]"), _matrix(d, f"D[{g}]")
        m, k = a.shape
        n, k2 = b.shape
        if k2 != k or tuple(d.shape) != (m, n):
            raise ValueError(f"group {g}: A {tuple(a.shape)}, B {tuple(b.shape)}, D {tuple(d.shape)}")
        dev = a.device if dev is None else dev
        if a.device != dev or b.device != dev or d.device != dev:
            raise ValueError("all groups must live on one device")
        descs[g] = GemmDesc(a.data_ptr(), b.data_ptr(), d.data_ptr(), m, n, k, lda, ldb, ldd)
    st = LIB.mg_check_list_host(descs, len(groups))
    check(st, "mg_check_list_host")
    raw = torch.frombuffer(bytearray(bytes(descs)), dtype=torch.uint8)
    return raw.to(dev)


def grouped_list_desc(desc: torch.Tensor, G: int) -> None:
    """mgemm_list on a device descriptor array (from list_descriptors)."""
    if desc.dtype != torch.uint8 or not desc.is_cuda or desc.numel() != 48 * G:
        raise ValueError("desc must be the device uint8 array of G descriptors")
    with torch.cuda.device(desc.device):
        st = LIB.mgemm_list(desc.data_ptr(), int(G), _stream(desc))
    check(st, "mgemm_list")


def grouped_list(groups, outs=None):
    """Independent GEMMs D_g = A_g @ B_g.T with per-group shapes in one launch.

    groups: [(A_g bf16 [m_g, k_g], B_g bf16 [n_g, k_g]), ...]; outs: optional
    [D_g bf16 [m_g, n_g], ...] (allocated when None).  Returns the D list."""
    if not groups:
        return []
    if outs is None:
        outs = [torch.empty((a.shape[0], b.shape[0]), dtype=torch.bfloat16, device=a.device)
                for a, b in groups]
    desc = list_descriptors(groups, outs)
    grouped_list_desc(desc, len(groups))
    return outs


def mx_scales_blocked(scales: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """E8M0 scales [..., rows, K/32] (uint8) -> the blocked layout
    [..., ceil(K/128), rows, 4] that fwd_mx reads (absent blocks 127)."""
    if not isinstance(scales, torch.Tensor) or scales.dtype != torch.uint8 or scales.dim() < 2:
        raise TypeError("scales must be a uint8 tensor [..., rows, K/32]")
    _need(scales, "scales", torch.uint8, scales.dim())
    *lead, rows, nb = scales.shape
    batch = 1
    for d in lead:
        batch *= d
    shape = (*lead, (nb + 3) // 4, rows, 4)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=scales.device)
    else:
        _need(out, "out", torch.uint8, len(shape))
        if tuple(out.shape) != shape:
            raise ValueError(f"out must be {shape}")
    _same_device(scales.device, out=out)
    with torch.cuda.device(scales.device):
        st = LIB.mg_mx_scales_blocked(scales.data_ptr(), out.data_ptr(), rows, 32 * nb, batch,
                                      _stream(scales))
    check(st, "mg_mx_scales_blocked")
    return out


def fwd_mx(x8: torch.Tensor, x_scale: torch.Tensor, w8: torch.Tensor, w_scale: torch.Tensor,
           offsets: torch.Tensor, max_m_per_e: int = 0,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """MXFP8 M-grouped forward: out[i] = X[i] @ W[e].T with X, W the E4M3
    codes x8 [M, K], w8 [E, N, K] (uint8) times their E8M0 block scales.

    x_scale: blocked [ceil(K/128), M, 4]; w_scale: blocked [E, ceil(K/128), N, 4]
    (mx_scales_blocked makes them from [M, K/32] and [E, N, K/32]).  out bf16
    [M, N]; rows past offsets[E] are left untouched."""
    _need(x8, "x8", torch.uint8, 2)
    _need(w8, "w8", torch.uint8, 3)
    M, K = x8.shape
    E, N, K2 = w8.shape
    if K2 != K:
        raise ValueError(f"x8 is [M, {K}] but w8 is [E, N, {K2}]")
    kt = (K + 127) // 128
    _need(x_scale, "x_scale", torch.uint8, 3)
    _need(w_scale, "w_scale", torch.uint8, 4)
    if tuple(x_scale.shape) != (kt, M, 4) or tuple(w_scale.shape) != (E, kt, N, 4):
        raise ValueError(f"blocked scales must be [{kt}, {M}, 4] and [{E}, {kt}, {N}, 4]")
    _offsets(offsets, E, x8.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x8.device)
    else:
        _need(out, "out", torch.bfloat16, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be [{M}, {N}]")
    _same_device(x8.device, x_scale=x_scale, w8=w8, w_scale=w_scale, out=out)
    with torch.cuda.device(x8.device):
        st = LIB.mgemm_fwd_mx(x8.data_ptr(), x_scale.data_ptr(), w8.data_ptr(), w_scale.data_ptr(),
                              offsets.data_ptr(), out.data_ptr(), M, N, K, E, int(max_m_per_e),
                              _stream(x8))
    check(st, "mgemm_fwd_mx")
    return out


def wgrad_mx(dyt8: torch.Tensor, dyt_scale: torch.Tensor, xt8: torch.Tensor,
             xt_scale: torch.Tensor, offsets: torch.Tensor, E: int | None = None,
             out: torch.Tensor | None = None, accumulate: bool = False) -> torch.Tensor:
    """MXFP8 K-grouped weight gradient: out[e] (=/+=) DYT[:, rows_e] @ XT[:, rows_e].T.

    dyt8 [N, M], xt8 [K, M]: uint8 E4M3 codes quantized along the tokens (token
    axis last); dyt_scale [M/128, N, 4], xt_scale [M/128, K, 4]: blocked E8M0
    scales (mx_scales_blocked of [N, M/32] and [K, M/32]).  offsets int32 [E+1]
    with every entry a multiple of 128.  out fp32 [E, N, K]."""
    _need(dyt8, "dyt8", torch.uint8, 2)
    _need(xt8, "xt8", torch.uint8, 2)
    N, M = dyt8.shape
    K, M2 = xt8.shape
    if M2 != M:
        raise ValueError(f"dyt8 is [N, {M}] but xt8 is [K, {M2}]")
    if E is None:
        E = offsets.numel() - 1
    _need(dyt_scale, "dyt_scale", torch.uint8, 3)
    _need(xt_scale, "xt_scale", torch.uint8, 3)
    if tuple(dyt_scale.shape) != (M // 128, N, 4) or tuple(xt_scale.shape) != (M // 128, K, 4):
        raise ValueError(f"blocked scales must be [{M // 128}, {N}, 4] and [{M // 128}, {K}, 4]")
    _offsets(offsets, E, dyt8.device)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an `out` to add into")
        out = torch.empty((E, N, K), dtype=torch.float32, device=dyt8.device)
    else:
        _need(out, "out", torch.float32, 3)
        if tuple(out.shape) != (E, N, K):
            raise ValueError(f"out must be [{E}, {N}, {K}]")
    _same_device(dyt8.device, dyt_scale=dyt_scale, xt8=xt8, xt_scale=xt_scale, out=out)
    with torch.cuda.device(dyt8.device):
        st = LIB.kgemm_wgrad_mx(dyt8.data_ptr(), dyt_scale.data_ptr(), xt8.data_ptr(),
                                xt_scale.data_ptr(), offsets.data_ptr(), out.data_ptr(),
                                M, N, K, E, 1 if accumulate else 0, _stream(dyt8))
    check(st, "kgemm_wgrad_mx")
    return out


def wgrad_mx_tm(dy8: torch.Tensor, dy_scale: torch.Tensor, x8: torch.Tensor,
                x_scale: torch.Tensor, offsets: torch.Tensor, E: int | None = None,
                out: torch.Tensor | None = None, accumulate: bool = False) -> torch.Tensor:
    """MXFP8 K-grouped weight gradient on token-major operands:
    out[e] (=/+=) DY[rows_e].T @ X[rows_e].

    dy8 [M, N], x8 [M, K]: uint8 E4M3 codes quantized along the tokens (token
    axis first, as the layer holds them); dy_scale [M/128, N, 4], x_scale
    [M/128, K, 4]: blocked E8M0 scales (mx_scales_blocked of [N, M/32] and
    [K, M/32]).  offsets int32 [E+1] with every entry a multiple of 128.
    out fp32 [E, N, K]."""
    _need(dy8, "dy8", torch.uint8, 2)
    _need(x8, "x8", torch.uint8, 2)
    M, N = dy8.shape
    M2, K = x8.shape
    if M2 != M:
        raise ValueError(f"dy8 is [{M}, N] but x8 is [{M2}, K]")
    if E is None:
        E = offsets.numel() - 1
    _need(dy_scale, "dy_scale", torch.uint8, 3)
    _need(x_scale, "x_scale", torch.uint8, 3)
    if tuple(dy_scale.shape) != (M // 128, N, 4) or tuple(x_scale.shape) != (M // 128, K, 4):
        raise ValueError(f"blocked scales must be [{M // 128}, {N}, 4] and [{M // 128}, {K}, 4]")
    _offsets(offsets, E, dy8.device)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an `out` to add into")
        out = torch.empty((E, N, K), dtype=torch.float32, device=dy8.device)
    else:
        _need(out, "out", torch.float32, 3)
        if tuple(out.shape) != (E, N, K):
            raise ValueError(f"out must be [{E}, {N}, {K}]")
    _same_device(dy8.device, dy_scale=dy_scale, x8=x8, x_scale=x_scale, out=out)
    with torch.cuda.device(dy8.device):
        st = LIB.kgemm_wgrad_mx_tm(dy8.data_ptr(), dy_scale.data_ptr(), x8.data_ptr(),
                                   x_scale.data_ptr(), offsets.data_ptr(), out.data_ptr(),
                                   M, N, K, E, 1 if accumulate else 0, _stream(dy8))
    check(st, "kgemm_wgrad_mx_tm")
    return out


def moe_combine(rows: torch.Tensor, token_rows: torch.Tensor,
                weights: torch.Tensor | None = None, out: torch.Tensor | None = None
                ) -> torch.Tensor:
    """out[t] = sum_j weights[t, j] rows[token_rows[t, j]] (bf16 [T, D]).

    rows bf16 [M, D]; token_rows int32 [T, k] (-1 = no row); weights fp32
    [T, k] or None (all 1).  The backward of the row gather of fwd_swiglu, or
    the layer's weighted output combine."""
    _need(rows, "rows", torch.bfloat16, 2)
    _need(token_rows, "token_rows", torch.int32, 2)
    M, D = rows.shape
    T, k = token_rows.shape
    wptr = 0
    if weights is not None:
        _need(weights, "weights", torch.float32, 2)
        if tuple(weights.shape) != (T, k):
            raise ValueError(f"weights must be [{T}, {k}]")
        wptr = weights.data_ptr()
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=rows.device)
    else:
        _need(out, "out", torch.bfloat16, 2)
        if tuple(out.shape) != (T, D):
            raise ValueError(f"out must be [{T}, {D}]")
    _same_device(rows.device, token_rows=token_rows, weights=weights, out=out)
    with torch.cuda.device(rows.device):
        st = LIB.mg_moe_combine(rows.data_ptr(), token_rows.data_ptr(), wptr, out.data_ptr(),
                                M, T, k, D, _stream(rows))
    check(st, "mg_moe_combine")
    return out


def Mgemm(x: torch.Tensor, w: torch.Tensor, cnt: torch.Tensor, max_M_per_E: int = 0,
          transpose_B: bool = True) -> torch.Tensor:
    """RapidGEMM-shaped M-grouped GEMM (README, "Kernels").

    w is stored [E, N, K].  transpose_B=True uses it transposed (the forward,
    x [M, K] -> [M, N]); transpose_B=False uses it as stored (the input
    gradient, x [M, N] -> [M, K]).  cnt: cumulative row offsets with a leading
    zero."""
    if transpose_B:
        return fwd(x, w, cnt, max_M_per_E)
    return dgrad(x, w, cnt, max_M_per_E)


def Kgemm(grad: torch.Tensor, X: torch.Tensor, cnt: torch.Tensor,
          descriptor: str | None = None) -> torch.Tensor:
    """RapidGEMM-shaped K-grouped fp32 weight gradient (README, "Kernels").

    descriptor names which weight is differentiated ("gw13": fused gate/up
    projection, "gw2": down projection); shapes come from the tensors, so it
    is only a label here."""
    if descriptor not in (None, "gw13", "gw2"):
        raise ValueError(f"descriptor must be 'gw13', 'gw2' or None, got {descriptor!r}")
    return wgrad(grad, X, cnt)
