"""fp64 oracle of the MXFP8 M-grouped forward and K-grouped weight gradient
(test infrastructure only).

The torchao PR #3416 ("[mxfp8 moe training] ... scale blocked format kernel
for groups along K", its "Changes" list) trains MoE layers with MXFP8 grouped
GEMMs: fp8 elements that share one e8m0 power-of-two scale per block, the
scales rearranged into a blocked layout for the grouped GEMM by a kernel of
their own, at a granularity of 128 rows x 4 scale columns.  The DeepGEMM
issue #10 thread explains why each GEMM of the backward needs its operands
quantized along its own reduction axis (activations are re-quantized for the
other axis, or kept in fp8 for the weight gradient).

Reading (the pages name the format, not its encoding): MXFP8 is the OCP
microscaling format -- blocks of 32 consecutive elements along the reduction
axis, one E8M0 scale 2^(s - 127) per block (s = 255 is NaN), E4M3 elements
(OCP FP8 E4M3: bias 7, no infinities, S.1111.111 is NaN, largest finite 448).

Storage of the inputs here (plain, unblocked):
  x8  uint8 [M, K]      E4M3 codes of expert-grouped rows,
  xs  uint8 [M, K/32]   E8M0 codes, xs[i, b] scales x8[i, 32b : 32b + 32],
  w8  uint8 [E, N, K]   E4M3 codes of the per-expert weights,
  ws  uint8 [E, N, K/32].
Forward, for offsets[e] <= i < offsets[e+1] (rows of expert e):
  Y[i, n] = sum_k dec(x8[i,k]) 2^(xs[i,k/32]-127) dec(w8[e,n,k]) 2^(ws[e,n,k/32]-127).
Every product of two E4M3 values times a power of two is exact in fp64, and
so is the scaling; the sum is one fp64 dot product per element.

The blocked scale layout of the GEMM call, [ceil(K/128)][rows][4]: for every
stretch of 128 reduction steps, the four scales of each row side by side
(bytes of absent blocks, when K is not a multiple of 128, hold 127).
"""
from __future__ import annotations

import math

import numpy as np

from .grouped_gemm import _check_offsets, expert_of_rows

MX_BLOCK = 32          # elements per shared scale along the reduction axis
MX_STAGE = 128         # reduction steps per row of the blocked scale layout


def e4m3_decode(codes) -> np.ndarray:
    """OCP FP8 E4M3 code -> value (float64), from the field definitions.

    sign s, exponent field E (4 bits, bias 7), mantissa field m (3 bits):
      E = 0:            (-1)^s 2^-6 (m / 8)         (subnormal, and zero)
      E = 15 and m = 7: NaN                         (no infinities)
      otherwise:        (-1)^s 2^(E-7) (1 + m / 8)
    """
    c = np.asarray(codes, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    E = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(E == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (E - 7).astype(np.int64)))
    val = s * val
    return np.where((E == 15) & ((c & 7) == 7), np.nan, val)


def e8m0_decode(codes) -> np.ndarray:
    """OCP E8M0 scale code -> 2^(code - 127) (float64); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, (c - 127).astype(np.int64)))


def mx_dequant(codes, scales) -> np.ndarray:
    """Values of an MX tensor [..., K] with scales [..., K/32] (float64)."""
    v = e4m3_decode(codes)
    K = v.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of the 32-element MX block")
    sc = e8m0_decode(scales)
    if sc.shape[-1] != K // MX_BLOCK:
        raise ValueError("scales must have K/32 entries per row")
    return v * np.repeat(sc, MX_BLOCK, axis=-1)


def grouped_fwd_mx(x8, xs, w8, ws, offsets) -> np.ndarray:
    """Y[i, :] = dequant(x)[i] @ dequant(w)[e].T for the rows of expert e (fp64).

    Rows at or past offsets[E] are NaN (they belong to no expert)."""
    x = mx_dequant(x8, xs)
    w = mx_dequant(w8, ws)
    M, K = x.shape
    E, N, K2 = w.shape
    assert K == K2
    o = _check_offsets(offsets, E, M)
    y = np.full((M, N), np.nan)
    for e in range(E):
        lo, hi = o[e], o[e + 1]
        if hi > lo:
            y[lo:hi] = x[lo:hi] @ w[e].T
    return y


def sample_fwd_mx(x8, xs, w8, ws, offsets, rows, cols):
    """Y[rows[j], cols[j]] of grouped_fwd_mx one element at a time, fp64.

    Only the rows and weight rows that are sampled are decoded.  Returns
    (value, sum of |products|) for the parity gate."""
    rows = np.asarray(rows); cols = np.asarray(cols)
    e = expert_of_rows(offsets, rows)
    assert (e >= 0).all()
    p = mx_dequant(np.asarray(x8)[rows], np.asarray(xs)[rows]) * \
        mx_dequant(np.asarray(w8)[e, cols], np.asarray(ws)[e, cols])
    return p.sum(axis=1), np.abs(p).sum(axis=1)


def mx_scales_blocked(scales) -> np.ndarray:
    """Plain scales [..., rows, K/32] -> the blocked layout [..., ceil(K/128), rows, 4].

    out[..., t, r, j] = scales[..., r, 4 t + j] where 4 t + j < K/32, else 127
    (the code of 1.0, so that an absent block's scale is finite)."""
    s = np.asarray(scales, dtype=np.uint8)
    *lead, rows, nb = s.shape
    nt = (nb + 3) // 4
    out = np.full((*lead, nt, rows, 4), 127, dtype=np.uint8)
    for t in range(nt):
        for j in range(4):
            b = 4 * t + j
            if b < nb:
                out[..., t, :, j] = s[..., :, b]
    return out


def blocked_bytes(rows: int, K: int) -> int:
    """Bytes of one blocked scale matrix of `rows` rows and reduction K."""
    return math.ceil(K / MX_STAGE) * rows * 4


def grouped_wgrad_mx(dyt8, dyts, xt8, xts, offsets, E: int, prior=None) -> np.ndarray:
    """MXFP8 K-grouped weight gradient (fp64, [E, N, K]).

    The torchao PR #3416 names this case -- groups along K, the token axis of
    the weight gradient -- and the DeepGEMM issue #10 thread the reason its
    operands are quantized along the tokens: each GEMM's operands are blocked
    along that GEMM's reduction axis.  So the operands come transposed, token
    axis last:
      dyt8 uint8 [N, M], dyts uint8 [N, M/32]   (dY^T and its scales),
      xt8  uint8 [K, M], xts  uint8 [K, M/32]   (X^T and its scales),
    and for the rows offsets[e] <= i < offsets[e+1] of expert e
      dW[e, n, k] = sum_i DYT[n, i] XT[k, i]      (dequantized values),
    plus `prior` when given; an expert with no rows gives zeros (or prior)."""
    dyt = mx_dequant(dyt8, dyts)
    xt = mx_dequant(xt8, xts)
    N, M = dyt.shape
    K, M2 = xt.shape
    assert M == M2
    o = _check_offsets(offsets, E, M)
    dw = np.zeros((E, N, K))
    for e in range(E):
        lo, hi = o[e], o[e + 1]
        if hi > lo:
            dw[e] = dyt[:, lo:hi] @ xt[:, lo:hi].T
    if prior is not None:
        dw = dw + prior
    return dw


def sample_wgrad_mx(dyt8, dyts, xt8, xts, offsets, experts, ns, ks):
    """dW[experts[j], ns[j], ks[j]] of grouped_wgrad_mx one element at a time,
    fp64, with sum |products|; an empty expert gives exactly (0, 0)."""
    o = np.asarray(offsets, dtype=np.int64)
    val = np.zeros(len(experts)); mag = np.zeros(len(experts))
    for j, (e, n, k) in enumerate(zip(experts, ns, ks)):
        lo, hi = o[e], o[e + 1]
        if hi <= lo:
            continue
        a = mx_dequant(np.asarray(dyt8)[n:n + 1], np.asarray(dyts)[n:n + 1])[0, lo:hi]
        b = mx_dequant(np.asarray(xt8)[k:k + 1], np.asarray(xts)[k:k + 1])[0, lo:hi]
        p = a * b
        val[j] = p.sum(); mag[j] = np.abs(p).sum()
    return val, mag
