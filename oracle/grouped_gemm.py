"""fp64 oracle of the M-grouped and K-grouped GEMMs (test infrastructure only).

Shapes follow the RapidGEMM README ("Kernels"): x [M, K] holds expert-grouped
rows, w [E, N, K] the per-expert weights, and a cumulative row-offset array
with a leading zero, offsets [E + 1], says that expert e owns rows
offsets[e] <= i < offsets[e+1].  Rows at or past offsets[E] belong to no
expert; the oracle marks them NaN in fwd/dgrad results.

Inputs are float64 arrays (bf16 inputs decoded exactly).  Each function is
the definition written out: one dense float64 matmul per expert.
"""
from __future__ import annotations

import numpy as np

from .bf16 import bf16_bits_to_f64


def _check_offsets(offsets, E: int, M: int) -> np.ndarray:
    o = np.asarray(offsets, dtype=np.int64)
    if o.shape != (E + 1,):
        raise ValueError(f"offsets must have E+1={E + 1} entries, got {o.shape}")
    if o[0] != 0 or (np.diff(o) < 0).any() or o[-1] > M:
        raise ValueError("offsets must start at 0, be non-decreasing and end <= M")
    return o


def grouped_fwd(x: np.ndarray, w: np.ndarray, offsets) -> np.ndarray:
    """Y[i, :] = x[i, :] @ w[e].T for offsets[e] <= i < offsets[e+1]  (fp64)."""
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


def grouped_dgrad(dy: np.ndarray, w: np.ndarray, offsets) -> np.ndarray:
    """dX[i, :] = dy[i, :] @ w[e] for offsets[e] <= i < offsets[e+1]  (fp64)."""
    M, N = dy.shape
    E, N2, K = w.shape
    assert N == N2
    o = _check_offsets(offsets, E, M)
    dx = np.full((M, K), np.nan)
    for e in range(E):
        lo, hi = o[e], o[e + 1]
        if hi > lo:
            dx[lo:hi] = dy[lo:hi] @ w[e]
    return dx


def grouped_wgrad(dy: np.ndarray, x: np.ndarray, offsets, E: int,
                  prior: np.ndarray | None = None) -> np.ndarray:
    """dW[e] = dy[rows_e].T @ x[rows_e]  (fp64, [E, N, K]); empty e gives 0.

    With `prior`, the result is prior + that (the accumulate-into-fp32 form of
    the TransformerEngine PR #2045 discussion of fuse_wgrad_accumulation)."""
    M, N = dy.shape
    M2, K = x.shape
    assert M == M2
    o = _check_offsets(offsets, E, M)
    dw = np.zeros((E, N, K))
    for e in range(E):
        lo, hi = o[e], o[e + 1]
        if hi > lo:
            dw[e] = dy[lo:hi].T @ x[lo:hi]
    if prior is not None:
        dw = dw + prior
    return dw


def _silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)); exp overflow gives -0."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def grouped_fwd_swiglu(x: np.ndarray, gather, w13: np.ndarray, offsets) -> np.ndarray:
    """Gate-up forward with the SwiGLU activation, on gathered rows (fp64).

    The DeepGEMM issue #10 thread names the fused kernels an MoE weight-gradient
    path needs -- with casting, with SwiGLU, with the MoE layout -- and the
    RapidGEMM README ("Kernels") calls the first FFN weight gradient gw13: the
    gate (w1) and up (w3) weights of each expert stacked as one [2I, K] matrix,
    w1 in rows 0..I-1 and w3 in rows I..2I-1.  Row i of the expert-grouped
    problem is token row gather[i] of x (gather None: x is already grouped).
    For offsets[e] <= i < offsets[e+1]:
        g = x[gather[i]] . w13[e, j],   u = x[gather[i]] . w13[e, I + j],
        h[i, j] = silu(g) * u,  silu(g) = g / (1 + exp(-g))        (j < I)
    Rows at or past offsets[E] are NaN."""
    rows = x if gather is None else x[np.asarray(gather, np.int64)]
    M, K = rows.shape
    E, N2, K2 = w13.shape
    assert K == K2 and N2 % 2 == 0
    I = N2 // 2
    o = _check_offsets(offsets, E, M)
    h = np.full((M, I), np.nan)
    for e in range(E):
        lo, hi = o[e], o[e + 1]
        if hi > lo:
            g = rows[lo:hi] @ w13[e, :I].T
            u = rows[lo:hi] @ w13[e, I:].T
            h[lo:hi] = _silu(g) * u
    return h


def _sigmoid(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def grouped_dgrad_swiglu(dy: np.ndarray, w2: np.ndarray, gu: np.ndarray, offsets):
    """Down-projection input gradient with the SwiGLU backward (fp64).

    The DeepGEMM issue #10 thread counts a kernel fused with SwiGLU among what a
    weight-gradient path needs besides the GEMMs.  With the forward
    h = silu(g) u (grouped_fwd_swiglu) followed by the down projection
    y = h W2[e]^T (W2 [E, N, I]), the backward takes dy [M, N] and the saved
    pre-activation gu [M, 2I] (g in columns 0..I-1, u in I..2I-1) and returns
    dgu [M, 2I]:
        dh = dy @ W2[e]                           (the grouped input gradient)
        dg = dh u silu'(g),  silu'(g) = s (1 + g (1 - s)),  s = 1 / (1 + exp(-g))
        du = dh silu(g)
    for the rows of expert e; rows at or past offsets[E] are NaN.  Also
    returns dh."""
    M, N = dy.shape
    E, N2, I = w2.shape
    assert N == N2 and gu.shape == (M, 2 * I)
    dh = grouped_dgrad(dy, w2, offsets)
    g, u = gu[:, :I], gu[:, I:]
    s = _sigmoid(g)
    dgu = np.concatenate([dh * u * s * (1.0 + g * (1.0 - s)), dh * g * s], axis=1)
    return dgu, dh


def sample_dgrad_swiglu(dy, w2, gu, offsets, rows, cols):
    """dg and du at (rows[j], cols[j]) (cols < I) one element at a time, fp64.

    Returns (dg, du, dh, sum |dy w2|) for the parity gate."""
    rows = np.asarray(rows); cols = np.asarray(cols)
    e = expert_of_rows(offsets, rows)
    assert (e >= 0).all()
    I = w2.shape[2]
    p = _f64(dy[rows]) * _f64(w2[e, :, cols])         # [S, N]
    dh = p.sum(axis=1)
    g = _f64(gu[rows, cols]); u = _f64(gu[rows, I + cols])
    s = _sigmoid(g)
    return dh * u * s * (1.0 + g * (1.0 - s)), dh * g * s, dh, np.abs(p).sum(axis=1)


def sample_fwd_swiglu(x: np.ndarray, gather, w13: np.ndarray, offsets, rows, cols):
    """h[rows[j], cols[j]] of grouped_fwd_swiglu one element at a time, fp64.

    Returns (h, g, u, sum |x w1|, sum |x w3|) for the parity gate."""
    rows = np.asarray(rows); cols = np.asarray(cols)
    e = expert_of_rows(offsets, rows)
    assert (e >= 0).all()
    I = w13.shape[1] // 2
    src = rows if gather is None else np.asarray(gather, np.int64)[rows]
    xr = _f64(x[src])
    pg = xr * _f64(w13[e, cols])
    pu = xr * _f64(w13[e, I + cols])
    g, u = pg.sum(axis=1), pu.sum(axis=1)
    return _silu(g) * u, g, u, np.abs(pg).sum(axis=1), np.abs(pu).sum(axis=1)


def grouped_list(groups) -> list:
    """A list of independent GEMMs, one per group: D_g = A_g @ B_g.T  (fp64).

    The TransformerEngine PR #2045 review asks for one C API over lists of
    per-group tensors, and the CUTLASS discussion #1452 ("Grouped GEMM where
    each subproblem is another grouped gemm instance") flattens nested grouped
    GEMMs such as LoRA x experts into such a list.  groups: sequence of
    (A [m, k], B [n, k]) float64 arrays; returns the list of D [m, n]."""
    out = []
    for a, b in groups:
        a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
        assert a.ndim == 2 and b.ndim == 2 and a.shape[1] == b.shape[1]
        out.append(a @ b.T)
    return out


def expert_of_rows(offsets, rows: np.ndarray) -> np.ndarray:
    """Expert index owning each row (rows past offsets[E] give -1)."""
    o = np.asarray(offsets, dtype=np.int64)
    e = np.searchsorted(o, rows, side="right") - 1
    return np.where(np.asarray(rows) < o[-1], e, -1)


def _f64(a: np.ndarray) -> np.ndarray:
    """Gathered operand pieces: bf16 bit patterns are decoded exactly."""
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else np.asarray(a, np.float64)


def sample_fwd(x: np.ndarray, w: np.ndarray, offsets, rows, cols):
    """Y[rows[j], cols[j]] one element at a time (vectorised over j), fp64.

    x, w may be float64 arrays or bf16 bit patterns (only the gathered rows are
    decoded).  Returns (value, sum of |products|); the second feeds the
    accumulation-error floor of the parity gate.  Rows must lie below
    offsets[E]."""
    rows = np.asarray(rows); cols = np.asarray(cols)
    e = expert_of_rows(offsets, rows)
    assert (e >= 0).all()
    p = _f64(x[rows]) * _f64(w[e, cols])        # [S, K]
    return p.sum(axis=1), np.abs(p).sum(axis=1)


def sample_dgrad(dy: np.ndarray, w: np.ndarray, offsets, rows, cols):
    """dX[rows[j], cols[j]] = sum_n dy[r, n] w[e, n, c], fp64, with sum |.|."""
    rows = np.asarray(rows); cols = np.asarray(cols)
    e = expert_of_rows(offsets, rows)
    assert (e >= 0).all()
    p = _f64(dy[rows]) * _f64(w[e, :, cols])    # [S, N]
    return p.sum(axis=1), np.abs(p).sum(axis=1)


def sample_wgrad(dy: np.ndarray, x: np.ndarray, offsets, experts, ns, ks):
    """dW[experts[j], ns[j], ks[j]] = sum over the expert's rows, fp64,
    with sum |.|; an empty expert gives exactly (0, 0)."""
    o = np.asarray(offsets, dtype=np.int64)
    val = np.zeros(len(experts)); mag = np.zeros(len(experts))
    for j, (e, n, k) in enumerate(zip(experts, ns, ks)):
        lo, hi = o[e], o[e + 1]
        p = _f64(dy[lo:hi, n]) * _f64(x[lo:hi, k])
        val[j] = p.sum(); mag[j] = np.abs(p).sum()
    return val, mag


def moe_combine(rows: np.ndarray, token_rows, weights=None) -> np.ndarray:
    """Token-order sum of routed rows (fp64): the inverse of the gather.

    The forward reads token t's activations into the rows i with gather[i] = t
    (one per routed expert, the MoE layout of the DeepGEMM issue #10 thread);
    the backward of that gather sums those rows' gradients back per token, and
    the output combine of the layer sums the experts' outputs per token with
    the router's weights.  token_rows int [T, k]: the rows of token t (-1 =
    none); weights [T, k] or None (all 1):
        out[t, :] = sum_j weights[t, j] rows[token_rows[t, j], :]."""
    tr = np.asarray(token_rows, dtype=np.int64)
    T, k = tr.shape
    D = rows.shape[1]
    w = np.ones((T, k)) if weights is None else np.asarray(weights, np.float64)
    out = np.zeros((T, D))
    for j in range(k):
        ok = tr[:, j] >= 0
        out[ok] += w[ok, j][:, None] * np.asarray(rows, np.float64)[tr[ok, j]]
    return out
