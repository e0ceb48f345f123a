"""GPU parity of the SwiGLU backward fused into the down projection's input
gradient, and of the pre-activation the fused forward saves for it (needs an
MI355X).

dgu (bf16) passes the gate of oracle/gate.py for outputs f * dh with dh an
fp32 sum: one bf16 ulp of the rounded oracle value, or within dh's fp32
summation error carried through the factor f.  The saved g | u must equal the
plain grouped forward's output on the same rows bit for bit.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_bf16_amd as mg
from oracle import (bf16_bits_to_f64, check_bf16_factor, grouped_dgrad, grouped_dgrad_swiglu,
                    sample_dgrad_swiglu)
from parity import SENTINEL, dev_bf16, dev_i32, host_bits, sentinel_bf16
from workloads import make_workload, normal_bf16_bits, offsets_from_sizes

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _factors(gu: np.ndarray, I: int):
    g, u = gu[:, :I], gu[:, I:]
    s = 1.0 / (1.0 + np.exp(-g))
    return np.concatenate([u * s * (1.0 + g * (1.0 - s)), g * s], axis=1)


# (expert sizes, N = model width, I = expert width, extra rows)
BW_CASES = [
    ([200, 0, 184, 128], 256, 128, 3),
    ([1, 255, 256, 257], 136, 264, 5),
    ([0, 513, 0, 1, 300], 520, 72, 0),
    ([700], 1032, 520, 2),
]


@pytest.mark.parametrize("case", range(len(BW_CASES)))
def test_dgrad_swiglu(case):
    sizes, N, I, extra = BW_CASES[case]
    _say("dgrad_swiglu", sizes, N, I, extra)
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + extra
    E = len(sizes)
    dyb = normal_bf16_bits((M, N), 1.0, 900 + case, 1)
    w2b = normal_bf16_bits((E, N, I), N ** -0.5, 900 + case, 2)
    gub = normal_bf16_bits((M, 2 * I), 2.0, 900 + case, 3)
    out = mg.dgrad_swiglu(dev_bf16(dyb), dev_bf16(w2b), dev_bf16(gub), dev_i32(off),
                          out=sentinel_bf16((M, 2 * I)))
    got = host_bits(out)
    o = int(off[-1])
    dy, w2, gu = bf16_bits_to_f64(dyb), bf16_bits_to_f64(w2b), bf16_bits_to_f64(gub)
    exact, _ = grouped_dgrad_swiglu(dy, w2, gu, off)
    S = grouped_dgrad(np.abs(dy), np.abs(w2), off)
    rep = check_bf16_factor(got[:o], exact[:o], _factors(gu, I)[:o],
                            np.concatenate([S, S], axis=1)[:o], N)
    assert rep.passed, str(rep)
    assert (got[o:] == SENTINEL).all(), "rows past offsets[E] were written"


def test_dgrad_swiglu_a3b_down_sampled():
    """The 30B-A3B down projection's backward (N 3072, I 1280, 32 experts,
    routed rows) in the launch a trainer makes: sampled elements, both
    halves, every expert's first and last row."""
    (wl,) = make_workload(4, "a3b_down")
    off = np.asarray(wl.offsets)
    M, N, I, E = wl.M, wl.N, wl.K, wl.E
    _say("dgrad_swiglu a3b", M, N, I, E)
    dyb = normal_bf16_bits((M, N), 1.0, 950, 1)
    w2b = normal_bf16_bits((E, N, I), N ** -0.5, 950, 2)
    gub = normal_bf16_bits((M, 2 * I), 2.0, 950, 3)
    out = mg.dgrad_swiglu(dev_bf16(dyb), dev_bf16(w2b), dev_bf16(gub), dev_i32(off),
                          max_m_per_e=int(np.diff(off).max()))
    got = host_bits(out)
    rng = np.random.default_rng(951)
    last = int(off[-1])
    live = np.diff(off) > 0
    edges = np.concatenate([off[:-1][live], off[1:][live] - 1])
    rows = np.concatenate([rng.integers(0, last, 2048), edges, edges])
    cols = np.concatenate([rng.integers(0, I, 2048), np.zeros_like(edges), np.full_like(edges, I - 1)])
    dg, du, dh, S = sample_dgrad_swiglu(dyb, w2b, gub, off, rows, cols)
    gu = bf16_bits_to_f64(gub)
    g, u = gu[rows, cols], gu[rows, I + cols]
    s = 1.0 / (1.0 + np.exp(-g))
    r1 = check_bf16_factor(got[rows, cols], dg, u * s * (1 + g * (1 - s)), S, N)
    r2 = check_bf16_factor(got[rows, I + cols], du, g * s, S, N)
    assert r1.passed, str(r1)
    assert r2.passed, str(r2)


@pytest.mark.parametrize("gathered", [False, True])
def test_fwd_swiglu_saves_the_plain_forward(gathered):
    """gu from the fused forward is bit for bit the plain grouped forward of
    the same rows with w13, and h does not change when gu is requested."""
    sizes, I, K = [300, 0, 17, 513], 264, 136
    off = offsets_from_sizes(sizes)
    M, E = int(off[-1]), len(sizes)
    T = 700 if gathered else M
    _say("fwd_swiglu gu", sizes, I, K, "gathered" if gathered else "")
    xb = normal_bf16_bits((T, K), 1.0, 960, 1)
    wb = normal_bf16_bits((E, 2 * I, K), K ** -0.5, 960, 2)
    gather = np.random.default_rng(961).integers(0, T, M).astype(np.int32) if gathered else None
    x, w = dev_bf16(xb), dev_bf16(wb)
    o = dev_i32(off)
    gi = None if gather is None else dev_i32(gather)
    gu = sentinel_bf16((M, 2 * I))
    h1 = mg.fwd_swiglu(x, w, o, gather=gi, gu_out=gu)
    h2 = mg.fwd_swiglu(x, w, o, gather=gi)
    xg = x if gather is None else x.index_select(0, gi.long()).contiguous()
    y = mg.fwd(xg, w, o)
    assert (host_bits(h1) == host_bits(h2)).all()
    assert (host_bits(gu) == host_bits(y)).all()


# ---------------------------------------------------------------- combine --

from oracle import check_bf16, moe_combine  # noqa: E402


def _inverse(tok: np.ndarray, T: int, k: int) -> np.ndarray:
    """token -> its rows (row i carries token tok[i]), -1 padded, rows ascending."""
    tr = -np.ones((T, k), np.int32)
    fill = np.zeros(T, np.int64)
    for i, t in enumerate(tok):
        tr[t, fill[t]] = i
        fill[t] += 1
    return tr


def _combine_gate(rows_bits, token_rows, weights, got_bits, sample=None):
    tr = np.asarray(token_rows, np.int64)
    if sample is not None:
        tr = tr[sample]
        got_bits = got_bits[sample]
    used = np.unique(tr[tr >= 0])
    remap = -np.ones(int(rows_bits.shape[0]), np.int64)
    remap[used] = np.arange(len(used))
    tr2 = np.where(tr >= 0, remap[np.maximum(tr, 0)], -1)
    R = bf16_bits_to_f64(rows_bits[used])
    w = None if weights is None else (weights if sample is None else weights[sample])
    exact = moe_combine(R, tr2, w)
    mag = moe_combine(np.abs(R), tr2, None if w is None else np.abs(w))
    return check_bf16(got_bits, exact, mag, tr.shape[1])


@pytest.mark.parametrize("weighted", [False, True])
def test_moe_combine_small(weighted):
    rng = np.random.default_rng(970 + weighted)
    T, k, M, D = 100, 4, 300, 264
    _say("moe_combine", T, k, M, D, "weighted" if weighted else "")
    rows = normal_bf16_bits((M, D), 1.0, 970, 1)
    tr = rng.integers(-1, M, (T, k)).astype(np.int32)     # -1: no row
    tr[3] = -1                                             # a token with no rows at all
    tr[5, 0] = M + 7                                       # an index out of range: skipped
    w = rng.random((T, k)).astype(np.float32) if weighted else None
    out = mg.moe_combine(dev_bf16(rows), dev_i32(tr),
                         None if w is None else torch.from_numpy(w).cuda())
    got = host_bits(out)
    tr_ok = np.where((tr >= 0) & (tr < M), tr, -1)
    rep = _combine_gate(rows, tr_ok, None if w is None else w.astype(np.float64), got)
    assert rep.passed, str(rep)
    assert (got[3] == 0).all()


def test_moe_combine_a3b_routing():
    """The 30B-A3B routing of one GPU's share: 16384 tokens, up to 8 local rows
    each, D = 3072 (the gate-up input gradient back to token order), with and
    without router weights; sampled tokens, and bitwise reproducible."""
    from workloads.synth import router_offsets
    off, tok = router_offsets(16384, 128, 8, 32, seed=4)
    T, k, D = 16384, 8, 3072
    M = int(off[-1])
    tr = _inverse(np.asarray(tok), T, k)
    _say("moe_combine a3b", T, k, M, D)
    rows = normal_bf16_bits((M, D), 1.0, 975, 1)
    w = np.random.default_rng(976).random((T, k)).astype(np.float32)
    r_d, t_d = dev_bf16(rows), dev_i32(tr)
    o1 = host_bits(mg.moe_combine(r_d, t_d))
    o2 = host_bits(mg.moe_combine(r_d, t_d))
    ow = host_bits(mg.moe_combine(r_d, t_d, torch.from_numpy(w).cuda()))
    assert (o1 == o2).all()
    sample = np.random.default_rng(977).choice(T, 512, replace=False)
    r1 = _combine_gate(rows, tr, None, o1, sample)
    r2 = _combine_gate(rows, tr, w.astype(np.float64), ow, sample)
    assert r1.passed, str(r1)
    assert r2.passed, str(r2)
    assert (o1[(tr < 0).all(axis=1)] == 0).all()           # tokens routed to no local expert
