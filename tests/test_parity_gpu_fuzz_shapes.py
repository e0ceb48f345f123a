"""Seeded random-shape fuzz of the core forward, dgrad and weight gradient,
the MXFP8 forward and weight gradients (on transposed and on token-major
operands), the gathered SwiGLU forward and its backward, the token-order
combine and the descriptor list against the oracle (needs an MI355X).
Ragged and empty experts, reductions of one block to several stages, widths
that are not multiples of the tile, strided views."""
import os

import numpy as np
import pytest
import torch

import moe_grouped_gemm_bf16_amd as mg
from oracle import (bf16_bits_to_f64, check_bf16, check_bf16_factor, check_bf16_mx,
                    check_fp32_mx, grouped_dgrad, grouped_dgrad_swiglu, grouped_fwd,
                    grouped_fwd_mx, grouped_wgrad, grouped_wgrad_mx, moe_combine, mx_dequant,
                    mx_scales_blocked)
from parity import SENTINEL, dev_bf16, dev_i32, host_bits, sentinel_bf16
from workloads import normal_bf16_bits, offsets_from_sizes
from workloads.synth import mx_e4m3_codes, mx_e8m0_codes

pytestmark = pytest.mark.gpu
# more seeds for a longer sweep: MG_FUZZ_SEEDS=<n>
SEEDS = range(int(os.environ.get("MG_FUZZ_SEEDS", "12")))


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _sizes(rng, E, hi, multiple=1):
    s = rng.integers(0, hi, E) * multiple
    s[rng.random(E) < 0.25] = 0
    return s.tolist()


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_fwd_mx(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.integers(1, 7))
    sizes = _sizes(rng, E, 400)
    N = 8 * int(rng.integers(1, 70))
    K = 32 * int(rng.integers(1, 20))
    print("[case] fuzz fwd_mx", seed, sizes, N, K, flush=True)
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + 2
    x8 = mx_e4m3_codes((M, K), 1100, seed, 1); w8 = mx_e4m3_codes((E, N, K), 1100, seed, 2)
    xs = mx_e8m0_codes((M, K // 32), 121, 2, 1100, seed, 3)
    ws = mx_e8m0_codes((E, N, K // 32), 121, 2, 1100, seed, 4)
    y = mg.fwd_mx(_u8(x8), _u8(mx_scales_blocked(xs)), _u8(w8), _u8(mx_scales_blocked(ws)),
                  dev_i32(off), out=sentinel_bf16((M, N)))
    got = host_bits(y)
    o = int(off[-1])
    exact = grouped_fwd_mx(x8, xs, w8, ws, off)[:o]
    mag = grouped_fwd(np.abs(mx_dequant(x8, xs)), np.abs(mx_dequant(w8, ws)), off)[:o]
    rep = check_bf16_mx(got[:o], exact, mag)
    assert rep.passed, str(rep)
    assert (got[o:] == SENTINEL).all()


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_wgrad_mx(seed):
    rng = np.random.default_rng(2000 + seed)
    E = int(rng.integers(1, 6))
    sizes = _sizes(rng, E, 5, multiple=128)
    N = 8 * int(rng.integers(1, 50)); K = 8 * int(rng.integers(1, 50))
    print("[case] fuzz wgrad_mx", seed, sizes, N, K, flush=True)
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + 128
    dyt8 = mx_e4m3_codes((N, M), 2100, seed, 1); xt8 = mx_e4m3_codes((K, M), 2100, seed, 2)
    dyts = mx_e8m0_codes((N, M // 32), 121, 2, 2100, seed, 3)
    xts = mx_e8m0_codes((K, M // 32), 121, 2, 2100, seed, 4)
    out = mg.wgrad_mx(_u8(dyt8), _u8(mx_scales_blocked(dyts)), _u8(xt8),
                      _u8(mx_scales_blocked(xts)), dev_i32(off), E)
    got = out.cpu().numpy()
    exact = grouped_wgrad_mx(dyt8, dyts, xt8, xts, off, E)
    mag = grouped_wgrad(np.abs(mx_dequant(dyt8, dyts)).T, np.abs(mx_dequant(xt8, xts)).T, off, E)
    sz = np.diff(np.asarray(off, np.int64))
    k_red = np.broadcast_to(np.maximum(sz, 1)[:, None, None], exact.shape)
    empty = np.broadcast_to((sz == 0)[:, None, None], exact.shape)
    rep = check_fp32_mx(got, exact, mag, k_red, empty_mask=empty)
    assert rep.passed, str(rep)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_wgrad_mx_token_major(seed):
    """The token-major MXFP8 weight gradient on random shapes (N, K multiples
    of 16): within the oracle's gate and bitwise equal to the call on the
    transposed codes."""
    rng = np.random.default_rng(2500 + seed)
    E = int(rng.integers(1, 6))
    sizes = _sizes(rng, E, 5, multiple=128)
    N = 16 * int(rng.integers(1, 40)); K = 16 * int(rng.integers(1, 40))
    print("[case] fuzz wgrad_mx_tm", seed, sizes, N, K, flush=True)
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + 128
    dyt8 = mx_e4m3_codes((N, M), 2600, seed, 1); xt8 = mx_e4m3_codes((K, M), 2600, seed, 2)
    dyts = mx_e8m0_codes((N, M // 32), 121, 2, 2600, seed, 3)
    xts = mx_e8m0_codes((K, M // 32), 121, 2, 2600, seed, 4)
    bd, bx, o = _u8(mx_scales_blocked(dyts)), _u8(mx_scales_blocked(xts)), dev_i32(off)
    out = mg.wgrad_mx_tm(_u8(dyt8.T), bd, _u8(xt8.T), bx, o, E,
                         out=torch.full((E, N, K), float("nan"), device="cuda"))
    ref = mg.wgrad_mx(_u8(dyt8), bd, _u8(xt8), bx, o, E)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    got = out.cpu().numpy()
    exact = grouped_wgrad_mx(dyt8, dyts, xt8, xts, off, E)
    mag = grouped_wgrad(np.abs(mx_dequant(dyt8, dyts)).T, np.abs(mx_dequant(xt8, xts)).T, off, E)
    sz = np.diff(np.asarray(off, np.int64))
    k_red = np.broadcast_to(np.maximum(sz, 1)[:, None, None], exact.shape)
    empty = np.broadcast_to((sz == 0)[:, None, None], exact.shape)
    rep = check_fp32_mx(got, exact, mag, k_red, empty_mask=empty)
    assert rep.passed, str(rep)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_dgrad_swiglu(seed):
    rng = np.random.default_rng(3000 + seed)
    E = int(rng.integers(1, 6))
    sizes = _sizes(rng, E, 500)
    N = 8 * int(rng.integers(1, 100)); I = 8 * int(rng.integers(1, 60))
    print("[case] fuzz dgrad_swiglu", seed, sizes, N, I, flush=True)
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + 1
    dyb = normal_bf16_bits((M, N), 1.0, 3100, seed, 1)
    w2b = normal_bf16_bits((E, N, I), N ** -0.5, 3100, seed, 2)
    gub = normal_bf16_bits((M, 2 * I), 2.0, 3100, seed, 3)
    out = mg.dgrad_swiglu(dev_bf16(dyb), dev_bf16(w2b), dev_bf16(gub), dev_i32(off),
                          out=sentinel_bf16((M, 2 * I)))
    got = host_bits(out)
    o = int(off[-1])
    dy, w2, gu = bf16_bits_to_f64(dyb), bf16_bits_to_f64(w2b), bf16_bits_to_f64(gub)
    exact, _ = grouped_dgrad_swiglu(dy, w2, gu, off)
    S = grouped_dgrad(np.abs(dy), np.abs(w2), off)
    g, u = gu[:, :I], gu[:, I:]
    s = 1 / (1 + np.exp(-g))
    fac = np.concatenate([u * s * (1 + g * (1 - s)), g * s], axis=1)
    rep = check_bf16_factor(got[:o], exact[:o], fac[:o], np.concatenate([S, S], axis=1)[:o], N)
    assert rep.passed, str(rep)
    assert (got[o:] == SENTINEL).all()


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_moe_combine(seed):
    rng = np.random.default_rng(4000 + seed)
    T = int(rng.integers(1, 400)); k = int(rng.integers(1, 10)); M = int(rng.integers(1, 900))
    D = 8 * int(rng.integers(1, 100))
    print("[case] fuzz moe_combine", seed, T, k, M, D, flush=True)
    rows = normal_bf16_bits((M, D), 1.0, 4100, seed, 1)
    tr = rng.integers(-1, M, (T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32) if seed % 2 else None
    out = mg.moe_combine(dev_bf16(rows), dev_i32(tr),
                         None if w is None else torch.from_numpy(w).cuda())
    got = host_bits(out)
    R = bf16_bits_to_f64(rows)
    wf = None if w is None else w.astype(np.float64)
    exact = moe_combine(R, tr, wf)
    mag = moe_combine(np.abs(R), tr, None if wf is None else np.abs(wf))
    rep = check_bf16(got, exact, mag, k)
    assert rep.passed, str(rep)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_core_ops(seed):
    """The three core calls on random shapes: the M-grouped forward and dgrad
    (rows past offsets[E] untouched) and the K-grouped weight gradient (with or
    without accumulation into a prior), every element against the oracle."""
    from parity import gate_dgrad_full, gate_fwd_full, gate_wgrad_full
    rng = np.random.default_rng(5000 + seed)
    E = int(rng.integers(1, 10))
    sizes = _sizes(rng, E, 600)
    if sum(sizes) == 0:
        sizes[0] = 40                     # (all experts empty has a test of its own)
    N = 8 * int(rng.integers(1, 80)); K = 8 * int(rng.integers(1, 80))
    acc = bool(seed % 2)
    print("[case] fuzz core", seed, sizes, N, K, "accumulate" if acc else "", flush=True)
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + 3
    xb = normal_bf16_bits((M, K), K ** -0.5, 5100, seed, 1)
    wb = normal_bf16_bits((E, N, K), K ** -0.5, 5100, seed, 2)
    dyb = normal_bf16_bits((M, N), 1.0, 5100, seed, 3)
    o = dev_i32(off)
    y = mg.fwd(dev_bf16(xb), dev_bf16(wb), o, out=sentinel_bf16((M, N)))
    dx = mg.dgrad(dev_bf16(dyb), dev_bf16(wb), o, out=sentinel_bf16((M, K)))
    prior = rng.standard_normal((E, N, K)).astype(np.float32) if acc else None
    dw = mg.wgrad(dev_bf16(dyb), dev_bf16(xb), o, E,
                  out=None if prior is None else torch.from_numpy(prior.copy()).cuda(),
                  accumulate=acc)
    torch.cuda.synchronize()
    yb, dxb = host_bits(y), host_bits(dx)
    o_end = int(off[-1])
    assert (yb[o_end:] == SENTINEL).all() and (dxb[o_end:] == SENTINEL).all()
    rep = gate_fwd_full(xb, wb, off, yb)
    assert rep.passed, f"fwd: {rep}"
    rep = gate_dgrad_full(dyb, wb, off, dxb)
    assert rep.passed, f"dgrad: {rep}"
    rep = gate_wgrad_full(dyb, xb, off, dw.cpu().numpy(),
                          prior=None if prior is None else prior.astype(np.float64))
    assert rep.passed, f"wgrad: {rep}"


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_grouped_list(seed):
    """The descriptor list on random groups: 1-8 independent GEMMs of random
    m, n, k (empty groups and k = 0 included), operands as views with padded
    row strides and outputs inside wider buffers, every element against the
    oracle and the padding columns untouched."""
    from oracle import check_bf16, grouped_list
    rng = np.random.default_rng(7000 + seed)
    G = int(rng.integers(1, 9))
    shapes = []
    for _ in range(G):
        m = int(rng.integers(0, 600)) if rng.random() > 0.15 else 0
        n = 8 * int(rng.integers(1, 80))
        k = 8 * int(rng.integers(0, 80)) if rng.random() > 0.1 else 0
        shapes.append((m, n, k))
    print("[case] fuzz list", seed, shapes, flush=True)
    bits, groups, outs, pads = [], [], [], []
    for g, (m, n, k) in enumerate(shapes):
        pa, pb, pd = (8 * int(v) for v in rng.integers(0, 4, 3))
        ab = normal_bf16_bits((m, k), 1.0, 7100, seed, g, 1)
        bb = normal_bf16_bits((n, k), k ** -0.5 if k else 1.0, 7100, seed, g, 2)
        abuf = torch.zeros((m, k + pa), dtype=torch.bfloat16, device="cuda")
        bbuf = torch.zeros((n, k + pb), dtype=torch.bfloat16, device="cuda")
        if m * k:
            abuf[:, :k] = dev_bf16(ab)
        if n * k:
            bbuf[:, :k] = dev_bf16(bb)
        dbuf = sentinel_bf16((m, n + pd))
        bits.append((ab, bb))
        groups.append((abuf[:, :k], bbuf[:, :k]))
        outs.append(dbuf[:, :n])
        pads.append((dbuf, pd))
    mg.grouped_list(groups, outs)
    torch.cuda.synchronize()
    a64 = [(bf16_bits_to_f64(a), bf16_bits_to_f64(b)) for a, b in bits]
    ref = grouped_list(a64)
    mag = grouped_list([(np.abs(a), np.abs(b)) for a, b in a64])
    for g, ((m, n, k), d, r, s, (dbuf, pd)) in enumerate(zip(shapes, outs, ref, mag, pads)):
        if m == 0:
            continue
        rep = check_bf16(host_bits(d), r, s, max(k, 1))
        assert rep.passed, f"group {g} {shapes[g]}: {rep}"
        if pd:
            assert (host_bits(dbuf)[:, n:] == SENTINEL).all(), f"group {g}: padding written"


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_fwd_swiglu(seed):
    """The gate-up forward with SwiGLU on random shapes: rows gathered from a
    random token map (or not), ragged and empty experts, and for odd seeds the
    saved pre-activation g | u as well; h on every element against the
    oracle, g | u against the oracle's plain forward, rows past offsets[E]
    untouched."""
    from oracle import check_bf16_swiglu, sample_fwd_swiglu
    rng = np.random.default_rng(8000 + seed)
    E = int(rng.integers(1, 8))
    sizes = _sizes(rng, E, 500)
    I = 8 * int(rng.integers(1, 50)); K = 8 * int(rng.integers(1, 60))
    gathered = bool(rng.integers(0, 2))
    save = bool(seed % 2)
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + 2
    T = int(rng.integers(1, 700)) if gathered else M
    print("[case] fuzz fwd_swiglu", seed, sizes, I, K, "T", T if gathered else None,
          "save" if save else "", flush=True)
    xb = normal_bf16_bits((T, K), 1.0, 8100, seed, 1)
    wb = normal_bf16_bits((E, 2 * I, K), K ** -0.5, 8100, seed, 2)
    gather = rng.integers(0, T, M).astype(np.int32) if gathered else None
    gu = sentinel_bf16((M, 2 * I)) if save else None
    h = mg.fwd_swiglu(dev_bf16(xb), dev_bf16(wb), dev_i32(off),
                      gather=None if gather is None else dev_i32(gather),
                      out=sentinel_bf16((M, I)), gu_out=gu)
    torch.cuda.synchronize()
    got = host_bits(h)
    o_end = int(off[-1])
    assert (got[o_end:] == SENTINEL).all()
    if o_end:
        rows = np.repeat(np.arange(o_end), I)
        cols = np.tile(np.arange(I), o_end)
        hh, g, u, sg, su = sample_fwd_swiglu(xb, gather, wb, off, rows, cols)
        rep = check_bf16_swiglu(got[rows, cols], hh, g, u, sg, su, K)
        assert rep.passed, f"h: {rep}"
    if save:
        gub = host_bits(gu)
        assert (gub[o_end:] == SENTINEL).all()
    if save and o_end:
        rows_x = xb if gather is None else xb[gather]
        x64, w64 = bf16_bits_to_f64(rows_x), bf16_bits_to_f64(wb)
        rep = check_bf16(gub[:o_end], grouped_fwd(x64, w64, off)[:o_end],
                         grouped_fwd(np.abs(x64), np.abs(w64), off)[:o_end], K)
        assert rep.passed, f"g | u: {rep}"
