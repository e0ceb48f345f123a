"""Pins of the MXFP8 oracle (CPU only).

The decoders are checked against torch's own float8 casts on every code and
against closed forms; the grouped forward against exact rational brute force
and power-of-two scale identities; the blocked scale layout against an
index-by-index loop; the parity gate against the mistakes it must catch.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import mx as omx
from workloads import synth


def _torch_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e8m0(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def test_e4m3_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = omx.e4m3_decode(codes), _torch_e4m3(codes)
    assert (np.isnan(ours) == np.isnan(ref)).all()
    ok = ~np.isnan(ref)
    assert (ours[ok] == ref[ok]).all()
    assert (np.signbit(ours[ok]) == np.signbit(ref[ok])).all()
    assert set(np.flatnonzero(np.isnan(ours))) == {0x7F, 0xFF}


def test_e4m3_closed_forms():
    d = lambda c: float(omx.e4m3_decode(np.array([c]))[0])
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert d(0x01) == 2.0 ** -9          # smallest subnormal: 2^-6 * 1/8
    assert d(0x07) == 7 * 2.0 ** -9
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x38) == 1.0                # E = 7: bias
    assert d(0x3C) == 1.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    pos = omx.e4m3_decode(np.arange(0x7F))
    assert (np.diff(pos) > 0).all()      # codes 0..0x7E are increasing


def test_e8m0_every_code_matches_torch_and_closed_forms():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = omx.e8m0_decode(codes), _torch_e8m0(codes)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert (ours[:255] == ref[:255]).all()
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127
    assert ours[128] == 2.0 and ours[126] == 0.5


def _brute_fwd_fraction(x8, xs, w8, ws, offsets):
    """Exact rationals: each code decoded by torch's cast, each scale 2^(s-127)."""
    xv = _torch_e4m3(x8); wv = _torch_e4m3(w8)
    M, K = x8.shape
    E, N, _ = w8.shape
    y = {}
    for e in range(E):
        for i in range(offsets[e], offsets[e + 1]):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    acc += (Fraction(xv[i, k]) * Fraction(2) ** (int(xs[i, k // 32]) - 127) *
                            Fraction(wv[e, n, k]) * Fraction(2) ** (int(ws[e, n, k // 32]) - 127))
                y[(i, n)] = acc
    return y


@pytest.mark.parametrize("seed", [0, 1])
def test_fwd_mx_brute_force_exact(seed):
    E, N, K = 3, 3, 96
    sizes = [3, 0, 4]
    offs = synth.offsets_from_sizes(sizes)
    M = int(offs[-1]) + 1                          # one row past the last expert
    x8 = synth.mx_e4m3_codes((M, K), 70, seed)
    w8 = synth.mx_e4m3_codes((E, N, K), 71, seed)
    xs = synth.mx_e8m0_codes((M, K // 32), 121, 4, 72, seed)
    ws = synth.mx_e8m0_codes((E, N, K // 32), 121, 4, 73, seed)
    y = omx.grouped_fwd_mx(x8, xs, w8, ws, offs)
    bf = _brute_fwd_fraction(x8, xs, w8, ws, offs)
    for (i, n), v in bf.items():
        assert y[i, n] == float(v)                 # exact: the fp64 sum does not round here
    assert np.isnan(y[M - 1]).all()                # row past offsets[E]


def test_fwd_mx_unit_scales_is_plain_grouped_fwd():
    E, N, K = 4, 16, 128
    offs = synth.offsets_from_sizes([5, 0, 9, 2])
    M = int(offs[-1])
    x8 = synth.mx_e4m3_codes((M, K), 80, 0)
    w8 = synth.mx_e4m3_codes((E, N, K), 81, 0)
    ones_x = np.full((M, K // 32), 127, np.uint8)
    ones_w = np.full((E, N, K // 32), 127, np.uint8)
    y = omx.grouped_fwd_mx(x8, ones_x, w8, ones_w, offs)
    ref = oracle.grouped_fwd(_torch_e4m3(x8), _torch_e4m3(w8), offs)
    np.testing.assert_array_equal(y, ref)


def test_fwd_mx_scale_shifts_are_exact_powers_of_two():
    E, N, K = 2, 8, 160                            # 5 blocks per row
    offs = synth.offsets_from_sizes([6, 5])
    M = int(offs[-1])
    x8 = synth.mx_e4m3_codes((M, K), 90, 0)
    w8 = synth.mx_e4m3_codes((E, N, K), 91, 0)
    xs = synth.mx_e8m0_codes((M, K // 32), 124, 3, 92, 0)
    ws = synth.mx_e8m0_codes((E, N, K // 32), 124, 3, 93, 0)
    y = omx.grouped_fwd_mx(x8, xs, w8, ws, offs)
    # every scale of row 4 up by 3: row 4 times 8, nothing else moves
    xs2 = xs.copy(); xs2[4] += 3
    y2 = omx.grouped_fwd_mx(x8, xs2, w8, ws, offs)
    np.testing.assert_array_equal(y2[4], 8.0 * y[4])
    np.testing.assert_array_equal(np.delete(y2, 4, 0), np.delete(y, 4, 0))
    # every scale of expert 1 down by 2: its rows times 1/4
    ws2 = ws.copy(); ws2[1] -= 2
    y3 = omx.grouped_fwd_mx(x8, xs, w8, ws2, offs)
    np.testing.assert_array_equal(y3[6:], 0.25 * y[6:])
    np.testing.assert_array_equal(y3[:6], y[:6])
    # one block (row 2, block 3) up by 1 adds exactly that block's contribution
    xs3 = xs.copy(); xs3[2, 3] += 1
    y4 = omx.grouped_fwd_mx(x8, xs3, w8, ws, offs)
    only = np.zeros_like(x8); only[2, 96:128] = x8[2, 96:128]
    part = omx.grouped_fwd_mx(only, xs, w8, ws, offs)
    np.testing.assert_allclose(y4[2] - y[2], part[2], rtol=1e-14, atol=0)
    assert np.abs(part[2]).max() > 0


def test_sample_fwd_mx_matches_full():
    E, N, K = 3, 24, 256
    offs = synth.offsets_from_sizes([10, 0, 13])
    M = int(offs[-1])
    x8 = synth.mx_e4m3_codes((M, K), 100, 0)
    w8 = synth.mx_e4m3_codes((E, N, K), 101, 0)
    xs = synth.mx_e8m0_codes((M, K // 32), 121, 5, 102, 0)
    ws = synth.mx_e8m0_codes((E, N, K // 32), 121, 5, 103, 0)
    y = omx.grouped_fwd_mx(x8, xs, w8, ws, offs)
    rows = np.array([0, 9, 10, 22]); cols = np.array([0, 23, 5, 11])
    v, s = omx.sample_fwd_mx(x8, xs, w8, ws, offs, rows, cols)
    np.testing.assert_array_equal(v, y[rows, cols])
    xv = omx.mx_dequant(x8, xs); wv = omx.mx_dequant(w8, ws)
    e = [0, 0, 2, 2]
    for j in range(4):
        assert s[j] == np.abs(xv[rows[j]] * wv[e[j], cols[j]]).sum()


@pytest.mark.parametrize("nb", [1, 3, 4, 5, 8])
def test_blocked_layout_index_by_index(nb):
    rows = 7
    s = synth.mx_e8m0_codes((2, rows, nb), 127, 100, 110, nb)
    out = omx.mx_scales_blocked(s)
    nt = (nb + 3) // 4
    assert out.shape == (2, nt, rows, 4)
    for b in range(2):
        for t in range(nt):
            for r in range(rows):
                for j in range(4):
                    want = s[b, r, 4 * t + j] if 4 * t + j < nb else 127
                    assert out[b, t, r, j] == want
    assert omx.blocked_bytes(rows, 32 * nb) == out[0].size


def test_mx_gate_accepts_rounding_and_rejects_block_mistakes():
    E, N, K = 1, 64, 2048
    M = 64
    offs = synth.offsets_from_sizes([M])
    x8 = synth.mx_e4m3_codes((M, K), 120, 0)
    w8 = synth.mx_e4m3_codes((E, N, K), 121, 0)
    # scales within a factor of 2 of each other, as block maxima of Gaussian
    # data are (with a wide spread most blocks are negligible next to the
    # few largest, and no tolerance that the matrix cores meet can see them)
    xs = synth.mx_e8m0_codes((M, K // 32), 121, 1, 122, 0)
    ws = synth.mx_e8m0_codes((E, N, K // 32), 121, 1, 123, 0)
    y = omx.grouped_fwd_mx(x8, xs, w8, ws, offs)
    xv = omx.mx_dequant(x8, xs); wv = omx.mx_dequant(w8, ws)
    S = np.abs(xv) @ np.abs(wv[0]).T
    good = oracle.f64_to_bf16_bits(y)
    assert oracle.check_bf16_mx(good, y, S).passed
    # within the floor: exact + 0.9 * 2^-12 S, rounded
    near = oracle.f64_to_bf16_bits(y + 0.9 * 2.0 ** -12 * S)
    assert oracle.check_bf16_mx(near, y, S).passed
    # a dropped 32-block
    x_drop = x8.copy(); x_drop[:, 640:672] = 0
    bad = oracle.f64_to_bf16_bits(omx.grouped_fwd_mx(x_drop, xs, w8, ws, offs))
    rep = oracle.check_bf16_mx(bad, y, S)
    assert not rep.passed and rep.fails > 0.8 * y.size
    # one block's scale off by one power of two
    xs_bad = xs.copy(); xs_bad[:, 7] += 1
    bad = oracle.f64_to_bf16_bits(omx.grouped_fwd_mx(x8, xs_bad, w8, ws, offs))
    rep = oracle.check_bf16_mx(bad, y, S)
    assert not rep.passed and rep.fails > 0.8 * y.size
    # scales read with the block index of the transposed layout
    ws_t = ws[:, :, ::-1].copy()
    bad = oracle.f64_to_bf16_bits(omx.grouped_fwd_mx(x8, xs, w8, ws_t, offs))
    assert oracle.check_bf16_mx(bad, y, S).fails > 0.9 * y.size


# ------------------------------------------------------------ MXFP8 wgrad --

def _wgrad_inputs(N, K, sizes, spread, seed, center=121):
    offs = synth.offsets_from_sizes(sizes)
    M = int(offs[-1])
    dyt8 = synth.mx_e4m3_codes((N, M), 130, seed)
    xt8 = synth.mx_e4m3_codes((K, M), 131, seed)
    dyts = synth.mx_e8m0_codes((N, M // 32), center, spread, 132, seed)
    xts = synth.mx_e8m0_codes((K, M // 32), center, spread, 133, seed)
    return offs, M, dyt8, dyts, xt8, xts


def test_wgrad_mx_brute_force_exact():
    N, K = 3, 2
    offs, M, dyt8, dyts, xt8, xts = _wgrad_inputs(N, K, [32, 0, 64], 4, 0)
    E = 3
    dw = omx.grouped_wgrad_mx(dyt8, dyts, xt8, xts, offs, E)
    dv, xv = _torch_e4m3(dyt8), _torch_e4m3(xt8)
    for e in range(E):
        for n in range(N):
            for k in range(K):
                acc = Fraction(0)
                for i in range(offs[e], offs[e + 1]):
                    acc += (Fraction(dv[n, i]) * Fraction(2) ** (int(dyts[n, i // 32]) - 127) *
                            Fraction(xv[k, i]) * Fraction(2) ** (int(xts[k, i // 32]) - 127))
                assert dw[e, n, k] == float(acc)
    assert (dw[1] == 0).all()
    prior = np.arange(E * N * K, dtype=np.float64).reshape(E, N, K)
    np.testing.assert_array_equal(omx.grouped_wgrad_mx(dyt8, dyts, xt8, xts, offs, E, prior),
                                  dw + prior)


def test_wgrad_mx_unit_scales_is_plain_wgrad_and_adjoint_of_fwd():
    N, K = 16, 24
    offs, M, dyt8, dyts, xt8, xts = _wgrad_inputs(N, K, [64, 0, 96, 32], 0, 1, center=127)
    E = 4
    dw = omx.grouped_wgrad_mx(dyt8, dyts, xt8, xts, offs, E)
    dy = _torch_e4m3(dyt8).T.copy(); x = _torch_e4m3(xt8).T.copy()
    np.testing.assert_array_equal(dw, oracle.grouped_wgrad(dy, x, offs, E))
    # with scales: sum_e <dW_e, W_e> = <dY, Y(X, W)> for any W (the forward's adjoint)
    offs, M, dyt8, dyts, xt8, xts = _wgrad_inputs(N, K, [64, 0, 96, 32], 3, 2)
    dw = omx.grouped_wgrad_mx(dyt8, dyts, xt8, xts, offs, E)
    dy = omx.mx_dequant(dyt8, dyts).T; x = omx.mx_dequant(xt8, xts).T
    w = np.random.default_rng(3).standard_normal((E, N, K))
    lhs = float((dw * w).sum())
    rhs = float((dy * oracle.grouped_fwd(x, w, offs)).sum())
    assert abs(lhs - rhs) <= 1e-12 * (np.abs(dw).sum() * np.abs(w).max())


def test_wgrad_mx_scale_shifts():
    N, K = 8, 12
    offs, M, dyt8, dyts, xt8, xts = _wgrad_inputs(N, K, [64, 96], 3, 4)
    E = 2
    dw = omx.grouped_wgrad_mx(dyt8, dyts, xt8, xts, offs, E)
    # all scales of X^T row 5 up by 2: column k = 5 of every expert times 4
    xts2 = xts.copy(); xts2[5] += 2
    dw2 = omx.grouped_wgrad_mx(dyt8, dyts, xt8, xts2, offs, E)
    np.testing.assert_array_equal(dw2[:, :, 5], 4.0 * dw[:, :, 5])
    np.testing.assert_array_equal(np.delete(dw2, 5, 2), np.delete(dw, 5, 2))
    # token block 3 (rows 96..127, expert 1) of every dY^T row down by 1: expert 0 unchanged
    dyts2 = dyts.copy(); dyts2[:, 3] -= 1
    dw3 = omx.grouped_wgrad_mx(dyt8, dyts2, xt8, xts, offs, E)
    np.testing.assert_array_equal(dw3[0], dw[0])
    only = np.zeros_like(dyt8); only[:, 96:128] = dyt8[:, 96:128]
    part = omx.grouped_wgrad_mx(only, dyts, xt8, xts, offs, E)
    np.testing.assert_allclose(dw[1] - dw3[1], 0.5 * part[1], rtol=1e-13, atol=0)


def test_sample_wgrad_mx_and_gate():
    N, K = 32, 40
    offs, M, dyt8, dyts, xt8, xts = _wgrad_inputs(N, K, [128, 0, 256], 1, 5)
    E = 3
    dw = omx.grouped_wgrad_mx(dyt8, dyts, xt8, xts, offs, E)
    es, ns, ks = np.array([0, 1, 2, 2]), np.array([0, 3, 31, 7]), np.array([39, 1, 0, 20])
    v, s = omx.sample_wgrad_mx(dyt8, dyts, xt8, xts, offs, es, ns, ks)
    np.testing.assert_array_equal(v, dw[es, ns, ks])
    assert s[1] == 0 and v[1] == 0
    mag = omx.grouped_wgrad_mx(dyt8, dyts, xt8, xts, offs, E) * 0
    dyv, xv = omx.mx_dequant(dyt8, dyts), omx.mx_dequant(xt8, xts)
    for e in range(E):
        lo, hi = offs[e], offs[e + 1]
        mag[e] = np.abs(dyv[:, lo:hi]) @ np.abs(xv[:, lo:hi]).T
    k_red = np.maximum(np.diff(offs), 1)[:, None, None]
    empty = np.broadcast_to((np.diff(offs) == 0)[:, None, None], dw.shape)
    assert oracle.check_fp32_mx(dw.astype(np.float32), dw, mag, k_red, empty_mask=empty).passed
    # a dropped 32-token block of expert 2 and a wrong expert fail
    d2 = dyt8.copy(); d2[:, 160:192] = 0
    bad = omx.grouped_wgrad_mx(d2, dyts, xt8, xts, offs, E)
    assert oracle.check_fp32_mx(bad, dw, mag, k_red, empty_mask=empty).fails > 0.8 * dw[2].size
    swapped = dw[[2, 1, 0]]
    assert not oracle.check_fp32_mx(swapped, dw, mag, k_red, empty_mask=empty).passed


def test_small_integer_inputs_decode_to_integers_and_sum_exactly():
    """The exact-result GPU cases rest on two facts checked here: the small
    integer codes decode (torch's float8 cast) to every integer in [-3, 3] and
    nothing else, and with scales constant along the reduction the oracle's
    forward equals integer brute force times the two scales."""
    c = synth.mx_small_int_codes((4096,), 3, 1)
    v = _torch_e4m3(c)
    assert sorted(set(v.tolist())) == [-3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0]
    s = synth.mx_e8m0_row_codes(9, 5, 127, 6, 3, 2)
    assert (s == s[:, :1]).all() and s.min() >= 121 and s.max() <= 133
    pc = synth.mx_e8m0_pair_codes((64, 8), 127, 3, 7)
    assert set(np.unique(pc).tolist()) == {127, 128}
    assert sorted(set(_torch_e8m0(pc).ravel().tolist())) == [1.0, 2.0]
    off = synth.offsets_from_sizes([3, 0, 2])
    M, N, K = 5, 3, 64
    x8 = synth.mx_small_int_codes((M, K), 3, 3)
    w8 = synth.mx_small_int_codes((3, N, K), 3, 4)
    xs = synth.mx_e8m0_row_codes(M, K // 32, 127, 6, 3, 5)
    ws = synth.mx_e8m0_row_codes(3 * N, K // 32, 127, 6, 3, 6).reshape(3, N, K // 32)
    got = oracle.grouped_fwd_mx(x8, xs, w8, ws, off)
    xi = _torch_e4m3(x8).astype(np.int64).tolist()
    wi = _torch_e4m3(w8).astype(np.int64).tolist()
    for i in range(M):
        e = int(np.searchsorted(off, i, side="right")) - 1
        for n in range(N):
            dot = sum(xi[i][k] * wi[e][n][k] for k in range(K))
            want = Fraction(dot) * Fraction(2) ** (int(xs[i, 0]) - 127) \
                * Fraction(2) ** (int(ws[e, n, 0]) - 127)
            assert Fraction(got[i, n]) == want
