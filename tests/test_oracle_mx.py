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
