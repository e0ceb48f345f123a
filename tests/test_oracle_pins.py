"""Pins of the oracle to things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle -- a transposed
operand, a wrong expert boundary, a dropped term, a double rounding in the
codec -- fails at least one of them:
  * exact rational brute force (fractions.Fraction triple loops) on tiny
    inputs, including bit-exact bf16 rounding done on rationals;
  * closed forms on one-hot inputs (Y picks a weight entry, dW counts pairs);
  * a hand-worked example in tests/golden/worked_e3.json;
  * the adjoint identity <dY, X W^T> = <dX, X> = sum_e <dW_e, W_e>, which
    ties the three contractions together (backward = dgrad + wgrad, DeepGEMM
    issue #10);
  * inserting an empty group changes nothing;
  * exhaustive and tie-case checks of the bf16 codec, and agreement with
    torch's own float32 -> bfloat16 rounding on float32-representable values;
  * for the gate-up forward with SwiGLU on gathered rows: scalar brute force,
    one-hot closed forms (swapping the gate and up halves must change the
    result), gather-as-permutation identities, sampler/gate consistency.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (bf16_bits_to_f64, bf16_ulp, f64_to_bf16_bits, grouped_dgrad,
                    grouped_fwd, grouped_wgrad, sample_dgrad, sample_fwd, sample_wgrad)
from oracle.bf16 import f64_round_bf16
from workloads import normal_bf16_bits, offsets_from_sizes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- rationals --

def frac_round_bf16(v: Fraction) -> Fraction:
    """Exact RNE of a rational to bf16 (normal and subnormal range), on
    Fractions only: independent of the oracle's float64 codec."""
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2; e += 1
    while a < 1:
        a *= 2; e -= 1
    # |v| = a * 2^e with 1 <= a < 2; bf16 spacing 2^(e-7), floored at 2^-133
    qexp = max(e, -126) - 7
    q = abs(v) / (Fraction(2) ** qexp)
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * Fraction(2) ** qexp


def frac_of(bits):
    return [[Fraction(float(x)) for x in row] for row in bf16_bits_to_f64(bits)]


def brute(xb, wb, dyb, sizes):
    """Triple loops over Fractions: Y, dX, dW exactly."""
    off = [0]
    for s in sizes:
        off.append(off[-1] + s)
    X = frac_of(xb)
    W = [frac_of(wb[e]) for e in range(len(sizes))]
    DY = frac_of(dyb)
    M, K = len(X), len(X[0])
    N = len(W[0])
    Y, DX = {}, {}
    DW = [[[Fraction(0)] * K for _ in range(N)] for _ in sizes]
    for e in range(len(sizes)):
        for i in range(off[e], off[e + 1]):
            for n in range(N):
                Y[i, n] = sum((X[i][k] * W[e][n][k] for k in range(K)), Fraction(0))
            for k in range(K):
                DX[i, k] = sum((DY[i][n] * W[e][n][k] for n in range(N)), Fraction(0))
            for n in range(N):
                for k in range(K):
                    DW[e][n][k] += DY[i][n] * X[i][k]
    return off, Y, DX, DW


@pytest.mark.parametrize("sizes,K,N,seed", [
    ([3, 0, 2], 5, 4, 11),
    ([1, 4], 8, 8, 12),
    ([0, 2, 1, 0, 3], 7, 3, 13),
    ([6], 8, 5, 14),
])
def test_brute_force_exact(sizes, K, N, seed):
    E, M = len(sizes), sum(sizes) + 1          # one trailing row owned by no expert
    xb = normal_bf16_bits((M, K), K ** -0.5, 900, seed, 1)
    wb = normal_bf16_bits((E, N, K), K ** -0.5, 900, seed, 2)
    dyb = normal_bf16_bits((M, N), 1.0, 900, seed, 3)
    off, Y, DX, DW = brute(xb, wb, dyb, sizes)
    x, w, dy = bf16_bits_to_f64(xb), bf16_bits_to_f64(wb), bf16_bits_to_f64(dyb)
    y = grouped_fwd(x, w, off)
    dx = grouped_dgrad(dy, w, off)
    dw = grouped_wgrad(dy, x, off, E)
    owned = off[-1]
    # bf16 x bf16 products are exact in fp64 and these short sums are too
    for (i, n), v in Y.items():
        assert y[i, n] == float(v)
        assert f64_to_bf16_bits(np.array(y[i, n])) == f64_to_bf16_bits(np.array(float(frac_round_bf16(v))))
    for (i, k), v in DX.items():
        assert dx[i, k] == float(v)
        assert f64_round_bf16(np.array(dx[i, k])) == float(frac_round_bf16(v))
    for e in range(E):
        assert np.array_equal(dw[e], np.array([[float(v) for v in r] for r in DW[e]]))
    assert np.isnan(y[owned:]).all() and np.isnan(dx[owned:]).all()
    # sampled element-wise forms agree with the brute force too
    rows = np.arange(owned)
    if owned:
        cols = rows % N
        v, _ = sample_fwd(xb, wb, off, rows, cols)
        assert np.array_equal(v, [float(Y[i, c]) for i, c in zip(rows, cols)])
        cols = rows % K
        v, _ = sample_dgrad(dyb, wb, off, rows, cols)
        assert np.array_equal(v, [float(DX[i, c]) for i, c in zip(rows, cols)])
    es = np.arange(E); ns = es % N; ks = (es * 3) % K
    v, _ = sample_wgrad(dyb, xb, off, es, ns, ks)
    assert np.array_equal(v, [float(DW[e][n][k]) for e, n, k in zip(es, ns, ks)])


# --------------------------------------------------------------- one-hot ----

def test_one_hot_closed_forms():
    """X one-hot at column p_i -> Y[i, n] = W[e(i), n, p_i];
    dY one-hot at q_i -> dX[i, k] = W[e(i), q_i, k];
    both one-hot -> dW[e, n, k] = #{i in e : q_i = n, p_i = k}."""
    rng = np.random.default_rng(5)
    sizes = [5, 0, 7, 3]
    E, K, N = 4, 6, 5
    off = offsets_from_sizes(sizes)
    M = off[-1]
    p = rng.integers(0, K, M); q = rng.integers(0, N, M)
    x = np.zeros((M, K)); x[np.arange(M), p] = 1.0
    dy = np.zeros((M, N)); dy[np.arange(M), q] = 1.0
    w = rng.integers(-8, 9, (E, N, K)).astype(np.float64)
    e_of = np.repeat(np.arange(E), sizes)
    y = grouped_fwd(x, w, off)
    dx = grouped_dgrad(dy, w, off)
    dw = grouped_wgrad(dy, x, off, E)
    for i in range(M):
        assert np.array_equal(y[i], w[e_of[i], :, p[i]])
        assert np.array_equal(dx[i], w[e_of[i], q[i], :])
    cnt = np.zeros((E, N, K))
    for i in range(M):
        cnt[e_of[i], q[i], p[i]] += 1
    assert np.array_equal(dw, cnt)


def test_hand_worked_golden():
    g = json.load(open(os.path.join(GOLDEN, "worked_e3.json")))
    x, w, dy = (np.array(g[k], dtype=np.float64) for k in ("x", "w", "dy"))
    off = g["offsets"]
    y = grouped_fwd(x, w, off)
    dx = grouped_dgrad(dy, w, off)
    dw = grouped_wgrad(dy, x, off, g["E"])
    owned = off[-1]
    assert np.array_equal(y[:owned], np.array(g["y_rows_owned"], float))
    assert np.array_equal(dx[:owned], np.array(g["dx_rows_owned"], float))
    assert np.isnan(y[owned:]).all() and np.isnan(dx[owned:]).all()
    assert np.array_equal(dw, np.array(g["dw"], float))
    adj = (dy[:owned] * y[:owned]).sum()
    assert adj == g["adjoint"] == (dx[:owned] * x[:owned]).sum() == (dw * w).sum()


# -------------------------------------------------------------- invariants --

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_adjoint_identity(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 7))
    sizes = rng.integers(0, 40, E); sizes[rng.integers(0, E)] = 0
    K, N = int(rng.integers(1, 50)), int(rng.integers(1, 50))
    off = offsets_from_sizes(sizes)
    M = off[-1] + 3
    x = rng.standard_normal((M, K)); w = rng.standard_normal((E, N, K))
    dy = rng.standard_normal((M, N))
    o = off[-1]
    y = grouped_fwd(x, w, off)[:o]
    dx = grouped_dgrad(dy, w, off)[:o]
    dw = grouped_wgrad(dy, x, off, E)
    a = (dy[:o] * y).sum(); b = (dx * x[:o]).sum(); c = (dw * w).sum()
    scale = max(1.0, np.abs(dy[:o]).sum() * np.abs(x).max() * np.abs(w).max() * K)
    assert abs(a - b) <= 1e-12 * scale and abs(a - c) <= 1e-12 * scale


def test_empty_group_insertion_and_concatenation():
    rng = np.random.default_rng(7)
    sizes = [4, 9, 0, 6]
    E, K, N = 4, 12, 10
    off = offsets_from_sizes(sizes)
    M = off[-1]
    x = rng.standard_normal((M, K)); w = rng.standard_normal((E, N, K))
    dy = rng.standard_normal((M, N))
    y, dx, dw = grouped_fwd(x, w, off), grouped_dgrad(dy, w, off), grouped_wgrad(dy, x, off, E)
    for pos in range(E + 1):
        s2 = sizes[:pos] + [0] + sizes[pos:]
        w2 = np.concatenate([w[:pos], rng.standard_normal((1, N, K)), w[pos:]])
        o2 = offsets_from_sizes(s2)
        assert np.array_equal(grouped_fwd(x, w2, o2), y)
        assert np.array_equal(grouped_dgrad(dy, w2, o2), dx)
        dw2 = grouped_wgrad(dy, x, o2, E + 1)
        assert np.array_equal(np.delete(dw2, pos, axis=0), dw)
        assert (dw2[pos] == 0).all()
    # the grouped result is the row concatenation of E single-expert problems
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        sub = offsets_from_sizes([hi - lo])
        assert np.array_equal(grouped_fwd(x[lo:hi], w[e:e + 1], sub), y[lo:hi])
        assert np.array_equal(grouped_dgrad(dy[lo:hi], w[e:e + 1], sub), dx[lo:hi])
        assert np.array_equal(grouped_wgrad(dy[lo:hi], x[lo:hi], sub, 1)[0], dw[e])


def test_wgrad_accumulate_prior():
    rng = np.random.default_rng(8)
    off = offsets_from_sizes([3, 0, 2])
    x = rng.standard_normal((5, 4)); dy = rng.standard_normal((5, 3))
    prior = rng.standard_normal((3, 3, 4))
    dw = grouped_wgrad(dy, x, off, 3)
    dwp = grouped_wgrad(dy, x, off, 3, prior=prior)
    assert np.array_equal(dwp, dw + prior)
    assert np.array_equal(dwp[1], prior[1])


def test_bad_offsets_rejected():
    x = np.zeros((4, 2)); w = np.zeros((2, 3, 2))
    for off in ([1, 2, 4], [0, 3, 2], [0, 2, 5], [0, 4]):
        with pytest.raises(ValueError):
            grouped_fwd(x, w, off)


# ------------------------------------------------------------------- codec --

def test_codec_exhaustive_round_trip():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    back = f64_to_bf16_bits(v)
    nan = np.isnan(v)
    assert np.array_equal(back[~nan], bits[~nan])
    assert (back[nan] == 0x7FC0).all()


def test_codec_ties_to_even_everywhere():
    # every midpoint between consecutive positive finite bf16 values
    b = np.arange(0, 0x7F7F, dtype=np.uint32).astype(np.uint16)
    lo = bf16_bits_to_f64(b); hi = bf16_bits_to_f64(b + 1)
    mid = (lo + hi) / 2                     # exact in fp64
    r = f64_to_bf16_bits(mid)
    expect = np.where(b % 2 == 0, b, b + 1).astype(np.uint16)
    assert np.array_equal(r, expect)
    assert np.array_equal(f64_to_bf16_bits(-mid), expect | np.uint16(0x8000))
    # just off the midpoint goes to the nearer side
    eps = (hi - lo) * 2.0 ** -20
    assert np.array_equal(f64_to_bf16_bits(mid - eps), b)
    assert np.array_equal(f64_to_bf16_bits(mid + eps), (b + 1).astype(np.uint16))


def test_codec_hand_picked():
    cases = [
        (1.0 + 2.0 ** -8, 0x3F80),           # tie -> even (1.0)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),       # tie -> even (1 + 2^-6)
        (-(1.0 + 2.0 ** -8), 0xBF80),
        (2.0 ** -133, 0x0001),               # smallest subnormal
        (2.0 ** -134, 0x0000),               # tie between 0 and 2^-133 -> 0
        (3 * 2.0 ** -134, 0x0002),           # tie between 2^-133 and 2^-132 -> even
        (2.0 ** -126, 0x0080),               # smallest normal
        (float(np.ldexp(255.0, 120)), 0x7F7F),            # largest finite
        (float(np.ldexp(511.0, 119)), 0x7F80),            # its upper tie -> inf
        (float(np.ldexp(511.0, 119)) * (1 - 2.0 ** -40), 0x7F7F),
        (0.0, 0x0000), (-0.0, 0x8000),
        (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
    ]
    for v, bits in cases:
        assert int(f64_to_bf16_bits(np.array(v))) == bits, (v, hex(bits))
    assert int(f64_to_bf16_bits(np.array(np.nan))) == 0x7FC0
    assert bf16_ulp(np.array(1.0)) == 2.0 ** -7
    assert bf16_ulp(np.array(1.99)) == 2.0 ** -7
    assert bf16_ulp(np.array(2.0)) == 2.0 ** -6
    assert bf16_ulp(np.array(0.0)) == 2.0 ** -133
    assert bf16_ulp(np.array(2.0 ** -130)) == 2.0 ** -133


def test_codec_agrees_with_torch_on_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(1e3),
        (rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
    ])
    f = f[np.isfinite(f)]
    t = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_bits(f.astype(np.float64)), t)


def test_rational_rounding_matches_codec_on_random_values():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000))
    for x in v:
        assert float(frac_round_bf16(Fraction(float(x)))) == float(f64_round_bf16(np.array(x)))


# ------------------------------------------- gate-up forward with SwiGLU --

def brute_swiglu(x, gather, w13, offsets):
    """Scalar loops with math.exp: an implementation written apart from the
    oracle's (no matmul, no vector code), for tiny inputs."""
    import math
    E, N2, K = w13.shape
    I = N2 // 2
    M = len(gather) if gather is not None else x.shape[0]
    out = [[None] * I for _ in range(M)]
    for e in range(E):
        for i in range(int(offsets[e]), int(offsets[e + 1])):
            src = int(gather[i]) if gather is not None else i
            for j in range(I):
                g = 0.0
                u = 0.0
                for k in range(K):
                    g += float(x[src, k]) * float(w13[e, j, k])
                    u += float(x[src, k]) * float(w13[e, I + j, k])
                out[i][j] = g / (1.0 + math.exp(-g)) * u
    return out


@pytest.mark.parametrize("sizes,T,K,I,seed", [
    ([3, 0, 2], 7, 5, 4, 1),
    ([1, 4], 5, 8, 3, 2),
    ([0, 0, 6, 1], 9, 3, 2, 3),
])
def test_swiglu_brute_force(sizes, T, K, I, seed):
    from oracle import grouped_fwd_swiglu
    rng = np.random.default_rng(seed)
    E = len(sizes)
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + 2                       # two rows past the last offset
    x = bf16_bits_to_f64(normal_bf16_bits((T, K), 1.0, seed, 1))
    w13 = bf16_bits_to_f64(normal_bf16_bits((E, 2 * I, K), 1.0, seed, 2))
    gather = rng.integers(0, T, M)              # repeats allowed (top-k routing)
    h = grouped_fwd_swiglu(x, gather, w13, off)
    ref = brute_swiglu(x, gather, w13, off)
    for i in range(M):
        for j in range(I):
            if ref[i][j] is None:
                assert np.isnan(h[i, j])
            else:
                assert h[i, j] == pytest.approx(ref[i][j], rel=1e-12, abs=1e-14)


def test_swiglu_closed_forms_and_halves():
    """One-hot rows pick single weights: h = silu(a) b exactly as math gives
    it; swapping the two halves of w13 gives silu(b) a (a transposed or
    mixed-up half fails here); silu(0) = 0 and silu is odd-symmetric around
    the sigmoid: silu(t) - silu(-t) = t."""
    import math
    from oracle import grouped_fwd_swiglu
    K, I, E = 4, 3, 2
    x = np.eye(K)                               # token t is one-hot at k = t
    w13 = np.zeros((E, 2 * I, K))
    for e in range(E):
        for j in range(I):
            for k in range(K):
                w13[e, j, k] = 0.5 * (1 + e) + 0.25 * j - 0.75 * k      # w1
                w13[e, I + j, k] = 1.0 - 0.125 * (j + k) + e           # w3
    gather = np.array([3, 0, 2, 1, 1])
    off = np.array([0, 2, 5])
    h = grouped_fwd_swiglu(x, gather, w13, off)
    swapped = np.concatenate([w13[:, I:], w13[:, :I]], axis=1)
    hs = grouped_fwd_swiglu(x, gather, swapped, off)
    for i in range(5):
        e = 0 if i < 2 else 1
        k = int(gather[i])
        for j in range(I):
            a, b = w13[e, j, k], w13[e, I + j, k]
            assert h[i, j] == pytest.approx(a / (1 + math.exp(-a)) * b, rel=1e-15)
            assert hs[i, j] == pytest.approx(b / (1 + math.exp(-b)) * a, rel=1e-15)
    zero_gate = w13.copy(); zero_gate[:, :I] = 0.0
    assert (grouped_fwd_swiglu(x, gather, zero_gate, off) == 0.0).all()
    t = np.linspace(-30.0, 30.0, 61)
    from oracle.grouped_gemm import _silu
    assert np.allclose(_silu(t) - _silu(-t), t, rtol=0, atol=1e-12)


def test_swiglu_gather_is_a_row_permutation():
    """Gathering token rows equals grouping them first; reordering the tokens
    (and remapping the index) changes nothing."""
    from oracle import grouped_fwd_swiglu
    rng = np.random.default_rng(11)
    T, K, I = 13, 6, 5
    off = offsets_from_sizes([4, 0, 7])
    x = bf16_bits_to_f64(normal_bf16_bits((T, K), 1.0, 11, 1))
    w13 = bf16_bits_to_f64(normal_bf16_bits((3, 2 * I, K), 1.0, 11, 2))
    gather = rng.integers(0, T, int(off[-1]))
    h = grouped_fwd_swiglu(x, gather, w13, off)
    np.testing.assert_array_equal(h, grouped_fwd_swiglu(x[gather], None, w13, off))
    perm = rng.permutation(T)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(h, grouped_fwd_swiglu(x[perm], inv[gather], w13, off))


def test_swiglu_sampler_and_gate():
    """The one-element sampler agrees with the full oracle, and the gate
    accepts the correctly rounded result but rejects a wrong expert's and a
    dropped term's."""
    from oracle import check_bf16_swiglu, grouped_fwd_swiglu, sample_fwd_swiglu
    rng = np.random.default_rng(5)
    T, K, I = 40, 64, 24
    off = offsets_from_sizes([10, 0, 25, 5])
    xb = normal_bf16_bits((T, K), K ** -0.5, 5, 1)
    wb = normal_bf16_bits((4, 2 * I, K), K ** -0.5, 5, 2)
    x, w13 = bf16_bits_to_f64(xb), bf16_bits_to_f64(wb)
    gather = rng.integers(0, T, int(off[-1]))
    h = grouped_fwd_swiglu(x, gather, w13, off)
    rows = np.repeat(np.arange(int(off[-1])), I)
    cols = np.tile(np.arange(I), int(off[-1]))
    hs, g, u, sg, su = sample_fwd_swiglu(xb, gather, wb, off, rows, cols)
    np.testing.assert_allclose(hs, h[rows, cols], rtol=1e-13, atol=1e-15)
    good = f64_to_bf16_bits(h[rows, cols])
    assert check_bf16_swiglu(good, hs, g, u, sg, su, K).passed
    wrong_expert = grouped_fwd_swiglu(x, gather, w13[[1, 0, 3, 2]], off)
    assert not check_bf16_swiglu(f64_to_bf16_bits(wrong_expert[rows, cols]), hs, g, u, sg, su, K).passed
    w_drop = w13.copy(); w_drop[:, :, K - 1] = 0.0
    dropped = grouped_fwd_swiglu(x, gather, w_drop, off)
    assert not check_bf16_swiglu(f64_to_bf16_bits(dropped[rows, cols]), hs, g, u, sg, su, K).passed


# ------------------------------------------------ per-group descriptor list --

def test_list_brute_force_exact():
    """Exact rational triple loops on tiny groups of different shapes,
    including empty and zero-reduction groups."""
    from oracle import grouped_list
    shapes = [(3, 4, 5), (0, 2, 3), (2, 0, 4), (1, 3, 0), (4, 1, 2)]
    groups = []
    for g, (m, n, k) in enumerate(shapes):
        a = bf16_bits_to_f64(normal_bf16_bits((m, k), 1.0, 60, g, 1))
        b = bf16_bits_to_f64(normal_bf16_bits((n, k), 1.0, 60, g, 2))
        groups.append((a, b))
    out = grouped_list(groups)
    for (a, b), d, (m, n, k) in zip(groups, out, shapes):
        assert d.shape == (m, n)
        for i in range(m):
            for j in range(n):
                ex = sum((Fraction(float(a[i, t])) * Fraction(float(b[j, t])) for t in range(k)),
                         Fraction(0))
                assert Fraction(float(d[i, j])) == ex or abs(float(d[i, j]) - float(ex)) <= 1e-15 * max(1.0, abs(float(ex)))
                assert f64_round_bf16(np.array([float(ex)]))[0] == f64_round_bf16(np.array([d[i, j]]))[0]


def test_list_one_hot_and_flattened_lora():
    """One-hot rows of A pick columns of B (a transposed B fails); and a nested
    LoRA x experts product flattens into one list: for each (adapter l, expert
    e) group, D = X_e A_l^T matches the rows of X_e times the adapter computed
    one dot product at a time."""
    from oracle import grouped_list
    k = 5
    a = np.eye(k)[[4, 0, 2]]                            # rows pick k = 4, 0, 2
    b = np.arange(3 * k, dtype=np.float64).reshape(3, k)
    (d,) = grouped_list([(a, b)])
    np.testing.assert_array_equal(d, b[:, [4, 0, 2]].T)
    rng = np.random.default_rng(3)
    xs = [rng.standard_normal((m, 8)) for m in (3, 0, 5)]     # three experts
    ads = [rng.standard_normal((2, 8)) for _ in range(2)]     # two rank-2 adapters
    flat = [(x, ad) for ad in ads for x in xs]
    out = grouped_list(flat)
    for (x, ad), dd in zip(flat, out):
        for i in range(x.shape[0]):
            for r in range(2):
                assert dd[i, r] == pytest.approx(float(sum(x[i, t] * ad[r, t] for t in range(8))),
                                                 rel=1e-12, abs=1e-12)
