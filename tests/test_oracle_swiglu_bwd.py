"""Pins of the SwiGLU backward through the down projection (CPU only).

The derivative is checked against central finite differences of silu(g) u
written with math.exp, the whole backward against the forward it
differentiates (a directional derivative of <dy, y(gu)>), and against a plain
loop on tiny inputs; the gate rejects swapped halves and a wrong expert.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle.bf16 import f64_to_bf16_bits


def _silu_u(g: float, u: float) -> float:
    return g / (1.0 + math.exp(-g)) * u


def test_derivative_matches_finite_differences():
    rng = np.random.default_rng(0)
    I = 16
    g = rng.standard_normal((3, I)) * 3.0
    u = rng.standard_normal((3, I))
    gu = np.concatenate([g, u], axis=1)
    # dh = 1 everywhere: N = 1, dy = 1, w2 = 1
    dy = np.ones((3, 1)); w2 = np.ones((1, 1, I))
    dgu, dh = oracle.grouped_dgrad_swiglu(dy, w2, gu, [0, 3])
    assert (dh == 1.0).all()
    eps = 1e-6
    for r in range(3):
        for j in range(I):
            fd_g = (_silu_u(g[r, j] + eps, u[r, j]) - _silu_u(g[r, j] - eps, u[r, j])) / (2 * eps)
            fd_u = (_silu_u(g[r, j], u[r, j] + eps) - _silu_u(g[r, j], u[r, j] - eps)) / (2 * eps)
            assert abs(dgu[r, j] - fd_g) <= 1e-7 * (1 + abs(fd_g))
            assert abs(dgu[r, I + j] - fd_u) <= 1e-7 * (1 + abs(fd_u))


def test_backward_is_the_derivative_of_the_forward():
    """<dgu, delta> = d/de <dy, Y(gu + e delta)> with Y = grouped_fwd(silu(g) u, W2)."""
    rng = np.random.default_rng(1)
    sizes = [5, 0, 7, 3]
    off = np.concatenate([[0], np.cumsum(sizes)])
    M, E, N, I = int(off[-1]), len(sizes), 6, 4
    dy = rng.standard_normal((M, N)); w2 = rng.standard_normal((E, N, I))
    gu = rng.standard_normal((M, 2 * I)); delta = rng.standard_normal((M, 2 * I))

    def loss(x):
        h = x[:, :I] / (1.0 + np.exp(-x[:, :I])) * x[:, I:]
        return float((dy * oracle.grouped_fwd(h, w2, off)).sum())

    eps = 1e-6
    fd = (loss(gu + eps * delta) - loss(gu - eps * delta)) / (2 * eps)
    dgu, _ = oracle.grouped_dgrad_swiglu(dy, w2, gu, off)
    assert abs(float((dgu * delta).sum()) - fd) <= 1e-6 * (1 + abs(fd))


def test_plain_loop_tiny():
    rng = np.random.default_rng(2)
    off = [0, 2, 2, 5]
    M, E, N, I = 5, 3, 3, 2
    dy = rng.standard_normal((M, N)); w2 = rng.standard_normal((E, N, I))
    gu = rng.standard_normal((M, 2 * I))
    dgu, dh = oracle.grouped_dgrad_swiglu(dy, w2, gu, off)
    for e in range(E):
        for i in range(off[e], off[e + 1]):
            for j in range(I):
                d = sum(dy[i, n] * w2[e, n, j] for n in range(N))
                g, u = gu[i, j], gu[i, I + j]
                s = 1.0 / (1.0 + math.exp(-g))
                assert math.isclose(dh[i, j], d, rel_tol=1e-13, abs_tol=1e-15)
                assert math.isclose(dgu[i, j], d * u * s * (1 + g * (1 - s)), rel_tol=1e-12, abs_tol=1e-14)
                assert math.isclose(dgu[i, I + j], d * g * s, rel_tol=1e-12, abs_tol=1e-14)


def test_sampler_and_gate():
    rng = np.random.default_rng(3)
    off = np.array([0, 40, 40, 100])
    M, E, N, I = 100, 3, 256, 32
    dy = rng.standard_normal((M, N)); w2 = rng.standard_normal((E, N, I)) / 16
    gu = rng.standard_normal((M, 2 * I)) * 2
    dgu, dh = oracle.grouped_dgrad_swiglu(dy, w2, gu, off)
    rows = np.array([0, 39, 40, 99]); cols = np.array([0, 31, 5, 17])
    dg, du, dhs, S = oracle.sample_dgrad_swiglu(dy, w2, gu, off, rows, cols)
    np.testing.assert_allclose(dg, dgu[rows, cols], rtol=1e-13)
    np.testing.assert_allclose(du, dgu[rows, I + cols], rtol=1e-13)
    np.testing.assert_allclose(dhs, dh[rows, cols], rtol=1e-13)
    g, u = gu[:, :I], gu[:, I:]
    s = 1 / (1 + np.exp(-g))
    fg, fu = u * s * (1 + g * (1 - s)), g * s
    absd = oracle.grouped_dgrad(np.abs(dy), np.abs(w2), off)
    fac = np.concatenate([fg, fu], axis=1)
    S2 = np.concatenate([absd, absd], axis=1)
    good = f64_to_bf16_bits(dgu)
    assert oracle.check_bf16_factor(good, dgu, fac, S2, N).passed
    swapped = f64_to_bf16_bits(np.concatenate([dgu[:, I:], dgu[:, :I]], axis=1))
    assert not oracle.check_bf16_factor(swapped, dgu, fac, S2, N).passed
    wrong = oracle.grouped_dgrad_swiglu(dy, w2[[2, 1, 0]], gu, off)[0]
    assert oracle.check_bf16_factor(f64_to_bf16_bits(wrong), dgu, fac, S2, N).fails > 0.8 * dgu[:40].size


# ---------------------------------------------------------------- combine --

def _router_maps(T, k, M_rows, seed):
    """A gather index (row -> token) with k rows per token, and its inverse."""
    rng = np.random.default_rng(seed)
    gather = np.repeat(np.arange(T), k)
    perm = rng.permutation(T * k)[:M_rows]
    gather = gather[perm]
    token_rows = -np.ones((T, k), np.int64)
    fill = np.zeros(T, np.int64)
    for i, t in enumerate(gather):
        token_rows[t, fill[t]] = i
        fill[t] += 1
    return gather, token_rows


def test_combine_is_the_adjoint_of_the_gather():
    """<combine(R), X> = <R, X[gather]>: the combine is the backward of the gather."""
    rng = np.random.default_rng(10)
    T, k, D = 50, 4, 24
    gather, token_rows = _router_maps(T, k, 170, 11)      # some tokens keep fewer than k rows
    R = rng.standard_normal((len(gather), D))
    X = rng.standard_normal((T, D))
    lhs = float((oracle.moe_combine(R, token_rows) * X).sum())
    rhs = float((R * X[gather]).sum())
    assert abs(lhs - rhs) <= 1e-12 * np.abs(R).sum() * np.abs(X).max()


def test_combine_plain_loop_with_weights():
    rng = np.random.default_rng(12)
    T, k, D = 7, 3, 5
    gather, token_rows = _router_maps(T, k, 18, 13)
    R = rng.standard_normal((len(gather), D))
    w = rng.random((T, k))
    out = oracle.moe_combine(R, token_rows, w)
    for t in range(T):
        for d in range(D):
            ref = sum(w[t, j] * R[token_rows[t, j], d] for j in range(k) if token_rows[t, j] >= 0)
            assert math.isclose(out[t, d], ref, rel_tol=1e-13, abs_tol=1e-15)
