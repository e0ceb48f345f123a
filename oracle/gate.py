"""Parity gates (test infrastructure only).

bf16 outputs (fwd, dgrad).  The strict gate is: every element g within one
bf16 ulp of b = bf16_rne(exact).  An fp32-accumulating implementation cannot
meet that on every element: where the exact value is the small remainder of a
cancelling sum, one bf16 ulp of it is smaller than the rounding error any
fp32 summation of the terms carries.  So an element also passes when g is the
correctly rounded bf16 of *some* value within the fp32 summation error of the
exact result:

    |g - exact| <= ulp(g) / 2 + 2^-24 * sqrt(K_red) * S,   S = sum_k |a_k b_k|,

K_red being the reduction length.  2^-24 sqrt(K_red) S is the typical (random
walk) size of the error of K_red fp32 roundings of partial sums bounded by S;
it is far above what a sane kernel produces on non-cancelling elements, and
far below the error of a dropped term, a wrong index or a wrong expert.  The
strict-failure count is reported next to the pass/fail verdict.

bf16 outputs of the fused SwiGLU forward, h = silu(g) u.  Same strict gate;
the floor carries the fp32 summation error of g and of u through the
activation to first order, plus a few fp32 roundings of exp, divide and
multiply:

    |h_got - h| <= ulp(h_got) / 2 + |silu'(g) u| dg + |silu(g)| du + 2^-20 |h|,
    dg = 2^-24 sqrt(K) S_g,  du = 2^-24 sqrt(K) S_u,
    silu'(g) = s (1 + g (1 - s)),  s = 1 / (1 + exp(-g)).

bf16 outputs of the SwiGLU backward, dg = dh u silu'(g) and du = dh silu(g)
with dh an fp32-accumulated sum and g, u given: the same strict gate, the
floor carrying dh's summation error through the factor f (u silu'(g) or
silu(g)) plus a few fp32 roundings:

    |got - exact| <= ulp(got) / 2 + |f| 2^-24 sqrt(K) S + 2^-20 |exact|.

bf16 outputs of the MXFP8 forward.  Same strict gate; the floor is that of
the fp8 dot products of gfx950's scaled matrix-core instruction, which do not
sum in fp32: measured on random E4M3 operands with random E8M0 scales, one
64-deep instruction lands within 1.1e-4 (about 2^-13) of the sum of the
absolute scaled products, as if the products were aligned to the largest one
and kept to about 14 fractional bits.  The errors of successive instructions
add at most linearly, so with a factor of two in hand:

    |g - exact| <= ulp(g) / 2 + 2^-12 * S,   S = sum_k |a_k b_k|  (scaled values).

A 32-element block dropped, scaled by a wrong power of two or taken from a
wrong row moves an element by about sqrt(32) times a typical product: with
block scales within a factor of two of each other (block maxima of Gaussian
data) and K = 2048, some 20 times this floor.  A block far smaller than the
largest ones of its sum is below it, as it is below the matrix cores' own
precision.

fp32 outputs of the MXFP8 weight gradient.  The same matrix-core precision
floor, applied per element: |g - exact| <= 2^-12 S + 2^-24 (8 + 2 sqrt(K_red)) S;
no Frobenius bound (a floor of 2^-12 of S is far above 1e-4 of the result's
norm when K_red is large); empty experts exactly zero (or the prior).

fp32 outputs (wgrad).  Relative Frobenius error <= 1e-4, over the whole
tensor and per expert (a large expert would otherwise hide a wrong small
one); an empty expert's block must be exactly zero (or exactly the prior
contents when accumulating).  Additionally every element must satisfy
|g - exact| <= 2^-24 (8 + 2 sqrt(K_red)) S, which catches single bad
elements that a Frobenius norm would average away.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .bf16 import bf16_bits_to_f64, bf16_ulp, f64_round_bf16

U32 = 2.0 ** -24


@dataclasses.dataclass
class GateReport:
    n: int
    passed: bool
    fails: int
    strict_fails: int = 0
    max_rel_frob: float = 0.0
    worst: str = ""

    def __str__(self):
        return (f"n={self.n} passed={self.passed} fails={self.fails} "
                f"strict_fails={self.strict_fails} rel_frob={self.max_rel_frob:.3e} {self.worst}")


def check_bf16(got_bits: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray,
               k_red) -> GateReport:
    """Gate for bf16 outputs against the fp64 oracle value `exact`."""
    g = bf16_bits_to_f64(got_bits)
    exact = np.asarray(exact, np.float64)
    b = f64_round_bf16(exact)
    strict = np.abs(g - b) <= bf16_ulp(b)
    floor = np.abs(g - exact) <= 0.5 * bf16_ulp(g) + U32 * np.sqrt(k_red) * abs_sum
    ok = (strict | floor) & np.isfinite(g)
    fails = int((~ok).sum())
    worst = ""
    if fails:
        i = int(np.argmax(np.where(ok, -np.inf, np.abs(g - exact))))
        worst = f"worst@{i}: got={g.flat[i]!r} exact={exact.flat[i]!r}"
    return GateReport(int(g.size), fails == 0, fails, int((~strict).sum()), 0.0, worst)


def check_bf16_swiglu(got_bits: np.ndarray, h: np.ndarray, g: np.ndarray, u: np.ndarray,
                      sum_g: np.ndarray, sum_u: np.ndarray, k_red) -> GateReport:
    """Gate for the bf16 output of the fused SwiGLU forward (see the header)."""
    got = bf16_bits_to_f64(got_bits)
    h = np.asarray(h, np.float64); g = np.asarray(g, np.float64); u = np.asarray(u, np.float64)
    b = f64_round_bf16(h)
    strict = np.abs(got - b) <= bf16_ulp(b)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-g))
    dsilu = sg * (1.0 + g * (1.0 - sg))
    dg = U32 * np.sqrt(k_red) * sum_g
    du = U32 * np.sqrt(k_red) * sum_u
    bound = 0.5 * bf16_ulp(got) + np.abs(dsilu * u) * dg + np.abs(g * sg) * du + 2.0 ** -20 * np.abs(h)
    ok = (strict | (np.abs(got - h) <= bound)) & np.isfinite(got)
    fails = int((~ok).sum())
    worst = ""
    if fails:
        i = int(np.argmax(np.where(ok, -np.inf, np.abs(got - h))))
        worst = f"worst@{i}: got={got.flat[i]!r} exact={h.flat[i]!r}"
    return GateReport(int(got.size), fails == 0, fails, int((~strict).sum()), 0.0, worst)


def check_bf16_factor(got_bits: np.ndarray, exact: np.ndarray, factor: np.ndarray,
                      abs_sum: np.ndarray, k_red) -> GateReport:
    """Gate for bf16 outputs f * dh with dh an fp32 sum (see the header)."""
    got = bf16_bits_to_f64(got_bits)
    exact = np.asarray(exact, np.float64)
    b = f64_round_bf16(exact)
    strict = np.abs(got - b) <= bf16_ulp(b)
    bound = (0.5 * bf16_ulp(got) + np.abs(factor) * U32 * np.sqrt(k_red) * abs_sum
             + 2.0 ** -20 * np.abs(exact))
    ok = (strict | (np.abs(got - exact) <= bound)) & np.isfinite(got)
    fails = int((~ok).sum())
    worst = ""
    if fails:
        i = int(np.argmax(np.where(ok, -np.inf, np.abs(got - exact))))
        worst = f"worst@{i}: got={got.flat[i]!r} exact={exact.flat[i]!r}"
    return GateReport(int(got.size), fails == 0, fails, int((~strict).sum()), 0.0, worst)


MX_FLOOR = 2.0 ** -12


def check_bf16_mx(got_bits: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray) -> GateReport:
    """Gate for the bf16 output of the MXFP8 forward (see the header)."""
    g = bf16_bits_to_f64(got_bits)
    exact = np.asarray(exact, np.float64)
    b = f64_round_bf16(exact)
    strict = np.abs(g - b) <= bf16_ulp(b)
    floor = np.abs(g - exact) <= 0.5 * bf16_ulp(g) + MX_FLOOR * abs_sum
    ok = (strict | floor) & np.isfinite(g)
    fails = int((~ok).sum())
    worst = ""
    if fails:
        i = int(np.argmax(np.where(ok, -np.inf, np.abs(g - exact))))
        worst = f"worst@{i}: got={g.flat[i]!r} exact={exact.flat[i]!r}"
    return GateReport(int(g.size), fails == 0, fails, int((~strict).sum()), 0.0, worst)


def check_fp32_mx(got: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray, k_red,
                  empty_mask=None, empty_expect=None) -> GateReport:
    """Gate for the fp32 output of the MXFP8 weight gradient (see the header)."""
    got = np.asarray(got, np.float64)
    exact = np.asarray(exact, np.float64)
    bound = (MX_FLOOR + U32 * (8.0 + 2.0 * np.sqrt(k_red))) * abs_sum
    ok = (np.abs(got - exact) <= bound) & np.isfinite(got)
    fails = int((~ok).sum())
    worst = ""
    if fails:
        i = int(np.argmax(np.where(ok, -np.inf, np.abs(got - exact))))
        worst = f"worst@{i}: got={got.flat[i]!r} exact={exact.flat[i]!r}"
    passed = fails == 0
    if empty_mask is not None:
        exp = 0.0 if empty_expect is None else empty_expect
        bad = int((got[empty_mask] != np.broadcast_to(exp, got.shape)[empty_mask]).sum())
        fails += bad
        passed = passed and bad == 0
    return GateReport(int(got.size), passed, fails, 0, rel_frob(got, exact), worst)


def rel_frob(got: np.ndarray, exact: np.ndarray) -> float:
    d = np.linalg.norm((np.asarray(got, np.float64) - exact).ravel())
    n = np.linalg.norm(np.asarray(exact, np.float64).ravel())
    return float(d / n) if n > 0 else float(d)


def check_fp32(got: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray, k_red,
               expert_slices=None, empty_mask=None, empty_expect=None,
               frob_tol: float = 1e-4) -> GateReport:
    """Gate for fp32 outputs.

    expert_slices: list of index tuples selecting each expert's block (or of
    boolean masks over samples); empty_mask / empty_expect: elements that must
    equal `empty_expect` exactly (zero, or the prior contents)."""
    got = np.asarray(got, np.float64)
    exact = np.asarray(exact, np.float64)
    elem_ok = np.abs(got - exact) <= U32 * (8.0 + 2.0 * np.sqrt(k_red)) * abs_sum
    elem_ok &= np.isfinite(got)
    fails = int((~elem_ok).sum())
    worst = ""
    if fails:
        i = int(np.argmax(np.where(elem_ok, -np.inf, np.abs(got - exact))))
        worst = f"worst@{i}: got={got.flat[i]!r} exact={exact.flat[i]!r}"
    frobs = [rel_frob(got, exact)]
    for sl in (expert_slices or []):
        if np.linalg.norm(exact[sl].ravel()) > 0:
            frobs.append(rel_frob(got[sl], exact[sl]))
    mx = max(frobs)
    passed = fails == 0 and mx <= frob_tol
    if empty_mask is not None:
        exp = 0.0 if empty_expect is None else empty_expect
        bad = int((got[empty_mask] != np.broadcast_to(exp, got.shape)[empty_mask]).sum())
        fails += bad
        passed = passed and bad == 0
    return GateReport(int(got.size), passed, fails, 0, mx, worst)
