"""Helpers of the GPU parity tests: move seeded bit patterns to the device and
back, run the oracle on the same bits, and apply the parity gates."""
from __future__ import annotations

import numpy as np
import torch

from oracle import (bf16_bits_to_f64, check_bf16, check_fp32, grouped_dgrad, grouped_fwd,
                    grouped_wgrad, sample_dgrad, sample_fwd, sample_wgrad)


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dev_i32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def sentinel_bf16(shape, device="cuda") -> torch.Tensor:
    """Output buffer pre-filled with a bf16 NaN pattern (0x7FAB) so that rows
    the library must not touch can be recognised afterwards."""
    t = torch.full(shape, 0x7FAB, dtype=torch.int16, device=device)
    return t.view(torch.bfloat16)


SENTINEL = 0x7FAB


def gate_fwd_full(xb, wb, off, got_bits):
    x, w = bf16_bits_to_f64(xb), bf16_bits_to_f64(wb)
    o = int(off[-1])
    exact = grouped_fwd(x, w, off)[:o]
    mag = grouped_fwd(np.abs(x), np.abs(w), off)[:o]
    return check_bf16(got_bits[:o], exact, mag, x.shape[1])


def gate_dgrad_full(dyb, wb, off, got_bits):
    dy, w = bf16_bits_to_f64(dyb), bf16_bits_to_f64(wb)
    o = int(off[-1])
    exact = grouped_dgrad(dy, w, off)[:o]
    mag = grouped_dgrad(np.abs(dy), np.abs(w), off)[:o]
    return check_bf16(got_bits[:o], exact, mag, dy.shape[1])


def gate_wgrad_full(dyb, xb, off, got, prior=None):
    dy, x = bf16_bits_to_f64(dyb), bf16_bits_to_f64(xb)
    E = len(off) - 1
    exact = grouped_wgrad(dy, x, off, E, prior=prior)
    mag = grouped_wgrad(np.abs(dy), np.abs(x), off, E)
    if prior is not None:
        mag = mag + np.abs(prior)
    sizes = np.diff(np.asarray(off, np.int64))
    k_red = np.broadcast_to(np.maximum(sizes, 1)[:, None, None], exact.shape)
    empty = np.broadcast_to((sizes == 0)[:, None, None], exact.shape)
    return check_fp32(got, exact, mag, k_red,
                      expert_slices=[(e,) for e in range(E) if sizes[e] > 0],
                      empty_mask=empty, empty_expect=(0.0 if prior is None else prior))


def sample_positions(rng, off, ncols, S):
    """S random (row, col) positions among the owned rows."""
    o = int(off[-1])
    rows = rng.integers(0, o, S)
    cols = rng.integers(0, ncols, S)
    return rows, cols


def gate_fwd_sampled(xb, wb, off, got_bits, S=4096, seed=0):
    rng = np.random.default_rng(seed)
    rows, cols = sample_positions(rng, off, wb.shape[1], S)
    exact, mag = sample_fwd(xb, wb, off, rows, cols)
    return check_bf16(got_bits[rows, cols], exact, mag, xb.shape[1])


def gate_dgrad_sampled(dyb, wb, off, got_bits, S=4096, seed=0):
    rng = np.random.default_rng(seed)
    rows, cols = sample_positions(rng, off, wb.shape[2], S)
    exact, mag = sample_dgrad(dyb, wb, off, rows, cols)
    return check_bf16(got_bits[rows, cols], exact, mag, dyb.shape[1])


def gate_wgrad_sampled(dyb, xb, off, got, S=2048, seed=0):
    """Sampled elements of every expert (S spread over experts, at least 16
    each), relative Frobenius per expert over its samples."""
    rng = np.random.default_rng(seed)
    E = len(off) - 1
    N, K = dyb.shape[1], xb.shape[1]
    per = max(16, S // E)
    es = np.repeat(np.arange(E), per)
    ns = rng.integers(0, N, es.size)
    ks = rng.integers(0, K, es.size)
    exact, mag = sample_wgrad(dyb, xb, off, es, ns, ks)
    g = got[es, ns, ks]
    sizes = np.diff(np.asarray(off, np.int64))
    k_red = np.maximum(sizes[es], 1)
    empty = sizes[es] == 0
    slices = [es == e for e in range(E) if sizes[e] > 0]
    return check_fp32(g, exact, mag, k_red, expert_slices=slices, empty_mask=empty)


# ------------------------------------------------ whole tensors, by expert --
#
# At the benchmark sizes every output element is checked, one expert at a
# time so that host memory stays bounded: the oracle runs on the expert's own
# rows (a one-expert problem with offsets [0, m_e]), the gate on that block,
# and the reports are merged.  Beside the gate, elements whose fp32 summation
# floor 2^-24 sqrt(K_red) sum|a b| is at most 1/8 of a bf16 ulp of the
# rounded result -- elements that do not cancel -- must meet the strict
# one-ulp gate: `nc_strict_fails` counts those that do not.

def _merge_bf16(reps, nc_fails):
    from oracle.gate import GateReport
    n = sum(r.n for r in reps)
    fails = sum(r.fails for r in reps)
    strict = sum(r.strict_fails for r in reps)
    worst = next((r.worst for r in reps if r.fails), "")
    rep = GateReport(n, fails == 0, fails, strict, 0.0, worst)
    rep.nc_strict_fails = nc_fails
    return rep


def _nc_strict(got_bits, exact, mag, k_red):
    from oracle.bf16 import bf16_ulp, f64_round_bf16
    b = f64_round_bf16(exact)
    ulp = bf16_ulp(b)
    nc = 2.0 ** -24 * np.sqrt(k_red) * mag <= ulp / 8
    g = bf16_bits_to_f64(got_bits)
    return int((nc & (np.abs(g - b) > ulp)).sum())


def _mgrouped_by_expert(ab, wb, off, got_bits, op):
    off = np.asarray(off, np.int64)
    red = ab.shape[1]
    reps, nc = [], 0
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        a = bf16_bits_to_f64(ab[lo:hi])
        w = bf16_bits_to_f64(wb[e:e + 1])
        o1 = np.array([0, hi - lo], np.int64)
        exact = op(a, w, o1)
        mag = op(np.abs(a), np.abs(w), o1)
        reps.append(check_bf16(got_bits[lo:hi], exact, mag, red))
        nc += _nc_strict(got_bits[lo:hi], exact, mag, red)
    return _merge_bf16(reps, nc)


def gate_fwd_experts(xb, wb, off, got_bits):
    """Every owned element of Y = X W_e^T, expert by expert."""
    return _mgrouped_by_expert(xb, wb, off, got_bits, grouped_fwd)


def gate_dgrad_experts(dyb, wb, off, got_bits):
    """Every owned element of dX = dY W_e, expert by expert."""
    return _mgrouped_by_expert(dyb, wb, off, got_bits, grouped_dgrad)


def gate_wgrad_experts(dyb, xb, off, got):
    """Every element of dW [E, N, K] (fp32), expert by expert: the element
    bound and the per-expert relative Frobenius error of check_fp32, the
    whole-tensor relative Frobenius error from the accumulated squares, and
    empty experts exactly zero."""
    from oracle.gate import GateReport
    off = np.asarray(off, np.int64)
    E = len(off) - 1
    fails, worst, mx = 0, "", 0.0
    d2 = n2 = 0.0
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        g = np.asarray(got[e], np.float64)
        if hi == lo:
            bad = int((g != 0).sum())
            fails += bad
            if bad and not worst:
                worst = f"empty expert {e} holds {bad} nonzero elements"
            continue
        dy, x = bf16_bits_to_f64(dyb[lo:hi]), bf16_bits_to_f64(xb[lo:hi])
        o1 = np.array([0, hi - lo], np.int64)
        exact = grouped_wgrad(dy, x, o1, 1)[0]
        mag = grouped_wgrad(np.abs(dy), np.abs(x), o1, 1)[0]
        r = check_fp32(g, exact, mag, hi - lo)
        fails += r.fails
        if r.fails and not worst:
            worst = f"expert {e}: {r.worst}"
        mx = max(mx, r.max_rel_frob)
        d2 += float(np.sum((g - exact) ** 2))
        n2 += float(np.sum(exact ** 2))
    whole = (d2 ** 0.5) / (n2 ** 0.5) if n2 > 0 else d2 ** 0.5
    mx = max(mx, whole)
    return GateReport(int(np.prod(got.shape)), fails == 0 and mx <= 1e-4, fails, 0, mx, worst)
