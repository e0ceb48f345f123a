"""The parity gate is fair, and the seeded inputs are what they claim (CPU).

Fair means: an honest fp32 accumulation of the same products (emulated here
on the CPU, in 16-wide partial sums like a matrix-core instruction) passes,
while planted mistakes -- a dropped 16-wide slice of the reduction, an
off-by-one expert boundary, a wrong expert's weights, one dropped token row
in wgrad -- fail.  The mistakes are planted in copies of the oracle's
results, on the CPU.
"""
import numpy as np
import pytest

from oracle import (bf16_bits_to_f64, check_bf16, check_fp32, f64_to_bf16_bits,
                    grouped_fwd, grouped_wgrad)
from workloads import (make_workload, normal_bf16_bits, offsets_from_sizes,
                       random_offsets, zipf_sizes)


def fp32_chunked(a, b, chunk=16):
    """C = A @ B^T with fp32 accumulation of exact-ish 16-wide partial sums."""
    acc = np.zeros((a.shape[0], b.shape[0]), np.float32)
    for k0 in range(0, a.shape[1], chunk):
        part = (a[:, k0:k0 + chunk] @ b[:, k0:k0 + chunk].T).astype(np.float32)
        acc = (acc + part).astype(np.float32)
    return acc.astype(np.float64)


def _problem(K, seed, sizes=(200, 0, 184, 128), N=96):
    off = offsets_from_sizes(list(sizes))
    M, E = int(off[-1]), len(sizes)
    x = bf16_bits_to_f64(normal_bf16_bits((M, K), K ** -0.5, 950, seed, 1))
    w = bf16_bits_to_f64(normal_bf16_bits((E, N, K), K ** -0.5, 950, seed, 2))
    return off, x, w


def _emulated_fwd(x, w, off, drop_chunk=None, shift=0, swap=False):
    y = np.zeros((x.shape[0], w.shape[1]))
    E = w.shape[0]
    for e in range(E):
        lo, hi = off[e] + (shift if e > 0 else 0), off[e + 1] + (shift if e + 1 < E else 0)
        lo, hi = max(lo, 0), min(hi, x.shape[0])
        if hi <= lo:
            continue
        we = w[(e + 1) % E] if (swap and e == E - 1) else w[e]
        a = x[lo:hi].copy()
        if drop_chunk is not None:
            a[:, drop_chunk * 16:(drop_chunk + 1) * 16] = 0
        y[lo:hi] = fp32_chunked(a, we)
    return y


@pytest.mark.parametrize("K", [256, 2048, 3072])
def test_fp32_emulation_passes_bf16_gate(K):
    off, x, w = _problem(K, K)
    exact = grouped_fwd(x, w, off)
    mag = grouped_fwd(np.abs(x), np.abs(w), off)
    got = f64_to_bf16_bits(_emulated_fwd(x, w, off))
    rep = check_bf16(got, exact, mag, K)
    assert rep.passed, str(rep)


@pytest.mark.parametrize("plant", ["drop_chunk", "boundary", "wrong_expert"])
def test_planted_mistakes_fail_bf16_gate(plant):
    K = 256
    off, x, w = _problem(K, 77)
    exact = grouped_fwd(x, w, off)
    mag = grouped_fwd(np.abs(x), np.abs(w), off)
    kw = {"drop_chunk": dict(drop_chunk=5), "boundary": dict(shift=1),
          "wrong_expert": dict(swap=True)}[plant]
    got = f64_to_bf16_bits(_emulated_fwd(x, w, off, **kw))
    rep = check_bf16(got, exact, mag, K)
    assert not rep.passed
    assert rep.fails > 50


def _wgrad_problem(seed):
    sizes = [300, 0, 17, 1, 120]
    off = offsets_from_sizes(sizes)
    M = int(off[-1])
    dy = bf16_bits_to_f64(normal_bf16_bits((M, 64), 1.0, 960, seed, 1))
    x = bf16_bits_to_f64(normal_bf16_bits((M, 80), 1.0, 960, seed, 2))
    return off, dy, x, len(sizes)


def _wgrad_fp32(dy, x, off, E, drop_row=None):
    dw = np.zeros((E, dy.shape[1], x.shape[1]))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        rows = [i for i in range(lo, hi) if i != drop_row]
        if rows:
            dw[e] = fp32_chunked(dy[rows].T.copy(), x[rows].T.copy())
    return dw


def _gate_wgrad(got, dy, x, off, E):
    exact = grouped_wgrad(dy, x, off, E)
    mag = grouped_wgrad(np.abs(dy), np.abs(x), off, E)
    sizes = np.diff(off)
    k_red = np.broadcast_to(np.maximum(sizes, 1)[:, None, None], exact.shape)
    empty = np.broadcast_to((sizes == 0)[:, None, None], exact.shape)
    return check_fp32(got, exact, mag, k_red, expert_slices=[(e,) for e in range(E)],
                      empty_mask=empty)


def test_fp32_emulation_passes_fp32_gate():
    off, dy, x, E = _wgrad_problem(1)
    rep = _gate_wgrad(_wgrad_fp32(dy, x, off, E), dy, x, off, E)
    assert rep.passed, str(rep)
    assert rep.max_rel_frob < 1e-6


def test_planted_mistakes_fail_fp32_gate():
    off, dy, x, E = _wgrad_problem(2)
    # one dropped token row in the 17-row expert (others are far larger)
    assert not _gate_wgrad(_wgrad_fp32(dy, x, off, E, drop_row=int(off[2]) + 3), dy, x, off, E).passed
    # an empty expert that is not exactly zero
    bad = _wgrad_fp32(dy, x, off, E); bad[1, 3, 4] = 1e-30
    assert not _gate_wgrad(bad, dy, x, off, E).passed
    # the 1-row expert's block taken from the wrong expert
    bad = _wgrad_fp32(dy, x, off, E); bad[3] = bad[2]
    assert not _gate_wgrad(bad, dy, x, off, E).passed


# ------------------------------------------------------------------ inputs --

def test_generators_are_deterministic():
    a = normal_bf16_bits((64, 33), 0.5, 1, 2, 3)
    b = normal_bf16_bits((64, 33), 0.5, 1, 2, 3)
    c = normal_bf16_bits((64, 33), 0.5, 1, 2, 4)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    v = bf16_bits_to_f64(normal_bf16_bits((200000,), 1.0, 9))
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01


def test_small_integer_operands_are_exact_and_their_sums_exact_in_fp32():
    """The exact-result GPU cases rest on these facts: the generator's bf16
    bits decode (torch's bf16 cast agrees) to every integer in [-3, 3], and a
    sum of R products of such values, |sum| <= 9 R, is exact in fp32 for the
    longest reduction those cases use (10804 tokens)."""
    import torch
    from workloads.synth import small_int_bf16_bits
    b = small_int_bf16_bits((4096,), 5, 6)
    v = bf16_bits_to_f64(b)
    assert sorted(set(v.tolist())) == [-3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0]
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(t, v)
    assert 9 * 10804 < 2 ** 24
    rng = np.random.default_rng(0)
    a = bf16_bits_to_f64(small_int_bf16_bits((10804,), 5, 7))
    c = bf16_bits_to_f64(small_int_bf16_bits((10804,), 5, 8))
    prods = (a * c)[rng.permutation(10804)]
    s32 = np.float32(0)
    for p in prods.astype(np.float32):
        s32 = np.float32(s32 + p)
    assert float(s32) == float(np.sum(a * c))


def test_workload_invariants():
    (tiny,) = make_workload(1)
    assert tiny.offsets.tolist() == [0, 200, 200, 384, 512]
    assert (tiny.E, tiny.N, tiny.K, tiny.M) == (4, 128, 256, 512)
    for cfg, g, m in ((2, 8, 4096), (3, 16, 2048)):
        (u,) = make_workload(cfg)
        assert u.offsets.tolist() == list(range(0, g * m + 1, m))
        assert (u.N, u.K) == (768, 2048)
    gate_up, down = make_workload(4)
    assert gate_up.offsets is down.offsets or np.array_equal(gate_up.offsets, down.offsets)
    assert (gate_up.N, gate_up.K, down.N, down.K) == (2560, 3072, 3072, 1280)
    assert abs(gate_up.rows - 32768) < 0.02 * 32768 and gate_up.E == 32
    gw13, gw2 = make_workload(5)
    s = gw13.sizes()
    assert s.sum() == 32768 and (s == 0).sum() == 4 and s.max() / s.sum() > 0.25
    assert sorted(s.tolist(), reverse=True)[:3] == [10804, 4703, 2891]
    assert (gw13.N, gw13.K, gw2.N, gw2.K) == (2560, 3072, 3072, 1280)


def test_zipf_and_random_offsets():
    s = zipf_sizes(1000, 10, 2, 1.2, seed=1)
    assert s.sum() == 1000 and (s == 0).sum() == 2
    o = random_offsets(9, 500, seed=3, special=[0, 1, 127, 128, 129])
    assert o[0] == 0 and o[-1] <= 500 and (np.diff(o) >= 0).all() and len(o) == 10
    assert sorted(np.diff(o).tolist())[:2] == [0, 1] or 0 in np.diff(o)


def test_lattice_operand_host_and_device_builders_agree():
    """The row-addressable operand for sizes past 4 GiB: the torch builder (run
    here on the CPU, in several row chunks) and the host view give the same
    values, rows and column slices alike, and every value is exact in bf16."""
    import torch
    from workloads.synth import LatticeMatrix, lattice_bf16, lattice_values
    M, K = 300, 40
    t = lattice_bf16(M, K, "cpu", chunk=64).float().numpy().astype(np.float64)
    h = LatticeMatrix(M, K)
    assert np.array_equal(t, h[np.arange(M)])
    assert np.array_equal(t[17:250, 9], h[17:250, 9])
    assert np.array_equal(t, lattice_values(np.arange(M)[:, None], np.arange(K)[None, :]))
    assert set(np.unique(t * 8).astype(int)) <= set(range(-8, 9))
    # neighbouring rows and columns differ (a misplaced read changes values)
    assert not np.array_equal(t[:-1], t[1:]) and not np.array_equal(t[:, :-1], t[:, 1:])


# ------------------------------------- whole-tensor gates, expert by expert --

def test_expert_gates_pass_fp32_emulation_and_catch_planted_mistakes():
    """The expert-by-expert whole-tensor gates (tests/parity.py) pass an fp32
    emulation with no strict failure on non-cancelling elements, and fail an
    element left at the output sentinel, one element 3 ulps off, and, for the
    fp32 weight gradient, a nonzero empty expert and one expert's block taken
    from another expert."""
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from parity import SENTINEL, gate_fwd_experts, gate_wgrad_experts
    from oracle.bf16 import bf16_ulp
    K = 512
    off, x, w = _problem(K, 77, sizes=(300, 0, 70, 257), N=136)
    xb = f64_to_bf16_bits(x)
    wb = f64_to_bf16_bits(w)
    got = f64_to_bf16_bits(_emulated_fwd(x, w, off))
    rep = gate_fwd_experts(xb, wb, off, got)
    assert rep.passed and rep.nc_strict_fails == 0, str(rep)
    bad = got.copy()
    bad[301, 5] = SENTINEL
    assert not gate_fwd_experts(xb, wb, off, bad).passed
    bad = got.copy()
    v = bf16_bits_to_f64(bad[[400]][:, [9]])
    bad[400, 9] = f64_to_bf16_bits(v + 3 * bf16_ulp(v))[0, 0]
    r = gate_fwd_experts(xb, wb, off, bad)
    assert not r.passed and r.nc_strict_fails == 1
    # fp32 weight gradient
    dy = bf16_bits_to_f64(normal_bf16_bits((int(off[-1]), 136), 1.0, 951, 1))
    dyb = f64_to_bf16_bits(dy)
    E = len(off) - 1
    dw = grouped_wgrad(dy, x, off, E).astype(np.float32)
    assert gate_wgrad_experts(dyb, xb, off, dw).passed
    b2 = dw.copy()
    b2[1, 3, 3] = 1e-30
    assert not gate_wgrad_experts(dyb, xb, off, b2).passed
    b3 = dw.copy()
    b3[2] = dw[3]
    assert not gate_wgrad_experts(dyb, xb, off, b3).passed
