"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Every case calls the C ABI (through the thin binding) on seeded inputs and
compares with the oracle on the same bits:
  * bf16 outputs (fwd, dgrad): within one bf16 ulp of the oracle rounded to
    bf16, or consistent with fp32 accumulation on cancelling sums (the gate
    in oracle/gate.py);
  * fp32 outputs (wgrad): relative Frobenius <= 1e-4 per expert and overall,
    element-wise accumulation bound, empty experts exactly zero (or exactly
    the prior contents when accumulating).
Sizes span several 256-wide tiles with ragged tails; the benchmark
workloads are checked on every output element (expert by expert), the
operands past 4 GiB and the longest reductions on sampled elements.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_bf16_amd as mg
from parity import (SENTINEL, dev_bf16, dev_i32, gate_dgrad_experts, gate_dgrad_full,
                    gate_fwd_experts, gate_fwd_full, gate_wgrad_experts, gate_wgrad_full,
                    gate_wgrad_sampled, host_bits, sentinel_bf16)
from workloads import make_workload, normal_bf16_bits, offsets_from_sizes

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(sizes, N, K, seed, extra_rows=0, x_scale=None, w_scale=None):
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + extra_rows
    E = len(sizes)
    xs = K ** -0.5 if x_scale is None else x_scale
    ws = K ** -0.5 if w_scale is None else w_scale
    xb = normal_bf16_bits((M, K), xs, 7000, seed, 1)
    wb = normal_bf16_bits((E, N, K), ws, 7000, seed, 2)
    dyb = normal_bf16_bits((M, N), 1.0, 7000, seed, 3)
    return off, M, E, xb, wb, dyb


def _run_mgrouped(off, M, xb, wb, dyb, N, K, hint=0):
    x, w, dy, o = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb), dev_i32(off)
    y = mg.fwd(x, w, o, hint, out=sentinel_bf16((M, N)))
    dx = mg.dgrad(dy, w, o, hint, out=sentinel_bf16((M, K)))
    torch.cuda.synchronize()
    return host_bits(y), host_bits(dx)


def _check_untouched(bits, off):
    assert (bits[int(off[-1]):] == SENTINEL).all(), "rows past offsets[E] were written"


# --------------------------------------------------------------- tiny config --

def test_tiny_config_all_three():
    (wl,) = make_workload(1)
    _say("tiny", wl.offsets.tolist())
    xb, wb, dyb = wl.x_bits(), wl.w_bits(), wl.dy_bits()
    yb, dxb = _run_mgrouped(wl.offsets, wl.M, xb, wb, dyb, wl.N, wl.K)
    r = gate_fwd_full(xb, wb, wl.offsets, yb); assert r.passed, str(r)
    r = gate_dgrad_full(dyb, wb, wl.offsets, dxb); assert r.passed, str(r)
    dw = mg.wgrad(dev_bf16(dyb), dev_bf16(xb), dev_i32(wl.offsets))
    torch.cuda.synchronize()
    r = gate_wgrad_full(dyb, xb, wl.offsets, dw.cpu().numpy()); assert r.passed, str(r)
    assert (dw[1] == 0).all()


# --------------------------------------------------------------- fuzz cases --

MG_CASES = [
    # sizes, N, K, extra rows past offsets[E]
    ([256], 256, 256, 0),
    ([1, 255, 256, 257], 264, 136, 5),
    ([0, 513, 0, 1, 300], 520, 200, 17),
    ([700, 0, 0], 72, 1032, 3),
    ([3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14], 8, 8, 0),
    ([64] * 9, 768, 64, 0),
    # the largest expert count, mostly tiny and empty experts
    ([int(v) for v in np.random.default_rng(7).integers(0, 6, 1024)], 8, 16, 2),
]


@pytest.mark.parametrize("case", range(len(MG_CASES)))
def test_mgrouped_fuzz(case):
    sizes, N, K, extra = MG_CASES[case]
    _say("mgrouped", sizes, N, K, extra)
    off, M, E, xb, wb, dyb = _inputs(sizes, N, K, 100 + case, extra)
    yb, dxb = _run_mgrouped(off, M, xb, wb, dyb, N, K)
    r = gate_fwd_full(xb, wb, off, yb); assert r.passed, "fwd " + str(r)
    r = gate_dgrad_full(dyb, wb, off, dxb); assert r.passed, "dgrad " + str(r)
    _check_untouched(yb, off)
    _check_untouched(dxb, off)


WG_CASES = [
    ([300, 0, 17, 1, 120], 264, 136),
    ([64, 63, 65, 128, 0], 256, 256),
    ([1000], 8, 520),
    ([0, 0, 2], 136, 8),
    # many skewed experts, a few empty: chunks of a handful of tiles, ranked
    ([int(v) for v in np.random.default_rng(8).zipf(1.3, 40) % 700] + [0, 0], 520, 264),
    # 256 tiles per expert: every XCD chunk holds exactly one tile per workgroup
    ([70, 0, 5], 4096, 4096),
    # the largest expert count
    ([int(v) for v in np.random.default_rng(9).integers(0, 9, 1024)], 8, 24),
    # one expert much heavier than the rest: its tiles are split in two token
    # halves (odd stage count, ragged last stage, ragged N and K, empty experts)
    ([2017, 33, 65, 129, 0, 0, 0, 700], 1544, 776),
    ([2500, 1, 0, 300, 0, 77, 1030, 5], 264, 1032),
    # near-uniform long experts whose tiles fill most but not all workgroups
    # (ragged N, K and token counts)
    ([3000, 2900, 3100, 2990, 3050, 2950, 3011, 2987], 760, 2000),
    ([2000 + 7 * i for i in range(17)], 256, 2048),
    # equal experts, E a multiple of 8: every XCD takes whole experts
    ([300] * 8, 264, 136),
    ([130] * 16, 520, 200),
    # ... and with one long tile per expert: each XCD's tile is split in two halves
    ([2000] * 8, 256, 256),
]


@pytest.mark.parametrize("case", range(len(WG_CASES)))
@pytest.mark.parametrize("accumulate", [False, True])
def test_wgrad_fuzz(case, accumulate):
    sizes, N, K = WG_CASES[case]
    _say("wgrad", sizes, N, K, "accumulate" if accumulate else "")
    off, M, E, xb, wb, dyb = _inputs(sizes, N, K, 200 + case, extra_rows=9,
                                     x_scale=1.0, w_scale=1.0)
    prior = None
    out = None
    if accumulate:
        prior = np.random.default_rng(case).standard_normal((E, N, K)).astype(np.float32)
        out = torch.from_numpy(prior.copy()).cuda()
    dw = mg.wgrad(dev_bf16(dyb), dev_bf16(xb), dev_i32(off), out=out, accumulate=accumulate)
    torch.cuda.synchronize()
    r = gate_wgrad_full(dyb, xb, off, dw.cpu().numpy(),
                        prior=None if prior is None else prior.astype(np.float64))
    assert r.passed, str(r)


def test_wgrad_first_call_captured_on_fresh_stream():
    """kgemm_wgrad's first call on a new stream, made while that stream is
    being captured into a graph: the call allocates nothing and enqueues no
    memory operation (it runs without the token split, which would otherwise
    take this heavy expert's tiles), and every replay -- three, with eager
    work between them -- matches the oracle."""
    sizes, N, K = [2017, 33, 65, 129, 0, 0, 0, 700], 1544, 776
    off, M, E, xb, wb, dyb = _inputs(sizes, N, K, 1800, extra_rows=3, x_scale=1.0, w_scale=1.0)
    dy, x, o = dev_bf16(dyb), dev_bf16(xb), dev_i32(off)
    out = torch.full((E, N, K), float("nan"), device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    _say("wgrad captured on a fresh stream", sizes, N, K)
    with torch.cuda.graph(g, stream=s):
        mg.wgrad(dy, x, o, out=out)
    torch.cuda.synchronize()
    other = torch.empty((E, N, K), device="cuda")
    for rep in range(3):
        out.fill_(float("nan"))
        mg.wgrad(dy, x, o, out=other)               # eager, on the current stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        r = gate_wgrad_full(dyb, xb, off, out.cpu().numpy())
        _say("replay", rep, str(r))
        assert r.passed, f"replay {rep}: {r}"


def test_captured_backward_follows_offsets_changed_in_place():
    """A graph of one forward, input gradient and weight gradient, captured
    once on a stream that already has its weight-gradient workspace (the
    captured weight gradient still runs without the token split), replayed
    after each of three routings has been written into the same device
    offsets array, with eager launches between the replays: the device-side
    scheduler reads the offsets at every launch, so each replay
    must match the oracle for the routing it finds, with no re-capture and no
    host synchronisation on the routing.  The routings keep the row total
    and include one that puts every row on a single expert."""
    N, K = 776, 1032
    routings = [[700, 0, 1300, 45, 2100, 256], [2100, 700, 0, 1300, 256, 45],
                [0, 0, 4401, 0, 0, 0]]
    M, E = sum(routings[0]), len(routings[0])
    assert all(sum(r) == M and len(r) == E for r in routings)
    off0, _, _, xb, wb, dyb = _inputs(routings[0], N, K, 1900)
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
    o = dev_i32(off0)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((E, N, K), device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        mg.wgrad(dy, x, o, out=dw)                  # allocates the stream's workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("captured fwd + dgrad + wgrad", N, K, routings)
    with torch.cuda.graph(g, stream=s):
        mg.fwd(x, w, o, out=y)
        mg.dgrad(dy, w, o, out=dx)
        mg.wgrad(dy, x, o, out=dw)
    torch.cuda.synchronize()
    scratch = torch.empty((E, N, K), device="cuda")
    for rep, sizes in enumerate(routings):
        off = offsets_from_sizes(sizes)
        o.copy_(dev_i32(off))                       # the new routing, in place
        y.fill_(float("nan"))
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
        mg.wgrad(dy, x, dev_i32(offsets_from_sizes(routings[rep - 1])), out=scratch)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, r in (("fwd", gate_fwd_full(xb, wb, off, host_bits(y))),
                        ("dgrad", gate_dgrad_full(dyb, wb, off, host_bits(dx))),
                        ("wgrad", gate_wgrad_full(dyb, xb, off, dw.cpu().numpy()))):
            _say("replay", rep, sizes, name, str(r))
            assert r.passed, f"replay {rep} {name}: {r}"


def test_host_threads_on_their_own_streams():
    """Four host threads, each on a stream of its own, launch the weight
    gradient (whose token split takes this heavy expert's tiles and a
    per-stream workspace, allocated on the stream's first call under the
    library's lock) and the forward five times each, at the same time: every
    result is bitwise the single-threaded one, which matches the oracle."""
    import threading
    sizes, N, K = [2017, 33, 65, 129, 0, 0, 0, 700], 1544, 776
    off, M, E, xb, wb, dyb = _inputs(sizes, N, K, 2100, x_scale=1.0, w_scale=1.0)
    dy, x, w, o = dev_bf16(dyb), dev_bf16(xb), dev_bf16(wb), dev_i32(off)
    ref_dw, ref_y = mg.wgrad(dy, x, o), mg.fwd(x, w, o)
    torch.cuda.synchronize()
    r = gate_wgrad_full(dyb, xb, off, ref_dw.cpu().numpy())
    assert r.passed, str(r)
    results, errors = {}, []

    def work(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [(mg.wgrad(dy, x, o), mg.fwd(x, w, o)) for _ in range(5)]
            s.synchronize()
            results[t] = outs
        except Exception as ex:                  # reported by the main thread
            errors.append(repr(ex))

    _say("four host threads, own streams", sizes, N, K)
    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    assert sorted(results) == [0, 1, 2, 3]
    for t, outs in results.items():
        for i, (dw, y) in enumerate(outs):
            assert torch.equal(dw, ref_dw), f"thread {t} call {i}: weight gradient differs"
            assert torch.equal(y.view(torch.int16), ref_y.view(torch.int16)), \
                f"thread {t} call {i}: forward differs"


def test_validation_and_split_switches():
    """MGEMM_VALIDATE=1 and MGEMM_SPLIT=0, which the library reads once per
    process, in a child process (tests/gpu_env_child.py): valid offsets pass
    and the unsplit weight gradient matches the oracle; decreasing offsets,
    offsets[E] > M, a missing leading zero and a device descriptor with
    k = 12 are rejected before any launch, their outputs untouched."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ, MGEMM_VALIDATE="1", MGEMM_SPLIT="0",
               PYTHONPATH=os.pathsep.join([os.path.dirname(here), here,
                                           os.environ.get("PYTHONPATH", "")]))
    _say("child with MGEMM_VALIDATE=1 MGEMM_SPLIT=0")
    p = subprocess.run([sys.executable, "-u", os.path.join(here, "gpu_env_child.py")],
                       env=env, capture_output=True, text=True, timeout=150)
    print(p.stdout[-3000:], p.stderr[-3000:], flush=True)
    assert p.returncode == 0 and "[child] ok" in p.stdout


def test_operands_beyond_4gib_sampled():
    """fwd, dgrad and wgrad where X [1052672, 2176] bf16 (4.58 GB) and the dgrad
    output dX of the same shape extend past 4 GiB, the last expert's rows lying
    beyond the 4 GiB byte offset: every tile base and store address must be
    64-bit.  X is the row-addressable lattice operand (built on the device in
    row chunks, recomputed on the host for the sampled rows); samples are
    concentrated in the rows past the boundary."""
    from oracle import check_bf16, sample_dgrad, sample_fwd
    from workloads.synth import LatticeMatrix, lattice_bf16
    M, K, N = (1 << 20) + 4096, 2176, 256
    sizes = [400000, 0, 350000, M - 750000]
    off = offsets_from_sizes(sizes)
    E = len(sizes)
    boundary = (1 << 32) // (2 * K)                  # first X row past 4 GiB
    assert off[-2] < boundary < M
    _say("beyond 4 GiB", M, K, N, sizes)
    x = lattice_bf16(M, K, "cuda")
    xh = LatticeMatrix(M, K)
    wb = normal_bf16_bits((E, N, K), K ** -0.5, 900, 1)
    dyb = normal_bf16_bits((M, N), 1.0, 900, 2)
    w, dy, o = dev_bf16(wb), dev_bf16(dyb), dev_i32(off)
    hint = int(max(sizes))
    rng = np.random.default_rng(900)
    rows = np.concatenate([rng.integers(0, M, 512), rng.integers(boundary, M, 1024),
                           np.arange(M - 64, M), np.arange(boundary - 32, boundary + 32)])
    rows_t = torch.from_numpy(rows).cuda()

    y = mg.fwd(x, w, o, hint)
    cols = rng.integers(0, N, rows.size)
    got = host_bits(y[rows_t, torch.from_numpy(cols).cuda()])
    exact, mag = sample_fwd(xh, wb, off, rows, cols)
    rep = check_bf16(got, exact, mag, K)
    assert rep.passed, f"fwd: {rep}"
    del y

    dx = mg.dgrad(dy, w, o, hint)
    cols = rng.integers(0, K, rows.size)
    got = host_bits(dx[rows_t, torch.from_numpy(cols).cuda()])
    exact, mag = sample_dgrad(dyb, wb, off, rows, cols)
    rep = check_bf16(got, exact, mag, N)
    assert rep.passed, f"dgrad: {rep}"
    del dx

    dw = mg.wgrad(dy, x, o, E)
    torch.cuda.synchronize()
    rep = gate_wgrad_sampled(dyb, xh, off, dw.cpu().numpy(), S=96, seed=900)
    assert rep.passed, f"wgrad: {rep}"


def test_longest_reductions_sampled():
    """The longest reductions the API takes (2^22 steps, 65536 stages in one
    tile): the forward with K = 2^22, the dgrad with N = 2^22, and the weight
    gradient over 2^22 tokens, on two ragged experts each, sampled against the
    oracle."""
    from oracle import check_bf16, sample_dgrad, sample_fwd
    R = 1 << 22
    rng = np.random.default_rng(901)
    sizes = [24, 16]
    off = offsets_from_sizes(sizes)
    M, E = int(off[-1]), 2
    rows = np.arange(M)
    _say("longest reductions: fwd K", R)
    xb = normal_bf16_bits((M, R), 1.0, 901, 1)
    wb = normal_bf16_bits((E, 16, R), R ** -0.5, 901, 2)
    y = mg.fwd(dev_bf16(xb), dev_bf16(wb), dev_i32(off))
    cols = rng.integers(0, 16, M)
    exact, mag = sample_fwd(xb, wb, off, rows, cols)
    rep = check_bf16(host_bits(y)[rows, cols], exact, mag, R)
    assert rep.passed, f"fwd: {rep}"
    del xb, wb, y
    _say("longest reductions: dgrad N", R)
    dyb = normal_bf16_bits((M, R), 1.0, 901, 3)
    wb = normal_bf16_bits((E, R, 16), R ** -0.5, 901, 4)
    dx = mg.dgrad(dev_bf16(dyb), dev_bf16(wb), dev_i32(off))
    exact, mag = sample_dgrad(dyb, wb, off, rows, cols)
    rep = check_bf16(host_bits(dx)[rows, cols], exact, mag, R)
    assert rep.passed, f"dgrad: {rep}"
    del dyb, wb, dx
    _say("longest reductions: wgrad tokens", R)
    off2 = offsets_from_sizes([R - 1000, 1000])
    dyb = normal_bf16_bits((R, 16), 1.0, 901, 5)
    xb = normal_bf16_bits((R, 24), 1.0, 901, 6)
    dw = mg.wgrad(dev_bf16(dyb), dev_bf16(xb), dev_i32(off2), 2)
    torch.cuda.synchronize()
    rep = gate_wgrad_sampled(dyb, xb, off2, dw.cpu().numpy(), S=64, seed=901)
    assert rep.passed, f"wgrad: {rep}"


def test_single_expert_is_plain_gemm():
    off, M, E, xb, wb, dyb = _inputs([777], 392, 328, 300)
    _say("E=1", M)
    yb, dxb = _run_mgrouped(off, M, xb, wb, dyb, 392, 328)
    assert gate_fwd_full(xb, wb, off, yb).passed
    assert gate_dgrad_full(dyb, wb, off, dxb).passed
    # and against torch's own fp32 GEMM of the same bf16 values
    y = dev_bf16(yb).float()
    ref = dev_bf16(xb).float() @ dev_bf16(wb)[0].float().t()
    assert torch.allclose(y, ref, rtol=2 ** -7, atol=1e-2)


def test_all_experts_empty_and_zero_reduction():
    off = offsets_from_sizes([0, 0, 0])
    M, N, K = 40, 64, 64
    xb = normal_bf16_bits((M, K), 0.1, 1, 1); wb = normal_bf16_bits((3, N, K), 0.1, 1, 2)
    _say("all empty")
    yb, dxb = _run_mgrouped(off, M, xb, wb, normal_bf16_bits((M, N), 1.0, 1, 3), N, K)
    assert (yb == SENTINEL).all() and (dxb == SENTINEL).all()
    dw = mg.wgrad(dev_bf16(normal_bf16_bits((M, N), 1.0, 1, 3)), dev_bf16(xb), dev_i32(off))
    prior = torch.full((3, N, K), 2.5, device="cuda")
    mg.wgrad(dev_bf16(normal_bf16_bits((M, N), 1.0, 1, 3)), dev_bf16(xb), dev_i32(off),
             out=prior, accumulate=True)
    torch.cuda.synchronize()
    assert (dw == 0).all() and (prior == 2.5).all()
    # K == 0: the forward is an empty sum, the owned rows become zero
    off2 = offsets_from_sizes([5, 3])
    x0 = torch.empty((8, 0), dtype=torch.bfloat16, device="cuda")
    w0 = torch.empty((2, 16, 0), dtype=torch.bfloat16, device="cuda")
    y0 = mg.fwd(x0, w0, dev_i32(off2), out=sentinel_bf16((10, 16))[:8])
    torch.cuda.synchronize()
    assert (y0.float() == 0).all()


def test_launch_hint_too_small_is_still_correct():
    off, M, E, xb, wb, dyb = _inputs([600, 1, 900], 520, 136, 400)
    _say("hint=1")
    yb, dxb = _run_mgrouped(off, M, xb, wb, dyb, 520, 136, hint=1)
    assert gate_fwd_full(xb, wb, off, yb).passed
    assert gate_dgrad_full(dyb, wb, off, dxb).passed


def test_side_stream_and_aliases():
    off, M, E, xb, wb, dyb = _inputs([130, 0, 260], 264, 264, 500)
    _say("side stream")
    x, w, dy, o = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb), dev_i32(off)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y = mg.Mgemm(x, w, o, 260, transpose_B=True)
        dx = mg.Mgemm(dy, w, o, 260, transpose_B=False)
        dw = mg.Kgemm(dy, x, o, "gw13")
    s.synchronize()
    assert gate_fwd_full(xb, wb, off, host_bits(y)).passed
    assert gate_dgrad_full(dyb, wb, off, host_bits(dx)).passed
    assert gate_wgrad_full(dyb, xb, off, dw.cpu().numpy()).passed


# ------------------------------------------------------ full-size workloads --
#
# Every output element of the benchmark workloads against the oracle (expert
# by expert, tests/parity.py): outputs pre-filled with a sentinel (bf16) or NaN
# (fp32), so that an element the kernel never wrote fails; each op launched
# twice into two live buffers and compared bitwise (run-to-run
# reproducibility); and no strict one-ulp failure among elements that do not
# cancel.

def _nan_f32(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _twice_mgrouped(fn, a, w, o, hint, shape):
    r1 = fn(a, w, o, hint, out=sentinel_bf16(shape))
    r2 = fn(a, w, o, hint, out=sentinel_bf16(shape))
    torch.cuda.synchronize()
    assert torch.equal(r1.view(torch.int16), r2.view(torch.int16)), "not bitwise reproducible"
    return host_bits(r1)


def _twice_wgrad(dy, x, o, shape):
    d1 = mg.wgrad(dy, x, o, out=_nan_f32(shape))
    d2 = mg.wgrad(dy, x, o, out=_nan_f32(shape))
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int32), d2.view(torch.int32)), "wgrad not bitwise reproducible"
    return d1.cpu().numpy()


def _assert_bf16_gate(what, rep):
    _say(what, str(rep), f"nc_strict_fails={rep.nc_strict_fails}")
    assert rep.passed, what + " " + str(rep)
    assert rep.nc_strict_fails == 0, f"{what}: strict failures on non-cancelling elements"


@pytest.mark.parametrize("cfg", [2, 3])
def test_uniform_workloads_whole(cfg):
    (wl,) = make_workload(cfg)
    _say(wl.name)
    xb, wb, dyb = wl.x_bits(), wl.w_bits(), wl.dy_bits()
    x, w, dy, o = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb), dev_i32(wl.offsets)
    hint = int(wl.sizes().max())
    yb = _twice_mgrouped(mg.fwd, x, w, o, hint, (wl.M, wl.N))
    dxb = _twice_mgrouped(mg.dgrad, dy, w, o, hint, (wl.M, wl.K))
    dw = _twice_wgrad(dy, x, o, (wl.E, wl.N, wl.K))
    del x, w, dy
    _assert_bf16_gate("fwd", gate_fwd_experts(xb, wb, wl.offsets, yb))
    _assert_bf16_gate("dgrad", gate_dgrad_experts(dyb, wb, wl.offsets, dxb))
    r = gate_wgrad_experts(dyb, xb, wl.offsets, dw)
    _say("wgrad", str(r))
    assert r.passed, "wgrad " + str(r)


@pytest.mark.parametrize("name", ["a3b_gate_up", "a3b_down"])
def test_a3b_router_workload_whole(name):
    (wl,) = make_workload(4, name)
    _say(wl.name, wl.rows)
    xb, wb, dyb = wl.x_bits(), wl.w_bits(), wl.dy_bits()
    x, w, dy, o = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb), dev_i32(wl.offsets)
    hint = int(wl.sizes().max())
    yb = _twice_mgrouped(mg.fwd, x, w, o, hint, (wl.M, wl.N))
    dxb = _twice_mgrouped(mg.dgrad, dy, w, o, hint, (wl.M, wl.K))
    del x, w, dy
    _assert_bf16_gate("fwd", gate_fwd_experts(xb, wb, wl.offsets, yb))
    _assert_bf16_gate("dgrad", gate_dgrad_experts(dyb, wb, wl.offsets, dxb))


@pytest.mark.parametrize("name", ["a3b_zipf_gw13", "a3b_zipf_gw2"])
def test_a3b_zipf_wgrad_whole(name):
    (wl,) = make_workload(5, name)
    _say(wl.name, wl.sizes().tolist())
    xb, dyb = wl.x_bits(), wl.dy_bits()
    x, dy, o = dev_bf16(xb), dev_bf16(dyb), dev_i32(wl.offsets)
    got = _twice_wgrad(dy, x, o, (wl.E, wl.N, wl.K))
    del x, dy
    empty = np.flatnonzero(wl.sizes() == 0)
    assert len(empty) == 4 and (got[empty] == 0).all()
    r = gate_wgrad_experts(dyb, xb, wl.offsets, got)
    _say("wgrad", str(r))
    assert r.passed, str(r)


# ------------------------------------------- exact results at full size --
# Operands that are integers in [-3, 3]: every product is an integer of
# magnitude <= 9 and every partial sum of a reduction of length R at most 9 R,
# below 2^24 for every reduction here (R <= 10804), so fp32 accumulation in any
# order is exact.  The kernels then owe the exact value itself -- bf16 outputs
# its round to nearest even, fp32 outputs the value -- on every element, with
# no tolerance: a wrong row, column, expert or reduction range changes bits.

def _exact_bf16(kind, exact, got_bits):
    from oracle import f64_to_bf16_bits
    want = f64_to_bf16_bits(exact)
    bad = int((got_bits != want).sum())
    _say(kind, "elements differing from the rounded exact value:", bad)
    assert bad == 0, f"{kind}: {bad} of {want.size} elements differ"


@pytest.mark.parametrize("name", ["a3b_gate_up", "a3b_down"])
def test_a3b_mgrouped_exact_on_small_integers(name):
    from oracle import bf16_bits_to_f64, grouped_dgrad, grouped_fwd
    from workloads.synth import small_int_bf16_bits
    (wl,) = make_workload(4, name)
    _say(wl.name, "exact", wl.rows)
    xb = small_int_bf16_bits((wl.M, wl.K), 9100, wl.tag, 1)
    wb = small_int_bf16_bits((wl.E, wl.N, wl.K), 9100, wl.tag, 2)
    dyb = small_int_bf16_bits((wl.M, wl.N), 9100, wl.tag, 3)
    hint = int(wl.sizes().max())
    y, dx = _run_mgrouped(wl.offsets, wl.M, xb, wb, dyb, wl.N, wl.K, hint)
    last = int(wl.offsets[-1])
    _check_untouched(y, wl.offsets)
    _check_untouched(dx, wl.offsets)
    x, w, dy = bf16_bits_to_f64(xb), bf16_bits_to_f64(wb), bf16_bits_to_f64(dyb)
    _exact_bf16("fwd", grouped_fwd(x, w, wl.offsets)[:last], y[:last])
    _exact_bf16("dgrad", grouped_dgrad(dy, w, wl.offsets)[:last], dx[:last])


@pytest.mark.parametrize("name", ["a3b_zipf_gw13", "a3b_zipf_gw2"])
def test_a3b_wgrad_exact_on_small_integers(name):
    from oracle import bf16_bits_to_f64, grouped_wgrad
    from workloads.synth import small_int_bf16_bits
    (wl,) = make_workload(5, name)
    _say(wl.name, "exact", wl.sizes().max())
    xb = small_int_bf16_bits((wl.M, wl.K), 9110, wl.tag, 1)
    dyb = small_int_bf16_bits((wl.M, wl.N), 9110, wl.tag, 2)
    dw = mg.wgrad(dev_bf16(dyb), dev_bf16(xb), dev_i32(wl.offsets), wl.E,
                  out=torch.full((wl.E, wl.N, wl.K), float("nan"), device="cuda"))
    got = dw.cpu().numpy().astype(np.float64)
    exact = grouped_wgrad(bf16_bits_to_f64(dyb), bf16_bits_to_f64(xb), wl.offsets, wl.E)
    bad = int((got != exact).sum())
    _say("wgrad elements differing from the exact value:", bad)
    assert bad == 0, f"{bad} of {got.size} elements differ"


# ------------------------------------- gate-up forward with SwiGLU, gathered --

SW_CASES = [
    # sizes, T (token rows; None = rows already grouped, no index), I, K, extra rows
    ([200, 0, 184, 128], 300, 128, 256, 3),
    ([1, 255, 256, 257], None, 264, 136, 5),      # I = 2 tiles + 8 columns
    ([0, 513, 0, 1, 300], 900, 520, 200, 0),      # repeated indices, empty experts
    ([700, 0, 0], 50, 72, 1032, 2),               # 14 uses of each token, long K
    ([64] * 9, 4096, 384, 64, 0),                 # indices spread over a tall x
]


def _swiglu_check(xb, gather, wb, off, got_bits, rows=None, cols=None):
    from oracle import check_bf16_swiglu, sample_fwd_swiglu
    I = wb.shape[1] // 2
    K = wb.shape[2]
    if rows is None:
        n = int(off[-1])
        rows = np.repeat(np.arange(n), I)
        cols = np.tile(np.arange(I), n)
    h, g, u, sg, su = sample_fwd_swiglu(xb, gather, wb, off, rows, cols)
    return check_bf16_swiglu(got_bits[rows, cols], h, g, u, sg, su, K)


@pytest.mark.parametrize("case", range(len(SW_CASES)))
def test_fwd_swiglu(case):
    sizes, T, I, K, extra = SW_CASES[case]
    _say("fwd_swiglu", sizes, T, I, K, extra)
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + extra
    E = len(sizes)
    rng = np.random.default_rng(400 + case)
    xb = normal_bf16_bits((T if T else M, K), 1.0, 400 + case, 1)
    wb = normal_bf16_bits((E, 2 * I, K), K ** -0.5, 400 + case, 2)
    gather = rng.integers(0, T, M).astype(np.int32) if T else None
    out = sentinel_bf16((M, I))
    h = mg.fwd_swiglu(dev_bf16(xb), dev_bf16(wb), dev_i32(off),
                      gather=None if gather is None else dev_i32(gather), out=out)
    torch.cuda.synchronize()
    got = host_bits(h)
    r = _swiglu_check(xb, gather, wb, off, got)
    assert r.passed, str(r)
    _check_untouched(got, off)


def test_fwd_swiglu_gather_equals_pregathered():
    """Gathering inside the operand loads gives bitwise the result of
    gathering the rows first (torch index_select) and running ungathered."""
    sizes, T, I, K = [300, 5, 0, 700], 640, 256, 512
    off = offsets_from_sizes(sizes)
    M = int(off[-1])
    xb = normal_bf16_bits((T, K), 1.0, 450, 1)
    wb = normal_bf16_bits((len(sizes), 2 * I, K), K ** -0.5, 450, 2)
    gather = np.random.default_rng(450).integers(0, T, M).astype(np.int32)
    x, w, o, gi = dev_bf16(xb), dev_bf16(wb), dev_i32(off), dev_i32(gather)
    h1 = mg.fwd_swiglu(x, w, o, gather=gi)
    h2 = mg.fwd_swiglu(x.index_select(0, gi.long()).contiguous(), w, o)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)


def test_a3b_gate_up_swiglu_gathered_sampled():
    """The 30B-A3B share's gate-up GEMM as a trainer would run it: 16384 tokens
    [16384, 3072] gathered through the router's row-to-token map into 32 expert
    groups, w13 [32, 2560, 3072], SwiGLU fused: h [M, 1280]."""
    from workloads.synth import router_offsets
    off, token_of_row = router_offsets(16384, 128, 8, 32, seed=4)
    (wl,) = [w for w in make_workload(4) if w.name == "a3b_gate_up"]
    assert np.array_equal(off, wl.offsets)
    T, K, I = 16384, 3072, 1280
    xb = normal_bf16_bits((T, K), 1.0, 4, 9, 1)
    wb = wl.w_bits()
    _say("a3b gate-up swiglu gathered", int(off[-1]))
    h = mg.fwd_swiglu(dev_bf16(xb), dev_bf16(wb), dev_i32(off), gather=dev_i32(token_of_row),
                      max_m_per_e=int(wl.sizes().max()))
    torch.cuda.synchronize()
    got = host_bits(h)
    rng = np.random.default_rng(7)
    rows = rng.integers(0, int(off[-1]), 4096)
    cols = rng.integers(0, I, 4096)
    # plus every column of the first and last row of each expert (tile edges)
    edge = np.concatenate([[off[e], off[e + 1] - 1] for e in range(32) if off[e + 1] > off[e]])
    rows = np.concatenate([rows, np.repeat(edge, 16)])
    cols = np.concatenate([cols, np.tile(np.arange(I - 16, I), edge.size)])
    r = _swiglu_check(xb, token_of_row, wb, off, got, rows, cols)
    assert r.passed, str(r)


# ------------------------------------------------ per-group descriptor list --

def _list_check(groups_bits, outs):
    """Every output element of every group against the oracle, bf16 gate."""
    from oracle import bf16_bits_to_f64, check_bf16, grouped_list
    a64 = [(bf16_bits_to_f64(a), bf16_bits_to_f64(b)) for a, b in groups_bits]
    ref = grouped_list(a64)
    mag = grouped_list([(np.abs(a), np.abs(b)) for a, b in a64])
    for g, ((a, b), d, r, s) in enumerate(zip(groups_bits, outs, ref, mag)):
        if r.size == 0:
            continue
        k = max(a.shape[1], 1)
        rep = check_bf16(host_bits(d), r, s, k)
        assert rep.passed, f"group {g}: {rep}"


def test_grouped_list_mixes_m_and_k_grouped():
    """One launch holding an expert layer's M-grouped forward (Y_e = X_e W_e^T,
    one group per expert) and its K-grouped weight gradient (dW_e = dY_e^T X_e,
    one group per expert on token-axis-last operands: A and B are expert e's
    column ranges of dY^T [N, M] and X^T [K, M], row stride M), against the
    oracle's grouped forward and grouped weight gradient (bf16 results here).
    Expert sizes are multiples of 8 so that the column views stay 16-byte
    aligned; the empty expert gives an empty forward group and a k = 0
    weight-gradient group (zeros)."""
    from oracle import bf16_bits_to_f64, check_bf16, grouped_fwd, grouped_wgrad
    sizes = [264, 0, 136, 520, 8]
    off = offsets_from_sizes(sizes)
    M, E, N, K = int(off[-1]), len(sizes), 200, 264
    xb = normal_bf16_bits((M, K), 1.0, 610, 1)
    wb = normal_bf16_bits((E, N, K), K ** -0.5, 610, 2)
    dyb = normal_bf16_bits((M, N), 1.0, 610, 3)
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
    xt, dyt = x.t().contiguous(), dy.t().contiguous()
    y = sentinel_bf16((M, N))
    dws = [sentinel_bf16((N, K)) for _ in range(E)]
    groups, outs = [], []
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        groups.append((x[lo:hi], w[e]))
        outs.append(y[lo:hi])
        groups.append((dyt[:, lo:hi], xt[:, lo:hi]))
        outs.append(dws[e])
    _say("grouped_list fwd + wgrad", sizes, N, K)
    mg.grouped_list(groups, outs)
    torch.cuda.synchronize()
    x64, w64, dy64 = bf16_bits_to_f64(xb), bf16_bits_to_f64(wb), bf16_bits_to_f64(dyb)
    rep = check_bf16(host_bits(y), grouped_fwd(x64, w64, off),
                     grouped_fwd(np.abs(x64), np.abs(w64), off), K)
    assert rep.passed, f"forward groups: {rep}"
    dw = grouped_wgrad(dy64, x64, off, E)
    dw_mag = grouped_wgrad(np.abs(dy64), np.abs(x64), off, E)
    for e in range(E):
        rep = check_bf16(host_bits(dws[e]), dw[e], dw_mag[e], max(sizes[e], 1))
        assert rep.passed, f"weight-gradient group {e}: {rep}"


def test_grouped_list_mixed_shapes():
    """Groups of different m, n, k in one launch: ragged tiles, row strides
    wider than the rows (views into bigger buffers), an empty group, a group
    with k = 0 (zeros), several tiles per group."""
    shapes = [(300, 264, 136), (0, 64, 64), (1, 8, 8), (513, 520, 200), (40, 16, 0),
              (256, 256, 512), (77, 1032, 72)]
    groups_bits, groups, outs = [], [], []
    for g, (m, n, k) in enumerate(shapes):
        ab = normal_bf16_bits((m, k), 1.0, 500 + g, 1)
        bb = normal_bf16_bits((n, k), k ** -0.5 if k else 1.0, 500 + g, 2)
        groups_bits.append((ab, bb))
        # A and B as views with padded rows (stride k + 16), D inside a wider buffer
        abuf = torch.zeros((m, k + 16), dtype=torch.bfloat16, device="cuda")
        bbuf = torch.zeros((n, k + 16), dtype=torch.bfloat16, device="cuda")
        if m * k:
            abuf[:, :k] = dev_bf16(ab)
        if n * k:
            bbuf[:, :k] = dev_bf16(bb)
        dbuf = sentinel_bf16((m, n + 24))
        groups.append((abuf[:, :k], bbuf[:, :k]))
        outs.append(dbuf[:, :n])
    _say("grouped_list mixed", shapes)
    mg.grouped_list(groups, outs)
    torch.cuda.synchronize()
    _list_check(groups_bits, outs)
    for g, (m, n, k) in enumerate(shapes):
        pad = host_bits(outs[g]._base)[:, n:] if m else None
        if pad is not None:
            assert (pad == SENTINEL).all(), f"group {g}: padding columns written"


def test_grouped_list_zero_width_operands():
    """Groups with k = 0 whose A and B are plain contiguous [m, 0] and [n, 0]
    tensors (torch gives such tensors a row stride of 1): the binding passes
    a row stride the library accepts and the outputs are zeros; a group with
    n = 0 beside them writes nothing."""
    a = torch.empty((300, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((264, 0), dtype=torch.bfloat16, device="cuda")
    a1 = torch.empty((1, 0), dtype=torch.bfloat16, device="cuda")
    b0 = torch.empty((0, 8), dtype=torch.bfloat16, device="cuda")
    a8 = dev_bf16(normal_bf16_bits((40, 8), 1.0, 520, 1))
    outs = [sentinel_bf16((300, 264)), sentinel_bf16((1, 264)), sentinel_bf16((40, 0))]
    _say("grouped_list zero-width operands")
    mg.grouped_list([(a, b), (a1, b), (a8, b0)], outs)
    torch.cuda.synchronize()
    assert (host_bits(outs[0]) == 0).all() and (host_bits(outs[1]) == 0).all()


def test_grouped_list_equals_mgrouped_forward():
    """Per-expert groups pointing into one X and one W give bitwise the
    M-grouped forward's result (same tiles, same reduction order)."""
    sizes, N, K = [300, 0, 517, 64, 1000], 520, 264
    off = offsets_from_sizes(sizes)
    M = int(off[-1])
    x = dev_bf16(normal_bf16_bits((M, K), K ** -0.5, 510, 1))
    w = dev_bf16(normal_bf16_bits((len(sizes), N, K), K ** -0.5, 510, 2))
    y = mg.fwd(x, w, dev_i32(off))
    ylist = torch.empty_like(y)
    groups = [(x[off[e]:off[e + 1]], w[e]) for e in range(len(sizes))]
    outs = [ylist[off[e]:off[e + 1]] for e in range(len(sizes))]
    mg.grouped_list(groups, outs)
    torch.cuda.synchronize()
    assert torch.equal(y, ylist)


def test_grouped_list_flattened_lora_experts():
    """Nested grouped GEMM flattened: 3 LoRA adapters x 4 experts = 12 groups,
    each expert's rows times each adapter's rank-16 down projection."""
    rng = np.random.default_rng(520)
    K, R = 1024, 16
    xs = [normal_bf16_bits((int(m), K), 1.0, 520, e, 1) for e, m in enumerate(rng.integers(0, 400, 4))]
    ads = [normal_bf16_bits((R, K), K ** -0.5, 520, l, 2) for l in range(3)]
    groups_bits = [(x, ad) for ad in ads for x in xs]
    groups = [(dev_bf16(a), dev_bf16(b)) for a, b in groups_bits]
    outs = mg.grouped_list(groups)
    torch.cuda.synchronize()
    _list_check(groups_bits, outs)
