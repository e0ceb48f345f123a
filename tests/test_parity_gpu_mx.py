"""GPU parity of the MXFP8 grouped forward, the MXFP8 K-grouped weight
gradient and the scale-layout kernel against the fp64 oracle (needs an
MI355X).

The GEMM gets the oracle's blocked scales (so its cases do not depend on the
layout kernel); the layout kernel is compared bit for bit with the oracle's
layout; one end-to-end case feeds the kernel-made layout to the GEMM.  bf16
outputs pass the MX gate of oracle/gate.py (one bf16 ulp of the rounded
exact value, or within the precision floor of the fp8 matrix-core products);
fp32 weight gradients pass the per-element MX fp32 gate, empty experts exactly
zero (or the prior contents when accumulating).
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_bf16_amd as mg
from oracle import check_bf16_mx, grouped_fwd, grouped_fwd_mx, mx_dequant, mx_scales_blocked
from oracle import sample_fwd_mx
from parity import SENTINEL, dev_i32, host_bits, sentinel_bf16
from workloads import make_workload, offsets_from_sizes
from workloads.synth import mx_e4m3_codes, mx_e8m0_codes

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def _mx_inputs(sizes, N, K, spread, seed, extra_rows=0, center=121):
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + extra_rows
    E = len(sizes)
    x8 = mx_e4m3_codes((M, K), 8000, seed, 1)
    w8 = mx_e4m3_codes((E, N, K), 8000, seed, 2)
    xs = mx_e8m0_codes((M, K // 32), center, spread, 8000, seed, 3)
    ws = mx_e8m0_codes((E, N, K // 32), center, spread, 8000, seed, 4)
    return off, M, E, x8, w8, xs, ws


def _run(off, M, N, x8, w8, xs, ws, hint=0):
    y = mg.fwd_mx(_u8(x8), _u8(mx_scales_blocked(xs)), _u8(w8), _u8(mx_scales_blocked(ws)),
                  dev_i32(off), hint, out=sentinel_bf16((M, N)))
    torch.cuda.synchronize()
    return host_bits(y)


def _gate_full(off, x8, w8, xs, ws, got):
    o = int(off[-1])
    exact = grouped_fwd_mx(x8, xs, w8, ws, off)[:o]
    mag = grouped_fwd(np.abs(mx_dequant(x8, xs)), np.abs(mx_dequant(w8, ws)), off)[:o]
    return check_bf16_mx(got[:o], exact, mag)


# (expert sizes, N, K, scale spread): ragged experts, empty ones, reductions
# of one 32-block, of less than one 128-step stage, with a ragged last stage,
# and of many stages
MX_CASES = [
    ([300, 0, 17, 513], 264, 256, 2),
    ([1, 255, 257], 136, 96, 1),
    ([700], 520, 416, 3),
    ([0, 0, 129], 8, 32, 0),
    ([64, 0, 100, 64, 300, 1, 64, 200], 256, 2048, 1),
    ([513, 511], 1032, 160, 2),
]


@pytest.mark.parametrize("case", range(len(MX_CASES)))
def test_fwd_mx(case):
    sizes, N, K, spread = MX_CASES[case]
    _say("fwd_mx", sizes, N, K, spread)
    off, M, E, x8, w8, xs, ws = _mx_inputs(sizes, N, K, spread, case, extra_rows=3)
    got = _run(off, M, N, x8, w8, xs, ws)
    rep = _gate_full(off, x8, w8, xs, ws, got)
    assert rep.passed, str(rep)
    assert (got[int(off[-1]):] == SENTINEL).all(), "rows past offsets[E] were written"


def test_fwd_mx_wide_scale_range_and_extreme_codes():
    """Scales across 2^-40 .. 2^40 per operand and elements at +-448, the
    subnormals and zeros: the exponent arithmetic of the scaled product."""
    sizes, N, K = [130, 70], 136, 256
    off, M, E, x8, w8, xs, ws = _mx_inputs(sizes, N, K, 40, 99, center=127)
    x8 = x8.copy(); w8 = w8.copy()
    x8[::7, ::5] = 0x7E; w8[:, ::3, 1::7] = 0xFE          # +448, -448
    x8[1::9, 2::11] = 0x01; w8[:, 2::5, ::13] = 0x07      # subnormals
    x8[3::4, 64:96] = 0                                   # a zero block
    _say("fwd_mx extremes", sizes, N, K)
    got = _run(off, M, N, x8, w8, xs, ws)
    rep = _gate_full(off, x8, w8, xs, ws, got)
    assert rep.passed, str(rep)


def test_fwd_mx_unit_scales_equal_torch_fp8_matmul_values():
    """With every scale 1.0 the result is the plain product of the decoded
    E4M3 values (pinned in the oracle against torch's float8 cast)."""
    sizes, N, K = [200, 56], 128, 512
    off, M, E, x8, w8, _, _ = _mx_inputs(sizes, N, K, 0, 5)
    xs = np.full((M, K // 32), 127, np.uint8)
    ws = np.full((E, N, K // 32), 127, np.uint8)
    _say("fwd_mx unit scales", sizes, N, K)
    got = _run(off, M, N, x8, w8, xs, ws)
    assert _gate_full(off, x8, w8, xs, ws, got).passed


@pytest.mark.parametrize("rows,K,batch", [(1, 32, 1), (257, 96, 1), (300, 416, 3), (64, 2048, 2),
                                          (1000, 160, 1)])
def test_scales_blocked_kernel_bit_exact(rows, K, batch):
    _say("mx_scales_blocked", rows, K, batch)
    s = mx_e8m0_codes((batch, rows, K // 32), 127, 127, 8100, rows, K)
    got = mg.mx_scales_blocked(_u8(s)).cpu().numpy()
    want = mx_scales_blocked(s)
    assert got.shape == want.shape
    np.testing.assert_array_equal(got, want)


def test_fwd_mx_end_to_end_with_layout_kernel():
    sizes, N, K = [90, 0, 333], 264, 288
    off, M, E, x8, w8, xs, ws = _mx_inputs(sizes, N, K, 2, 11)
    _say("fwd_mx end to end", sizes, N, K)
    bx = mg.mx_scales_blocked(_u8(xs))
    bw = mg.mx_scales_blocked(_u8(ws))
    y = mg.fwd_mx(_u8(x8), bx, _u8(w8), bw, dev_i32(off))
    torch.cuda.synchronize()
    assert _gate_full(off, x8, w8, xs, ws, host_bits(y)).passed


def test_fwd_mx_zero_reduction_and_empty_experts():
    M, N, E = 40, 64, 3
    off = offsets_from_sizes([0, 25, 0])
    _say("fwd_mx K=0 and empty experts")
    x8 = torch.zeros((M, 0), dtype=torch.uint8, device="cuda")
    w8 = torch.zeros((E, N, 0), dtype=torch.uint8, device="cuda")
    bx = torch.zeros((0, M, 4), dtype=torch.uint8, device="cuda")
    bw = torch.zeros((E, 0, N, 4), dtype=torch.uint8, device="cuda")
    y = mg.fwd_mx(x8, bx, w8, bw, dev_i32(off), out=sentinel_bf16((M, N)))
    got = host_bits(y)
    assert (got[:25] == 0).all() and (got[25:] == SENTINEL).all()
    # all experts empty: nothing is written
    off0 = offsets_from_sizes([0, 0, 0])
    K = 64
    y = mg.fwd_mx(torch.zeros((M, K), dtype=torch.uint8, device="cuda"),
                  torch.zeros((1, M, 4), dtype=torch.uint8, device="cuda"),
                  torch.zeros((E, N, K), dtype=torch.uint8, device="cuda"),
                  torch.zeros((E, 1, N, 4), dtype=torch.uint8, device="cuda"),
                  dev_i32(off0), out=sentinel_bf16((M, N)))
    assert (host_bits(y) == SENTINEL).all()


def test_fwd_mx_rejects_bad_shapes():
    x8 = torch.zeros((8, 48), dtype=torch.uint8, device="cuda")      # K not a multiple of 32
    w8 = torch.zeros((1, 8, 48), dtype=torch.uint8, device="cuda")
    bx = torch.zeros((1, 8, 4), dtype=torch.uint8, device="cuda")
    bw = torch.zeros((1, 1, 8, 4), dtype=torch.uint8, device="cuda")
    with pytest.raises(mg.MgemmError):
        mg.fwd_mx(x8, bx, w8, bw, dev_i32(offsets_from_sizes([8])))


@pytest.mark.parametrize("name", ["a3b_gate_up", "a3b_down"])
def test_a3b_mx_sampled(name):
    """The 30B-A3B expert shapes with MXFP8 operands, in the launch the bench
    times: sampled elements against the oracle, untouched rows, and two runs
    bit-identical."""
    (wl,) = make_workload(4, name)
    off = np.asarray(wl.offsets)
    M, N, K, E = wl.M, wl.N, wl.K, wl.E
    _say("a3b mx", name, M, N, K, E)
    x8 = mx_e4m3_codes((M, K), 8200, 1)
    w8 = mx_e4m3_codes((E, N, K), 8200, 2)
    xs = mx_e8m0_codes((M, K // 32), 121, 1, 8200, 3)
    ws = mx_e8m0_codes((E, N, K // 32), 121, 1, 8200, 4)
    dx8, dw8 = _u8(x8), _u8(w8)
    bx, bw = _u8(mx_scales_blocked(xs)), _u8(mx_scales_blocked(ws))
    o = dev_i32(off)
    y1 = mg.fwd_mx(dx8, bx, dw8, bw, o, out=sentinel_bf16((M, N)))
    y2 = mg.fwd_mx(dx8, bx, dw8, bw, o, out=sentinel_bf16((M, N)))
    g1, g2 = host_bits(y1), host_bits(y2)
    assert (g1 == g2).all(), "not deterministic"
    last = int(off[-1])
    assert (g1[last:] == SENTINEL).all()
    rng = np.random.default_rng(8201)
    rows = rng.integers(0, last, 2048)
    cols = rng.integers(0, N, 2048)
    # the first and last rows and columns of every expert too
    edges = np.concatenate([off[:-1][np.diff(off) > 0], off[1:][np.diff(off) > 0] - 1])
    rows = np.concatenate([rows, edges, edges])
    cols = np.concatenate([cols, np.zeros_like(edges), np.full_like(edges, N - 1)])
    val, mag = sample_fwd_mx(x8, xs, w8, ws, off, rows, cols)
    rep = check_bf16_mx(g1[rows, cols], val, mag)
    assert rep.passed, str(rep)


# ------------------------------------------------------------ MXFP8 wgrad --

from oracle import check_fp32_mx, grouped_wgrad, grouped_wgrad_mx, sample_wgrad_mx  # noqa: E402


def _wg_inputs(sizes, N, K, spread, seed, center=121):
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + 128                       # one stage of rows owned by no expert
    dyt8 = mx_e4m3_codes((N, M), 8400, seed, 1)
    xt8 = mx_e4m3_codes((K, M), 8400, seed, 2)
    dyts = mx_e8m0_codes((N, M // 32), center, spread, 8400, seed, 3)
    xts = mx_e8m0_codes((K, M // 32), center, spread, 8400, seed, 4)
    return off, M, dyt8, dyts, xt8, xts


def _wg_gate(off, dyt8, dyts, xt8, xts, got, prior=None):
    E = len(off) - 1
    exact = grouped_wgrad_mx(dyt8, dyts, xt8, xts, off, E, prior=prior)
    mag = grouped_wgrad(np.abs(mx_dequant(dyt8, dyts)).T, np.abs(mx_dequant(xt8, xts)).T, off, E)
    sizes = np.diff(np.asarray(off, np.int64))
    k_red = np.broadcast_to(np.maximum(sizes, 1)[:, None, None], exact.shape)
    empty = np.broadcast_to((sizes == 0)[:, None, None], exact.shape)
    return check_fp32_mx(got, exact, mag, k_red, empty_mask=empty,
                         empty_expect=None if prior is None else prior)


# (expert sizes in multiples of 128, N, K, scale spread)
WG_MX_CASES = [
    ([128, 0, 384, 256], 264, 136, 2),
    ([1024], 520, 264, 1),
    ([0, 128], 8, 8, 0),
    ([128, 128, 128, 128, 128, 0, 640], 256, 256, 1),
    ([2048, 128, 0, 256], 136, 520, 3),
]


@pytest.mark.parametrize("case", range(len(WG_MX_CASES)))
@pytest.mark.parametrize("accumulate", [False, True])
def test_wgrad_mx(case, accumulate):
    sizes, N, K, spread = WG_MX_CASES[case]
    _say("wgrad_mx", sizes, N, K, spread, "accumulate" if accumulate else "")
    off, M, dyt8, dyts, xt8, xts = _wg_inputs(sizes, N, K, spread, case)
    E = len(sizes)
    prior = None
    if accumulate:
        prior = np.random.default_rng(case).standard_normal((E, N, K)).astype(np.float32)
        out = torch.from_numpy(prior.copy()).cuda()
    else:
        out = torch.full((E, N, K), float("nan"), dtype=torch.float32, device="cuda")
    mg.wgrad_mx(_u8(dyt8), _u8(mx_scales_blocked(dyts)), _u8(xt8), _u8(mx_scales_blocked(xts)),
                dev_i32(off), E, out=out, accumulate=accumulate)
    got = out.cpu().numpy()
    rep = _wg_gate(off, dyt8, dyts, xt8, xts, got,
                   prior=None if prior is None else prior.astype(np.float64))
    assert rep.passed, str(rep)


def test_wgrad_mx_is_deterministic_and_layout_kernel_end_to_end():
    sizes, N, K = [256, 0, 512], 136, 264
    off, M, dyt8, dyts, xt8, xts = _wg_inputs(sizes, N, K, 2, 77)
    _say("wgrad_mx end to end", sizes, N, K)
    a = (_u8(dyt8), mg.mx_scales_blocked(_u8(dyts)), _u8(xt8), mg.mx_scales_blocked(_u8(xts)))
    o = dev_i32(off)
    r1 = mg.wgrad_mx(*a, o).cpu().numpy()
    r2 = mg.wgrad_mx(*a, o).cpu().numpy()
    assert (r1 == r2).all()
    assert _wg_gate(off, dyt8, dyts, xt8, xts, r1).passed


def test_wgrad_mx_rejects_bad_shapes():
    z = lambda *sh: torch.zeros(sh, dtype=torch.uint8, device="cuda")
    # M = 96 is not a multiple of 128 (the binding's shapes are consistent, so
    # the library's own check raises)
    with pytest.raises(mg.MgemmError):
        mg.wgrad_mx(z(8, 96), z(0, 8, 4), z(8, 96), z(0, 8, 4),
                    dev_i32(offsets_from_sizes([96])), 1)


# ------------------------------------ MXFP8 wgrad on token-major operands --

# (expert sizes in multiples of 128, N, K, scale spread); N and K multiples of 16
WG_MX_TM_CASES = [
    ([128, 0, 384, 256], 272, 144, 2),
    ([1024], 528, 272, 1),
    ([0, 128], 16, 16, 0),
    ([128, 128, 128, 128, 128, 0, 640], 256, 256, 1),
    ([2048, 128, 0, 256], 144, 528, 3),
    ([384, 256], 1040, 48, 1),
]


@pytest.mark.parametrize("case", range(len(WG_MX_TM_CASES)))
@pytest.mark.parametrize("accumulate", [False, True])
def test_wgrad_mx_token_major(case, accumulate):
    """kgemm_wgrad_mx_tm on dY [M, N] and X [M, K] codes as the layer holds
    them: within the oracle's MXFP8 gate, and bitwise equal to kgemm_wgrad_mx
    on the transposed codes with the same scales (empty experts, a stage of
    rows owned by no expert, ragged N and K)."""
    sizes, N, K, spread = WG_MX_TM_CASES[case]
    _say("wgrad_mx_tm", sizes, N, K, spread, "accumulate" if accumulate else "")
    off, M, dyt8, dyts, xt8, xts = _wg_inputs(sizes, N, K, spread, 50 + case)
    E = len(sizes)
    prior = None
    outs = []
    for _ in range(2):
        if accumulate:
            prior = np.random.default_rng(case).standard_normal((E, N, K)).astype(np.float32)
            outs.append(torch.from_numpy(prior.copy()).cuda())
        else:
            outs.append(torch.full((E, N, K), float("nan"), dtype=torch.float32, device="cuda"))
    bd, bx = _u8(mx_scales_blocked(dyts)), _u8(mx_scales_blocked(xts))
    o = dev_i32(off)
    mg.wgrad_mx_tm(_u8(np.ascontiguousarray(dyt8.T)), bd, _u8(np.ascontiguousarray(xt8.T)), bx,
                   o, E, out=outs[0], accumulate=accumulate)
    mg.wgrad_mx(_u8(dyt8), bd, _u8(xt8), bx, o, E, out=outs[1], accumulate=accumulate)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32)), \
        "token-major result differs from the transposed-operand one"
    rep = _wg_gate(off, dyt8, dyts, xt8, xts, outs[0].cpu().numpy(),
                   prior=None if prior is None else prior.astype(np.float64))
    assert rep.passed, str(rep)


def test_wgrad_mx_token_major_rejects_bad_shapes():
    z = lambda *sh: torch.zeros(sh, dtype=torch.uint8, device="cuda")
    with pytest.raises(mg.MgemmError):        # N = 24 is not a multiple of 16
        mg.wgrad_mx_tm(z(128, 24), z(1, 24, 4), z(128, 16), z(1, 16, 4),
                       dev_i32(offsets_from_sizes([128])), 1)


@pytest.mark.parametrize("name", ["a3b_zipf_gw13", "a3b_zipf_gw2"])
def test_a3b_zipf_wgrad_mx_token_major(name):
    """The skewed 30B-A3B weight gradients on token-major MXFP8 operands:
    bitwise equal to the transposed-operand call on every element."""
    (wl,) = make_workload(5, name)
    sizes = [((int(s) + 127) // 128) * 128 for s in wl.sizes()]
    off = offsets_from_sizes(sizes)
    M, N, K, E = int(off[-1]), wl.N, wl.K, wl.E
    _say("a3b wgrad mx token-major", name, M, N, K, E)
    dyt8 = mx_e4m3_codes((N, M), 8600, wl.tag, 1)
    xt8 = mx_e4m3_codes((K, M), 8600, wl.tag, 2)
    bd = _u8(mx_scales_blocked(mx_e8m0_codes((N, M // 32), 121, 1, 8600, wl.tag, 3)))
    bx = _u8(mx_scales_blocked(mx_e8m0_codes((K, M // 32), 121, 1, 8600, wl.tag, 4)))
    o = dev_i32(off)
    a = mg.wgrad_mx_tm(_u8(np.ascontiguousarray(dyt8.T)), bd, _u8(np.ascontiguousarray(xt8.T)),
                       bx, o, E, out=torch.full((E, N, K), float("nan"), device="cuda"))
    b = mg.wgrad_mx(_u8(dyt8), bd, _u8(xt8), bx, o, E)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("name", ["a3b_zipf_gw13", "a3b_zipf_gw2"])
def test_a3b_zipf_wgrad_mx_sampled(name):
    """The skewed 30B-A3B weight gradients with MXFP8 operands, experts padded
    to whole 128-token stages: sampled elements against the oracle, empty
    experts exactly zero."""
    (wl,) = make_workload(5, name)
    sizes = [((int(s) + 127) // 128) * 128 for s in wl.sizes()]
    off = offsets_from_sizes(sizes)
    M, N, K, E = int(off[-1]), wl.N, wl.K, wl.E
    _say("a3b wgrad mx", name, M, N, K, E)
    dyt8 = mx_e4m3_codes((N, M), 8500, wl.tag, 1)
    xt8 = mx_e4m3_codes((K, M), 8500, wl.tag, 2)
    dyts = mx_e8m0_codes((N, M // 32), 121, 1, 8500, wl.tag, 3)
    xts = mx_e8m0_codes((K, M // 32), 121, 1, 8500, wl.tag, 4)
    dw = mg.wgrad_mx(_u8(dyt8), _u8(mx_scales_blocked(dyts)), _u8(xt8),
                     _u8(mx_scales_blocked(xts)), dev_i32(off), E)
    got = dw.cpu().numpy()
    sz = np.asarray(sizes)
    assert (got[sz == 0] == 0).all()
    rng = np.random.default_rng(8501)
    live = np.flatnonzero(sz > 0)
    es = np.concatenate([rng.choice(live, 384), live, live])
    ns = np.concatenate([rng.integers(0, N, 384), np.zeros_like(live), np.full_like(live, N - 1)])
    ks = np.concatenate([rng.integers(0, K, 384), np.full_like(live, K - 1), np.zeros_like(live)])
    val, mag = sample_wgrad_mx(dyt8, dyts, xt8, xts, off, es, ns, ks)
    k_red = np.maximum(sz[es], 1)
    rep = check_fp32_mx(got[es, ns, ks], val, mag, k_red)
    assert rep.passed, str(rep)


def test_mx_dgrad_is_forward_on_requantized_transposed_weights():
    """The MXFP8 input gradient dX = dY W_e as the forward call: dY quantized
    along N, the weights stored transposed [E, K, N] and quantized along N.
    Checked against the oracle's grouped dgrad definition on the dequantized
    values (W_e = the transpose of the dequantized [K, N] matrix)."""
    from oracle import grouped_dgrad
    sizes, N, K = [200, 0, 137, 300], 256, 264
    off = offsets_from_sizes(sizes)
    M, E = int(off[-1]), len(sizes)
    _say("mx dgrad via forward", sizes, N, K)
    dy8 = mx_e4m3_codes((M, N), 8600, 1)
    dys = mx_e8m0_codes((M, N // 32), 121, 1, 8600, 2)
    wt8 = mx_e4m3_codes((E, K, N), 8600, 3)
    wts = mx_e8m0_codes((E, K, N // 32), 121, 1, 8600, 4)
    dx = mg.fwd_mx(_u8(dy8), _u8(mx_scales_blocked(dys)), _u8(wt8), _u8(mx_scales_blocked(wts)),
                   dev_i32(off), out=sentinel_bf16((M, K)))
    got = host_bits(dx)
    dyv = mx_dequant(dy8, dys)
    w = np.ascontiguousarray(np.transpose(mx_dequant(wt8, wts), (0, 2, 1)))   # [E, N, K]
    exact = grouped_dgrad(dyv, w, off)
    mag = grouped_dgrad(np.abs(dyv), np.abs(w), off)
    rep = check_bf16_mx(got, exact, mag)
    assert rep.passed, str(rep)


def test_mx_longest_reductions_sampled():
    """The MXFP8 forward with K = 2^22 (32768 stages of 128 fp8 steps in one
    tile) and the MXFP8 weight gradient over 2^22 tokens, two experts each,
    sampled against the oracle under the MX gates."""
    R = 1 << 22
    rng = np.random.default_rng(8800)
    off = offsets_from_sizes([24, 16])
    M, N = int(off[-1]), 16
    _say("mx longest reductions: fwd K", R)
    x8 = mx_e4m3_codes((M, R), 8800, 1)
    w8 = mx_e4m3_codes((2, N, R), 8800, 2)
    xs = mx_e8m0_codes((M, R // 32), 121, 1, 8800, 3)
    ws = mx_e8m0_codes((2, N, R // 32), 121, 1, 8800, 4)
    got = _run(off, M, N, x8, w8, xs, ws)
    rows = np.arange(M)
    cols = rng.integers(0, N, M)
    val, mag = sample_fwd_mx(x8, xs, w8, ws, off, rows, cols)
    rep = check_bf16_mx(got[rows, cols], val, mag)
    assert rep.passed, f"fwd: {rep}"
    del x8, w8, xs, ws
    _say("mx longest reductions: wgrad tokens", R)
    off2 = offsets_from_sizes([R - 1024, 1024])
    K = 24
    dyt8 = mx_e4m3_codes((N, R), 8800, 5)
    xt8 = mx_e4m3_codes((K, R), 8800, 6)
    dyts = mx_e8m0_codes((N, R // 32), 121, 1, 8800, 7)
    xts = mx_e8m0_codes((K, R // 32), 121, 1, 8800, 8)
    dw = mg.wgrad_mx(_u8(dyt8), _u8(mx_scales_blocked(dyts)), _u8(xt8),
                     _u8(mx_scales_blocked(xts)), dev_i32(off2), 2)
    torch.cuda.synchronize()
    got = dw.cpu().numpy()
    es = np.repeat(np.arange(2), 24)
    ns = rng.integers(0, N, es.size)
    ks = rng.integers(0, K, es.size)
    val, mag = sample_wgrad_mx(dyt8, dyts, xt8, xts, off2, es, ns, ks)
    k_red = np.maximum(np.diff(np.asarray(off2, np.int64))[es], 1)
    rep = check_fp32_mx(got[es, ns, ks], val, mag, k_red)
    assert rep.passed, f"wgrad: {rep}"


# ------------------------------------------------ exact small-integer cases --
# Codes of integers in [-3, 3], each row of X and of W (each row of dY^T and
# X^T in the weight gradient) scaled by one power of two along its whole
# reduction axis.  The products that make one output element are then integers
# times one common power of two, and every partial sum is at most 9 x (the
# reduction length) of those units: fewer than 24 significant bits, and fewer
# than 10 within one matrix-core instruction.  Any summation order is exact, so
# the kernels owe the exact value itself: fp32 outputs bit for bit, bf16 outputs
# its round to nearest even, with no tolerance.  A scale taken from the wrong
# row or column, or a code from the wrong place, changes the bits.

from oracle import f64_to_bf16_bits  # noqa: E402
from workloads.synth import mx_e8m0_pair_codes, mx_e8m0_row_codes, mx_small_int_codes  # noqa: E402

MX_EXACT_FWD = [([300, 0, 17, 513], 264, 2048), ([1, 255, 257], 136, 96), ([700], 520, 416)]


def _fwd_exact_inputs(sizes, N, K, seed):
    off = offsets_from_sizes(sizes)
    M, E = int(off[-1]), len(sizes)
    x8 = mx_small_int_codes((M, K), 8900, seed, 1)
    w8 = mx_small_int_codes((E, N, K), 8900, seed, 2)
    xs = mx_e8m0_row_codes(M, K // 32, 127, 6, 8900, seed, 3)
    ws = mx_e8m0_row_codes(E * N, K // 32, 127, 6, 8900, seed, 4).reshape(E, N, K // 32)
    return off, M, x8, w8, xs, ws


@pytest.mark.parametrize("case", range(len(MX_EXACT_FWD)))
def test_fwd_mx_exact_on_small_integers(case):
    sizes, N, K = MX_EXACT_FWD[case]
    _say("fwd_mx exact", sizes, N, K)
    off, M, x8, w8, xs, ws = _fwd_exact_inputs(sizes, N, K, case)
    got = _run(off, M, N, x8, w8, xs, ws)
    want = f64_to_bf16_bits(grouped_fwd_mx(x8, xs, w8, ws, off))
    bad = int((got != want).sum())
    assert bad == 0, f"{bad} of {got.size} elements differ from the rounded exact value"


@pytest.mark.parametrize("name", ["a3b_gate_up", "a3b_down"])
def test_a3b_mx_exact_whole_tensor(name):
    """The 30B-A3B expert shapes in the launch the bench times, every element
    of the output equal to the round to nearest even of the exact value."""
    (wl,) = make_workload(4, name)
    off = np.asarray(wl.offsets)
    M, N, K, E = wl.M, wl.N, wl.K, wl.E
    _say("a3b mx exact", name, M, N, K, E)
    x8 = mx_small_int_codes((M, K), 8910, 1)
    w8 = mx_small_int_codes((E, N, K), 8910, 2)
    xs = mx_e8m0_row_codes(M, K // 32, 127, 6, 8910, 3)
    ws = mx_e8m0_row_codes(E * N, K // 32, 127, 6, 8910, 4).reshape(E, N, K // 32)
    got = _run(off, M, N, x8, w8, xs, ws)
    last = int(off[-1])
    assert (got[last:] == SENTINEL).all()
    want = f64_to_bf16_bits(grouped_fwd_mx(x8, xs, w8, ws, off)[:last])
    bad = int((got[:last] != want).sum())
    assert bad == 0, f"{bad} of {want.size} elements differ from the rounded exact value"


MX_EXACT_WG = [([128, 0, 384, 1024], 272, 144), ([2048, 128, 0, 256], 144, 528)]   # N, K: x16


@pytest.mark.parametrize("case", range(len(MX_EXACT_WG)))
def test_wgrad_mx_exact_on_small_integers(case):
    """Both MXFP8 weight-gradient calls (transposed and token-major operands)
    equal to the exact fp32 value on every element; empty experts exactly 0."""
    sizes, N, K = MX_EXACT_WG[case]
    off = offsets_from_sizes(sizes)
    M, E = int(off[-1]) + 128, len(sizes)
    _say("wgrad_mx exact", sizes, N, K)
    dyt8 = mx_small_int_codes((N, M), 8920, case, 1)
    xt8 = mx_small_int_codes((K, M), 8920, case, 2)
    dyts = mx_e8m0_row_codes(N, M // 32, 127, 6, 8920, case, 3)
    xts = mx_e8m0_row_codes(K, M // 32, 127, 6, 8920, case, 4)
    exact = grouped_wgrad_mx(dyt8, dyts, xt8, xts, off, E)
    assert (exact.astype(np.float32).astype(np.float64) == exact).all()
    bd, bx = _u8(mx_scales_blocked(dyts)), _u8(mx_scales_blocked(xts))
    o = dev_i32(off)
    a = mg.wgrad_mx(_u8(dyt8), bd, _u8(xt8), bx, o, E,
                    out=torch.full((E, N, K), float("nan"), device="cuda"))
    b = mg.wgrad_mx_tm(_u8(np.ascontiguousarray(dyt8.T)), bd, _u8(np.ascontiguousarray(xt8.T)),
                       bx, o, E, out=torch.full((E, N, K), float("nan"), device="cuda"))
    torch.cuda.synchronize()
    for got, what in ((a.cpu().numpy(), "transposed"), (b.cpu().numpy(), "token-major")):
        bad = int((got.astype(np.float64) != exact).sum())
        assert bad == 0, f"{what}: {bad} of {got.size} elements differ from the exact value"


def test_fwd_mx_exact_with_block_scales_along_the_reduction():
    """Small-integer codes with every 32-block scaled by 2^0 or 2^1 at random
    (X and W): each product is an integer, every partial sum at most 36 K,
    inside one instruction at most 2304 -- still exact in any order.  The
    rounded exact value is owed bit for bit, which pins the addressing of the
    block scales along K (a block scale from the wrong block is off by 2x)."""
    sizes, N, K = [300, 0, 17, 513], 264, 1024
    off = offsets_from_sizes(sizes)
    M, E = int(off[-1]), len(sizes)
    _say("fwd_mx exact, block scales along K", sizes, N, K)
    x8 = mx_small_int_codes((M, K), 8930, 1)
    w8 = mx_small_int_codes((E, N, K), 8930, 2)
    xs = mx_e8m0_pair_codes((M, K // 32), 127, 8930, 3)
    ws = mx_e8m0_pair_codes((E, N, K // 32), 127, 8930, 4)
    got = _run(off, M, N, x8, w8, xs, ws)
    want = f64_to_bf16_bits(grouped_fwd_mx(x8, xs, w8, ws, off))
    bad = int((got != want).sum())
    assert bad == 0, f"{bad} of {got.size} elements differ from the rounded exact value"


def test_wgrad_mx_exact_with_block_scales_along_the_tokens():
    """The same for both MXFP8 weight-gradient calls: 32-token blocks scaled
    by 2^0 or 2^1 at random, the exact fp32 value owed on every element."""
    sizes, N, K = [128, 0, 384, 1024], 272, 144
    off = offsets_from_sizes(sizes)
    M, E = int(off[-1]) + 128, len(sizes)
    _say("wgrad_mx exact, block scales along the tokens", sizes, N, K)
    dyt8 = mx_small_int_codes((N, M), 8940, 1)
    xt8 = mx_small_int_codes((K, M), 8940, 2)
    dyts = mx_e8m0_pair_codes((N, M // 32), 127, 8940, 3)
    xts = mx_e8m0_pair_codes((K, M // 32), 127, 8940, 4)
    exact = grouped_wgrad_mx(dyt8, dyts, xt8, xts, off, E)
    assert (exact.astype(np.float32).astype(np.float64) == exact).all()
    bd, bx = _u8(mx_scales_blocked(dyts)), _u8(mx_scales_blocked(xts))
    o = dev_i32(off)
    a = mg.wgrad_mx(_u8(dyt8), bd, _u8(xt8), bx, o, E,
                    out=torch.full((E, N, K), float("nan"), device="cuda"))
    b = mg.wgrad_mx_tm(_u8(np.ascontiguousarray(dyt8.T)), bd, _u8(np.ascontiguousarray(xt8.T)),
                       bx, o, E, out=torch.full((E, N, K), float("nan"), device="cuda"))
    torch.cuda.synchronize()
    for got, what in ((a.cpu().numpy(), "transposed"), (b.cpu().numpy(), "token-major")):
        bad = int((got.astype(np.float64) != exact).sum())
        assert bad == 0, f"{what}: {bad} of {got.size} elements differ from the exact value"
