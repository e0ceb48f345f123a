"""Benchmark of the MoE grouped GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole path over one batch of seeded synthetic
input: the M-grouped forward Y = X W_e^T, the M-grouped input gradient
dX = dY W_e and the K-grouped fp32 weight gradient dW_e = dY_e^T X_e, each one
launch of libmgemm.so.  The default workload is one GPU's expert share of the
30B-A3B layout (RapidGEMM README, *Model layout* / *Settings*: 32 local experts,
d_model 3072, expert FFN 1280): the forward and input gradient of the gate-up
(K 3072 -> N 2560) and down (K 1280 -> N 3072) GEMMs on router-assigned rows,
and both weight gradients (gw13, gw2) on the Zipf-skewed split -- six launches
per step.  `--workload uniform_g8` / `uniform_g16` run the grouped-GEMM shapes
of the TransformerEngine PR #2045 perf table instead, (g, m, n, k) =
(8, 4096, 768, 2048) / (16, 2048, 768, 2048).

Prints ONE JSON line: whole-step TFLOP/s (algorithmic flops 2*M*N*K per op,
M = rows owned by experts), the fraction of the bf16 dense matrix-core peak,
per-op HIP-event timings (warm, and with the L2 and the Infinity Cache flushed
before every launch: the flushed median is each op's headline), each op's
fraction of the peak beside its target, the roofline entry of the dominant
kernel and the oracle's CPU time on the host's cores.  Inputs are resident in HBM before
the timed region; nothing is skipped inside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0        # MI355X published dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0         # MI355X published dense fp8 matrix-core peak
BF16_FLOP_PER_CLK = 256 * 4096   # 256 CUs x 4096 dense bf16 flop per clock and CU
KERNEL_SRC = os.path.join(ROOT, "moe_grouped_gemm_bf16_amd", "csrc", "mgemm_kernels.hip")
KERNEL_NAMES = {"fwd": "grouped_gemm_kernel<0>", "dgrad": "grouped_gemm_kernel<1>",
                "wgrad": "grouped_gemm_kernel<2>", "fwd_swiglu": "grouped_gemm_kernel<3>",
                "list": "grouped_gemm_kernel<4>", "fwd_mx": "grouped_gemm_kernel<5>",
                "wgrad_mx": "grouped_gemm_kernel<6>", "dgrad_swiglu": "grouped_gemm_kernel<7>",
                "wgrad_mx_tm": "grouped_gemm_kernel<8>"}


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="a3b", choices=["a3b", "uniform_g8", "uniform_g16"])
    p.add_argument("--no-clock", action="store_true",
                   help="skip the clock sampling phase after the timed steps (profiler runs)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle timing (used for profiler passes)")
    p.add_argument("--cold", type=int, default=50,
                   help="time each op N times after flushing the caches (0: skip)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one plain 1 GiB device copy (for HBM counter calibration)")
    p.add_argument("--comparators", action="store_true",
                   help="also time library baselines on the same inputs (reported only)")
    p.add_argument("--lists", action="store_true",
                   help="also time the descriptor-list call against the M-grouped one "
                        "(reported only)")
    p.add_argument("--fusions", action="store_true",
                   help="also time the gate-up forward with gathered rows and fused SwiGLU "
                        "against the unfused sequence (reported only)")
    p.add_argument("--mx", action="store_true",
                   help="also time the MXFP8 grouped forward against the bf16 one on the same "
                        "shapes (reported only)")
    p.add_argument("--ceiling", action="store_true",
                   help="also run the matrix-core ceiling probe (libmgemm_probe.so): the rate "
                        "of the bf16 products alone, no memory traffic (reported only)")
    return p.parse_args()


# ------------------------------------------------------------------ workload --

class Op:
    """One launch of the path: a name, its workload, a launcher and its flops."""

    def __init__(self, name, kind, wl, launch, flops, bytes_, tensors=None):
        self.name, self.kind, self.wl, self.launch = name, kind, wl, launch
        self.flops, self.bytes = flops, bytes_
        self.tensors = tensors or {}
        self.times_ms = []


def build_ops(workload: str, torch, mg):
    from workloads import make_workload

    def up(bits):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    ops, inputs = [], []
    if workload == "a3b":
        mg_wls = make_workload(4)          # gate-up and down, router-assigned rows
        wg_wls = make_workload(5)          # gw13 and gw2, Zipf split
    else:
        cfg = 2 if workload == "uniform_g8" else 3
        mg_wls = make_workload(cfg)
        wg_wls = mg_wls
    for wl in mg_wls:
        x, w, dy = up(wl.x_bits()), up(wl.w_bits()), up(wl.dy_bits())
        off = torch.from_numpy(wl.offsets).cuda()
        y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
        dx = torch.empty((wl.M, wl.K), dtype=torch.bfloat16, device="cuda")
        hint = int(wl.sizes().max())
        rows = wl.rows
        ab = 2 * (rows * wl.K + wl.E * wl.N * wl.K + rows * wl.N)   # read X, W; write Y
        ops.append(Op(f"fwd:{wl.name}", "fwd", wl,
                      (lambda x=x, w=w, off=off, y=y, h=hint: mg.fwd(x, w, off, h, out=y)),
                      wl.flops(), ab, dict(a=x, w=w, off=off)))
        ops.append(Op(f"dgrad:{wl.name}", "dgrad", wl,
                      (lambda dy=dy, w=w, off=off, dx=dx, h=hint: mg.dgrad(dy, w, off, h, out=dx)),
                      wl.flops(), ab, dict(a=dy, w=w, off=off)))
        inputs.append((x, w, dy, off, y, dx))
    for wl in wg_wls:
        if workload == "a3b" or "wgrad" in wl.ops:
            if workload == "a3b":
                x, dy = up(wl.x_bits()), up(wl.dy_bits())
                off = torch.from_numpy(wl.offsets).cuda()
            else:
                x, _, dy, off, _, _ = inputs[0]
            dw = torch.empty((wl.E, wl.N, wl.K), dtype=torch.float32, device="cuda")
            rows = wl.rows
            ab = 2 * rows * (wl.N + wl.K) + 4 * wl.E * wl.N * wl.K        # read dY, X; write fp32 dW
            ops.append(Op(f"wgrad:{wl.name}", "wgrad", wl,
                          (lambda dy=dy, x=x, off=off, dw=dw: mg.wgrad(dy, x, off, out=dw)),
                          wl.flops(), ab, dict(dy=dy, x=x, off=off)))
            inputs.append((x, dy, off, dw))
    return ops, inputs


# -------------------------------------------------------------- comparators --

def comparators(ops, torch, reps=20):
    """Library baselines on the same device inputs, reported beside the kernels
    (never part of `value`): a loop of one hipBLASLt GEMM per expert (torch 2-D
    matmul, the analogue of the multi-stream per-group baseline of the
    TransformerEngine PR #2045 perf table) and torch._grouped_mm where this torch
    has it.  Operands that the libraries want in the other orientation are made
    contiguous before the timed region.  Both emit bf16 for wgrad (the kernel
    under test writes fp32).  Each is timed with the host's enqueue hidden
    (`us`, the GPU's time) and back to back (`us_host_inclusive`)."""
    out = {}
    for op in ops:
        t, o = op.tensors, [int(v) for v in op.wl.offsets]
        E = len(o) - 1
        spans = [(e, o[e], o[e + 1]) for e in range(E) if o[e + 1] > o[e]]
        ends = t["off"][1:].contiguous()
        rec = {}
        if op.kind == "fwd":
            wt = t["w"].transpose(1, 2).contiguous()          # [E, K, N]
            a = t["a"]
            loop = lambda: [torch.matmul(a[i:j], wt[e]) for e, i, j in spans]
            grp = lambda: torch._grouped_mm(a, wt, offs=ends)
        elif op.kind == "dgrad":
            w, a = t["w"], t["a"]
            loop = lambda: [torch.matmul(a[i:j], w[e]) for e, i, j in spans]
            grp = lambda: torch._grouped_mm(a, w, offs=ends)
        else:
            dyt, x = t["dy"].t().contiguous(), t["x"]           # dY^T [N, M]
            loop = lambda: [torch.matmul(dyt[:, i:j], x[i:j]) for e, i, j in spans]
            grp = lambda: torch._grouped_mm(dyt, x, offs=ends)
        th, us = time_library(torch, loop, reps)
        rec["hipblaslt_per_expert_loop"] = {"us": round(us, 1), "us_host_inclusive": round(th, 1),
                                            "tflops": round(op.flops / us / 1e6, 1)}
        if hasattr(torch, "_grouped_mm"):
            try:
                th, us = time_library(torch, grp, reps)
                rec["torch_grouped_mm"] = {"us": round(us, 1), "us_host_inclusive": round(th, 1),
                                           "tflops": round(op.flops / us / 1e6, 1)}
            except Exception as exc:                       # not supported by this PyTorch
                rec["torch_grouped_mm"] = {"error": f"{type(exc).__name__}: {str(exc)[:120]}"}
        if op.kind == "wgrad":
            rec["note"] = "comparators write bf16 dW; the kernel writes fp32"
        out[op.name] = rec
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ fusions --

def fusions(torch, mg, reps=20):
    """The 30B-A3B share's gate-up GEMM as a trainer runs it: 16384 token rows
    x [16384, 3072] gathered by the router's row-to-token map into 32 expert
    groups, w13 [32, 2560, 3072], SwiGLU: h [M, 1280].  Fused: one
    mgemm_fwd_swiglu launch.  Unfused: torch index_select of the rows, the
    plain grouped forward to [M, 2560], torch silu(g) * u.  Reported beside
    the step, never part of `value`."""
    import numpy as np
    from workloads import make_workload, normal_bf16_bits
    from workloads.synth import router_offsets
    off_np, tok = router_offsets(16384, 128, 8, 32, seed=4)
    (wl,) = [w for w in make_workload(4) if w.name == "a3b_gate_up"]
    T, K, I = 16384, 3072, 1280
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    x, w13 = up(normal_bf16_bits((T, K), 1.0, 4, 9, 1)), up(wl.w_bits())
    off = torch.from_numpy(off_np).cuda()
    gi = torch.from_numpy(tok).cuda()
    gl = gi.long()
    M = int(off_np[-1])
    hint = int(np.diff(off_np).max())
    h = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda")

    def fused():
        mg.fwd_swiglu(x, w13, off, gather=gi, max_m_per_e=hint, out=h)

    def unfused():
        xg = x.index_select(0, gl)
        mg.fwd(xg, w13, off, hint, out=y)
        torch.nn.functional.silu(y[:, :I]) * y[:, I:]

    # the two are timed interleaved (one of each per round), so that both see
    # the same clock and cache state
    for _ in range(5):
        fused()
        unfused()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(2)] for _ in range(reps)]
    for pair in ev:
        for (a, b), fn in zip(pair, (fused, unfused)):
            a.record()
            fn()
            b.record()
    torch.cuda.synchronize()
    tf = statistics.median(p[0][0].elapsed_time(p[0][1]) for p in ev) * 1e3
    tu = statistics.median(p[1][0].elapsed_time(p[1][1]) for p in ev) * 1e3
    flops = 2 * M * (2 * I) * K
    out = {"fwd_swiglu_gathered:a3b_gate_up": {
        "rows": M, "tokens": T, "fused_us": round(tf, 1), "tflops": round(flops / tf / 1e6, 1),
        "pct_peak": round(100 * flops / tf / 1e6 / PEAK_BF16_TFLOPS, 1),
        "unfused_us": round(tu, 1), "speedup": round(tu / tf, 3),
        "unfused": "torch index_select + mgemm_fwd [M, 2560] + torch silu(g) * u"}}

    # the backward through the down projection: dh = dy W2[e] with the SwiGLU
    # backward fused (dgu [M, 2I]) against mgemm_dgrad to dh and the same
    # activation backward in torch; and the fused forward saving g | u
    (wd,) = [w for w in make_workload(4) if w.name == "a3b_down"]
    N = wd.N
    dy = up(normal_bf16_bits((M, N), 1.0, 4, 9, 2))
    w2 = up(wd.w_bits())
    gu = torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda")
    mg.fwd_swiglu(x, w13, off, gather=gi, max_m_per_e=hint, out=h, gu_out=gu)
    dgu = torch.empty_like(gu)
    dh = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")

    def bfused():
        mg.dgrad_swiglu(dy, w2, gu, off, hint, out=dgu)

    def bunfused():
        mg.dgrad(dy, w2, off, hint, out=dh)
        g = gu[:, :I].float(); u = gu[:, I:].float(); d = dh.float()
        sg = torch.sigmoid(g)
        torch.cat([d * u * sg * (1 + g * (1 - sg)), d * g * sg], dim=1).to(torch.bfloat16)

    def fsave():
        mg.fwd_swiglu(x, w13, off, gather=gi, max_m_per_e=hint, out=h, gu_out=gu)

    pairs = (("dgrad_swiglu:a3b_down", bfused, bunfused, 2 * M * N * I,
              "mgemm_dgrad to dh [M, 1280] + torch SwiGLU backward"),
             ("fwd_swiglu_saving_gu:a3b_gate_up", fsave, fused, flops,
              "the same fused forward without saving g | u"))
    for name, fa, fb, fl, what in pairs:
        for _ in range(5):
            fa(); fb()
        torch.cuda.synchronize()
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(2)] for _ in range(reps)]
        for pair in ev:
            for (a, b), fn in zip(pair, (fa, fb)):
                a.record()
                fn()
                b.record()
        torch.cuda.synchronize()
        ta = statistics.median(p[0][0].elapsed_time(p[0][1]) for p in ev) * 1e3
        tb = statistics.median(p[1][0].elapsed_time(p[1][1]) for p in ev) * 1e3
        out[name] = {"fused_us": round(ta, 1), "tflops": round(fl / ta / 1e6, 1),
                     "pct_peak": round(100 * fl / ta / 1e6 / PEAK_BF16_TFLOPS, 1),
                     "reference_us": round(tb, 1), "ratio": round(tb / ta, 3),
                     "reference": what}
    # the token-order combine (the gather's inverse): the gate-up input gradient
    # rows [M, 3072] summed back per token, unweighted and with router weights;
    # HBM-bound, reported against the 8 TB/s roofline
    tr = -np.ones((T, 8), np.int32)
    fill = np.zeros(T, np.int64)
    for i, t in enumerate(tok):
        tr[t, fill[t]] = i
        fill[t] += 1
    trd = torch.from_numpy(tr).cuda()
    wts = torch.rand((T, 8), device="cuda")
    rows = up(normal_bf16_bits((M, K), 1.0, 4, 9, 3))
    xo = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    for name, fn, extra in (("moe_combine:a3b_dx", lambda: mg.moe_combine(rows, trd, out=xo), 0),
                            ("moe_combine_weighted:a3b_y",
                             lambda: mg.moe_combine(rows, trd, wts, out=xo), T * 8 * 4)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        tc = statistics.median(a.elapsed_time(b) for a, b in ev) * 1e3
        nbytes = M * K * 2 + T * 8 * 4 + T * K * 2 + extra
        out[name] = {"us": round(tc, 1), "algo_GBps": round(nbytes / tc / 1e3, 1),
                     "pct_hbm": round(100 * nbytes / tc / 1e3 / PEAK_HBM_GBS, 1),
                     "rows": M, "tokens": T}
    return out


# -------------------------------------------------------------------- lists --

def lists(torch, mg, reps=20):
    """The descriptor-list call (one launch over per-group pointers and shapes)
    on the 30B-A3B share: (1) the gate-up forward as 32 per-expert groups
    against the M-grouped call on the same data; (2) gate-up and down forwards
    of all 32 experts mixed in one 64-group launch against two M-grouped
    launches; (3) on uniform_g8, M- and K-grouped problems in one launch: the
    8 experts' forwards and their weight gradients (dW_e = dY_e^T X_e on
    token-axis-last copies of dY and X, made before the timed region; bf16
    results) against the M-grouped forward plus the K-grouped weight gradient
    (fp32 results).  Timed interleaved; reported beside the step only."""
    import numpy as np
    from workloads import make_workload
    wls = {w.name: w for w in make_workload(4)}
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    ins = {}
    for name in ("a3b_gate_up", "a3b_down"):
        wl = wls[name]
        off = [int(v) for v in wl.offsets]
        x, w = up(wl.x_bits()), up(wl.w_bits())
        y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
        groups = [(x[off[e]:off[e + 1]], w[e]) for e in range(wl.E)]
        outs = [y[off[e]:off[e + 1]] for e in range(wl.E)]
        ins[name] = (wl, x, w, torch.from_numpy(wl.offsets).cuda(), y, groups, outs,
                     int(wl.sizes().max()))
    gu, dn = ins["a3b_gate_up"], ins["a3b_down"]
    d_gu = mg.list_descriptors(gu[5], gu[6])
    d_mix = mg.list_descriptors(gu[5] + dn[5], gu[6] + dn[6])
    (wu,) = make_workload(2)
    ou = [int(v) for v in wu.offsets]
    xu, wwu, dyu = up(wu.x_bits()), up(wu.w_bits()), up(wu.dy_bits())
    xut, dyut = xu.t().contiguous(), dyu.t().contiguous()
    yu = torch.empty((wu.M, wu.N), dtype=torch.bfloat16, device="cuda")
    dwu = torch.empty((wu.E, wu.N, wu.K), dtype=torch.bfloat16, device="cuda")
    dwu32 = torch.empty((wu.E, wu.N, wu.K), dtype=torch.float32, device="cuda")
    offu = torch.from_numpy(wu.offsets).cuda()
    mk_groups, mk_outs = [], []
    for e in range(wu.E):
        mk_groups += [(xu[ou[e]:ou[e + 1]], wwu[e]), (dyut[:, ou[e]:ou[e + 1]], xut[:, ou[e]:ou[e + 1]])]
        mk_outs += [yu[ou[e]:ou[e + 1]], dwu[e]]
    d_mk = mg.list_descriptors(mk_groups, mk_outs)
    cases = {
        "gate_up_32_groups": (lambda: mg.grouped_list_desc(d_gu, 32),
                              lambda: mg.fwd(gu[1], gu[2], gu[3], gu[7], out=gu[4]),
                              gu[0].flops()),
        "gate_up_and_down_64_groups": (lambda: mg.grouped_list_desc(d_mix, 64),
                                       lambda: (mg.fwd(gu[1], gu[2], gu[3], gu[7], out=gu[4]),
                                                mg.fwd(dn[1], dn[2], dn[3], dn[7], out=dn[4])),
                                       gu[0].flops() + dn[0].flops()),
        "uniform_g8_fwd_and_wgrad_16_groups": (
            lambda: mg.grouped_list_desc(d_mk, 2 * wu.E),
            lambda: (mg.fwd(xu, wwu, offu, out=yu), mg.wgrad(dyu, xu, offu, wu.E, out=dwu32)),
            2 * wu.flops()),
    }
    out = {}
    for name, (fl, fm, flops) in cases.items():
        for _ in range(5):
            fl(); fm()
        torch.cuda.synchronize()
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(2)] for _ in range(reps)]
        for pair in ev:
            for (a, b), fn in zip(pair, (fl, fm)):
                a.record()
                fn()
                b.record()
        torch.cuda.synchronize()
        tl = statistics.median(p[0][0].elapsed_time(p[0][1]) for p in ev) * 1e3
        tm = statistics.median(p[1][0].elapsed_time(p[1][1]) for p in ev) * 1e3
        out[name] = {"list_us": round(tl, 1), "tflops": round(flops / tl / 1e6, 1),
                     "pct_peak": round(100 * flops / tl / 1e6 / PEAK_BF16_TFLOPS, 1),
                     "mgrouped_us": round(tm, 1), "ratio": round(tm / tl, 3)}
    return out


# ----------------------------------------------------------------------- mx --

def time_alone(torch, fn, reps, warm=3, hide_host=False):
    """Median HIP-event time (us) of fn launched on its own.  By default the
    launches go back to back, so a library loop's host cost between its
    launches is part of its time; with hide_host each repetition is enqueued
    behind a GPU sleep of ~10 ms (torch.cuda._sleep), so that the host has
    queued the whole loop before the first event runs and the time is the
    GPU's alone."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if hide_host:
            torch.cuda.synchronize()
            torch.cuda._sleep(20_000_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in ts) * 1e3


def time_library(torch, fn, reps):
    """A library loop's time two ways: back to back (host cost included) and
    with the host's enqueue hidden (the GPU's time alone)."""
    host = time_alone(torch, fn, reps)
    gpu = time_alone(torch, fn, reps, hide_host=hasattr(torch.cuda, "_sleep"))
    return host, gpu


def per_expert_scaled_mm(torch, x8, xs, w8, ws, offsets):
    """A loop of torch._scaled_mm calls, one per non-empty expert, on MXFP8
    codes with E8M0 scales per 32 reduction steps (uint8 [rows, K/32]).
    Returns {"fn": the loop, "compare": a function of the grouped call's
    output giving the relative Frobenius difference from the loop's} when the
    call works here, else {"error": ...}.  Where the library refuses an
    expert's row count, each
    expert's rows are copied once (outside any timing) into a block padded
    with zero codes to a multiple of 128 rows, and the loop runs on those."""
    if not hasattr(torch, "_scaled_mm") or not hasattr(torch, "float8_e8m0fnu"):
        return {"error": "torch._scaled_mm with E8M0 scales not in this build"}
    ends = [int(v) for v in offsets]
    live = [e for e in range(len(ends) - 1) if ends[e + 1] > ends[e]]
    wf, we = w8.view(torch.float8_e4m3fn), ws.view(torch.float8_e8m0fnu)

    def run(blocks):
        return [torch._scaled_mm(xa, wf[e].t(), scale_a=sa, scale_b=we[e],
                                 out_dtype=torch.bfloat16) for e, xa, sa in blocks]

    blocks = [(e, x8[ends[e]:ends[e + 1]].view(torch.float8_e4m3fn),
               xs[ends[e]:ends[e + 1]].view(torch.float8_e8m0fnu)) for e in live]
    padded = False
    try:
        ys = run(blocks)
        torch.cuda.synchronize()
    except Exception as exc:                       # the library refuses some shapes
        first = f"{type(exc).__name__}: {str(exc)[:400]}"
        padded = True
        pb = []
        for e in live:
            m = ends[e + 1] - ends[e]
            mp = (m + 127) // 128 * 128
            xa = torch.zeros((mp, x8.shape[1]), dtype=torch.uint8, device=x8.device)
            sa = torch.full((mp, xs.shape[1]), 127, dtype=torch.uint8, device=xs.device)
            xa[:m] = x8[ends[e]:ends[e + 1]]
            sa[:m] = xs[ends[e]:ends[e + 1]]
            pb.append((e, xa.view(torch.float8_e4m3fn), sa.view(torch.float8_e8m0fnu)))
        blocks = pb
        try:
            ys = run(blocks)
            torch.cuda.synchronize()
        except Exception as exc2:
            return {"error": first, "padded_error": f"{type(exc2).__name__}: {str(exc2)[:200]}"}
    def compare(y_grouped):
        num = den = 0.0
        for e, ye in zip(live, ys):
            g = y_grouped[ends[e]:ends[e + 1]].float()
            num += float((ye[:g.shape[0]].float() - g).pow(2).sum())
            den += float(g.pow(2).sum())
        return float(f"{(num / max(den, 1e-300)) ** 0.5:.3e}")

    rec = {"fn": lambda: run(blocks), "compare": compare}
    if padded:
        rec["rows_padded_to_128"] = sum(int(xa.shape[0]) for _, xa, _ in blocks)
        rec["unpadded_error"] = first
    return rec


def per_expert_scaled_mm_wgrad(torch, dyt8, dyts, xt8, xts, offsets):
    """The MXFP8 weight gradient as a loop of torch._scaled_mm calls, one per
    non-empty expert: dW_e = DYT[:, rows_e] XT[:, rows_e]^T, on contiguous
    per-expert copies of the codes and plain E8M0 scales (made once, outside
    any timing).  The library's block-scaled path writes bf16 only, so its dW
    is bf16 where the grouped call's is fp32.  Returns {"fn": ..., "compare":
    ...} as per_expert_scaled_mm does, or {"error": ...}."""
    if not hasattr(torch, "_scaled_mm") or not hasattr(torch, "float8_e8m0fnu"):
        return {"error": "torch._scaled_mm with E8M0 scales not in this build"}
    ends = [int(v) for v in offsets]
    live = [e for e in range(len(ends) - 1) if ends[e + 1] > ends[e]]
    blocks = []
    for e in live:
        lo, hi = ends[e], ends[e + 1]
        blocks.append((e, dyt8[:, lo:hi].contiguous().view(torch.float8_e4m3fn),
                       dyts[:, lo // 32:hi // 32].contiguous().view(torch.float8_e8m0fnu),
                       xt8[:, lo:hi].contiguous().view(torch.float8_e4m3fn),
                       xts[:, lo // 32:hi // 32].contiguous().view(torch.float8_e8m0fnu)))

    def run():
        return [torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
                for _, a, sa, b, sb in blocks]

    try:
        ys = run()
        torch.cuda.synchronize()
    except Exception as exc:
        return {"error": f"{type(exc).__name__}: {str(exc)[:400]}"}
    def compare(dw_grouped):
        num = den = 0.0
        for (e, *_), ye in zip(blocks, ys):
            g = dw_grouped[e]
            num += float((ye.float() - g).pow(2).sum())
            den += float(g.pow(2).sum())
        return float(f"{(num / max(den, 1e-300)) ** 0.5:.3e}")

    return {"fn": run, "compare": compare, "out_dtype": "bf16"}


def mx(torch, mg, reps=20):
    """The MXFP8 grouped forward (E4M3 operands, E8M0 scales per 32 steps) on
    the uniform g8 shape and the 30B-A3B share's two expert GEMMs, timed
    interleaved with the bf16 forward of the same shape and with a loop of
    per-expert torch._scaled_mm calls on the same codes (the library
    comparator); plus the blocked scale layout kernel on the gate-up operands.
    Reported beside the step only (`value` is the bf16 path)."""
    import numpy as np
    from workloads import make_workload
    from workloads.synth import mx_e4m3_codes, mx_e8m0_codes
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    wls = [make_workload(2)[0]] + make_workload(4)
    out = {}
    for wl in wls:
        M, N, K, E = wl.M, wl.N, wl.K, wl.E
        off = torch.from_numpy(wl.offsets).cuda()
        hint = int(wl.sizes().max())
        x8 = u8(mx_e4m3_codes((M, K), 8300, wl.cfg, wl.tag, 1))
        w8 = u8(mx_e4m3_codes((E, N, K), 8300, wl.cfg, wl.tag, 2))
        xs = u8(mx_e8m0_codes((M, K // 32), 121, 1, 8300, wl.cfg, wl.tag, 3))
        ws = u8(mx_e8m0_codes((E, N, K // 32), 121, 1, 8300, wl.cfg, wl.tag, 4))
        bx, bw = mg.mx_scales_blocked(xs), mg.mx_scales_blocked(ws)
        x, w = up(wl.x_bits()), up(wl.w_bits())
        y8 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y = torch.empty_like(y8)
        fns = [lambda: mg.fwd_mx(x8, bx, w8, bw, off, hint, out=y8),
               lambda: mg.fwd(x, w, off, hint, out=y),
               lambda: (mg.mx_scales_blocked(xs, out=bx), mg.mx_scales_blocked(ws, out=bw))]
        # library comparator: one torch._scaled_mm (hipBLASLt) per expert on the
        # same codes with the plain [rows, K/32] E8M0 scales, where this build
        # supports it; its agreement with the grouped call is reported
        cmp_rec = per_expert_scaled_mm(torch, x8, xs, w8, ws, wl.offsets)
        compare = cmp_rec.pop("compare", None)
        cmp_fn = cmp_rec.pop("fn", None)
        for _ in range(5):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in fns] for _ in range(reps)]
        for row in ev:
            for (a, b), fn in zip(row, fns):
                a.record()
                fn()
                b.record()
        torch.cuda.synchronize()
        t = [statistics.median(r[i][0].elapsed_time(r[i][1]) for r in ev) * 1e3
             for i in range(len(fns))]
        flops = wl.flops()
        sc_bytes = 2 * (xs.numel() + ws.numel())          # read plain, write blocked (same size)
        out[f"fwd_mx:{wl.name}"] = {
            "mx_us": round(t[0], 1), "tflops": round(flops / t[0] / 1e6, 1),
            "pct_fp8_peak": round(100 * flops / t[0] / 1e6 / PEAK_FP8_TFLOPS, 1),
            "bf16_us": round(t[1], 1), "speedup_vs_bf16": round(t[1] / t[0], 3),
            "scale_layout_us": round(t[2], 1),
            "scale_layout_GBps": round(sc_bytes / t[2] / 1e3, 1)}
        if cmp_fn is not None:                    # timed on its own, after the others
            th, tg = time_library(torch, cmp_fn, reps)
            cmp_rec["us"] = round(tg, 1)
            cmp_rec["us_host_inclusive"] = round(th, 1)
            cmp_rec["speedup_of_grouped"] = round(tg / t[0], 3)
        if compare is not None:                   # y8: the grouped call's last result
            cmp_rec["rel_frobenius_vs_grouped"] = compare(y8)
        out[f"fwd_mx:{wl.name}"]["per_expert_scaled_mm"] = cmp_rec
        del x8, w8, xs, ws, bx, bw, x, w, y8, y
        torch.cuda.empty_cache()
    # weight gradients: uniform g8 and the skewed 30B-A3B ones, experts padded to
    # whole 128-token stages (the MXFP8 call's requirement), the bf16 call on the
    # same offsets
    from workloads import offsets_from_sizes
    for wl in [make_workload(2)[0]] + make_workload(5):
        sizes = [((int(v) + 127) // 128) * 128 for v in wl.sizes()]
        offn = offsets_from_sizes(sizes)
        M, N, K, E = int(offn[-1]), wl.N, wl.K, wl.E
        off = torch.from_numpy(offn).cuda()
        dyt8 = u8(mx_e4m3_codes((N, M), 8310, wl.cfg, wl.tag, 1))
        xt8 = u8(mx_e4m3_codes((K, M), 8310, wl.cfg, wl.tag, 2))
        dyts = u8(mx_e8m0_codes((N, M // 32), 121, 1, 8310, wl.cfg, wl.tag, 3))
        xts = u8(mx_e8m0_codes((K, M // 32), 121, 1, 8310, wl.cfg, wl.tag, 4))
        bd, bx = mg.mx_scales_blocked(dyts), mg.mx_scales_blocked(xts)
        dy = torch.randn((M, N), device="cuda").to(torch.bfloat16)
        x = torch.randn((M, K), device="cuda").to(torch.bfloat16)
        dy8, x8 = dyt8.t().contiguous(), xt8.t().contiguous()      # token-major codes
        d8 = torch.empty((E, N, K), dtype=torch.float32, device="cuda")
        d16 = torch.empty_like(d8)
        dtm = torch.empty_like(d8)
        fns = [lambda: mg.wgrad_mx(dyt8, bd, xt8, bx, off, E, out=d8),
               lambda: mg.wgrad(dy, x, off, E, out=d16),
               lambda: mg.wgrad_mx_tm(dy8, bd, x8, bx, off, E, out=dtm)]
        cmp_rec = per_expert_scaled_mm_wgrad(torch, dyt8, dyts, xt8, xts, offn)
        compare = cmp_rec.pop("compare", None)
        cmp_fn = cmp_rec.pop("fn", None)
        for _ in range(3):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in fns] for _ in range(reps)]
        for row in ev:
            for (a, b), fn in zip(row, fns):
                a.record()
                fn()
                b.record()
        torch.cuda.synchronize()
        t = [statistics.median(r[i][0].elapsed_time(r[i][1]) for r in ev) * 1e3
             for i in range(len(fns))]
        flops = 2 * M * N * K
        out[f"wgrad_mx:{wl.name}"] = {
            "rows": M, "mx_us": round(t[0], 1), "tflops": round(flops / t[0] / 1e6, 1),
            "pct_fp8_peak": round(100 * flops / t[0] / 1e6 / PEAK_FP8_TFLOPS, 1),
            "bf16_us": round(t[1], 1), "speedup_vs_bf16": round(t[1] / t[0], 3),
            "token_major_us": round(t[2], 1),
            "token_major_pct_fp8_peak": round(100 * flops / t[2] / 1e6 / PEAK_FP8_TFLOPS, 1)}
        if cmp_fn is not None:                    # timed on its own, after the others
            th, tg = time_library(torch, cmp_fn, reps)
            cmp_rec["us"] = round(tg, 1)
            cmp_rec["us_host_inclusive"] = round(th, 1)
            cmp_rec["speedup_of_grouped"] = round(tg / t[0], 3)
        if compare is not None:                   # d8: the grouped call's last result
            cmp_rec["rel_frobenius_vs_grouped"] = compare(d8)
        out[f"wgrad_mx:{wl.name}"]["per_expert_scaled_mm"] = cmp_rec
        del dyt8, xt8, dyts, xts, dy8, x8, bd, bx, dy, x, d8, d16, dtm
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ ceiling --

def ceiling(torch, seconds=3.0, iters=16384):
    """The matrix-core ceiling probe: one workgroup of 8 waves per compute
    unit issuing only v_mfma_f32_32x32x16_bf16 on register-held random
    operands (include/mgemm_probe.h).  Launches repeat for `seconds` to reach
    the steady power state; the last second's HIP-event rate is reported with
    the graphics clock sampled while the probe runs again."""
    import ctypes
    path = os.path.join(ROOT, "moe_grouped_gemm_bf16_amd", "libmgemm_probe.so")
    if not os.path.exists(path):
        return {"error": "libmgemm_probe.so not built"}
    lib = ctypes.CDLL(path)
    lib.mg_probe_mfma_bf16.restype = ctypes.c_int
    lib.mg_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.mg_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.mg_probe_mfma_bf16_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def launch():
        if lib.mg_probe_mfma_bf16(blocks, iters, out.data_ptr(), st) != 0:
            raise RuntimeError("probe launch failed")

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds - 1.0:
        for _ in range(10):
            launch()
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    a.record()
    t1 = time.perf_counter()
    while time.perf_counter() - t1 < 1.0:
        for _ in range(10):
            launch()
        n += 10
        torch.cuda.synchronize()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n
    tflops = lib.mg_probe_mfma_bf16_flops(blocks, iters) / us / 1e6
    clock = ClockSampler().measure(launch, torch, seconds=2.5)
    rec = {"tflops": round(tflops, 1), "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 1),
           "us_per_launch": round(us, 1), "launches_timed": n, "workgroups": blocks,
           "products_per_wave": iters * 8}
    if clock:
        rec["gfx_mhz_median"] = clock.get("gfx_mhz_median")
    return rec


# ------------------------------------------------------------- CPU baseline --

def cpu_baseline(workload: str):
    """The oracle as it stands, timed on this host's cores over whole steps
    of the default workload (all three ops, all experts), repeated until at
    least 10 s of CPU work have run; for the a3b workload, over the gate-up
    fwd + dgrad + wgrad of 4 of the 32 experts (a bounded sample).  The record
    names the CPU model and the BLAS library the oracle's products ran on."""
    import numpy as np
    from oracle import (bf16_bits_to_f64, f64_to_bf16_bits, grouped_dgrad, grouped_fwd,
                        grouped_wgrad)
    from workloads import make_workload
    blas = None
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        cores = max(i.get("num_threads", 1) for i in info) if info else 1
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                             None)
    except OSError:  # pragma: no cover
        pass
    flops, secs = 0, 0.0
    td = time.perf_counter()      # generating the inputs and decoding them to fp64: reported apart
    if workload == "a3b":
        wl = make_workload(4, "a3b_gate_up")[0]
        sel = 4
        o = wl.offsets
        rows = int(o[sel])
        X = bf16_bits_to_f64(wl.x_bits()[:rows]); W = bf16_bits_to_f64(wl.w_bits()[:sel])
        DY = bf16_bits_to_f64(wl.dy_bits()[:rows]); off = o[:sel + 1]
        sample = f"gate-up fwd+dgrad+wgrad of experts 0-3 ({rows} rows) of the 30B-A3B share"
    else:
        wl = make_workload(2 if workload == "uniform_g8" else 3)[0]
        X, W, DY = (bf16_bits_to_f64(b) for b in (wl.x_bits(), wl.w_bits(), wl.dy_bits()))
        off = wl.offsets
        rows = int(off[-1])
        sample = f"one whole step (fwd+dgrad+wgrad, all {wl.E} experts) of {wl.name}"
    E = len(off) - 1
    decode_secs = time.perf_counter() - td
    reps = 0
    t = time.perf_counter()
    while reps == 0 or time.perf_counter() - t < 10.0:
        f64_to_bf16_bits(grouped_fwd(X, W, off))
        f64_to_bf16_bits(grouped_dgrad(DY, W, off))
        grouped_wgrad(DY, X, off, E).astype(np.float32)
        reps += 1
    secs = time.perf_counter() - t
    flops = reps * 3 * 2 * rows * wl.N * wl.K
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "sample": f"{sample}, {reps} times", "seconds": round(secs, 3),
            "cpu_model": cpu_model, "blas": blas, "input_seconds": round(decode_secs, 3)}


# -------------------------------------------------------------------- traffic --

def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_src_sha256_16") != kernel_hash():
        return None
    return rec.get("bytes_per_launch", {}).get(kernel)


class ClockSampler:
    """Graphics clock while the step runs: amdsmi's per-XCD current gfx
    clocks (MHz) read every 2 ms on a thread of its own (ctypes calls, which
    release the interpreter lock).  The firmware refreshes that table only
    about once a second, so the step is repeated for `seconds` after the
    timed region and only samples taken after the table first changed inside
    that window count, at or above the 500 MHz minimum clock (an idle reading
    otherwise).  Best effort: without amdsmi, without a refresh in the window,
    or if every read fails, it reports nothing."""

    def __init__(self):
        self.samples, self._stop, self._th, self._h, self._smi = [], threading.Event(), None, None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:
            self._smi = None

    def _run(self):
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
                c = [v for v in m.get("current_gfxclks", []) if isinstance(v, (int, float)) and v > 0]
                if c:
                    self.samples.append((time.perf_counter(), statistics.fmean(c)))
            except Exception:
                pass
            self._stop.wait(0.002)

    def measure(self, step, torch, seconds=2.5):
        if self._smi is None:
            return None
        self._th = threading.Thread(target=self._run, daemon=True)
        t0 = time.perf_counter()
        self._th.start()
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                step()
            torch.cuda.synchronize()
        self._stop.set()
        self._th.join(timeout=5.0)            # (a read that never returns is left behind)
        if self._th.is_alive():
            return None
        try:
            self._smi.amdsmi_shut_down()
        except Exception:
            pass
        vals = [v for _, v in self.samples]
        first_new = next((i for i, v in enumerate(vals) if v != vals[0]), None)
        late = [v for v in vals[first_new:] if v >= 500.0] if first_new is not None else []
        if not late:
            return None
        return {"gfx_mhz_median": round(statistics.median(late), 1),
                "gfx_mhz_min": round(min(late), 1), "gfx_mhz_max": round(max(late), 1),
                "samples": len(late),
                "source": "amdsmi current_gfxclks (mean over the XCDs) every 2 ms while the "
                          "step repeats for 2.5 s after the timed steps; samples after the "
                          "table's first refresh in that window"}


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_grouped_gemm_bf16_amd as mg

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    ops, _keep = build_ops(args.workload, torch, mg)
    print(f"[bench] {args.workload}: {len(ops)} launches per step", file=sys.stderr, flush=True)

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for op in ops:
            op.launch()
    torch.cuda.synchronize()

    # Per-launch statistics from an untimed pass of K steps with HIP events
    # around every launch (event markers between launches lengthen a step by
    # several percent, so the timed steps below carry only the two around the
    # dominant kernel, whose duration the roofline entry needs).
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in ops] for _ in range(args.steps)]
    for s in range(args.steps):
        for i, op in enumerate(ops):
            ev[s][i][0].record(stream)
            op.launch()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    for s in range(args.steps):
        for i, op in enumerate(ops):
            op.times_ms.append(ev[s][i][0].elapsed_time(ev[s][i][1]))
    dom_i = max(range(len(ops)), key=lambda i: statistics.fmean(ops[i].times_ms))

    # the timed region: exactly K steps
    dev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, op in enumerate(ops):
            if i == dom_i:
                dev[s][0].record(stream)
            op.launch()
            if i == dom_i:
                dev[s][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom_times_ms = [a.elapsed_time(b) for a, b in dev]

    def one_step():
        for op in ops:
            op.launch()
    clock = None if args.no_clock else ClockSampler().measure(one_step, torch)

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    step_flops = sum(op.flops for op in ops)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    per_op = {}
    for op in ops:
        avg = statistics.fmean(op.times_ms)
        per_op[op.name] = {
            "avg_us": round(avg * 1e3, 2),
            "median_us": round(statistics.median(op.times_ms) * 1e3, 2),
            "min_us": round(min(op.times_ms) * 1e3, 2),
            "top10_mean_us": round(statistics.fmean(
                sorted(op.times_ms)[:max(1, len(op.times_ms) // 10)]) * 1e3, 2),
            "tflops": round(op.flops / (avg * 1e-3) / 1e12, 1),
            "pct_peak": round(100 * op.flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1),
            "median_pct_peak": round(
                100 * op.flops / (statistics.median(op.times_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1),
            "algo_GBps": round(op.bytes / (avg * 1e-3) / 1e9, 1),
        }

    if args.cold > 0:
        # Flushed launches: a 512 MiB fill (twice the 256 MB Infinity Cache,
        # far beyond the L2s) runs before every launch, outside its events;
        # one synchronisation at the end.
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        for op in ops:
            cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.cold)]
            for e0, e1 in cev:
                flush.fill_(1)
                e0.record(stream)
                op.launch()
                e1.record(stream)
            torch.cuda.synchronize()
            ts = sorted(e0.elapsed_time(e1) for e0, e1 in cev)
            med = statistics.median(ts)
            per_op[op.name].update({
                "cold_median_us": round(med * 1e3, 2),
                "cold_min_us": round(ts[0] * 1e3, 2),
                "cold_top10_mean_us": round(statistics.fmean(ts[:max(1, len(ts) // 10)]) * 1e3, 2),
                "cold_tflops": round(op.flops / (med * 1e-3) / 1e12, 1),
                "cold_pct_peak": round(100 * op.flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1),
            })
        del flush

    # each op against its target fraction of the peak (M-grouped forward and
    # input gradient 60%, K-grouped weight gradient 50%), on the flushed
    # median when measured, else the warm median
    targets = {}
    for op in ops:
        r = per_op[op.name]
        t_us = r.get("cold_median_us", r["median_us"])
        pct = 100 * op.flops / (t_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS
        goal = 50.0 if op.kind == "wgrad" else 60.0
        targets[op.name] = {"pct_peak": round(pct, 1), "target_pct": goal,
                            "target_us": round(op.flops / (goal / 100 * PEAK_BF16_TFLOPS * 1e12) * 1e6, 1),
                            "us": t_us, "timing": "flushed median" if "cold_median_us" in r else "warm median",
                            "met": pct >= goal}

    dom = ops[dom_i]
    dom_avg_s = statistics.fmean(dom_times_ms) * 1e-3      # in the timed region
    achieved = dom.flops / dom_avg_s / 1e12
    traffic = load_traffic(args.workload, dom.name)
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": f"{KERNEL_NAMES[dom.kind]} ({dom.name})",
                "avg_us_timed_region": round(dom_avg_s * 1e6, 2),
                "algorithmic_bytes": dom.bytes}

    comp = None
    if args.comparators:
        print("[bench] timing library comparators", file=sys.stderr, flush=True)
        comp = comparators(ops, torch)

    listed = None
    if args.lists:
        print("[bench] timing the descriptor-list call", file=sys.stderr, flush=True)
        listed = lists(torch, mg)

    mxr = None
    if args.mx:
        print("[bench] timing the MXFP8 forward", file=sys.stderr, flush=True)
        mxr = mx(torch, mg)

    ceil_rec = None
    if args.ceiling:
        print("[bench] running the matrix-core ceiling probe", file=sys.stderr, flush=True)
        ceil_rec = ceiling(torch)

    fused = None
    if args.fusions:
        print("[bench] timing the fused gate-up forward", file=sys.stderr, flush=True)
        fused = fusions(torch, mg)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.workload)

    wl0 = ops[0].wl
    if args.workload == "a3b":
        config = {"workload": "a3b_expert_share", "experts": 32, "d_model": 3072,
                  "expert_ffn": 1280, "fwd_dgrad_rows": ops[0].wl.rows,
                  "wgrad_rows": ops[-1].wl.rows, "ops": [o.name for o in ops]}
    else:
        config = {"workload": wl0.name, "g": wl0.E, "m": int(wl0.sizes()[0]), "n": wl0.N,
                  "k": wl0.K, "ops": [o.name for o in ops]}
    line = {
        "metric": "grouped-GEMM TFLOP/s + % bf16 MFMA peak (fwd, dgrad, wgrad), 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)-scaled bf16 inputs, see workloads/synth.py)",
        "config": config,
        "per_op": per_op,
        "targets": targets,
        "roofline": roofline,
        "clock": clock,
        "pct_of_clock_adjusted_peak": (
            round(100 * value / (BF16_FLOP_PER_CLK * clock["gfx_mhz_median"] * 1e6 / 1e12), 2)
            if clock else None),
        "cpu_baseline": cpu,
        "kernel_src_sha256_16": kernel_hash(),
    }
    if comp is not None:
        line["comparators"] = comp
    if fused is not None:
        line["fused_ops"] = fused
    if listed is not None:
        line["list_ops"] = listed
    if mxr is not None:
        line["mx_ops"] = mxr
    if ceil_rec is not None:
        line["mfma_ceiling"] = ceil_rec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
