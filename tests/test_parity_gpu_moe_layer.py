"""One MoE FFN layer, forward and backward, composed from the library's calls
and checked against torch autograd in fp32 on the CPU (needs an MI355X).

Forward: h = fwd_swiglu(x gathered by the router, w13) saving g | u, rows of
the down projection fwd(h, w2), the weighted combine back to tokens.
Backward: the combine's backward (dy gathered per row, times the row's
router weight -- test glue in torch), dgrad_swiglu, the gate-up input
gradient, the combine back to tokens, and the two weight gradients.  The
reference differentiates the same computation from the same bf16 inputs in
fp32; the library rounds every intermediate to bf16 (h, g | u, y rows,
dgu), so the bound is a relative one, 2e-2 in Frobenius norm per tensor --
far below what a swapped half, a transposed operand, a wrong expert or a
missing router weight would give.  The per-call numerics are gated tightly
elsewhere.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_bf16_amd as mg
from parity import dev_i32
from workloads import offsets_from_sizes

pytestmark = pytest.mark.gpu


def _rel(a: torch.Tensor, b: torch.Tensor) -> float:
    a = a.double(); b = b.double()
    return float((a - b).norm() / b.norm())


def test_moe_ffn_layer_forward_and_backward():
    torch.manual_seed(0)
    T, D, I, E, k = 512, 256, 136, 6, 2
    print("[case] moe layer", T, D, I, E, k, flush=True)
    # router stand-in: top-k of random logits over E experts, rows sorted by expert
    logits = torch.randn(T, E)
    top = logits.topk(k, dim=1)
    wts = torch.softmax(top.values, dim=1)                      # [T, k]
    pairs = [(int(top.indices[t, j]), t, j) for t in range(T) for j in range(k)]
    pairs.sort()
    gather = np.array([t for _, t, _ in pairs], np.int32)      # row -> token
    sizes = np.bincount([e for e, _, _ in pairs], minlength=E)
    off = offsets_from_sizes(sizes.tolist())
    token_rows = -np.ones((T, k), np.int32)
    row_w = np.zeros(len(pairs), np.float32)
    for i, (e, t, j) in enumerate(pairs):
        token_rows[t, j] = i
        row_w[i] = float(wts[t, j])
    M = len(pairs)

    bf = torch.bfloat16
    x = (torch.randn(T, D) / 2).to(bf)
    w13 = (torch.randn(E, 2 * I, D) * D ** -0.5).to(bf)
    w2 = (torch.randn(E, D, I) * I ** -0.5).to(bf)
    dy = torch.randn(T, D).to(bf)

    # ---- library, on the GPU
    xd, w13d, w2d, dyd = x.cuda(), w13.cuda(), w2.cuda(), dy.cuda()
    o, gi, trd = dev_i32(off), dev_i32(gather), dev_i32(token_rows)
    wd = wts.float().contiguous().cuda()
    gu = torch.empty((M, 2 * I), dtype=bf, device="cuda")
    h = mg.fwd_swiglu(xd, w13d, o, gather=gi, gu_out=gu)
    y_rows = mg.fwd(h, w2d, o)
    y = mg.moe_combine(y_rows, trd, wd)
    # backward of the weighted combine: each row gets its token's dy times its weight
    dy_rows = (dyd.float()[gi.long()] * torch.from_numpy(row_w).cuda()[:, None]).to(bf)
    dgu = mg.dgrad_swiglu(dy_rows, w2d, gu, o)
    dx_rows = mg.dgrad(dgu, w13d, o)
    dx = mg.moe_combine(dx_rows, trd)
    dw2 = mg.wgrad(dy_rows, h, o, E)
    x_rows = xd[gi.long()].contiguous()
    dw13 = mg.wgrad(dgu, x_rows, o, E)
    torch.cuda.synchronize()

    # ---- reference: torch autograd, fp32, CPU
    xr = x.float().requires_grad_(True)
    w13r = w13.float().requires_grad_(True)
    w2r = w2.float().requires_grad_(True)
    g_idx = torch.from_numpy(gather).long()
    yr = torch.zeros(T, D)
    xg = xr[g_idx]
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        a = xg[lo:hi] @ w13r[e].t()
        hr = torch.nn.functional.silu(a[:, :I]) * a[:, I:]
        ye = hr @ w2r[e].t()
        tok = g_idx[lo:hi]
        rw = torch.from_numpy(row_w[lo:hi])[:, None]
        yr = yr.index_add(0, tok, ye * rw)
    (yr * dy.float()).sum().backward()

    checks = {"y": (y.cpu(), yr.detach()), "dx": (dx.cpu(), xr.grad),
              "dw13": (dw13.cpu(), w13r.grad), "dw2": (dw2.cpu(), w2r.grad)}
    for name, (got, ref) in checks.items():
        r = _rel(got.float(), ref)
        print(f"[case] {name}: relative Frobenius {r:.3e}", flush=True)
        assert r < 2e-2, f"{name}: relative Frobenius {r:.3e}"
