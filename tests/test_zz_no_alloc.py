"""kgemm_wgrad_noalloc (the weight gradient for callers that cannot allocate:
its token-split workspace is the library's static device array) against
kgemm_wgrad on the GPU: two calls in a row, the second on a smaller input,
each bitwise equal to kgemm_wgrad's result on the same input and within the
fp32 gate of the oracle; with and without accumulation; and the same call
captured into a graph and replayed, every replay checked."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_bf16_amd as mg
from parity import dev_bf16, dev_i32, gate_wgrad_full
from workloads import normal_bf16_bits, offsets_from_sizes

pytestmark = pytest.mark.gpu

# One expert much heavier than the rest, so that its tiles are split in two
# token halves and the static workspace is used; the second input is smaller
# (fewer rows, experts and tiles) and splits too.
CASES = [
    ([2017, 33, 65, 129, 0, 0, 0, 700], 1544, 776),
    ([1500, 20, 0, 300], 520, 264),
]


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(i):
    sizes, N, K = CASES[i]
    off = offsets_from_sizes(sizes)
    M = int(off[-1]) + 3
    dyb = normal_bf16_bits((M, N), 1.0, 1700, i, 1)
    xb = normal_bf16_bits((M, K), 1.0, 1700, i, 2)
    return off, len(sizes), N, K, dyb, xb


@pytest.mark.parametrize("accumulate", [False, True])
def test_noalloc_matches_wgrad_on_two_calls(accumulate):
    ins = [_inputs(i) for i in range(len(CASES))]
    dev = []
    for i, (off, E, N, K, dyb, xb) in enumerate(ins):
        prior = np.random.default_rng(1700 + i).standard_normal((E, N, K)).astype(np.float32)
        dev.append((dev_bf16(dyb), dev_bf16(xb), dev_i32(off), prior))
    outs = []
    for i, (dy, x, o, prior) in enumerate(dev):          # two calls in a row
        _say("noalloc", CASES[i], "accumulate" if accumulate else "")
        out = torch.from_numpy(prior.copy()).cuda() if accumulate else \
            torch.full(tuple(prior.shape), float("nan"), device="cuda")
        outs.append(mg.wgrad_noalloc(dy, x, o, out=out, accumulate=accumulate))
    torch.cuda.synchronize()
    for i, (dy, x, o, prior) in enumerate(dev):
        ref = torch.from_numpy(prior.copy()).cuda() if accumulate else None
        ref = mg.wgrad(dy, x, o, out=ref, accumulate=accumulate)
        torch.cuda.synchronize()
        assert torch.equal(outs[i].view(torch.int32), ref.view(torch.int32)), \
            f"call {i}: kgemm_wgrad_noalloc differs from kgemm_wgrad"
        off, E, N, K, dyb, xb = ins[i]
        r = gate_wgrad_full(dyb, xb, off, outs[i].cpu().numpy(),
                            prior=prior.astype(np.float64) if accumulate else None)
        _say("call", i, str(r))
        assert r.passed, str(r)


def test_noalloc_captured_and_replayed():
    """Captured into a graph (the caller that cannot allocate), replayed three
    times with eager work between the replays: every replay bitwise equal to
    the eager call's result."""
    off, E, N, K, dyb, xb = _inputs(1)
    dy, x, o = dev_bf16(dyb), dev_bf16(xb), dev_i32(off)
    eager = mg.wgrad_noalloc(dy, x, o, out=torch.empty((E, N, K), device="cuda"))
    out = torch.full((E, N, K), float("nan"), device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mg.wgrad_noalloc(dy, x, o, out=out)
    torch.cuda.synchronize()
    # the eager work between replays: the first case, through the same array
    off0, E0, N0, K0, dyb0, xb0 = _inputs(0)
    dy0, x0, o0 = dev_bf16(dyb0), dev_bf16(xb0), dev_i32(off0)
    other = torch.empty((E0, N0, K0), device="cuda")
    for rep in range(3):
        _say("replay", rep)
        out.fill_(float("nan"))
        mg.wgrad_noalloc(dy0, x0, o0, out=other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"replay {rep}"
