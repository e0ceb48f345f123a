"""Child process of test_parity_gpu.test_validation_and_split_switches: run
with MGEMM_VALIDATE=1 and MGEMM_SPLIT=0 in its environment (the library reads
both once per process).  Prints one line per check and exits non-zero on the
first failure."""
import sys

import numpy as np
import torch

import moe_grouped_gemm_bf16_amd as mg
from moe_grouped_gemm_bf16_amd._lib import MG_ERR_OFFSETS, MG_ERR_SHAPE, MgemmError
from parity import SENTINEL, dev_bf16, dev_i32, gate_fwd_full, gate_wgrad_full, host_bits, sentinel_bf16
from workloads import normal_bf16_bits, offsets_from_sizes


def expect_error(status, fn, what):
    try:
        fn()
    except MgemmError as ex:
        assert ex.status == status, f"{what}: status {ex.status}, expected {status}"
        print("[child] rejected as expected:", what, flush=True)
        return
    raise AssertionError(f"{what}: not rejected")


def main():
    sizes, N, K = [2017, 33, 65, 129, 0, 0, 0, 700], 1544, 776
    off = offsets_from_sizes(sizes)
    M, E = int(off[-1]) + 3, len(sizes)
    xb = normal_bf16_bits((M, K), 1.0, 2200, 1)
    wb = normal_bf16_bits((E, N, K), K ** -0.5, 2200, 2)
    dyb = normal_bf16_bits((M, N), 1.0, 2200, 3)
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)

    # valid offsets pass the validation; the weight gradient runs without
    # the token split and still matches the oracle
    y = mg.fwd(x, w, dev_i32(off), out=sentinel_bf16((M, N)))
    dw = mg.wgrad(dy, x, dev_i32(off))
    torch.cuda.synchronize()
    r = gate_fwd_full(xb, wb, off, host_bits(y))
    assert r.passed, f"fwd: {r}"
    r = gate_wgrad_full(dyb, xb, off, dw.cpu().numpy())
    assert r.passed, f"wgrad without the split: {r}"
    print("[child] valid offsets: fwd and unsplit wgrad match the oracle", flush=True)

    # offsets breaking the precondition are rejected before any launch
    bad = off.copy()
    bad[3], bad[4] = bad[4], bad[3]              # decreasing
    out = sentinel_bf16((M, N))
    expect_error(MG_ERR_OFFSETS, lambda: mg.fwd(x, w, dev_i32(bad), out=out), "decreasing offsets (fwd)")
    torch.cuda.synchronize()
    assert (host_bits(out) == SENTINEL).all(), "a rejected call wrote its output"
    past = off.copy()
    past[-1] = M + 1                             # offsets[E] > M
    expect_error(MG_ERR_OFFSETS, lambda: mg.wgrad(dy, x, dev_i32(past)), "offsets[E] > M (wgrad)")
    first = off.copy()
    first[0] = 1                                 # no leading zero
    expect_error(MG_ERR_OFFSETS, lambda: mg.dgrad(dy, w, dev_i32(first)), "offsets[0] != 0 (dgrad)")

    # a descriptor list whose device copy breaks the rules (k not a multiple
    # of 8), built past the binding's own host check
    a, b = dev_bf16(xb[:40, :16]), dev_bf16(wb[0, :24, :16])
    d = sentinel_bf16((40, 24))
    desc = mg.list_descriptors([(a, b)], [d])
    raw = desc.cpu().numpy().copy()
    fields = raw.view(np.int32)                  # a, b, d pointers (6 words), m, n, k, lda, ldb, ldd
    fields[8] = 12                               # k = 12
    expect_error(MG_ERR_SHAPE, lambda: mg.grouped_list_desc(torch.from_numpy(raw).cuda(), 1),
                 "descriptor with k = 12 (list)")
    torch.cuda.synchronize()
    assert (host_bits(d) == SENTINEL).all(), "a rejected list wrote its output"
    print("[child] ok", flush=True)


if __name__ == "__main__":
    main()
    sys.exit(0)
