"""Oracle for the MoE grouped GEMM: plain, slow, obviously correct CPU code.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, the smoke check and the bench's CPU-baseline leg call it.  It
shares no code with the HIP path (no kernels, headers, helpers or tables); the
two meet only through the seeded inputs of the `workloads` package.

What it computes (fp64 throughout, per-expert dense GEMMs, one library matmul
per expert; nothing blocked, fused or reordered):
  * M-grouped forward (RapidGEMM README, "Kernels", Mgemm): for the rows
    offsets[e] <= i < offsets[e+1] of expert e,  Y[i, n] = sum_k X[i, k] W[e, n, k].
  * M-grouped input gradient (same passage, the input-gradient form; the
    DeepGEMM issue #10 thread: a GEMM's backward is two GEMMs, dgrad and wgrad):
    dX[i, k] = sum_n dY[i, n] W[e, n, k].
  * K-grouped weight gradient (RapidGEMM README, "Kernels", Kgemm: the grouped
    FP32 weight gradient; DeepGEMM issue #10: wgrad is x^T dy):
    dW[e, n, k] = sum_{offsets[e] <= i < offsets[e+1]} dY[i, n] X[i, k],
    laid out like W so that it can update W.
  * Gate-up forward with SwiGLU on gathered rows (DeepGEMM issue #10: the
    fused-with-SwiGLU and MoE-layout kernels; RapidGEMM README "Kernels": the
    stacked gate/up weight gw13 refers to): row i reads token row gather[i],
    h[i, j] = silu(x . w1[e, j]) * (x . w3[e, j]) with w1, w3 the two halves of
    the expert's [2I, K] weight.
  * Its backward through the down projection: dh = dy W2[e] (the grouped input
    gradient), then the SwiGLU backward dg = dh u silu'(g), du = dh silu(g) on
    the saved pre-activation g | u (the DeepGEMM issue #10 thread: a kernel
    fused with SwiGLU is part of a weight-gradient path).
  * The token-order combine that inverts the gather: out[t] = sum_j w[t, j]
    rows[token_rows[t, j]] (the backward of the dispatch gather, or the
    layer's weighted output combine).
  * A list of independent GEMMs D_g = A_g B_g^T with per-group shapes (the
    TransformerEngine PR #2045 review: one C API over lists of tensors; the
    CUTLASS discussion #1452: nested grouped GEMMs flattened into one list).
  * MXFP8 M-grouped forward (torchao PR #3416: MXFP8 MoE grouped GEMMs with
    e8m0 block scales in a blocked layout; DeepGEMM issue #10: operands
    quantized along each GEMM's reduction axis): E4M3 elements, one E8M0
    scale per 32 reduction steps, decoded exactly and summed in fp64; the
    MXFP8 K-grouped weight gradient on token-major-last (transposed) operands
    quantized along the tokens; and the blocked scale layout
    [ceil(K/128)][rows][4] the GEMM calls read.
  * bf16 outputs are the fp64 result rounded once, directly, to bf16 with
    round-to-nearest-even.

Pins (tests/test_oracle_pins.py): exact rational brute force on tiny inputs,
closed forms on one-hot inputs, a hand-worked example (tests/golden/), the
adjoint identity tying fwd/dgrad/wgrad together, empty-group insertion,
exhaustive codec round trips and tie cases; for the SwiGLU forward, scalar
brute force with math.exp, one-hot closed forms that tell the gate half from
the up half, gather-as-permutation identities, and a gate that rejects a wrong
expert or a dropped term; for the SwiGLU backward, central finite
differences of silu(g) u and the chain-rule identity <dgu, [dg0, du0]> =
<dh, d(silu(g) u)> for a perturbation; for the combine, the adjoint identity
with the gather (<combine(R), X> = <R, X[gather]>) and a plain loop; for the descriptor list, exact rational brute force on
groups of mixed shapes (empty and zero-reduction ones included), a one-hot
transpose check and the flattened LoRA x experts identity; for MXFP8, the
element and scale decoders against torch's float8_e4m3fn / float8_e8m0fnu
casts on every code, closed forms, exact rational brute force on tiny inputs,
power-of-two scale shifts that move whole rows or experts exactly, the
blocked layout against an index-by-index brute force, and for the MXFP8
weight gradient exact rational brute force, the unit-scale reduction to the
plain K-grouped wgrad and the adjoint identity with the MXFP8 forward.  Every function here
is pinned; none is "parity
unpinned".
"""
from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits, bf16_ulp  # noqa: F401
from .grouped_gemm import (  # noqa: F401
    grouped_fwd,
    grouped_dgrad,
    grouped_wgrad,
    sample_fwd,
    sample_dgrad,
    sample_wgrad,
    grouped_fwd_swiglu,
    sample_fwd_swiglu,
    grouped_dgrad_swiglu,
    sample_dgrad_swiglu,
    moe_combine,
    grouped_list,
)
from .mx import (  # noqa: F401
    e4m3_decode,
    e8m0_decode,
    mx_dequant,
    grouped_fwd_mx,
    sample_fwd_mx,
    grouped_wgrad_mx,
    sample_wgrad_mx,
    mx_scales_blocked,
)
from .gate import (check_bf16, check_bf16_swiglu, check_bf16_mx, check_fp32,  # noqa: F401
                   check_fp32_mx, check_bf16_factor, GateReport)
