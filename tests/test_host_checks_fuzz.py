"""Property tests of the library's host-side checks (CPU, no device use).

mg_check_offsets_host and mg_check_list_host are compared, on many generated
inputs, with the rules include/mgemm.h states for the offsets array and for
mg_gemm_desc, written out here from the header's text.
"""
import ctypes

import numpy as np
from hypothesis import given, settings, strategies as st

from moe_grouped_gemm_bf16_amd import _lib
from moe_grouped_gemm_bf16_amd._lib import GemmDesc

L = _lib.LIB
OK, NUL, SHAPE, ALIGN, DEV, LAUNCH, OFFS = range(7)
MAX_E, MAX_DIM, MAX_ROWS = 1024, 1 << 22, (1 << 31) - 1


def offsets_rule(off, E, M):
    """The header: 1 <= E <= 1024, 0 <= M < 2^31; offsets[0] == 0,
    non-decreasing, offsets[E] <= M."""
    if not (1 <= E <= MAX_E) or not (0 <= M <= MAX_ROWS):
        return SHAPE
    if off[0] != 0 or any(off[e + 1] < off[e] for e in range(E)) or off[E] > M:
        return OFFS
    return OK


@st.composite
def offsets_case(draw):
    E = draw(st.integers(0, 12))
    steps = draw(st.lists(st.integers(-3, 40), min_size=E + 1, max_size=E + 1))
    off = np.cumsum(steps).astype(np.int64)
    if draw(st.booleans()):
        off = off - off[0]                   # usually a leading zero
    off = np.clip(off, -(1 << 31), (1 << 31) - 1).astype(np.int32)
    M = draw(st.one_of(st.integers(-2, 600), st.sampled_from([MAX_ROWS, MAX_ROWS + 1])))
    return off, E, M


@settings(max_examples=400, derandomize=True, deadline=None, database=None)
@given(offsets_case())
def test_offsets_check_follows_the_header(case):
    off, E, M = case
    arr = np.ascontiguousarray(np.concatenate([off, [0]]) if off.size == 0 else off, np.int32)
    got = L.mg_check_offsets_host(arr.ctypes.data, E, M)
    assert got == offsets_rule([int(v) for v in arr], E, M), (off, E, M)


P = 0x100000                       # a 16-byte aligned address, never dereferenced


def group_rule(d):
    """The header, per group: m, n, k >= 0; k, n and the strides multiples of
    8; lda >= k, ldb >= k, ldd >= n; strides <= 2^22 -- else SHAPE.  A group
    with m == 0 or n == 0 does nothing (no pointer is checked); otherwise d
    must be non-NULL and 16-byte aligned, and so must a and b when k > 0.
    Size errors come before NULL pointers, NULL pointers before misalignment."""
    a, b, dd, m, n, k, lda, ldb, ldd = d
    if m < 0 or n < 0 or k < 0:
        return SHAPE
    if n % 8 or k % 8 or lda % 8 or ldb % 8 or ldd % 8:
        return SHAPE
    if lda < k or ldb < k or ldd < n or max(lda, ldb, ldd) > MAX_DIM:
        return SHAPE
    if m == 0 or n == 0:
        return OK
    ptrs = [dd] + ([a, b] if k > 0 else [])
    if any(p == 0 for p in ptrs):
        return NUL
    if any(p % 16 for p in ptrs):
        return ALIGN
    return OK


def list_rule(descs):
    if not (1 <= len(descs) <= MAX_E):
        return SHAPE
    for d in descs:
        r = group_rule(d)
        if r != OK:
            return r
    return OK


ptr = st.sampled_from([0, P, P + 8, P + 16, P + 4])
dim = st.sampled_from([-8, -1, 0, 3, 8, 16, 24, 40, 64])
ld = st.sampled_from([0, 8, 12, 16, 24, 64, MAX_DIM, MAX_DIM + 8])
group = st.tuples(ptr, ptr, ptr, dim, dim, dim, ld, ld, ld)


@settings(max_examples=600, derandomize=True, deadline=None, database=None)
@given(st.lists(group, min_size=1, max_size=5))
def test_list_check_follows_the_header(descs):
    arr = (GemmDesc * len(descs))(*[GemmDesc(*d) for d in descs])
    got = L.mg_check_list_host(arr, len(descs))
    assert got == list_rule(descs), descs
