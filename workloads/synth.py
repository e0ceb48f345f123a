"""Seeded synthetic workloads for the MoE grouped GEMM.

Every grouped-GEMM problem is described in its *forward* orientation:
  X [M, K]  expert-contiguous token rows (bf16)
  W [E, N, K] per-expert weights (bf16)
  Y / dY [M, N], dX [M, K], dW [E, N, K]
with the rows of expert e being offsets[e] <= i < offsets[e+1] and a leading
zero in `offsets` (the RapidGEMM README, "Kernels": the cumulative row-offset
tensor with a leading zero).

The five workloads follow the shapes the pages use:
  * tiny: E=4, K=256, N=128, expert sizes [200, 0, 184, 128];
  * the two grouped-GEMM shapes of the TransformerEngine PR #2045 perf table,
    (g, m, n, k) = (8, 4096, 768, 2048) and (16, 2048, 768, 2048);
  * one GPU's expert share of the 30B-A3B layout of the RapidGEMM README
    ("Model layout" and "Settings" tables: d_model 3072, 128 experts, top-8,
    expert FFN width 1280, EP=4 so 32 experts per GPU, 4096 tokens per rank),
    routed by a seeded Gaussian router stand-in, for fwd/dgrad;
  * the same 32-expert layout with a Zipf(s=1.2) token split that has empty
    experts and one expert above 25% of the rows, for wgrad.

Inputs are drawn from seeded PCG64 streams as float32 normals, scaled, and
rounded to bf16 bit patterns (round to nearest even).  Only bit patterns and
offset arrays leave this module.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

_CHUNK = 1 << 24  # elements generated per chunk, to bound host memory


def _stream(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even.

    Input generation only; the inputs are finite normals so no NaN handling is
    needed here."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_bf16_bits(shape: Sequence[int], scale: float, *key: int) -> np.ndarray:
    """bf16 bit patterns of N(0, 1) * scale, from the PCG64 stream `key`."""
    n = int(np.prod(shape, dtype=np.int64))
    rng = _stream(*key)
    out = np.empty(n, dtype=np.uint16)
    s = np.float32(scale)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            v *= s
        out[lo:hi] = _f32_to_bf16_bits(v)
    return out.reshape(tuple(shape))


def small_int_bf16_bits(shape: Sequence[int], *key: int) -> np.ndarray:
    """bf16 bit patterns of integers uniform in [-3, 3] (each exact in bf16)."""
    rng = _stream(*key)
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = _f32_to_bf16_bits(rng.integers(-3, 4, hi - lo).astype(np.float32))
    return out.reshape(tuple(shape))


def offsets_from_sizes(sizes: Sequence[int]) -> np.ndarray:
    """Per-expert row counts -> int32 cumulative offsets with a leading zero."""
    sizes = np.asarray(sizes, dtype=np.int64)
    if (sizes < 0).any():
        raise ValueError("expert sizes must be >= 0")
    off = np.zeros(len(sizes) + 1, dtype=np.int64)
    np.cumsum(sizes, out=off[1:])
    if off[-1] > np.iinfo(np.int32).max:
        raise ValueError("total rows exceed int32")
    return off.astype(np.int32)


def router_offsets(n_tokens: int, n_experts_total: int, top_k: int,
                   local_experts: int, seed: int):
    """Router stand-in: top-k of seeded Gaussian logits, kept for local experts.

    Top-k of softmax equals top-k of the logits (softmax is monotone).  Ties
    break toward the lower expert index (stable sort).  The kept
    (token, expert) pairs are sorted by (expert, token).  Returns
    (offsets int32 [local_experts + 1], token_of_row int32 [M])."""
    rng = _stream(seed, 101)
    logits = rng.standard_normal((n_tokens, n_experts_total))
    topk = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    experts = topk.reshape(-1)
    tokens = np.repeat(np.arange(n_tokens, dtype=np.int64), top_k)
    keep = experts < local_experts
    experts, tokens = experts[keep], tokens[keep]
    order = np.lexsort((tokens, experts))
    counts = np.bincount(experts, minlength=local_experts)
    return offsets_from_sizes(counts), tokens[order].astype(np.int32)


def zipf_sizes(total: int, n_experts: int, n_empty: int, s: float,
               seed: int) -> np.ndarray:
    """Zipf(s) row counts with `n_empty` forced-empty experts.

    The non-empty experts get weights r^-s for ranks r = 1..(E - n_empty);
    `total` rows are split by largest-remainder rounding (ties toward the
    lower rank); a seeded permutation maps rank -> expert id, so the empty
    experts and the heavy one land at arbitrary ids."""
    live = n_experts - n_empty
    w = np.arange(1, live + 1, dtype=np.float64) ** (-s)
    quota = total * w / w.sum()
    base = np.floor(quota).astype(np.int64)
    short = total - int(base.sum())
    frac = quota - base
    order = np.lexsort((np.arange(live), -frac))  # largest fraction first
    base[order[:short]] += 1
    ranked = np.zeros(n_experts, dtype=np.int64)
    ranked[:live] = base
    perm = _stream(seed, 202).permutation(n_experts)
    sizes = np.zeros(n_experts, dtype=np.int64)
    sizes[perm] = ranked
    return sizes


def random_offsets(E: int, M: int, seed: int, special: Sequence[int] = ()) -> np.ndarray:
    """Ragged offsets for fuzzing: random sizes summing to at most M.

    `special` sizes (e.g. 0, 1, tile-1, tile, tile+1) are placed first, the
    rest are random; total rows never exceed M."""
    rng = _stream(seed, 303)
    sizes = list(special)[:E]
    rest = E - len(sizes)
    left = M - sum(sizes)
    if left < 0:
        raise ValueError("special sizes exceed M")
    if rest > 0:
        cuts = np.sort(rng.integers(0, left + 1, size=rest))
        parts = np.diff(np.concatenate([[0], cuts]))
        sizes += [int(p) for p in parts]
    sizes = np.asarray(sizes, dtype=np.int64)
    rng.shuffle(sizes)
    return offsets_from_sizes(sizes)


@dataclasses.dataclass
class Workload:
    """One grouped-GEMM problem in forward orientation."""
    name: str
    cfg: int
    tag: int
    E: int
    N: int
    K: int
    offsets: np.ndarray              # int32 [E + 1]
    M: int                           # rows allocated in X / Y (>= offsets[E])
    x_scale: float
    w_scale: float
    dy_scale: float = 1.0
    ops: tuple = ("fwd", "dgrad", "wgrad")

    @property
    def rows(self) -> int:
        return int(self.offsets[-1])

    def sizes(self) -> np.ndarray:
        return np.diff(self.offsets.astype(np.int64))

    def x_bits(self) -> np.ndarray:
        return normal_bf16_bits((self.M, self.K), self.x_scale, self.cfg, self.tag, 1)

    def w_bits(self) -> np.ndarray:
        return normal_bf16_bits((self.E, self.N, self.K), self.w_scale, self.cfg, self.tag, 2)

    def dy_bits(self) -> np.ndarray:
        return normal_bf16_bits((self.M, self.N), self.dy_scale, self.cfg, self.tag, 3)

    def flops(self) -> int:
        """Algorithmic flops of one op: 2 * (real rows) * N * K."""
        return 2 * self.rows * self.N * self.K


def _tiny() -> List[Workload]:
    K, N = 256, 128
    return [Workload("tiny_e4", 1, 0, 4, N, K, offsets_from_sizes([200, 0, 184, 128]), 512,
                     K ** -0.5, K ** -0.5)]


def _uniform(cfg: int, g: int, m: int, n: int, k: int) -> List[Workload]:
    return [Workload(f"uniform_g{g}_m{m}_n{n}_k{k}", cfg, 0, g, n, k,
                     offsets_from_sizes([m] * g), g * m, k ** -0.5, k ** -0.5)]


def _a3b_router() -> List[Workload]:
    off, _ = router_offsets(16384, 128, 8, 32, seed=4)
    M = int(off[-1])
    return [
        Workload("a3b_gate_up", 4, 0, 32, 2560, 3072, off, M, 3072 ** -0.5, 3072 ** -0.5,
                 ops=("fwd", "dgrad")),
        Workload("a3b_down", 4, 1, 32, 3072, 1280, off, M, 1280 ** -0.5, 1280 ** -0.5,
                 ops=("fwd", "dgrad")),
    ]


def _a3b_zipf() -> List[Workload]:
    off = offsets_from_sizes(zipf_sizes(32768, 32, 4, 1.2, seed=5))
    M = int(off[-1])
    return [
        Workload("a3b_zipf_gw13", 5, 0, 32, 2560, 3072, off, M, 1.0, 1.0, ops=("wgrad",)),
        Workload("a3b_zipf_gw2", 5, 1, 32, 3072, 1280, off, M, 1.0, 1.0, ops=("wgrad",)),
    ]


CONFIGS: Dict[int, Callable[[], List[Workload]]] = {
    1: _tiny,
    2: lambda: _uniform(2, 8, 4096, 768, 2048),
    3: lambda: _uniform(3, 16, 2048, 768, 2048),
    4: _a3b_router,
    5: _a3b_zipf,
}


def make_workload(cfg: int, name: Optional[str] = None) -> List[Workload]:
    """All problems of workload `cfg` (or only the one called `name`)."""
    ws = CONFIGS[cfg]()
    if name is not None:
        ws = [w for w in ws if w.name == name]
        if not ws:
            raise KeyError(name)
    return ws


def mx_e4m3_codes(shape: Sequence[int], *key: int) -> np.ndarray:
    """uint8 OCP E4M3 codes of roughly Gaussian values of the size MX blocks
    hold (|v| mostly in [2^3, 2^8]): sign and 3-bit mantissa from one uniform
    random byte, the 4-bit exponent field floor(log2(64 |N(0, 1)|)) + 7
    clipped to [0, 15]; the NaN code S.1111.111 is never drawn (it becomes
    S.1111.110)."""
    n = int(np.prod(shape, dtype=np.int64))
    rng = _stream(*key)
    out = np.empty(n, dtype=np.uint8)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        v = np.abs(rng.standard_normal(hi - lo, dtype=np.float32)) * np.float32(64.0)
        _, e = np.frexp(v)                        # v = f 2^e, f in [0.5, 1): floor(log2 v) = e - 1
        ex = np.clip(e + 6, 0, 15).astype(np.uint8)
        c = (rng.integers(0, 256, hi - lo, dtype=np.uint8) & np.uint8(0x87)) | (ex << np.uint8(3))
        c[(c & np.uint8(0x7F)) == np.uint8(0x7F)] -= np.uint8(1)
        out[lo:hi] = c
    return out.reshape(tuple(shape))


def mx_e8m0_codes(shape: Sequence[int], center: int, spread: int, *key: int) -> np.ndarray:
    """uint8 E8M0 scale codes, uniform in [center - spread, center + spread]."""
    rng = _stream(*key)
    c = rng.integers(center - spread, center + spread + 1, int(np.prod(shape, dtype=np.int64)))
    return np.clip(c, 0, 254).astype(np.uint8).reshape(tuple(shape))


# E4M3 codes of the integers 0..3 from their fields (sign bit 7, exponent field
# bits 6..3 with bias 7, mantissa bits 2..0): 0 is all zeros, 1 = 2^0 (E = 7),
# 2 = 2^1 (E = 8), 3 = 2^1 * 1.5 (E = 8, m = 4).
_E4M3_SMALL_INT = np.array([0x00, 0x38, 0x40, 0x44], dtype=np.uint8)


def mx_small_int_codes(shape: Sequence[int], *key: int) -> np.ndarray:
    """uint8 E4M3 codes of integers uniform in [-3, 3] (zero without a sign
    bit).  Products of two such values are integers of magnitude <= 9."""
    rng = _stream(*key)
    n = int(np.prod(shape, dtype=np.int64))
    mag = rng.integers(0, 4, n)
    neg = (rng.integers(0, 2, n) == 1) & (mag > 0)
    c = _E4M3_SMALL_INT[mag] | np.where(neg, np.uint8(0x80), np.uint8(0))
    return c.astype(np.uint8).reshape(tuple(shape))


def mx_e8m0_pair_codes(shape: Sequence[int], lo: int, *key: int) -> np.ndarray:
    """uint8 E8M0 scale codes drawn uniformly from {lo, lo + 1}: neighbouring
    32-blocks scaled by the same power of two or by twice it."""
    rng = _stream(*key)
    c = lo + rng.integers(0, 2, int(np.prod(shape, dtype=np.int64)))
    return c.astype(np.uint8).reshape(tuple(shape))


def mx_e8m0_row_codes(rows: int, blocks: int, center: int, spread: int, *key: int) -> np.ndarray:
    """uint8 E8M0 scale codes [rows, blocks], uniform in [center - spread,
    center + spread] per row and the same for every block of a row."""
    c = mx_e8m0_codes((rows, 1), center, spread, *key)
    return np.ascontiguousarray(np.broadcast_to(c, (rows, blocks)))


# -- a row-addressable operand for sizes past 4 GiB ---------------------------
# Element (i, k) = ((37 i + 11 k + 5) mod 17 - 8) / 8: a multiple of 1/8 in
# [-1, 1], exact in bf16, so that a tensor of billions of elements can be built
# on the device in row chunks and any of its rows (or a column range) recomputed
# on the host without materialising it.  Neighbouring rows and columns differ,
# so a row or column read from the wrong place changes the result.

def lattice_values(i, k) -> np.ndarray:
    """Values (float64) at broadcast int64 indices i, k."""
    i = np.asarray(i, np.int64); k = np.asarray(k, np.int64)
    return ((37 * i + 11 * k + 5) % 17 - 8) / 8.0


class LatticeMatrix:
    """Host view of the [M, K] lattice operand: m[rows] gives those rows,
    m[row_slice, col] one column over a row range (float64)."""

    def __init__(self, M: int, K: int):
        self.shape = (M, K)

    def __getitem__(self, idx):
        M, K = self.shape
        if isinstance(idx, tuple):
            rows, col = idx
            return lattice_values(np.arange(M)[rows], int(col))
        return lattice_values(np.asarray(idx, np.int64)[:, None], np.arange(K)[None, :])


def lattice_bf16(M: int, K: int, device, chunk: int = 1 << 16):
    """The [M, K] lattice operand as a torch bf16 tensor on `device`, built in
    row chunks (exact: every value is a multiple of 1/8 in [-1, 1])."""
    import torch
    out = torch.empty((M, K), dtype=torch.bfloat16, device=device)
    k = torch.arange(K, dtype=torch.int64, device=device)[None, :]
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        i = torch.arange(r0, r1, dtype=torch.int64, device=device)[:, None]
        v = (37 * i + 11 * k + 5) % 17 - 8
        out[r0:r1] = (v.to(torch.float32) / 8.0).to(torch.bfloat16)
    return out
