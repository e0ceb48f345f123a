// gfx950 (CDNA4) kernels of the MoE grouped GEMM.
//
// One kernel template serves the three contractions of the path:
//   FWD   (M-grouped, RapidGEMM README "Kernels", Mgemm forward):
//         Y[i, n]   = sum_k X[i, k]  W[e, n, k]          rows i of expert e
//   DGRAD (M-grouped, the same call's input-gradient form; backward of a GEMM
//         is dgrad + wgrad, DeepGEMM issue #10):
//         dX[i, k]  = sum_n dY[i, n] W[e, n, k]
//   WGRAD (K-grouped, RapidGEMM README "Kernels", Kgemm, FP32 weight gradient):
//         dW[e,n,k] = sum_{i of e} dY[i, n] X[i, k]      fp32 out
// Expert e owns rows offsets[e] <= i < offsets[e+1] (cumulative offsets with a
// leading zero).
//
// Every output tile is computed as D = P * Q^T over a reduction axis R, where
// P indexes the output's contiguous dimension (so each lane of the matrix-core
// result holds four consecutive output elements) and Q the other one:
//            P (contiguous out dim)        Q                 R
//   FWD      n  from W[e] [n][k]           m from X [m][k]   k  (both R-contiguous)
//   DGRAD    k  from W[e] [n][k]           m from dY[m][n]   n  (P is R-strided)
//   WGRAD    k  from X  [i][k]             n from dY[i][n]   i  (both R-strided)
//   FWD_MX   as FWD, with E4M3 operands and one E8M0 scale per 32 k (MXFP8;
//            torchao PR #3416): the same 128-byte staged rows hold 128 k, and
//            the scaled fp8 matrix-core product applies the scales
//   DGRAD_SWIGLU as DGRAD (down projection: dH = dY W2[e]), the epilogue applying
//            the SwiGLU backward on the saved pre-activation g | u: dg = dh u
//            silu'(g), du = dh silu(g) (DeepGEMM issue #10: a kernel fused with
//            SwiGLU is part of a weight-gradient path)
//   WGRAD_MX K-grouped like WGRAD, on E4M3 operands quantized along the
//            tokens and stored token axis last: P = k from X^T [k][i],
//            Q = n from dY^T [n][i], R = i (both R-contiguous, as FWD_MX)
//
// Operand staging: HBM -> LDS by direct-to-LDS buffer loads (no registers),
// in LDS stages of kBK reduction steps, the next stage in flight while one is
// consumed.  R-contiguous operands are staged as [outer][kBK] rows and read
// with 128-bit LDS loads; R-strided operands are staged as they lie in HBM,
// [kBK][outer], and read with the LDS transpose load (ds_read_b64_tr_b16),
// which hands each lane 4 consecutive reduction values of one outer index --
// the transposes wgrad and dgrad need are done by the LDS read, not by a pass.
// Buffer descriptors whose range ends at the last valid byte make ragged
// rows, reduction tails and out-of-range columns arrive in LDS as zeros.
//
// Scheduling: all experts in one persistent launch, one workgroup per compute
// unit.  Each workgroup reads the offsets once, derives per-expert tile counts
// and their prefix sums on the device (no host synchronisation; empty experts
// give no M-tiles) and walks its own list of tiles.  The LDS stage ring runs
// on across tile boundaries: the first stages of the next tile load while the
// current tile's last products and its stores run.  Workgroup b runs on XCD
// b % 8 (the dispatcher deals workgroups to the XCDs round-robin), and every
// XCD owns a part of the tile space chosen so that the tiles it runs at the
// same time share operand panels in its L2:
//   M-grouped: a contiguous range of tile ids in a grouped raster order
//     (groups of gm M-tiles of one expert, M-tile fastest), so the tiles in
//     flight on an XCD cover ~gm M-tiles x a few P-tiles of one expert.
//   K-grouped: for every expert, one of 8 compact chunks of its tile grid
//     (P-bands of bw P-tiles, P-tile fastest within a band); experts are taken
//     heaviest first and the workgroups of an XCD share its list longest-
//     processing-time first, which balances tiles whose cost is the expert's
//     row count.  A tile too heavy to balance by placement (an expert holding
//     a large share of the rows) is split into two halves of its token range
//     whose fp32 partial sums are added by whichever half ends second.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdlib>
#include <mutex>
#include <type_traits>
#include <vector>

#include "mgemm.h"
#include "mgemm_launch.h"

namespace mg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

#ifndef MG_BK
#define MG_BK 64
#endif
// Reduction steps per LDS stage.  64 makes every R-contiguous row of a stage
// one full 128-byte line, so each L2 request carries 128 bytes.
constexpr int kBK = MG_BK;
constexpr int kStages = kBK == 32 ? 4 : 2;   // LDS stages (256x256 tile: 128 KiB)
constexpr int kRowB = kBK * 2;               // bytes per R-contiguous staged row
constexpr int kRowChunks = kBK / 8;          // 16-byte chunks per such row

#ifndef MG_WAVES
#define MG_WAVES 8
#endif
constexpr uint32_t kOOB = 0x80000000u;   // offset bit past any buffer range

// Tile configuration: BP x BQ output tile, WP x WQ waves, each wave owning a
// (BP/WP) x (BQ/WQ) sub-tile of 32x32 matrix-core blocks.
template <int BP_, int BQ_, int WP_, int WQ_>
struct TileCfg {
  static constexpr int BP = BP_, BQ = BQ_, WP = WP_, WQ = WQ_;
  static constexpr int NW = WP * WQ, NT = 64 * NW;
  static constexpr int WTP = BP / WP, WTQ = BQ / WQ;
  static constexpr int MP = WTP / 32, MQ = WTQ / 32;
  static constexpr int P_BYTES = BP * kBK * 2, Q_BYTES = BQ * kBK * 2;
  static constexpr int STAGE = P_BYTES + Q_BYTES;
  static constexpr int LDS = kStages * STAGE;
  static constexpr int SEGS = STAGE / 1024;          // 1 KiB direct-to-LDS loads per stage
  static constexpr int SEGS_P = P_BYTES / 1024;
  static constexpr int SEGS_PER_WAVE = SEGS / NW;
  static_assert(WTP % 32 == 0 && WTQ % 32 == 0, "wave tile must be 32-aligned");
  static_assert(SEGS % NW == 0 && SEGS_P % SEGS_PER_WAVE == 0, "segments per wave");
  static_assert(LDS <= 160 * 1024 - 16 * 1024, "LDS budget");
};

// 128-bit raw buffer descriptor: base, stride 0, range `bytes`.  Loads past
// the range return zero.  All inputs are wave-uniform.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  r.y = (int32_t)(__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xFFFFu);
  r.z = (int32_t)__builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000;
  return r;
}

// Direct-to-LDS 16-byte load: lane l's 16 bytes land at LDS byte address
// lds_addr + 16 l (lds_addr wave-uniform).  Issued as inline assembly so that
// the compiler does not serialise it against the LDS reads of other stages;
// completion is awaited explicitly with vmcnt before the stage's barrier.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory");
}

// Direct-to-LDS 4-byte load: lane l's dword lands at lds_addr + 4 l.
__device__ __forceinline__ void dma4(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(
      (const __attribute__((address_space(3))) void*)p);
}

// LDS layouts of one stage (byte offsets within an operand tile):
//  R-contiguous tile [outer][kBK]: rows of kRowB bytes in 16-B chunks; chunk c
//    of row r sits at chunk c ^ rc_swz(r), which uses row bits 0-4 only.  32
//    consecutive rows read at one chunk hit distinct banks in groups of 8 or
//    16 lanes.
//  R-strided tile [kBK][outer]: rows of outer*2 bytes in 16-B chunks; chunk c
//    of reduction row r sits at c ^ rs_swz(r % 4).  A transpose load touches
//    4 rows x 2 chunks per 16 lanes (4 chunks per 32 lanes), all distinct.
__device__ __forceinline__ int rc_swz(int row) {
  return kRowChunks == 4 ? (((row >> 1) ^ (row >> 2)) & 3) : ((row & 7) ^ ((row >> 3) & 3));
}
__device__ __forceinline__ int rs_swz(int r4) { return (0xCA60 >> (4 * r4)) & 15; }  // 0,6,10,12

// ------------------------------------------------------------- scheduler --

// Exclusive prefix sum over the block of per-thread values; returns the
// thread's exclusive prefix and writes the block total to *total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    int s = scratch[w];
    before += (w < wave) ? s : 0;
    all += s;
  }
  *total = all;
  return before + incl - x;
}

// The same over 64-bit values (block total to *total).
template <int NT>
__device__ __forceinline__ int64_t block_exclusive_scan64(int64_t x, int64_t* scratch,
                                                          int64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  __syncthreads();
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int64_t v = scratch[w];
    before += (w < wave) ? v : 0;
    all += v;
  }
  *total = all;
  return before + incl - x;
}

// Descriptor g of the list, read through the constant address space: the
// kernel never writes the descriptors, and with a wave-uniform g this
// compiles to scalar loads (waited on with lgkmcnt), not vector loads whose
// wait would also cover the in-flight operand loads.
typedef __attribute__((address_space(4))) const ListDesc ConstListDesc;
__device__ __forceinline__ ListDesc list_desc(const ListDesc* list, int g) {
  const ConstListDesc* p = reinterpret_cast<const ConstListDesc*>(
      reinterpret_cast<uintptr_t>(list)) + __builtin_amdgcn_readfirstlane(g);
  ListDesc d;
  d.a = p->a;
  d.b = p->b;
  d.d = p->d;
  d.m = p->m;
  d.n = p->n;
  d.k = p->k;
  d.lda = p->lda;
  d.ldb = p->ldb;
  d.ldd = p->ldd;
  return d;
}

struct Tile {
  int e;        // expert
  int q0;       // first Q index of the tile (global row for M-grouped, n for K-grouped)
  int q_end;    // one past the last valid Q index
  int p0;       // first P index
  int r_begin;  // reduction range [r_begin, r_end) of this work item
  int r_end;
  int split;    // K-grouped: -1 for a whole tile, else 2 x split-tile id + half
};

// Scheduler state kept in LDS / registers for the whole launch.
struct Sched {
  int* scan;    // [16] scan scratch
  int* pref;    // [E+1] M-grouped: exclusive prefix of M-tiles per expert
  int* offs;    // [E+1] copy of the offsets
  int* inv;     // [E]   K-grouped: rank (heaviest first) -> expert
  int* mine;    // [2E]  K-grouped: this workgroup's (rank | rho << 16, count) entries
  int* keys;    // [64]  K-grouped: balancing scratch
  int nmine;    // K-grouped: entries in `mine`
  int total;    // number of tiles
  int E, tilesP, tilesQ, red;
  int gm;       // M-grouped: M-tiles per raster group
  int bw;       // K-grouped: P-tiles per band
  int per;      // K-grouped: tiles per expert
  bool split;   // K-grouped: heavy tiles may be split in two token halves
  bool whole;   // K-grouped: each XCD takes whole experts (see kchunk_start)
  const ListDesc* list;   // descriptor list (E groups), else null
};

// Offsets are read clamped to [0, M] and made non-decreasing per expert, so
// that even offsets breaking the documented precondition cannot move any read
// or write outside the tensors (the results are then meaningless, not unsafe).
__device__ __forceinline__ int clamp_off(const int32_t* offsets, int i, int M) {
  const int o = offsets[i];
  return o < 0 ? 0 : (o > M ? M : o);
}

// M-grouped set-up: tiles are, for every expert, ceil(m_e / BQ) M-tiles times
// tilesP P-tiles; empty experts contribute none.
template <int NT, int BQ>
__device__ void setup_mgrouped(const int32_t* __restrict__ offsets, int E, int M, Sched& S) {
  constexpr int kPer = (kMaxExperts + NT - 1) / NT;
  const int e0 = threadIdx.x * kPer;
  int cnt[kPer];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = e0 + j;
    cnt[j] = 0;
    if (e < E) {
      const int lo = clamp_off(offsets, e, M);
      const int hi = max(lo, clamp_off(offsets, e + 1, M));
      S.offs[e] = lo;
      if (e == E - 1) S.offs[E] = hi;
      const int m = hi - lo;
      cnt[j] = m > 0 ? (m + BQ - 1) / BQ : 0;
      mine += cnt[j];
    }
  }
  int mtiles;
  int run = block_exclusive_scan<NT>(mine, S.scan, &mtiles);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = e0 + j;
    if (e < E) S.pref[e] = run;
    run += cnt[j];
  }
  if (threadIdx.x == 0) S.pref[E] = mtiles;
  __syncthreads();
  S.total = mtiles * S.tilesP;
}

// Descriptor-list set-up: group g has ceil(m / BQ) x ceil(n / BP) tiles (none
// when m or n is not positive); S.pref holds their exclusive prefix.
template <int NT, int BP, int BQ>
__device__ void setup_list(const ListDesc* __restrict__ desc, int G, Sched& S) {
  constexpr int kPer = (kMaxExperts + NT - 1) / NT;
  const int g0 = threadIdx.x * kPer;
  int cnt[kPer];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int g = g0 + j;
    cnt[j] = 0;
    if (g < G) {
      const int m = desc[g].m, n = desc[g].n;
      cnt[j] = m > 0 && n > 0 ? ((m + BQ - 1) / BQ) * ((n + BP - 1) / BP) : 0;
      mine += cnt[j];
    }
  }
  int total;
  int run = block_exclusive_scan<NT>(mine, S.scan, &total);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int g = g0 + j;
    if (g < G) S.pref[g] = run;
    run += cnt[j];
  }
  if (threadIdx.x == 0) S.pref[G] = total;
  __syncthreads();
  S.total = total;
  // Groups may differ in k, so tiles differ in cost (stages + 3 for the
  // store): the XCDs get contiguous tile ranges of equal total cost rather
  // than equal tile counts.  XCD x starts at T_x, the number of tiles whose
  // cost midpoint lies below x / 8 of the total W: a tile u of a group whose
  // tiles cost w each and start at cumulative cost c0 counts when
  // 8 (c0 + u w) + 4 w < x W.  T_x is kept in S.keys[x] (x = 0..8).
  int64_t cost = 0;
  int64_t w[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int g = g0 + j;
    w[j] = 0;
    if (g < G) {
      w[j] = (int64_t)((max(desc[g].k, 0) + kBK - 1) / kBK + 3);
      cost += (int64_t)cnt[j] * w[j];
    }
  }
  int64_t* scratch64 = reinterpret_cast<int64_t*>(S.keys + 16);
  int64_t wtot;
  int64_t crun = block_exclusive_scan64<NT>(cost, scratch64, &wtot);
  int below[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (g0 + j < G && cnt[j] > 0) {
      for (int x = 1; x < 8; ++x) {
        const int64_t num = (int64_t)x * wtot - 8 * crun - 4 * w[j];
        const int64_t q = num <= 0 ? 0 : (num + 8 * w[j] - 1) / (8 * w[j]);
        below[x] += (int)(q < cnt[j] ? q : cnt[j]);
      }
      crun += (int64_t)cnt[j] * w[j];
    }
  }
  if (threadIdx.x < 9) S.keys[threadIdx.x] = threadIdx.x == 8 ? total : 0;
  __syncthreads();
  for (int x = 1; x < 8; ++x) {
    int v = below[x];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if ((threadIdx.x & 63) == 0 && v != 0) atomicAdd(&S.keys[x], v);
  }
  __syncthreads();
}

// Tile id L of the list -> tile: the group holding L (binary search on the
// prefix; groups without tiles share their successor's prefix), then, within
// the group, raster groups of gm M-tiles, M-tile fastest.
template <int BP, int BQ>
__device__ __forceinline__ void decode_list(int L, const Sched& S, const ListDesc* desc, Tile& t) {
  int lo = 0, hi = S.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S.pref[mid] <= L) lo = mid; else hi = mid - 1;
  }
  const int g = __builtin_amdgcn_readfirstlane(lo);
  const ListDesc dg = list_desc(desc, g);
  const int m = dg.m, n = dg.n, k = dg.k;
  const int local = L - S.pref[g];
  const int mt = (m + BQ - 1) / BQ, tilesP = (n + BP - 1) / BP;
  const int gg = local / (S.gm * tilesP);
  const int rem = local - gg * S.gm * tilesP;
  const int gh = min(S.gm, mt - gg * S.gm);
  const int tp = rem / gh;
  t.e = g;
  t.q0 = (gg * S.gm + (rem - tp * gh)) * BQ;
  t.q_end = m;
  t.p0 = tp * BP;
  t.r_begin = 0;
  t.r_end = max(k, 0);
}

// K-grouped: chunk k (0..7) of an expert's tile grid is the band-order index
// range [k per / 8, (k+1) per / 8).
// With `whole` (equal experts, E a multiple of 8), chunk 0 is the expert's
// whole grid and the others are empty: XCD x then takes the experts of rank
// x, x + 8, ..., so that all tiles of an expert share its X and dY panels in
// one L2 (with 8 chunks each expert's panels are read by every XCD).
__device__ __forceinline__ int kchunk_start(int k, int per, bool whole) {
  return whole ? (k == 0 ? 0 : per) : (k * per) >> 3;
}
__device__ __forceinline__ int kchunk_size(int k, int per, bool whole) {
  return kchunk_start(k + 1, per, whole) - kchunk_start(k, per, whole);
}

// K-grouped set-up: every expert has tilesQ x tilesP tiles whose cost grows
// with its row count; experts are ranked heaviest first (ties: lower index
// first) so that long reductions start early and short ones fill the tail.
// The row counts are staged in S.mine (free until the balancing below),
// padded with -1 so that the rank loop reads them four at a time.
template <int NT>
__device__ void setup_kgrouped(const int32_t* __restrict__ offsets, int E, int M, Sched& S) {
  for (int e = threadIdx.x; e <= E; e += NT) S.offs[e] = clamp_off(offsets, e, M);
  __syncthreads();
  // whole experts per XCD when every expert has the same, nonzero row count
  // and E is a multiple of 8 (the XCDs then get equal shares)
  int same = 1;
  for (int e = threadIdx.x; e < E; e += NT)
    same &= S.offs[e + 1] - S.offs[e] == S.offs[1] - S.offs[0] ? 1 : 0;
  same = __syncthreads_and(same);
  S.whole = S.whole && same != 0 && (E & 7) == 0 && S.offs[1] > S.offs[0];
  int* sizes = S.mine;
  for (int e = threadIdx.x; e < E + 4; e += NT)
    sizes[e] = e < E ? max(S.offs[e + 1] - S.offs[e], 0) : -1;
  __syncthreads();
  const int4* s4 = reinterpret_cast<const int4*>(sizes);
  for (int e = threadIdx.x; e < E; e += NT) {
    const int me = sizes[e];
    int rank = 0;
    for (int f4 = 0; f4 < (E + 3) / 4; ++f4) {
      const int4 v = s4[f4];
      const int f = 4 * f4;
      rank += (v.x > me || (v.x == me && f < e)) ? 1 : 0;
      rank += (v.y > me || (v.y == me && f + 1 < e)) ? 1 : 0;
      rank += (v.z > me || (v.z == me && f + 2 < e)) ? 1 : 0;
      rank += (v.w > me || (v.w == me && f + 3 < e)) ? 1 : 0;
    }
    S.inv[rank] = e;
  }
  __syncthreads();
  S.total = E * S.per;
}

// K-grouped token split.  A tile of an expert whose cost exceeds the XCD's
// average load per workgroup cannot be balanced by placement alone: it is
// split into two halves of its token range when such tiles are few enough
// (at most kSplitPerXcd and at most half the XCD's workgroups) for each half
// to share a workgroup with lighter tiles.  The halves add their fp32
// partial sums at the end (see the consumer's epilogue).  kSplitCost: extra
// cost, in stages, charged to a half for writing and reading the partial.
constexpr int kSplitPerXcd = 16;
constexpr int kSplitMinStages = 16;
constexpr int kSplitCost = 4;

// K-grouped balancing.  XCD x's list is chunk (x - r) mod 8 of expert inv[r]
// for r = 0, 1, ...: runs of equal-cost tiles, heaviest first.  Its nx
// workgroups take them longest-processing-time first: the c tiles of a chunk
// go `full` = c / nx to every workgroup and one more to the `rem` = c % nx
// least loaded ones (ties: lower workgroup index).  A workgroup whose load
// has rank rho among them takes the chunk's tiles rho, rho + nx, ...; it
// records (r, rho, count) for its own list.  Cost of a tile: its stages plus
// three for the store, scaled so that every load fits 25 bits; the keys
// (load, index) are ranked by comparing each with all the others.  When every
// tile costs the same this is plain round-robin over the list, done without
// ranking.  One wave does the work; the per-rank quantities are computed 64
// ranks at a time, one per lane, and read back with readlane.
template <int NT>
__device__ void balance_kgrouped(int x, int me, int nx, Sched& S) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // pass 1: the XCD's total cost, for the split decision
    uint64_t tot0 = 0;
    for (int r = lane; r < S.E; r += 64) {
      const int e = S.inv[r];
      const int m = max(S.offs[e + 1] - S.offs[e], 0);
      tot0 += (uint64_t)kchunk_size((x - r) & 7, S.per, S.whole) * (uint64_t)((m + kBK - 1) / kBK + 3);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) tot0 += __shfl_xor(tot0, d, 64);
    tot0 = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(tot0 >> 32)) << 32) |
           __builtin_amdgcn_readfirstlane((uint32_t)tot0);
    const uint64_t avg = tot0 / (uint64_t)nx;
    // tiles heavier than the average load (and long enough to halve)
    auto heavy = [&](int m) {
      const int st = (m + kBK - 1) / kBK;
      return st >= kSplitMinStages && (uint64_t)(st + 3) > avg;
    };
    int nheavy = 0;
    for (int r = lane; r < S.E; r += 64) {
      const int e = S.inv[r];
      if (heavy(max(S.offs[e + 1] - S.offs[e], 0))) nheavy += kchunk_size((x - r) & 7, S.per, S.whole);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) nheavy += __shfl_xor(nheavy, d, 64);
    nheavy = __builtin_amdgcn_readfirstlane(nheavy);
    const bool split_on = S.split && nheavy > 0 && nheavy <= kSplitPerXcd && 2 * nheavy <= nx;
    // a run's pieces: c tiles of cost w, or 2c halves of cost about w / 2
    auto piece = [&](int m, int c, int& np, uint32_t& w, bool& sp) {
      const int st = (m + kBK - 1) / kBK;
      sp = split_on && heavy(m);
      np = sp ? 2 * c : c;
      w = (uint32_t)(sp ? (st + 1) / 2 + 3 + kSplitCost : st + 3);
    };
    // pass 2: totals over the pieces
    uint64_t tot = 0;
    int ntiles = 0;
    uint32_t wlo = 0xFFFFFFFFu, whi = 0;
    for (int r = lane; r < S.E; r += 64) {
      const int e = S.inv[r];
      const int m = max(S.offs[e + 1] - S.offs[e], 0);
      int c;
      uint32_t w;
      bool sp;
      piece(m, kchunk_size((x - r) & 7, S.per, S.whole), c, w, sp);
      tot += (uint64_t)c * w;
      ntiles += c;
      if (c > 0) { wlo = min(wlo, w); whi = max(whi, w); }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      tot += __shfl_xor(tot, d, 64);
      ntiles += __shfl_xor(ntiles, d, 64);
      wlo = min(wlo, (uint32_t)__shfl_xor((int)wlo, d, 64));
      whi = max(whi, (uint32_t)__shfl_xor((int)whi, d, 64));
    }
    // (the reductions are wave-uniform; say so, so that what follows is scalar)
    tot = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(tot >> 32)) << 32) |
          __builtin_amdgcn_readfirstlane((uint32_t)tot);
    ntiles = __builtin_amdgcn_readfirstlane(ntiles);
    wlo = __builtin_amdgcn_readfirstlane(wlo);
    whi = __builtin_amdgcn_readfirstlane(whi);
    // scaled tile cost (c >> sh) + 1: a load never exceeds (tot >> sh) + ntiles;
    // keys need loads below 2^25, else (only for lists of tens of millions of
    // tiles) the round-robin below is used, which is balanced to one tile
    int sh = 0;
    while ((tot >> sh) >= (1ull << 15)) ++sh;
    const uint64_t maxload = (tot >> sh) + (uint64_t)ntiles;
    const bool equal = wlo >= whi || (maxload >> 25) != 0;
    uint32_t load = 0;
    int n = 0, pos = 0;       // pos: list position mod nx (equal costs)
    int sbase = 0;            // split tiles of this XCD so far
    for (int b0 = 0; b0 < S.E; b0 += 64) {
      const int rl = b0 + lane;
      int cl = 0, fl = 0, rl_rem = 0, spl = 0, ctl = 0;
      uint32_t wl = 0;
      if (rl < S.E) {
        const int e = S.inv[rl];
        const int m = max(S.offs[e + 1] - S.offs[e], 0);
        uint32_t w;
        bool sp;
        ctl = kchunk_size((x - rl) & 7, S.per, S.whole);
        piece(m, ctl, cl, w, sp);
        spl = sp ? 1 : 0;
        wl = (w >> sh) + 1u;
        fl = cl / nx;
        rl_rem = cl - fl * nx;
      }
      const int nb = min(64, S.E - b0);
      for (int i = 0; i < nb; ++i) {
        const int c = __builtin_amdgcn_readlane(cl, i);
        if (c == 0) continue;
        const int full = __builtin_amdgcn_readlane(fl, i);
        const int rem = __builtin_amdgcn_readlane(rl_rem, i);
        int rho;
        if (equal) {
          rho = me - pos;
          rho += rho < 0 ? nx : 0;
          pos += rem;
          pos -= pos >= nx ? nx : 0;
        } else {
          const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)wl, i);
          int rank = lane;
          if (rem > 0) {
            // rank of each bin's key among the nx keys (all distinct)
            const uint32_t key = lane < nx ? ((load << 6) | (uint32_t)lane) : 0xFFFFFFFFu;
            S.keys[lane] = (int)key;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const uint4* kv = reinterpret_cast<const uint4*>(S.keys);
            int r0 = 0, r1 = 0;
            if (nx <= 32) {
              uint4 q[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) q[j] = kv[j];
#pragma unroll
              for (int j = 0; j < 8; j += 2) {
                r0 += (q[j].x < key) + (q[j].y < key) + (q[j].z < key) + (q[j].w < key);
                r1 += (q[j + 1].x < key) + (q[j + 1].y < key) + (q[j + 1].z < key) +
                      (q[j + 1].w < key);
              }
            } else {
              uint4 q[16];
#pragma unroll
              for (int j = 0; j < 16; ++j) q[j] = kv[j];
#pragma unroll
              for (int j = 0; j < 16; j += 2) {
                r0 += (q[j].x < key) + (q[j].y < key) + (q[j].z < key) + (q[j].w < key);
                r1 += (q[j + 1].x < key) + (q[j + 1].y < key) + (q[j + 1].z < key) +
                      (q[j + 1].w < key);
              }
            }
            rank = r0 + r1;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (rank < rem) load += w;
          }
          load += (uint32_t)full * w;
          rho = __builtin_amdgcn_readlane(rank, me);
        }
        const int cnt = full + (rho < rem ? 1 : 0);
        const int sp = __builtin_amdgcn_readlane(spl, i);
        if (cnt > 0) {
          if (lane == 0) {
            S.mine[2 * n] = (b0 + i) | (rho << 16) | (sbase << 22) | (sp << 27);
            S.mine[2 * n + 1] = cnt;
          }
          ++n;
        }
        if (sp) sbase += __builtin_amdgcn_readlane(ctl, i);
      }
    }
    if (lane == 0) S.keys[0] = n;
  }
  __syncthreads();
  S.nmine = S.keys[0];
}

// M-grouped tile id L -> tile.  Ids run expert by expert; within an expert,
// in groups of gm M-tiles (the last group may be shorter), M-tile fastest,
// then P-tile.
template <int PSTEP, int BQ>
__device__ __forceinline__ void decode_mgrouped(int L, const Sched& S, Tile& t) {
  const int tilesP = S.tilesP;
  // the expert whose id range [pref[e] tilesP, pref[e+1] tilesP) holds L: the
  // largest e with pref[e] tilesP <= L (empty experts share their successor's
  // prefix)
  int lo = 0, hi = S.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S.pref[mid] * tilesP <= L) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int local = L - S.pref[e] * tilesP;
  const int mt = S.pref[e + 1] - S.pref[e];
  const int g = local / (S.gm * tilesP);
  const int rem = local - g * S.gm * tilesP;
  const int gh = min(S.gm, mt - g * S.gm);
  const int tp = rem / gh;
  const int m = g * S.gm + (rem - tp * gh);
  t.e = e;
  t.q0 = S.offs[e] + m * BQ;
  t.q_end = max(S.offs[e + 1], S.offs[e]);
  t.p0 = tp * PSTEP;
  t.r_begin = 0;
  t.r_end = S.red;
}

// Tile u of chunk k of the expert with rank r -> tile.  Within the expert's
// grid the tiles run in band order: P-bands of bw P-tiles each (the last may
// be narrower); within a band, Q-tile slow and P-tile fast.
template <int BP, int BQ>
__device__ __forceinline__ void decode_kgrouped(int r, int k, int u_in_chunk, const Sched& S,
                                                bool whole, Tile& t) {
  const int e = S.inv[r];
  const int u = kchunk_start(k, S.per, whole) + u_in_chunk;
  const int nbw = S.bw * S.tilesQ;
  const int b = min(u / nbw, (S.tilesP - 1) / S.bw);
  const int local = u - b * nbw;
  const int wb = min(S.bw, S.tilesP - b * S.bw);
  const int tq = local / wb;
  const int tp = b * S.bw + (local - tq * wb);
  t.e = e;
  t.q0 = tq * BQ;
  t.p0 = tp * BP;
  t.r_begin = S.offs[e];
  t.r_end = max(S.offs[e + 1], S.offs[e]);
  t.q_end = 0x7FFFFFFF;
}

// The tile list of one workgroup: XCD x = blockIdx % 8, index c = blockIdx / 8
// among the nx = gridDim / 8 workgroups of that XCD (gridDim is a multiple
// of 8).  M-grouped: ids lo + c, lo + c + nx, ... of the XCD's range.
// K-grouped: the balanced entries of `mine`.
template <int MODE, int BP, int BQ>
struct TileSeq {
  int x, c, nx, count, lo, j, ie;
  static constexpr bool MXW = MODE == kWgradMx || MODE == kWgradMxT;   // MXFP8 weight gradient
  static constexpr bool KG = MODE == kWgrad || MXW;                      // K-grouped
  static constexpr int SBK = MXW ? 128 : kBK;                            // reduction steps per stage

  __device__ __forceinline__ void init(const Sched& S) {
    x = blockIdx.x & 7;
    c = blockIdx.x >> 3;
    nx = gridDim.x >> 3;
    j = 0;
    ie = 0;
    if (!KG) {
      if (MODE == kList) {              // cost-balanced ranges from the set-up
        lo = S.keys[x];
        count = S.keys[x + 1] - lo;
      } else {
        const int q8 = S.total >> 3, r8 = S.total & 7;
        count = q8 + (x < r8 ? 1 : 0);
        lo = x * q8 + (x < r8 ? x : r8);
      }
    }
  }

  // Next tile of this workgroup; false once the list is exhausted.
  __device__ __forceinline__ bool next(const Sched& S, Tile& t) {
    t.split = -1;
    if (KG) {
      if (ie >= S.nmine) return false;
      // entry: rank (bits 0-9), rho (16-21), first split-tile index (22-26), split (27)
      const int rr = S.mine[2 * ie], cnt = S.mine[2 * ie + 1];
      const int r = rr & 0x3FF, rho = (rr >> 16) & 63, sbase = (rr >> 22) & 31;
      const bool sp = (rr >> 27) & 1;
      const int v = rho + j * nx;                 // piece of the chunk
      const int u = sp ? v >> 1 : v;
      decode_kgrouped<BP, BQ>(r, (x - r) & 7, u, S, MODE == kWgrad && S.whole, t);
      if (MXW) {
        // whole 128-token stages (a no-op for offsets that are multiples of
        // 128, as documented; others give wrong sums but only aligned,
        // in-bounds loads: M is a multiple of 128)
        t.r_begin &= ~(SBK - 1);
        t.r_end = (t.r_end + SBK - 1) & ~(SBK - 1);
      }
      if (sp) {
        // halves of the token range, split at a stage boundary
        const int st = (t.r_end - t.r_begin + SBK - 1) / SBK;
        const int mid = t.r_begin + ((st + 1) / 2) * SBK;
        if (v & 1) t.r_begin = mid;
        else t.r_end = mid;
        t.split = ((x * kSplitPerXcd + sbase + u) << 1) | (v & 1);
      }
      if (++j == cnt) { j = 0; ++ie; }
    } else {
      const int s = c + j * nx;
      if (s >= count) return false;
      ++j;
      // the fused SwiGLU forward's tile covers BP / 2 output columns (gate + up rows)
      if (MODE == kList) decode_list<BP, BQ>(lo + s, S, S.list, t);
      else decode_mgrouped<(MODE == kFwdSwiglu ? BP / 2 : BP), BQ>(lo + s, S, t);
    }
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.q0 = __builtin_amdgcn_readfirstlane(t.q0);
    t.q_end = __builtin_amdgcn_readfirstlane(t.q_end);
    t.p0 = __builtin_amdgcn_readfirstlane(t.p0);
    t.r_begin = __builtin_amdgcn_readfirstlane(t.r_begin);
    t.r_end = __builtin_amdgcn_readfirstlane(t.r_end);
    t.split = __builtin_amdgcn_readfirstlane(t.split);
    return true;
  }
};

// ------------------------------------------------------------------ kernel --

// Fragment reads.  A 32x32x16 matrix-core operand gives lane l the 8
// reduction values 8*(l/32) + 0..7 of outer index l % 32 (within one k-slice
// of 16).  Both operands use the same assignment, so the products pair up.

// R-contiguous tile [outer][kBK]: one 128-bit read.
__device__ __forceinline__ bf16x8 frag_rc(const char* tile, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(tile + off);
}

// R-strided tile [kBK][outer]: two transpose loads of 4 reduction rows each.
// Within each 16-lane group, lane i's element j comes from the 8-byte word
// addressed by lane 4j + i/4, element i % 4; so lane i addresses row
// R0 + i/4, outer columns o0 + 4 (i % 4) .. +3, and receives column o0 + i of
// rows R0 .. R0 + 3.
__device__ __forceinline__ bf16x8 frag_rs(const char* tile, uint32_t off, uint32_t off4) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)(
                       (__attribute__((address_space(3))) void*)tile) + off));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)(
                       (__attribute__((address_space(3))) void*)tile) + off + off4));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

// Scaled fp8 product whose A and B scales are bytes i and j of sa and sb (the
// byte select is an immediate: i and j are constants once the caller's loops
// are unrolled, and the switch folds).
template <int I, int J>
__device__ __forceinline__ f32x16 mfma_mx_ij(const i32x8& a, const i32x8& b, const f32x16& c,
                                             uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, I, (int)sa, J, (int)sb);
}
__device__ __forceinline__ f32x16 mfma_mx(int i, int j, const i32x8& a, const i32x8& b,
                                          const f32x16& c, uint32_t sa, uint32_t sb) {
  switch (4 * i + j) {
    case 0: return mfma_mx_ij<0, 0>(a, b, c, sa, sb);
    case 1: return mfma_mx_ij<0, 1>(a, b, c, sa, sb);
    case 2: return mfma_mx_ij<0, 2>(a, b, c, sa, sb);
    case 3: return mfma_mx_ij<0, 3>(a, b, c, sa, sb);
    case 4: return mfma_mx_ij<1, 0>(a, b, c, sa, sb);
    case 5: return mfma_mx_ij<1, 1>(a, b, c, sa, sb);
    case 6: return mfma_mx_ij<1, 2>(a, b, c, sa, sb);
    case 7: return mfma_mx_ij<1, 3>(a, b, c, sa, sb);
    case 8: return mfma_mx_ij<2, 0>(a, b, c, sa, sb);
    case 9: return mfma_mx_ij<2, 1>(a, b, c, sa, sb);
    case 10: return mfma_mx_ij<2, 2>(a, b, c, sa, sb);
    case 11: return mfma_mx_ij<2, 3>(a, b, c, sa, sb);
    case 12: return mfma_mx_ij<3, 0>(a, b, c, sa, sb);
    case 13: return mfma_mx_ij<3, 1>(a, b, c, sa, sb);
    case 14: return mfma_mx_ij<3, 2>(a, b, c, sa, sb);
    default: return mfma_mx_ij<3, 3>(a, b, c, sa, sb);
  }
}

// The persistent body of one workgroup: a producer walks the tile list
// issuing LDS stages (tiles with an empty reduction have none), a consumer
// walks the same list consuming them and storing each tile's result.  Stage
// g of the launch lives in LDS buffer g % kStages.
template <int MODE, class C>
__device__ __forceinline__ void run_tiles(const KernelArgs& a, const Sched& S, char* lds,
                                          int Pdim, int Qdim) {
  constexpr bool SWI = MODE == kFwdSwiglu;
  constexpr bool LIST = MODE == kList;
  constexpr bool MXT = MODE == kWgradMxT;      // MXFP8 weight gradient on token-major operands
  constexpr bool MX = MODE == kFwdMx || MODE == kWgradMx || MXT;
  constexpr bool KG = MODE == kWgrad || MODE == kWgradMx || MXT;   // K-grouped, fp32 out
  constexpr bool DG = MODE == kDgrad || MODE == kDgradSwiglu;
  constexpr bool P_RS = DG || MODE == kWgrad || MXT;   // P is R-strided for dgrad and wgrad
  constexpr bool Q_RS = MODE == kWgrad || MXT;        // Q is R-strided for wgrad
  constexpr int SPW = C::SEGS_PER_WAVE;
  // element bytes, and reduction steps per stage (a staged row is kRowB bytes)
  constexpr int ES = MX ? 1 : 2;
  constexpr int BKE = kRowB / ES;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  int ldP, ldQ;
  if (MODE == kWgradMx) { ldP = (int)a.M; ldQ = (int)a.M; }   // X^T, dY^T rows of M tokens
  else if (MXT) { ldP = (int)a.K; ldQ = (int)a.N; }           // X8, dY8 rows of K, N codes
  else if (MODE == kFwd || SWI || LIST || MX) { ldP = (int)a.K; ldQ = (int)a.K; }   // LIST: per tile
  else if (DG) { ldP = (int)a.K; ldQ = (int)a.N; }
  else { ldP = (int)a.K; ldQ = (int)a.N; }

  // ---- direct-to-LDS plan: each stage is C::SEGS 1-KiB segments (the P tile
  // first, then the Q tile); wave w loads segments w*SPW .. w*SPW + SPW - 1.
  // The per-lane part (offset within the tile, column) is the same for every
  // tile; the base, the valid extents and the descriptor follow the tile.
  const bool wP = wave * SPW < C::SEGS_P;                    // wave-uniform
  const bool rs = wP ? P_RS : Q_RS;
  const int outer = wP ? C::BP : C::BQ;
  int ld = wP ? ldP : ldQ;              // LIST: the tile's group's row stride
  const int seg0 = wP ? wave * SPW : wave * SPW - C::SEGS_P;
  const uint32_t lds_base = lds_u32(lds) + (wP ? 0u : (uint32_t)C::P_BYTES) + seg0 * 1024u;
  uint32_t voff[SPW];
  int col[SPW];    // R-contiguous: reduction column; R-strided: outer column
  int orow[SPW];   // fused SwiGLU forward: the row's output column (P) or row (Q) in the tile
  // Fused SwiGLU forward: the P tile holds, for each wave row wp, the gate rows
  // (w13 rows p0 + 64 wp + 0..63) in its blocks 0-1 and the matching up rows
  // (w13 rows I + p0 + 64 wp + 0..63) in its blocks 2-3, so that acc[i][j]
  // and acc[i + 2][j] hold g and u of the same outputs.
  const int I2 = (int)(a.N / 2);
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int p = (seg0 + j) * 1024 + lane * 16;             // byte within the tile
    if (MXT) {                                               // [128 tokens][outer] fp8
      // rows of outer bytes in 16-byte chunks; chunk c of token row r sits at
      // chunk c ^ (2 (r % 8)), so that the transpose reads of 8 consecutive
      // rows at two neighbouring chunks hit 16 distinct chunks
      const int r = p / outer, pc = (p >> 4) % (outer / 16);
      const int c = pc ^ (2 * (r & 7));
      voff[j] = (uint32_t)(r * ld + 16 * c);
      col[j] = 16 * c;
      orow[j] = 0;
    } else if (rs) {                                         // [kBK][outer]
      const int r = p / (outer * 2), pc = (p >> 4) % (outer / 8);
      const int c = pc ^ rs_swz(r & 3);
      voff[j] = (uint32_t)(r * ld + 8 * c) * 2u;
      col[j] = 8 * c;
      orow[j] = 0;
    } else {                                                 // [outer][kBK]
      const int row = p / kRowB, pc = (p >> 4) % kRowChunks;
      const int c = pc ^ rc_swz(row);
      int grow = row;
      orow[j] = row;
      if (SWI && wP) {
        const int wr = row >> 7, blk = (row >> 5) & 3, in = row & 31;
        orow[j] = 64 * wr + 32 * (blk & 1) + in;
        grow = (blk < 2 ? 0 : I2) + orow[j];
      }
      voff[j] = (uint32_t)(grow * ld * ES + 16 * c);
      col[j] = 16 * c / ES;
    }
  }
  // MXFP8: every stage also carries the operands' scales, [BP][4] bytes of P
  // then [BQ][4] of Q, behind the data stages; a wave loads the dwords of
  // kScRows rows of its operand, 64 rows per 4-byte direct-to-LDS load, with
  // the stage's first kScLoads loads.
  constexpr int kScStage = MX ? (C::BP + C::BQ) * 4 : 0;
  constexpr int kScRows = C::BP / (C::SEGS_P / SPW);
  constexpr int kScLoads = MX ? kScRows / 64 : 0;
  static_assert(!MX || (kScRows % 64 == 0 && kScLoads <= SPW &&
                        C::BQ == kScRows * ((C::SEGS - C::SEGS_P) / SPW)), "scale rows per wave");
  const int w4 = seg0 / SPW;                // wave index within its operand
  // MXFP8 data loads, without per-load tables: load d of a wave covers rows
  // 8 (seg0 + d) + lane / 8 of its operand tile, and with seg0 a multiple of
  // 8 the swizzled chunk of that row is (lane % 8) ^ (lane / 8) ^ (d % 4).
  static_assert(!MX || MXT || (SPW % 8 == 0 && kRowChunks == 8), "MXFP8 load plan");
  const int mx_c0 = (lane & 7) ^ (lane >> 3);
  const uint32_t mx_rowoff = (uint32_t)(seg0 * 8 + (lane >> 3)) * (uint32_t)ld;
  // Token-major fp8 loads, without per-load tables: load d of a wave covers
  // token rows 4 (seg0 + d) + lane / 16 of its operand tile, logical chunk
  // lane % 16, which with seg0 a multiple of 2 sits at chunk
  // (lane % 16) ^ (2 ((4 (d % 2) + lane / 16) % 8)).
  static_assert(!MXT || (SPW % 2 == 0 && C::BP == 256), "token-major fp8 load plan");
  const uint32_t mxt_row = (uint32_t)(4 * seg0 + (lane >> 4)) * (uint32_t)ld;
  const uint32_t mxt_c0 = 16u * (uint32_t)((lane & 15) ^ (2 * ((lane >> 4) & 7)));
  const uint32_t mxt_c1 = 16u * (uint32_t)((lane & 15) ^ (2 * ((4 + (lane >> 4)) & 7)));
  const uint32_t sc_base = lds_u32(lds) + (uint32_t)C::LDS +
                           (wP ? 0u : (uint32_t)C::BP * 4u) + (uint32_t)(4 * kScRows) * w4;

  // Operand bases and valid extents of a tile.
  auto tile_src = [&](const Tile& t, const char*& src, int& nouter) {
    const char* P = reinterpret_cast<const char*>(a.p_src);
    const char* Q = reinterpret_cast<const char*>(a.q_src);
    if (MODE == kWgradMx) {        // P = X^T rows k (R = i), Q = dY^T rows n (R = i)
      P += (int64_t)t.p0 * a.M + t.r_begin;
      Q += (int64_t)t.q0 * a.M + t.r_begin;
    } else if (MXT) {              // P = X8 [i][k] R-strided, Q = dY8 [i][n] R-strided
      P += (int64_t)t.r_begin * a.K + t.p0;
      Q += (int64_t)t.r_begin * a.N + t.q0;
    } else if (MODE == kFwd || MX) {   // P = W[e] rows n (R = k), Q = X rows m (R = k)
      P += ((int64_t)t.e * a.N + t.p0) * a.K * ES;
      Q += (int64_t)t.q0 * a.K * ES;
    } else if (SWI) {              // P = W13[e] rows from p0 (gate; up at + I), Q = X rows
      P += ((int64_t)t.e * a.N + t.p0) * a.K * 2;
      if (a.gather == nullptr) Q += (int64_t)t.q0 * a.K * 2;
    } else if (LIST) {             // P = B_g rows n, Q = A_g rows m (R = k), own strides
      const ListDesc dg = list_desc(S.list, t.e);
      P = reinterpret_cast<const char*>(dg.b) + (int64_t)t.p0 * dg.ldb * 2;
      Q = reinterpret_cast<const char*>(dg.a) + (int64_t)t.q0 * dg.lda * 2;
    } else if (DG) {               // P = W[e] [n][k] R-strided, Q = dY rows m (R = n)
      P += ((int64_t)t.e * a.N * a.K + t.p0) * 2;
      Q += (int64_t)t.q0 * a.N * 2;
    } else {                       // P = X [i][k] R-strided, Q = dY [i][n] R-strided
      P += ((int64_t)t.r_begin * a.K + t.p0) * 2;
      Q += ((int64_t)t.r_begin * a.N + t.q0) * 2;
    }
    const int nP = (LIST ? list_desc(S.list, t.e).n : Pdim) - t.p0;
    const int nQ = KG ? Qdim - t.q0 : t.q_end - t.q0;
    src = wP ? P : Q;
    nouter = wP ? nP : nQ;
  };

  // ---- producer state (wave-uniform)
  TileSeq<MODE, C::BP, C::BQ> pseq;
  pseq.init(S);
  const char* p_src = nullptr;
  int p_nouter = 0, p_red = 0, p_nk = 0, p_kt = 0;
  i32x4 p_rc = {0, 0, 0, 0};
  bool p_live = false;
  uint32_t tvoff[SPW];            // fused SwiGLU forward: this tile's row offsets
  uint32_t tmask = 0;             // and which of the lane's rows are valid
  i32x4 sc_rc = {0, 0, 0, 0};     // MXFP8: the tile's scale descriptor,
  uint32_t sc_off = 0, sc_stride = 0;   // the lane's first scale row at stage 0, bytes per stage,
  uint32_t sc_ok = 0;                   // and which of the lane's rows (+ 64 i) are in the tile
#pragma unroll
  for (int j = 0; j < SPW; ++j) tvoff[j] = voff[j];
  auto p_next_tile = [&]() {
    Tile t;
    p_live = false;
    while (pseq.next(S, t)) {
      const int red = t.r_end - t.r_begin;
      const int nk = (red + BKE - 1) / BKE;
      if (nk <= 0) continue;                  // nothing to stage: the consumer stores zeros
      if (LIST) {
        // the group's row stride, and the lanes' row offsets under it
        const ListDesc dg = list_desc(S.list, t.e);
        ld = wP ? dg.ldb : dg.lda;
#pragma unroll
        for (int j = 0; j < SPW; ++j) tvoff[j] = (uint32_t)(orow[j] * ld + col[j]) * 2u;
        tmask = (1u << SPW) - 1u;             // rows past the group's end: descriptor range
      }
      tile_src(t, p_src, p_nouter);
      p_red = red;
      p_nk = nk;
      p_kt = 0;
      const int rows = p_nouter < outer ? (p_nouter > 0 ? p_nouter : 0) : outer;
      p_rc = make_rsrc(p_src, (uint32_t)rows * (uint32_t)ld * (uint32_t)ES);
      if (MX) {
        // blocked scales: stage s of row r at (s rows_total + r) 4 bytes; W's
        // per expert.  A row past the tile's valid rows reads zero.
        const int row = kScRows * w4 + lane;
        const int base = wP ? t.p0 : t.q0;
        if (MODE == kWgradMx || MXT) {
          // the operands' scales over all M tokens: the tile's stages start
          // at token stage r_begin / 128 (expert boundaries are multiples of 128)
          const int rows_total = wP ? Pdim : Qdim, ks = (int)((a.M + 127) / 128);
          const int end = rows_total;
          sc_rc = make_rsrc(wP ? a.p_scale : a.q_scale,
                            (uint32_t)ks * (uint32_t)rows_total * 4u);
          sc_off = (uint32_t)((t.r_begin >> 7) * rows_total + base + row) * 4u;
          sc_stride = (uint32_t)rows_total * 4u;
          sc_ok = 0;
#pragma unroll
          for (int i = 0; i < kScLoads; ++i) sc_ok |= (base + row + 64 * i < end ? 1u : 0u) << i;
        } else {
        const int ks = nk;                    // stages of the whole reduction (red = K)
        const int end = wP ? Pdim : t.q_end;
        if (wP)
          sc_rc = make_rsrc(a.p_scale + (int64_t)t.e * ks * a.N * 4,
                            (uint32_t)ks * (uint32_t)a.N * 4u);
        else
          sc_rc = make_rsrc(a.q_scale, (uint32_t)ks * (uint32_t)a.M * 4u);
        sc_off = (uint32_t)(base + row) * 4u;
        sc_stride = (uint32_t)(wP ? a.N : a.M) * 4u;
        sc_ok = 0;
#pragma unroll
        for (int i = 0; i < kScLoads; ++i) sc_ok |= (base + row + 64 * i < end ? 1u : 0u) << i;
        }
      }
      if (SWI) {
        tmask = 0;
        if (wP) {
          // gate and up rows of this tile: the descriptor spans the expert's
          // rows from p0 on; a column past I is masked
          p_rc = make_rsrc(p_src, (uint32_t)(a.N - t.p0) * (uint32_t)ld * 2u);
#pragma unroll
          for (int j = 0; j < SPW; ++j) tmask |= (t.p0 + orow[j] < I2 ? 1u : 0u) << j;
        } else if (a.gather != nullptr) {
          // gathered rows: offsets from the index, descriptor over all of x
          p_rc = make_rsrc(p_src, (uint32_t)a.T * (uint32_t)ld * 2u);
#pragma unroll
          for (int j = 0; j < SPW; ++j) {
            const bool ok = t.q0 + orow[j] < t.q_end;
            const int src = ok ? a.gather[t.q0 + orow[j]] : 0;
            tvoff[j] = (uint32_t)src * (uint32_t)ld * 2u + (uint32_t)col[j] * 2u;
            tmask |= (ok ? 1u : 0u) << j;
          }
        } else {
#pragma unroll
          for (int j = 0; j < SPW; ++j) tmask |= (orow[j] < p_nouter ? 1u : 0u) << j;
        }
      }
      p_live = true;
      return;
    }
    // No tile left: the refills that follow read nothing (see dma_begin).
    // (Not in the MXFP8 weight gradient, which sits at its register limit.)
    if (MODE != kWgradMx) {
      p_rc = make_rsrc(p_src, 0u);
      if (MX) sc_rc = make_rsrc(p_src, 0u);
    }
  };
  p_next_tile();

  // Vector-memory loads this wave has issued (uniform), and the count right
  // after each stage's loads: the loads of stage g are complete once at most
  // `issued - after[g % kStages]` operations are outstanding (loads complete
  // in order; stores are not counted, which only makes the wait stricter).
  int issued = 0, gp = 0;
  int after[kStages];
#pragma unroll
  for (int s = 0; s < kStages; ++s) after[s] = 0;

  auto stage_rsrc = [&](int r0) {
    if (!rs) return p_rc;
    const int rr = min(p_red - r0, BKE), oc = min(p_nouter, outer);
    const uint32_t bytes = rr > 0 && oc > 0 ? ((uint32_t)(rr - 1) * ld + oc) * (uint32_t)ES : 0u;
    return make_rsrc(p_src + (int64_t)r0 * ld * ES, bytes);
  };
  // Load d of the stage whose data go to `dst` (and, MXFP8, whose scales go
  // to `sdst`, loaded with the first loads); returns the vector-memory
  // operations issued.
  auto dma_one = [&](const i32x4& rsrc, uint32_t dst, uint32_t sdst, int d, int r0) {
    uint32_t off;
    if (MX && !MXT) {
      const int cj = 16 * (mx_c0 ^ (d & 3));
      uint32_t ro = mx_rowoff;
      // The weight gradient runs at the register limit: left alone, the
      // compiler keeps all SPW sums ro + d 8 ld live through the tile, they
      // spill, and every refill then waits on the reloads (vmcnt down to 0,
      // draining the stage in flight).  An opaque copy keeps them per load.
      if constexpr (MODE == kWgradMx) asm volatile("" : "+v"(ro));
      off = (ro + (uint32_t)d * 8u * (uint32_t)ld + (uint32_t)(cj + r0)) |
            (r0 + cj < p_red ? 0u : kOOB);
    } else if (MXT) {
      uint32_t ro = mxt_row;
      asm volatile("" : "+v"(ro));
      const uint32_t cj = (d & 1) ? mxt_c1 : mxt_c0;
      off = (ro + (uint32_t)d * 4u * (uint32_t)ld + cj) | ((int)cj < p_nouter ? 0u : kOOB);
    } else if (SWI || LIST)
      off = (tvoff[d] + (uint32_t)r0 * 2u) |
            (r0 + col[d] < p_red && ((tmask >> d) & 1u) ? 0u : kOOB);
    else
      off = rs ? (voff[d] | (col[d] < p_nouter ? 0u : kOOB))
               : ((voff[d] + (uint32_t)r0 * ES) | (r0 + col[d] < p_red ? 0u : kOOB));
    dma16(rsrc, dst + d * 1024u, off);
    if (MX && d < kScLoads) {
      const uint32_t so = (sc_off + 256u * d + (uint32_t)(r0 / BKE) * sc_stride) |
                          ((sc_ok >> d) & 1u ? 0u : kOOB);
      dma4(sc_rc, sdst + 256u * d, so);
      return 2;
    }
    return 1;
  };
  auto p_advance = [&]() {
    after[gp % kStages] = issued;
    ++gp;
    if (++p_kt == p_nk) p_next_tile();
  };
  // Issue the producer's next stage in one go.
  auto produce = [&]() {
    if (!p_live) return;
    const int r0 = p_kt * BKE;
    const uint32_t dst = lds_base + (uint32_t)((gp % kStages) * C::STAGE);
    const uint32_t sdst = sc_base + (uint32_t)((gp % kStages) * kScStage);
    const i32x4 rsrc = stage_rsrc(r0);
#pragma unroll
    for (int d = 0; d < SPW; ++d) issued += dma_one(rsrc, dst, sdst, d, r0);
    p_advance();
  };

  // ---- fragment addresses (byte offsets within an operand tile)
  const int wp = wave / C::WQ, wq = wave % C::WQ;
  const int l32 = lane & 31, h = lane >> 5, L = lane & 15, g16 = (lane >> 4) & 1;
  // k-slices per stage: 16 bf16 steps (one 16-byte read per lane), or, MXFP8,
  // 64 fp8 steps (two 16-byte reads per lane)
  constexpr int KR = kBK / 16;                 // 16-byte fragment reads per staged row and lane
  constexpr int KK = MX ? KR / 2 : KR;
  static_assert(KK % 2 == 0, "fragment double buffer parity");
  uint32_t offP[P_RS ? C::MP : KR], offQ[Q_RS ? C::MQ : KR];
  // R-contiguous: row = base + 32 i + l32 (swizzle depends on l32 only),
  // chunk 2 kk + h; entry kk, then + 32 kRowB i.
  // R-strided: row 8 h + L/4 (+ 16 kk + 4 t), outer base + 32 i + 16 g16 + 4 (L % 4).
  auto rs_off = [&](int obase, int i, int outer_) {
    const int o = obase + 32 * i + 16 * g16 + 4 * (L & 3);
    const int r = 8 * h + (L >> 2);
    return (uint32_t)(r * outer_ * 2 + (((o >> 3) ^ rs_swz(L >> 2)) << 4) + 8 * (L & 1));
  };
  auto rc_off = [&](int obase, int kk) {
    const int row = obase + l32;
    return (uint32_t)(row * kRowB + (((2 * kk + h) ^ rc_swz(l32)) << 4));
  };
  if (P_RS) {
#pragma unroll
    for (int i = 0; i < C::MP; ++i) offP[i] = rs_off(wp * C::WTP, i, C::BP);
  } else {
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) offP[kk] = rc_off(wp * C::WTP, kk);
  }
  if (Q_RS) {
#pragma unroll
    for (int j = 0; j < C::MQ; ++j) offQ[j] = rs_off(wq * C::WTQ, j, C::BQ);
  } else {
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) offQ[kk] = rc_off(wq * C::WTQ, kk);
  }
  // Token-major fp8 tiles [128 tokens][256 outer bytes] (MXFP8 weight gradient
  // on token-major operands), read with the 8-bit LDS transpose load: within
  // each 16-lane group, lane i receives byte i % 8 of the 8-byte words that
  // lanes 2 j + i / 8 address, j = 0..7.  So lane L of the group addresses
  // token row 16 h + L / 2 (+ 8 q for its q-th read) at outer bytes
  // o0 + 8 (L % 2), and lane i receives outer o0 + i of 8 consecutive tokens.
  // The fragment of outer block i sits 2 i chunks further, which with the
  // row swizzle is an XOR of 32 i on the lane's base.
  auto mxt_off = [&](int obase) {
    const int L = lane & 15, g16 = (lane >> 4) & 1;
    const int row = 16 * h + (L >> 1);
    const int chunk = ((obase >> 4) + g16) ^ (2 * (L >> 1));
    return (uint32_t)(row * 256 + 16 * chunk + 8 * (L & 1));
  };
  const uint32_t mxt_offP = MXT ? mxt_off(wp * C::WTP) : 0u;
  const uint32_t mxt_offQ = MXT ? mxt_off(wq * C::WTQ) : 0u;
  static_assert(!MXT || (C::BP == 256 && C::BQ == 256), "token-major fp8 rows of 256 bytes");

  f32x16 acc[C::MP][C::MQ];
#pragma unroll
  for (int i = 0; i < C::MP; ++i)
#pragma unroll
    for (int j = 0; j < C::MQ; ++j) acc[i][j] = f32x16{};

  // MXFP8 fragments.  The scaled 32x32x64 fp8 product takes from lane l
  // (outer index l % 32, h = l / 32) 32 bytes: bytes 0-15 are reduction
  // steps 16 h + 0..15 and bytes 16-31 steps 32 + 16 h + 0..15, so the first
  // 32 steps form one scale block and the last 32 the other; the scale of
  // block b of outer index r comes from lane r + 32 b.  Slice kk of a staged
  // row (bytes 64 kk .. 64 kk + 63 = MX blocks 2 kk, 2 kk + 1) is therefore
  // read as chunks 4 kk + h and 4 kk + 2 + h -- the bf16 reads of slices 2 kk
  // and 2 kk + 1 -- and lane l passes the scale byte 2 kk + h of its row.
  // The scales of a slice are packed one byte per block: byte i of sp is the
  // scale of P block i, byte j of sq that of Q block j, and the product picks
  // its byte with the instruction's scale byte select.
  typedef typename std::conditional<MX, i32x8, bf16x8>::type FragT;
  struct Frags {
    FragT p[C::MP], q[C::MQ];
    uint32_t sp, sq;
  };
  static_assert(!MX || (C::MP == 4 && C::MQ == 4), "one scale byte per block in a dword");
  // MXFP8 reads in two parts, so that the products can run between them: the
  // scale dwords of the rows (32 apart) ...
  auto mx_read_sc = [&](int g, uint32_t (&raw)[8]) {
    const char* sc = lds + C::LDS + (g % kStages) * kScStage;
    const uint32_t* rp = reinterpret_cast<const uint32_t*>(sc + (wp * C::WTP + l32) * 4);
    const uint32_t* rq = reinterpret_cast<const uint32_t*>(sc + C::BP * 4 + (wq * C::WTQ + l32) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      raw[i] = rp[32 * i];
      raw[4 + i] = rq[32 * i];
    }
  };
  // ... then their bytes 2 kk + h packed one per block, and the fragments
  auto mx_pack_read_fr = [&](int g, int kk, const uint32_t (&raw)[8], Frags& f) {
    if constexpr (MX) {
      const int sh = 8 * (2 * kk + h);
      auto pk = [&](int o) {
        const uint32_t lo = __builtin_amdgcn_perm(raw[o + 1] >> sh, raw[o] >> sh, 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm(raw[o + 3] >> sh, raw[o + 2] >> sh, 0x0c0c0400u);
        return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      };
      f.sp = pk(0);
      f.sq = pk(4);
      const char* tp = lds + (g % kStages) * C::STAGE;
      const char* tq = tp + C::P_BYTES;
      if constexpr (MXT) {
        // four transpose reads of 8 tokens each: tokens 16 h + 0..15 and
        // 32 + 16 h + 0..15 of the slice, the operand layout of the scaled product
        auto frag8t = [&](const char* tile, uint32_t off) {
          typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
          typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
          auto tr = [&](uint32_t o) {
            return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2*)((__attribute__((address_space(3))) char*)(
                                 (__attribute__((address_space(3))) void*)tile) + o));
          };
          const uint32_t base = off + (uint32_t)(kk * 64 * 256);
          const i32x2 a0 = tr(base), a1 = tr(base + 8 * 256), a2 = tr(base + 32 * 256),
                      a3 = tr(base + 40 * 256);
          const i32x4 lo = __builtin_shufflevector(a0, a1, 0, 1, 2, 3);
          const i32x4 hi = __builtin_shufflevector(a2, a3, 0, 1, 2, 3);
          return (i32x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
#pragma unroll
        for (int i = 0; i < C::MP; ++i) f.p[i] = frag8t(tp, mxt_offP ^ (uint32_t)(32 * i));
#pragma unroll
        for (int j = 0; j < C::MQ; ++j) f.q[j] = frag8t(tq, mxt_offQ ^ (uint32_t)(32 * j));
        return;
      }
      // chunk 2 kk' + h of a 128-byte row: offP[kk'] = offP[0] ^ (kk' << 5) (the
      // row base has no low bits and (2 kk' + h) ^ swz = (h ^ swz) ^ 2 kk'), which
      // keeps one address register per operand instead of four
      const uint32_t p0 = offP[0] ^ (uint32_t)(64 * kk), p1 = offP[0] ^ (uint32_t)(64 * kk + 32);
      const uint32_t q0 = offQ[0] ^ (uint32_t)(64 * kk), q1 = offQ[0] ^ (uint32_t)(64 * kk + 32);
      auto frag8 = [&](const char* tile, uint32_t off0, uint32_t off1) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(tile + off0);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(tile + off1);
        return (i32x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
#pragma unroll
      for (int i = 0; i < C::MP; ++i) f.p[i] = frag8(tp, p0 + i * 32 * kRowB, p1 + i * 32 * kRowB);
#pragma unroll
      for (int j = 0; j < C::MQ; ++j) f.q[j] = frag8(tq, q0 + j * 32 * kRowB, q1 + j * 32 * kRowB);
    }
  };
  auto read = [&](int g, int kk, Frags& f) {
    const char* tp = lds + (g % kStages) * C::STAGE;
    const char* tq = tp + C::P_BYTES;
    if constexpr (MX) {
      uint32_t raw[8];
      mx_read_sc(g, raw);
      mx_pack_read_fr(g, kk, raw, f);
      return;
    } else {
#pragma unroll
    for (int i = 0; i < C::MP; ++i)
      f.p[i] = P_RS ? frag_rs(tp, offP[i] + kk * 16 * C::BP * 2, 4 * C::BP * 2)
                    : frag_rc(tp, offP[kk] + i * 32 * kRowB);
#pragma unroll
    for (int j = 0; j < C::MQ; ++j)
      f.q[j] = Q_RS ? frag_rs(tq, offQ[j] + kk * 16 * C::BQ * 2, 4 * C::BQ * 2)
                    : frag_rc(tq, offQ[kk] + j * 32 * kRowB);
    }
  };
  // bf16 stage schedule (see the pipeline below): products of slice 1 before
  // the release; loads issued by the ends of slice 1, slice 2 and slice 3's
  // first part; products of slice 3 before the publish
  constexpr bool kEarly = !MX && KK == 4 && SPW == 8;
  constexpr int kRel = 2, kL1 = 2, kL2 = 5, kL3 = 6, kPub = 3;
  // MXFP8 stage schedule (16 products per slice, 16 data loads per stage):
  // products of slice 0 before the release; loads issued by the end of slice
  // 0 and before the publish; products of slice 1 before the publish
  constexpr int kMxRel = 4, kMxL0 = 6, kMxL1 = 10, kMxPub = 8;
  // Operations of the following stage's refill issued before the publish
  // wait in steady state: kL3 (bf16), half a stage's loads (other bf16
  // configurations), or MXFP8's kMxL1 data loads and the scale loads (issued
  // with the first data loads).
  constexpr int kSteady = kEarly ? kL3 : MX ? kMxL1 + (kScLoads < kMxL1 ? kScLoads : kMxL1)
                                           : SPW / 2;
  // wait until this wave's loads of stage g have landed
  auto wait_stage = [&](int g) {
    int n = issued - after[g % kStages];
    n = n < 0 ? 0 : n;
    // The steady-state count is tested first, on the fall-through path: the
    // chain below costs several taken branches per stage, which measurably
    // slows the stage loop.  (The counts that occur otherwise are exact
    // steps: fewer loads at a tile or list end, or a whole stage's.)
    if (__builtin_expect(n == kSteady, 1)) {
      wait_vmcnt<kSteady>();
      return;
    }
    if (n >= 24) wait_vmcnt<24>();
    else if (n >= 16) { if (n >= 20) wait_vmcnt<20>(); else if (n >= 18) wait_vmcnt<18>(); else wait_vmcnt<16>(); }
    else if (n >= 8) { if (n >= 12) wait_vmcnt<12>(); else if (n >= 10) wait_vmcnt<10>(); else wait_vmcnt<8>(); }
    else if (n >= 4) { if (n >= 6) wait_vmcnt<6>(); else wait_vmcnt<4>(); }
    else if (n >= 2) wait_vmcnt<2>();
    else wait_vmcnt<0>();
  };

  constexpr int kMM = C::MP * C::MQ;            // products per k-slice per wave
  // Products x0 .. x1-1 of one k-slice with the producer's loads d0 .. d1-1
  // (of the stage set up in `sd`) spread evenly between them.
  struct StageDma {
    int r0;
    uint32_t dst, sdst;
    i32x4 rsrc;
    bool on;
  };
  auto dma_begin = [&]() {
    StageDma sd;
    sd.on = p_live;
    sd.r0 = 0;
    sd.dst = 0;
    sd.sdst = 0;
    sd.rsrc = p_rc;
    if (sd.on) {
      sd.r0 = p_kt * BKE;
      sd.dst = lds_base + (uint32_t)((gp % kStages) * C::STAGE);
      sd.sdst = sc_base + (uint32_t)((gp % kStages) * kScStage);
      sd.rsrc = stage_rsrc(sd.r0);
    } else if (MODE != kWgradMx) {
      // No stage left to stage: the refill's loads still go out, through the
      // producer's descriptors of range zero (they read nothing and write
      // zeros), into the buffer the producer would fill next, which no stage
      // still to be consumed occupies.  The stage loop then carries no branch
      // around its loads (1-3% on the bf16 launches, 2-17% on the MXFP8
      // forward and token-major weight gradient); the kernel waits for these
      // loads before it ends.
      sd.dst = lds_base + (uint32_t)((gp % kStages) * C::STAGE);
      sd.sdst = sc_base + (uint32_t)((gp % kStages) * kScStage);
      sd.rsrc = p_rc;
    }
    return sd;
  };
  auto mma_part = [&](const Frags& f, int x0, int x1, const StageDma& sd, int d0, int d1) {
    int d = d0;
#pragma unroll
    for (int x = x0; x < x1; ++x) {
      const int i = x / C::MQ, j = x % C::MQ;
      if constexpr (MX) {
        acc[i][j] = mfma_mx(i, j, f.p[i], f.q[j], acc[i][j], f.sp, f.sq);
        // An empty use of the result (in its accumulator register) keeps the
        // product where it is written: the scaled product's builtin has no
        // side effects, and without the use the compiler moves a slice's
        // products past the loads, waits and barriers that follow, towards
        // their next use, and the one wave of the SIMD then waits at each
        // barrier with no product queued.  (The bf16 products stay in place.)
        const float pin = acc[i][j][0];
        asm volatile("" ::"a"(pin));
      } else
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.p[i], f.q[j], acc[i][j], 0, 0, 0);
      // after product x, (x - x0 + 1) (d1 - d0) / (x1 - x0) loads are due
      while (d < d1 && (d - d0) * (x1 - x0) < (x - x0 + 1) * (d1 - d0)) {
        if (MODE != kWgradMx || sd.on) {
          __builtin_amdgcn_sched_barrier(0);
          issued += dma_one(sd.rsrc, sd.dst, sd.sdst, d, sd.r0);
          __builtin_amdgcn_sched_barrier(0);
        }
        ++d;
      }
    }
    if (sd.on && d1 == SPW && d0 < d1) p_advance();   // this part issued the stage's last load
  };

  // Result block (i, j) of the matrix cores: lane l holds Q index l % 32 and,
  // in accumulator registers 4g .. 4g+3, the four consecutive P indices of
  // 16-byte chunk 2g + l/32 (P indices 8g + 4(l/32) + 0..3).  A store
  // instruction then touches 32 output rows; the memory pipeline handles about
  // one row per cycle, so the lanes are first regrouped with the lane-half
  // swaps of gfx950 so that each store covers 16 rows x 64 contiguous bytes:
  //  fp32: v_permlane16_swap between chunk pairs (2g', 2g'+1) leaves register
  //    group g holding row (l % 16) + 16 (g % 2), chunk (l / 32) + 2 ((l / 16) % 2)
  //    + 4 (g / 2): 4 stores of 16 B per block;
  //  bf16: 8-byte chunks; v_permlane16_swap between groups (g, g+2) then
  //    v_permlane32_swap between (2g', 2g'+1) leave lane l holding rows (l % 16)
  //    and (l % 16) + 16, chunks c, c+1 with c = 4 ((l / 16) % 2) + 2 (l / 32):
  //    2 stores of 16 B per block.
  auto swap16 = [](uint32_t& x, uint32_t& y) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    x = r[0];
    y = r[1];
  };
  auto swap32 = [](uint32_t& x, uint32_t& y) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    x = r[0];
    y = r[1];
  };
  const int l16 = lane & 15, pa = (lane >> 4) & 1, pb = lane >> 5;
  // Where a tile's bf16 result goes: the output, its row stride and column
  // bound (the descriptor list's group has its own; read once per tile, as
  // the stores could otherwise be taken to alias the descriptors).
  struct OutView {
    uint16_t* out;
    int ldo, pbound;
  };
  auto out_view = [&](const Tile& t) {
    OutView v;
    if (LIST) {
      const ListDesc dg = list_desc(S.list, t.e);
      v.out = reinterpret_cast<uint16_t*>(dg.d);
      v.ldo = dg.ldd;
      v.pbound = dg.n;
    } else {
      v.out = reinterpret_cast<uint16_t*>(a.out);
      v.ldo = Pdim;
      v.pbound = Pdim;
    }
    return v;
  };
  // Result block (i, j) held in `blk` (the register layout of acc[i][j]).
  auto store_block = [&](const Tile& t, const OutView& ov, int i, int j, const f32x16& blk) {
    if (KG) {
      float* out = reinterpret_cast<float*>(a.out) + (int64_t)t.e * a.N * a.K;
      const int c = pb + 2 * pa;                          // chunk of groups 0 and 1
      // (each element goes through a named float: this compiler lowers
      // __builtin_bit_cast of an ext_vector element as a copy of element 0)
      uint32_t v[4][4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = blk[4 * g + e];
          v[g][e] = __builtin_bit_cast(uint32_t, f);
        }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        swap16(v[0][e], v[1][e]);
        swap16(v[2][e], v[3][e]);
      }
      const int n0 = t.q0 + wq * C::WTQ + j * 32 + l16;
      const int k0 = t.p0 + wp * C::WTP + i * 32 + 4 * c;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 16 * (g & 1), k = k0 + 16 * (g >> 1);
        if (n >= Qdim || k >= Pdim) continue;
        f32x4 r = {__builtin_bit_cast(float, v[g][0]), __builtin_bit_cast(float, v[g][1]),
                   __builtin_bit_cast(float, v[g][2]), __builtin_bit_cast(float, v[g][3])};
        f32x4* dst = reinterpret_cast<f32x4*>(out + (int64_t)n * a.K + k);
        if (a.accumulate) r += *dst;
        *dst = r;
      }
    } else {
      uint16_t* out = ov.out;
      const int ldo = ov.ldo;
      const int pbound = ov.pbound;
      const int c = 4 * pa + 2 * pb;                      // first of the lane's two chunks
      uint32_t v[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2 lo = __builtin_convertvector((f32x2){blk[4 * g], blk[4 * g + 1]}, bf16x2);
        const bf16x2 hi =
            __builtin_convertvector((f32x2){blk[4 * g + 2], blk[4 * g + 3]}, bf16x2);
        v[g][0] = __builtin_bit_cast(uint32_t, lo);
        v[g][1] = __builtin_bit_cast(uint32_t, hi);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        swap16(v[0][e], v[2][e]);
        swap16(v[1][e], v[3][e]);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        swap32(v[0][e], v[1][e]);
        swap32(v[2][e], v[3][e]);
      }
      const int m0 = t.q0 + wq * C::WTQ + j * 32 + l16;
      const int col = t.p0 + wp * (SWI ? C::WTP / 2 : C::WTP) + i * 32 + 4 * c;
      if (col >= pbound) return;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int m = m0 + 16 * half;
        if (m >= t.q_end) continue;
        const u32x4 pk = {v[2 * half][0], v[2 * half][1], v[2 * half + 1][0],
                          v[2 * half + 1][1]};
        *reinterpret_cast<u32x4*>(out + (int64_t)m * ldo + col) = pk;
      }
    }
  };
  // h = silu(g) u = g u / (1 + e^-g), in fp32 (e^-g = 2^(-g log2 e) with the
  // hardware base-2 exponential; an overflow gives h = -0 or 0, never NaN
  // for finite g and u)
  auto swiglu = [](const f32x16& g, const f32x16& u) {
    f32x16 h;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float gv = g[e];
      const float ex = __builtin_amdgcn_exp2f(-gv * 1.4426950408889634f);
      h[e] = gv / (1.0f + ex) * u[e];
    }
    return h;
  };
  // SwiGLU backward on result block (i, j) (dh, fp32): the lanes are regrouped
  // as for the bf16 store, but on the fp32 values, so that each lane holds 8
  // consecutive columns of two rows; it loads those columns of g and u (16
  // bytes each) and stores dg and du.
  auto store_dswiglu = [&](const Tile& t, int i, int j, const f32x16& blk) {
    const int I = (int)a.K;
    uint32_t v[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = blk[4 * g + e];
        v[g][e] = __builtin_bit_cast(uint32_t, f);
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      swap16(v[0][e], v[2][e]);
      swap16(v[1][e], v[3][e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      swap32(v[0][e], v[1][e]);
      swap32(v[2][e], v[3][e]);
    }
    const int c = 4 * pa + 2 * pb;
    const int m0 = t.q0 + wq * C::WTQ + j * 32 + l16;
    const int col = t.p0 + wp * C::WTP + i * 32 + 4 * c;
    if (col >= I) return;
    const uint16_t* gu = reinterpret_cast<const uint16_t*>(a.aux);
    uint16_t* dgu = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int m = m0 + 16 * half;
      if (m >= t.q_end) continue;
      const int64_t row = (int64_t)m * (2 * I);
      const u32x4 gw = *reinterpret_cast<const u32x4*>(gu + row + col);
      const u32x4 uw = *reinterpret_cast<const u32x4*>(gu + row + I + col);
      u32x4 dg, du;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // columns 2q, 2q + 1: fp32 dh from v[2 half + q / 2][2 (q % 2) + 0..1]
        const float dh0 = __builtin_bit_cast(float, v[2 * half + q / 2][2 * (q % 2)]);
        const float dh1 = __builtin_bit_cast(float, v[2 * half + q / 2][2 * (q % 2) + 1]);
        const float g0 = __builtin_bit_cast(float, gw[q] << 16);
        const float g1 = __builtin_bit_cast(float, gw[q] & 0xFFFF0000u);
        const float u0 = __builtin_bit_cast(float, uw[q] << 16);
        const float u1 = __builtin_bit_cast(float, uw[q] & 0xFFFF0000u);
        const float s0 = 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g0 * 1.4426950408889634f));
        const float s1 = 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g1 * 1.4426950408889634f));
        const bf16x2 a2 = __builtin_convertvector(
            (f32x2){dh0 * u0 * (s0 * (1.0f + g0 * (1.0f - s0))), dh1 * u1 * (s1 * (1.0f + g1 * (1.0f - s1)))},
            bf16x2);
        const bf16x2 b2 = __builtin_convertvector((f32x2){dh0 * (g0 * s0), dh1 * (g1 * s1)}, bf16x2);
        dg[q] = __builtin_bit_cast(uint32_t, a2);
        du[q] = __builtin_bit_cast(uint32_t, b2);
      }
      *reinterpret_cast<u32x4*>(dgu + row + col) = dg;
      *reinterpret_cast<u32x4*>(dgu + row + I + col) = du;
    }
  };
  auto store_tile = [&](const Tile& t) {
    if (MODE == kDgradSwiglu) {
#pragma unroll
      for (int j = 0; j < C::MQ; ++j)
#pragma unroll
        for (int i = 0; i < C::MP; ++i) store_dswiglu(t, i, j, acc[i][j]);
      return;
    }
    if (KG && a.accumulate && t.r_end <= t.r_begin) return;   // adds nothing
    const OutView ov = out_view(t);
    if (SWI) {
#pragma unroll
      for (int j = 0; j < C::MQ; ++j)
#pragma unroll
        for (int i = 0; i < C::MP / 2; ++i)
          store_block(t, ov, i, j, swiglu(acc[i][j], acc[i + C::MP / 2][j]));
      if (a.aux != nullptr) {
        // the pre-activation g | u for the backward: gu [M, 2I]
        const int I2 = Pdim;
        const OutView og = {reinterpret_cast<uint16_t*>(a.aux), 2 * I2, I2};
        const OutView ou = {reinterpret_cast<uint16_t*>(a.aux) + I2, 2 * I2, I2};
#pragma unroll
        for (int j = 0; j < C::MQ; ++j)
#pragma unroll
          for (int i = 0; i < C::MP / 2; ++i) {
            store_block(t, og, i, j, acc[i][j]);
            store_block(t, ou, i, j, acc[i + C::MP / 2][j]);
          }
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < C::MQ; ++j)
#pragma unroll
      for (int i = 0; i < C::MP; ++i) store_block(t, ov, i, j, acc[i][j]);
  };

  // ---- end of a half of a split K-grouped tile.  Each half writes its fp32
  // accumulators to its own workspace slot (in register order: entry
  // (i MQ + j) 4 + g of thread tid at ((i MQ + j) 4 + g) NT + tid), waits for
  // the writes and swaps the launch's odd mark into the tile's ticket word:
  // the half that finds the mark already there ends second and stores (own +
  // other) -- a commutative sum, so the result does not depend on which half
  // ends last -- plus the prior value when accumulating, then clears the
  // word.  The mark is 2 g + 1 for the launch count g of the workspace, so a
  // word left behind by an earlier launch (one cleared, or one that never
  // completed) never equals it; clearing keeps repeated launches with one
  // mark (a replayed graph) correct.  Nothing waits for another workgroup.
  // The slots are written and read with device-scope accesses (cache policy
  // sc1: the store is acknowledged once it is visible device-wide, the load
  // misses every cache that is not coherent device-wide), the stores are
  // waited for (vmcnt) before the exchange, and the exchange is a
  // device-scope atomic, so no cache is written back or invalidated.
  constexpr int kSlotFloats = C::BP * C::BQ;
  constexpr int kCoherent = 16;                 // cache policy bit sc1
  auto finish_half = [&](const Tile& t) {
    const int sid = t.split >> 1, half = t.split & 1;
    // (an opaque zero added to the constant entry offsets keeps the compiler
    // from hoisting 32 of them into registers for the whole kernel)
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    auto slot_rsrc = [&](int slot) {
      return __builtin_amdgcn_make_buffer_rsrc(a.ws + (int64_t)slot * kSlotFloats, (short)0,
                                               kSlotFloats * 4, 0x00020000);
    };
    {
      const auto rs = slot_rsrc(2 * sid + half);
#pragma unroll
      for (int ii = 0; ii < C::MP; ++ii)
#pragma unroll
        for (int jj = 0; jj < C::MQ; ++jj)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 v = {acc[ii][jj][4 * g4], acc[ii][jj][4 * g4 + 1], acc[ii][jj][4 * g4 + 2],
                             acc[ii][jj][4 * g4 + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(i32x4, v), rs, tid * 16,
                z + ((ii * C::MQ + jj) * 4 + g4) * C::NT * 16, kCoherent);
          }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t* ticket = a.tickets + sid;
    if (tid == 0)
      S.scan[8] = __hip_atomic_exchange(ticket, a.ticket_mark, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == a.ticket_mark ? 1 : 0;
    __syncthreads();
    if (S.scan[8] == 0) return;                 // the other half finishes the tile
    const OutView ov = out_view(t);
    const auto rs = slot_rsrc(2 * sid + (half ^ 1));
#pragma unroll
    for (int jj = 0; jj < C::MQ; ++jj)
#pragma unroll
      for (int ii = 0; ii < C::MP; ++ii) {
        f32x4 v[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          v[g4] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         rs, tid * 16, z + ((ii * C::MQ + jj) * 4 + g4) * C::NT * 16, kCoherent));
        const f32x8 lo = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
        const f32x8 hi = __builtin_shufflevector(v[2], v[3], 0, 1, 2, 3, 4, 5, 6, 7);
        const f32x16 other = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10,
                                                     11, 12, 13, 14, 15);
        store_block(t, ov, ii, jj, acc[ii][jj] + other);
      }
    if (tid == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // ---- pipeline.  Stage g is consumed in KK k-slices; while slice kk's
  // products run, the next slice is read.  Two barriers per stage:
  //  - release: once every wave holds the stage's remaining slices in
  //    registers (each waits for its own LDS reads before arriving), stage g's
  //    buffer is free and the producer's stage g + kStages is issued into it,
  //    its loads spread between the remaining products -- it does not wait
  //    for stage g+1 to land;
  //  - publish: in the last slice, once this wave's loads of stage g+1 have
  //    landed; stage g+1's first slice is read while the rest of the last
  //    slice's products run.
  // bf16 (four slices, eight loads per wave and stage): slices 2 and 3 are
  // both read during slice 1, and the release comes after slice 1's second
  // product, so the refill gets about two slices more lead than with a
  // release in the last slice, and its loads are spread at about one per 2.5
  // products (denser bursts slow the products and the fragment reads that
  // share the CU's memory path).  Slices 0 and 2 go to fr[0], slice 1 to
  // fr[1], slice 3 to fr3.  MXFP8 (two slices of 64 steps): the release
  // follows slice 0's fourth product, once slice 1 is in registers.  The other
  // compile-time configurations read one slice ahead and release in the last
  // slice.
#pragma unroll
  for (int s = 0; s < kStages; ++s) produce();   // every buffer is free at the start
  TileSeq<MODE, C::BP, C::BQ> cseq;
  cseq.init(S);
  Frags fr[2];
  Frags fr3;                                   // bf16: slice 3 of the stage
  const StageDma sd_none = {0, 0u, 0u, p_rc, false};
  StageDma refill = sd_none;                   // the refill being issued
  int g = 0;
  if (gp > 0) {
    wait_stage(0);
    __syncthreads();
    read(0, 0, fr[0]);
  }
  Tile ct;
  while (cseq.next(S, ct)) {
    const int nk = (ct.r_end - ct.r_begin + BKE - 1) / BKE;
    for (int kt = 0; kt < nk; ++kt, ++g) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        Frags& cur = fr[kk & 1];
        Frags& nxt = fr[(kk + 1) & 1];
        if constexpr (MX) {
          // Two slices of 64 steps per stage.  Slice 0: the next slice's scale
          // reads go first; they are packed after two products, when they have
          // landed, and only then are the fragment reads issued (a pack right
          // behind all the reads would wait for most of them: the LDS counter
          // tracks at most 15 in order, and one wave per SIMD leaves the
          // matrix core idle meanwhile).  Once slice 1 is in registers (after
          // kMxRel products) the stage's buffer is released and the refill
          // issued, spread over the rest of slice 0 and slice 1; the publish
          // of the next stage follows slice 1's kMxPub-th product.
          static_assert(KK == 2, "MXFP8 stages of two 64-step slices");
          constexpr int X2 = 2;
          uint32_t raw[8];
          if (kk == 0) {
            mx_read_sc(g, raw);
            __builtin_amdgcn_sched_barrier(0);
            mma_part(cur, 0, X2, sd_none, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            mx_pack_read_fr(g, 1, raw, nxt);
            __builtin_amdgcn_sched_barrier(0);
            mma_part(cur, X2, kMxRel, sd_none, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();                    // release stage g's buffer
            refill = dma_begin();
            __builtin_amdgcn_sched_barrier(0);
            mma_part(cur, kMxRel, kMM, refill, 0, kMxL0);
            __builtin_amdgcn_sched_barrier(0);
          } else {
            const bool more = g + 1 < gp;
            mma_part(cur, 0, kMxPub, refill, kMxL0, kMxL1);
            __builtin_amdgcn_sched_barrier(0);
            if (more) {
              wait_stage(g + 1);
              __syncthreads();                  // publish stage g+1
              mx_read_sc(g + 1, raw);
            }
            __builtin_amdgcn_sched_barrier(0);
            mma_part(cur, kMxPub, kMxPub + X2, refill, kMxL1, kMxL1 + 2);
            __builtin_amdgcn_sched_barrier(0);
            if (more) mx_pack_read_fr(g + 1, 0, raw, nxt);
            __builtin_amdgcn_sched_barrier(0);
            mma_part(cur, kMxPub + X2, kMM, refill, kMxL1 + 2, SPW);
            __builtin_amdgcn_sched_barrier(0);
          }
          continue;
        }
        if constexpr (kEarly) {
          if (kk == 0) {
            read(g, 1, fr[1]);
            __builtin_amdgcn_sched_barrier(0);
            mma_part(fr[0], 0, kMM, sd_none, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          } else if (kk == 1) {
            read(g, 2, fr[0]);
            read(g, 3, fr3);
            __builtin_amdgcn_sched_barrier(0);
            mma_part(fr[1], 0, kRel, sd_none, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();                    // release stage g's buffer
            refill = dma_begin();
            __builtin_amdgcn_sched_barrier(0);
            mma_part(fr[1], kRel, kMM, refill, 0, kL1);
            __builtin_amdgcn_sched_barrier(0);
          } else if (kk == 2) {
            mma_part(fr[0], 0, kMM, refill, kL1, kL2);
            __builtin_amdgcn_sched_barrier(0);
          } else {
            const bool more = g + 1 < gp;
            mma_part(fr3, 0, kPub, refill, kL2, kL3);
            __builtin_amdgcn_sched_barrier(0);
            if (more) {
              wait_stage(g + 1);
              __syncthreads();                  // publish stage g+1
              read(g + 1, 0, fr[0]);
            }
            __builtin_amdgcn_sched_barrier(0);
            mma_part(fr3, kPub, kMM, refill, kL3, SPW);
            __builtin_amdgcn_sched_barrier(0);
          }
          continue;
        }
        if (kk + 1 < KK) {
          read(g, kk + 1, nxt);
          __builtin_amdgcn_sched_barrier(0);
          mma_part(cur, 0, kMM, sd_none, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        } else {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __syncthreads();
          const bool more = g + 1 < gp;
          const StageDma sd = dma_begin();
          __builtin_amdgcn_sched_barrier(0);
          mma_part(cur, 0, kMM / 2, sd, 0, SPW / 2);
          __builtin_amdgcn_sched_barrier(0);
          if (more) {
            wait_stage(g + 1);
            __syncthreads();
            read(g + 1, 0, nxt);
          }
          __builtin_amdgcn_sched_barrier(0);
          mma_part(cur, kMM / 2, kMM, sd, SPW / 2, SPW);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (MODE == kWgrad && ct.split >= 0) finish_half(ct);
    else store_tile(ct);
#pragma unroll
    for (int i = 0; i < C::MP; ++i)
#pragma unroll
      for (int j = 0; j < C::MQ; ++j) acc[i][j] = f32x16{};
  }
  // the last refill loads (issued with no stage left) land in this
  // workgroup's LDS: wait for them before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int MODE, class C>
__global__ __launch_bounds__(C::NT)
void grouped_gemm_kernel(KernelArgs a) {
  constexpr bool KG = MODE == kWgrad || MODE == kWgradMx || MODE == kWgradMxT;
  constexpr bool MXM = MODE == kFwdMx || MODE == kWgradMx || MODE == kWgradMxT;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS + (MXM ? kStages * (C::BP + C::BQ) * 4 : 0)];
  // keys [64] | scan [16] | mine [2 kMaxExperts + 8] | pref [E+1] | offs [E+1] | inv [E]
  // (keys and mine 16-byte aligned: they are read four entries at a time)
  __shared__ __attribute__((aligned(16))) int sched[64 + 16 + 2 * kMaxExperts + 8 +
                                                   2 * (kMaxExperts + 1) + kMaxExperts];

  int Pdim, Qdim;
  if (MODE == kFwd || MODE == kFwdMx) {
    Pdim = (int)a.N; Qdim = (int)a.M;
  } else if (MODE == kFwdSwiglu) {
    Pdim = (int)(a.N / 2); Qdim = (int)a.M;      // outputs: I = N / 2 columns
  } else if (MODE == kList) {
    Pdim = 0; Qdim = 0;                          // per group, from the descriptors
  } else if (MODE == kDgrad || MODE == kDgradSwiglu) {
    Pdim = (int)a.K; Qdim = (int)a.M;
  } else {
    Pdim = (int)a.K; Qdim = (int)a.N;
  }
  const int E = a.E;
  Sched S;
  S.keys = sched;
  S.scan = sched + 64;
  S.mine = sched + 80;
  S.pref = S.mine + 2 * kMaxExperts + 8;
  S.offs = S.pref + (E + 1);
  S.inv = S.offs + (E + 1);
  S.nmine = 0;
  S.E = E;
  constexpr int kPStep = MODE == kFwdSwiglu ? C::BP / 2 : C::BP;
  S.tilesP = MODE == kList ? 1 : (Pdim + kPStep - 1) / kPStep;
  S.list = MODE == kList ? a.list : nullptr;
  S.tilesQ = (Qdim + C::BQ - 1) / C::BQ;
  S.red = MODE == kFwd || MODE == kFwdSwiglu || MODE == kFwdMx ? (int)a.K : (int)a.N;
  // raster group: about sqrt(nx) M-tiles, more when there are few P-tiles,
  // so that the nx tiles an XCD runs at once span ~gm x (nx / gm) panels
  const int nx = gridDim.x >> 3;
  int gm = 1;
  while (gm * gm < nx) ++gm;
  S.gm = max(gm, (nx + S.tilesP - 1) / S.tilesP);
  S.per = S.tilesQ * S.tilesP;
  // band width ~ sqrt(per / 8): a chunk of per/8 tiles is then ~bw x bw
  int bw = 1;
  while (bw < S.tilesP && 2 * (2 * bw + 1) * (2 * bw + 1) <= S.per) ++bw;
  S.bw = bw;
  // (the MXFP8 weight gradient does not split: its registers are all taken)
  S.split = MODE == kWgrad && a.ws != nullptr && a.tickets != nullptr;
  S.whole = MODE == kWgrad;                  // (the set-up keeps it only for equal experts)
  if (KG) {
    setup_kgrouped<C::NT>(a.offsets, E, (int)a.M, S);
    balance_kgrouped<C::NT>(blockIdx.x & 7, blockIdx.x >> 3, nx, S);
  } else if (MODE == kList) {
    setup_list<C::NT, C::BP, C::BQ>(a.list, E, S);
  } else {
    setup_mgrouped<C::NT, C::BQ>(a.offsets, E, (int)a.M, S);
  }
  run_tiles<MODE, C>(a, S, lds, Pdim, Qdim);
}


// ------------------------------------------------------------ host launch --

#if MG_WAVES == 8
using Cfg = TileCfg<256, 256, 2, 4>;    // 8 waves (2 per SIMD), 128x64 per wave
#else
using Cfg = TileCfg<256, 256, 2, 2>;    // 4 waves (1 per SIMD), 128x128 per wave
#endif
// MXFP8: one wave per SIMD, 128x128 per wave.  Its 32-byte fp8 fragments,
// double-buffered, and 16 accumulator blocks need more than the 256
// registers a wave has when two share a SIMD; alone it has 512.
using CfgMx = TileCfg<256, 256, 2, 2>;
static_assert(CfgMx::BP == Cfg::BP && CfgMx::BQ == Cfg::BQ, "one tile size for the launch sizing");

// Compute units of the current device (one resident workgroup each).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Token-split workspace: the ticket words (one per split tile) followed by two
// fp32 slots of one tile per split tile.
constexpr int kSplitTiles = 8 * kSplitPerXcd;
constexpr size_t kTicketBytes = 4096;
constexpr size_t kWorkspaceBytes =
    kTicketBytes + (size_t)2 * kSplitTiles * Cfg::BP * Cfg::BQ * sizeof(float);
static_assert(kSplitTiles * sizeof(uint32_t) <= kTicketBytes, "ticket area");
constexpr int kMaxDevices = 64;

// Per (device, stream): allocated on the first weight-gradient launch of the
// pair that is not being captured into a graph, its tickets cleared there
// (synchronously, not on the caller's stream), and kept until the process
// ends.  Launches on one stream run in order and share it; launches on
// different streams never do.  `launches` numbers the pair's launches for
// the ticket marks.
struct Workspace {
  int dev;
  hipStream_t stream;
  char* base;
  uint32_t launches;
};
static std::mutex g_ws_mutex;
static std::vector<Workspace> g_ws;

// The pair's workspace and this launch's ticket mark, or nullptr (no split).
static char* stream_workspace(hipStream_t s, uint32_t* mark) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  for (Workspace& w : g_ws)
    if (w.dev == dev && w.stream == s) {
      *mark = 2u * (++w.launches & 0x7FFFFFFFu) + 1u;
      return w.base;
    }
  void* p = nullptr;
  if (hipMalloc(&p, kWorkspaceBytes) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;                       // no workspace: launches do not split
  }
  if (hipMemset(p, 0, kTicketBytes) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(p);
    return nullptr;
  }
  g_ws.push_back({dev, s, static_cast<char*>(p), 1u});
  *mark = 3u;
  return static_cast<char*>(p);
}

// The static workspace: one array per device, zero at load, which the
// no-allocation entry point uses in place of the per-stream one.  Its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current); in host code the array's own name is not a device address.
static_assert(kWorkspaceBytes == MG_NOALLOC_SCRATCH_BYTES, "the size kgemm_wgrad_noalloc states");
static __device__ __align__(256) char scratch[kWorkspaceBytes];
static std::mutex g_scratch_mutex;
static char* g_scratch_ptr[kMaxDevices];
static uint32_t g_scratch_launches[kMaxDevices];

static int static_workspace(char** base, uint32_t* mark) {
  int dev = 0;
  int err = (int)hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = (int)hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr) return err != hipSuccess ? err : (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *base = g_scratch_ptr[dev];
  *mark = 2u * (++g_scratch_launches[dev] & 0x7FFFFFFFu) + 1u;
  return hipSuccess;
}

// MGEMM_SPLIT=0 turns the token split off (every tile is then computed whole).
static bool split_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("MGEMM_SPLIT");
    return !(v != nullptr && v[0] == '0');
  }();
  return on;
}

// Whether work enqueued on `s` now would be captured into a graph.
static bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) {
    (void)hipGetLastError();
    return true;                          // unknown: take the path that allocates nothing
  }
  return st != hipStreamCaptureStatusNone;
}

int launch_grouped(int mode, const KernelArgs& a_in, int64_t max_m_per_e, hipStream_t s,
                   WsKind ws_kind) {
  KernelArgs a = a_in;
  a.ws = nullptr;
  a.tickets = nullptr;
  a.ticket_mark = 0;
  const bool kg = mode == kWgrad || mode == kWgradMx || mode == kWgradMxT;
  // (only the bf16 weight gradient splits; a stream being captured never
  // gets a per-stream workspace: the graph could be replayed on another
  // stream next to direct launches on this one)
  if (mode == kWgrad && a.M > 0 && split_enabled()) {
    char* w = nullptr;
    uint32_t mark = 0;
    if (ws_kind == kWsStatic) {
      const int err = static_workspace(&w, &mark);
      if (err != hipSuccess) return err;
    } else if (!capturing(s)) {
      w = stream_workspace(s, &mark);
    }
    if (w != nullptr) {
      a.tickets = reinterpret_cast<uint32_t*>(w);
      a.ws = reinterpret_cast<float*>(w + kTicketBytes);
      a.ticket_mark = mark;
    }
  }
  int64_t tiles;
  if (mode == kList) {
    tiles = int64_t(1) << 30;                 // unknown on the host: one workgroup per CU
  } else if (kg) {
    const int64_t tilesP = (a.K + Cfg::BP - 1) / Cfg::BP;
    const int64_t tilesQ = (a.N + Cfg::BQ - 1) / Cfg::BQ;
    tiles = (int64_t)a.E * tilesQ * tilesP;
  } else {
    const int64_t Pdim = mode == kFwd || mode == kFwdMx ? a.N : (mode == kFwdSwiglu ? a.N / 2 : a.K);
    const int64_t pstep = mode == kFwdSwiglu ? Cfg::BP / 2 : Cfg::BP;
    const int64_t tilesP = (Pdim + pstep - 1) / pstep;
    int64_t mt = (a.M + Cfg::BQ - 1) / Cfg::BQ + a.E;       // sum_e ceil(m_e/BQ) <= this
    if (max_m_per_e > 0) {
      const int64_t alt = (int64_t)a.E * ((max_m_per_e + Cfg::BQ - 1) / Cfg::BQ);
      if (alt < mt) mt = alt;
    }
    tiles = mt * tilesP;
  }
  if (tiles <= 0) return 0;
  // one workgroup per compute unit at most, and a multiple of 8 so that
  // workgroup b stays on XCD b % 8's part of the tile space
  // (at most 64 per XCD: the K-grouped balancing keeps one lane per workgroup)
  const int cus = device_cus() & ~7;
  const int64_t cap = cus < 8 ? 8 : (cus > 512 ? 512 : cus);
  int64_t grid = (tiles + 7) & ~int64_t(7);
  if (grid > cap) grid = cap;
  dim3 g((unsigned)grid), b(Cfg::NT);
  switch (mode) {
    case kFwd: hipLaunchKernelGGL((grouped_gemm_kernel<kFwd, Cfg>), g, b, 0, s, a); break;
    case kDgrad: hipLaunchKernelGGL((grouped_gemm_kernel<kDgrad, Cfg>), g, b, 0, s, a); break;
    case kFwdSwiglu:
      hipLaunchKernelGGL((grouped_gemm_kernel<kFwdSwiglu, Cfg>), g, b, 0, s, a);
      break;
    case kList: hipLaunchKernelGGL((grouped_gemm_kernel<kList, Cfg>), g, b, 0, s, a); break;
    case kFwdMx:
      hipLaunchKernelGGL((grouped_gemm_kernel<kFwdMx, CfgMx>), g, dim3(CfgMx::NT), 0, s, a);
      break;
    case kWgradMx:
      hipLaunchKernelGGL((grouped_gemm_kernel<kWgradMx, CfgMx>), g, dim3(CfgMx::NT), 0, s, a);
      break;
    case kWgradMxT:
      hipLaunchKernelGGL((grouped_gemm_kernel<kWgradMxT, CfgMx>), g, dim3(CfgMx::NT), 0, s, a);
      break;
    case kDgradSwiglu:
      hipLaunchKernelGGL((grouped_gemm_kernel<kDgradSwiglu, Cfg>), g, b, 0, s, a);
      break;
    default: hipLaunchKernelGGL((grouped_gemm_kernel<kWgrad, Cfg>), g, b, 0, s, a); break;
  }
  return (int)hipGetLastError();
}

// Blocked MXFP8 scales: entry [b][t][r] (a dword) holds the four scales of
// row r for reduction steps 128 t .. 128 t + 127 (127, the code of 1.0, for
// blocks past K / 32).  The torchao PR #3416 rearranges e8m0 scales into the
// layout its grouped GEMM reads with a kernel of its own; this is that step
// for the layout the MXFP8 forward above stages per LDS stage.  A workgroup
// moves a tile of 64 rows x 16 dwords through LDS, so that it reads each
// row's bytes contiguously and writes each output row of dwords contiguously.
constexpr int kScTileR = 64, kScTileT = 16;
__global__ __launch_bounds__(256) void mx_scales_blocked_kernel(const uint8_t* __restrict__ src,
                                                                 uint32_t* __restrict__ dst,
                                                                 int64_t rows, int64_t nb,
                                                                 int64_t nt, int64_t rblocks) {
  __shared__ uint32_t tile[kScTileR][kScTileT + 1];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x / rblocks;
  const int64_t r0 = (blockIdx.x % rblocks) * kScTileR, t0 = (int64_t)blockIdx.y * kScTileT;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tid / kScTileT + 16 * i, tq = tid % kScTileT;
    const int64_t r = r0 + row, t = t0 + tq;
    uint32_t v = 0;
    if (r < rows && t < nt) {
      const uint8_t* p = src + (b * rows + r) * nb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t blk = 4 * t + j;
        v |= (uint32_t)(blk < nb ? p[blk] : 127u) << (8 * j);
      }
    }
    tile[row][tq] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tq = tid / kScTileR + 4 * i, row = tid % kScTileR;
    const int64_t r = r0 + row, t = t0 + tq;
    if (r < rows && t < nt) dst[(b * nt + t) * rows + r] = tile[row][tq];
  }
}

int launch_mx_scales_blocked(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K,
                             int64_t batch, hipStream_t s) {
  const int64_t nb = K / 32, nt = (K + 127) / 128;
  if (batch <= 0 || rows <= 0 || nt <= 0) return 0;
  const int64_t rblocks = (rows + kScTileR - 1) / kScTileR;
  const int64_t gx = batch * rblocks, gy = (nt + kScTileT - 1) / kScTileT;
  if (gx >= (int64_t(1) << 31) || gy > 65535) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_scales_blocked_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s,
                     src, reinterpret_cast<uint32_t*>(dst), rows, nb, nt, rblocks);
  return (int)hipGetLastError();
}

}  // namespace mg
