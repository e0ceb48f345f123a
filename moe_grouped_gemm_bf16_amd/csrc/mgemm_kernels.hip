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
//
// Operand staging: HBM -> LDS by direct-to-LDS buffer loads (no registers),
// in 4 LDS stages of 32 reduction steps, 3 of them in flight while one is
// consumed.  R-contiguous operands are staged as [outer][32] rows and read
// with 128-bit LDS loads; R-strided operands are staged as they lie in HBM,
// [32][outer], and read with the LDS transpose load (ds_read_b64_tr_b16),
// which hands each lane 4 consecutive reduction values of one outer index --
// the transposes wgrad and dgrad need are done by the LDS read, not by a pass.
// Buffer descriptors whose range ends at the last valid byte make ragged
// rows, reduction tails and out-of-range columns arrive in LDS as zeros.
//
// Scheduling: all experts in one launch.  Each workgroup reads the offsets,
// derives per-expert tile counts and their prefix sums on the device (no host
// synchronisation, empty experts give no M-tiles) and loops over its tiles.
// M-grouped tiles all cost the same, so they are laid out XCD by XCD (the
// dispatcher deals workgroups round-robin over the 8 XCDs) to keep operand
// panels in one XCD's L2.  K-grouped tiles cost in proportion to the expert's
// rows, so they are ordered heaviest expert first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mgemm_launch.h"

namespace mg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

#ifndef MG_BK
#define MG_BK 64
#endif
#ifndef MG_DMA_SLOTS
#define MG_DMA_SLOTS 1
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
//  R-strided tile [32][outer]: rows of outer*2 bytes in 16-B chunks; chunk c
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

struct Tile {
  int e;        // expert
  int q0;       // first Q index of the tile (global row for M-grouped, n for K-grouped)
  int q_end;    // one past the last valid Q index
  int p0;       // first P index
  int r_begin;  // reduction range [r_begin, r_end)
  int r_end;
};

// Scheduler state kept in LDS for the whole launch.
struct Sched {
  int* scan;    // [16] scan scratch
  int* pref;    // [E+1] M-grouped: exclusive prefix of M-tiles per expert
  int* offs;    // [E+1] copy of the offsets
  int* inv;     // [E]   K-grouped: rank (heaviest first) -> expert
  int total;    // number of tiles
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
__device__ void setup_mgrouped(const int32_t* __restrict__ offsets, int E, int M, int tilesP,
                               Sched& S) {
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
  S.total = mtiles * tilesP;
}

// Tile of virtual workgroup id v (v = blockIdx.x + j * gridDim.x; gridDim.x is
// a multiple of 8, so v stays on blockIdx.x's XCD).  The tiles are laid out
// XCD by XCD: XCD x owns a contiguous range of tile ids, so tiles that run
// together on one XCD share operand panels in its L2.  Within the range, the
// P-tile index runs fastest.  Returns false once v is past this XCD's range.
template <int BP, int BQ>
__device__ __forceinline__ bool tile_mgrouped(int v, int E, int tilesP, int red,
                                              const Sched& S, Tile& t) {
  const int T = S.total;
  const int x = v & 7, s = v >> 3;
  const int q8 = T >> 3, r8 = T & 7;
  if (s >= q8 + (x < r8 ? 1 : 0)) return false;
  const int L = x * q8 + (x < r8 ? x : r8) + s;
  const int mt = L / tilesP, tp = L - mt * tilesP;
  // the expert whose M-tile range [pref[e], pref[e+1]) holds mt: the largest e
  // with pref[e] <= mt (empty experts share their successor's prefix)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S.pref[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  t.e = lo;
  t.q0 = S.offs[lo] + (mt - S.pref[lo]) * BQ;
  t.q_end = max(S.offs[lo + 1], S.offs[lo]);
  t.p0 = tp * BP;
  t.r_begin = 0;
  t.r_end = red;
  return true;
}

// K-grouped set-up: every expert has tilesQ x tilesP tiles whose cost grows
// with its row count; experts are ranked heaviest first (ties: lower index
// first) so that long reductions start early and short ones fill the tail.
template <int NT>
__device__ void setup_kgrouped(const int32_t* __restrict__ offsets, int E, int M, int per,
                               Sched& S) {
  for (int e = threadIdx.x; e <= E; e += NT) S.offs[e] = clamp_off(offsets, e, M);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += NT) {
    const int me = max(S.offs[e + 1] - S.offs[e], 0);
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const int mf = max(S.offs[f + 1] - S.offs[f], 0);
      rank += (mf > me || (mf == me && f < e)) ? 1 : 0;
    }
    S.inv[rank] = e;
  }
  __syncthreads();
  S.total = E * per;
}

template <int BP, int BQ>
__device__ __forceinline__ bool tile_kgrouped(int v, int tilesP, int per, const Sched& S,
                                              Tile& t) {
  if (v >= S.total) return false;
  const int rank = v / per, w = v - rank * per;
  const int e = S.inv[rank];
  const int tq = w / tilesP, tp = w - tq * tilesP;
  t.e = e;
  t.q0 = tq * BQ;
  t.p0 = tp * BP;
  t.r_begin = S.offs[e];
  t.r_end = max(S.offs[e + 1], S.offs[e]);
  t.q_end = 0x7FFFFFFF;
  return true;
}

// ------------------------------------------------------------------ kernel --

// Fragment reads.  A 32x32x16 matrix-core operand gives lane l the 8
// reduction values 8*(l/32) + 0..7 of outer index l % 32 (within one k-slice
// of 16).  Both operands use the same assignment, so the products pair up.

// R-contiguous tile [outer][32] (64-byte rows): one 128-bit read.
__device__ __forceinline__ bf16x8 frag_rc(const char* tile, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(tile + off);
}

// R-strided tile [32][outer]: two transpose loads of 4 reduction rows each.
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

template <int MODE, class C>
__device__ __forceinline__ void run_tile(const KernelArgs& a, const Tile& t, char* lds,
                                         int Pdim, int Qdim) {
  constexpr bool P_RS = MODE != kFwd;      // P is R-strided for dgrad and wgrad
  constexpr bool Q_RS = MODE == kWgrad;    // Q is R-strided for wgrad
  constexpr int SPW = C::SEGS_PER_WAVE;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  // ---- operand sources for this tile
  const uint16_t* P = reinterpret_cast<const uint16_t*>(a.p_src);
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q_src);
  int ldP, ldQ;
  if (MODE == kFwd) {            // P = W[e] rows n (R = k), Q = X rows m (R = k)
    ldP = (int)a.K; ldQ = (int)a.K;
    P += ((int64_t)t.e * a.N + t.p0) * a.K;
    Q += (int64_t)t.q0 * a.K;
  } else if (MODE == kDgrad) {   // P = W[e] [n][k] R-strided, Q = dY rows m (R = n)
    ldP = (int)a.K; ldQ = (int)a.N;
    P += (int64_t)t.e * a.N * a.K + t.p0;
    Q += (int64_t)t.q0 * a.N;
  } else {                       // P = X [i][k] R-strided, Q = dY [i][n] R-strided
    ldP = (int)a.K; ldQ = (int)a.N;
    P += (int64_t)t.r_begin * a.K + t.p0;
    Q += (int64_t)t.r_begin * a.N + t.q0;
  }
  const int red_len = t.r_end - t.r_begin;
  const int nk = (red_len + kBK - 1) / kBK;
  const int nP = Pdim - t.p0;                  // valid P rows (R-contiguous) or columns
  const int nQ = MODE == kWgrad ? Qdim - t.q0 : t.q_end - t.q0;

  // ---- direct-to-LDS plan: each stage is C::SEGS 1-KiB segments (the P tile
  // first, then the Q tile); wave w loads segments w*SPW .. w*SPW + SPW - 1.
  const bool wP = wave * SPW < C::SEGS_P;                    // wave-uniform
  const bool rs = wP ? P_RS : Q_RS;
  const int outer = wP ? C::BP : C::BQ;
  const int nouter = wP ? nP : nQ;
  const int ld = wP ? ldP : ldQ;
  const uint16_t* src = wP ? P : Q;
  const int seg0 = wP ? wave * SPW : wave * SPW - C::SEGS_P;
  const uint32_t lds_base = lds_u32(lds) + (wP ? 0u : (uint32_t)C::P_BYTES) + seg0 * 1024u;
  uint32_t voff[SPW];
  int col[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int p = (seg0 + j) * 1024 + lane * 16;             // byte within the tile
    if (rs) {                                                // [32][outer]
      const int r = p / (outer * 2), pc = (p >> 4) % (outer / 8);
      const int c = pc ^ rs_swz(r & 3);
      voff[j] = ((uint32_t)(r * ld + 8 * c) * 2u) | (8 * c < nouter ? 0u : kOOB);
      col[j] = 0;
    } else {                                                 // [outer][32]
      const int row = p / kRowB, pc = (p >> 4) % kRowChunks;
      const int c = pc ^ rc_swz(row);
      voff[j] = (uint32_t)(row * ld + 8 * c) * 2u;
      col[j] = 8 * c;
    }
  }
  const int rc_rows = nouter < outer ? (nouter > 0 ? nouter : 0) : outer;
  const i32x4 rc_rsrc = make_rsrc(src, (uint32_t)rc_rows * (uint32_t)ld * 2u);
  auto rs_rsrc = [&](int r0) {
    const int rr = min(red_len - r0, kBK), oc = min(nouter, outer);
    const uint32_t bytes = rr > 0 && oc > 0 ? ((uint32_t)(rr - 1) * ld + oc) * 2u : 0u;
    return make_rsrc(src + (int64_t)r0 * ld, bytes);
  };

  // Vector-memory operations this wave has issued (uniform), and the count
  // right after each stage's loads: the loads of stage s are complete once at
  // most `issued - after[s % kStages]` operations are outstanding.
  int issued = 0;
  int after[kStages];
#pragma unroll
  for (int s = 0; s < kStages; ++s) after[s] = 0;

  auto issue = [&](int kt) {
    const int r0 = kt * kBK;
    const uint32_t dst = lds_base + (uint32_t)((kt % kStages) * C::STAGE);
    if (rs) {
      const i32x4 rsrc = rs_rsrc(r0);
#pragma unroll
      for (int j = 0; j < SPW; ++j) dma16(rsrc, dst + j * 1024u, voff[j]);
    } else {
#pragma unroll
      for (int j = 0; j < SPW; ++j)
        dma16(rc_rsrc, dst + j * 1024u,
              (voff[j] + (uint32_t)r0 * 2u) | (r0 + col[j] < red_len ? 0u : kOOB));
    }
    issued += SPW;
    after[kt % kStages] = issued;
  };

  // ---- fragment addresses (byte offsets within an operand tile)
  const int wp = wave / C::WQ, wq = wave % C::WQ;
  const int l32 = lane & 31, h = lane >> 5, L = lane & 15, g16 = (lane >> 4) & 1;
  constexpr int KK = kBK / 16;                 // 16-wide k-slices per stage
  uint32_t offP[P_RS ? C::MP : KK], offQ[Q_RS ? C::MQ : KK];
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
    for (int kk = 0; kk < KK; ++kk) offP[kk] = rc_off(wp * C::WTP, kk);
  }
  if (Q_RS) {
#pragma unroll
    for (int j = 0; j < C::MQ; ++j) offQ[j] = rs_off(wq * C::WTQ, j, C::BQ);
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) offQ[kk] = rc_off(wq * C::WTQ, kk);
  }

  f32x16 acc[C::MP][C::MQ];
#pragma unroll
  for (int i = 0; i < C::MP; ++i)
#pragma unroll
    for (int j = 0; j < C::MQ; ++j) acc[i][j] = f32x16{};

  struct Frags {
    bf16x8 p[C::MP], q[C::MQ];
  };
  auto read = [&](int kt, int kk, Frags& f) {
    const char* tp = lds + (kt % kStages) * C::STAGE;
    const char* tq = tp + C::P_BYTES;
#pragma unroll
    for (int i = 0; i < C::MP; ++i)
      f.p[i] = P_RS ? frag_rs(tp, offP[i] + kk * 16 * C::BP * 2, 4 * C::BP * 2)
                    : frag_rc(tp, offP[kk] + i * 32 * kRowB);
#pragma unroll
    for (int j = 0; j < C::MQ; ++j)
      f.q[j] = Q_RS ? frag_rs(tq, offQ[j] + kk * 16 * C::BQ * 2, 4 * C::BQ * 2)
                    : frag_rc(tq, offQ[kk] + j * 32 * kRowB);
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < C::MP; ++i)
#pragma unroll
      for (int j = 0; j < C::MQ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.p[i], f.q[j], acc[i][j], 0, 0, 0);
  };
  // wait until this wave's loads of stage s have landed
  auto wait_stage = [&](int s) {
    int n = issued - after[s % kStages];
    n = n < 0 ? 0 : n;
    if (n >= 24) wait_vmcnt<24>();
    else if (n >= 16) { if (n >= 20) wait_vmcnt<20>(); else wait_vmcnt<16>(); }
    else if (n >= 8) { if (n >= 12) wait_vmcnt<12>(); else wait_vmcnt<8>(); }
    else if (n >= 4) { if (n >= 6) wait_vmcnt<6>(); else wait_vmcnt<4>(); }
    else if (n >= 2) wait_vmcnt<2>();
    else wait_vmcnt<0>();
  };

  // ---- pipeline.  Stage s lives in LDS buffer s % kStages and is consumed
  // in KK k-slices.  While slice kk's products run, slice kk+1 is read; the
  // last slice's products run while the barrier that publishes stage kt+1
  // is crossed and stage kt+1's first slice is read, so the matrix cores
  // stay busy across it.  That barrier also releases stage kt's buffer for
  // every wave (each wave waits for its own LDS reads before arriving), so
  // the loads of stage kt+kStages start right after it, spread between the
  // products of the following MG_DMA_SLOTS slices (a burst of loads would
  // stall on the memory queue).
  constexpr int kMM = C::MP * C::MQ;
  constexpr int kSlots = MG_DMA_SLOTS < KK ? MG_DMA_SLOTS : KK;
  constexpr int kPer = (SPW + kSlots - 1) / kSlots;   // loads per slot
  // Products of one k-slice, with loads [d0, d0 + nd) of stage dma_kt spread
  // evenly between them.
  auto mma_dma = [&](const Frags& f, int dma_kt, int d0, int nd) {
    const bool doit = nd > 0 && dma_kt < nk;
    const int r0 = dma_kt * kBK;
    const uint32_t dst = lds_base + (uint32_t)((dma_kt % kStages) * C::STAGE);
    i32x4 rsrc = rc_rsrc;
    if (rs && doit) rsrc = rs_rsrc(r0);
    const int every = nd > 0 && kMM / nd > 0 ? kMM / nd : 1;
    int d = d0;
#pragma unroll
    for (int x = 0; x < kMM; ++x) {
      const int i = x / C::MQ, j = x % C::MQ;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.p[i], f.q[j], acc[i][j], 0, 0, 0);
      if ((x + 1) % every == 0 && d < d0 + nd) {
        if (doit) {
          __builtin_amdgcn_sched_barrier(0);
          const uint32_t off = rs ? voff[d]
                                  : (voff[d] + (uint32_t)r0 * 2u) | (r0 + col[d] < red_len ? 0u : kOOB);
          dma16(rsrc, dst + d * 1024u, off);
          ++issued;
          __builtin_amdgcn_sched_barrier(0);
        }
        ++d;
      }
    }
    if (doit && d0 + nd == SPW) after[dma_kt % kStages] = issued;
  };
  auto slot_lo = [&](int slot) { return min(slot * kPer, SPW); };
  auto slot_n = [&](int slot) { return min((slot + 1) * kPer, SPW) - min(slot * kPer, SPW); };

  __syncthreads();                     // the previous tile's readers are done
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nk) issue(s);
  Frags fr[2];
  if (nk > 0) {
    wait_stage(0);
    __syncthreads();
    read(0, 0, fr[0]);
  }
  // slot 0 of stage kStages-1 (its buffer is still untouched)
  {
    const int s0 = kStages - 1;
    if (s0 < nk) {
      const int r0 = s0 * kBK;
      const uint32_t dst = lds_base + (uint32_t)((s0 % kStages) * C::STAGE);
      const i32x4 rsrc = rs ? rs_rsrc(r0) : rc_rsrc;
      for (int d = slot_lo(0); d < slot_lo(0) + slot_n(0); ++d) {
        const uint32_t off = rs ? voff[d]
                                : (voff[d] + (uint32_t)r0 * 2u) | (r0 + col[d] < red_len ? 0u : kOOB);
        dma16(rsrc, dst + d * 1024u, off);
        ++issued;
      }
      if (slot_n(0) == SPW) after[s0 % kStages] = issued;
    }
  }
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      Frags& cur = fr[kk & 1];
      Frags& nxt = fr[(kk + 1) & 1];
      int dma_kt, slot;
      if (kk + 1 < KK) {
        read(kt, kk + 1, nxt);
        dma_kt = kt + kStages - 1;      // slots 1.. of the stage begun after the last barrier
        slot = kk + 1;
      } else {
        if (kt + 1 < nk) {
          wait_stage(kt + 1);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __syncthreads();
          read(kt + 1, 0, nxt);
        }
        dma_kt = kt + kStages;          // its buffer (stage kt's) was just released
        slot = 0;
      }
      __builtin_amdgcn_sched_barrier(0);
      if (slot < kSlots) mma_dma(cur, dma_kt, slot_lo(slot), slot_n(slot));
      else mma_dma(cur, dma_kt, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue.  Result block (i, j): lane holds Q index l32 and P indices
  // 8*g + 4*h + 0..3 for g = 0..3 (accumulator registers 4g..4g+3).
  if (MODE == kWgrad) {
    float* out = reinterpret_cast<float*>(a.out) + (int64_t)t.e * a.N * a.K;
#pragma unroll
    for (int j = 0; j < C::MQ; ++j) {
      const int n = t.q0 + wq * C::WTQ + j * 32 + l32;
      if (n >= Qdim) continue;
      float* orow = out + (int64_t)n * a.K;
#pragma unroll
      for (int i = 0; i < C::MP; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int k = t.p0 + wp * C::WTP + i * 32 + g * 8 + h * 4;
          if (k >= Pdim) continue;
          f32x4 r = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                     acc[i][j][4 * g + 3]};
          f32x4* dst = reinterpret_cast<f32x4*>(orow + k);
          if (a.accumulate) r += *dst;
          *dst = r;
        }
      }
    }
  } else {
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    const int ldo = Pdim;
#pragma unroll
    for (int j = 0; j < C::MQ; ++j) {
      const int m = t.q0 + wq * C::WTQ + j * 32 + l32;
      if (m >= t.q_end) continue;
      uint16_t* orow = out + (int64_t)m * ldo;
#pragma unroll
      for (int i = 0; i < C::MP; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = t.p0 + wp * C::WTP + i * 32 + g * 8 + h * 4;
          if (c >= Pdim) continue;
          bf16x2 lo = __builtin_convertvector(
              (f32x2){acc[i][j][4 * g], acc[i][j][4 * g + 1]}, bf16x2);
          bf16x2 hi = __builtin_convertvector(
              (f32x2){acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]}, bf16x2);
          u32x2 pk = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          *reinterpret_cast<u32x2*>(orow + c) = pk;
        }
      }
    }
  }
}

template <int MODE, class C>
__global__ __launch_bounds__(C::NT)
void grouped_gemm_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];
  __shared__ int sched[16 + 2 * (kMaxExperts + 1) + kMaxExperts];

  int Pdim, Qdim;
  if (MODE == kFwd) {
    Pdim = (int)a.N; Qdim = (int)a.M;
  } else if (MODE == kDgrad) {
    Pdim = (int)a.K; Qdim = (int)a.M;
  } else {
    Pdim = (int)a.K; Qdim = (int)a.N;
  }
  const int tilesP = (Pdim + C::BP - 1) / C::BP;
  const int tilesQ = (Qdim + C::BQ - 1) / C::BQ;
  const int E = a.E;
  Sched S;
  S.scan = sched;
  S.pref = sched + 16;
  S.offs = S.pref + (E + 1);
  S.inv = S.offs + (E + 1);
  if (MODE == kWgrad) setup_kgrouped<C::NT>(a.offsets, E, (int)a.M, tilesQ * tilesP, S);
  else setup_mgrouped<C::NT, C::BQ>(a.offsets, E, (int)a.M, tilesP, S);
  const int red = MODE == kFwd ? (int)a.K : (int)a.N;

  for (int v = blockIdx.x;; v += gridDim.x) {
    Tile t;
    const bool have = MODE == kWgrad
                          ? tile_kgrouped<C::BP, C::BQ>(v, tilesP, tilesQ * tilesP, S, t)
                          : tile_mgrouped<C::BP, C::BQ>(v, E, tilesP, red, S, t);
    if (!have) break;
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.q0 = __builtin_amdgcn_readfirstlane(t.q0);
    t.q_end = __builtin_amdgcn_readfirstlane(t.q_end);
    t.p0 = __builtin_amdgcn_readfirstlane(t.p0);
    t.r_begin = __builtin_amdgcn_readfirstlane(t.r_begin);
    t.r_end = __builtin_amdgcn_readfirstlane(t.r_end);
    run_tile<MODE, C>(a, t, lds, Pdim, Qdim);
  }
}


// ------------------------------------------------------------ host launch --

#if MG_WAVES == 8
using Cfg = TileCfg<256, 256, 2, 4>;    // 8 waves (2 per SIMD), 128x64 per wave
#else
using Cfg = TileCfg<256, 256, 2, 2>;    // 4 waves (1 per SIMD), 128x128 per wave
#endif

int launch_grouped(int mode, const KernelArgs& a, int64_t max_m_per_e, hipStream_t s) {
  int grid;
  if (mode == kWgrad) {
    const int tilesP = (int)((a.K + Cfg::BP - 1) / Cfg::BP);
    const int tilesQ = (int)((a.N + Cfg::BQ - 1) / Cfg::BQ);
    grid = a.E * tilesQ * tilesP;
  } else {
    const int64_t Pdim = mode == kFwd ? a.N : a.K;
    const int tilesP = (int)((Pdim + Cfg::BP - 1) / Cfg::BP);
    int64_t mt = (a.M + Cfg::BQ - 1) / Cfg::BQ + a.E;       // sum_e ceil(m_e/BQ) <= this
    if (max_m_per_e > 0) {
      const int64_t alt = (int64_t)a.E * ((max_m_per_e + Cfg::BQ - 1) / Cfg::BQ);
      if (alt < mt) mt = alt;
    }
    // a multiple of 8 so that every virtual id a workgroup visits stays on its XCD
    grid = (int)((mt * tilesP + 7) & ~int64_t(7));
  }
  if (grid <= 0) return 0;
  dim3 g(grid), b(Cfg::NT);
  switch (mode) {
    case kFwd: hipLaunchKernelGGL((grouped_gemm_kernel<kFwd, Cfg>), g, b, 0, s, a); break;
    case kDgrad: hipLaunchKernelGGL((grouped_gemm_kernel<kDgrad, Cfg>), g, b, 0, s, a); break;
    default: hipLaunchKernelGGL((grouped_gemm_kernel<kWgrad, Cfg>), g, b, 0, s, a); break;
  }
  return (int)hipGetLastError();
}

}  // namespace mg
