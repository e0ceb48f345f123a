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
// Both operands are staged in LDS as [outer][R] with R contiguous, so a single
// matrix-core loop serves all three; R-strided operands are transposed in
// registers (8x8 blocks of bf16) on the way from HBM to LDS.
//
// Scheduling: one workgroup per output tile, all experts in one launch.  Each
// workgroup reads the offsets, derives per-expert tile counts and their prefix
// sums on the device (no host synchronisation, empty experts give no M-tiles),
// and decodes its own tile.  M-grouped tiles all cost the same, so they are
// laid out XCD by XCD (the dispatcher deals workgroups round-robin over the 8
// XCDs) to keep operand panels in one XCD's L2.  K-grouped tiles cost in
// proportion to the expert's rows, so they are ordered heaviest expert first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mgemm_launch.h"

namespace mg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBP = 256;           // tile extent along P
constexpr int kBQ = 256;           // tile extent along Q
constexpr int kBK = 64;            // reduction slice per stage
constexpr int kThreads = 512;      // 8 waves: 2 along P x 4 along Q
constexpr int kWavesP = 2;
constexpr int kWavesQ = 4;
constexpr int kWaveP = kBP / kWavesP;   // 128
constexpr int kWaveQ = kBQ / kWavesQ;   // 64
constexpr int kBlkP = kWaveP / 32;      // 4 matrix-core blocks of 32 along P
constexpr int kBlkQ = kWaveQ / 32;      // 2 along Q
constexpr int kTileBytes = kBP * kBK * 2;          // one operand stage: 32 KiB
constexpr int kLdsBytes = 4 * kTileBytes;          // 2 operands x 2 stages
constexpr uint32_t kOOB = 0x80000000u;             // offset bit past any range

static_assert(kBP == 256 && kBQ == 256 && kBK == 64, "loaders assume 256x256x64");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer: stride 0, range `bytes`; loads past the range return zero.
  // Base and range are wave-uniform; say so, so that the descriptor lives in
  // scalar registers.
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// LDS layout of one operand stage: 256 rows (outer index) x 64 bf16 (R), 128 B
// per row, in 16-byte chunks whose position is XOR-swizzled by row bits 0-2
// and 3-5.  Matrix-core reads (32 consecutive rows, one chunk) and the
// transposed writes (rows 8 apart) both land on distinct banks.
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  int sw = (row ^ (row >> 3)) & 7;
  return (uint32_t)(row * 128 + ((chunk ^ sw) << 4));
}

// ---------------------------------------------------------------- loaders --
// Each loader is run by 256 threads (one half of the workgroup, `lt` in
// 0..255) and fetches one 256 x 64 operand stage into 8 x 16 bytes/thread.

// R-contiguous source: rows 0..255 from `base` (row stride ld elements), R
// columns [r0, r0 + 64).  Rows >= nrows and columns >= r_end read as zero.
__device__ __forceinline__ void load_rc(u32x4 (&v)[8], const uint16_t* base, int ld, int nrows,
                                        int r0, int r_end, int lt) {
  const int rows = nrows < kBP ? (nrows > 0 ? nrows : 0) : kBP;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)rows * (uint32_t)ld * 2u);
  const int c = lt & 7;
  const int rc = r0 + c * 8;
  // a chunk past the reduction end gets an offset past any range (bit 31 set;
  // ranges are below 2^31 bytes), so it reads as zero
  const uint32_t oob = rc < r_end ? 0u : kOOB;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (lt >> 3) + 32 * j;
    v[j] = bload(rs, ((uint32_t)(row * ld + rc) * 2u) | oob);
  }
}

__device__ __forceinline__ void store_rc(char* lds, const u32x4 (&v)[8], int lt) {
  const int c = lt & 7;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (lt >> 3) + 32 * j;
    *reinterpret_cast<u32x4*>(lds + lds_off(row, c)) = v[j];
  }
}

// R-strided source: R rows [0, 64) from `base` (row stride ld elements), outer
// columns 0..255.  R rows >= nred and outer columns >= nouter read as zero;
// the buffer range ends exactly at the last valid element, so no byte outside
// the rows' valid columns is ever addressed.  Thread lt owns the 8x8 block
// (R rows 8*(lt>>5) .. +7) x (outer 8*(lt&31) .. +7).
__device__ __forceinline__ void load_rs(u32x4 (&v)[8], const uint16_t* base, int ld, int nred,
                                        int nouter, int lt) {
  const int rr = nred < kBK ? (nred > 0 ? nred : 0) : kBK;
  const int oc = nouter < kBP ? nouter : kBP;
  const uint32_t bytes = rr > 0 && oc > 0 ? ((uint32_t)(rr - 1) * (uint32_t)ld + (uint32_t)oc) * 2u : 0u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
  const int ob = lt & 31, rb = lt >> 5;
  const uint32_t oob = ob * 8 < oc ? 0u : kOOB;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t off = ((uint32_t)((rb * 8 + j) * ld + ob * 8) * 2u) | oob;
    v[j] = bload(rs, off);
  }
}

// Transpose the 8x8 bf16 block in registers and write it as 8 LDS rows
// (outer 8*ob + c) holding R chunk rb.
__device__ __forceinline__ void store_rs(char* lds, const u32x4 (&v)[8], int lt) {
  const int ob = lt & 31, rb = lt >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int d = c >> 1;
    u32x4 o;
    if ((c & 1) == 0) {
      o.x = __builtin_amdgcn_perm(v[1][d], v[0][d], 0x05040100u);
      o.y = __builtin_amdgcn_perm(v[3][d], v[2][d], 0x05040100u);
      o.z = __builtin_amdgcn_perm(v[5][d], v[4][d], 0x05040100u);
      o.w = __builtin_amdgcn_perm(v[7][d], v[6][d], 0x05040100u);
    } else {
      o.x = __builtin_amdgcn_perm(v[1][d], v[0][d], 0x07060302u);
      o.y = __builtin_amdgcn_perm(v[3][d], v[2][d], 0x07060302u);
      o.z = __builtin_amdgcn_perm(v[5][d], v[4][d], 0x07060302u);
      o.w = __builtin_amdgcn_perm(v[7][d], v[6][d], 0x07060302u);
    }
    *reinterpret_cast<u32x4*>(lds + lds_off(ob * 8 + c, rb)) = o;
  }
}

// ------------------------------------------------------------- scheduler --

// Exclusive prefix sum over the block of per-thread values; returns the
// thread's exclusive prefix and writes the block total to *total.
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
  for (int w = 0; w < kThreads / 64; ++w) {
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

// M-grouped set-up: tiles are, for every expert, ceil(m_e / BQ) M-tiles times
// tilesP P-tiles; empty experts contribute none.
// Offsets are read clamped to [0, M] and made non-decreasing per expert, so
// that even offsets breaking the documented precondition cannot move any read
// or write outside the tensors (the results are then meaningless, not unsafe).
__device__ __forceinline__ int clamp_off(const int32_t* offsets, int i, int M) {
  const int o = offsets[i];
  return o < 0 ? 0 : (o > M ? M : o);
}

__device__ void setup_mgrouped(const int32_t* __restrict__ offsets, int E, int M, int tilesP,
                               Sched& S) {
  constexpr int kPer = kMaxExperts / kThreads;
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
      cnt[j] = m > 0 ? (m + kBQ - 1) / kBQ : 0;
      mine += cnt[j];
    }
  }
  int mtiles;
  int run = block_exclusive_scan(mine, S.scan, &mtiles);
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
  t.q0 = S.offs[lo] + (mt - S.pref[lo]) * kBQ;
  t.q_end = max(S.offs[lo + 1], S.offs[lo]);
  t.p0 = tp * kBP;
  t.r_begin = 0;
  t.r_end = red;
  return true;
}

// K-grouped set-up: every expert has tilesQ x tilesP tiles whose cost grows
// with its row count; experts are ranked heaviest first (ties: lower index
// first) so that long reductions start early and short ones fill the tail.
__device__ void setup_kgrouped(const int32_t* __restrict__ offsets, int E, int M, int per,
                               Sched& S) {
  for (int e = threadIdx.x; e <= E; e += kThreads) S.offs[e] = clamp_off(offsets, e, M);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
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

__device__ __forceinline__ bool tile_kgrouped(int v, int tilesP, int per, const Sched& S,
                                              Tile& t) {
  if (v >= S.total) return false;
  const int rank = v / per, w = v - rank * per;
  const int e = S.inv[rank];
  const int tq = w / tilesP, tp = w - tq * tilesP;
  t.e = e;
  t.q0 = tq * kBQ;
  t.p0 = tp * kBP;
  t.r_begin = S.offs[e];
  t.r_end = max(S.offs[e + 1], S.offs[e]);
  t.q_end = 0x7FFFFFFF;
  return true;
}

// ------------------------------------------------------------------ kernel --

template <int MODE>
__device__ __forceinline__ void run_tile(const KernelArgs& a, const Tile& t, char* lds,
                                         int Pdim, int Qdim) {
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
  const int nrowsP = Pdim - t.p0;              // valid P rows (R-contiguous) or columns
  const int nrowsQ = t.q_end - t.q0;           // for R-contiguous Q (M-grouped)

  const bool loadsP = wave < 4;                // waves 0-3 stage P, 4-7 stage Q
  const int lt = tid & 255;
  // stage s: P at s * 2 * kTileBytes, Q right after it

  u32x4 v[8];
  auto gload = [&](int kt) {
    const int r0 = kt * kBK;
    if (loadsP) {
      if (MODE == kFwd) load_rc(v, P, ldP, nrowsP, r0, red_len, lt);
      else load_rs(v, P + (int64_t)r0 * ldP, ldP, red_len - r0, nrowsP, lt);
    } else {
      if (MODE == kWgrad) load_rs(v, Q + (int64_t)r0 * ldQ, ldQ, red_len - r0, Qdim - t.q0, lt);
      else load_rc(v, Q, ldQ, nrowsQ, r0, red_len, lt);
    }
  };
  auto lstore = [&](int buf) {
    char* base = lds + buf * (2 * kTileBytes) + (loadsP ? 0 : kTileBytes);
    if (loadsP ? MODE == kFwd : MODE != kWgrad) store_rc(base, v, lt);
    else store_rs(base, v, lt);
  };

  f32x16 acc[kBlkP][kBlkQ];
#pragma unroll
  for (int i = 0; i < kBlkP; ++i)
#pragma unroll
    for (int j = 0; j < kBlkQ; ++j) acc[i][j] = f32x16{};

  const int wp = wave / kWavesQ, wq = wave % kWavesQ;
  const int lrow = lane & 31, lhalf = lane >> 5;

  if (nk > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const char* sp = lds + cur * (2 * kTileBytes);
    const char* sq = sp + kTileBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int chunk = kk * 2 + lhalf;
      bf16x8 fp[kBlkP], fq[kBlkQ];
#pragma unroll
      for (int i = 0; i < kBlkP; ++i)
        fp[i] = *reinterpret_cast<const bf16x8*>(sp + lds_off(wp * kWaveP + i * 32 + lrow, chunk));
#pragma unroll
      for (int j = 0; j < kBlkQ; ++j)
        fq[j] = *reinterpret_cast<const bf16x8*>(sq + lds_off(wq * kWaveQ + j * 32 + lrow, chunk));
#pragma unroll
      for (int i = 0; i < kBlkP; ++i)
#pragma unroll
        for (int j = 0; j < kBlkQ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp[i], fq[j], acc[i][j], 0, 0, 0);
      // keep each k-slice's fragment reads next to its own products (bounds
      // the fragment registers live at once)
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Result block (i, j): lane holds Q index lrow and P indices
  // 8*g + 4*lhalf + 0..3 for g = 0..3 (accumulator registers 4g..4g+3).
  if (MODE == kWgrad) {
    float* out = reinterpret_cast<float*>(a.out) + (int64_t)t.e * a.N * a.K;
#pragma unroll
    for (int j = 0; j < kBlkQ; ++j) {
      const int n = t.q0 + wq * kWaveQ + j * 32 + lrow;
      if (n >= Qdim) continue;
      float* orow = out + (int64_t)n * a.K;
#pragma unroll
      for (int i = 0; i < kBlkP; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int k = t.p0 + wp * kWaveP + i * 32 + g * 8 + lhalf * 4;
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
    for (int j = 0; j < kBlkQ; ++j) {
      const int m = t.q0 + wq * kWaveQ + j * 32 + lrow;
      if (m >= t.q_end) continue;
      uint16_t* orow = out + (int64_t)m * ldo;
#pragma unroll
      for (int i = 0; i < kBlkP; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = t.p0 + wp * kWaveP + i * 32 + g * 8 + lhalf * 4;
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

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  __shared__ int sched[16 + 2 * (kMaxExperts + 1) + kMaxExperts];

  int Pdim, Qdim;
  if (MODE == kFwd) {
    Pdim = (int)a.N; Qdim = (int)a.M;
  } else if (MODE == kDgrad) {
    Pdim = (int)a.K; Qdim = (int)a.M;
  } else {
    Pdim = (int)a.K; Qdim = (int)a.N;
  }
  const int tilesP = (Pdim + kBP - 1) / kBP;
  const int tilesQ = (Qdim + kBQ - 1) / kBQ;
  const int E = a.E;
  Sched S;
  S.scan = sched;
  S.pref = sched + 16;
  S.offs = S.pref + (E + 1);
  S.inv = S.offs + (E + 1);
  if (MODE == kWgrad) setup_kgrouped(a.offsets, E, (int)a.M, tilesQ * tilesP, S);
  else setup_mgrouped(a.offsets, E, (int)a.M, tilesP, S);
  const int red = MODE == kFwd ? (int)a.K : (int)a.N;

  for (int v = blockIdx.x;; v += gridDim.x) {
    Tile t;
    const bool have = MODE == kWgrad ? tile_kgrouped(v, tilesP, tilesQ * tilesP, S, t)
                                     : tile_mgrouped(v, E, tilesP, red, S, t);
    if (!have) break;
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.q0 = __builtin_amdgcn_readfirstlane(t.q0);
    t.q_end = __builtin_amdgcn_readfirstlane(t.q_end);
    t.p0 = __builtin_amdgcn_readfirstlane(t.p0);
    t.r_begin = __builtin_amdgcn_readfirstlane(t.r_begin);
    t.r_end = __builtin_amdgcn_readfirstlane(t.r_end);
    run_tile<MODE>(a, t, lds, Pdim, Qdim);
  }
}

// ------------------------------------------------------------ host launch --

static int tiles_upper_bound_m(int64_t M, int E, int64_t max_m_per_e, int tilesP) {
  int64_t mt = (M + kBQ - 1) / kBQ + E;             // sum_e ceil(m_e/BQ) <= this
  if (max_m_per_e > 0) {
    int64_t alt = (int64_t)E * ((max_m_per_e + kBQ - 1) / kBQ);
    if (alt < mt) mt = alt;
  }
  return (int)(mt * tilesP);
}

int launch_grouped(int mode, const KernelArgs& a, int64_t max_m_per_e, hipStream_t s) {
  int grid;
  if (mode == kWgrad) {
    const int tilesP = (int)((a.K + kBP - 1) / kBP), tilesQ = (int)((a.N + kBQ - 1) / kBQ);
    grid = a.E * tilesQ * tilesP;
  } else {
    // a multiple of 8 so that every virtual id a workgroup visits stays on its XCD
    const int64_t Pdim = mode == kFwd ? a.N : a.K;
    const int tilesP = (int)((Pdim + kBP - 1) / kBP);
    grid = tiles_upper_bound_m(a.M, a.E, max_m_per_e, tilesP);
    grid = (grid + 7) & ~7;
  }
  if (grid <= 0) return 0;
  dim3 g(grid), b(kThreads);
  switch (mode) {
    case kFwd: hipLaunchKernelGGL(grouped_gemm_kernel<kFwd>, g, b, 0, s, a); break;
    case kDgrad: hipLaunchKernelGGL(grouped_gemm_kernel<kDgrad>, g, b, 0, s, a); break;
    default: hipLaunchKernelGGL(grouped_gemm_kernel<kWgrad>, g, b, 0, s, a); break;
  }
  return (int)hipGetLastError();
}

}  // namespace mg
