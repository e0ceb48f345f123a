// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mg {

enum { kFwd = 0, kDgrad = 1, kWgrad = 2, kFwdSwiglu = 3, kList = 4, kFwdMx = 5, kWgradMx = 6,
       kDgradSwiglu = 7, kWgradMxT = 8 };

// Largest expert count a launch accepts: the device-side scheduler keeps the
// per-expert tile prefix in LDS, two entries per thread of a 512-thread block.
constexpr int kMaxExperts = 1024;

// One group of the descriptor-list call (same layout as mg_gemm_desc of the
// C ABI): D [m, n] = A [m, k] B [n, k]^T, row strides in elements.
struct ListDesc {
  const void* a;
  const void* b;
  void* d;
  int32_t m, n, k;
  int32_t lda, ldb, ldd;
};

struct KernelArgs {
  const void* p_src;        // FWD/DGRAD: W [E,N,K]; FWD_SWIGLU: W13 [E,N=2I,K]; WGRAD: X [M,K];
                            // FWD_MX: W8 [E,N,K] E4M3 codes; WGRAD_MX: X^T [K,M] E4M3 codes;
                            // WGRAD_MX_T: X8 [M,K] E4M3 codes (token-major)
  const void* q_src;        // FWD: X [M,K]; FWD_SWIGLU: X [M or T,K]; DGRAD/WGRAD: dY [M,N];
                            // FWD_MX: X8 [M,K] E4M3 codes; WGRAD_MX: dY^T [N,M] E4M3 codes;
                            // WGRAD_MX_T: dY8 [M,N] E4M3 codes (token-major)
  const int32_t* offsets;   // [E+1], device
  void* out;                // FWD: Y [M,N] bf16; FWD_SWIGLU: H [M,N/2] bf16; DGRAD: dX [M,K] bf16;
                            // DGRAD_SWIGLU: dGU [M,2K] bf16 (dg | du);
                            // WGRAD, WGRAD_MX, WGRAD_MX_T: dW [E,N,K] fp32
  int64_t M, N, K;
  int32_t E;
  int32_t accumulate;       // WGRAD only: add into `out`
  const ListDesc* list;     // LIST: E descriptors (device)
  const int32_t* gather;    // FWD_SWIGLU: row i of the problem is row gather[i] of x (or NULL)
  int64_t T;                // FWD_SWIGLU with gather: rows of x
  float* ws;                // WGRAD token split: 2 slots of 256 x 256 fp32 per split tile
  uint32_t* tickets;        // one word per split tile (see ticket_mark)
  uint32_t ticket_mark;     // this launch's odd ticket value, 2 g + 1 for a launch count g
  const uint8_t* p_scale;   // FWD_MX: W's E8M0 scales, blocked [E][ceil(K/128)][N][4];
                            // WGRAD_MX, WGRAD_MX_T: X's, blocked [M/128][K][4]
  const uint8_t* q_scale;   // FWD_MX: X's E8M0 scales, blocked [ceil(K/128)][M][4];
                            // WGRAD_MX, WGRAD_MX_T: dY's, blocked [M/128][N][4]
  void* aux;                // FWD_SWIGLU: optional gu [M, N] bf16 out (pre-activation g | u);
                            // DGRAD_SWIGLU: gu [M, 2K] bf16 in
};

// Token-order combine: out[t, :] = sum_j w[t, j] rows[token_rows[t, j], :]
// (bf16 rows [M, D], token_rows int32 [T, k], weights fp32 [T, k] or NULL, out
// bf16 [T, D]).  Returns a hipError_t value.
int launch_moe_combine(const uint16_t* rows, const int32_t* token_rows, const float* weights,
                       uint16_t* out, int64_t M, int64_t T, int32_t k, int64_t D, hipStream_t s);

// Rearrange E8M0 scales [batch][rows][K/32] into the blocked layout
// [batch][ceil(K/128)][rows][4] (absent blocks 127).  Returns a hipError_t value.
int launch_mx_scales_blocked(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K,
                             int64_t batch, hipStream_t s);

// Where the weight gradient's token split takes its workspace from.
enum WsKind {
  kWsStream = 0,   // a device allocation per (device, stream), made on first use
  kWsStatic = 1,   // the library's static device array (one per device); never allocates
};

// Enqueue one grouped GEMM on stream `s`.  Returns a hipError_t value.
int launch_grouped(int mode, const KernelArgs& a, int64_t max_m_per_e, hipStream_t s,
                   WsKind ws = kWsStream);

}  // namespace mg
