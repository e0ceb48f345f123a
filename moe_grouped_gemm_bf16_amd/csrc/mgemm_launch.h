// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mg {

enum { kFwd = 0, kDgrad = 1, kWgrad = 2, kFwdSwiglu = 3, kList = 4 };

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
  const void* p_src;        // FWD/DGRAD: W [E,N,K]; FWD_SWIGLU: W13 [E,N=2I,K]; WGRAD: X [M,K]
  const void* q_src;        // FWD: X [M,K]; FWD_SWIGLU: X [M or T,K]; DGRAD/WGRAD: dY [M,N]
  const int32_t* offsets;   // [E+1], device
  void* out;                // FWD: Y [M,N] bf16; FWD_SWIGLU: H [M,N/2] bf16; DGRAD: dX [M,K] bf16;
                            // WGRAD: dW [E,N,K] fp32
  int64_t M, N, K;
  int32_t E;
  int32_t accumulate;       // WGRAD only: add into `out`
  const ListDesc* list;     // LIST: E descriptors (device)
  const int32_t* gather;    // FWD_SWIGLU: row i of the problem is row gather[i] of x (or NULL)
  int64_t T;                // FWD_SWIGLU with gather: rows of x
  float* ws;                // WGRAD token split: 2 slots of 256 x 256 fp32 per split tile
  uint32_t* tickets;        // one zeroed counter per split tile (every launch leaves them zeroed)
};

// Enqueue one grouped GEMM on stream `s`.  Returns a hipError_t value.
int launch_grouped(int mode, const KernelArgs& a, int64_t max_m_per_e, hipStream_t s);

}  // namespace mg
