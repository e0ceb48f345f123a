// C-ABI entry points of libmgemm.so: argument validation, device check and
// dispatch to the gfx950 kernels.  No host workspace, no host<->device copy
// and no synchronisation on the normal path: the offsets stay on the device
// and are read by the kernels' own tile scheduler (a host workspace copied to
// the device per call, freed before the asynchronous copy has run, is the
// lifetime race discussed in the TransformerEngine PR #2045 review; this
// design has no such buffer).  The only allocation is the device workspace of
// the weight gradient's token split, made once per (device, stream) by the
// launch layer and kept for the life of the process (never while the stream
// is being captured); kgemm_wgrad_noalloc takes it from a static device array
// instead.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mgemm.h"
#include "mgemm_launch.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 22;     // N, K: 256-row tile offsets fit int32
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int kMaxDevices = 64;

std::atomic<int> g_arch_state[kMaxDevices];       // 0 unknown, 1 gfx950, 2 other

mg_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MG_ERR_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MG_ERR_DEVICE;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? MG_OK : MG_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mg_status check_sizes(int64_t M, int64_t N, int64_t K, int32_t E) {
  if (E < 1 || E > mg::kMaxExperts) return MG_ERR_SHAPE;
  if (M < 0 || N < 0 || K < 0 || M > kMaxRows || N > kMaxDim || K > kMaxDim) return MG_ERR_SHAPE;
  if ((N & 7) || (K & 7)) return MG_ERR_SHAPE;
  return MG_OK;
}

// Optional debug validation of the device offsets (MGEMM_VALIDATE=1): copies
// them to the host on the caller's stream and synchronises it.
mg_status maybe_validate(const int32_t* offsets, int32_t E, int64_t M, hipStream_t s,
                         int32_t multiple = 1) {
  static const bool on = [] {
    const char* v = std::getenv("MGEMM_VALIDATE");
    return v != nullptr && v[0] == '1';
  }();
  if (!on) return MG_OK;
  std::vector<int32_t> h(static_cast<size_t>(E) + 1);
  if (hipMemcpyAsync(h.data(), offsets, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MG_ERR_DEVICE;
  mg_status st = mg_check_offsets_host(h.data(), E, M);
  if (st != MG_OK) return st;
  for (int32_t e = 0; e <= E; ++e)
    if (h[static_cast<size_t>(e)] % multiple != 0) return MG_ERR_OFFSETS;
  return MG_OK;
}

static_assert(sizeof(mg_gemm_desc) == sizeof(mg::ListDesc) &&
                  offsetof(mg_gemm_desc, m) == offsetof(mg::ListDesc, m) &&
                  offsetof(mg_gemm_desc, ldd) == offsetof(mg::ListDesc, ldd),
              "mg_gemm_desc and the kernel's descriptor must have one layout");

mg_status launch(int mode, const mg::KernelArgs& a, int64_t max_m_per_e, hipStream_t s,
                 mg::WsKind ws = mg::kWsStream) {
  int err = mg::launch_grouped(mode, a, max_m_per_e, s, ws);
  return err == hipSuccess ? MG_OK : MG_ERR_LAUNCH;
}

// Shared body of the two M-grouped calls.  `a_in` is x (fwd) or dy (dgrad).
mg_status mgrouped(int mode, const void* a_in, const void* w, const int32_t* offsets, void* out,
                   int64_t M, int64_t N, int64_t K, int32_t E, int64_t max_m_per_e,
                   void* stream) {
  mg_status st = check_sizes(M, N, K, E);
  if (st != MG_OK) return st;
  if (max_m_per_e < 0) return MG_ERR_SHAPE;
  const int64_t pdim = mode == mg::kFwd ? N : K;
  // tile-count bound used by the scheduler must fit in int32
  if (((M + 255) / 256 + E) * ((pdim + 255) / 256) > kMaxRows) return MG_ERR_SHAPE;
  if (M == 0 || pdim == 0) return MG_OK;
  const int64_t red = mode == mg::kFwd ? K : N;   // an empty reduction reads no input
  if (!offsets || !out || (red > 0 && (!a_in || !w))) return MG_ERR_NULL;
  if ((red > 0 && (!aligned16(a_in) || !aligned16(w))) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return MG_ERR_ALIGN;
  if ((st = check_device()) != MG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = maybe_validate(offsets, E, M, s)) != MG_OK) return st;
  mg::KernelArgs a{};
  a.p_src = w;
  a.q_src = a_in;
  a.offsets = offsets;
  a.out = out;
  a.M = M; a.N = N; a.K = K; a.E = E;
  a.accumulate = 0;
  return launch(mode, a, max_m_per_e, s);
}

}  // namespace

extern "C" {

mg_status mgemm_fwd(const void* x, const void* w, const int32_t* offsets, void* y, int64_t M,
                    int64_t N, int64_t K, int32_t E, int64_t max_m_per_e, void* stream) {
  return mgrouped(mg::kFwd, x, w, offsets, y, M, N, K, E, max_m_per_e, stream);
}

mg_status mgemm_dgrad(const void* dy, const void* w, const int32_t* offsets, void* dx, int64_t M,
                      int64_t N, int64_t K, int32_t E, int64_t max_m_per_e, void* stream) {
  return mgrouped(mg::kDgrad, dy, w, offsets, dx, M, N, K, E, max_m_per_e, stream);
}

mg_status mgemm_fwd_swiglu_gu(const void* x, const int32_t* gather, const void* w13,
                              const int32_t* offsets, void* h, void* gu, int64_t M, int64_t T,
                              int64_t I, int64_t K, int32_t E, int64_t max_m_per_e,
                              void* stream) {
  mg_status st = check_sizes(M, 2 * I, K, E);
  if (st != MG_OK) return st;
  if (max_m_per_e < 0 || I < 0 || (I & 7)) return MG_ERR_SHAPE;   // h rows 16-byte aligned
  if (gather != nullptr && (T < 0 || T > kMaxRows)) return MG_ERR_SHAPE;
  // 32-bit buffer offsets: one expert's w13 and (when gathering) all of x
  constexpr int64_t k4G = int64_t(1) << 32;
  if (2 * I * K * 2 >= k4G || (gather != nullptr && T * K * 2 >= k4G)) return MG_ERR_SHAPE;
  if (((M + 255) / 256 + E) * ((I + 127) / 128) > kMaxRows) return MG_ERR_SHAPE;
  if (M == 0 || I == 0) return MG_OK;
  if (!offsets || !h || (K > 0 && (!x || !w13))) return MG_ERR_NULL;
  if ((K > 0 && (!aligned16(x) || !aligned16(w13))) || !aligned16(h) || !aligned16(gu) ||
      (reinterpret_cast<uintptr_t>(offsets) & 3u) || (reinterpret_cast<uintptr_t>(gather) & 3u))
    return MG_ERR_ALIGN;
  if ((st = check_device()) != MG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = maybe_validate(offsets, E, M, s)) != MG_OK) return st;
  mg::KernelArgs a{};
  a.p_src = w13;
  a.q_src = x;
  a.offsets = offsets;
  a.out = h;
  a.aux = gu;
  a.M = M; a.N = 2 * I; a.K = K; a.E = E;
  a.accumulate = 0;
  a.gather = gather;
  a.T = gather != nullptr ? T : M;
  return launch(mg::kFwdSwiglu, a, max_m_per_e, s);
}

mg_status mgemm_fwd_swiglu(const void* x, const int32_t* gather, const void* w13,
                           const int32_t* offsets, void* h, int64_t M, int64_t T, int64_t I,
                           int64_t K, int32_t E, int64_t max_m_per_e, void* stream) {
  return mgemm_fwd_swiglu_gu(x, gather, w13, offsets, h, nullptr, M, T, I, K, E, max_m_per_e,
                             stream);
}

mg_status mgemm_dgrad_swiglu(const void* dy, const void* w2, const void* gu,
                             const int32_t* offsets, void* dgu, int64_t M, int64_t N, int64_t I,
                             int32_t E, int64_t max_m_per_e, void* stream) {
  mg_status st = check_sizes(M, N, I, E);      // the down projection: K = I
  if (st != MG_OK) return st;
  if (max_m_per_e < 0) return MG_ERR_SHAPE;
  if (((M + 255) / 256 + E) * ((I + 255) / 256) > kMaxRows) return MG_ERR_SHAPE;
  if (M == 0 || I == 0) return MG_OK;
  if (!offsets || !dgu || !gu || (N > 0 && (!dy || !w2))) return MG_ERR_NULL;
  if ((N > 0 && (!aligned16(dy) || !aligned16(w2))) || !aligned16(gu) || !aligned16(dgu) ||
      (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return MG_ERR_ALIGN;
  if ((st = check_device()) != MG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = maybe_validate(offsets, E, M, s)) != MG_OK) return st;
  mg::KernelArgs a{};
  a.p_src = w2;
  a.q_src = dy;
  a.offsets = offsets;
  a.out = dgu;
  a.aux = const_cast<void*>(gu);
  a.M = M; a.N = N; a.K = I; a.E = E;
  a.accumulate = 0;
  return launch(mg::kDgradSwiglu, a, max_m_per_e, s);
}

mg_status mgemm_list(const mg_gemm_desc* desc, int32_t G, void* stream) {
  if (G < 1 || G > mg::kMaxExperts) return MG_ERR_SHAPE;
  if (!desc) return MG_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(desc) & 7u) return MG_ERR_ALIGN;
  mg_status st = check_device();
  if (st != MG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  static const bool validate = [] {
    const char* v = std::getenv("MGEMM_VALIDATE");
    return v != nullptr && v[0] == '1';
  }();
  if (validate) {
    std::vector<mg_gemm_desc> h(static_cast<size_t>(G));
    if (hipMemcpyAsync(h.data(), desc, h.size() * sizeof(mg_gemm_desc), hipMemcpyDeviceToHost,
                       s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return MG_ERR_DEVICE;
    if ((st = mg_check_list_host(h.data(), G)) != MG_OK) return st;
  }
  mg::KernelArgs a{};
  a.list = reinterpret_cast<const mg::ListDesc*>(desc);
  a.E = G;
  return launch(mg::kList, a, 0, s);
}

mg_status mgemm_fwd_mx(const void* x, const void* x_scale, const void* w, const void* w_scale,
                       const int32_t* offsets, void* y, int64_t M, int64_t N, int64_t K, int32_t E,
                       int64_t max_m_per_e, void* stream) {
  mg_status st = check_sizes(M, N, K, E);
  if (st != MG_OK) return st;
  if (max_m_per_e < 0 || (K & 31)) return MG_ERR_SHAPE;       // whole 32-element scale blocks
  // blocked scales are addressed with 31-bit offsets
  const int64_t ks = (K + 127) / 128;
  constexpr int64_t k2G = int64_t(1) << 31;
  if (ks * M * 4 >= k2G || ks * N * 4 >= k2G) return MG_ERR_SHAPE;
  if (((M + 255) / 256 + E) * ((N + 255) / 256) > kMaxRows) return MG_ERR_SHAPE;
  if (M == 0 || N == 0) return MG_OK;
  if (!offsets || !y || (K > 0 && (!x || !w || !x_scale || !w_scale))) return MG_ERR_NULL;
  if ((K > 0 && (!aligned16(x) || !aligned16(w) ||
                 (reinterpret_cast<uintptr_t>(x_scale) & 3u) ||
                 (reinterpret_cast<uintptr_t>(w_scale) & 3u))) ||
      !aligned16(y) || (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return MG_ERR_ALIGN;
  if ((st = check_device()) != MG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = maybe_validate(offsets, E, M, s)) != MG_OK) return st;
  mg::KernelArgs a{};
  a.p_src = w;
  a.q_src = x;
  a.p_scale = static_cast<const uint8_t*>(w_scale);
  a.q_scale = static_cast<const uint8_t*>(x_scale);
  a.offsets = offsets;
  a.out = y;
  a.M = M; a.N = N; a.K = K; a.E = E;
  return launch(mg::kFwdMx, a, max_m_per_e, s);
}

mg_status kgemm_wgrad_mx_tm(const void* dy8, const void* dy_scale, const void* x8,
                            const void* x_scale, const int32_t* offsets, float* dw, int64_t M,
                            int64_t N, int64_t K, int32_t E, int32_t accumulate, void* stream) {
  mg_status st = check_sizes(M, N, K, E);
  if (st != MG_OK) return st;
  // tokens in 128-step stages; rows of N and K code bytes start 16-byte
  // aligned; 32-bit buffer offsets over 128 token rows and the blocked scales
  constexpr int64_t k2G = int64_t(1) << 31;
  const int64_t ks = M / 128;
  if ((M & 127) || (N & 15) || (K & 15) || ks * N * 4 >= k2G || ks * K * 4 >= k2G)
    return MG_ERR_SHAPE;
  if (N == 0 || K == 0) return MG_OK;
  if (!offsets || !dw || (M > 0 && (!dy8 || !x8 || !dy_scale || !x_scale))) return MG_ERR_NULL;
  if ((M > 0 && (!aligned16(dy8) || !aligned16(x8) ||
                 (reinterpret_cast<uintptr_t>(dy_scale) & 3u) ||
                 (reinterpret_cast<uintptr_t>(x_scale) & 3u))) ||
      !aligned16(dw) || (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return MG_ERR_ALIGN;
  if ((st = check_device()) != MG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = maybe_validate(offsets, E, M, s, 128)) != MG_OK) return st;
  mg::KernelArgs a{};
  a.p_src = x8;
  a.q_src = dy8;
  a.p_scale = static_cast<const uint8_t*>(x_scale);
  a.q_scale = static_cast<const uint8_t*>(dy_scale);
  a.offsets = offsets;
  a.out = dw;
  a.M = M; a.N = N; a.K = K; a.E = E;
  a.accumulate = accumulate ? 1 : 0;
  return launch(mg::kWgradMxT, a, 0, s);
}

mg_status kgemm_wgrad_mx(const void* dyt, const void* dyt_scale, const void* xt,
                         const void* xt_scale, const int32_t* offsets, float* dw, int64_t M,
                         int64_t N, int64_t K, int32_t E, int32_t accumulate, void* stream) {
  mg_status st = check_sizes(M, N, K, E);
  if (st != MG_OK) return st;
  // tokens in 128-step stages; 32-bit buffer offsets over a 256-row tile of
  // M-byte rows and over the blocked scales
  constexpr int64_t k2G = int64_t(1) << 31;
  const int64_t ks = M / 128;
  if ((M & 127) || 256 * M >= 2 * k2G || ks * N * 4 >= k2G || ks * K * 4 >= k2G)
    return MG_ERR_SHAPE;
  if (N == 0 || K == 0) return MG_OK;
  if (!offsets || !dw || (M > 0 && (!dyt || !xt || !dyt_scale || !xt_scale))) return MG_ERR_NULL;
  if ((M > 0 && (!aligned16(dyt) || !aligned16(xt) ||
                 (reinterpret_cast<uintptr_t>(dyt_scale) & 3u) ||
                 (reinterpret_cast<uintptr_t>(xt_scale) & 3u))) ||
      !aligned16(dw) || (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return MG_ERR_ALIGN;
  if ((st = check_device()) != MG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = maybe_validate(offsets, E, M, s, 128)) != MG_OK) return st;
  mg::KernelArgs a{};
  a.p_src = xt;
  a.q_src = dyt;
  a.p_scale = static_cast<const uint8_t*>(xt_scale);
  a.q_scale = static_cast<const uint8_t*>(dyt_scale);
  a.offsets = offsets;
  a.out = dw;
  a.M = M; a.N = N; a.K = K; a.E = E;
  a.accumulate = accumulate ? 1 : 0;
  return launch(mg::kWgradMx, a, 0, s);
}

mg_status mg_moe_combine(const void* rows, const int32_t* token_rows, const float* weights,
                         void* out, int64_t M, int64_t T, int32_t k, int64_t D, void* stream) {
  if (M < 0 || T < 0 || D < 0 || k < 1 || k > 64 || (D & 7) || M > kMaxRows || T > kMaxRows ||
      D > kMaxDim)
    return MG_ERR_SHAPE;
  if (T == 0 || D == 0) return MG_OK;
  if (!token_rows || !out || (M > 0 && !rows)) return MG_ERR_NULL;
  if ((M > 0 && !aligned16(rows)) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(token_rows) & 3u) ||
      (reinterpret_cast<uintptr_t>(weights) & 3u))
    return MG_ERR_ALIGN;
  mg_status st;
  if ((st = check_device()) != MG_OK) return st;
  const int err = mg::launch_moe_combine(static_cast<const uint16_t*>(rows), token_rows, weights,
                                         static_cast<uint16_t*>(out), M, T, k, D,
                                         static_cast<hipStream_t>(stream));
  return err == hipSuccess ? MG_OK : MG_ERR_LAUNCH;
}

mg_status mg_mx_scales_blocked(const void* scales, void* blocked, int64_t rows, int64_t K,
                               int64_t batch, void* stream) {
  if (rows < 0 || K < 0 || batch < 0 || (K & 31) || rows > kMaxRows || K > kMaxDim ||
      batch > kMaxRows)
    return MG_ERR_SHAPE;
  const int64_t total = batch * ((K + 127) / 128) * rows;    // output dwords
  if (total >= (int64_t(1) << 40) || batch * ((rows + 63) / 64) >= (int64_t(1) << 31))
    return MG_ERR_SHAPE;
  if (total == 0) return MG_OK;
  if (!scales || !blocked) return MG_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(blocked) & 3u) return MG_ERR_ALIGN;
  mg_status st;
  if ((st = check_device()) != MG_OK) return st;
  const int err = mg::launch_mx_scales_blocked(static_cast<const uint8_t*>(scales),
                                               static_cast<uint8_t*>(blocked), rows, K, batch,
                                               static_cast<hipStream_t>(stream));
  return err == hipSuccess ? MG_OK : MG_ERR_LAUNCH;
}

namespace {

mg_status wgrad_common(const void* dy, const void* x, const int32_t* offsets, float* dw,
                       int64_t M, int64_t N, int64_t K, int32_t E, int32_t accumulate,
                       void* stream, mg::WsKind ws) {
  mg_status st = check_sizes(M, N, K, E);
  if (st != MG_OK) return st;
  if ((int64_t)E * ((N + 255) / 256) * ((K + 255) / 256) > kMaxRows) return MG_ERR_SHAPE;
  if (N == 0 || K == 0) return MG_OK;
  if (!offsets || !dw || (M > 0 && (!dy || !x))) return MG_ERR_NULL;
  if ((M > 0 && (!aligned16(dy) || !aligned16(x))) || !aligned16(dw) ||
      (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return MG_ERR_ALIGN;
  if ((st = check_device()) != MG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = maybe_validate(offsets, E, M, s)) != MG_OK) return st;
  mg::KernelArgs a{};
  a.p_src = x;
  a.q_src = dy;
  a.offsets = offsets;
  a.out = dw;
  a.M = M; a.N = N; a.K = K; a.E = E;
  a.accumulate = accumulate ? 1 : 0;
  return launch(mg::kWgrad, a, 0, s, ws);
}

}  // namespace

mg_status kgemm_wgrad(const void* dy, const void* x, const int32_t* offsets, float* dw,
                      int64_t M, int64_t N, int64_t K, int32_t E, int32_t accumulate,
                      void* stream) {
  return wgrad_common(dy, x, offsets, dw, M, N, K, E, accumulate, stream, mg::kWsStream);
}

mg_status kgemm_wgrad_noalloc(const void* dy, const void* x, const int32_t* offsets, float* dw,
                              int64_t M, int64_t N, int64_t K, int32_t E, int32_t accumulate,
                              void* stream) {
  return wgrad_common(dy, x, offsets, dw, M, N, K, E, accumulate, stream, mg::kWsStatic);
}

static_assert(MG_NOALLOC_SCRATCH_BYTES > 0, "scratch size");

const char* mg_status_str(int32_t status) {
  switch (status) {
    case MG_OK: return "MG_OK";
    case MG_ERR_NULL: return "MG_ERR_NULL: a required pointer is NULL";
    case MG_ERR_SHAPE:
      return "MG_ERR_SHAPE: sizes outside the entry point's rules (E in [1,1024]; N, K multiples "
             "of 8, of 16 for the token-major MXFP8 weight gradient; MXFP8 token counts and "
             "offsets multiples of 128 where the call reduces over tokens)";
    case MG_ERR_ALIGN: return "MG_ERR_ALIGN: data pointers must be 16-byte aligned";
    case MG_ERR_DEVICE: return "MG_ERR_DEVICE: current device is not gfx950 (or HIP failed)";
    case MG_ERR_LAUNCH: return "MG_ERR_LAUNCH: kernel launch failed";
    case MG_ERR_OFFSETS: return "MG_ERR_OFFSETS: offsets must start at 0, not decrease, end <= M";
    default: return "unknown mg_status";
  }
}

int32_t mg_abi_version(void) { return 1; }

mg_status mg_check_list_host(const mg_gemm_desc* desc_host, int32_t G) {
  if (!desc_host) return MG_ERR_NULL;
  if (G < 1 || G > mg::kMaxExperts) return MG_ERR_SHAPE;
  for (int32_t g = 0; g < G; ++g) {
    const mg_gemm_desc& d = desc_host[g];
    if (d.m < 0 || d.n < 0 || d.k < 0) return MG_ERR_SHAPE;
    if ((d.n & 7) || (d.k & 7) || (d.lda & 7) || (d.ldb & 7) || (d.ldd & 7)) return MG_ERR_SHAPE;
    if (d.lda < d.k || d.ldb < d.k || d.ldd < d.n || d.lda > kMaxDim || d.ldb > kMaxDim ||
        d.ldd > kMaxDim)
      return MG_ERR_SHAPE;
    if (d.m == 0 || d.n == 0) continue;
    if (!d.d || (d.k > 0 && (!d.a || !d.b))) return MG_ERR_NULL;
    if (!aligned16(d.d) || (d.k > 0 && (!aligned16(d.a) || !aligned16(d.b)))) return MG_ERR_ALIGN;
  }
  return MG_OK;
}

mg_status mg_check_offsets_host(const int32_t* offsets_host, int32_t E, int64_t M) {
  if (!offsets_host) return MG_ERR_NULL;
  if (E < 1 || E > mg::kMaxExperts || M < 0 || M > kMaxRows) return MG_ERR_SHAPE;
  if (offsets_host[0] != 0) return MG_ERR_OFFSETS;
  for (int32_t e = 0; e < E; ++e)
    if (offsets_host[e + 1] < offsets_host[e]) return MG_ERR_OFFSETS;
  if (offsets_host[E] > M) return MG_ERR_OFFSETS;
  return MG_OK;
}

}  // extern "C"
