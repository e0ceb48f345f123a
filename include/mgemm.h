/* mgemm.h -- C ABI of the MoE grouped GEMM library for AMD Instinct MI355X
 * (gfx950).  Library: libmgemm.so.
 *
 * The operations follow the problem statement of the RapidGEMM README
 * ("Kernels"): an M-grouped GEMM that computes the grouped forward or
 * input-gradient product from expert-grouped rows x [M, K], per-expert
 * weights w [E, N, K] and a cumulative row-offset array with a leading zero;
 * and a K-grouped GEMM that computes the grouped FP32 weight gradient from the
 * same expert-grouped rows.  The backward of a GEMM is two GEMMs, dgrad and
 * wgrad (DeepGEMM issue #10).  One C entry point per operation serves every
 * front end, as the TransformerEngine PR #2045 review asks of its grouped-GEMM
 * API.
 *
 * Conventions shared by all calls
 *   - (M, N, K, E) always describe the FORWARD problem: X [M, K],
 *     W [E, N, K], Y [M, N].  All tensors are dense, row-major, contiguous.
 *   - bf16 tensors are passed as pointers to 16-bit bf16 bit patterns.
 *   - offsets: int32 DEVICE array of E + 1 entries, offsets[0] == 0,
 *     non-decreasing, offsets[E] <= M.  Expert e owns rows
 *     offsets[e] <= i < offsets[e+1]; experts may be empty and row counts are
 *     arbitrary (no multiple-of-tile requirement).  The library never reads
 *     the offsets on the host: this is a precondition, checked only when the
 *     environment variable MGEMM_VALIDATE=1 (debug; it copies the offsets to
 *     the host and synchronises the stream).
 *   - All data pointers are DEVICE pointers, 16-byte aligned; N and K must be
 *     multiples of 8 (every row starts 16-byte aligned).  1 <= E <= 1024.
 *     M < 2^31, N and K <= 2^22 (the longest reduction one tile runs), and
 *     a call's count of 256 x 256 output tiles below 2^31.  Each call below
 *     adds its own limits.  Outputs must not alias inputs.
 *   - stream: a hipStream_t (NULL = the null stream).  Each call only
 *     enqueues work on that stream and returns; it never synchronises or
 *     keeps a caller pointer after returning.  The caller owns every buffer
 *     and must keep it alive until the stream has run the work.  The one
 *     allocation: the first kgemm_wgrad call on a (device, stream) pair that
 *     is not being captured into a graph allocates a 64 MiB device workspace
 *     for that pair (hipMalloc, its counters cleared with a synchronous
 *     hipMemset -- nothing is enqueued on the caller's stream for it) and
 *     keeps it until the process ends; calls on one stream share it in stream
 *     order, calls on different streams never share one.  A kgemm_wgrad call
 *     made while its stream is being captured allocates nothing and runs
 *     without the token split (so it enqueues exactly one kernel and no
 *     memory operation).  If the allocation fails the call still runs,
 *     without the split.  MGEMM_SPLIT=0 turns the split (and the workspace)
 *     off.  kgemm_wgrad_noalloc never allocates (a static device array).
 *   - Host-detectable errors are returned before anything is enqueued.
 *     Launch failures return MG_ERR_LAUNCH.  Faults during execution surface
 *     at the caller's next synchronisation, like any stream work.  Nothing
 *     throws across this ABI.
 *   - Thread safety: calls may be made concurrently from several threads; the
 *     shared state is a per-device architecture check done once, the
 *     mutex-protected table of per-stream workspaces and the per-device
 *     address of kgemm_wgrad_noalloc's static array.
 */
#ifndef MGEMM_H
#define MGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mg_status {
  MG_OK = 0,
  MG_ERR_NULL = 1,     /* a required pointer is NULL                          */
  MG_ERR_SHAPE = 2,    /* sizes outside the entry point's rules: E < 1 or > 1024,
                          negative or too large sizes, N or K not a multiple of
                          8 (16 for kgemm_wgrad_mx_tm), MXFP8 token counts or
                          offsets not multiples of 128 where required         */
  MG_ERR_ALIGN = 3,    /* a data pointer is not 16-byte aligned               */
  MG_ERR_DEVICE = 4,   /* current device is not gfx950, or HIP query failed   */
  MG_ERR_LAUNCH = 5,   /* the kernel launch was rejected                      */
  MG_ERR_OFFSETS = 6   /* offsets violate the precondition (validation only)  */
} mg_status;

/* M-grouped forward (RapidGEMM README, "Kernels", Mgemm forward form):
 *   y[i, n] = sum_k x[i, k] * w[e, n, k]   for offsets[e] <= i < offsets[e+1]
 * x: bf16 [M, K]; w: bf16 [E, N, K]; y: bf16 [M, N] (written).
 * Products accumulate in fp32; y is the fp32 sum rounded to nearest even.
 * Rows i >= offsets[E] of y are not touched.  M == 0 or N == 0 is a no-op;
 * K == 0 writes zeros to the owned rows.
 * max_m_per_e: optional hint, an upper bound on any expert's row count, used
 * only to size the launch (0 = unknown).  Results never depend on it: with a
 * hint that is too small each workgroup simply processes more tiles.  A
 * negative value gives MG_ERR_SHAPE. */
mg_status mgemm_fwd(const void* x, const void* w, const int32_t* offsets, void* y,
                    int64_t M, int64_t N, int64_t K, int32_t E, int64_t max_m_per_e,
                    void* stream);

/* M-grouped input gradient (the same call's input-gradient form):
 *   dx[i, k] = sum_n dy[i, n] * w[e, n, k]   for offsets[e] <= i < offsets[e+1]
 * dy: bf16 [M, N]; w: bf16 [E, N, K]; dx: bf16 [M, K] (written).
 * fp32 accumulation, round to nearest even.  Rows i >= offsets[E] of dx are
 * not touched.  M == 0 or K == 0 is a no-op; N == 0 writes zeros.
 * max_m_per_e: launch-size hint, as for mgemm_fwd. */
mg_status mgemm_dgrad(const void* dy, const void* w, const int32_t* offsets, void* dx,
                      int64_t M, int64_t N, int64_t K, int32_t E, int64_t max_m_per_e,
                      void* stream);

/* Gate-up forward with the SwiGLU activation fused into the epilogue, on rows
 * gathered through an index (the fused-with-SwiGLU and MoE-layout kernels of
 * the DeepGEMM issue #10 thread; w13 stacks each expert's gate and up weights
 * as the RapidGEMM README's gw13 gradient does):
 *   g = x[r] . w13[e, j],  u = x[r] . w13[e, I + j],  r = gather ? gather[i] : i
 *   h[i, j] = silu(g) * u = g u / (1 + exp(-g))   for offsets[e] <= i < offsets[e+1]
 * x: bf16 [T, K] when gather != NULL (token-major rows; gather: int32 DEVICE
 * array [M] of row indices in [0, T), repeats allowed), else bf16 [M, K]
 * (already expert-grouped; T is ignored).  w13: bf16 [E, 2I, K], gate rows
 * 0..I-1, up rows I..2I-1.  h: bf16 [M, I] (written).  fp32 accumulation, the
 * activation in fp32, one rounding to bf16 (nearest even).  Rows i >=
 * offsets[E] of h are not touched; an index outside [0, T) reads zeros.
 * I and K multiples of 8; 2 I K and (with gather) T K below 2^31 elements.
 * M == 0 or I == 0 is a no-op.  Allocates nothing.  max_m_per_e: launch-size
 * hint, as for mgemm_fwd. */
mg_status mgemm_fwd_swiglu(const void* x, const int32_t* gather, const void* w13,
                           const int32_t* offsets, void* h, int64_t M, int64_t T, int64_t I,
                           int64_t K, int32_t E, int64_t max_m_per_e, void* stream);

/* mgemm_fwd_swiglu that also writes the pre-activation the backward needs:
 * gu: bf16 [M, 2I] (written when not NULL): gu[i, j] = g, gu[i, I + j] = u,
 * each the fp32 accumulator rounded to nearest even (the values h was computed
 * from, before that rounding).  16-byte aligned.  Otherwise exactly
 * mgemm_fwd_swiglu, which is this call with gu == NULL. */
mg_status mgemm_fwd_swiglu_gu(const void* x, const int32_t* gather, const void* w13,
                              const int32_t* offsets, void* h, void* gu, int64_t M, int64_t T,
                              int64_t I, int64_t K, int32_t E, int64_t max_m_per_e,
                              void* stream);

/* Down-projection input gradient fused with the SwiGLU backward (DeepGEMM
 * issue #10: a kernel fused with SwiGLU is part of a weight-gradient path).
 * With the forward h = silu(g) u (mgemm_fwd_swiglu_gu) and y = h W2[e]^T:
 *   dh[i, j]  = sum_n dy[i, n] w2[e, n, j]        (fp32, not stored)
 *   dgu[i, j]     = dh u silu'(g),  silu'(g) = s (1 + g (1 - s)),  s = 1/(1 + e^-g)
 *   dgu[i, I + j] = dh silu(g)
 * with g = gu[i, j], u = gu[i, I + j], for offsets[e] <= i < offsets[e+1].
 * dy: bf16 [M, N]; w2: bf16 [E, N, I] (the down weights, N = model width);
 * gu: bf16 [M, 2I] (the saved pre-activation); dgu: bf16 [M, 2I] (written,
 * the gradient of gu, ready for the gate-up weight and input gradients).
 * The activation backward in fp32, one rounding to bf16.  Rows i >=
 * offsets[E] of dgu are not touched.  I and N multiples of 8; all pointers
 * 16-byte aligned.  M == 0 or I == 0 is a no-op; N == 0 writes zeros.
 * Allocates nothing.  max_m_per_e: launch-size hint, as for mgemm_fwd. */
mg_status mgemm_dgrad_swiglu(const void* dy, const void* w2, const void* gu,
                             const int32_t* offsets, void* dgu, int64_t M, int64_t N, int64_t I,
                             int32_t E, int64_t max_m_per_e, void* stream);

/* Token-order combine of routed rows, the inverse of the gather of
 * mgemm_fwd_swiglu (the MoE layout of the DeepGEMM issue #10 thread): the
 * backward of the dispatch gather sums each token's row gradients, the
 * layer's output combine sums its experts' outputs with the router weights:
 *   out[t, :] = sum_{j < k} weights[t, j] rows[token_rows[t, j], :]
 * rows: bf16 [M, D]; token_rows: int32 [T, k] DEVICE array, entry -1 (or any
 * index outside [0, M)) = no row; weights: fp32 [T, k] DEVICE or NULL (all
 * 1); out: bf16 [T, D] (written; must not overlap rows).  fp32 accumulation in
 * ascending j (bitwise reproducible), one rounding to nearest even.  D a
 * multiple of 8, 1 <= k <= 64; rows and out 16-byte aligned, token_rows and
 * weights 4-byte aligned.  T == 0 or D == 0 is a no-op.  Allocates nothing. */
mg_status mg_moe_combine(const void* rows, const int32_t* token_rows, const float* weights,
                         void* out, int64_t M, int64_t T, int32_t k, int64_t D, void* stream);

/* One group of mgemm_list: D [m, n] = A [m, k] B [n, k]^T (bf16 in and out,
 * fp32 accumulation, round to nearest even), row-major with row strides in
 * elements.  All three pointers are DEVICE pointers, 16-byte aligned; k, n and
 * the strides multiples of 8, lda >= k, ldb >= k, ldd >= n, strides <= 2^22.
 * m, n, k >= 0: a group with m == 0 or n == 0 does nothing; k == 0 writes
 * zeros. */
typedef struct mg_gemm_desc {
  const void* a;
  const void* b;
  void* d;
  int32_t m, n, k;
  int32_t lda, ldb, ldd;
} mg_gemm_desc;

/* A list of independent GEMMs with per-group shapes and pointers in one
 * launch (the TransformerEngine PR #2045 review asks for one C API over lists
 * of per-group tensors; the CUTLASS discussion #1452 flattens nested grouped
 * GEMMs -- LoRA adapters x MoE experts -- into such a list).  desc: DEVICE
 * array of G descriptors, 8-byte aligned, 1 <= G <= 1024; read by the kernel's
 * own scheduler, never on the host (checked on the host only under
 * MGEMM_VALIDATE=1, with mg_check_list_host).  The D regions must not overlap
 * each other or any input.  Allocates nothing.  M- and K-grouped problems mix
 * in one list: a K-grouped weight gradient dW_e = dY_e^T X_e is the entry
 * a = dY^T + offsets[e], b = X^T + offsets[e] (token-axis-last copies [N, M]
 * and [K, M], lda = ldb = M), m = N, n = K, k = the expert's token count. */
mg_status mgemm_list(const mg_gemm_desc* desc, int32_t G, void* stream);

/* Host-side check of a descriptor list held in HOST memory (no device use):
 * MG_OK, or MG_ERR_SHAPE / MG_ERR_NULL / MG_ERR_ALIGN for the first group that
 * breaks the rules above (within a group a size error is reported before a
 * NULL pointer, and a NULL pointer before a misaligned one; pointers of a
 * group with m == 0 or n == 0, and a and b when k == 0, are not checked). */
mg_status mg_check_list_host(const mg_gemm_desc* desc_host, int32_t G);

/* MXFP8 M-grouped forward (torchao PR #3416: MoE training with MXFP8
 * grouped GEMMs whose e8m0 block scales are first rearranged into the layout
 * the GEMM reads; MXFP8 taken as the OCP microscaling format: E4M3 elements,
 * one E8M0 scale 2^(s - 127) per 32 consecutive reduction steps):
 *   y[i, n] = sum_k X[i, k] W[e, n, k]   for offsets[e] <= i < offsets[e+1],
 *   X[i, k] = e4m3(x[i, k]) 2^(xs(i, k/32) - 127),  W likewise with ws.
 * x: uint8 E4M3 codes [M, K]; w: uint8 E4M3 codes [E, N, K]; y: bf16 [M, N]
 * (written, round to nearest even).
 * x_scale: uint8 E8M0 codes in the BLOCKED layout [ceil(K/128)][M][4] (entry
 * [t][i][j] scales x[i, 128 t + 32 j .. + 31]); w_scale: [E][ceil(K/128)][N][4]
 * likewise per expert.  mg_mx_scales_blocked makes this layout from the plain
 * [rows][K/32] one.  Pointers: x, w, y 16-byte aligned, scales 4-byte aligned.
 * K a multiple of 32, N a multiple of 8; ceil(K/128) M and ceil(K/128) N
 * below 2^29.  The products are those of the gfx950 scaled fp8 matrix-core
 * instruction, accumulated in fp32: each 64-step product is exact to about
 * 2^-13 of the sum of its absolute terms, not to fp32 rounding.  The MX
 * input gradient is the same call on dy and the weights transposed to
 * [E, K, N] and quantized along N (each GEMM's operands are quantized along
 * its own reduction axis, DeepGEMM issue #10).  M == 0 or N == 0 is a no-op;
 * K == 0 writes zeros.  Allocates nothing.  max_m_per_e: launch-size hint, as
 * for mgemm_fwd. */
mg_status mgemm_fwd_mx(const void* x, const void* x_scale, const void* w, const void* w_scale,
                       const int32_t* offsets, void* y, int64_t M, int64_t N, int64_t K, int32_t E,
                       int64_t max_m_per_e, void* stream);

/* MXFP8 K-grouped weight gradient in FP32 (torchao PR #3416: MXFP8 grouped
 * GEMMs with groups along K, the token axis of the weight gradient; DeepGEMM
 * issue #10: its operands are quantized along the tokens, and FP8 wgrad needs
 * token counts that are multiples of 128):
 *   dw[e, n, k] (= or +=) sum_{offsets[e] <= i < offsets[e+1]} DYT[n, i] XT[k, i]
 * with DYT, XT the dequantized E4M3 codes times their E8M0 block scales.
 * dyt: uint8 E4M3 [N, M] (dY transposed, token axis last); xt: uint8 E4M3 [K, M];
 * dyt_scale: blocked [M/128][N][4] (entry [t][n][j] scales dyt[n, 128 t + 32 j
 * .. + 31]); xt_scale: blocked [M/128][K][4]; dw: fp32 [E, N, K].
 * M a multiple of 128, and every offsets[e] a multiple of 128 (experts padded
 * to whole 128-token stages; checked only under MGEMM_VALIDATE=1 -- otherwise
 * each expert's range is widened to whole stages: wrong sums, but never
 * misaligned or out-of-bounds accesses); N and K
 * multiples of 8; 256 M < 2^32; M/128 N and M/128 K below 2^29.  Pointers:
 * dyt, xt, dw 16-byte aligned, scales 4-byte aligned.  accumulate as for
 * kgemm_wgrad; an expert with no rows gets zeros (or is left as it was).  The
 * products are the scaled fp8 matrix-core products (about 2^-13 of the sum of
 * the absolute terms per 64 tokens), accumulated in fp32.  N == 0 or K == 0 is
 * a no-op.  Allocates nothing, and never splits a tile's token range. */
mg_status kgemm_wgrad_mx(const void* dyt, const void* dyt_scale, const void* xt,
                         const void* xt_scale, const int32_t* offsets, float* dw, int64_t M,
                         int64_t N, int64_t K, int32_t E, int32_t accumulate, void* stream);

/* kgemm_wgrad_mx on operands as the layer holds them, token-major: the same
 * weight gradient, with
 *   dw[e, n, k] (= or +=) sum_{offsets[e] <= i < offsets[e+1]} DY[i, n] X[i, k]
 * where DY, X are the dequantized E4M3 codes dy8 [M, N] and x8 [M, K] (rows of
 * tokens, quantized along the tokens: one E8M0 scale per 32 consecutive tokens
 * of a column) -- no transposed copies: the kernel stages 128-token blocks of
 * the rows and transposes them in its LDS reads (the weight gradient needs
 * transposed operands, DeepGEMM issue #10).  dy_scale: blocked [M/128][N][4]
 * (entry [t][n][j] scales dy8[128 t + 32 j .. + 31, n], i.e.
 * mg_mx_scales_blocked of the per-column scales [N][M/32]); x_scale: blocked
 * [M/128][K][4].  M a multiple of 128 and every offsets[e] a multiple of 128
 * (as for kgemm_wgrad_mx); N and K multiples of 16; M/128 N and M/128 K below
 * 2^29.  Pointers: dy8, x8, dw 16-byte aligned, scales 4-byte aligned.
 * Results bitwise equal to kgemm_wgrad_mx on the transposed codes with the
 * same scales.  N == 0 or K == 0 is a no-op.  Allocates nothing. */
mg_status kgemm_wgrad_mx_tm(const void* dy8, const void* dy_scale, const void* x8,
                            const void* x_scale, const int32_t* offsets, float* dw, int64_t M,
                            int64_t N, int64_t K, int32_t E, int32_t accumulate, void* stream);

/* Blocked layout of MXFP8 scales (the torchao PR #3416 "scale blocked format"
 * step, for the layout above): scales: uint8 [batch][rows][K/32] (DEVICE);
 * blocked: uint8 [batch][ceil(K/128)][rows][4] (DEVICE, 4-byte aligned,
 * written; must not overlap scales), entry [b][t][r][j] = scales[b][r][4t + j],
 * or 127 (the code of 1.0) where 4t + j >= K/32.  K a multiple of 32.
 * Enqueued on `stream`; allocates nothing. */
mg_status mg_mx_scales_blocked(const void* scales, void* blocked, int64_t rows, int64_t K,
                               int64_t batch, void* stream);

/* K-grouped weight gradient in FP32 (RapidGEMM README, "Kernels", Kgemm;
 * wgrad is x^T dy, DeepGEMM issue #10, laid out like w so it can update w):
 *   dw[e, n, k] (= or +=) sum_{offsets[e] <= i < offsets[e+1]} dy[i, n] * x[i, k]
 * dy: bf16 [M, N]; x: bf16 [M, K]; dw: fp32 [E, N, K].
 * accumulate == 0: dw is overwritten, and an expert with no rows gets zeros.
 * accumulate != 0: the sum is added to dw's contents (fp32 gradient
 * accumulation, as in the TransformerEngine PR #2045 review of
 * fuse_wgrad_accumulation), and an empty expert's block is left as it was.
 * Rows i >= offsets[E] do not contribute.  N == 0 or K == 0 is a no-op.
 * An expert much heavier than the rest may have its token range split in two
 * halves whose fp32 partial sums are added as (half + half), then + dw when
 * accumulating: results are bitwise reproducible from call to call (a call
 * captured into a graph computes such tiles whole, which may differ from an
 * uncaptured call in the last bits).  This is the call that uses the
 * per-stream workspace described above.  The halves meet through one ticket
 * word per split tile, tagged with a per-launch mark, so a word left behind
 * by a launch that did not complete cannot mislead a later one. */
mg_status kgemm_wgrad(const void* dy, const void* x, const int32_t* offsets, float* dw,
                      int64_t M, int64_t N, int64_t K, int32_t E, int32_t accumulate,
                      void* stream);

/* Bytes of kgemm_wgrad_noalloc's static device array: 4 KiB of ticket words
 * and two 256 x 256 fp32 slots for each of at most 128 split tiles. */
#define MG_NOALLOC_SCRATCH_BYTES (4096 + 2 * 128 * 256 * 256 * 4)

/* kgemm_wgrad for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as kgemm_wgrad (bitwise the
 * same results as an uncaptured kgemm_wgrad call), but the token split's
 * workspace is a static device array of MG_NOALLOC_SCRATCH_BYTES that each
 * GPU the library runs on holds from load until the process ends; the call
 * allocates nothing, enqueues only the kernel (no memset) and also splits
 * while its stream is being captured.  The array's need is bounded by
 * construction (at most 128 split tiles per launch, whatever the sizes), so
 * no size is rejected for it.  Every call on one GPU shares that GPU's array:
 * calls that may run at the same time on one GPU (other streams, other
 * threads, replays of graphs holding this call) race on it and can give
 * wrong results; order them on one stream.  Returns MG_ERR_LAUNCH if the
 * array's device address cannot be obtained. */
mg_status kgemm_wgrad_noalloc(const void* dy, const void* x, const int32_t* offsets, float* dw,
                              int64_t M, int64_t N, int64_t K, int32_t E, int32_t accumulate,
                              void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* mg_status_str(int32_t status);

/* Version of this ABI; bumped on any incompatible change. */
int32_t mg_abi_version(void);

/* Host-side check of an offsets array held in HOST memory (no device use):
 * MG_OK if offsets[0] == 0, non-decreasing, offsets[E] <= M; MG_ERR_OFFSETS
 * otherwise; MG_ERR_NULL / MG_ERR_SHAPE for a NULL pointer or bad E / M. */
mg_status mg_check_offsets_host(const int32_t* offsets_host, int32_t E, int64_t M);

#ifdef __cplusplus
}
#endif

#endif /* MGEMM_H */
