/*
 * kda.h -- C ABI of libkda, the MI355X (gfx950) chunked forward of Kimi Delta
 * Attention.
 *
 * Source of the operation: FlashKDA pages. "Core Kernel API / flash_kda.fwd"
 * (ccm-staging.vinena.studio, FlashKDA Delta Attention skill) gives the call
 *   fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
 *       initial_state=None, final_state=None, cu_seqlens=None);
 * "Kernel API and Constraints" (trend.ondo.sh, MoonshotAI/FlashKDA) fixes
 * K = V = 128, cu_seqlens only with B = 1, and initial/final states that are
 * bf16 or fp32 or absent and of one dtype; the summary paragraph of the
 * ccm-staging page fixes bf16 activations and describes varlen packing.
 *
 * The pages print no formula. libkda computes, per sequence n and head h, the
 * gated delta rule with per-channel decay along the key axis:
 *   q^ = q / sqrt(|q|^2 + 1e-6),  k^ = k / sqrt(|k|^2 + 1e-6)
 *   log a_c = max(-exp(A_log[h]) * softplus(g_c + dt_bias[h,c]), lower_bound)
 *   S_t = (I - beta_t k^ k^T) Diag(a_t) S_{t-1} + beta_t k^ v_t^T   (S is K x V)
 *   out_t = scale * S_t^T q^
 * evaluated chunkwise (64 tokens per chunk) on the GPU.
 *
 * Conventions for every entry point:
 *  - Device pointers unless stated otherwise; all buffers belong to the caller.
 *    libkda never allocates, frees or retains device memory.
 *  - Activations are row-major contiguous:
 *      q, k, g : bf16 [B, T, H, 128]      v, out : bf16 [B, T, H, 128]
 *      beta    : bf16 [B, T, H]           A_log  : fp32 [H]
 *      dt_bias : fp32 [H, 128]
 *      initial_state, final_state : [N, H, 128(K), 128(V)], bf16 or fp32,
 *                                   S[n][h][k][v] with o = S^T q over k.
 *    With cu_seqlens (int32 [N+1], device, sorted, cu[0] = 0, cu[N] = T) the
 *    batch is B = 1 and sequence n owns tokens [cu[n], cu[n+1]); otherwise
 *    N = B and sequence n is batch row n.
 *  - Calls are asynchronous on `stream`; nothing synchronises the host and
 *    cu_seqlens is never read on the host (its validity is a precondition).
 *  - Errors are detected before anything is enqueued and returned as a
 *    kda_status; on KDA_ERR_HIP the contents of out/final_state are undefined.
 *  - The library is stateless apart from the optional profiling switch and is
 *    safe to call from several host threads on different streams.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef KDA_API
#define KDA_API __attribute__((visibility("default")))
#endif

/* Status codes returned by kda_fwd and kda_decode. */
typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL                         */
    KDA_ERR_HEAD_DIM = 2,    /* head dims other than K = V = 128 (kda_fwd and
                                kda_fwd_noalloc: other than K = V = 128 or 64)      */
    KDA_ERR_SHAPE = 3,       /* B, T, H <= 0, num_seqs <= 0 with cu_seqlens,
                                B != 1 with cu_seqlens, or sizes past the limits
                                below (KDA_MAX_HEADS, 32-bit grids and offsets)     */
    KDA_ERR_STATE_DTYPE = 4, /* state_dtype inconsistent with the state pointers   */
    KDA_ERR_ARG = 5,         /* scale or lower_bound non-finite, lower_bound > 0,
                                or a tensor that must be 16-byte aligned is not
                                (see "Alignment" below)                            */
    KDA_ERR_WORKSPACE = 6,   /* workspace NULL, not 256-byte aligned, or smaller
                                than kda_fwd_workspace_size                        */
    KDA_ERR_ALIAS = 7,       /* out overlaps an input, or the states overlap only
                                partially                                          */
    KDA_ERR_HIP = 8,         /* a HIP launch/runtime error after validation         */
    KDA_ERR_SCRATCH = 9      /* kda_fwd_noalloc: the call needs more workspace than
                                KDA_NOALLOC_SCRATCH_BYTES                           */
} kda_status;

/* dtype of initial_state / final_state (one dtype for both). */
typedef enum {
    KDA_STATE_NONE = 0,      /* both state pointers NULL                            */
    KDA_STATE_BF16 = 1,
    KDA_STATE_FP32 = 2
} kda_state_dtype;

/* Size limits (checked, KDA_ERR_SHAPE): H <= KDA_MAX_HEADS (a chunk's rows are
 * addressed with 32-bit byte offsets); with cu_seqlens, T <= INT32_MAX (int32
 * offsets); for kda_fwd, (chunk slots) * H and 8 * N * H at most INT32_MAX, and for
 * kda_decode N * H at most INT32_MAX (launch grids). */
#define KDA_MAX_HEADS 65536

/* Alignment (checked, KDA_ERR_ARG): q, k, v, g, out, dt_bias and the state tensors
 * (initial_state, final_state, the decode state, dfinal_state, dinitial_state) and
 * the fp32 gradients of kda_bwd must be 16-byte aligned: the kernels move them in
 * 16-byte pieces. beta, A_log, cu_seqlens and dout need only their element
 * alignment. Tensors allocated by torch are 256-byte aligned. */

/* Most negative lower_bound of the fast form of kda_fwd. Inside one 16-token
 * sub-chunk the fast form anchors the decay factors at the middle token, so the
 * largest factor is exp(8 * |lower_bound|); -10 keeps it inside the bf16/fp32
 * range (exp(88.7)). Below it, kda_fwd builds every factor from exponents <= 0
 * and evaluates the 16 x 16 diagonal blocks of the in-chunk matrices element by
 * element (about 1.5 times the chunk preparation time); any finite
 * lower_bound <= 0 is accepted. */
#define KDA_LOWER_BOUND_NARROW (-10.0f)

/*
 * kda_fwd -- chunked KDA forward (the flash_kda.fwd call of the pages).
 *
 *  q, k, v, g, beta : bf16 inputs, layouts above; must not overlap `out`.
 *  scale            : multiplies the output only (finite).
 *  out              : bf16 [B, T, H, 128], written in full (round to nearest even).
 *  A_log, dt_bias   : fp32 gate parameters.
 *  lower_bound      : clamp of log a in natural-log units, finite and <= 0;
 *                     0 means no decay (see KDA_LOWER_BOUND_NARROW).
 *  initial_state    : NULL (zero state) or [N, H, 128, 128] of state_dtype.
 *  final_state      : NULL (not returned) or [N, H, 128, 128] of state_dtype;
 *                     receives S after the last token of each sequence (bf16 is
 *                     rounded to nearest even from the fp32 state). It may be
 *                     the same pointer as initial_state (in-place update) but
 *                     may not overlap it otherwise.
 *  state_dtype      : KDA_STATE_NONE iff both state pointers are NULL.
 *  cu_seqlens       : NULL, or int32 [num_seqs + 1] on the device (B must be 1).
 *  num_seqs         : number of packed sequences when cu_seqlens != NULL, else
 *                     ignored (N = B).
 *  B, T, H, K, V    : sizes; K = V = 128 (the pages' head dims, "Kernel API and
 *                     Constraints") or K = V = 64, where every 128 in the layouts
 *                     above reads 64 (q, k, g, v, out rows of 64, dt_bias [H, 64],
 *                     states [N, H, 64, 64]). T counts packed tokens when
 *                     cu_seqlens is given.
 *  workspace        : device scratch of at least kda_fwd_workspace_size(...)
 *                     bytes, 256-byte aligned; contents on entry are ignored and
 *                     on return hold per-chunk intermediates (internal format).
 *  stream           : hipStream_t (as void*) the kernels are enqueued on; NULL
 *                     means the default stream.
 */
KDA_API int kda_fwd(const void *q, const void *k, const void *v, const void *g,
            const void *beta, float scale, void *out, const float *A_log,
            const float *dt_bias, float lower_bound, const void *initial_state,
            void *final_state, int state_dtype, const int32_t *cu_seqlens,
            int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K,
            int64_t V, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_fwd_noalloc -- kda_fwd without a workspace argument, for callers that
 * cannot allocate device memory at call time: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The workspace kda_fwd
 * would take from the caller comes from a scratch array built into the library
 * (a file-scope device array of KDA_NOALLOC_SCRATCH_BYTES, one per GPU the
 * library runs on, held until the process ends); nothing is allocated or freed
 * by the call. The kernels, their results and every argument rule are those of
 * kda_fwd, and the output is the same bit for bit.
 *
 *  Arguments as for kda_fwd, without workspace / workspace_bytes.
 *  Errors as for kda_fwd, plus KDA_ERR_SCRATCH (checked before any HIP call)
 *  when kda_fwd_workspace_size(B, T, H, num_seqs) > KDA_NOALLOC_SCRATCH_BYTES,
 *  and KDA_ERR_HIP if the scratch's device address cannot be obtained.
 *  The first call on a GPU looks up that GPU's scratch address (the device of
 *  `stream`, or the current device for the NULL stream).
 *  Every call on one GPU uses that GPU's one scratch array: calls that may
 *  overlap in time on one GPU (other streams, other host threads) race and
 *  must be serialised by the caller; calls in order on one stream are safe.
 *  The scratch needs no clearing between calls: every call writes each part
 *  it reads before reading it.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
KDA_API int kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
            const void *beta, float scale, void *out, const float *A_log,
            const float *dt_bias, float lower_bound, const void *initial_state,
            void *final_state, int state_dtype, const int32_t *cu_seqlens,
            int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K,
            int64_t V, void *stream);

/*
 * kda_fwd_workspace_size -- bytes of workspace kda_fwd needs (host only).
 *  In the pages' call ("Core Kernel API / flash_kda.fwd", ccm-staging page) the
 *  caller hands in every result buffer (out, final_state); libkda keeps that
 *  convention for the scratch its chunked kernels pass between them, which is
 *  one more caller-owned buffer whose size this call reports (chunk table,
 *  per-chunk records, segment maps of the segment-parallel scan).
 *  num_seqs = 0 means no cu_seqlens (N = B); otherwise B must be 1 and T is the
 *  packed token count. Returns 0 for invalid sizes (those kda_fwd rejects with
 *  KDA_ERR_SHAPE).
 */
KDA_API size_t kda_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t num_seqs);

/*
 * kda_decode -- one token per sequence: the single-token step of the same
 * recurrence with the state updated in place (the decode use of flash_kda.fwd
 * with T = 1 per sequence; the pages' argument list and state constraints as
 * for kda_fwd). No chunking is involved, so any finite lower_bound <= 0 is
 * accepted and no workspace is needed.
 *
 *  q, k, v, g : bf16 [N, H, 128] (token of sequence n);  beta : bf16 [N, H]
 *  out        : bf16 [N, H, 128], written in full (round to nearest even);
 *               must not overlap an input or the state.
 *  scale, A_log, dt_bias : as for kda_fwd.
 *  lower_bound: clamp of log a in natural-log units, finite and <= 0.
 *  state      : [N, H, 128(K), 128(V)] of state_dtype (KDA_STATE_BF16 or
 *               KDA_STATE_FP32), read and overwritten with the state after the
 *               token (bf16 rounded to nearest even from fp32); must not
 *               overlap an input.
 *  N, H, K, V : sizes; K and V must be 128.
 *  stream     : hipStream_t (as void*); NULL means the default stream.
 * Errors as for kda_fwd (KDA_ERR_STATE_DTYPE if state_dtype is NONE or
 * unknown, KDA_ERR_NULL if state is NULL); nothing is enqueued on error.
 */
KDA_API int kda_decode(const void *q, const void *k, const void *v, const void *g,
               const void *beta, float scale, void *out, const float *A_log,
               const float *dt_bias, float lower_bound, void *state, int state_dtype,
               int64_t N, int64_t H, int64_t K, int64_t V, void *stream);

/*
 * kda_bwd -- gradients of the forward above (the pages show only the forward;
 * this is its derivative, for training). For
 *   L = sum(dout * out) + sum(dfinal_state * final_state)
 * with out and final_state the results of kda_fwd on the same inputs, it
 * writes dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta, dL/dA_log, dL/ddt_bias and
 * dL/dinitial_state. lower_bound clamps: an element whose unclamped
 * -exp(A_log) softplus(g + dt_bias) lies below lower_bound passes no gradient
 * to g, dt_bias or A_log. Arithmetic is fp32 throughout.
 *
 *  q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, cu_seqlens, num_seqs,
 *  B, T, H, K, V : as for kda_fwd (any finite lower_bound <= 0).
 *  dout          : bf16 [B, T, H, 128], the gradient of out.
 *  initial_state : NULL (zero state) or [N, H, 128, 128] of state_dtype
 *                  (KDA_STATE_NONE iff NULL).
 *  dfinal_state  : NULL (zero) or fp32 [N, H, 128, 128], the gradient of the
 *                  final state.
 *  dq, dk, dv, dg: fp32 [B, T, H, 128];  dbeta : fp32 [B, T, H];
 *  dA_log        : fp32 [H];  ddt_bias : fp32 [H, 128] (sums over all tokens).
 *  dinitial_state: NULL (not returned) or fp32 [N, H, 128, 128].
 *  All outputs are written in full and may not overlap an input, each other or
 *  the workspace. The per-head sums are taken in a fixed order (deterministic).
 *  workspace     : at least kda_bwd_workspace_size(...) bytes, 256-byte
 *                  aligned (per chunk and head: 258 KiB of chunk quantities and
 *                  the fp32 state and state gradient at the chunk's ends).
 * Errors as for kda_fwd.
 */
KDA_API int kda_bwd(const void *q, const void *k, const void *v, const void *g,
            const void *beta, float scale, const void *dout, const float *A_log,
            const float *dt_bias, float lower_bound, const void *initial_state,
            int state_dtype, const float *dfinal_state, const int32_t *cu_seqlens,
            int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
            float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dA_log,
            float *ddt_bias, float *dinitial_state, void *workspace,
            size_t workspace_bytes, void *stream);

/* kda_bwd_workspace_size -- bytes of workspace kda_bwd needs (host only); sizes
 * as for kda_fwd_workspace_size, 0 for invalid sizes. */
KDA_API size_t kda_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t num_seqs);

/* kda_status_string -- static, NUL-terminated description of a kda_status code
 * (host only; "unknown kda status" for other values). The pages' debugging
 * advice ("Accuracy Verification and Debugging", trend.ondo.sh page) is to log
 * whether the fast kernel was selected or why a call was rejected; these
 * strings state the reason for each rejection, and the Python binding raises
 * them as its error messages. */
KDA_API const char *kda_status_string(int status);

/*
 * Kernel-level timing for measurement tools (host only, not thread-safe).
 *  kda_profile_enable(1) clears the record and makes later kda_fwd / kda_decode calls
 *  bracket each kernel they enqueue with hipEvents on the call's stream (up to
 *  8192 launches); kda_profile_enable(0) stops recording. kda_profile_read
 *  synchronises on the recorded events and aggregates them per kernel: it
 *  writes up to `cap` distinct kernel names (static strings), their summed
 *  durations in ms and launch counts, and returns the number of kernels, or -1
 *  on a HIP error. Events are created on first use and kept for the process.
 */
KDA_API int kda_profile_enable(int on);
KDA_API int kda_profile_read(const char **names, float *total_ms, int *counts, int cap);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
