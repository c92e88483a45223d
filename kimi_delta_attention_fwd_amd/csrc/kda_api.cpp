/*
 * kda_api.cpp -- C ABI of libkda (declared in include/kda.h): argument
 * validation, workspace carving and kernel launches on the caller's stream.
 *
 * The checks mirror the constraints the FlashKDA pages state for
 * flash_kda.fwd ("Kernel API and Constraints", trend.ondo.sh page: K = V = 128,
 * cu_seqlens only with B = 1, initial and final states bf16/fp32/None of one
 * dtype; "Core Kernel API / flash_kda.fwd", ccm-staging page: the argument
 * list). Everything is checked on the host before any HIP call, so every error
 * path can be exercised without a GPU.
 */
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "kda.h"
#include "kda_internal.h"

extern "C" hipError_t kda_launch_chunk_map(const int32_t *cu, int64_t nseq, int64_t T, int32_t *chunk_off,
                                           hipStream_t st);
extern "C" hipError_t kda_launch_prep(const void *q, const void *k, const void *v, const void *g,
                                      const void *beta, const float *A_log, const float *dt_bias,
                                      float scale, float lower_bound, const int32_t *cu,
                                      const int32_t *chunk_off, int64_t nseq, int64_t T, int64_t H,
                                      int64_t nslots, int64_t K, int64_t V, void *records, int64_t trim_max,
                                      hipStream_t st);
extern "C" int64_t kda_scan_many_max_chunks(const int32_t *cu, int64_t nseq, int64_t H, int64_t K, int64_t V,
                                            int64_t segc);
extern "C" hipError_t kda_launch_scan(const void *records, const int32_t *cu, const int32_t *chunk_off,
                                      int64_t nseq, int64_t T, int64_t H, int64_t nslots, int64_t K, int64_t V,
                                      void *out, const void *init_state, void *final_state, int state_fp32,
                                      int64_t segc, void *seg_area, hipStream_t st);
extern "C" hipError_t kda_launch_bwd(int stage, const void *q, const void *k, const void *v, const void *g,
                                     const void *beta, const void *dout, const float *A_log,
                                     const float *dt_bias, float scale, float lower_bound,
                                     const void *init, int init_fp32, const float *dfinal,
                                     const int32_t *cu, const int32_t *chunk_off, int64_t nseq, int64_t T,
                                     int64_t H, int64_t nslots, unsigned char *area, float *dq, float *dk,
                                     float *dv, float *dg, float *dbeta, float *dA_log, float *ddt_bias,
                                     float *dinit, hipStream_t st);
extern "C" hipError_t kda_launch_decode(const void *q, const void *k, const void *v, const void *g,
                                        const void *beta, const float *A_log, const float *dt_bias, float scale,
                                        float lower_bound, void *state, int state_fp32, void *out, int64_t N,
                                        int64_t H, hipStream_t st);

namespace {

struct Range {
    uintptr_t lo, hi; /* [lo, hi) */
};

Range rng(const void *p, size_t bytes)
{
    const uintptr_t a = (uintptr_t)p;
    return Range{a, a + bytes};
}

bool overlap(const Range &a, const Range &b)
{
    return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi;
}

/* ---- optional kernel timing: events around each launch, aggregated per kernel ---- */
constexpr int kMaxProf = 8192; /* launches recorded per enable() */
bool g_prof_on = false;
int g_prof_n = 0;
const char *g_prof_names[kMaxProf];
hipEvent_t g_ev[kMaxProf][2];
int g_ev_made = 0;

struct ProfScope {
    int idx;
    hipStream_t st;
    ProfScope(const char *name, hipStream_t s) : idx(-1), st(s)
    {
        if (!g_prof_on || g_prof_n >= kMaxProf) return;
        if (g_prof_n >= g_ev_made) {
            if (hipEventCreate(&g_ev[g_ev_made][0]) != hipSuccess) return;
            if (hipEventCreate(&g_ev[g_ev_made][1]) != hipSuccess) return;
            g_ev_made++;
        }
        idx = g_prof_n++;
        g_prof_names[idx] = name;
        (void)hipEventRecord(g_ev[idx][0], st);
    }
    ~ProfScope()
    {
        if (idx >= 0) (void)hipEventRecord(g_ev[idx][1], st);
    }
};

} // namespace

extern "C" const char *kda_status_string(int status)
{
    switch (status) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_HEAD_DIM:
        return "KDA_ERR_HEAD_DIM: K and V must both be 128 (kda_fwd and kda_fwd_noalloc also take K = V = 64)";
    case KDA_ERR_SHAPE:
        return "KDA_ERR_SHAPE: B, T, H must be positive and within the size limits (KDA_MAX_HEADS, 32-bit grids); with cu_seqlens B must be 1 and num_seqs positive";
    case KDA_ERR_STATE_DTYPE:
        return "KDA_ERR_STATE_DTYPE: state_dtype must be NONE exactly when no state is given, else BF16 or FP32";
    case KDA_ERR_ARG:
        return "KDA_ERR_ARG: scale and lower_bound must be finite with lower_bound <= 0, and the tensors kda.h "
               "lists under Alignment 16-byte aligned";
    case KDA_ERR_WORKSPACE:
        return "KDA_ERR_WORKSPACE: workspace is NULL, not 256-byte aligned, or smaller than kda_fwd_workspace_size";
    case KDA_ERR_ALIAS:
        return "KDA_ERR_ALIAS: out/final_state/state/workspace overlap an input or each other, or the states overlap partially";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch or runtime error occurred";
    case KDA_ERR_SCRATCH:
        return "KDA_ERR_SCRATCH: kda_fwd_noalloc needs more workspace than its built-in scratch "
               "(KDA_NOALLOC_SCRATCH_BYTES, 256 MiB) for these sizes; call kda_fwd with a caller workspace";
    default: return "unknown kda status";
    }
}

/* head dims of kda_fwd: K = V = 128 (the pages' dims) or K = V = 64 */
static bool fwd_head_dims_ok(int64_t K, int64_t V)
{
    return (K == KDA_DK && V == KDA_DV) || (K == 64 && V == 64);
}

/* 16-byte alignment of the tensors the kernels move in 16-byte pieces (NULL passes) */
static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

/* the size limits of kda.h (KDA_MAX_HEADS, 32-bit grids and offsets) */
static bool fwd_sizes_ok(int64_t B, int64_t T, int64_t H, int64_t num_seqs)
{
    if (H > KDA_MAX_HEADS) return false;
    if (num_seqs > 0 && T > INT32_MAX) return false;
    if (B > INT32_MAX || T > ((int64_t)1 << 40)) return false; /* keeps the products below in range */
    const int64_t N = num_seqs > 0 ? num_seqs : B;
    if (N > INT32_MAX || 8 * N * H > INT32_MAX) return false;
    if (num_seqs == 0 && (T + KDA_CHUNK - 1) / KDA_CHUNK > INT32_MAX / B) return false;
    return kda_max_chunks(B, T, num_seqs) * H <= INT32_MAX;
}

extern "C" size_t kda_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t num_seqs)
{
    if (B <= 0 || T <= 0 || H <= 0 || num_seqs < 0) return 0;
    if (num_seqs > 0 && B != 1) return 0;
    if (!fwd_sizes_ok(B, T, H, num_seqs)) return 0;
    const int64_t nslots = kda_max_chunks(B, T, num_seqs);
    return kda_chunk_map_bytes(num_seqs, T) + (size_t)nslots * (size_t)H * KDA_REC_BYTES +
           kda_seg_bytes(B, T, H, num_seqs);
}

extern "C" int kda_profile_enable(int on)
{
    g_prof_on = on != 0;
    if (g_prof_on) g_prof_n = 0;
    return KDA_OK;
}

extern "C" int kda_profile_read(const char **names, float *total_ms, int *counts, int cap)
{
    int nk = 0;
    for (int i = 0; i < g_prof_n; i++) {
        if (hipEventSynchronize(g_ev[i][1]) != hipSuccess) return -1;
        float t = 0.f;
        if (hipEventElapsedTime(&t, g_ev[i][0], g_ev[i][1]) != hipSuccess) return -1;
        int j = 0;
        while (j < nk && strcmp(names[j], g_prof_names[i]) != 0) j++;
        if (j == nk) {
            if (nk >= cap) continue;
            names[nk] = g_prof_names[i];
            total_ms[nk] = 0.f;
            counts[nk] = 0;
            nk++;
        }
        total_ms[j] += t;
        counts[j] += 1;
    }
    return nk;
}

extern "C" hipError_t kda_noalloc_scratch(void *stream, void **ptr);

/* kda_fwd and kda_fwd_noalloc: validation, then the launches. With noalloc the
   workspace is the library's scratch array of the stream's GPU, looked up after
   every argument check has passed (workspace / workspace_bytes are ignored). */
static int fwd_run(const void *q, const void *k, const void *v, const void *g, const void *beta,
                   float scale, void *out, const float *A_log, const float *dt_bias,
                   float lower_bound, const void *initial_state, void *final_state,
                   int state_dtype, const int32_t *cu_seqlens, int64_t num_seqs, int64_t B,
                   int64_t T, int64_t H, int64_t K, int64_t V, void *workspace,
                   size_t workspace_bytes, void *stream, bool noalloc)
{
    /* ---- validation (host only, nothing enqueued yet) ---- */
    if (!fwd_head_dims_ok(K, V)) return KDA_ERR_HEAD_DIM;
    if (B <= 0 || T <= 0 || H <= 0) return KDA_ERR_SHAPE;
    if (cu_seqlens && (B != 1 || num_seqs <= 0)) return KDA_ERR_SHAPE;
    if (!fwd_sizes_ok(B, T, H, cu_seqlens ? num_seqs : 0)) return KDA_ERR_SHAPE;
    if (!q || !k || !v || !g || !beta || !out || !A_log || !dt_bias) return KDA_ERR_NULL;
    if (state_dtype == KDA_STATE_NONE) {
        if (initial_state || final_state) return KDA_ERR_STATE_DTYPE;
    } else if (state_dtype == KDA_STATE_BF16 || state_dtype == KDA_STATE_FP32) {
        if (!initial_state && !final_state) return KDA_ERR_STATE_DTYPE;
    } else {
        return KDA_ERR_STATE_DTYPE;
    }
    if (!std::isfinite(scale) || !std::isfinite(lower_bound) || lower_bound > 0.f) return KDA_ERR_ARG;
    for (const void *p : {q, k, v, g, (const void *)out, (const void *)dt_bias, initial_state,
                          (const void *)final_state})
        if (!aligned16(p)) return KDA_ERR_ARG;
    const int64_t nseq_arg = cu_seqlens ? num_seqs : 0;
    const size_t need = kda_fwd_workspace_size(B, T, H, nseq_arg);
    if (noalloc) {
        if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
        workspace = nullptr;
        workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    } else if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) {
        return KDA_ERR_WORKSPACE;
    }

    const int64_t N = cu_seqlens ? num_seqs : B;
    const size_t act = (size_t)B * T * H * K * 2, actv = (size_t)B * T * H * V * 2;
    const size_t sbytes = (size_t)N * H * K * V * (state_dtype == KDA_STATE_FP32 ? 4 : 2);
    const Range r_out = rng(out, actv);
    const Range inputs[] = {rng(q, act), rng(k, act), rng(v, actv), rng(g, act),
                            rng(beta, (size_t)B * T * H * 2), rng(A_log, (size_t)H * 4),
                            rng(dt_bias, (size_t)H * K * 4),
                            rng(cu_seqlens, cu_seqlens ? (size_t)(num_seqs + 1) * 4 : 0),
                            rng(initial_state, initial_state ? sbytes : 0)};
    const Range r_fin = rng(final_state, final_state ? sbytes : 0);
    if (noalloc) {
        /* the scratch array is the library's own: no caller tensor can overlap it */
        if (kda_noalloc_scratch(stream, &workspace) != hipSuccess) return KDA_ERR_HIP;
    }
    const Range r_ws = noalloc ? Range{0, 0} : rng(workspace, need);
    for (const Range &in : inputs) {
        if (overlap(r_out, in)) return KDA_ERR_ALIAS;
        if (overlap(r_ws, in)) return KDA_ERR_ALIAS;
        if (&in != &inputs[8] && overlap(r_fin, in)) return KDA_ERR_ALIAS;
    }
    if (overlap(r_out, r_fin) || overlap(r_out, r_ws) || overlap(r_fin, r_ws)) return KDA_ERR_ALIAS;
    if (initial_state && final_state && initial_state != final_state && overlap(inputs[8], r_fin))
        return KDA_ERR_ALIAS;

    /* ---- launches ---- */
    hipStream_t st = (hipStream_t)stream;
    unsigned char *ws = (unsigned char *)workspace;
    int32_t *chunk_off = nullptr;
    if (cu_seqlens) {
        chunk_off = (int32_t *)ws;
        ProfScope ps("kda_chunk_map", st);
        if (kda_launch_chunk_map(cu_seqlens, num_seqs, T, chunk_off, st) != hipSuccess) return KDA_ERR_HIP;
    }
    void *records = ws + kda_chunk_map_bytes(nseq_arg, T);
    const int64_t nslots = kda_max_chunks(B, T, nseq_arg);
    /* the segment-parallel scan (few long chains) exists for K = V = 128 only */
    const int64_t segc = (K == KDA_DK && V == KDA_DV) ? kda_seg_len(B, T, H, nseq_arg) : 0;
    {
        ProfScope ps("kda_prep", st);
        if (kda_launch_prep(q, k, v, g, beta, A_log, dt_bias, scale, lower_bound, cu_seqlens, chunk_off,
                            N, T, H, nslots, K, V, records,
                            kda_scan_many_max_chunks(cu_seqlens, N, H, K, V, segc), st) != hipSuccess)
            return KDA_ERR_HIP;
    }
    {
        ProfScope ps("kda_scan", st);
        if (kda_launch_scan(records, cu_seqlens, chunk_off, N, T, H, nslots, K, V, out,
                            state_dtype == KDA_STATE_NONE ? nullptr : initial_state, final_state,
                            state_dtype == KDA_STATE_FP32 ? 1 : 0, segc,
                            (unsigned char *)records + (size_t)nslots * (size_t)H * KDA_REC_BYTES, st) != hipSuccess)
            return KDA_ERR_HIP;
    }
    return KDA_OK;
}

extern "C" int kda_fwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                       float scale, void *out, const float *A_log, const float *dt_bias,
                       float lower_bound, const void *initial_state, void *final_state,
                       int state_dtype, const int32_t *cu_seqlens, int64_t num_seqs, int64_t B,
                       int64_t T, int64_t H, int64_t K, int64_t V, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    return fwd_run(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, final_state,
                   state_dtype, cu_seqlens, num_seqs, B, T, H, K, V, workspace, workspace_bytes, stream, false);
}

extern "C" int kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g, const void *beta,
                               float scale, void *out, const float *A_log, const float *dt_bias,
                               float lower_bound, const void *initial_state, void *final_state,
                               int state_dtype, const int32_t *cu_seqlens, int64_t num_seqs, int64_t B,
                               int64_t T, int64_t H, int64_t K, int64_t V, void *stream)
{
    return fwd_run(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, final_state,
                   state_dtype, cu_seqlens, num_seqs, B, T, H, K, V, nullptr, 0, stream, true);
}

extern "C" int kda_decode(const void *q, const void *k, const void *v, const void *g, const void *beta,
                          float scale, void *out, const float *A_log, const float *dt_bias, float lower_bound,
                          void *state, int state_dtype, int64_t N, int64_t H, int64_t K, int64_t V, void *stream)
{
    /* ---- validation (host only, nothing enqueued yet) ---- */
    if (K != KDA_DK || V != KDA_DV) return KDA_ERR_HEAD_DIM;
    if (N <= 0 || H <= 0) return KDA_ERR_SHAPE;
    if (H > KDA_MAX_HEADS || N > INT32_MAX || N * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (!q || !k || !v || !g || !beta || !out || !A_log || !dt_bias || !state) return KDA_ERR_NULL;
    if (state_dtype != KDA_STATE_BF16 && state_dtype != KDA_STATE_FP32) return KDA_ERR_STATE_DTYPE;
    if (!std::isfinite(scale) || !std::isfinite(lower_bound) || lower_bound > 0.f) return KDA_ERR_ARG;
    for (const void *p : {q, k, v, g, (const void *)out, (const void *)dt_bias, (const void *)state})
        if (!aligned16(p)) return KDA_ERR_ARG;
    const size_t vec = (size_t)N * H * KDA_DK * 2;
    const size_t sbytes = (size_t)N * H * KDA_DK * KDA_DV * (state_dtype == KDA_STATE_FP32 ? 4 : 2);
    const Range r_out = rng(out, vec), r_state = rng(state, sbytes);
    const Range inputs[] = {rng(q, vec), rng(k, vec), rng(v, vec), rng(g, vec), rng(beta, (size_t)N * H * 2),
                            rng(A_log, (size_t)H * 4), rng(dt_bias, (size_t)H * KDA_DK * 4)};
    for (const Range &in : inputs)
        if (overlap(r_out, in) || overlap(r_state, in)) return KDA_ERR_ALIAS;
    if (overlap(r_out, r_state)) return KDA_ERR_ALIAS;

    hipStream_t st = (hipStream_t)stream;
    ProfScope ps("kda_decode", st);
    if (kda_launch_decode(q, k, v, g, beta, A_log, dt_bias, scale, lower_bound, state,
                          state_dtype == KDA_STATE_FP32 ? 1 : 0, out, N, H, st) != hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

/* ---- backward ---- */
extern "C" size_t kda_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t num_seqs)
{
    if (B <= 0 || T <= 0 || H <= 0 || num_seqs < 0) return 0;
    if (num_seqs > 0 && B != 1) return 0;
    if (!fwd_sizes_ok(B, T, H, num_seqs)) return 0;
    const int64_t items = kda_max_chunks(B, T, num_seqs) * H;
    return kda_chunk_map_bytes(num_seqs, T) + (size_t)items * KDA_BR_FLOATS * 4 +
           2 * (size_t)items * KDA_DK * KDA_DV * 4 + kda_bwd_part_bytes(items) +
           kda_bwd_grad_wgs(items) * (size_t)KDA_BWD_SCR_FLOATS * 4;
}

extern "C" int kda_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                       float scale, const void *dout, const float *A_log, const float *dt_bias,
                       float lower_bound, const void *initial_state, int state_dtype,
                       const float *dfinal_state, const int32_t *cu_seqlens, int64_t num_seqs, int64_t B,
                       int64_t T, int64_t H, int64_t K, int64_t V, float *dq, float *dk, float *dv, float *dg,
                       float *dbeta, float *dA_log, float *ddt_bias, float *dinitial_state, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    if (K != KDA_DK || V != KDA_DV) return KDA_ERR_HEAD_DIM;
    if (B <= 0 || T <= 0 || H <= 0) return KDA_ERR_SHAPE;
    if (cu_seqlens && (B != 1 || num_seqs <= 0)) return KDA_ERR_SHAPE;
    if (!fwd_sizes_ok(B, T, H, cu_seqlens ? num_seqs : 0)) return KDA_ERR_SHAPE;
    if (!q || !k || !v || !g || !beta || !dout || !A_log || !dt_bias) return KDA_ERR_NULL;
    if (!dq || !dk || !dv || !dg || !dbeta || !dA_log || !ddt_bias) return KDA_ERR_NULL;
    if (state_dtype == KDA_STATE_NONE) {
        if (initial_state) return KDA_ERR_STATE_DTYPE;
    } else if (state_dtype == KDA_STATE_BF16 || state_dtype == KDA_STATE_FP32) {
        if (!initial_state) return KDA_ERR_STATE_DTYPE;
    } else {
        return KDA_ERR_STATE_DTYPE;
    }
    if (!std::isfinite(scale) || !std::isfinite(lower_bound) || lower_bound > 0.f) return KDA_ERR_ARG;
    for (const void *p : {q, k, v, g, (const void *)dt_bias, initial_state, (const void *)dfinal_state,
                          (const void *)dq, (const void *)dk, (const void *)dv, (const void *)dg,
                          (const void *)dbeta, (const void *)ddt_bias, (const void *)dinitial_state})
        if (!aligned16(p)) return KDA_ERR_ARG;
    const int64_t nseq_arg = cu_seqlens ? num_seqs : 0;
    const size_t need = kda_bwd_workspace_size(B, T, H, nseq_arg);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) return KDA_ERR_WORKSPACE;

    const int64_t N = cu_seqlens ? num_seqs : B;
    const size_t act = (size_t)B * T * H * KDA_DK * 2, g32 = 2 * act, fstate = (size_t)N * H * KDA_DK * KDA_DV * 4;
    const size_t sbytes = (size_t)N * H * KDA_DK * KDA_DV * (state_dtype == KDA_STATE_FP32 ? 4 : 2);
    const Range inputs[] = {rng(q, act), rng(k, act), rng(v, act), rng(g, act), rng(beta, (size_t)B * T * H * 2),
                            rng(dout, act), rng(A_log, (size_t)H * 4), rng(dt_bias, (size_t)H * KDA_DK * 4),
                            rng(cu_seqlens, cu_seqlens ? (size_t)(num_seqs + 1) * 4 : 0),
                            rng(initial_state, initial_state ? sbytes : 0),
                            rng(dfinal_state, dfinal_state ? fstate : 0)};
    const Range outputs[] = {rng(dq, g32), rng(dk, g32), rng(dv, g32), rng(dg, g32),
                             rng(dbeta, (size_t)B * T * H * 4), rng(dA_log, (size_t)H * 4),
                             rng(ddt_bias, (size_t)H * KDA_DK * 4),
                             rng(dinitial_state, dinitial_state ? fstate : 0), rng(workspace, need)};
    for (const Range &o : outputs) {
        for (const Range &in : inputs)
            if (overlap(o, in)) return KDA_ERR_ALIAS;
        for (const Range &o2 : outputs)
            if (&o2 != &o && overlap(o, o2)) return KDA_ERR_ALIAS;
    }

    hipStream_t st = (hipStream_t)stream;
    unsigned char *ws = (unsigned char *)workspace;
    int32_t *chunk_off = nullptr;
    if (cu_seqlens) {
        chunk_off = (int32_t *)ws;
        ProfScope ps("kda_chunk_map", st);
        if (kda_launch_chunk_map(cu_seqlens, num_seqs, T, chunk_off, st) != hipSuccess) return KDA_ERR_HIP;
    }
    unsigned char *area = ws + kda_chunk_map_bytes(nseq_arg, T);
    const int64_t nslots = kda_max_chunks(B, T, nseq_arg);
    static const char *names[4] = {"kda_bwd_chunk", "kda_bwd_scan", "kda_bwd_grad", "kda_bwd_reduce"};
    for (int stage = 0; stage < 4; stage++) {
        ProfScope ps(names[stage], st);
        if (kda_launch_bwd(stage, q, k, v, g, beta, dout, A_log, dt_bias, scale, lower_bound, initial_state,
                           state_dtype == KDA_STATE_FP32 ? 1 : 0, dfinal_state, cu_seqlens, chunk_off, N, T, H,
                           nslots, area, dq, dk, dv, dg, dbeta, dA_log, ddt_bias, dinitial_state,
                           st) != hipSuccess)
            return KDA_ERR_HIP;
    }
    return KDA_OK;
}
