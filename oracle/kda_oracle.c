/*
 * kda_oracle.c -- fp64 CPU reference for the Kimi Delta Attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU leg do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (plain definition, one token at a time, in double):
 *   The pages (FlashKDA: "Kernel API and Constraints" on the trend.ondo.sh
 *   page; "Core Kernel API / flash_kda.fwd" on the ccm-staging page) name the
 *   call fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
 *   initial_state, final_state, cu_seqlens), fix K = V = 128, bf16 inputs,
 *   cu_seqlens with B = 1 and states of matching dtype, and describe the kernel
 *   as handling the recurrent state updates of delta attention. They print no
 *   formula, so this oracle takes the gated delta rule with per-channel decay:
 *
 *     q^ = q / sqrt(sum q^2 + 1e-6),  k^ = k / sqrt(sum k^2 + 1e-6)
 *     x_c  = g_c + dt_bias[h, c]
 *     la_c = max(-exp(A_log[h]) * softplus(x_c), lower_bound),  alpha_c = exp(la_c)
 *     S_t  = (I - beta_t k^ k^T) Diag(alpha) S_{t-1} + beta_t k^ v_t^T
 *     o_t  = scale * S_t^T q^
 *
 *   S is K x V (rows indexed by the key channel). The state entering a
 *   sequence is initial_state (or zero); final_state receives S after its last
 *   token. The product (I - b k k^T) Diag(alpha) S + b k v^T is evaluated as
 *   decay (S <- Diag(alpha) S), erase-and-write (S <- S + k (b (v - S^T k))^T),
 *   then read (o = scale S^T q), which is the same expression expanded.
 *
 * Layouts: q, k, g [B, T, H, K]; v, out [B, T, H, V]; beta [B, T, H];
 * A_log [H]; dt_bias [H, K]; states [N, H, K, V]. With cu_seqlens (B = 1) the
 * N sequences are rows [cu[n], cu[n+1]) of the packed token axis; otherwise
 * N = B and sequence n is batch row n.
 *
 * Work split: OpenMP over (sequence, head, block of 32 value columns). The
 * columns of S evolve independently given k^, alpha and beta, so each task runs
 * the unmodified per-token recurrence on its own columns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F64 = 0, ORC_BF16 = 1, ORC_F32 = 2 };

static double orc_load(const void *p, int64_t i, int dt)
{
    if (dt == ORC_F64)
        return ((const double *)p)[i];
    if (dt == ORC_F32)
        return (double)((const float *)p)[i];
    /* bf16 bit pattern: the upper 16 bits of an IEEE binary32 */
    uint32_t u = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* softplus(x) = ln(1 + e^x), written in a form that does not overflow */
static double orc_softplus(double x)
{
    return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

#define ORC_VBLK 32

/*
 * Returns 0 on success, -1 on an argument error (sizes, B != 1 with
 * cu_seqlens, inconsistent cu_seqlens), -2 on allocation failure.
 */
int kda_oracle_fwd(const void *q, const void *k, const void *v, const void *g,
                   const void *beta, int in_dtype, double scale, double *out,
                   const double *A_log, const double *dt_bias,
                   double lower_bound, const void *initial_state,
                   int state_dtype, double *final_state,
                   const int32_t *cu_seqlens, int64_t num_seqs, int64_t B,
                   int64_t T, int64_t H, int64_t K, int64_t V, int nthreads)
{
    if (B <= 0 || T < 0 || H <= 0 || K <= 0 || V <= 0)
        return -1;
    int64_t N = B;
    if (cu_seqlens) {
        if (B != 1 || num_seqs <= 0 || cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T)
            return -1;
        for (int64_t n = 0; n < num_seqs; n++)
            if (cu_seqlens[n + 1] < cu_seqlens[n])
                return -1;
        N = num_seqs;
    }
    const int64_t nvb = (V + ORC_VBLK - 1) / ORC_VBLK;
    const int64_t ntask = N * H * nvb;
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t task = 0; task < ntask; task++) {
        const int64_t n = task / (H * nvb);
        const int64_t h = (task / nvb) % H;
        const int64_t v0 = (task % nvb) * ORC_VBLK;
        const int64_t vb = (V - v0) < ORC_VBLK ? (V - v0) : ORC_VBLK;
        double *S = (double *)calloc((size_t)(K * vb), sizeof(double));
        double *qn = (double *)malloc((size_t)K * sizeof(double));
        double *kn = (double *)malloc((size_t)K * sizeof(double));
        double *alpha = (double *)malloc((size_t)K * sizeof(double));
        double *e = (double *)malloc((size_t)vb * sizeof(double));
        if (!S || !qn || !kn || !alpha || !e) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = -2;
            free(S); free(qn); free(kn); free(alpha); free(e);
            continue;
        }
        /* the sequence's token rows on the flattened [B*T] axis */
        int64_t bos, eos;
        if (cu_seqlens) {
            bos = cu_seqlens[n];
            eos = cu_seqlens[n + 1];
        } else {
            bos = n * T;
            eos = n * T + T;
        }
        if (initial_state)
            for (int64_t c = 0; c < K; c++)
                for (int64_t j = 0; j < vb; j++)
                    S[c * vb + j] = orc_load(initial_state, ((n * H + h) * K + c) * V + v0 + j, state_dtype);
        const double decay_rate = exp(A_log[h]);
        for (int64_t t = bos; t < eos; t++) {
            const int64_t row = t * H + h; /* (token, head) row index */
            /* L2 normalisation of q and k */
            double sq = 0.0, sk = 0.0;
            for (int64_t c = 0; c < K; c++) {
                qn[c] = orc_load(q, row * K + c, in_dtype);
                kn[c] = orc_load(k, row * K + c, in_dtype);
                sq += qn[c] * qn[c];
                sk += kn[c] * kn[c];
            }
            const double iq = 1.0 / sqrt(sq + 1e-6), ik = 1.0 / sqrt(sk + 1e-6);
            for (int64_t c = 0; c < K; c++) {
                qn[c] *= iq;
                kn[c] *= ik;
            }
            /* per-channel gate */
            for (int64_t c = 0; c < K; c++) {
                const double x = orc_load(g, row * K + c, in_dtype) + dt_bias[h * K + c];
                const double la = fmax(-decay_rate * orc_softplus(x), lower_bound);
                alpha[c] = exp(la);
            }
            const double b = orc_load(beta, row, in_dtype);
            /* decay: S <- Diag(alpha) S */
            for (int64_t c = 0; c < K; c++)
                for (int64_t j = 0; j < vb; j++)
                    S[c * vb + j] *= alpha[c];
            /* erase and write: S <- S + k^ (b (v - S^T k^))^T */
            for (int64_t j = 0; j < vb; j++) {
                double s = 0.0;
                for (int64_t c = 0; c < K; c++)
                    s += S[c * vb + j] * kn[c];
                e[j] = b * (orc_load(v, row * V + v0 + j, in_dtype) - s);
            }
            for (int64_t c = 0; c < K; c++)
                for (int64_t j = 0; j < vb; j++)
                    S[c * vb + j] += kn[c] * e[j];
            /* read: o = scale S^T q^ */
            for (int64_t j = 0; j < vb; j++) {
                double s = 0.0;
                for (int64_t c = 0; c < K; c++)
                    s += S[c * vb + j] * qn[c];
                out[row * V + v0 + j] = scale * s;
            }
        }
        if (final_state)
            for (int64_t c = 0; c < K; c++)
                for (int64_t j = 0; j < vb; j++)
                    final_state[((n * H + h) * K + c) * V + v0 + j] = S[c * vb + j];
        free(S); free(qn); free(kn); free(alpha); free(e);
    }
    return err;
}

/* Threads OpenMP would use by default (for reporting). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
