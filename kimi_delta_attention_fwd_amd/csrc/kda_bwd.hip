/*
 * kda_bwd.hip -- gfx950 kernels of the backward of the chunked Kimi Delta
 * Attention forward: gradients of q, k, v, g, beta, A_log, dt_bias and the
 * initial state for L = <dout, out> + <dfinal, final_state>.
 *
 * The FlashKDA pages show only the forward ("Core Kernel API / flash_kda.fwd",
 * ccm-staging page); these are the derivatives of the forward recurrence
 * described in kda.h, taken through its chunked form (kda_internal.h). All
 * arithmetic is fp32 on the vector ALUs:
 *
 *   kda_bwd_chunk_kernel  one workgroup per (chunk, head): q^, k^, log a, G, A, P,
 *                         T = (I + A)^-1 (forward substitution), W, U, Q', K~,
 *                         e^{G_L}, stored as fp32 per-chunk areas.
 *   kda_bwd_scan_kernel   one workgroup per (sequence, head, 16 value columns);
 *                         value columns are independent in both directions:
 *                         forward  S <- diag(e^{G_L}) S + K~^T (U - W S), storing S
 *                                  at every chunk start;
 *                         reverse  dS <- diag(e^{G_L}) dS - W^T (K~ dS) + Q'^T dout,
 *                                  storing dS at every chunk end; the last one is
 *                                  the initial-state gradient.
 *   kda_bwd_grad_kernel   per (chunk, head), given S and dS at its ends:
 *                         dQ' = dout S^T, dW = -dD S^T - P^T dQ', dK~ = D dS^T,
 *                         dP = dout U^T - dQ' W^T, dU = P^T dout + dD (dD = K~ dS,
 *                         D = U - W S), then through W = T X_W, U = T X_U,
 *                         dA = -T^T dT T^T, the pairwise decay factors
 *                         e^{G_i - G_j} (<= 1, formed per element), the in-chunk
 *                         cumsum, the gate and the L2 norms.
 *   kda_bwd_reduce_kernel sums the per-chunk gate partials of each head into
 *                         d A_log and d dt_bias (fixed order: deterministic).
 */
#include "kda.h"
#include "kda_device.h"

namespace {

constexpr int NT = 256;   /* threads of every backward workgroup */
constexpr int LDK = 129;  /* padded LDS row stride of [64][128] arrays */
constexpr int LDT = 65;   /* padded LDS row stride of [64][64] arrays  */

__device__ __forceinline__ float softplus_f(float x)
{
    return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid_f(float x)
{
    return 1.f / (1.f + expf(-x));
}

/* chunks and first chunk slot of sequence seq, and its first token row */
__device__ __forceinline__ void bwd_seq(int64_t seq, const int32_t *cu, const int32_t *chunk_off, int64_t T,
                                        int64_t &nchunk, int64_t &slot0, int64_t &row0, int64_t &len)
{
    if (cu == nullptr) {
        nchunk = (T + KDA_CHUNK - 1) / KDA_CHUNK;
        slot0 = seq * nchunk;
        row0 = seq * T;
        len = T;
    } else {
        len = (int64_t)cu[seq + 1] - cu[seq];
        nchunk = (len + KDA_CHUNK - 1) / KDA_CHUNK;
        slot0 = chunk_off[seq];
        row0 = cu[seq];
    }
}

/* C[i][j] = (acc ? C[i][j] : 0) + alpha * sum_k a(i, k) b(k, j) for i < M, j < N,
 * with a(i, k) = TA ? A[k][i] : A[i][k] and b(k, j) = TB ? B[j][k] : B[k][j]
 * (row strides lda, ldb, ldc). N is a power of two. Callers separate products
 * that share an output or read one another's output with a barrier. */
template <bool TA, bool TB>
__device__ __forceinline__ void wg_gemm(float *C, int ldc, const float *A, int lda, const float *B, int ldb,
                                        int M, int N, int Kd, float alpha, bool acc)
{
    for (int e = threadIdx.x; e < M * N; e += NT) {
        const int i = e / N, j = e - i * N;
        float s = 0.f;
        for (int kk = 0; kk < Kd; kk++) {
            const float a = TA ? A[kk * lda + i] : A[i * lda + kk];
            const float b = TB ? B[j * ldb + kk] : B[kk * ldb + j];
            s = fmaf(a, b, s);
        }
        C[i * ldc + j] = acc ? C[i * ldc + j] + alpha * s : alpha * s;
    }
}

} // namespace

/* ------------------------------------------------------------------------- */
/* chunk quantities, one workgroup per (chunk slot, head), grid H * nslots     */
/* ------------------------------------------------------------------------- */
extern "C" __global__ void __launch_bounds__(NT)
kda_bwd_chunk_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                     const uint16_t *__restrict__ v, const uint16_t *__restrict__ g,
                     const uint16_t *__restrict__ beta, const float *__restrict__ A_log,
                     const float *__restrict__ dt_bias, float scale, float lower_bound,
                     const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, int64_t nseq,
                     int64_t T, int H, int64_t nslots, float *__restrict__ brec)
{
    __shared__ float sQ[KDA_CHUNK * LDK], sK[KDA_CHUNK * LDK], sG[KDA_CHUNK * LDK];
    __shared__ float sA[KDA_CHUNK * LDT], sT[KDA_CHUNK * LDT], sP[KDA_CHUNK * LDT];
    __shared__ float sB[KDA_CHUNK];

    const int64_t item = blockIdx.x;
    const int h = (int)(item / nslots);
    const int64_t slot = item - (int64_t)h * nslots;
    int64_t t0, seq;
    int L;
    if (!locate_chunk(slot, cu, chunk_off, nseq, T, t0, L, seq)) return;
    float *R = brec + item * KDA_BR_FLOATS;
    const int t = threadIdx.x;

    /* 1. norms and gate: thread t covers row t / 4, channels 32 (t % 4) + [0, 32) */
    {
        const int i = t >> 2, c0 = (t & 3) * 32;
        const float rate = expf(A_log[h]);
        if (i < L) {
            const int64_t base = ((t0 + i) * H + h) * KDA_DK + c0;
            float qx[32], kx[32];
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int c = 0; c < 32; c++) {
                qx[c] = bf2f(q[base + c]);
                kx[c] = bf2f(k[base + c]);
                sq = fmaf(qx[c], qx[c], sq);
                sk = fmaf(kx[c], kx[c], sk);
            }
            sq += __shfl_xor(sq, 1);
            sq += __shfl_xor(sq, 2);
            sk += __shfl_xor(sk, 1);
            sk += __shfl_xor(sk, 2);
            const float nq = sqrtf(sq + 1e-6f), nk = sqrtf(sk + 1e-6f);
#pragma unroll
            for (int c = 0; c < 32; c++) {
                sQ[i * LDK + c0 + c] = qx[c] / nq;
                sK[i * LDK + c0 + c] = kx[c] / nk;
                const float x = bf2f(g[base + c]) + dt_bias[h * KDA_DK + c0 + c];
                sG[i * LDK + c0 + c] = fmaxf(-rate * softplus_f(x), lower_bound);
            }
            if ((t & 3) == 0) {
                const float b = bf2f(beta[(t0 + i) * H + h]);
                sB[i] = b;
                R[KDA_BR_BETA + i] = b;
                R[KDA_BR_NQ + i] = nq;
                R[KDA_BR_NK + i] = nk;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 32; c++) {
                sQ[i * LDK + c0 + c] = 0.f;
                sK[i * LDK + c0 + c] = 0.f;
                sG[i * LDK + c0 + c] = 0.f;
            }
            if ((t & 3) == 0) {
                sB[i] = 0.f;
                R[KDA_BR_BETA + i] = 0.f;
                R[KDA_BR_NQ + i] = 1.f;
                R[KDA_BR_NK + i] = 1.f;
            }
        }
    }
    for (int e = t; e < KDA_CHUNK * KDA_CHUNK; e += NT) {
        const int i = e >> 6, j = e & 63;
        sA[i * LDT + j] = 0.f;
        sP[i * LDT + j] = 0.f;
        sT[i * LDT + j] = 0.f;
    }
    __syncthreads();

    /* 2. in-chunk inclusive cumsum of log a per channel */
    if (t < KDA_DK) {
        float acc = 0.f;
        for (int i = 0; i < KDA_CHUNK; i++) {
            acc += sG[i * LDK + t];
            sG[i * LDK + t] = acc;
        }
    }
    __syncthreads();

    /* 3. A (j < i) and P (j <= i) over the 2080 lower-triangle pairs */
    for (int e = t; e < KDA_CHUNK * (KDA_CHUNK + 1) / 2; e += NT) {
        int i = (int)((sqrtf(8.f * (float)e + 1.f) - 1.f) * 0.5f);
        while (i * (i + 1) / 2 > e) i--;
        while ((i + 1) * (i + 2) / 2 <= e) i++;
        const int j = e - i * (i + 1) / 2;
        float a = 0.f, p = 0.f;
        if (i < L) {
            for (int c = 0; c < KDA_DK; c++) {
                const float E = expf(sG[i * LDK + c] - sG[j * LDK + c]);
                const float kj = sK[j * LDK + c] * E;
                a = fmaf(sK[i * LDK + c], kj, a);
                p = fmaf(sQ[i * LDK + c], kj, p);
            }
        }
        sA[i * LDT + j] = j < i ? sB[i] * a : 0.f;
        sP[i * LDT + j] = scale * p;
    }
    __syncthreads();

    /* 4. T = (I + A)^-1, row by row: T[r][j] = delta_rj - sum_{j <= m < r} A[r][m] T[m][j] */
    for (int r = 0; r < KDA_CHUNK; r++) {
        if (t < KDA_CHUNK) {
            const int j = t;
            float s = 0.f;
            if (j == r) {
                s = 1.f;
            } else if (j < r) {
                for (int m = j; m < r; m++) s = fmaf(-sA[r * LDT + m], sT[m * LDT + j], s);
            }
            sT[r * LDT + j] = s;
        }
        __syncthreads();
    }

    /* 5. store T, P, q^, k^, G */
    for (int e = t; e < KDA_CHUNK * KDA_CHUNK; e += NT) {
        const int i = e >> 6, j = e & 63;
        R[KDA_BR_T + e] = sT[i * LDT + j];
        R[KDA_BR_P + e] = sP[i * LDT + j];
    }
    for (int e = t; e < KDA_CHUNK * KDA_DK; e += NT) {
        const int i = e >> 7, c = e & 127;
        R[KDA_BR_QN + e] = sQ[i * LDK + c];
        R[KDA_BR_KN + e] = sK[i * LDK + c];
        R[KDA_BR_G + e] = sG[i * LDK + c];
    }

    /* 6. W = T X_W (X_W = beta k^ e^G) in threads 0-127, U = T X_U (X_U = beta v) in
     *    128-255, one channel column each; then Q' = scale q^ e^G - P W (first half)
     *    and K~, e^{G_L} (second half) */
    const int c = t & 127, half = t >> 7;
    float acc[KDA_CHUNK];
#pragma unroll
    for (int i = 0; i < KDA_CHUNK; i++) acc[i] = 0.f;
    for (int m = 0; m < L; m++) {
        const float x = half == 0 ? sB[m] * sK[m * LDK + c] * expf(sG[m * LDK + c])
                                  : sB[m] * bf2f(v[((t0 + m) * H + h) * KDA_DV + c]);
#pragma unroll
        for (int i = 0; i < KDA_CHUNK; i++) acc[i] = fmaf(sT[i * LDT + m], x, acc[i]);
    }
    float *dst = R + (half == 0 ? KDA_BR_W : KDA_BR_U);
#pragma unroll
    for (int i = 0; i < KDA_CHUNK; i++) dst[i * KDA_DK + c] = acc[i];
    if (half == 0) {
        /* acc holds column c of W: Q'[i][c] = scale q^ e^G - sum_m P[i][m] W[m][c] */
        float qp[KDA_CHUNK];
#pragma unroll
        for (int i = 0; i < KDA_CHUNK; i++) qp[i] = scale * sQ[i * LDK + c] * expf(sG[i * LDK + c]);
        for (int m = 0; m < L; m++) {
            const float wm = R[KDA_BR_W + m * KDA_DK + c];
#pragma unroll
            for (int i = 0; i < KDA_CHUNK; i++) qp[i] = fmaf(-sP[i * LDT + m], wm, qp[i]);
        }
#pragma unroll
        for (int i = 0; i < KDA_CHUNK; i++) R[KDA_BR_QP + i * KDA_DK + c] = qp[i];
    } else {
        const float gl = sG[(L - 1) * LDK + c];
#pragma unroll
        for (int i = 0; i < KDA_CHUNK; i++)
            R[KDA_BR_KT + i * KDA_DK + c] = sK[i * LDK + c] * expf(gl - sG[i * LDK + c]);
        R[KDA_BR_GL + c] = expf(gl);
    }
}

/* ------------------------------------------------------------------------- */
/* state checkpoints and state gradients: one workgroup per (sequence, head,  */
/* 16 value columns), grid N * H * 8. Thread t owns column 16 tile + t % 16   */
/* and key rows t / 16 + 16 m (m < 8) of S and dS.                            */
/* ------------------------------------------------------------------------- */
extern "C" __global__ void __launch_bounds__(NT)
kda_bwd_scan_kernel(const float *__restrict__ brec, const int32_t *__restrict__ cu,
                    const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H, int64_t nslots,
                    const void *__restrict__ init, int init_fp32, const float *__restrict__ dfinal,
                    const uint16_t *__restrict__ dout, float *__restrict__ ckpt, float *__restrict__ dse,
                    float *__restrict__ dinit)
{
    __shared__ float sS[KDA_DK * 16], sD[KDA_CHUNK * 16], sO[KDA_CHUNK * 16];
    const int tile = blockIdx.x & 7;
    const int64_t chain = blockIdx.x >> 3;
    const int64_t seq = chain / H;
    const int h = (int)(chain - seq * H);
    if (seq >= nseq) return;
    int64_t nchunk, slot0, row0, len;
    bwd_seq(seq, cu, chunk_off, T, nchunk, slot0, row0, len);
    const int t = threadIdx.x, j = t & 15, rb = t >> 4, col = tile * 16 + j;
    const int64_t sbase = (seq * H + h) * (int64_t)(KDA_DK * KDA_DV);

    float S[8];
#pragma unroll
    for (int m = 0; m < 8; m++) {
        const int64_t o = sbase + (int64_t)(rb + 16 * m) * KDA_DV + col;
        S[m] = init == nullptr ? 0.f
             : init_fp32 ? ((const float *)init)[o] : bf2f(((const uint16_t *)init)[o]);
    }
    for (int64_t c = 0; c < nchunk; c++) {
        const int64_t item = (int64_t)h * nslots + slot0 + c;
        const float *R = brec + item * KDA_BR_FLOATS;
        float *ck = ckpt + item * (int64_t)(KDA_DK * KDA_DV);
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const int r = rb + 16 * m;
            ck[r * KDA_DV + col] = S[m];
            sS[r * 16 + j] = S[m];
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const int i = rb + 16 * m;
            float s = R[KDA_BR_U + i * KDA_DV + col];
            for (int r = 0; r < KDA_DK; r++) s = fmaf(-R[KDA_BR_W + i * KDA_DK + r], sS[r * 16 + j], s);
            sD[i * 16 + j] = s;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const int r = rb + 16 * m;
            float s = R[KDA_BR_GL + r] * S[m];
            for (int i = 0; i < KDA_CHUNK; i++) s = fmaf(R[KDA_BR_KT + i * KDA_DK + r], sD[i * 16 + j], s);
            S[m] = s;
        }
        __syncthreads();
    }

    float dS[8];
#pragma unroll
    for (int m = 0; m < 8; m++)
        dS[m] = dfinal == nullptr ? 0.f : dfinal[sbase + (int64_t)(rb + 16 * m) * KDA_DV + col];
    for (int64_t c = nchunk - 1; c >= 0; c--) {
        const int64_t item = (int64_t)h * nslots + slot0 + c;
        const float *R = brec + item * KDA_BR_FLOATS;
        float *dk = dse + item * (int64_t)(KDA_DK * KDA_DV);
        const int64_t rem = len - c * KDA_CHUNK;
        const int L = (int)(rem < KDA_CHUNK ? rem : KDA_CHUNK);
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const int r = rb + 16 * m;
            dk[r * KDA_DV + col] = dS[m];
            sS[r * 16 + j] = dS[m];
        }
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const int i = rb + 16 * m;
            sO[i * 16 + j] = i < L ? bf2f(dout[((row0 + c * KDA_CHUNK + i) * H + h) * KDA_DV + col]) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const int i = rb + 16 * m;
            float s = 0.f;
            for (int r = 0; r < KDA_DK; r++) s = fmaf(R[KDA_BR_KT + i * KDA_DK + r], sS[r * 16 + j], s);
            sD[i * 16 + j] = s;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const int r = rb + 16 * m;
            float s = R[KDA_BR_GL + r] * dS[m];
            for (int i = 0; i < L; i++) {
                s = fmaf(-R[KDA_BR_W + i * KDA_DK + r], sD[i * 16 + j], s);
                s = fmaf(R[KDA_BR_QP + i * KDA_DK + r], sO[i * 16 + j], s);
            }
            dS[m] = s;
        }
        __syncthreads();
    }
    if (dinit != nullptr) {
#pragma unroll
        for (int m = 0; m < 8; m++) dinit[sbase + (int64_t)(rb + 16 * m) * KDA_DV + col] = dS[m];
    }
}

/* ------------------------------------------------------------------------- */
/* gradients of one (chunk, head) per loop trip; grid <= KDA_BWD_GRAD_WGS,     */
/* each workgroup with its own KDA_BWD_SCR_FLOATS of scratch                   */
/* ------------------------------------------------------------------------- */
extern "C" __global__ void __launch_bounds__(NT)
kda_bwd_grad_kernel(const uint16_t *__restrict__ v, const uint16_t *__restrict__ g,
                    const uint16_t *__restrict__ dout, const float *__restrict__ A_log,
                    const float *__restrict__ dt_bias, float scale, float lower_bound,
                    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, int64_t nseq,
                    int64_t T, int H, int64_t nslots, const float *__restrict__ brec,
                    const float *__restrict__ ckpt, const float *__restrict__ dse, float *__restrict__ part,
                    float *__restrict__ scratch, float *__restrict__ dq, float *__restrict__ dk,
                    float *__restrict__ dv, float *__restrict__ dg, float *__restrict__ dbeta)
{
    __shared__ float sG[KDA_CHUNK * LDK], sK[KDA_CHUNK * LDK];
    __shared__ float sdA[KDA_CHUNK * LDT], sdP[KDA_CHUNK * LDT];
    __shared__ float sBeta[KDA_CHUNK], sGL[KDA_DK], sGL2[KDA_DK], sRed[KDA_DK];

    float *scr = scratch + (size_t)blockIdx.x * KDA_BWD_SCR_FLOATS;
    float *D = scr, *dD = scr + 8192, *dQp = scr + 2 * 8192, *dW = scr + 3 * 8192, *dKt = scr + 4 * 8192;
    float *dU = scr + 5 * 8192, *XW = scr + 6 * 8192, *XU = scr + 7 * 8192, *dXW = scr + 8 * 8192;
    float *dXU = scr + 9 * 8192, *dqn = scr + 10 * 8192, *dkn = scr + 11 * 8192, *dG = scr + 12 * 8192;
    float *DO = scr + 13 * 8192;
    float *dP = scr + 14 * 8192, *dT = dP + 4096, *X1 = dP + 2 * 4096;

    const int t = threadIdx.x, c = t & 127, half = t >> 7;
    const int64_t nitems = (int64_t)H * nslots;
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int h = (int)(item / nslots);
        const int64_t slot = item - (int64_t)h * nslots;
        int64_t t0, seq;
        int L;
        if (!locate_chunk(slot, cu, chunk_off, nseq, T, t0, L, seq)) continue;
        const float *R = brec + item * KDA_BR_FLOATS;
        const float *S0 = ckpt + item * (int64_t)(KDA_DK * KDA_DV);
        const float *dS = dse + item * (int64_t)(KDA_DK * KDA_DV);
        const float rate = expf(A_log[h]);

        /* s0: dout, X_W, X_U, D <- U; LDS copies of G and k^ */
        for (int e = t; e < KDA_CHUNK * KDA_DK; e += NT) {
            const int i = e >> 7, cc = e & 127;
            const float b = R[KDA_BR_BETA + i];
            const bool ok = i < L;
            const int64_t row = ((t0 + i) * H + h) * KDA_DV + cc;
            DO[e] = ok ? bf2f(dout[row]) : 0.f;
            XU[e] = ok ? b * bf2f(v[row]) : 0.f;
            const float gg = R[KDA_BR_G + e], kk = R[KDA_BR_KN + e];
            XW[e] = b * kk * expf(gg);
            D[e] = R[KDA_BR_U + e];
            sG[i * LDK + cc] = gg;
            sK[i * LDK + cc] = kk;
        }
        if (t < KDA_CHUNK) sBeta[t] = R[KDA_BR_BETA + t];
        __syncthreads();

        /* s1: D = U - W S, dD = K~ dS, dQ' = dout S^T */
        wg_gemm<false, false>(D, KDA_DV, R + KDA_BR_W, KDA_DK, S0, KDA_DV, KDA_CHUNK, KDA_DV, KDA_DK, -1.f, true);
        wg_gemm<false, false>(dD, KDA_DV, R + KDA_BR_KT, KDA_DK, dS, KDA_DV, KDA_CHUNK, KDA_DV, KDA_DK, 1.f, false);
        wg_gemm<false, true>(dQp, KDA_DK, DO, KDA_DV, S0, KDA_DV, KDA_CHUNK, KDA_DK, KDA_DV, 1.f, false);
        __syncthreads();

        /* s2: dW = -dD S^T, dK~ = D dS^T, dP = dout U^T, dU = P^T dout */
        wg_gemm<false, true>(dW, KDA_DK, dD, KDA_DV, S0, KDA_DV, KDA_CHUNK, KDA_DK, KDA_DV, -1.f, false);
        wg_gemm<false, true>(dKt, KDA_DK, D, KDA_DV, dS, KDA_DV, KDA_CHUNK, KDA_DK, KDA_DV, 1.f, false);
        wg_gemm<false, true>(dP, KDA_CHUNK, DO, KDA_DV, R + KDA_BR_U, KDA_DV, KDA_CHUNK, KDA_CHUNK, KDA_DV, 1.f, false);
        wg_gemm<true, false>(dU, KDA_DV, R + KDA_BR_P, KDA_CHUNK, DO, KDA_DV, KDA_CHUNK, KDA_DV, KDA_CHUNK, 1.f, false);
        __syncthreads();

        /* s3: Q' = scale q^ e^G - P W: dP -= dQ' W^T, dW -= P^T dQ'; dU += dD */
        wg_gemm<false, true>(dP, KDA_CHUNK, dQp, KDA_DK, R + KDA_BR_W, KDA_DK, KDA_CHUNK, KDA_CHUNK, KDA_DK, -1.f, true);
        wg_gemm<true, false>(dW, KDA_DK, R + KDA_BR_P, KDA_CHUNK, dQp, KDA_DK, KDA_CHUNK, KDA_DK, KDA_CHUNK, -1.f, true);
        for (int e = t; e < KDA_CHUNK * KDA_DV; e += NT) dU[e] += dD[e];
        __syncthreads();

        /* s4: dT = dW X_W^T (+ dU X_U^T below), dX_W = T^T dW, dX_U = T^T dU; masked dP to LDS */
        wg_gemm<false, true>(dT, KDA_CHUNK, dW, KDA_DK, XW, KDA_DK, KDA_CHUNK, KDA_CHUNK, KDA_DK, 1.f, false);
        wg_gemm<true, false>(dXW, KDA_DK, R + KDA_BR_T, KDA_CHUNK, dW, KDA_DK, KDA_CHUNK, KDA_DK, KDA_CHUNK, 1.f, false);
        wg_gemm<true, false>(dXU, KDA_DV, R + KDA_BR_T, KDA_CHUNK, dU, KDA_DV, KDA_CHUNK, KDA_DV, KDA_CHUNK, 1.f, false);
        for (int e = t; e < KDA_CHUNK * KDA_CHUNK; e += NT) {
            const int i = e >> 6, jj = e & 63;
            sdP[i * LDT + jj] = jj <= i ? dP[e] : 0.f;
        }
        __syncthreads();
        wg_gemm<false, true>(dT, KDA_CHUNK, dU, KDA_DV, XU, KDA_DV, KDA_CHUNK, KDA_CHUNK, KDA_DV, 1.f, true);
        __syncthreads();

        /* s5: X1 = T^T dT */
        wg_gemm<true, false>(X1, KDA_CHUNK, R + KDA_BR_T, KDA_CHUNK, dT, KDA_CHUNK, KDA_CHUNK, KDA_CHUNK, KDA_CHUNK, 1.f, false);
        __syncthreads();

        /* s6: dA = -X1 T^T on the strict lower triangle */
        for (int e = t; e < KDA_CHUNK * KDA_CHUNK; e += NT) {
            const int i = e >> 6, jj = e & 63;
            float s = 0.f;
            if (jj < i)
                for (int n = 0; n < KDA_CHUNK; n++) s = fmaf(X1[i * KDA_CHUNK + n], R[KDA_BR_T + jj * KDA_CHUNK + n], s);
            sdA[i * LDT + jj] = -s;
        }
        /* s6b: d G_L from the carried decay: e^{G_L} sum_j dS[c][j] S[c][j] */
        if (half == 0) {
            float s = 0.f;
            for (int jj = 0; jj < KDA_DV; jj++) s = fmaf(dS[c * KDA_DV + jj], S0[c * KDA_DV + jj], s);
            sGL[c] = R[KDA_BR_GL + c] * s;
        }
        __syncthreads();

        /* s7: per-element terms (Q', K~, X_W, X_U); thread (c, half) takes rows of parity half */
        {
            const float gl = sG[(L - 1) * LDK + c];
            float glacc = 0.f;
            for (int i = half; i < L; i += 2) {
                const int e = i * KDA_DK + c;
                const float gam = expf(sG[i * LDK + c]), kn = sK[i * LDK + c], qn = R[KDA_BR_QN + e];
                const float b = sBeta[i];
                float aq = scale * dQp[e] * gam;
                float ag = scale * qn * gam * dQp[e];
                const float kt = R[KDA_BR_KT + e], dkt = dKt[e];
                float ak = dkt * expf(gl - sG[i * LDK + c]);
                ag -= dkt * kt;
                glacc = fmaf(dkt, kt, glacc);
                const float dxw = dXW[e], dxu = dXU[e];
                ak = fmaf(b * gam, dxw, ak);
                ag = fmaf(b * kn * gam, dxw, ag);
                const float vv = bf2f(v[((t0 + i) * H + h) * KDA_DV + c]);
                dv[((t0 + i) * H + h) * KDA_DV + c] = b * dxu;
                XU[e] = kn * gam * dxw + vv * dxu;   /* d beta partial of (i, c); X_U is no longer needed */
                dqn[e] = aq;
                dkn[e] = ak;
                dG[e] = ag;
            }
            if (half == 1) sGL2[c] = glacc;
            __syncthreads();
            if (half == 0) sGL[c] += glacc + sGL2[c];
        }
        __syncthreads();

        /* s8: pairwise factors, row side: rows i of parity half, j <= i */
        for (int i = half; i < L; i += 2) {
            const int e = i * KDA_DK + c;
            const float gi = sG[i * LDK + c], kni = sK[i * LDK + c], qni = R[KDA_BR_QN + e];
            const float bi = sBeta[i];
            float ag = 0.f, ak = 0.f, aq = 0.f, ab = 0.f;
            for (int jj = 0; jj <= i; jj++) {
                const float E = expf(gi - sG[jj * LDK + c]);
                const float knj = sK[jj * LDK + c] * E;
                const float a = sdA[i * LDT + jj], p = sdP[i * LDT + jj];
                const float ta = a * bi * kni * knj, tp = p * scale * qni * knj;
                ag += ta + tp;
                ak = fmaf(a * bi, knj, ak);
                aq = fmaf(p * scale, knj, aq);
                ab = fmaf(a * kni, knj, ab);
            }
            dG[e] += ag;
            dkn[e] += ak;
            dqn[e] += aq;
            XU[e] += ab;
        }
        __syncthreads();

        /* s9: pairwise factors, column side: rows j of parity half, i >= j */
        for (int jj = half; jj < L; jj += 2) {
            const int e = jj * KDA_DK + c;
            const float gj = sG[jj * LDK + c], knj = sK[jj * LDK + c];
            float ag = 0.f, ak = 0.f;
            for (int i = jj; i < L; i++) {
                const float E = expf(sG[i * LDK + c] - gj);
                const float a = sdA[i * LDT + jj], p = sdP[i * LDT + jj];
                const float tt = (a * sBeta[i] * sK[i * LDK + c] + p * scale * R[KDA_BR_QN + i * KDA_DK + c]) * E;
                ak += tt;
                ag = fmaf(-tt, knj, ag);
            }
            dG[e] += ag;
            dkn[e] += ak;
        }
        __syncthreads();

        /* s10: d log a = reverse cumsum of dG (G_L's gradient on the last row), then the gate */
        if (half == 0) {
            float run = sGL[c], pdt = 0.f, pa = 0.f;
            for (int i = L - 1; i >= 0; i--) {
                run += dG[i * KDA_DK + c];
                const float x = bf2f(g[((t0 + i) * H + h) * KDA_DK + c]) + dt_bias[h * KDA_DK + c];
                const float free_la = -rate * softplus_f(x);
                const float dla = free_la < lower_bound ? 0.f : run;
                const float dx = -dla * rate * sigmoid_f(x);
                dg[((t0 + i) * H + h) * KDA_DK + c] = dx;
                pdt += dx;
                pa = fmaf(dla, free_la, pa);
            }
            part[item * KDA_BWD_PART_FLOATS + c] = pdt;
            sRed[c] = pa;
        }
        __syncthreads();
        if (t == 0) {
            float s = 0.f;
            for (int cc = 0; cc < KDA_DK; cc++) s += sRed[cc];
            part[item * KDA_BWD_PART_FLOATS + KDA_DK] = s;
        }

        /* s11: through the L2 norms; thread t: row t / 4, channels 32 (t % 4) + [0, 32) */
        {
            const int i = t >> 2, c0 = (t & 3) * 32;
            float sq = 0.f, sk = 0.f, sb = 0.f;
            if (i < L) {
                for (int cc = 0; cc < 32; cc++) {
                    const int e = i * KDA_DK + c0 + cc;
                    sq = fmaf(R[KDA_BR_QN + e], dqn[e], sq);
                    sk = fmaf(R[KDA_BR_KN + e], dkn[e], sk);
                    sb += XU[e];
                }
            }
            /* xor butterflies: every lane of a quad adds the same pairs (deterministic) */
            sq += __shfl_xor(sq, 1);
            sq += __shfl_xor(sq, 2);
            sk += __shfl_xor(sk, 1);
            sk += __shfl_xor(sk, 2);
            sb += __shfl_xor(sb, 1);
            sb += __shfl_xor(sb, 2);
            if (i < L) {
                const float inq = 1.f / R[KDA_BR_NQ + i], ink = 1.f / R[KDA_BR_NK + i];
                const int64_t row = ((t0 + i) * H + h) * KDA_DK + c0;
                for (int cc = 0; cc < 32; cc++) {
                    const int e = i * KDA_DK + c0 + cc;
                    dq[row + cc] = (dqn[e] - R[KDA_BR_QN + e] * sq) * inq;
                    dk[row + cc] = (dkn[e] - R[KDA_BR_KN + e] * sk) * ink;
                }
                if ((t & 3) == 0) dbeta[(t0 + i) * H + h] = sb;
            }
        }
        __syncthreads();
    }
}

/* ------------------------------------------------------------------------- */
/* per-head sums of the gate partials, grid H, 128 threads                     */
/* ------------------------------------------------------------------------- */
extern "C" __global__ void __launch_bounds__(128)
kda_bwd_reduce_kernel(const float *__restrict__ part, const int32_t *__restrict__ chunk_off, int64_t nseq,
                      int64_t nslots, float *__restrict__ dA_log, float *__restrict__ ddt_bias)
{
    const int h = blockIdx.x, c = threadIdx.x;
    const int64_t nvalid = chunk_off == nullptr ? nslots : (int64_t)chunk_off[nseq];
    float s = 0.f, sa = 0.f;
    for (int64_t slot = 0; slot < nvalid; slot++) {
        const float *p = part + ((int64_t)h * nslots + slot) * KDA_BWD_PART_FLOATS;
        s += p[c];
        if (c == 0) sa += p[KDA_DK];
    }
    ddt_bias[h * KDA_DK + c] = s;
    if (c == 0) dA_log[h] = sa;
}

/* ------------------------------------------------------------------------- */
/* launcher: stage 0 chunk quantities, 1 scan, 2 gradients, 3 gate sums        */
/* ------------------------------------------------------------------------- */
extern "C" hipError_t kda_launch_bwd(int stage, const void *q, const void *k, const void *v, const void *g,
                                     const void *beta, const void *dout, const float *A_log,
                                     const float *dt_bias, float scale, float lower_bound,
                                     const void *init, int init_fp32, const float *dfinal,
                                     const int32_t *cu, const int32_t *chunk_off, int64_t nseq, int64_t T,
                                     int64_t H, int64_t nslots, unsigned char *area, float *dq, float *dk,
                                     float *dv, float *dg, float *dbeta, float *dA_log, float *ddt_bias,
                                     float *dinit, hipStream_t st)
{
    const int64_t items = H * nslots;
    float *brec = (float *)area;
    float *ckpt = brec + (size_t)items * KDA_BR_FLOATS;
    float *dse = ckpt + (size_t)items * KDA_DK * KDA_DV;
    float *part = dse + (size_t)items * KDA_DK * KDA_DV;
    float *scratch = (float *)((unsigned char *)part + kda_bwd_part_bytes(items));
    switch (stage) {
    case 0:
        hipLaunchKernelGGL(kda_bwd_chunk_kernel, dim3((unsigned)items), dim3(NT), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)g,
                           (const uint16_t *)beta, A_log, dt_bias, scale, lower_bound, cu, chunk_off, nseq, T,
                           (int)H, nslots, brec);
        break;
    case 1:
        hipLaunchKernelGGL(kda_bwd_scan_kernel, dim3((unsigned)(nseq * H * 8)), dim3(NT), 0, st, brec, cu,
                           chunk_off, nseq, T, (int)H, nslots, init, init_fp32, dfinal, (const uint16_t *)dout,
                           ckpt, dse, dinit);
        break;
    case 2:
        hipLaunchKernelGGL(kda_bwd_grad_kernel, dim3((unsigned)kda_bwd_grad_wgs(items)), dim3(NT), 0, st,
                           (const uint16_t *)v, (const uint16_t *)g, (const uint16_t *)dout, A_log, dt_bias, scale,
                           lower_bound, cu, chunk_off, nseq, T, (int)H, nslots, brec, ckpt, dse, part, scratch,
                           dq, dk, dv, dg, dbeta);
        break;
    case 3:
        hipLaunchKernelGGL(kda_bwd_reduce_kernel, dim3((unsigned)H), dim3(128), 0, st, part, chunk_off, nseq,
                           nslots, dA_log, ddt_bias);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
