/*
 * kda_bwd.hip -- gfx950 kernels of the backward of the chunked Kimi Delta
 * Attention forward: gradients of q, k, v, g, beta, A_log, dt_bias and the
 * initial state for L = <dout, out> + <dfinal, final_state>.
 *
 * The FlashKDA pages show only the forward ("Core Kernel API / flash_kda.fwd",
 * ccm-staging page); these are the derivatives of the forward recurrence
 * described in kda.h, taken through its chunked form (kda_internal.h). All
 * arithmetic is fp32: the matrix products of the scan and of the gradient
 * kernel on fp32 MFMA (v_mfma_f32_16x16x4f32), the rest on the vector ALUs:
 *
 *   kda_bwd_chunk_kernel  one workgroup per (chunk, head): q^, k^, log a, G, A, P
 *                         (16 x 16 blocks below the diagonal on MFMA with the decay
 *                         split at a block boundary, diagonal blocks per element),
 *                         T = (I + A)^-1 (forward substitution by 16-row blocks),
 *                         W, U, Q' (MFMA), K~, e^{G_L}, stored as fp32 per-chunk areas.
 *   kda_bwd_scan_kernel   one workgroup per (sequence, head, 16 value columns),
 *                         fp32 MFMA; value columns are independent in both directions:
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
 *                         e^{G_i - G_j} (<= 1; partners in other 16-row blocks on
 *                         MFMA with the factor split at a block boundary, own-block
 *                         partners per element), the in-chunk cumsum, the gate and
 *                         the L2 norms.
 *   kda_bwd_reduce_kernel sums the per-chunk gate partials of each head into
 *                         d A_log and d dt_bias (fixed order: deterministic).
 */
#include "kda.h"
#include "kda_device.h"

namespace {

constexpr int NT = 256;   /* threads of the chunk and scan workgroups */
constexpr int NTG = 512;  /* threads of a gradient workgroup (eight waves) */
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

__device__ __forceinline__ f32x4 mfma4(float a, float b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

/* LDS staging of one 32-wide contraction slice for wg_gemm: A^T [32][WS_LSA] and
 * B [32][WS_LSB] (rows = contraction index); two such buffers */
constexpr int WS_LSA = 68, WS_LSB = 132;
constexpr int WS_STAGE = 32 * WS_LSA + 32 * WS_LSB;

/* one operand slice of wg_gemm (contraction indices 32 sl .. 32 sl + 31) into this
 * thread's registers: 16 bytes of A and N / 64 times 16 bytes of B */
template <bool TA, bool TB, int N, int lda, int ldb>
__device__ __forceinline__ void wg_slice_load(float4 &ra, float4 (&rbq)[N / 64], const float *A, const float *B,
                                              int sl, int tid)
{
    const int kb = 32 * sl;
    if (TA) ra = *(const float4 *)(A + (kb + (tid >> 4)) * lda + 4 * (tid & 15));
    else ra = *(const float4 *)(A + (tid >> 3) * lda + kb + 4 * (tid & 7));
#pragma unroll
    for (int p = 0; p < N / 64; p++) {
        const int idx = tid + 512 * p;
        if (TB) rbq[p] = *(const float4 *)(B + (idx >> 3) * ldb + kb + 4 * (idx & 7));
        else rbq[p] = *(const float4 *)(B + (kb + idx / (N / 4)) * ldb + 4 * (idx % (N / 4)));
    }
}

/* the registers of wg_slice_load into one LDS staging buffer (A^T and B rows by
 * contraction index) */
template <bool TA, bool TB, int N>
__device__ __forceinline__ void wg_slice_store(float *sa, const float4 &ra, const float4 (&rbq)[N / 64], int tid)
{
    float *sb = sa + 32 * WS_LSA;
    if (TA) {
        *(float4 *)(sa + (tid >> 4) * WS_LSA + 4 * (tid & 15)) = ra;
    } else {
        const int i = tid >> 3, c = 4 * (tid & 7);
        sa[c * WS_LSA + i] = ra.x; sa[(c + 1) * WS_LSA + i] = ra.y;
        sa[(c + 2) * WS_LSA + i] = ra.z; sa[(c + 3) * WS_LSA + i] = ra.w;
    }
#pragma unroll
    for (int p = 0; p < N / 64; p++) {
        const int idx = tid + 512 * p;
        if (TB) {
            const int j = idx >> 3, c = 4 * (idx & 7);
            sb[c * WS_LSB + j] = rbq[p].x; sb[(c + 1) * WS_LSB + j] = rbq[p].y;
            sb[(c + 2) * WS_LSB + j] = rbq[p].z; sb[(c + 3) * WS_LSB + j] = rbq[p].w;
        } else {
            *(float4 *)(sb + (idx / (N / 4)) * WS_LSB + 4 * (idx % (N / 4))) = rbq[p];
        }
    }
}

/* C[i][j] = (acc ? C[i][j] : 0) + alpha * sum_k a(i, k) b(k, j) for i < 64, j < N,
 * with a(i, k) = TA ? A[k][i] : A[i][k] and b(k, j) = TB ? B[j][k] : B[k][j], dense
 * row-major operands (A is [64][KD], [KD][64] if TA; B is [KD][N], [N][KD] if TB;
 * C is [64][N]), on fp32 MFMA (16 x 16 x 4 blocks) by the eight waves of a
 * gradient workgroup. Wave w holds row blocks 2 (w % 2) + {0, 1} and N / 64 column
 * blocks starting at (w / 2) N / 64. The contraction runs in 32-wide slices: each
 * operand slice is read from global memory once per workgroup, 16 bytes per thread
 * (coalesced), into an LDS buffer from which the waves read their fragments (lane
 * group gq takes contraction indices 8 gq .. 8 gq + 7 of the slice); the next slice
 * is loaded into registers while the current one is multiplied, then written to the
 * other buffer (one barrier per slice). Every row stride and base is a multiple of
 * 4 floats. stage: 2 * WS_STAGE floats of LDS, 16-byte aligned. Every thread of the
 * workgroup calls it (it holds barriers); callers separate products that share an
 * output or read one another's output with a barrier. */
template <bool TA, bool TB, int N, int KD>
__device__ __forceinline__ void wg_gemm(float *C, const float *A, const float *B, float alpha, bool acc,
                                          float *stage)
{
    static_assert(N % 64 == 0 && KD % 32 == 0, "block shape");
    constexpr int lda = TA ? 64 : KD, ldb = TB ? KD : N, ldc = N;
    constexpr int NBW = N / 64, NSL = KD / 32, NBQ = N / 64; /* B float4 pieces per thread */
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int l = tid & 63, w = tid >> 6, gq = l >> 4, r16 = l & 15;
    const int rb0 = 2 * (w & 1), cb0 = (w >> 1) * NBW;
    float4 ra, rbq[NBQ];
    f32x4 d[2][NBW];
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int cb = 0; cb < NBW; cb++) d[rb][cb] = zero4();
    wg_slice_load<TA, TB, N, lda, ldb>(ra, rbq, A, B, 0, tid);
    wg_slice_store<TA, TB, N>(stage, ra, rbq, tid);
    __syncthreads();
#pragma unroll
    for (int sl = 0; sl < NSL; sl++) {
        if (sl + 1 < NSL) wg_slice_load<TA, TB, N, lda, ldb>(ra, rbq, A, B, sl + 1, tid);
        const float *sa = stage + (sl & 1) * WS_STAGE, *sb = sa + 32 * WS_LSA;
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const int k = 8 * gq + s;
            float a[2], b[NBW];
#pragma unroll
            for (int rb = 0; rb < 2; rb++) a[rb] = sa[k * WS_LSA + 16 * (rb0 + rb) + r16];
#pragma unroll
            for (int cb = 0; cb < NBW; cb++) b[cb] = sb[k * WS_LSB + 16 * (cb0 + cb) + r16];
#pragma unroll
            for (int rb = 0; rb < 2; rb++)
#pragma unroll
                for (int cb = 0; cb < NBW; cb++) d[rb][cb] = mfma4(a[rb], b[cb], d[rb][cb]);
        }
        if (sl + 1 < NSL) wg_slice_store<TA, TB, N>(stage + ((sl + 1) & 1) * WS_STAGE, ra, rbq, tid);
        __syncthreads();
    }
    if (acc) {
        float cv[2][NBW][4];
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int cb = 0; cb < NBW; cb++)
#pragma unroll
                for (int e = 0; e < 4; e++) cv[rb][cb][e] = C[(16 * (rb0 + rb) + 4 * gq + e) * ldc + 16 * (cb0 + cb) + r16];
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int cb = 0; cb < NBW; cb++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    C[(16 * (rb0 + rb) + 4 * gq + e) * ldc + 16 * (cb0 + cb) + r16] = fmaf(alpha, d[rb][cb][e], cv[rb][cb][e]);
    } else {
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int cb = 0; cb < NBW; cb++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    C[(16 * (rb0 + rb) + 4 * gq + e) * ldc + 16 * (cb0 + cb) + r16] = alpha * d[rb][cb][e];
    }
}

} // namespace

/* ------------------------------------------------------------------------- */
/* chunk quantities, one workgroup per (chunk slot, head), grid H * nslots     */
/* ------------------------------------------------------------------------- */
extern "C" __global__ void __launch_bounds__(NTG)
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

    /* 1. norms and gate: thread t covers row t / 8, channels 16 (t % 8) + [0, 16), read
     *    as 16-byte pieces */
    {
        const int i = t >> 3, c0 = (t & 7) * 16;
        const float rate = expf(A_log[h]);
        if (i < L) {
            const int64_t base = ((t0 + i) * H + h) * KDA_DK + c0;
            uint4 uq[2], uk[2], ug[2];
#pragma unroll
            for (int p = 0; p < 2; p++) {
                uq[p] = *(const uint4 *)(q + base + 8 * p);
                uk[p] = *(const uint4 *)(k + base + 8 * p);
                ug[p] = *(const uint4 *)(g + base + 8 * p);
            }
            float qx[16], kx[16], gx[16];
#pragma unroll
            for (int p = 0; p < 2; p++)
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const uint32_t wq = u == 0 ? uq[p].x : u == 1 ? uq[p].y : u == 2 ? uq[p].z : uq[p].w;
                    const uint32_t wk = u == 0 ? uk[p].x : u == 1 ? uk[p].y : u == 2 ? uk[p].z : uk[p].w;
                    const uint32_t wg = u == 0 ? ug[p].x : u == 1 ? ug[p].y : u == 2 ? ug[p].z : ug[p].w;
                    qx[8 * p + 2 * u] = bf2f((uint16_t)(wq & 0xffff));
                    qx[8 * p + 2 * u + 1] = bf2f((uint16_t)(wq >> 16));
                    kx[8 * p + 2 * u] = bf2f((uint16_t)(wk & 0xffff));
                    kx[8 * p + 2 * u + 1] = bf2f((uint16_t)(wk >> 16));
                    gx[8 * p + 2 * u] = bf2f((uint16_t)(wg & 0xffff));
                    gx[8 * p + 2 * u + 1] = bf2f((uint16_t)(wg >> 16));
                }
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int c = 0; c < 16; c++) {
                sq = fmaf(qx[c], qx[c], sq);
                sk = fmaf(kx[c], kx[c], sk);
            }
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) {
                sq += __shfl_xor(sq, o);
                sk += __shfl_xor(sk, o);
            }
            const float nq = sqrtf(sq + 1e-6f), nk = sqrtf(sk + 1e-6f);
#pragma unroll
            for (int c = 0; c < 16; c++) {
                sQ[i * LDK + c0 + c] = qx[c] / nq;
                sK[i * LDK + c0 + c] = kx[c] / nk;
                const float x = gx[c] + dt_bias[h * KDA_DK + c0 + c];
                sG[i * LDK + c0 + c] = fmaxf(-rate * softplus_f(x), lower_bound);
            }
            if ((t & 7) == 0) {
                const float b = bf2f(beta[(t0 + i) * H + h]);
                sB[i] = b;
                R[KDA_BR_BETA + i] = b;
                R[KDA_BR_NQ + i] = nq;
                R[KDA_BR_NK + i] = nk;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 16; c++) {
                sQ[i * LDK + c0 + c] = 0.f;
                sK[i * LDK + c0 + c] = 0.f;
                sG[i * LDK + c0 + c] = 0.f;
            }
            if ((t & 7) == 0) {
                sB[i] = 0.f;
                R[KDA_BR_BETA + i] = 0.f;
                R[KDA_BR_NQ + i] = 1.f;
                R[KDA_BR_NK + i] = 1.f;
            }
        }
    }
    for (int e = t; e < KDA_CHUNK * KDA_CHUNK; e += NTG) {
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

    /* 3. A (j < i) and P (j <= i). Pairs inside the four diagonal 16 x 16 blocks
     *    (136 each) element by element; the six blocks below them on fp32 MFMA with
     *    the decay split at the end of the block before row i's (anchor a, G_a):
     *      A_ij = beta_i sum_c (k^_ic e^{G_ic - G_ac}) (k^_jc e^{G_ac - G_jc}),
     *      P_ij = scale sum_c (q^_ic e^{G_ic - G_ac}) (k^_jc e^{G_ac - G_jc}),
     *    both factors <= 1 for j <= a < i. Rows past the chunk have k^ = q^ = 0. */
    for (int e = t; e < 4 * 136; e += NTG) {
        const int bd = e / 136, r = e - bd * 136;
        int ii = (int)((sqrtf(8.f * (float)r + 1.f) - 1.f) * 0.5f);
        while (ii * (ii + 1) / 2 > r) ii--;
        while ((ii + 1) * (ii + 2) / 2 <= r) ii++;
        const int i = 16 * bd + ii, j = 16 * bd + r - ii * (ii + 1) / 2;
        float a = 0.f, p = 0.f;
        for (int c = 0; c < KDA_DK; c++) {
            const float E = exp2_fast((sG[i * LDK + c] - sG[j * LDK + c]) * LOG2E_F);
            const float kj = sK[j * LDK + c] * E;
            a = fmaf(sK[i * LDK + c], kj, a);
            p = fmaf(sQ[i * LDK + c], kj, p);
        }
        sA[i * LDT + j] = j < i ? sB[i] * a : 0.f;
        sP[i * LDT + j] = scale * p;
    }
    {
        /* block (ib, jb), jb < ib: list index w, one per wave (waves 6 and 7 idle) */
        const int w = t >> 6, l = t & 63, gq = l >> 4, r16 = l & 15;
        for (int bi = w; bi < 6; bi += 8) {
            const int ib = bi == 0 ? 1 : bi < 3 ? 2 : 3;
            const int jb = bi == 0 ? 0 : bi < 3 ? bi - 1 : bi - 3;
            const int ia = 16 * ib - 1, i = 16 * ib + r16, j = 16 * jb + r16;
            f32x4 accA = zero4(), accP = zero4();
            for (int c0 = 0; c0 < KDA_DK; c0 += 4) {
                const int c = c0 + gq;
                const float ga = sG[ia * LDK + c];
                const float fi = exp2_fast(fminf(sG[i * LDK + c] - ga, 0.f) * LOG2E_F);
                const float bj = sK[j * LDK + c] * exp2_fast(fminf(ga - sG[j * LDK + c], 0.f) * LOG2E_F);
                accA = mfma4(sK[i * LDK + c] * fi, bj, accA);
                accP = mfma4(sQ[i * LDK + c] * fi, bj, accP);
            }
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int ro = 16 * ib + 4 * gq + e;
                sA[ro * LDT + j] = sB[ro] * accA[e];
                sP[ro * LDT + j] = scale * accP[e];
            }
        }
    }
    __syncthreads();

    /* 4. T = (I + A)^-1 by forward substitution in blocks of 16 rows: wave w inverts
     *    the diagonal block (I + A_ww) with column j in registers of lanes j, j + 16, ...
     *    (T_ww[r][j] = delta_rj - sum_{m < r} A_ww[r][m] T_ww[m][j]); then, for
     *    i - b = 1, 2, 3, T_ib = -T_ii sum_{b <= m < i} A_im T_mb on fp32 MFMA, wave b
     *    taking block (b + d, b) */
    {
        const int w = t >> 6, l = t & 63, gq = l >> 4, r16 = l & 15;
        if (w < 4) { /* waves 4-7 have no diagonal block */
            float tc[16];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float s = r == r16 ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; m++) s = fmaf(-sA[(16 * w + r) * LDT + 16 * w + m], tc[m], s);
                tc[r] = s;
            }
            if (gq == 0) {
#pragma unroll
                for (int r = 0; r < 16; r++) sT[(16 * w + r) * LDT + 16 * w + r16] = tc[r];
            }
        }
        __syncthreads();
        for (int d = 1; d < 4; d++) {
            const int bb = w, ib = w + d;
            if (ib < 4) {
                /* X = sum_m A_im T_mb: contraction index 16 m + 4 s + gq at step s */
                f32x4 x = zero4();
                for (int m = bb; m < ib; m++) {
#pragma unroll
                    for (int s4 = 0; s4 < 4; s4++) {
                        const int kk = 16 * m + 4 * s4 + gq;
                        x = mfma4(sA[(16 * ib + r16) * LDT + kk], sT[kk * LDT + 16 * bb + r16], x);
                    }
                }
                /* T_ib = -T_ii X; X in accumulator layout is the B operand for the
                 * contraction index 4 gq + s at step s */
                f32x4 y = zero4();
#pragma unroll
                for (int s4 = 0; s4 < 4; s4++)
                    y = mfma4(-sT[(16 * ib + r16) * LDT + 16 * ib + 4 * gq + s4], x[s4], y);
#pragma unroll
                for (int e = 0; e < 4; e++) sT[(16 * ib + 4 * gq + e) * LDT + 16 * bb + r16] = y[e];
            }
            __syncthreads();
        }
    }

    /* 5. store T, P, q^, k^, G */
    for (int e = t; e < KDA_CHUNK * KDA_CHUNK; e += NTG) {
        const int i = e >> 6, j = e & 63;
        R[KDA_BR_T + e] = sT[i * LDT + j];
        R[KDA_BR_P + e] = sP[i * LDT + j];
    }
    for (int e = t; e < KDA_CHUNK * KDA_DK; e += NTG) {
        const int i = e >> 7, c = e & 127;
        R[KDA_BR_QN + e] = sQ[i * LDK + c];
        R[KDA_BR_KN + e] = sK[i * LDK + c];
        R[KDA_BR_G + e] = sG[i * LDK + c];
    }

    /* 6. W = T X_W (X_W = beta k^ e^G), U = T X_U (X_U = beta v) and
     *    Q' = scale q^ e^G - P W on fp32 MFMA: wave w takes columns 16 w .. 16 w + 15
     *    (one 16-column block) of all 64 rows; the contraction index of the first two
     *    products is 16 kb + 4 s + gq at step s, and W's accumulators serve as the B
     *    operand of P W (contraction index 16 kb + 4 gq + s). Rows m >= L contribute
     *    nothing (beta_m = 0 there, and v is not read). Then K~ and e^{G_L}. */
    {
        const int w = t >> 6, l = t & 63, gq = l >> 4, r16 = l & 15;
        f32x4 wacc[4][1], uacc[4][1];
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
#pragma unroll
            for (int cbi = 0; cbi < 1; cbi++) {
                wacc[rb][cbi] = zero4();
                uacc[rb][cbi] = zero4();
            }
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
#pragma unroll
            for (int s4 = 0; s4 < 4; s4++) {
                const int m = 16 * kb + 4 * s4 + gq;
                float ta[4];
#pragma unroll
                for (int rb = 0; rb < 4; rb++) ta[rb] = sT[(16 * rb + r16) * LDT + m];
#pragma unroll
                for (int cbi = 0; cbi < 1; cbi++) {
                    const int c = 16 * (w + cbi) + r16;
                    const float xw = sB[m] * sK[m * LDK + c] * expf(sG[m * LDK + c]);
                    /* unconditional load from a row inside the chunk, then a select:
                     * a load under a branch would wait for every outstanding load */
                    const float vm = bf2f(v[((t0 + (m < L ? m : L - 1)) * H + h) * KDA_DV + c]);
                    const float xu = m < L ? sB[m] * vm : 0.f;
#pragma unroll
                    for (int rb = 0; rb < 4; rb++) {
                        wacc[rb][cbi] = mfma4(ta[rb], xw, wacc[rb][cbi]);
                        uacc[rb][cbi] = mfma4(ta[rb], xu, uacc[rb][cbi]);
                    }
                }
            }
        }
        f32x4 qacc[4][1];
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
#pragma unroll
            for (int cbi = 0; cbi < 1; cbi++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int row = 16 * rb + 4 * gq + e, c = 16 * (w + cbi) + r16;
                    R[KDA_BR_W + row * KDA_DK + c] = wacc[rb][cbi][e];
                    R[KDA_BR_U + row * KDA_DV + c] = uacc[rb][cbi][e];
                    qacc[rb][cbi][e] = scale * sQ[row * LDK + c] * expf(sG[row * LDK + c]);
                }
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
#pragma unroll
            for (int s4 = 0; s4 < 4; s4++) {
                const int m = 16 * kb + 4 * gq + s4;
#pragma unroll
                for (int ib = 0; ib < 4; ib++) {
                    const float pa = -sP[(16 * ib + r16) * LDT + m];
#pragma unroll
                    for (int cbi = 0; cbi < 1; cbi++) qacc[ib][cbi] = mfma4(pa, wacc[kb][cbi][s4], qacc[ib][cbi]);
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
#pragma unroll
            for (int cbi = 0; cbi < 1; cbi++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    R[KDA_BR_QP + (16 * rb + 4 * gq + e) * KDA_DK + 16 * (w + cbi) + r16] = qacc[rb][cbi][e];
    }
    for (int e = t; e < KDA_CHUNK * KDA_DK; e += NTG) {
        const int i = e >> 7, c = e & 127;
        R[KDA_BR_KT + e] = sK[i * LDK + c] * expf(sG[(L - 1) * LDK + c] - sG[i * LDK + c]);
    }
    if (t < KDA_DK) R[KDA_BR_GL + t] = expf(sG[(L - 1) * LDK + t]);
}

/* ------------------------------------------------------------------------- */
/* state checkpoints and state gradients: one workgroup of 4 waves per        */
/* (sequence, head, 16 value columns), grid N * H * 8, on fp32 MFMA. Lane      */
/* (r16, gq) of wave w holds rows 16 (2 w + rb) + 4 gq + e (rb < 2, e < 4),    */
/* column 16 tile + r16 of S and dS (the 16 x 16 accumulator layout). Record   */
/* rows past a chunk's last token are zero, so every product runs over all 64. */
/* ------------------------------------------------------------------------- */

/* LDS slot of row r, column j of the 128 x 16 state tile and of the 64 x 16
 * chunk tile: the four lane groups read rows 32 (resp. 16) apart, which the
 * row offsets spread over the banks */
__host__ __device__ constexpr int s_lds(int r, int j) { return r * 16 + (r >> 5) * 8 + j; }
__host__ __device__ constexpr int d_lds(int i, int j) { return i * 16 + (i >> 4) * 8 + j; }

/* one chunk's operands of the forward state pass, for lane (r16, gq) of wave w:
 * W row 16 w + r16, columns 32 gq .. 32 gq + 31; K~[16 gq + s][16 (2 w + rb) + r16];
 * U rows 16 w + 4 gq + e, column col; e^{G_L} of rows 16 (2 w + rb) + 4 gq + e */
struct FwdOps {
    float4 wv[8];
    float kt[2][16];
    f32x4 u, gl[2];
};

__device__ __forceinline__ void load_fwd(FwdOps &o, const float *R, int w, int gq, int r16, int col)
{
    const float *wrow = R + KDA_BR_W + (16 * w + r16) * KDA_DK + 32 * gq;
#pragma unroll
    for (int i = 0; i < 8; i++) o.wv[i] = *(const float4 *)(wrow + 4 * i);
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int s = 0; s < 16; s++) o.kt[rb][s] = R[KDA_BR_KT + (16 * gq + s) * KDA_DK + 16 * (2 * w + rb) + r16];
#pragma unroll
    for (int e = 0; e < 4; e++) o.u[e] = R[KDA_BR_U + (16 * w + 4 * gq + e) * KDA_DV + col];
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int e = 0; e < 4; e++) o.gl[rb][e] = R[KDA_BR_GL + 16 * (2 * w + rb) + 4 * gq + e];
}

/* one chunk's early operands of the reverse pass: K~ row 16 w + r16, columns
 * 32 gq .. 32 gq + 31; dout rows 16 gq + s (zero past the chunk's L rows; the
 * load itself is unconditional, from a row clamped into the chunk, because a
 * load under a branch waits for every outstanding load), column col; e^{G_L}
 * of the lane's state rows */
struct RevOps {
    float4 kv[8];
    float o[16];
    f32x4 gl[2];
};

__device__ __forceinline__ void load_rev(RevOps &o, const float *R, const uint16_t *dout, int64_t row0, int64_t len,
                                         int64_t c, int H, int h, int w, int gq, int r16, int col)
{
    const float *krow = R + KDA_BR_KT + (16 * w + r16) * KDA_DK + 32 * gq;
#pragma unroll
    for (int i = 0; i < 8; i++) o.kv[i] = *(const float4 *)(krow + 4 * i);
    const int64_t rem = len - c * KDA_CHUNK;
    const int L = (int)(rem < KDA_CHUNK ? rem : KDA_CHUNK);
#pragma unroll
    for (int s = 0; s < 16; s++) {
        const int i = 16 * gq + s;
        const float x = bf2f(dout[((row0 + c * KDA_CHUNK + (i < L ? i : L - 1)) * H + h) * KDA_DV + col]);
        o.o[s] = i < L ? x : 0.f;
    }
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int e = 0; e < 4; e++) o.gl[rb][e] = R[KDA_BR_GL + 16 * (2 * w + rb) + 4 * gq + e];
}

extern "C" __global__ void __launch_bounds__(NT)
kda_bwd_scan_kernel(const float *__restrict__ brec, const int32_t *__restrict__ cu,
                    const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H, int64_t nslots,
                    const void *__restrict__ init, int init_fp32, const float *__restrict__ dfinal,
                    const uint16_t *__restrict__ dout, float *__restrict__ ckpt, float *__restrict__ dse,
                    float *__restrict__ dinit)
{
    __shared__ float sS[s_lds(127, 15) + 1], sD[d_lds(63, 15) + 1];
    /* XCD-aware: consecutive workgroups go to the 8 XCDs in turn, so the 8 value
     * tiles of chain c are workgroups 64 (c / 8) + 8 tile + c % 8, all on XCD c % 8,
     * and read each chunk's operands through one L2 */
    const int64_t bq = blockIdx.x >> 3;
    const int tile = (int)(bq & 7);
    const int64_t chain = (bq >> 3) * 8 + (blockIdx.x & 7);
    const int64_t seq = chain / H;
    const int h = (int)(chain - seq * H);
    if (seq >= nseq) return;
    int64_t nchunk, slot0, row0, len;
    bwd_seq(seq, cu, chunk_off, T, nchunk, slot0, row0, len);
    const int t = threadIdx.x, w = t >> 6, l = t & 63, gq = l >> 4, r16 = l & 15, col = tile * 16 + r16;
    const int64_t sbase = (seq * H + h) * (int64_t)(KDA_DK * KDA_DV);

    f32x4 S[2];
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int64_t o = sbase + (int64_t)(16 * (2 * w + rb) + 4 * gq + e) * KDA_DV + col;
            S[rb][e] = init == nullptr ? 0.f
                     : init_fp32 ? ((const float *)init)[o] : bf2f(((const uint16_t *)init)[o]);
        }

    /* forward: S_c is stored, D = U - W S_c, S_{c+1} = diag(e^{G_L}) S_c + K~^T D.
     * Two operand sets with fixed roles: the next chunk's are loaded while this one
     * is computed. */
    FwdOps opA, opB;
    auto fwd_step = [&](const FwdOps &cur, FwdOps &nxt, int64_t c) {
        const int64_t item = (int64_t)h * nslots + slot0 + c;
        float *ck = ckpt + item * (int64_t)(KDA_DK * KDA_DV);
        if (c + 1 < nchunk) load_fwd(nxt, brec + (item + 1) * KDA_BR_FLOATS, w, gq, r16, col);
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 16 * (2 * w + rb) + 4 * gq + e;
                ck[r * KDA_DV + col] = S[rb][e];
                sS[s_lds(r, r16)] = S[rb][e];
            }
        __syncthreads();
        /* B operands read from LDS in one batch, then the MFMAs (four chains) */
        float bs[32];
#pragma unroll
        for (int s = 0; s < 32; s++) bs[s] = sS[s_lds(32 * gq + s, r16)];
        f32x4 dp[4] = {cur.u, zero4(), zero4(), zero4()};
#pragma unroll
        for (int s = 0; s < 32; s++) {
            const float4 f = cur.wv[s >> 2];
            const float a = (s & 3) == 0 ? f.x : (s & 3) == 1 ? f.y : (s & 3) == 2 ? f.z : f.w;
            dp[s & 3] = mfma4(-a, bs[s], dp[s & 3]);
        }
        const f32x4 dacc = (dp[0] + dp[1]) + (dp[2] + dp[3]);
#pragma unroll
        for (int e = 0; e < 4; e++) sD[d_lds(16 * w + 4 * gq + e, r16)] = dacc[e];
        __syncthreads();
        float bd[16];
#pragma unroll
        for (int s = 0; s < 16; s++) bd[s] = sD[d_lds(16 * gq + s, r16)];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            f32x4 acc0 = cur.gl[rb] * S[rb], acc1 = zero4();
#pragma unroll
            for (int s = 0; s < 16; s += 2) {
                acc0 = mfma4(cur.kt[rb][s], bd[s], acc0);
                acc1 = mfma4(cur.kt[rb][s + 1], bd[s + 1], acc1);
            }
            S[rb] = acc0 + acc1;
        }
    };
    if (nchunk > 0) load_fwd(opA, brec + ((int64_t)h * nslots + slot0) * KDA_BR_FLOATS, w, gq, r16, col);
    for (int64_t c = 0; c < nchunk; c += 2) {
        fwd_step(opA, opB, c);
        if (c + 1 < nchunk) fwd_step(opB, opA, c + 1);
    }

    /* reverse: dS_{c+1} is stored, dD = K~ dS_{c+1},
     * dS_c = diag(e^{G_L}) dS_{c+1} - W^T dD + Q'^T dout_c. K~, dout and e^{G_L}
     * are loaded one chunk ahead; W and Q' at the top of the chunk (they are first
     * needed after the dD product). */
    f32x4 dS[2];
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int e = 0; e < 4; e++)
            dS[rb][e] = dfinal == nullptr ? 0.f
                      : dfinal[sbase + (int64_t)(16 * (2 * w + rb) + 4 * gq + e) * KDA_DV + col];
    RevOps rA, rB;
    auto rev_step = [&](const RevOps &rcur, RevOps &rnxt, int64_t c) {
        const int64_t item = (int64_t)h * nslots + slot0 + c;
        const float *R = brec + item * KDA_BR_FLOATS;
        float *dk = dse + item * (int64_t)(KDA_DK * KDA_DV);
        float wt[2][16], qt[2][16];
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int s = 0; s < 16; s++) {
                const int idx = (16 * gq + s) * KDA_DK + 16 * (2 * w + rb) + r16;
                wt[rb][s] = R[KDA_BR_W + idx];
                qt[rb][s] = R[KDA_BR_QP + idx];
            }
        if (c > 0) load_rev(rnxt, R - KDA_BR_FLOATS, dout, row0, len, c - 1, H, h, w, gq, r16, col);
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 16 * (2 * w + rb) + 4 * gq + e;
                dk[r * KDA_DV + col] = dS[rb][e];
                sS[s_lds(r, r16)] = dS[rb][e];
            }
        __syncthreads();
        float bs[32];
#pragma unroll
        for (int s = 0; s < 32; s++) bs[s] = sS[s_lds(32 * gq + s, r16)];
        f32x4 dp[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int s = 0; s < 32; s++) {
            const float4 f = rcur.kv[s >> 2];
            const float a = (s & 3) == 0 ? f.x : (s & 3) == 1 ? f.y : (s & 3) == 2 ? f.z : f.w;
            dp[s & 3] = mfma4(a, bs[s], dp[s & 3]);
        }
        const f32x4 dacc = (dp[0] + dp[1]) + (dp[2] + dp[3]);
#pragma unroll
        for (int e = 0; e < 4; e++) sD[d_lds(16 * w + 4 * gq + e, r16)] = dacc[e];
        __syncthreads();
        float bd[16];
#pragma unroll
        for (int s = 0; s < 16; s++) bd[s] = sD[d_lds(16 * gq + s, r16)];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            f32x4 acc0 = rcur.gl[rb] * dS[rb], acc1 = zero4();
#pragma unroll
            for (int s = 0; s < 16; s++) {
                acc0 = mfma4(-wt[rb][s], bd[s], acc0);
                acc1 = mfma4(qt[rb][s], rcur.o[s], acc1);
            }
            dS[rb] = acc0 + acc1;
        }
    };
    if (nchunk > 0)
        load_rev(rA, brec + ((int64_t)h * nslots + slot0 + nchunk - 1) * KDA_BR_FLOATS, dout, row0, len, nchunk - 1, H,
                 h, w, gq, r16, col);
    for (int64_t c = nchunk - 1; c >= 0; c -= 2) {
        rev_step(rA, rB, c);
        if (c > 0) rev_step(rB, rA, c - 1);
    }
    if (dinit != nullptr) {
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                dinit[sbase + (int64_t)(16 * (2 * w + rb) + 4 * gq + e) * KDA_DV + col] = dS[rb][e];
    }
}

/* ------------------------------------------------------------------------- */
/* gradients of one (chunk, head) per loop trip; grid <= KDA_BWD_GRAD_WGS,     */
/* each workgroup with its own KDA_BWD_SCR_FLOATS of scratch                   */
/* ------------------------------------------------------------------------- */
extern "C" __global__ void __launch_bounds__(NTG)
kda_bwd_grad_kernel(const uint16_t *__restrict__ v, const uint16_t *__restrict__ g,
                    const uint16_t *__restrict__ dout, const float *__restrict__ A_log,
                    const float *__restrict__ dt_bias, float scale, float lower_bound,
                    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, int64_t nseq,
                    int64_t T, int H, int64_t nslots, const float *__restrict__ brec,
                    const float *__restrict__ ckpt, const float *__restrict__ dse, float *__restrict__ part,
                    float *__restrict__ scratch, float *__restrict__ dq, float *__restrict__ dk,
                    float *__restrict__ dv, float *__restrict__ dg, float *__restrict__ dbeta)
{
    /* G, k^, q^ for the per-element phases; during the matrix products the same
     * LDS holds the products' operand slices */
    __shared__ __attribute__((aligned(16))) float sGKQ[3 * KDA_CHUNK * LDK];
    float *const sG = sGKQ, *const sK = sGKQ + KDA_CHUNK * LDK, *const sQ = sGKQ + 2 * KDA_CHUNK * LDK;
    float *const stage = sGKQ;
    static_assert(2 * WS_STAGE <= 3 * KDA_CHUNK * LDK, "staging fits");
    __shared__ float sdA[KDA_CHUNK * LDT], sdP[KDA_CHUNK * LDT];
    __shared__ float sBeta[KDA_CHUNK], sGL[KDA_DK], sRed[KDA_DK];
    __shared__ float sQx[3][KDA_DK], sTot[4][KDA_DK], sX[3][2][KDA_DK]; /* row-quarter exchanges */

    float *const scr0 = scratch + (size_t)blockIdx.x * KDA_BWD_SCR_FLOATS;

    /* thread t: channel c = t % 128 and row quarter qtr = t / 128 in the per-element phases */
    const int t = threadIdx.x, c = t & 127, qtr = t >> 7;
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
        /* the scratch base is re-derived per item (opaque to the compiler), so the
         * per-lane operand addresses of the products are not hoisted out of the item
         * loop, where they would hold hundreds of registers */
        float *scr = scr0;
        asm volatile("" : "+s"(scr));
        float *D = scr, *dD = scr + 8192, *dQp = scr + 2 * 8192, *dW = scr + 3 * 8192, *dKt = scr + 4 * 8192;
        float *dU = scr + 5 * 8192, *XW = scr + 6 * 8192, *XU = scr + 7 * 8192, *dXW = scr + 8 * 8192;
        float *dXU = scr + 9 * 8192, *dqn = scr + 10 * 8192, *dkn = scr + 11 * 8192, *dG = scr + 12 * 8192;
        float *DO = scr + 13 * 8192;
        float *dP = scr + 14 * 8192, *dT = dP + 4096, *X1 = dP + 2 * 4096;
        const float rate = expf(A_log[h]);

        /* s0: dout, X_W, X_U, D <- U. Eight elements per pass with all their loads
         * issued before any store (the scratch stores could otherwise alias the record
         * loads for the compiler) */
        for (int e0 = t; e0 < KDA_CHUNK * KDA_DK; e0 += 8 * NTG) {
            float xb[8], xo[8], xv[8], xg[8], xk[8], xu[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int e = e0 + u * NTG, i = e >> 7, cc = e & 127;
                const bool ok = i < L;
                /* loads are unconditional (rows clamped into the chunk) and selected after */
                const int64_t row = ((t0 + (ok ? i : L - 1)) * H + h) * KDA_DV + cc;
                xb[u] = R[KDA_BR_BETA + i];
                const float fo = bf2f(dout[row]), fv = bf2f(v[row]);
                xo[u] = ok ? fo : 0.f;
                xv[u] = ok ? fv : 0.f;
                xg[u] = R[KDA_BR_G + e];
                xk[u] = R[KDA_BR_KN + e];
                xu[u] = R[KDA_BR_U + e];
            }
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int e = e0 + u * NTG;
                DO[e] = xo[u];
                XU[e] = xb[u] * xv[u];
                XW[e] = xb[u] * xk[u] * exp2_fast(xg[u] * LOG2E_F);
                D[e] = xu[u];
            }
        }
        if (t < KDA_CHUNK) sBeta[t] = R[KDA_BR_BETA + t];
        __syncthreads();

        /* s1: D = U - W S, dD = K~ dS, dQ' = dout S^T */
        wg_gemm<false, false, KDA_DV, KDA_DK>(D, R + KDA_BR_W, S0, -1.f, true, stage);
        wg_gemm<false, false, KDA_DV, KDA_DK>(dD, R + KDA_BR_KT, dS, 1.f, false, stage);
        wg_gemm<false, true, KDA_DK, KDA_DV>(dQp, DO, S0, 1.f, false, stage);
        __syncthreads();

        /* s2: dW = -dD S^T, dK~ = D dS^T, dP = dout U^T, dU = P^T dout */
        wg_gemm<false, true, KDA_DK, KDA_DV>(dW, dD, S0, -1.f, false, stage);
        wg_gemm<false, true, KDA_DK, KDA_DV>(dKt, D, dS, 1.f, false, stage);
        wg_gemm<false, true, KDA_CHUNK, KDA_DV>(dP, DO, R + KDA_BR_U, 1.f, false, stage);
        wg_gemm<true, false, KDA_DV, KDA_CHUNK>(dU, R + KDA_BR_P, DO, 1.f, false, stage);
        __syncthreads();

        /* s3: Q' = scale q^ e^G - P W: dP -= dQ' W^T, dW -= P^T dQ'; dU += dD */
        wg_gemm<false, true, KDA_CHUNK, KDA_DK>(dP, dQp, R + KDA_BR_W, -1.f, true, stage);
        wg_gemm<true, false, KDA_DK, KDA_CHUNK>(dW, R + KDA_BR_P, dQp, -1.f, true, stage);
        for (int e = t; e < KDA_CHUNK * KDA_DV; e += NTG) dU[e] += dD[e];
        __syncthreads();

        /* s4: dT = dW X_W^T (+ dU X_U^T below), dX_W = T^T dW, dX_U = T^T dU; masked dP to LDS */
        wg_gemm<false, true, KDA_CHUNK, KDA_DK>(dT, dW, XW, 1.f, false, stage);
        wg_gemm<true, false, KDA_DK, KDA_CHUNK>(dXW, R + KDA_BR_T, dW, 1.f, false, stage);
        wg_gemm<true, false, KDA_DV, KDA_CHUNK>(dXU, R + KDA_BR_T, dU, 1.f, false, stage);
        for (int e = t; e < KDA_CHUNK * KDA_CHUNK; e += NTG) {
            const int i = e >> 6, jj = e & 63;
            sdP[i * LDT + jj] = jj <= i ? scale * dP[e] : 0.f; /* scale folded in */
        }
        __syncthreads();
        wg_gemm<false, true, KDA_CHUNK, KDA_DV>(dT, dU, XU, 1.f, true, stage);
        __syncthreads();

        /* s5: X1 = T^T dT */
        wg_gemm<true, false, KDA_CHUNK, KDA_CHUNK>(X1, R + KDA_BR_T, dT, 1.f, false, stage);
        __syncthreads();

        /* s6: dA = -X1 T^T (into dT, which is no longer needed), kept on the strict lower triangle */
        wg_gemm<false, true, KDA_CHUNK, KDA_CHUNK>(dT, X1, R + KDA_BR_T, -1.f, false, stage);
        /* s6b: d G_L from the carried decay: e^{G_L} sum_j dS[r][j] S[r][j]; thread t takes
         * row t / 4, columns 32 (t % 4) .. + 31 as 16-byte pieces */
        {
            const int r = t >> 2, hf = t & 3;
            const float4 *a4 = (const float4 *)(dS + r * KDA_DV + 32 * hf);
            const float4 *b4 = (const float4 *)(S0 + r * KDA_DV + 32 * hf);
            float s = 0.f;
#pragma unroll
            for (int jj = 0; jj < 8; jj++) {
                const float4 x = a4[jj], y = b4[jj];
                s = fmaf(x.x, y.x, s);
                s = fmaf(x.y, y.y, s);
                s = fmaf(x.z, y.z, s);
                s = fmaf(x.w, y.w, s);
            }
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            if (hf == 0) sGL[r] = R[KDA_BR_GL + r] * s;
        }
        __syncthreads();
        for (int e = t; e < KDA_CHUNK * KDA_CHUNK; e += NTG) {
            const int i = e >> 6, jj = e & 63;
            sdA[i * LDT + jj] = jj < i ? dT[e] : 0.f;
        }
        /* s6c: the products are done with the staging LDS: G (in log2 units), k^ and
         * q^ go there for the per-element phases, eight elements per pass */
        for (int e0 = t; e0 < KDA_CHUNK * KDA_DK; e0 += 8 * NTG) {
            float xg[8], xk[8], xq[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int e = e0 + u * NTG;
                xg[u] = R[KDA_BR_G + e];
                xk[u] = R[KDA_BR_KN + e];
                xq[u] = R[KDA_BR_QN + e];
            }
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int e = e0 + u * NTG, i = e >> 7, cc = e & 127;
                sG[i * LDK + cc] = xg[u] * LOG2E_F;
                sK[i * LDK + cc] = xk[u];
                sQ[i * LDK + cc] = xq[u];
            }
        }
        __syncthreads();

        /* s7: per-element terms (Q', K~, X_W, X_U); thread (c, qtr) takes rows i with
         * i % 4 = qtr, four rows per pass with all their loads issued first */
        {
            const float gl = sG[(L - 1) * LDK + c];
            float glacc = 0.f;
            for (int i0 = qtr; i0 < L; i0 += 16) {
                float xdq[4], xkt[4], xdkt[4], xdxw[4], xdxu[4], xv[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    /* unconditional loads from a row clamped into the chunk (rows past it
                     * are not used) */
                    const int i = i0 + 4 * u, ic = i < L ? i : L - 1, e = ic * KDA_DK + c;
                    xdq[u] = dQp[e];
                    xkt[u] = R[KDA_BR_KT + e];
                    xdkt[u] = dKt[e];
                    xdxw[u] = dXW[e];
                    xdxu[u] = dXU[e];
                    xv[u] = bf2f(v[((t0 + ic) * H + h) * KDA_DV + c]);
                }
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int i = i0 + 4 * u, e = i * KDA_DK + c;
                    if (i < L) {
                        const float gam = exp2_fast(sG[i * LDK + c]), kn = sK[i * LDK + c], qn = sQ[i * LDK + c];
                        const float b = sBeta[i];
                        float aq = scale * xdq[u] * gam;
                        float ag = scale * qn * gam * xdq[u];
                        float ak = xdkt[u] * exp2_fast(gl - sG[i * LDK + c]);
                        ag -= xdkt[u] * xkt[u];
                        glacc = fmaf(xdkt[u], xkt[u], glacc);
                        ak = fmaf(b * gam, xdxw[u], ak);
                        ag = fmaf(b * kn * gam, xdxw[u], ag);
                        dv[((t0 + i) * H + h) * KDA_DV + c] = b * xdxu[u];
                        XU[e] = kn * gam * xdxw[u] + xv[u] * xdxu[u]; /* d beta partial of (i, c); X_U is no longer needed */
                        dqn[e] = aq;
                        dkn[e] = ak;
                        dG[e] = ag;
                    }
                }
            }
            if (qtr > 0) sQx[qtr - 1][c] = glacc;
            __syncthreads();
            if (qtr == 0) sGL[c] += glacc + (sQx[0][c] + sQx[1][c]) + sQx[2][c];
        }
        __syncthreads();

        /* s8a: the pairwise sums over partners in other 16-row blocks, on fp32 MFMA.
         * With the factor split at a block boundary (anchor row a, value G_a),
         * e^{G_i - G_j} = e^{G_i - G_a} e^{G_a - G_j}, both factors <= 1 for j <= a < i:
         *   row side, row block ib >= 1, a = 16 ib - 1:
         *     SA_off[i] = e^{G_i - G_a} sum_{j <= a} dA_ij (k^_j e^{G_a - G_j}), SP_off likewise
         *     with scale dP;
         *   column side, block jb <= 2, a = 16 jb + 15:
         *     CT_off[j] = e^{G_a - G_j} sum_{i > a} (dA_ij beta_i k^_i + scale dP_ij q^_i) e^{G_i - G_a}.
         * Wave w takes channels 16 w .. 16 w + 15 (one 16-column block); the contraction
         * index at step s of lane group gq is k0 + gq. Results go to scratch arrays no
         * longer needed (D, dD, dW) as SA_off, SP_off, CT_off; rows without such
         * partners get 0. Exponents are in log2 units and clamped at 0. */
        {
            float *OA = D, *OP = dD, *OC = dW;
            int tid = t;
            asm volatile("" : "+v"(tid));
            const int w = tid >> 6, l = tid & 63, gq = l >> 4, r16 = l & 15;
            {
                const int cc = 16 * w + r16;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    OA[(4 * gq + e) * KDA_DK + cc] = 0.f;
                    OP[(4 * gq + e) * KDA_DK + cc] = 0.f;
                    OC[(48 + 4 * gq + e) * KDA_DK + cc] = 0.f;
                }
                for (int ib = 1; ib < 4; ib++) {
                    const float ga = sG[(16 * ib - 1) * LDK + cc];
                    f32x4 sa = zero4(), sp = zero4();
                    for (int k0 = 0; k0 < 16 * ib; k0 += 4) {
                        const int j = k0 + gq;
                        const float bv = sK[j * LDK + cc] * exp2_fast(fminf(ga - sG[j * LDK + cc], 0.f));
                        sa = mfma4(sdA[(16 * ib + r16) * LDT + j], bv, sa);
                        sp = mfma4(sdP[(16 * ib + r16) * LDT + j], bv, sp);
                    }
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int i = 16 * ib + 4 * gq + e;
                        const float f = exp2_fast(fminf(sG[i * LDK + cc] - ga, 0.f));
                        OA[i * KDA_DK + cc] = sa[e] * f;
                        OP[i * KDA_DK + cc] = sp[e] * f;
                    }
                }
                for (int jb = 0; jb < 3; jb++) {
                    const float ga = sG[(16 * jb + 15) * LDK + cc];
                    f32x4 ct = zero4();
                    for (int k0 = 16 * (jb + 1); k0 < KDA_CHUNK; k0 += 4) {
                        const int i = k0 + gq;
                        const float f = exp2_fast(fminf(sG[i * LDK + cc] - ga, 0.f));
                        ct = mfma4(sdA[i * LDT + 16 * jb + r16], sBeta[i] * sK[i * LDK + cc] * f, ct);
                        ct = mfma4(sdP[i * LDT + 16 * jb + r16], sQ[i * LDK + cc] * f, ct);
                    }
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int j = 16 * jb + 4 * gq + e;
                        OC[j * KDA_DK + cc] = ct[e] * exp2_fast(fminf(ga - sG[j * LDK + cc], 0.f));
                    }
                }
            }
        }
        __syncthreads();

        /* s8: pairwise factors, row side: rows i with i % 4 = qtr, j <= i. With
         * E = e^{G_i - G_j} per channel, SA = sum_j dA_ij k^_j E and SP = sum_j scale dP_ij k^_j E
         * give every row-side term: d k^_i += beta_i SA, d q^_i += SP,
         * dG_i += beta_i k^_i SA + q^_i SP, and the d beta partial k^_i SA. Partners in
         * the row's own 16-row block are summed here, the rest come from s8a. */
        for (int i = qtr; i < L; i += 4) {
            const int e = i * KDA_DK + c;
            const float g0 = dG[e], k0 = dkn[e], q0 = dqn[e], b0 = XU[e];
            const float gi = sG[i * LDK + c];
            float sa = D[e], sp = dD[e];
            /* two blocks of 8 partners with all LDS reads first; partners past i have
             * dA = dP = 0 there and a clamped (finite) factor, so they add exactly 0 */
#pragma unroll
            for (int j0 = (i & ~15); j0 < (i & ~15) + 16; j0 += 8) {
                float xg[8], xk[8], xa[8], xp[8];
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    xg[u] = sG[(j0 + u) * LDK + c];
                    xk[u] = sK[(j0 + u) * LDK + c];
                    xa[u] = sdA[i * LDT + j0 + u];
                    xp[u] = sdP[i * LDT + j0 + u];
                }
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const float knj = xk[u] * exp2_fast(fminf(gi - xg[u], 0.f));
                    sa = fmaf(xa[u], knj, sa);
                    sp = fmaf(xp[u], knj, sp);
                }
            }
            const float kni = sK[i * LDK + c], qni = sQ[i * LDK + c], bi = sBeta[i];
            dG[e] = g0 + fmaf(bi * kni, sa, qni * sp);
            dkn[e] = k0 + bi * sa;
            dqn[e] = q0 + sp;
            XU[e] = b0 + kni * sa;
        }
        __syncthreads();

        /* s9: pairwise factors, column side: rows j with j % 4 = qtr, i >= j:
         * CT = sum_i (dA_ij beta_i k^_i + scale dP_ij q^_i) E; d k^_j += CT, dG_j -= k^_j CT.
         * Rows i in the row's own 16-row block are summed here, the rest come from s8a. */
        for (int jj = qtr; jj < L; jj += 4) {
            const int e = jj * KDA_DK + c;
            const float g0 = dG[e], k0 = dkn[e];
            const float gj = sG[jj * LDK + c], knj = sK[jj * LDK + c];
            float ct = dW[e];
            /* two blocks of 8 rows, LDS reads first; rows before jj or past the chunk
             * have dA = dP = 0 there and add exactly 0 */
#pragma unroll
            for (int i0 = (jj & ~15); i0 < (jj & ~15) + 16; i0 += 8) {
                float xg[8], xk[8], xq[8], xb[8], xa[8], xp[8];
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const int i = i0 + u;
                    xg[u] = sG[i * LDK + c];
                    xk[u] = sK[i * LDK + c];
                    xq[u] = sQ[i * LDK + c];
                    xb[u] = sBeta[i];
                    xa[u] = sdA[i * LDT + jj];
                    xp[u] = sdP[i * LDT + jj];
                }
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const float coef = fmaf(xa[u] * xb[u], xk[u], xp[u] * xq[u]);
                    ct = fmaf(coef, exp2_fast(fminf(xg[u] - gj, 0.f)), ct);
                }
            }
            dG[e] = fmaf(-knj, ct, g0);
            dkn[e] = k0 + ct;
        }
        __syncthreads();

        /* s10: d log a = reverse cumsum of dG (G_L's gradient on the last row), then the
         * gate; thread (c, qtr) takes rows 16 qtr .. 16 qtr + 15, starting from the
         * totals of the quarters below it in the chunk (higher rows) */
        {
            const int r0 = 16 * qtr, n = L - r0; /* rows of this quarter: u < n */
            float xg[16], tot = 0.f;
#pragma unroll
            for (int u = 0; u < 16; u++) {
                const float x = dG[(r0 + u) * KDA_DK + c]; /* row < 64: always inside the scratch tile */
                xg[u] = u < n ? x : 0.f;
                tot += xg[u];
            }
            sTot[qtr][c] = tot;
            __syncthreads();
            float run = sGL[c], pdt = 0.f, pa = 0.f;
            for (int q = 3; q > qtr; q--) run += sTot[q][c];
            const float bias = dt_bias[h * KDA_DK + c];
            float xx[16]; /* gate inputs, loaded unconditionally from rows clamped into the chunk */
#pragma unroll
            for (int u = 0; u < 16; u++) {
                const int ic = r0 + u < L ? r0 + u : L - 1;
                xx[u] = bf2f(g[((t0 + ic) * H + h) * KDA_DK + c]);
            }
#pragma unroll
            for (int u = 15; u >= 0; u--) {
                if (u < n) {
                    const int i = r0 + u;
                    run += xg[u];
                    const float x = xx[u] + bias;
                    const float free_la = -rate * softplus_f(x);
                    const float dla = free_la < lower_bound ? 0.f : run;
                    const float dx = -dla * rate * sigmoid_f(x);
                    dg[((t0 + i) * H + h) * KDA_DK + c] = dx;
                    pdt += dx;
                    pa = fmaf(dla, free_la, pa);
                }
            }
            if (qtr > 0) {
                sX[qtr - 1][0][c] = pdt;
                sX[qtr - 1][1][c] = pa;
            }
            __syncthreads();
            if (qtr == 0) {
                part[item * KDA_BWD_PART_FLOATS + c] = pdt + (sX[0][0][c] + sX[1][0][c]) + sX[2][0][c];
                sRed[c] = pa + (sX[0][1][c] + sX[1][1][c]) + sX[2][1][c];
            }
        }
        __syncthreads();
        if (t == 0) {
            float s = 0.f;
            for (int cc = 0; cc < KDA_DK; cc++) s += sRed[cc];
            part[item * KDA_BWD_PART_FLOATS + KDA_DK] = s;
        }

        /* s11: through the L2 norms; thread t: row t / 8, channels 32 m + 4 (t % 8) + [0, 4)
         * for m < 4 (16-byte pieces of the scratch rows) */
        {
            const int i = t >> 3, q8 = t & 7;
            float xq[4][4], xk[4][4];
            float sq = 0.f, sk = 0.f, sb = 0.f;
            if (i < L) {
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    const int e = i * KDA_DK + 32 * m + 4 * q8;
                    const float4 fq = *(const float4 *)(dqn + e), fk = *(const float4 *)(dkn + e);
                    const float4 fb = *(const float4 *)(XU + e);
                    xq[m][0] = fq.x; xq[m][1] = fq.y; xq[m][2] = fq.z; xq[m][3] = fq.w;
                    xk[m][0] = fk.x; xk[m][1] = fk.y; xk[m][2] = fk.z; xk[m][3] = fk.w;
                    sb += (fb.x + fb.y) + (fb.z + fb.w);
                }
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        const int cc = 32 * m + 4 * q8 + u;
                        sq = fmaf(sQ[i * LDK + cc], xq[m][u], sq);
                        sk = fmaf(sK[i * LDK + cc], xk[m][u], sk);
                    }
            }
            /* xor butterflies over the row's 8 lanes: every lane adds the same pairs
             * (deterministic) */
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) {
                sq += __shfl_xor(sq, o);
                sk += __shfl_xor(sk, o);
                sb += __shfl_xor(sb, o);
            }
            if (i < L) {
                const float inq = 1.f / R[KDA_BR_NQ + i], ink = 1.f / R[KDA_BR_NK + i];
                const int64_t row = ((t0 + i) * H + h) * KDA_DK;
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        const int cc = 32 * m + 4 * q8 + u;
                        dq[row + cc] = (xq[m][u] - sQ[i * LDK + cc] * sq) * inq;
                        dk[row + cc] = (xk[m][u] - sK[i * LDK + cc] * sk) * ink;
                    }
                if (q8 == 0) dbeta[(t0 + i) * H + h] = sb;
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
        hipLaunchKernelGGL(kda_bwd_chunk_kernel, dim3((unsigned)items), dim3(NTG), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)g,
                           (const uint16_t *)beta, A_log, dt_bias, scale, lower_bound, cu, chunk_off, nseq, T,
                           (int)H, nslots, brec);
        break;
    case 1:
        hipLaunchKernelGGL(kda_bwd_scan_kernel, dim3((unsigned)((nseq * H + 7) / 8 * 64)), dim3(NT), 0, st, brec, cu,
                           chunk_off, nseq, T, (int)H, nslots, init, init_fp32, dfinal, (const uint16_t *)dout,
                           ckpt, dse, dinit);
        break;
    case 2:
        hipLaunchKernelGGL(kda_bwd_grad_kernel, dim3((unsigned)kda_bwd_grad_wgs(items)), dim3(NTG), 0, st,
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
