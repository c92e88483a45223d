/*
 * kda_decode.hip -- gfx950 single-token step of Kimi Delta Attention: one
 * token per sequence, the recurrent state read and written in place. This is
 * the recurrence itself (the FlashKDA pages, "Core Kernel API / flash_kda.fwd"
 * on the ccm-staging page, give the arguments; "Kernel API and Constraints" on
 * the trend.ondo.sh page fixes K = V = 128 and bf16/fp32 states), evaluated
 * without chunking:
 *   a_c = exp(max(-exp(A_log[h]) softplus(g_c + dt_bias[h, c]), lower_bound))
 *   S  <- Diag(a) S;   e = S^T k^;   S <- S + beta k^ (v - e)^T;   out = scale S^T q^
 * with q^, k^ the L2-normalised q, k (eps 1e-6). It is bound by the state
 * traffic: 64 KB read and 64 KB written per (sequence, head) in fp32.
 */
#include "kda_device.h"

/*
 * One workgroup of 256 threads per (sequence, head). Thread (cq = tid / 32,
 * jq = tid % 32) holds state rows 16 cq .. 16 cq + 15, columns 4 jq .. 4 jq + 3
 * in fp32 registers; a wave's load of one row index covers two whole 512-byte
 * state rows. The per-channel vectors (decay, k^, scale q^) are formed by wave 0
 * and shared through LDS; the two reductions over key rows (e and out) go
 * through an 8 x 32 LDS table of partial sums.
 */
extern "C" __global__ void __launch_bounds__(256)
kda_decode_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                  const uint16_t *__restrict__ gt, const uint16_t *__restrict__ beta,
                  const float *__restrict__ A_log, const float *__restrict__ dt_bias, float scale,
                  float lower_bound, void *__restrict__ state, int state_fp32, uint16_t *__restrict__ out, int H)
{
    __shared__ float s_a[KDA_DK], s_k[KDA_DK], s_q[KDA_DK];
    __shared__ f32x4 s_red[8][32];
    const int64_t nh = blockIdx.x; /* n * H + h */
    const int h = (int)(nh % H);
    const int tid = threadIdx.x, jq = tid & 31, cq = tid >> 5, l = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t vec0 = (size_t)nh * KDA_DK;

    /* state tile first: the longest latency */
    f32x4 S[16];
    if (state_fp32) {
        const float *sp = (const float *)state + (size_t)nh * KDA_DK * KDA_DV;
#pragma unroll
        for (int rr = 0; rr < 16; rr++) S[rr] = *(const f32x4 *)&sp[(16 * cq + rr) * KDA_DV + 4 * jq];
    } else {
        const uint16_t *sp = (const uint16_t *)state + (size_t)nh * KDA_DK * KDA_DV;
#pragma unroll
        for (int rr = 0; rr < 16; rr++) {
            const u32x2 u = *(const u32x2 *)&sp[(16 * cq + rr) * KDA_DV + 4 * jq];
            S[rr] = f32x4{bf2f((uint16_t)(u[0] & 0xffff)), bf2f((uint16_t)(u[0] >> 16)),
                          bf2f((uint16_t)(u[1] & 0xffff)), bf2f((uint16_t)(u[1] >> 16))};
        }
    }
    const u32x2 vu = *(const u32x2 *)&v[vec0 + 4 * jq];
    const f32x4 vv = {bf2f((uint16_t)(vu[0] & 0xffff)), bf2f((uint16_t)(vu[0] >> 16)),
                      bf2f((uint16_t)(vu[1] & 0xffff)), bf2f((uint16_t)(vu[1] >> 16))};
    const float bt = bf2f(beta[nh]);

    if (wave == 0) {
        /* lane l: channels 2 l, 2 l + 1 */
        const uint32_t wq = *(const uint32_t *)&q[vec0 + 2 * l];
        const uint32_t wk = *(const uint32_t *)&k[vec0 + 2 * l];
        const uint32_t wg = *(const uint32_t *)&gt[vec0 + 2 * l];
        const float q0 = bf2f((uint16_t)(wq & 0xffff)), q1 = bf2f((uint16_t)(wq >> 16));
        const float k0 = bf2f((uint16_t)(wk & 0xffff)), k1 = bf2f((uint16_t)(wk >> 16));
        float sq = q0 * q0 + q1 * q1, sk = k0 * k0 + k1 * k1;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            sq += __shfl_xor(sq, m);
            sk += __shfl_xor(sk, m);
        }
        const float iq = scale / sqrtf(sq + 1e-6f), ik = 1.f / sqrtf(sk + 1e-6f);
        const float decay_rate = __expf(A_log[h]);
        const float lb2 = lower_bound * LOG2E_F;
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const int c = 2 * l + e;
            /* log2 a = max(-exp(A_log) softplus(x) log2(e), lower_bound log2(e)),
               softplus(x) log2(e) = max(t, 0) + log2(1 + 2^{-|t|}), t = x log2(e) */
            const float t = (bf2f((uint16_t)(e ? (wg >> 16) : (wg & 0xffff))) + dt_bias[(size_t)h * KDA_DK + c]) * LOG2E_F;
            const float sp2 = fmaxf(t, 0.f) + log2_fast(1.f + exp2_fast(-fabsf(t)));
            s_a[c] = exp2_fast(fmaxf(-decay_rate * sp2, lb2));
            s_k[c] = (e ? k1 : k0) * ik;
            s_q[c] = (e ? q1 : q0) * iq;
        }
    }
    __syncthreads();

    /* decay, then e_j = sum_c k^_c S[c][j] over this thread's rows */
    f32x4 pe = zero4();
#pragma unroll
    for (int rr = 0; rr < 16; rr++) {
        const int c = 16 * cq + rr;
        S[rr] *= s_a[c];
        pe += s_k[c] * S[rr];
    }
    s_red[cq][jq] = pe;
    __syncthreads();
    f32x4 e4 = zero4();
#pragma unroll
    for (int i = 0; i < 8; i++) e4 += s_red[i][jq];
    const f32x4 dl = bt * (vv - e4);
    /* write, then out_j = scale sum_c q^_c S[c][j] */
    f32x4 po = zero4();
#pragma unroll
    for (int rr = 0; rr < 16; rr++) {
        const int c = 16 * cq + rr;
        S[rr] += s_k[c] * dl;
        po += s_q[c] * S[rr];
    }
    __syncthreads(); /* every thread has read the e partials */
    s_red[cq][jq] = po;

    if (state_fp32) {
        float *sp = (float *)state + (size_t)nh * KDA_DK * KDA_DV;
#pragma unroll
        for (int rr = 0; rr < 16; rr++) *(f32x4 *)&sp[(16 * cq + rr) * KDA_DV + 4 * jq] = S[rr];
    } else {
        uint16_t *sp = (uint16_t *)state + (size_t)nh * KDA_DK * KDA_DV;
#pragma unroll
        for (int rr = 0; rr < 16; rr++) {
            u32x2 u;
            u[0] = pack_bf16x2(S[rr][0], S[rr][1]);
            u[1] = pack_bf16x2(S[rr][2], S[rr][3]);
            *(u32x2 *)&sp[(16 * cq + rr) * KDA_DV + 4 * jq] = u;
        }
    }
    __syncthreads();
    if (cq == 0) {
        f32x4 o4 = zero4();
#pragma unroll
        for (int i = 0; i < 8; i++) o4 += s_red[i][jq];
        u32x2 u;
        u[0] = pack_bf16x2(o4[0], o4[1]);
        u[1] = pack_bf16x2(o4[2], o4[3]);
        *(u32x2 *)&out[vec0 + 4 * jq] = u;
    }
}

/* launcher (called by kda_api.cpp after validation) */
extern "C" hipError_t kda_launch_decode(const void *q, const void *k, const void *v, const void *g, const void *beta,
                                        const float *A_log, const float *dt_bias, float scale, float lower_bound,
                                        void *state, int state_fp32, void *out, int64_t N, int64_t H, hipStream_t st)
{
    hipLaunchKernelGGL(kda_decode_kernel, dim3((unsigned)(N * H)), dim3(256), 0, st, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)g, (const uint16_t *)beta, A_log,
                       dt_bias, scale, lower_bound, state, state_fp32, (uint16_t *)out, (int)H);
    return hipGetLastError();
}
