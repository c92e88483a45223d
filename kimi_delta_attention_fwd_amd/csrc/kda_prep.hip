/*
 * kda_prep.hip -- gfx950 kernels of the chunked Kimi Delta Attention forward:
 *
 *   kda_chunk_map_kernel : varlen chunk table (prefix sum of ceil(len / 64)).
 *   kda_prep_kernel      : one workgroup per (chunk, head); gate, q/k L2 norm,
 *                          in-chunk cumsum, tril A and P, T = (I + A)^-1 by
 *                          forward substitution in LDS, W, U, Q', K~^T.
 *
 * The operation is the gated delta rule of the FlashKDA pages (ccm-staging
 * page, "Core Kernel API / flash_kda.fwd"; trend.ondo.sh page, "Kernel API and
 * Constraints"); the chunk algebra and the record layout are described in
 * kda_internal.h. Exponentials are taken base 2 (v_exp_f32) on log2-scaled sums.
 */
#include "kda.h"
#include "kda_device.h"

/* ------------------------------------------------------------------------- */
/* varlen chunk table: chunk_off[n] = sum_{m < n} ceil(len_m / 64), then the  */
/* count and the ascending indices of sequences of more than                  */
/* KDA_MANY_MAX_CHUNKS chunks (long_list[0] = count, long_list[1 + i]); the   */
/* list holds max_long entries, which valid cu_seqlens never exceed            */
/* ------------------------------------------------------------------------- */
extern "C" __global__ void __launch_bounds__(1024)
kda_chunk_map_kernel(const int32_t *__restrict__ cu, int64_t nseq, int32_t *__restrict__ chunk_off,
                     int64_t max_long)
{
    __shared__ int32_t s_wave[16], s_wave_l[16];
    __shared__ int32_t s_carry, s_carry_l;
    int32_t *long_list = chunk_off + nseq + 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) { s_carry = 0; s_carry_l = 0; chunk_off[0] = 0; }
    __syncthreads();
    for (int64_t base = 0; base < nseq; base += 1024) {
        const int64_t n = base + tid;
        int32_t x = 0, f = 0;
        if (n < nseq) {
            const int32_t len = cu[n + 1] - cu[n];
            x = (len + KDA_CHUNK - 1) / KDA_CHUNK;
            f = x > KDA_MANY_MAX_CHUNKS;
        }
        const int32_t f0 = f;
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t y = __shfl_up(x, d), yf = __shfl_up(f, d);
            if (lane >= d) { x += y; f += yf; }
        }
        if (lane == 63) { s_wave[wave] = x; s_wave_l[wave] = f; }
        __syncthreads();
        int32_t add = s_carry, add_l = s_carry_l;
        for (int w = 0; w < wave; w++) { add += s_wave[w]; add_l += s_wave_l[w]; }
        if (n < nseq) chunk_off[n + 1] = add + x;
        if (f0 && add_l + f - 1 < max_long) long_list[1 + add_l + f - 1] = (int32_t)n;
        __syncthreads();
        if (tid == 1023) { s_carry = add + x; s_carry_l = add_l + f; }
        __syncthreads();
    }
    if (tid == 0) long_list[0] = (int32_t)(s_carry_l < max_long ? s_carry_l : max_long);
}

/* ------------------------------------------------------------------------- */
/* prep: one workgroup of 4 waves per (chunk slot, head)                       */
/* ------------------------------------------------------------------------- */
/*
 * Wave w owns tokens 16 w .. 16 w + 15 of the chunk (sub-chunk w); lane l holds
 * token 16 w + l % 16 and the 32 key channels 32 kb + 8 (l / 16) + i, i < 8
 * (natural order: the loads are 16 bytes per lane; where an operand must be in
 * the accumulator-pair order kperm, a 0/1 selector MFMA reorders it).
 *
 * Decay factors (log2 units; c = in-sub-chunk inclusive cumsum, m_w = c at the
 * sub-chunk's 8th token, B_w = G before sub-chunk w, Gm_w = B_w + m_w):
 *   diagonal block w:   (k^ 2^{c - m_w}) . (k^ 2^{m_w - c})          |exp| <= 8 |lb|
 *   block (i, b < i):   (k^ 2^{c - m_i} 2^{m_i}) . (k^ 2^{m_b - c} 2^{B_i - Gm_b})
 *                       both sides <= 1 (anchored at the start of sub-chunk i), so a
 *                       factor only underflows where the pairwise decay is negligible
 *   Q~ = q^ 2^{G} = (q^ 2^{c - m_w}) 2^{Gm_w},   R = k^ 2^{G} likewise,
 *   K~ = k^ 2^{G_L - G} = (k^ 2^{m_w - c}) 2^{G_L - Gm_w}.
 * beta enters through A's rows and through T's columns (TB = T diag(beta)):
 * W = TB (K^ o e^G), U = TB V.
 */
#define KDA_TS 68 /* row stride (floats) of the fp32 64x64 tiles: 16-byte rows, rows spread over the banks */

/* DK = 32 NKB key channels, DV = 32 NVB value columns */
template <int NKB, int NVB> struct PrepShared {
    float beta[KDA_CHUNK];
    union {
        struct { /* phases A-D */
            float tot[4][32 * NKB]; /* in-sub-chunk inclusive cumsum at token 15 (log2)  */
            float mid[4][32 * NKB]; /* ... at token 7 (the anchor m_w)                    */
            float fq[4][32 * NKB];  /* 2^{Gm_w}                                           */
            float fk[4][32 * NKB];  /* 2^{G_L - Gm_w}                                     */
            float fm[4][32 * NKB];  /* 2^{m_w}                                            */
            float fy[6][32 * NKB];  /* 2^{B_i - Gm_b}, pair (i, b) -> i (i - 1) / 2 + b     */
            bf16x8 yd[4][NKB][64];  /* diagonal key side k^ 2^{m_w - c}, per sub-chunk    */
        } p1;
        struct { /* phases E-F */
            float t[KDA_CHUNK][KDA_TS]; /* T = (I + A)^-1, blocks on or below the diagonal */
            bf16x8 tbt[6][64];          /* (T diag(beta))^T fragments, index kda_tbt_idx  */
        } p2;
    } u;
    bf16x8 rt[2 * NKB][2][64];  /* R^T fragments (key tile, token block)                 */
    bf16x8 vt[2 * NVB][2][64];  /* V^T fragments (value tile, token block)               */
    float a[KDA_CHUNK][KDA_TS]; /* A (strictly lower; beta_r on row r)                 */
};

/* (T diag(beta))^T fragment (column block jt, row block pair jb): lane = column
   16 jt + l % 16, 8 values over rows 32 jb + kperm(l / 16, i); only jb >= jt / 2 is
   nonzero */
__device__ __forceinline__ int kda_tbt_idx(int jt, int jb) { return jt < 2 ? 2 * jt + jb : 2 + jt; }

/* lane N of each 16-lane row of the wave, to the whole row (DPP row_newbcast) */
template <int N> __device__ __forceinline__ float row_bcast(float x)
{
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, false));
}

/* wide form's diagonal block: this lane's partial sums over its channels against
   partner token JJ .. 15 of its row (lane 16 g + JJ holds the partner's values of
   the same channels), the decay exp2 of a clamped log2 difference */
template <int JJ> struct WidePartners {
    static __device__ __forceinline__ void add(float kh, float qh, float c, float (&sa)[16], float (&sp)[16])
    {
        const float kp = row_bcast<JJ>(kh), cp = row_bcast<JJ>(c);
        const float t = kp * exp2_fast(fminf(c - cp, 0.f));
        sa[JJ] += kh * t;
        sp[JJ] += qh * t;
        WidePartners<JJ + 1>::add(kh, qh, c, sa, sp);
    }
};
template <> struct WidePartners<16> {
    static __device__ __forceinline__ void add(float, float, float, float (&)[16], float (&)[16]) {}
};

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

/* R-form fragment (lane = token, 8 values over a 32-wide block) -> C-form 16x16 tile
   (lane = column of the block, 4 regs = tokens 4 g + e) with a 0/1 selector MFMA */
__device__ __forceinline__ void store_transposed(const bf16x8 &fr, const bf16x8 (&sel)[2], uint16_t *dst0,
                                                 uint16_t *dst1)
{
    const f32x4 d0 = mfma(fr, sel[0], zero4());
    const f32x4 d1 = mfma(fr, sel[1], zero4());
    uint2 u0, u1;
    u0.x = pack_bf16x2(d0[0], d0[1]);
    u0.y = pack_bf16x2(d0[2], d0[3]);
    u1.x = pack_bf16x2(d1[0], d1[1]);
    u1.y = pack_bf16x2(d1[2], d1[3]);
    *(uint2 *)dst0 = u0;
    *(uint2 *)dst1 = u1;
}

/* The prep body. WIDE (lower_bound below KDA_LOWER_BOUND_NARROW) builds every
   decay factor from exponents <= 0 and evaluates the 16x16 diagonal blocks of A
   and P element by element, so no factor overflows for any lower_bound:
     row sides k^ 2^{c}, q^ 2^{c};  Q~ = q^ 2^{B_w + c},  R = k^ 2^{B_w + c};
     K~ = k^ 2^{G_L - B_w - c};  off-diagonal key side k^ 2^{tot_w - c} 2^{B_i - B_{b+1}};
     diagonal (r, j <= r): sum_c k^_r k^_j 2^{min(c_r - c_j, 0)} (partner token j's
     values from the lanes of the same channel group).
   (c = in-sub-chunk inclusive cumsum, tot_w = its value at the sub-chunk's last
   row, B_w = G before sub-chunk w, all log2.) */
template <bool WIDE, int NKB, int NVB>
__device__ __forceinline__ void prep_body(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *gt,
                                          const uint16_t *beta, const float *__restrict__ A_log,
                                          const float *__restrict__ dt_bias, float scale, float lower_bound,
                                          const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off,
                                          int64_t nseq, int64_t T, int H, int64_t nslots,
                                          unsigned char *__restrict__ rec_base, int64_t trim_max)
{
    constexpr int DK = 32 * NKB, DV = 32 * NVB, NE = 8 * NKB; /* NE: key channels per lane */
    using RL = RecLayout<NKB, 2 * NVB>;
    __shared__ PrepShared<NKB, NVB> sh;
    const int64_t slot = blockIdx.x / H;
    const int h = (int)(blockIdx.x - slot * H);
    int64_t t0, seq;
    int L;
    if (!locate_chunk(slot, cu, chunk_off, nseq, T, t0, L, seq)) return;
    unsigned char *rec = rec_base + ((size_t)h * nslots + slot) * RL::BYTES;

    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, r16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6); /* wave-uniform: branches on it are scalar */
    const int r = 16 * w + r16;
    const bool valid = r < L;
    /* A partial chunk of a sequence of at most trim_max chunks is scanned by
       the many-chain kernel, which reads the fragments of token tiles past the
       chunk's tokens as zeros without touching memory. Those fragments are
       left unwritten: W, Q' and P of row tile w >= nmt (skip_row), and, when
       L <= 32, K~^T token block 1 and U token tiles 2, 3 (skip_hi). Both
       flags are wave-uniform. */
    bool skip_row = false, skip_hi = false;
    if (L < KDA_CHUNK) {
        const int64_t len = cu == nullptr ? T : (int64_t)cu[seq + 1] - cu[seq];
        if ((len + KDA_CHUNK - 1) / KDA_CHUNK <= trim_max) {
            const int nmt = (L + 15) >> 4;
            skip_row = w >= nmt;
            skip_hi = w >= 2 && nmt <= 2;
        }
    }

    /* ---- phase A: load this lane's token row, norms, gate, cumsum ---- */
    /* Token rows past the chunk end fall outside the descriptors' ranges and load
       as zeros, so every lane loads unconditionally (no branch, no early wait). */
    const size_t act0 = ((size_t)t0 * H + h) * DK; /* element offset of (t0, h, 0) in q, k, g */
    const size_t actv0 = ((size_t)t0 * H + h) * DV; /* ... in v */
    const uint32_t row_bytes = (uint32_t)H * DK * 2, row_bytes_v = (uint32_t)H * DV * 2;
    const uint32_t act_bytes = (uint32_t)(L - 1) * row_bytes + DK * 2;
    const uint32_t act_bytes_v = (uint32_t)(L - 1) * row_bytes_v + DV * 2;
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + act0, act_bytes), rk = buf_rsrc(k + act0, act_bytes);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gt + act0, act_bytes), rv = buf_rsrc(v + actv0, act_bytes_v);
    const __amdgpu_buffer_rsrc_t rb = buf_rsrc(beta + (size_t)t0 * H + h, (uint32_t)(L - 1) * H * 2 + 2);
    const uint32_t voff = (uint32_t)r * row_bytes, voff_v = (uint32_t)r * row_bytes_v;
    float qf[NE], kf[NE], la[NE];
    bf16x8 vfr[NVB];
    const float bt = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)r * H * 2, 0, 0));
    const float decay_rate = __expf(A_log[h]);
    const float lb2 = lower_bound * LOG2E_F;
    /* 16 bytes per lane and tensor: operand slot i of key block kb holds channel
       32 kb + 8 g + i (natural order) */
    u32x4 uqa[NKB], uka[NKB], uga[NKB], uva[NVB];
    static_assert(NKB == NVB || NKB == 2 * NVB || NVB == 2 * NKB, "head dims");
#pragma unroll
    for (int kb = 0; kb < (NKB > NVB ? NKB : NVB); kb++) {
        if (kb < NKB) {
            const uint32_t o = voff + (uint32_t)(32 * kb + 8 * g) * 2;
            uqa[kb] = __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0);
            uka[kb] = __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0);
            uga[kb] = __builtin_amdgcn_raw_buffer_load_b128(rg, o, 0, 0);
        }
        if (kb < NVB)
            uva[kb] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v + (uint32_t)(32 * kb + 8 * g) * 2, 0, 0);
    }
    /* All 17 loads are in flight before any of them is consumed. (The activation
       pointers are deliberately not __restrict__: loads through restrict const
       pointers count as invariant, and the compiler then re-issues some of them
       next to their late first use, which costs a second memory round trip.) */
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < NKB; kb++) {
        const float *dbp = dt_bias + (size_t)h * DK + 32 * kb + 8 * g;
        const float4 db0 = *(const float4 *)dbp, db1 = *(const float4 *)(dbp + 4);
        const float dbs[8] = {db0.x, db0.y, db0.z, db0.w, db1.x, db1.y, db1.z, db1.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int sh16 = (i & 1) * 16, wi = i >> 1;
            const int j = kb * 8 + i;
            qf[j] = bf2f((uint16_t)(uqa[kb][wi] >> sh16));
            kf[j] = bf2f((uint16_t)(uka[kb][wi] >> sh16));
            /* log2 a = max(-exp(A_log) softplus(x) log2(e), lower_bound log2(e)) with
               softplus(x) log2(e) = max(t, 0) + log2(1 + 2^{-|t|}),  t = x log2(e) */
            const float t = (bf2f((uint16_t)(uga[kb][wi] >> sh16)) + dbs[i]) * LOG2E_F;
            const float sp2 = fmaxf(t, 0.f) + log2_fast(1.f + exp2_fast(-fabsf(t)));
            const float l2 = fmaxf(-decay_rate * sp2, lb2);
            la[j] = valid ? l2 : 0.f; /* padded rows: no decay */
        }
    }
    /* v stays in bf16 */
#pragma unroll
    for (int vb = 0; vb < NVB; vb++) vfr[vb] = __builtin_bit_cast(bf16x8, uva[vb]);
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < NE; j++) { sq += qf[j] * qf[j]; sk += kf[j] * kf[j]; }
    sq += __shfl_xor(sq, 16); sq += __shfl_xor(sq, 32);
    sk += __shfl_xor(sk, 16); sk += __shfl_xor(sk, 32);
    const float iq = scale / sqrtf(sq + 1e-6f), ik = 1.f / sqrtf(sk + 1e-6f);
#pragma unroll
    for (int j = 0; j < NE; j++) la[j] = row_scan16(la[j]);
    if (r16 == 7 || r16 == 15) {
        float *dst = (r16 == 15) ? sh.u.p1.tot[w] : sh.u.p1.mid[w];
#pragma unroll
        for (int kb = 0; kb < NKB; kb++) {
            *(float4 *)&dst[32 * kb + 8 * g] = make_float4(la[8 * kb], la[8 * kb + 1], la[8 * kb + 2], la[8 * kb + 3]);
            *(float4 *)&dst[32 * kb + 8 * g + 4] =
                make_float4(la[8 * kb + 4], la[8 * kb + 5], la[8 * kb + 6], la[8 * kb + 7]);
        }
    }
    if (g == 0) sh.beta[r] = bt;
    __syncthreads();

    /* ---- phase B: per (sub-chunk, channel) factors ---- */
    for (int p = tid; p < 4 * DK; p += 256) {
        const int ww = p / DK, ch = p % DK;
        float B = 0.f, GL = 0.f;
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const float tm = sh.u.p1.tot[m][ch];
            if (m < ww) B += tm;
            GL += tm;
        }
        if constexpr (WIDE) { /* log2 values: B_w and G_L - B_w */
            sh.u.p1.fq[ww][ch] = B;
            sh.u.p1.fk[ww][ch] = GL - B;
        } else {
            const float gm = B + sh.u.p1.mid[ww][ch];
            sh.u.p1.fq[ww][ch] = exp2_fast(gm);
            sh.u.p1.fk[ww][ch] = exp2_fast(GL - gm);
            sh.u.p1.fm[ww][ch] = exp2_fast(sh.u.p1.mid[ww][ch]);
        }
        if (ww == 0) ((float *)(rec + RL::GL))[ch] = exp2_fast(GL);
    }
    for (int p = tid; p < 6 * DK; p += 256) {
        const int pp = p / DK, ch = p % DK;
        const int i = pp < 1 ? 1 : (pp < 3 ? 2 : 3);
        const int b = pp - i * (i - 1) / 2;
        float Bi = 0.f, Bb = 0.f;
        for (int m = 0; m < i; m++) {
            const float tm = sh.u.p1.tot[m][ch];
            Bi += tm;
            if (m < b) Bb += tm;
        }
        if constexpr (WIDE) sh.u.p1.fy[pp][ch] = exp2_fast(Bi - (Bb + sh.u.p1.tot[b][ch])); /* 2^{B_i - B_{b+1}} */
        else sh.u.p1.fy[pp][ch] = exp2_fast(Bi - (Bb + sh.u.p1.mid[b][ch]));
    }
    __syncthreads();

    /* ---- phase C: decay-scaled operands (R-form), transposes ---- */
    bf16x8 xdk_f[NKB], xdq_f[NKB], yd_f[NKB], qt_f[NKB], xok_f[NKB], xoq_f[NKB];
    bf16x8 sel[2]; /* 0/1 selectors: slot i of lane group g is channel 8 g + i of a 32-wide block */
    {
#pragma unroll
        for (int hh = 0; hh < 2; hh++)
#pragma unroll
            for (int i = 0; i < 8; i++) sel[hh][i] = (__bf16)(8 * g + i == 16 * hh + r16 ? 1.f : 0.f);
        const int jb = w >> 1, jh = w & 1;
#pragma unroll
        for (int kb = 0; kb < NKB; kb++) {
            bf16x8 rf, kt;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int j = kb * 8 + i;
                const int ch = 32 * kb + 8 * g + i;
                if constexpr (WIDE) {
                    const float c = la[j];
                    const float kh = kf[j] * ik, qh = qf[j] * iq;
                    const float ec = exp2_fast(c), eg = exp2_fast(sh.u.p1.fq[w][ch] + c);
                    const float ek = exp2_fast(sh.u.p1.fk[w][ch] - c), ey = exp2_fast(sh.u.p1.tot[w][ch] - c);
                    xok_f[kb][i] = (__bf16)(kh * ec);
                    xoq_f[kb][i] = (__bf16)(qh * ec);
                    yd_f[kb][i] = (__bf16)(kh * ey);
                    qt_f[kb][i] = (__bf16)(qh * eg);
                    rf[i] = (__bf16)(kh * eg);
                    kt[i] = (__bf16)(kh * ek);
                } else {
                    const float d = la[j] - sh.u.p1.mid[w][ch];
                    const float e1 = exp2_fast(d), e2 = exp2_fast(-d);
                    const float kh = kf[j] * ik;
                    const float xk = kh * e1, xq = qf[j] * iq * e1, ykv = kh * e2;
                    const float fq = sh.u.p1.fq[w][ch], fm = sh.u.p1.fm[w][ch];
                    xok_f[kb][i] = (__bf16)(xk * fm); /* k^ 2^{c}: anchored at the sub-chunk start */
                    xoq_f[kb][i] = (__bf16)(xq * fm);
                    xdk_f[kb][i] = (__bf16)xk;
                    xdq_f[kb][i] = (__bf16)xq;
                    yd_f[kb][i] = (__bf16)ykv;
                    qt_f[kb][i] = (__bf16)(xq * fq);
                    rf[i] = (__bf16)(xk * fq);
                    kt[i] = (__bf16)(ykv * sh.u.p1.fk[w][ch]);
                }
            }
            sh.u.p1.yd[w][kb][l] = yd_f[kb];
            /* key tiles 2 kb and 2 kb + 1 of R, V and K~ */
            store_transposed(rf, sel, (uint16_t *)&sh.rt[2 * kb][jb][l] + 4 * jh,
                             (uint16_t *)&sh.rt[2 * kb + 1][jb][l] + 4 * jh);
            if (kb < NVB)
                store_transposed(vfr[kb], sel, (uint16_t *)&sh.vt[2 * kb][jb][l] + 4 * jh,
                                 (uint16_t *)&sh.vt[2 * kb + 1][jb][l] + 4 * jh);
            if (!skip_hi)
                store_transposed(kt, sel,
                                 (uint16_t *)(rec + RL::KT + ((size_t)((2 * kb) * 2 + jb) * 64 + l) * 16 + jh * 8),
                                 (uint16_t *)(rec + RL::KT + ((size_t)((2 * kb + 1) * 2 + jb) * 64 + l) * 16 + jh * 8));
        }
#pragma unroll
        for (int vb = NKB; vb < NVB; vb++) /* value tiles past the key tiles (DV > DK) */
            store_transposed(vfr[vb], sel, (uint16_t *)&sh.vt[2 * vb][jb][l] + 4 * jh,
                             (uint16_t *)&sh.vt[2 * vb + 1][jb][l] + 4 * jh);
    }
    __syncthreads(); /* yd, rt, vt visible */

    /* ---- phase D: tril A and P for row block w (lane = token r, regs = j) ---- */
    f32x4 at[4], pt[4];
#pragma unroll
    for (int b = 0; b < 4; b++) { at[b] = zero4(); pt[b] = zero4(); }
    {
        f32x4 ad = zero4(), pd = zero4();
        if constexpr (WIDE) {
            /* partial sums over this lane's 32 channels for partner token jj of the
               sub-chunk (lane 16 g + jj holds the same channels), then the sum over
               the 4 channel groups; lane (g, r16) keeps partners 4 g .. 4 g + 3 */
            float sa[16], sp[16];
#pragma unroll
            for (int jj = 0; jj < 16; jj++) { sa[jj] = 0.f; sp[jj] = 0.f; }
#pragma unroll
            for (int j = 0; j < NE; j++) WidePartners<0>::add(kf[j] * ik, qf[j] * iq, la[j], sa, sp);
#pragma unroll
            for (int jj = 0; jj < 16; jj++) {
                sa[jj] += __shfl_xor(sa[jj], 16);
                sa[jj] += __shfl_xor(sa[jj], 32);
                sp[jj] += __shfl_xor(sp[jj], 16);
                sp[jj] += __shfl_xor(sp[jj], 32);
            }
#pragma unroll
            for (int e = 0; e < 4; e++)
#pragma unroll
                for (int jj = 0; jj < 16; jj++)
                    if (jj == 4 * g + e) { ad[e] = sa[jj]; pd[e] = sp[jj]; }
        } else {
#pragma unroll
            for (int kb = 0; kb < NKB; kb++) {
                ad = mfma(yd_f[kb], xdk_f[kb], ad);
                pd = mfma(yd_f[kb], xdq_f[kb], pd);
            }
        }
        for (int b = 0; b < w; b++) {
            /* key side k^_j 2^{m_b - c_j} 2^{B_w - Gm_b} = k^_j 2^{B_w - G_j} <= 1 */
            const float *fy = sh.u.p1.fy[w * (w - 1) / 2 + b];
            f32x4 ta = zero4(), tp = zero4();
#pragma unroll
            for (int kb = 0; kb < NKB; kb++) {
                const bf16x8 yb = sh.u.p1.yd[b][kb][l];
                bf16x8 ys;
#pragma unroll
                for (int i = 0; i < 8; i++) ys[i] = (__bf16)((float)yb[i] * fy[32 * kb + 8 * g + i]);
                ta = mfma(ys, xok_f[kb], ta);
                tp = mfma(ys, xoq_f[kb], tp);
            }
#pragma unroll
            for (int bb = 0; bb < 4; bb++)
                if (bb == b) { at[bb] = ta; pt[bb] = tp; }
        }
        /* masks (select, never multiply: masked entries may be inf/nan) */
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int jj = 4 * g + e;
            const float av = ad[e] * bt;
            ad[e] = (jj < r16) ? av : 0.f;
            pd[e] = (jj <= r16) ? pd[e] : 0.f;
        }
#pragma unroll
        for (int bb = 0; bb < 4; bb++)
            if (bb == w) { at[bb] = ad; pt[bb] = pd; }
    }
#pragma unroll
    for (int b = 0; b < 4; b++) {
        if (b < w) {
#pragma unroll
            for (int e = 0; e < 4; e++) at[b][e] *= bt;
        }
        *(float4 *)&sh.a[r][16 * b + 4 * g] = make_float4(at[b][0], at[b][1], at[b][2], at[b][3]);
    }
    bf16x8 pf[2];
    pf[0] = pack8(pt[0], pt[1]);
    pf[1] = pack8(pt[2], pt[3]);
    if (!skip_row) {
        bf16x8 *pdst = (bf16x8 *)(rec + RL::P);
        if (w < 2) {
            pdst[KDA_PIDX(w, 0) * 64 + l] = pf[0];
        } else {
            pdst[(2 + 2 * (w - 2)) * 64 + l] = pf[0];
            pdst[(2 + 2 * (w - 2) + 1) * 64 + l] = pf[1];
        }
    }
    __syncthreads(); /* A visible; p1 (tot/mid/yd) dead from here on */

    /* ---- phase E: T = (I + A)^-1 in fp32 ---- */
    float(*tt)[KDA_TS] = sh.u.p2.t;
    {
        /* 16x16 diagonal blocks by forward substitution (column c per lane) */
        const int c = r16;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; rr++) {
            float acc = (rr == c) ? 1.f : 0.f;
#pragma unroll
            for (int jj = 0; jj < rr; jj++) acc -= sh.a[16 * w + rr][16 * w + jj] * x[jj];
            x[rr] = acc;
        }
        if (g == 0) {
#pragma unroll
            for (int rr = 0; rr < 16; rr++) tt[16 * w + rr][16 * w + c] = x[rr];
        }
    }
    __syncthreads();
    /* Block column w below the diagonal, by block forward substitution with fp32
       MFMAs: T_iw = -T_ii sum_{w <= k < i} A_ik T_kw. Blocks are held in the 16x16
       accumulator layout (lane = column, 4 registers = rows 4 g + e), which is also
       the B-operand layout when the contraction index is split as 4 g + s over the
       4 steps s; A operands are rows of A and T_ii read 4 at a time from LDS. */
    {
        f32x4 tb[4];
#pragma unroll
        for (int e = 0; e < 4; e++) tb[w][e] = tt[16 * w + 4 * g + e][16 * w + r16];
#pragma unroll
        for (int i = 1; i < 4; i++) {
            if (i <= w) continue;
            f32x4 xs = zero4();
#pragma unroll
            for (int kk = 0; kk < i; kk++) {
                if (kk < w) continue;
                const float4 av = *(const float4 *)&sh.a[16 * i + r16][16 * kk + 4 * g];
                xs = mfma_f32(av.x, tb[kk][0], xs);
                xs = mfma_f32(av.y, tb[kk][1], xs);
                xs = mfma_f32(av.z, tb[kk][2], xs);
                xs = mfma_f32(av.w, tb[kk][3], xs);
            }
            const float4 tv = *(const float4 *)&tt[16 * i + r16][16 * i + 4 * g];
            f32x4 y = zero4();
            y = mfma_f32(tv.x, xs[0], y);
            y = mfma_f32(tv.y, xs[1], y);
            y = mfma_f32(tv.z, xs[2], y);
            y = mfma_f32(tv.w, xs[3], y);
            tb[i] = -y;
        }
        /* off-diagonal blocks to LDS (rows of T for the W and U operands) */
#pragma unroll
        for (int i = 1; i < 4; i++) {
            if (i <= w) continue;
#pragma unroll
            for (int e = 0; e < 4; e++) tt[16 * i + 4 * g + e][16 * w + r16] = tb[i][e];
        }
        /* (T diag(beta))^T fragments of column block w; blocks above the diagonal are 0 */
        const float bj = sh.beta[16 * w + r16];
#pragma unroll
        for (int jb = 0; jb < 2; jb++) {
            if (jb < (w >> 1)) continue;
            f32x4 lo = zero4(), hi = zero4();
            if (2 * jb >= w) lo = tb[2 * jb] * bj;
            if (2 * jb + 1 >= w) hi = tb[2 * jb + 1] * bj;
            sh.u.p2.tbt[kda_tbt_idx(w, jb)][l] = pack8(lo, hi);
        }
    }
    __syncthreads();

    /* ---- phase F: TB = T diag(beta); W, U, P TB and Q' for row block w ---- */
    const int nkb = (w >= 2) ? 2 : 1; /* token blocks holding j <= 16 w + 15 */
    bf16x8 tbf[2];
#pragma unroll
    for (int jb = 0; jb < 2; jb++) {
        if (jb >= nkb) { tbf[jb] = pack8(zero4(), zero4()); continue; }
        const int j0 = 32 * jb + 4 * g, j1 = j0 + 16;
        const float4 t0v = *(const float4 *)&tt[r][j0], t1v = *(const float4 *)&tt[r][j1];
        const float4 b0v = *(const float4 *)&sh.beta[j0], b1v = *(const float4 *)&sh.beta[j1];
        const float tv[8] = {t0v.x * b0v.x, t0v.y * b0v.y, t0v.z * b0v.z, t0v.w * b0v.w,
                             t1v.x * b1v.x, t1v.y * b1v.y, t1v.z * b1v.z, t1v.w * b1v.w};
#pragma unroll
        for (int i = 0; i < 8; i++) tbf[jb][i] = (__bf16)((32 * jb + kperm(g, i) <= r) ? tv[i] : 0.f);
    }
    /* W (stored negated), lane = token, regs = key channel */
#pragma unroll
    for (int kb = 0; kb < NKB; kb++) {
        if (skip_row) break;
        f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
        for (int jb = 0; jb < 2; jb++)
            if (jb < nkb) {
                d0 = mfma(sh.rt[2 * kb][jb][l], tbf[jb], d0);
                d1 = mfma(sh.rt[2 * kb + 1][jb][l], tbf[jb], d1);
            }
        ((bf16x8 *)(rec + RL::W))[(w * NKB + kb) * 64 + l] = pack8(-d0, -d1);
    }
    /* U, lane = value column, regs = token */
#pragma unroll
    for (int nt = 0; nt < 2 * NVB; nt++) {
        if (skip_hi) break;
        f32x4 d = zero4();
#pragma unroll
        for (int jb = 0; jb < 2; jb++)
            if (jb < nkb) d = mfma(tbf[jb], sh.vt[nt][jb][l], d);
        uint2 u;
        u.x = pack_bf16x2(d[0], d[1]);
        u.y = pack_bf16x2(d[2], d[3]);
        *(uint2 *)(rec + RL::U + ((size_t)(nt * 64 + l) * 16 + w * 4) * 2) = u;
    }
    if (skip_row) return;
    /* P TB, lane = token r, regs = j' */
    f32x4 ptt[4];
#pragma unroll
    for (int jt = 0; jt < 4; jt++) {
        ptt[jt] = zero4();
        if (jt > w) continue;
#pragma unroll
        for (int jb = 0; jb < 2; jb++) {
            if (jb >= nkb || jb < (jt >> 1)) continue;
            ptt[jt] = mfma(sh.u.p2.tbt[kda_tbt_idx(jt, jb)][l], pf[jb], ptt[jt]);
        }
    }
    bf16x8 ptf[2];
    ptf[0] = pack8(-ptt[0], -ptt[1]);
    ptf[1] = pack8(-ptt[2], -ptt[3]);
    /* Q' = Q~ - (P TB) R, lane = token, regs = key channel */
#pragma unroll
    for (int kb = 0; kb < NKB; kb++) {
        /* Q~ into the accumulator layout (rows = channels 32 kb + 16 hh + 4 g + e,
           column = token) by 0/1 selector MFMAs (exact) */
        f32x4 d0 = mfma(sel[0], qt_f[kb], zero4()), d1 = mfma(sel[1], qt_f[kb], zero4());
#pragma unroll
        for (int jb = 0; jb < 2; jb++)
            if (jb < nkb) {
                d0 = mfma(sh.rt[2 * kb][jb][l], ptf[jb], d0);
                d1 = mfma(sh.rt[2 * kb + 1][jb][l], ptf[jb], d1);
            }
        ((bf16x8 *)(rec + RL::Q))[(w * NKB + kb) * 64 + l] = pack8(d0, d1);
    }
}

#define KDA_PREP_KERNEL(name, WIDE, NKB, NVB)                                                                      \
    extern "C" __global__ void __launch_bounds__(256, 2)                                                            \
        name(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *gt, const uint16_t *beta,     \
             const float *__restrict__ A_log, const float *__restrict__ dt_bias, float scale, float lower_bound,     \
             const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H,  \
             int64_t nslots, unsigned char *__restrict__ rec_base, int64_t trim_max)                              \
    {                                                                                                               \
        prep_body<WIDE, NKB, NVB>(q, k, v, gt, beta, A_log, dt_bias, scale, lower_bound, cu, chunk_off, nseq, T, H, \
                                  nslots, rec_base, trim_max);                                                      \
    }

/* K = V = 128; the wide form below lower_bound KDA_LOWER_BOUND_NARROW */
KDA_PREP_KERNEL(kda_prep_kernel, false, 4, 4)
KDA_PREP_KERNEL(kda_prep_wide_kernel, true, 4, 4)
/* K = V = 64 */
KDA_PREP_KERNEL(kda_prep_k64_kernel, false, 2, 2)
KDA_PREP_KERNEL(kda_prep_wide_k64_kernel, true, 2, 2)

/* ------------------------------------------------------------------------- */
/* launchers (called by kda_api.cpp after validation)                          */
/* ------------------------------------------------------------------------- */
extern "C" hipError_t kda_launch_chunk_map(const int32_t *cu, int64_t nseq, int64_t T, int32_t *chunk_off,
                                           hipStream_t st)
{
    hipLaunchKernelGGL(kda_chunk_map_kernel, dim3(1), dim3(1024), 0, st, cu, nseq, chunk_off, kda_max_long_seqs(T));
    return hipGetLastError();
}

extern "C" hipError_t kda_launch_prep(const void *q, const void *k, const void *v, const void *g,
                                      const void *beta, const float *A_log, const float *dt_bias,
                                      float scale, float lower_bound, const int32_t *cu,
                                      const int32_t *chunk_off, int64_t nseq, int64_t T, int64_t H,
                                      int64_t nslots, int64_t K, int64_t V, void *records, int64_t trim_max,
                                      hipStream_t st)
{
    const int64_t blocks = nslots * H;
    const bool wide = lower_bound < KDA_LOWER_BOUND_NARROW;
    auto kern = wide ? kda_prep_wide_kernel : kda_prep_kernel;
    if (K == 64 && V == 64) kern = wide ? kda_prep_wide_k64_kernel : kda_prep_k64_kernel;
    else if (K != KDA_DK || V != KDA_DV) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern,
                       dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v,
                       (const uint16_t *)g, (const uint16_t *)beta, A_log, dt_bias, scale,
                       lower_bound, cu, chunk_off, nseq, T, (int)H, nslots, (unsigned char *)records, trim_max);
    return hipGetLastError();
}

