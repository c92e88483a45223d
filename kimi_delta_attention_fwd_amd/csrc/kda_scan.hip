/*
 * kda_scan.hip -- gfx950 scan kernel of the chunked Kimi Delta Attention
 * forward: the sequential chunk loop per (sequence, head, 16 value columns)
 * with the fp32 state slice in MFMA accumulators. The records it consumes are
 * produced by kda_prep_kernel (layout in kda_internal.h).
 */
#include "kda_device.h"

/* ------------------------------------------------------------------------- */
/* scan: one workgroup of 3 waves per (sequence, head, 16-column value tile)   */
/* ------------------------------------------------------------------------- */
/*
 * wave 0 (state):  D = U - W S and S <- diag(e^{G_L}) S + K~^T D; the fp32 state
 *                  slice (128 key rows x 16 value columns) lives in its MFMA
 *                  accumulators.
 * wave 1 (output): out = Q' S + P U from the bf16 copy of the chunk's entering
 *                  state that wave 0 leaves in a two-slot LDS ring.
 * wave 2 (L2 warm): touches its eighth of the record four chunks ahead with
 *                  LDS-DMA loads into a scratch LDS buffer, so that the eight
 *                  workgroups of a chain find their records in L2.
 * The three waves meet at one barrier per chunk. Waves 0 and 1 double-buffer
 * their record operands in registers: all loads for chunk c + 1 are issued at
 * the start of chunk c (two register sets alternate over a two-chunk unroll).
 * Records and out are accessed through buffer descriptors (SGPR base per chunk,
 * one lane offset), which keeps address arithmetic off the vector ALU.
 * The warming loads are issued through inline assembly, so the compiler does
 * not track them and no wave ever waits for them, except wave 2 once before it
 * exits (its LDS must not be released with DMA writes in flight).
 */
struct ScanSetS {
    bf16x8 W[16], K[16], U[2];
    f32x4 gl[8]; /* e^{G_L} for key rows 16 mt + 4 g + e */
};
struct ScanSetO {
    bf16x8 Q[16], P[6], U[2];
};

/* buffer descriptor over one chunk record: SGPR base, lane offsets in VGPRs */
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_rsrc(const unsigned char *rec)
{
    return buf_rsrc(rec, KDA_REC_BYTES);
}

__device__ __forceinline__ bf16x8 bufld(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ void load_set(ScanSetS &X, const unsigned char *rec, int ubase, int l, int g)
{
    const __amdgpu_buffer_rsrc_t r = rec_rsrc(rec);
#pragma unroll
    for (int f = 0; f < 16; f++) X.W[f] = bufld(r, l * 16, KDA_REC_W + f * 1024);
    X.U[0] = bufld(r, l * 32, ubase);
    X.U[1] = bufld(r, l * 32, ubase + 16);
#pragma unroll
    for (int mt = 0; mt < 8; mt++)
        X.gl[mt] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, g * 16, KDA_REC_GL + mt * 64, 0));
#pragma unroll
    for (int f = 0; f < 16; f++) X.K[f] = bufld(r, l * 16, KDA_REC_KT + f * 1024);
}

__device__ __forceinline__ void load_set(ScanSetO &X, const unsigned char *rec, int ubase, int l, int g)
{
    const __amdgpu_buffer_rsrc_t r = rec_rsrc(rec);
#pragma unroll
    for (int f = 0; f < 16; f++) X.Q[f] = bufld(r, l * 16, KDA_REC_Q + f * 1024);
#pragma unroll
    for (int f = 0; f < 6; f++) X.P[f] = bufld(r, l * 16, KDA_REC_P + f * 1024);
    X.U[0] = bufld(r, l * 32, ubase);
    X.U[1] = bufld(r, l * 32, ubase + 16);
}

__device__ __forceinline__ void chunk_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

/* state wave: X holds chunk c; loads chunk c + 1 (at nrec) into Y */
__device__ __forceinline__ void state_step(ScanSetS &X, ScanSetS &Y, f32x4 (&S)[8], const unsigned char *nrec,
                                           int ubase, bf16x8 *slot, int l, int g)
{
    load_set(Y, nrec, ubase, l, g);
    bf16x8 sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
        sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
        slot[kb * 64 + l] = sb[kb];
    }
    chunk_barrier();
    f32x4 D[4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        const int o = (mt & 1) * 4;
        const bf16x8 &u = X.U[mt >> 1];
        D[mt] = f32x4{(float)u[o], (float)u[o + 1], (float)u[o + 2], (float)u[o + 3]};
    }
    /* D = U - W S */
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int mt = 0; mt < 4; mt++) D[mt] = mfma(X.W[mt * 4 + kb], sb[kb], D[mt]);
    /* S <- diag(e^{G_L}) S + K~^T D */
#pragma unroll
    for (int mt = 0; mt < 8; mt++) S[mt] *= X.gl[mt];
    bf16x8 db[2];
    db[0] = pack8(D[0], D[1]);
    db[1] = pack8(D[2], D[3]);
#pragma unroll
    for (int jb = 0; jb < 2; jb++)
#pragma unroll
        for (int mt = 0; mt < 8; mt++) S[mt] = mfma(X.K[mt * 2 + jb], db[jb], S[mt]);
}

/* output wave: X holds chunk c (tokens t0 .. t0 + L - 1); loads chunk c + 1 into Y.
   out is written through a buffer descriptor bounded at row L - 1: rows past
   the sequence end fall outside it and the hardware drops their stores. */
__device__ __forceinline__ void output_step(ScanSetO &X, ScanSetO &Y, const unsigned char *nrec, int ubase,
                                            const bf16x8 *slot, uint16_t *out, int64_t t0, int L, int H,
                                            int h, int nt, int l, int g, int n16)
{
    load_set(Y, nrec, ubase, l, g);
    chunk_barrier();
    bf16x8 sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) sb[kb] = slot[kb * 64 + l];
    /* out^T = S^T Q'^T + U^T P^T   (lane = token, regs = 4 value columns) */
    f32x4 O[4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) O[mt] = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int mt = 0; mt < 4; mt++) O[mt] = mfma(sb[kb], X.Q[mt * 4 + kb], O[mt]);
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int jb = 0; jb <= (mt >> 1); jb++) O[mt] = mfma(X.U[jb], X.P[KDA_PIDX(mt, jb)], O[mt]);
    const int row_bytes = H * KDA_DV * 2;
    const __amdgpu_buffer_rsrc_t ro =
        buf_rsrc(out + ((size_t)t0 * H + h) * KDA_DV, (uint32_t)((L - 1) * row_bytes + KDA_DV * 2));
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        u32x2 u;
        u[0] = f2bf_bits(O[mt][0]) | ((uint32_t)f2bf_bits(O[mt][1]) << 16);
        u[1] = f2bf_bits(O[mt][2]) | ((uint32_t)f2bf_bits(O[mt][3]) << 16);
        __builtin_amdgcn_raw_buffer_store_b64(u, ro, (16 * mt + n16) * row_bytes + (16 * nt + 4 * g) * 2, 0, 0);
    }
}

/* one 1 KiB LDS-DMA load (64 lanes x 16 bytes) that nobody waits for; m0 is not
   otherwise used in this kernel (LDS instructions on gfx9 do not read it) */
__device__ __forceinline__ void warm_l2(const unsigned char *p, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(p), "s"(lds_addr) : "memory", "m0");
}

#define KDA_WARM_AHEAD 4

extern "C" __global__ void __launch_bounds__(192)
kda_scan_kernel(const unsigned char *__restrict__ rec_base, const int32_t *__restrict__ cu,
                const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H, int64_t nslots,
                uint16_t *__restrict__ out, const void *__restrict__ init_state,
                void *__restrict__ final_state, int state_fp32)
{
    __shared__ bf16x8 ring[2][4 * 64];                          /* 8 KiB: S(c) in bf16 */
    __shared__ __attribute__((aligned(16))) unsigned char warm_sink[1024];
    const int wave = threadIdx.x >> 6;
    const int l = threadIdx.x & 63, g = l >> 4, n16 = l & 15;
    /* the 8 value tiles of a chain run on one XCD (blockIdx % 8) and share its L2 */
    const int64_t b = blockIdx.x;
    const int64_t xcd = b & 7, qd = b >> 3;
    const int nt = (int)(qd & 7);
    const int64_t chain = (qd >> 3) * 8 + xcd;
    const int64_t nchain = nseq * H;
    if (chain >= nchain) return;
    const int64_t seq = chain / H;
    const int h = (int)(chain - seq * H);
    const int vcol = 16 * nt + n16;

    int64_t bos, eos, slot0;
    if (cu == nullptr) {
        bos = seq * T;
        eos = bos + T;
        slot0 = seq * ((T + KDA_CHUNK - 1) / KDA_CHUNK);
    } else {
        bos = cu[seq];
        eos = cu[seq + 1];
        slot0 = chunk_off[seq];
    }
    const int64_t nchunk = (eos - bos + KDA_CHUNK - 1) / KDA_CHUNK;
    const unsigned char *rec0 = rec_base + ((size_t)h * nslots + slot0) * KDA_REC_BYTES;
    /* record of chunk c, clamped to the last one (its reload is harmless) */
    auto rec_of = [&](int64_t c) { return rec0 + (size_t)(c < nchunk ? c : nchunk - 1) * KDA_REC_BYTES; };
    const int ubase = KDA_REC_U + nt * 2048; /* this tile's 2 KiB of U; lane l reads 32 bytes */

    if (wave == 0) {
        /* ---------------- state wave ---------------- */
        f32x4 S[8];
        const size_t sbase = (size_t)chain * KDA_DK * KDA_DV;
#pragma unroll
        for (int mt = 0; mt < 8; mt++) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const size_t idx = sbase + (size_t)(16 * mt + 4 * g + e) * KDA_DV + vcol;
                float sv = 0.f;
                if (init_state)
                    sv = state_fp32 ? ((const float *)init_state)[idx] : bf2f(((const uint16_t *)init_state)[idx]);
                S[mt][e] = sv;
            }
        }
        if (nchunk > 0) {
            ScanSetS X, Y;
            int64_t c = 0;
            if (nchunk & 1) {
                load_set(X, rec_of(0), ubase, l, g);
                state_step(X, Y, S, rec_of(1), ubase, ring[0], l, g);
                c = 1;
            } else {
                load_set(Y, rec_of(0), ubase, l, g);
            }
            for (; c < nchunk; c += 2) {
                state_step(Y, X, S, rec_of(c + 1), ubase, ring[c & 1], l, g);
                state_step(X, Y, S, rec_of(c + 2), ubase, ring[(c + 1) & 1], l, g);
            }
        }
        if (final_state) {
            const size_t sbase2 = (size_t)chain * KDA_DK * KDA_DV;
#pragma unroll
            for (int mt = 0; mt < 8; mt++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const size_t idx = sbase2 + (size_t)(16 * mt + 4 * g + e) * KDA_DV + vcol;
                    if (state_fp32) ((float *)final_state)[idx] = S[mt][e];
                    else ((uint16_t *)final_state)[idx] = f2bf_bits(S[mt][e]);
                }
        }
    } else if (wave == 1) {
        /* ---------------- output wave ---------------- */
        if (nchunk > 0) {
            ScanSetO X, Y;
            int64_t c = 0;
            auto t0_of = [&](int64_t cc) { return bos + cc * KDA_CHUNK; };
            auto len_of = [&](int64_t cc) {
                const int64_t rem = eos - t0_of(cc);
                return (int)(rem < KDA_CHUNK ? rem : KDA_CHUNK);
            };
            if (nchunk & 1) {
                load_set(X, rec_of(0), ubase, l, g);
                output_step(X, Y, rec_of(1), ubase, ring[0], out, t0_of(0), len_of(0), H, h, nt, l, g, n16);
                c = 1;
            } else {
                load_set(Y, rec_of(0), ubase, l, g);
            }
            for (; c < nchunk; c += 2) {
                output_step(Y, X, rec_of(c + 1), ubase, ring[c & 1], out, t0_of(c), len_of(c), H, h, nt, l, g,
                            n16);
                output_step(X, Y, rec_of(c + 2), ubase, ring[(c + 1) & 1], out, t0_of(c + 1), len_of(c + 1), H,
                            h, nt, l, g, n16);
            }
        }
    } else {
        /* ---------------- L2-warming wave ---------------- */
        const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)warm_sink;
        for (int64_t c = 0; c < nchunk; c++) {
            const int64_t cw = c + KDA_WARM_AHEAD;
            if (cw < nchunk) {
                const unsigned char *r = rec0 + (size_t)cw * KDA_REC_BYTES;
                /* this tile's eighth of the shared operands, 1 KiB pieces */
                for (int i = nt; i < KDA_REC_U / 1024 + 1; i += 8) warm_l2(r + i * 1024 + l * 16, lds);
                /* and its own 2 KiB of U */
                warm_l2(r + KDA_REC_U + nt * 2048 + l * 16, lds);
                warm_l2(r + KDA_REC_U + nt * 2048 + 1024 + l * 16, lds);
            }
            chunk_barrier();
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

/* ------------------------------------------------------------------------- */
/* launcher (called by kda_api.cpp after validation)                           */
/* ------------------------------------------------------------------------- */
extern "C" hipError_t kda_launch_scan(const void *records, const int32_t *cu, const int32_t *chunk_off,
                                      int64_t nseq, int64_t T, int64_t H, int64_t nslots, void *out,
                                      const void *init_state, void *final_state, int state_fp32,
                                      hipStream_t st)
{
    const int64_t nchain = nseq * H;
    const int64_t blocks = (nchain + 7) / 8 * 64;
    hipLaunchKernelGGL(kda_scan_kernel, dim3((unsigned)blocks), dim3(192), 0, st,
                       (const unsigned char *)records, cu, chunk_off, nseq, T, (int)H, nslots,
                       (uint16_t *)out, init_state, final_state, state_fp32);
    return hipGetLastError();
}
