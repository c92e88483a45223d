/*
 * kda_scan_pair.hip -- the state scan of the chunked Kimi Delta Attention
 * forward with one workgroup of 6 waves per (chain, pair of 16-column value
 * tiles): four CUs per chain.
 *
 * The operation is the chunk update of kda_internal.h over the records
 * kda_prep_kernel writes (the recurrent state updates the FlashKDA pages
 * describe: ccm-staging page, summary and "Core Kernel API / flash_kda.fwd"):
 *   D = U - W S,  out = Q' S + P U,  S <- diag(e^{G_L}) S + K~^T D,
 * per chain in chunk order, S in fp32, bf16 operands, fp32 accumulation.
 *
 * Why pairs. The chunk's shared operands (W, K~, Q', P: 54 KiB) are the same
 * for every value tile of a chain. With one CU per tile the eight tiles of a
 * chain each pull them from L2, and the scan runs at the aggregate L2-to-CU
 * rate (about 17 TB/s over 256 CUs: 1 us per chunk at 32 chains). Here they
 * cross from L2 to a CU once per pair of tiles and are read from LDS.
 *
 *   waves 0, 1 (state of tile 2 p + w): D = U - W S and the state update, S in
 *        fp32 accumulators; W and K~ from LDS; U and e^{G_L} from memory into
 *        registers one chunk ahead; the bf16 copy of the entering state goes to
 *        a two-slot LDS ring for the output wave of the tile.
 *   waves 2, 3 (output of tile 2 p + w - 2): out = Q' S + P U from the ring, Q'
 *        and P from LDS, U from memory one chunk ahead.
 *   waves 4, 5 (copy): after the barrier of chunk c, LDS-DMA
 *        (global_load_lds_dwordx4) of Q' and P of chunk c + 1 into the two-slot
 *        Q'P ring, then of W and K~ of chunk c + 2 into their three-slot rings,
 *        then L2 warming of the workgroup's quarter of the record KDA_PAIR_WARM
 *        chunks ahead (one 4-byte load per 128-byte line); each then waits until
 *        only the chunk c + 2 copies and the warming are outstanding, so that
 *        everything chunk c + 1 needs has landed before its barrier (loads
 *        complete in issue order).
 * One barrier per chunk; a slot is refilled only after the barrier that ends
 * its last reader's chunk. Chunk indices past a sequence's end are clamped to
 * its last chunk, so every chunk issues the same copies and waits.
 * The arithmetic and its order are the three-wave kernel's (kda_scan.hip), so
 * both give the same bits.
 */
#include "kda_device.h"

#define KDA_PQP_BYTES (16384 + 6144)  /* Q' (16 fragments) then P (6)            */
#define KDA_PAIR_WARM 4               /* L2 warming distance (chunks)            */
#define KDA_PWARM_RANGE 18048         /* a quarter of a record: 141 lines        */
/* copies per chunk and copy wave: 11 of Q'P (1 KiB each), 8 of W, 8 of K~, and
   2 (wave 4) or 1 (wave 5) warming loads */
#define KDA_PCP_QP 11
#define KDA_PCP0_TAIL (8 + 8 + 2) /* issued after the Q'P copies of a round */
#define KDA_PCP1_TAIL (8 + 8 + 1)
static_assert(2 * KDA_PCP_QP == 22, "Q' and P are 22 KiB");
static_assert(4 * KDA_PWARM_RANGE >= KDA_REC_BYTES && KDA_PWARM_RANGE % 128 == 0, "warming ranges cover a record");
static_assert(2 * KDA_PCP0_TAIL + KDA_PCP_QP < 63, "copies in flight within the vmcnt range");

/* one 1 KiB LDS-DMA copy (lane l: 16 bytes to lds_addr + 16 l); lds_addr is the
   same in every lane (an SGPR operand). The compiler keeps nothing of its own in
   m0 in this file (checked on the generated code by tests/test_isa_guards.py). */
__device__ __forceinline__ void pair_copy(const unsigned char *p, uint32_t lds_addr)
{
    const uint32_t a = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(p), "s"(a) : "memory", "m0");
}

/* one 4-byte LDS-DMA load per lane (touches 64 lines of 128 B) */
__device__ __forceinline__ void pair_touch(const unsigned char *p, uint32_t lds_addr)
{
    const uint32_t a = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(p), "s"(a) : "memory", "m0");
}

template <int N> __device__ __forceinline__ void pair_wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void pair_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ uint32_t lds_u32(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char *)p;
}

__device__ __forceinline__ bf16x8 lds_frag(const unsigned char *base, int off)
{
    return *(const bf16x8 *)(base + off);
}

struct PairNext {
    bf16x8 U[2];
    f32x4 gl[8];
};

/* the tile's U (and, for the state wave, e^{G_L}) of the chunk at rec */
template <bool WITH_GL>
__device__ __forceinline__ void pair_load_next(PairNext &X, const unsigned char *rec, int nt, int l, int g)
{
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(rec, KDA_REC_BYTES);
    X.U[0] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, l * 32, KDA_REC_U + nt * 2048, 0));
    X.U[1] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, l * 32, KDA_REC_U + nt * 2048 + 16, 0));
    if (WITH_GL) {
#pragma unroll
        for (int mt = 0; mt < 8; mt++)
            X.gl[mt] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, g * 16, KDA_REC_GL + mt * 64, 0));
    }
}

/* state wave, chunk c: X holds U and e^{G_L} of chunk c, Y receives those of
   chunk c + 1 (nrec); ws / ks: the W / K~ slots of chunk c; ring: the slot of
   chunk c */
__device__ __forceinline__ void pair_state_step(const PairNext &X, PairNext &Y, f32x4 (&S)[8],
                                                const unsigned char *nrec, const unsigned char *ws,
                                                const unsigned char *ks, bf16x8 *ring, int nt, int l, int g)
{
    pair_load_next<true>(Y, nrec, nt, l, g);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
        sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
        ring[kb * 64 + l] = sb[kb];
    }
    pair_barrier();
    bf16x8 W[16];
#pragma unroll
    for (int f = 0; f < 16; f++) W[f] = lds_frag(ws, f * 1024 + l * 16);
    __builtin_amdgcn_sched_barrier(0);
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
        for (int mt = 0; mt < 4; mt++) D[mt] = mfma(W[mt * 4 + kb], sb[kb], D[mt]);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 kt[16];
#pragma unroll
    for (int f = 0; f < 16; f++) kt[f] = lds_frag(ks, f * 1024 + l * 16);
    /* S <- diag(e^{G_L}) S + K~^T D */
#pragma unroll
    for (int mt = 0; mt < 8; mt++) S[mt] *= X.gl[mt];
    bf16x8 db[2];
    db[0] = pack8(D[0], D[1]);
    db[1] = pack8(D[2], D[3]);
#pragma unroll
    for (int jb = 0; jb < 2; jb++)
#pragma unroll
        for (int mt = 0; mt < 8; mt++) S[mt] = mfma(kt[mt * 2 + jb], db[jb], S[mt]);
}

/* output wave, chunk c: X holds U of chunk c, Y receives that of chunk c + 1 */
__device__ __forceinline__ void pair_output_step(const PairNext &X, PairNext &Y, const unsigned char *nrec,
                                                 const unsigned char *qs, const bf16x8 *ring, int nt,
                                                 const __amdgpu_buffer_rsrc_t &ro, int row_bytes, int l, int g,
                                                 int n16)
{
    pair_load_next<false>(Y, nrec, nt, l, g);
    __builtin_amdgcn_sched_barrier(0);
    pair_barrier();
    bf16x8 sb[4], Q[16], P[6];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) sb[kb] = ring[kb * 64 + l];
#pragma unroll
    for (int f = 0; f < 16; f++) Q[f] = lds_frag(qs, f * 1024 + l * 16);
#pragma unroll
    for (int f = 0; f < 6; f++) P[f] = lds_frag(qs, 16384 + f * 1024 + l * 16);
    /* out^T = S^T Q'^T + U^T P^T   (lane = token, regs = 4 value columns) */
    f32x4 O[4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) O[mt] = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int mt = 0; mt < 4; mt++) O[mt] = mfma(sb[kb], Q[mt * 4 + kb], O[mt]);
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int jb = 0; jb <= (mt >> 1); jb++) O[mt] = mfma(X.U[jb], P[KDA_PIDX(mt, jb)], O[mt]);
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        u32x2 o;
        o[0] = pack_bf16x2(O[mt][0], O[mt][1]);
        o[1] = pack_bf16x2(O[mt][2], O[mt][3]);
        __builtin_amdgcn_raw_buffer_store_b64(o, ro, (16 * mt + n16) * row_bytes + (16 * nt + 4 * g) * 2, 0, 0);
    }
}

extern "C" __global__ void __launch_bounds__(384)
kda_scan_pair_kernel(const unsigned char *__restrict__ rec_base, const int32_t *__restrict__ cu,
                     const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H, int64_t nslots,
                     uint16_t *__restrict__ out, const void *init_state, void *final_state, int state_fp32,
                     const int32_t *__restrict__ long_list)
{
    __shared__ __attribute__((aligned(1024))) unsigned char wslots[3][16384];
    __shared__ __attribute__((aligned(1024))) unsigned char kslots[3][16384];
    __shared__ __attribute__((aligned(1024))) unsigned char qslots[2][KDA_PQP_BYTES];
    __shared__ bf16x8 ring[2][2][4 * 64]; /* [tile in pair][chunk parity]: S(c) in bf16 */
    __shared__ __attribute__((aligned(16))) unsigned char warm_sink[256];
    const int wave = threadIdx.x >> 6;
    const int l = threadIdx.x & 63, g = l >> 4, n16 = l & 15;
    /* the 4 tile pairs of a chain run on one XCD (blockIdx % 8) and share its L2 */
    const int64_t b = blockIdx.x;
    const int64_t xcd = b & 7, qd = b >> 3;
    const int tp = (int)(qd & 3);
    const int64_t ci = (qd >> 2) * 8 + xcd;
    int64_t seq;
    int h;
    if (long_list == nullptr) {
        if (ci >= nseq * H) return;
        seq = ci / H;
        h = (int)(ci - seq * H);
    } else {
        const int64_t slot = ci / H;
        if (slot >= long_list[0]) return;
        seq = long_list[1 + slot];
        h = (int)(ci - slot * H);
    }
    const int64_t chain = seq * H + h;
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
    const size_t sbase = (size_t)chain * KDA_DK * KDA_DV;

    if (wave < 2) {
        /* ---------------- state of tile nt ---------------- */
        const int ti = wave, nt = 2 * tp + ti;
        const int vcol = 16 * nt + n16;
        f32x4 S[8];
#pragma unroll
        for (int mt = 0; mt < 8; mt++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const size_t idx = sbase + (size_t)(16 * mt + 4 * g + e) * KDA_DV + vcol;
                float sv = 0.f;
                if (init_state)
                    sv = state_fp32 ? ((const float *)init_state)[idx] : bf2f(((const uint16_t *)init_state)[idx]);
                S[mt][e] = sv;
            }
        if (nchunk > 0) {
            /* U and e^{G_L} of chunk c in register set c % 2 after an odd leading
               chunk (no conditional step in the loop body) */
            PairNext A, B;
            int64_t c0 = 0;
            if (nchunk & 1) {
                pair_load_next<true>(B, rec_of(0), nt, l, g);
                pair_state_step(B, A, S, rec_of(1), wslots[0], kslots[0], ring[ti][0], nt, l, g);
                c0 = 1;
            } else {
                pair_load_next<true>(A, rec_of(0), nt, l, g);
            }
            for (int64_t c = c0; c < nchunk; c += 2) {
                pair_state_step(A, B, S, rec_of(c + 1), wslots[c % 3], kslots[c % 3], ring[ti][c & 1], nt, l, g);
                pair_state_step(B, A, S, rec_of(c + 2), wslots[(c + 1) % 3], kslots[(c + 1) % 3],
                                ring[ti][(c + 1) & 1], nt, l, g);
            }
        }
        if (final_state) {
#pragma unroll
            for (int mt = 0; mt < 8; mt++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const size_t idx = sbase + (size_t)(16 * mt + 4 * g + e) * KDA_DV + vcol;
                    if (state_fp32) ((float *)final_state)[idx] = S[mt][e];
                    else ((uint16_t *)final_state)[idx] = f2bf_bits(S[mt][e]);
                }
        }
    } else if (wave < 4) {
        /* ---------------- output of tile nt ---------------- */
        const int ti = wave - 2, nt = 2 * tp + ti;
        const int row_bytes = H * KDA_DV * 2;
        /* out rows of chunk c through a descriptor bounded at the chunk's last token */
        auto out_rsrc = [&](int64_t c) {
            const int64_t t0 = bos + c * KDA_CHUNK;
            const int64_t rem = eos - t0;
            const int L = (int)(rem < KDA_CHUNK ? rem : KDA_CHUNK);
            return buf_rsrc(out + ((size_t)t0 * H + h) * KDA_DV, (uint32_t)((L - 1) * row_bytes + KDA_DV * 2));
        };
        if (nchunk > 0) {
            PairNext A, B;
            int64_t c0 = 0;
            if (nchunk & 1) {
                pair_load_next<false>(B, rec_of(0), nt, l, g);
                pair_output_step(B, A, rec_of(1), qslots[0], ring[ti][0], nt, out_rsrc(0), row_bytes, l, g, n16);
                c0 = 1;
            } else {
                pair_load_next<false>(A, rec_of(0), nt, l, g);
            }
            for (int64_t c = c0; c < nchunk; c += 2) {
                pair_output_step(A, B, rec_of(c + 1), qslots[c & 1], ring[ti][c & 1], nt, out_rsrc(c), row_bytes,
                                 l, g, n16);
                pair_output_step(B, A, rec_of(c + 2), qslots[(c + 1) & 1], ring[ti][(c + 1) & 1], nt,
                                 out_rsrc(c + 1), row_bytes, l, g, n16);
            }
        }
    } else {
        /* ---------------- copy waves ---------------- */
        const int cw = wave - 4;
        const uint32_t sink = lds_u32(warm_sink);
        /* this workgroup's quarter of a record: lines of 128 B, clamped into the
           quarter and into the record */
        auto warm_ptr = [&](const unsigned char *wr, int j) {
            const int line = 64 * j + l;
            int off = tp * KDA_PWARM_RANGE + (line * 128 < KDA_PWARM_RANGE ? line * 128 : KDA_PWARM_RANGE - 128);
            off = off < KDA_REC_BYTES ? off : KDA_REC_BYTES - 128;
            return wr + off;
        };
        /* Q' and P of chunk c into Q'P slot c % 2: pieces 11 cw .. 11 cw + 10 of
           the slot's 22 (Q' KiB 0-15, then P KiB 0-5) */
        auto copy_qp = [&](int64_t c) {
            const unsigned char *r = rec_of(c);
            const uint32_t dst = lds_u32(qslots[c & 1]);
#pragma unroll
            for (int j = 0; j < KDA_PCP_QP; j++) {
                const int i = KDA_PCP_QP * cw + j;
                const int src = i < 16 ? KDA_REC_Q + i * 1024 : KDA_REC_P + (i - 16) * 1024;
                pair_copy(r + src + l * 16, dst + i * 1024);
            }
        };
        /* W and K~ of chunk c into their slots c % 3 (half each), then the warming
           of chunk c + KDA_PAIR_WARM - 2 */
        auto copy_wk = [&](int64_t c) {
            const unsigned char *r = rec_of(c);
            const uint32_t dw = lds_u32(wslots[c % 3]) + cw * 8192, dk = lds_u32(kslots[c % 3]) + cw * 8192;
#pragma unroll
            for (int i = 0; i < 8; i++) pair_copy(r + KDA_REC_W + cw * 8192 + i * 1024 + l * 16, dw + i * 1024);
#pragma unroll
            for (int i = 0; i < 8; i++) pair_copy(r + KDA_REC_KT + cw * 8192 + i * 1024 + l * 16, dk + i * 1024);
            const unsigned char *wr = rec_of(c + KDA_PAIR_WARM - 2);
            if (cw == 0) {
                pair_touch(warm_ptr(wr, 0), sink);
                pair_touch(warm_ptr(wr, 1), sink);
            } else {
                pair_touch(warm_ptr(wr, 2), sink);
            }
        };
        if (nchunk > 0) {
            copy_qp(0);
            copy_wk(0);
            copy_wk(1);
            /* chunk 0 has landed when at most chunk 1's W, K~ and warming are outstanding */
            if (cw == 0) pair_wait_vm<KDA_PCP0_TAIL>(); else pair_wait_vm<KDA_PCP1_TAIL>();
            for (int64_t c = 0; c < nchunk; c++) {
                pair_barrier();
                copy_qp(c + 1);
                copy_wk(c + 2);
                if (cw == 0) pair_wait_vm<KDA_PCP0_TAIL>(); else pair_wait_vm<KDA_PCP1_TAIL>();
            }
        }
        pair_wait_vm<0>(); /* no copy may still be landing when the workgroup's LDS is released */
    }
}

/* the pair scan for max_chains chains (or the long sequences of a packed batch,
   listed by the chunk-table kernel, when long_list is given) */
extern "C" hipError_t kda_launch_scan_pair(const void *records, const int32_t *cu, const int32_t *chunk_off,
                                           int64_t nseq, int64_t T, int64_t H, int64_t nslots, void *out,
                                           const void *init_state, void *final_state, int state_fp32,
                                           int64_t max_chains, const int32_t *long_list, hipStream_t st)
{
    hipLaunchKernelGGL(kda_scan_pair_kernel, dim3((unsigned)((max_chains + 7) / 8 * 32)), dim3(384), 0, st,
                       (const unsigned char *)records, cu, chunk_off, nseq, T, (int)H, nslots, (uint16_t *)out,
                       init_state, final_state, state_fp32, long_list);
    return hipGetLastError();
}
