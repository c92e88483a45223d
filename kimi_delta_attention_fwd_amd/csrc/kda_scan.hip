/*
 * kda_scan.hip -- gfx950 scan kernels of the chunked Kimi Delta Attention
 * forward: the sequential chunk loop per (sequence, head) with the fp32 state in
 * MFMA accumulators, over the records kda_prep_kernel writes (layout in
 * kda_internal.h). kda_launch_scan picks one of three forms from the sizes
 * alone (no device data is read on the host):
 *   kda_scan_kernel       3 waves per (chain, 16 value columns): fewer than 128
 *                         chains, and the long sequences of packed batches
 *                         (kda_scan_k64_kernel: the same at K = V = 64);
 *   kda_scan_many_kernel  8 waves per chain, the chunk's shared operands in
 *                         LDS: 128 chains or more;
 *   kda_seg_map_kernel, kda_seg_chain_kernel, kda_scan_seg_kernel
 *                         segment-parallel: at most 10 long chains.
 * All of them evaluate the same chunk update in the same order (bf16 operands,
 * fp32 accumulation), so a chain gives the same bits on the first two; the
 * segment-parallel form differs from them by rounding only.
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
 * wave 2 (L2 warm): touches its eighth of the record three chunks ahead with
 *                  LDS-DMA loads into a scratch LDS buffer, so that the eight
 *                  workgroups of a chain find their records in L2; in the plain
 *                  128-channel scan it also copies each chunk's K~^T two chunks
 *                  ahead into a three-slot LDS ring that the state wave reads.
 * The three waves meet at one barrier per chunk. Waves 0 and 1 double-buffer
 * their record operands in registers: all loads for chunk c + 1 are issued at
 * the start of chunk c (two register sets alternate over a two-chunk unroll).
 * Records and out are accessed through buffer descriptors (SGPR base per chunk,
 * one lane offset), which keeps address arithmetic off the vector ALU.
 * The warming loads are issued through inline assembly, so the compiler does
 * not track them and no wave ever waits for them, except wave 2 once before it
 * exits (its LDS must not be released with DMA writes in flight).
 */
/* NKB = DK / 32 key blocks (W, Q', K~^T hold 4 NKB fragments each). Register
   sets of one chunk's operands: every operand of the state update (the
   segment-map kernel); W alone (the scan's state wave, which reads K~^T, e^{G_L}
   and U from the warming wave's LDS ring); Q' and P (the output wave, U from the
   ring). */
template <int NKB> struct ScanSetS {
    bf16x8 W[4 * NKB], K[4 * NKB], U[2];
    f32x4 gl[2 * NKB]; /* e^{G_L} for key rows 16 mt + 4 g + e */
};
template <int NKB> struct ScanSetW {
    bf16x8 W[4 * NKB];
};
template <int NKB> struct ScanSetO {
    bf16x8 Q[4 * NKB], P[6];
};
/* A ring slot holds the chunk's K~^T (4 NKB fragments), then 1 KiB from e^{G_L}
   on, then this tile's 2 KiB of U (lane l's 32 bytes at 32 l) */
template <int NKB> __device__ __forceinline__ const bf16x8 *slot_gl(const bf16x8 *slot) { return slot + 4 * NKB * 64; }
template <int NKB> __device__ __forceinline__ const bf16x8 *slot_u(const bf16x8 *slot) { return slot + 4 * NKB * 64 + 64; }

__device__ __forceinline__ bf16x8 bufld(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

/* one chunk record (layout RecLayout<NKB, NVT>) through a buffer descriptor:
   SGPR base, lane offsets in VGPRs */
template <int NKB, int NVT>
__device__ __forceinline__ void load_set(ScanSetS<NKB> &X, const unsigned char *rec, int ubase, int l, int g)
{
    using RL = RecLayout<NKB, NVT>;
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(rec, RL::BYTES);
#pragma unroll
    for (int f = 0; f < 4 * NKB; f++) X.W[f] = bufld(r, l * 16, RL::W + f * 1024);
    X.U[0] = bufld(r, l * 32, ubase);
    X.U[1] = bufld(r, l * 32, ubase + 16);
#pragma unroll
    for (int mt = 0; mt < 2 * NKB; mt++)
        X.gl[mt] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, g * 16, RL::GL + mt * 64, 0));
#pragma unroll
    for (int f = 0; f < 4 * NKB; f++) X.K[f] = bufld(r, l * 16, RL::KT + f * 1024);
}

template <int NKB, int NVT>
__device__ __forceinline__ void load_set(ScanSetW<NKB> &X, const unsigned char *rec, int l)
{
    using RL = RecLayout<NKB, NVT>;
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(rec, RL::BYTES);
#pragma unroll
    for (int f = 0; f < 4 * NKB; f++) X.W[f] = bufld(r, l * 16, RL::W + f * 1024);
}

template <int NKB, int NVT>
__device__ __forceinline__ void load_set(ScanSetO<NKB> &X, const unsigned char *rec, int l)
{
    using RL = RecLayout<NKB, NVT>;
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(rec, RL::BYTES);
#pragma unroll
    for (int f = 0; f < 4 * NKB; f++) X.Q[f] = bufld(r, l * 16, RL::Q + f * 1024);
#pragma unroll
    for (int f = 0; f < 6; f++) X.P[f] = bufld(r, l * 16, RL::P + f * 1024);
}

__device__ __forceinline__ void chunk_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

/* state wave: X holds chunk c's W, kt_lds is chunk c's ring slot; loads chunk
   c + 1's W (at nrec) into Y */
template <int NKB, int NVT>
__device__ __forceinline__ void state_step(ScanSetW<NKB> &X, ScanSetW<NKB> &Y, f32x4 (&S)[2 * NKB],
                                           const unsigned char *nrec, bf16x8 *slot, int l, int g,
                                           const bf16x8 *kt_lds)
{
    load_set<NKB, NVT>(Y, nrec, l);
    bf16x8 sb[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; kb++) {
        sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
        slot[kb * 64 + l] = sb[kb];
    }
    chunk_barrier();
    f32x4 D[4];
    bf16x8 uu[2];
#pragma unroll
    for (int jb = 0; jb < 2; jb++) uu[jb] = slot_u<NKB>(kt_lds)[2 * l + jb];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        const int o = (mt & 1) * 4;
        const bf16x8 &u = uu[mt >> 1];
        D[mt] = f32x4{(float)u[o], (float)u[o + 1], (float)u[o + 2], (float)u[o + 3]};
    }
    /* D = U - W S */
#pragma unroll
    for (int kb = 0; kb < NKB; kb++)
#pragma unroll
        for (int mt = 0; mt < 4; mt++) D[mt] = mfma(X.W[mt * NKB + kb], sb[kb], D[mt]);
    /* S <- diag(e^{G_L}) S + K~^T D (e^{G_L} after K~^T in the LDS slot, key-channel order) */
#pragma unroll
    for (int mt = 0; mt < 2 * NKB; mt++) S[mt] *= ((const f32x4 *)slot_gl<NKB>(kt_lds))[4 * mt + g];
    bf16x8 db[2];
    db[0] = pack8(D[0], D[1]);
    db[1] = pack8(D[2], D[3]);
    /* K~^T from the chunk's LDS slot, 2 NKB fragments at a time */
#pragma unroll
    for (int jb = 0; jb < 2; jb++) {
        bf16x8 kf[2 * NKB];
#pragma unroll
        for (int mt = 0; mt < 2 * NKB; mt++) kf[mt] = kt_lds[(mt * 2 + jb) * 64 + l];
#pragma unroll
        for (int mt = 0; mt < 2 * NKB; mt++) S[mt] = mfma(kf[mt], db[jb], S[mt]);
    }
}

/* output wave: X holds chunk c's Q' and P (tokens t0 .. t0 + L - 1), kslot is its
   ring slot (U), slot the entering state; loads chunk c + 1 into Y. out is written
   through a buffer descriptor bounded at row L - 1: rows past the sequence end
   fall outside it and the hardware drops their stores. */
template <int NKB, int NVT>
__device__ __forceinline__ void output_step(ScanSetO<NKB> &X, ScanSetO<NKB> &Y, const unsigned char *nrec,
                                            const bf16x8 *slot, uint16_t *out, int64_t t0, int L, int H, int h,
                                            int nt, int l, int g, int n16, const bf16x8 *kslot)
{
    constexpr int DV = 16 * NVT;
    load_set<NKB, NVT>(Y, nrec, l);
    chunk_barrier();
    bf16x8 sb[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; kb++) sb[kb] = slot[kb * 64 + l];
    /* out^T = S^T Q'^T + U^T P^T   (lane = token, regs = 4 value columns) */
    f32x4 O[4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) O[mt] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; kb++)
#pragma unroll
        for (int mt = 0; mt < 4; mt++) O[mt] = mfma(sb[kb], X.Q[mt * NKB + kb], O[mt]);
    bf16x8 uu[2];
#pragma unroll
    for (int jb = 0; jb < 2; jb++) uu[jb] = slot_u<NKB>(kslot)[2 * l + jb];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int jb = 0; jb <= (mt >> 1); jb++) O[mt] = mfma(uu[jb], X.P[KDA_PIDX(mt, jb)], O[mt]);
    const int row_bytes = H * DV * 2;
    const __amdgpu_buffer_rsrc_t ro =
        buf_rsrc(out + ((size_t)t0 * H + h) * DV, (uint32_t)((L - 1) * row_bytes + DV * 2));
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        u32x2 u;
        u[0] = pack_bf16x2(O[mt][0], O[mt][1]);
        u[1] = pack_bf16x2(O[mt][2], O[mt][3]);
        __builtin_amdgcn_raw_buffer_store_b64(u, ro, (16 * mt + n16) * row_bytes + (16 * nt + 4 * g) * 2, 0, 0);
    }
}

/* one 1 KiB LDS-DMA load (64 lanes x 16 bytes) that nobody waits for; m0 is not
   otherwise used in this kernel (LDS instructions on gfx9 do not read it; the
   generated code is checked for that by tests/test_isa_guards.py) */
__device__ __forceinline__ void warm_l2(const unsigned char *p, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(p), "s"(lds_addr) : "memory", "m0");
}

/* padding of the LDS-ring warming loop (0-7 nops measured alike) */
#ifndef KDA_WARM_NOPS
#define KDA_WARM_NOPS 2
#endif
#define KDA_STR2(x) #x
#define KDA_STR(x) KDA_STR2(x)

/* chunks between the one a workgroup computes and the one its warming wave
   touches (long prefill scan: 2 or 3 -> 1.021 ms, 4 -> 1.038, 6 -> 1.106,
   8 -> 1.150) */
#define KDA_WARM_AHEAD 3

/* chunks between the one the state wave computes and the one whose ring slot the
   warming wave fills (the ring has KDA_KRING_AHEAD + 1 slots) */
#ifndef KDA_KRING_AHEAD
#define KDA_KRING_AHEAD 3
#endif
#define KDA_KRING_SLOTS (KDA_KRING_AHEAD + 1)

/* the scan body over DK = 32 NKB key channels and NVT value tiles of 16 columns
   (record layout RecLayout<NKB, NVT>); SEG instantiates the segment-parallel
   rescan (one workgroup per (chain, segment, tile)), which the plain kernel
   compiles without */
template <bool SEG, int NKB, int NVT>
__device__ __forceinline__ void scan_body(const unsigned char *__restrict__ rec_base, const int32_t *__restrict__ cu,
                                          const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H,
                                          int64_t nslots, uint16_t *__restrict__ out,
                                          const void *init_state, void *final_state,
                                          int state_fp32, const int32_t *__restrict__ long_list, int64_t nseg,
                                          int64_t segc, const float *__restrict__ seg_init)
{
    using RL = RecLayout<NKB, NVT>;
    constexpr int DK = 32 * NKB, DV = 16 * NVT;
    static_assert((NVT & (NVT - 1)) == 0, "value tiles: a power of two");
    __shared__ bf16x8 ring[2][NKB * 64];                        /* S(c) in bf16 (8 KiB at DK = 128) */
    __shared__ __attribute__((aligned(16))) unsigned char warm_sink[1024];
    /* the ring: K~^T of chunk c, 1 KiB from e^{G_L} on and this tile's U in
       kring[c % KDA_KRING_SLOTS] (slot_gl, slot_u), copied by the warming wave
       KDA_KRING_AHEAD chunks ahead */
    __shared__ __attribute__((aligned(16))) bf16x8 kring[KDA_KRING_SLOTS][4 * NKB * 64 + 64 + 128];
    const int wave = threadIdx.x >> 6;
    const int l = threadIdx.x & 63, g = l >> 4, n16 = l & 15;
    /* the NVT value tiles of a chain run on one XCD (blockIdx % 8) and share its L2 */
    const int64_t b = blockIdx.x;
    const int64_t xcd = b & 7, qd = b >> 3;
    const int nt = (int)(qd & (NVT - 1));
    const int64_t cs = (qd / NVT) * 8 + xcd;
    /* cs = ci * nseg + segment; ci is the chain (sequence * H + head), or with a
       long-sequence list (long_list[0] entries, then sequence indices) the list
       slot * H + head */
    const int64_t seg = SEG ? cs % nseg : 0;
    const int64_t ci = SEG ? cs / nseg : cs;
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
    int64_t nchunk = (eos - bos + KDA_CHUNK - 1) / KDA_CHUNK;
    /* a segment of the segment-parallel scan: chunks seg * segc .. from the
       entering state the chaining pass left in seg_init (fp32; segment 0's is a
       copy of the initial state, so an in-place final state cannot race with
       it); only the sequence's last segment writes the final state */
    const void *ist = init_state;
    int ist_fp32 = state_fp32;
    size_t ibase = (size_t)chain * DK * DV;
    void *fst = final_state;
    if (SEG) {
        const int64_t nseg_seq = nchunk > segc ? (nchunk + segc - 1) / segc : 1;
        if (seg >= nseg_seq) return;
        const int64_t c_first = seg * segc;
        nchunk = nchunk - c_first < segc ? nchunk - c_first : segc;
        bos += c_first * KDA_CHUNK;
        slot0 += c_first;
        ist = seg_init;
        ist_fp32 = 1;
        ibase = ((size_t)chain * nseg + seg) * DK * DV;
        if (seg < nseg_seq - 1) fst = nullptr;
    }
    const unsigned char *rec0 = rec_base + ((size_t)h * nslots + slot0) * RL::BYTES;
    /* record of chunk c, clamped to the last one (its reload is harmless) */
    auto rec_of = [&](int64_t c) { return rec0 + (size_t)(c < nchunk ? c : nchunk - 1) * RL::BYTES; };
    const int ubase = RL::U + nt * 2048; /* this tile's 2 KiB of U; lane l reads 32 bytes */

    if (wave == 0) {
        /* ---------------- state wave ---------------- */
        f32x4 S[2 * NKB];
#pragma unroll
        for (int mt = 0; mt < 2 * NKB; mt++) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const size_t idx = ibase + (size_t)(16 * mt + 4 * g + e) * DV + vcol;
                float sv = 0.f;
                if (ist)
                    sv = ist_fp32 ? ((const float *)ist)[idx] : bf2f(((const uint16_t *)ist)[idx]);
                S[mt][e] = sv;
            }
        }
        if (nchunk > 0) {
            ScanSetW<NKB> X, Y;
            int64_t c = 0;
            if (nchunk & 1) {
                load_set<NKB, NVT>(X, rec_of(0), l);
                state_step<NKB, NVT>(X, Y, S, rec_of(1), ring[0], l, g, kring[0]);
                c = 1;
            } else {
                load_set<NKB, NVT>(Y, rec_of(0), l);
            }
            for (; c < nchunk; c += 2) {
                state_step<NKB, NVT>(Y, X, S, rec_of(c + 1), ring[c & 1], l, g, kring[c % KDA_KRING_SLOTS]);
                state_step<NKB, NVT>(X, Y, S, rec_of(c + 2), ring[(c + 1) & 1], l, g,
                                     kring[(c + 1) % KDA_KRING_SLOTS]);
            }
        }
        if (fst) {
            const size_t sbase2 = (size_t)chain * DK * DV;
#pragma unroll
            for (int mt = 0; mt < 2 * NKB; mt++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const size_t idx = sbase2 + (size_t)(16 * mt + 4 * g + e) * DV + vcol;
                    if (state_fp32) ((float *)fst)[idx] = S[mt][e];
                    else ((uint16_t *)fst)[idx] = f2bf_bits(S[mt][e]);
                }
        }
    } else if (wave == 1) {
        /* ---------------- output wave ---------------- */
        if (nchunk > 0) {
            ScanSetO<NKB> X, Y;
            int64_t c = 0;
            auto t0_of = [&](int64_t cc) { return bos + cc * KDA_CHUNK; };
            auto len_of = [&](int64_t cc) {
                const int64_t rem = eos - t0_of(cc);
                return (int)(rem < KDA_CHUNK ? rem : KDA_CHUNK);
            };
            if (nchunk & 1) {
                load_set<NKB, NVT>(X, rec_of(0), l);
                output_step<NKB, NVT>(X, Y, rec_of(1), ring[0], out, t0_of(0), len_of(0), H, h, nt, l, g, n16,
                                      kring[0]);
                c = 1;
            } else {
                load_set<NKB, NVT>(Y, rec_of(0), l);
            }
            for (; c < nchunk; c += 2) {
                output_step<NKB, NVT>(Y, X, rec_of(c + 1), ring[c & 1], out, t0_of(c), len_of(c), H, h, nt, l, g,
                                      n16, kring[c % KDA_KRING_SLOTS]);
                output_step<NKB, NVT>(X, Y, rec_of(c + 2), ring[(c + 1) & 1], out, t0_of(c + 1), len_of(c + 1), H,
                                      h, nt, l, g, n16, kring[(c + 1) % KDA_KRING_SLOTS]);
            }
        }
    } else {
        /* ---------------- L2-warming wave ---------------- */
        const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)warm_sink;
        /* After barrier c: touches this tile's share of chunk c + KDA_WARM_AHEAD's
           record into L2 and copies K~^T, e^{G_L} and U of chunk c +
           KDA_KRING_AHEAD into its ring slot (LDS-DMA), the state wave being done
           with chunk c - 1's slot; then waits for chunk c + 1's copy before
           barrier c + 1. Every trip issues the same number of loads (chunk indices
           clamped to the last), so the waits count exactly: NTJ + 2 touches
           (7 + 2 at 128 key channels) and 4 NKB + 1 + 2 copies. The output wave
           reads U from the same slot, between the same barriers as the state
           wave. */
        /* NPIECE 1 KiB pieces up to e^{G_L}, NTJ of them per tile, and its U */
        constexpr int NPIECE = RL::U / 1024 + 1, NTJ = (NPIECE + NVT - 1) / NVT;
        constexpr int NTOUCH = NTJ + 2, NCOPY = 4 * NKB + 3;
        static_assert((KDA_KRING_AHEAD - 1) * (NTOUCH + NCOPY) <= 63 && KDA_KRING_AHEAD >= 2,
                      "the waits below count at most 63 loads");
        auto kt_copy = [&](int64_t cc) {
            const int64_t ck = cc < nchunk ? cc : nchunk - 1;
            const unsigned char *src = rec0 + (size_t)ck * RL::BYTES + RL::KT + l * 16;
            const uint32_t dst =
                (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16x8 *)kring[cc % KDA_KRING_SLOTS];
#pragma unroll
            for (int i = 0; i < 4 * NKB; i++) warm_l2(src + i * 1024, dst + i * 1024);
            warm_l2(src - RL::KT + RL::GL, dst + 4 * NKB * 1024); /* e^{G_L} and 512 bytes after it */
            warm_l2(src - RL::KT + ubase, dst + (4 * NKB + 1) * 1024); /* this tile's U */
            warm_l2(src - RL::KT + ubase + 1024, dst + (4 * NKB + 2) * 1024);
        };
        /* this tile's share of chunk cw's record into L2, in 1 KiB pieces */
        auto touch = [&](int64_t cw) {
            cw = cw < nchunk ? cw : nchunk - 1;
            const unsigned char *r = rec0 + (size_t)cw * RL::BYTES;
#pragma unroll
            for (int j = 0; j < NTJ; j++) {
                const int i = nt + NVT * j < NPIECE ? nt + NVT * j : NPIECE - 1;
                warm_l2(r + i * 1024 + l * 16, lds);
            }
            warm_l2(r + RL::U + nt * 2048 + l * 16, lds);
            warm_l2(r + RL::U + nt * 2048 + 1024 + l * 16, lds);
        };
        if (nchunk == 0) return; /* no chunk: no barrier, nothing to copy */
        /* units of NTOUCH + NCOPY loads, so that KDA_KRING_AHEAD - 1 units were
           issued after any copy when the loop waits for it */
        kt_copy(0);
#pragma unroll
        for (int k = 1; k < KDA_KRING_AHEAD; k++) {
            touch(k);
            kt_copy(k);
        }
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((KDA_KRING_AHEAD - 1) * (NTOUCH + NCOPY)) : "memory");
        for (int64_t c = 0; c < nchunk; c++) {
            asm volatile(".p2align 5\n\t.rept " KDA_STR(KDA_WARM_NOPS) "\n\ts_nop 0\n\t.endr");
            chunk_barrier();
            touch(c + KDA_WARM_AHEAD);
            kt_copy(c + KDA_KRING_AHEAD);
            /* chunk c + 1's copy has landed */
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((KDA_KRING_AHEAD - 1) * (NTOUCH + NCOPY)) : "memory");
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

/* K~^T, e^{G_L} and U through the warming wave's LDS ring: the state wave then
   issues 16 loads per chunk instead of 42, so two chunks of its loads fit the 63
   a wave can have outstanding, and the kernel needs 280 registers (338 with
   e^{G_L} and U in registers). Long prefill scan 1.063 -> 1.026 ms with K~^T
   alone (and no longer sensitive to the warming loop's code placement), 1.004 ms
   with e^{G_L}, 0.990 ms with U, 0.977 ms with four ring slots filled three
   chunks ahead instead of three two ahead. */
extern "C" __global__ void __launch_bounds__(192)
kda_scan_kernel(const unsigned char *__restrict__ rec_base, const int32_t *__restrict__ cu,
                const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H, int64_t nslots,
                uint16_t *__restrict__ out, const void *init_state,
                void *final_state, int state_fp32, const int32_t *__restrict__ long_list)
{
    scan_body<false, 4, 8>(rec_base, cu, chunk_off, nseq, T, H, nslots, out, init_state, final_state, state_fp32,
                           long_list, 1, 0, nullptr);
}

/* K = V = 64: four value tiles per chain */
extern "C" __global__ void __launch_bounds__(192)
kda_scan_k64_kernel(const unsigned char *__restrict__ rec_base, const int32_t *__restrict__ cu,
                    const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H, int64_t nslots,
                    uint16_t *__restrict__ out, const void *init_state, void *final_state, int state_fp32)
{
    scan_body<false, 2, 4>(rec_base, cu, chunk_off, nseq, T, H, nslots, out, init_state, final_state, state_fp32,
                           nullptr, 1, 0, nullptr);
}

/* the rescan of the segment-parallel scan: workgroup (chain, segment slot, tile) */
extern "C" __global__ void __launch_bounds__(192)
kda_scan_seg_kernel(const unsigned char *__restrict__ rec_base, const int32_t *__restrict__ cu,
                    const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H, int64_t nslots,
                    uint16_t *__restrict__ out, void *final_state, int state_fp32, int64_t nseg,
                    int64_t segc, const float *__restrict__ seg_init)
{
    scan_body<true, 4, 8>(rec_base, cu, chunk_off, nseq, T, H, nslots, out, nullptr, final_state, state_fp32, nullptr,
                          nseg, segc, seg_init);
}

/* ------------------------------------------------------------------------- */
/* segment-parallel scan: segment maps and their chaining                      */
/* ------------------------------------------------------------------------- */
/*
 * With few chains (fixed-length batches of B * H <= 10 long sequences, e.g. one
 * GPU's share of heads) the three-wave kernel leaves most CUs idle: each chain
 * is one dependent walk over all its chunks. The chunk update is affine in the
 * state, S -> (diag(e^{G_L}) - K~^T W) S + K~^T U, so a segment of chunks maps
 * its entering state S to M S + B. kda_seg_map_kernel runs every segment but
 * the last from the states [0 | I] (B: 8 value tiles with U; M: 8 identity
 * tiles with U taken as 0), all segments at once; kda_seg_chain_kernel walks the
 * G - 1 maps of a chain in fp32 to get every segment's entering state; the
 * three-wave kernel then rescans each segment from its entering state, writing
 * out (and, for the last segment, the final state). The maps use the same
 * chunk arithmetic as the scan (bf16 operands, fp32 accumulation), so the
 * result differs from the plain scan only by rounding.
 */

/* state-only chunk step: X holds chunk c, loads chunk c + 1 (at nrec) into Y */
__device__ __forceinline__ void map_step(ScanSetS<4> &X, ScanSetS<4> &Y, f32x4 (&S)[8], const unsigned char *nrec,
                                         int ubase, int l, int g, bool homog)
{
    load_set<4, 8>(Y, nrec, ubase, l, g);
    bf16x8 sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
    f32x4 D[4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        const int o = (mt & 1) * 4;
        const bf16x8 &u = X.U[mt >> 1];
        D[mt] = homog ? zero4() : f32x4{(float)u[o], (float)u[o + 1], (float)u[o + 2], (float)u[o + 3]};
    }
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int mt = 0; mt < 4; mt++) D[mt] = mfma(X.W[mt * 4 + kb], sb[kb], D[mt]);
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

/* chunks and first chunk slot of sequence seq (fixed-length batch or packed) */
__device__ __forceinline__ void seq_chunks(int64_t seq, const int32_t *cu, const int32_t *chunk_off, int64_t T,
                                           int64_t &nchunk, int64_t &slot0)
{
    if (cu == nullptr) {
        nchunk = (T + KDA_CHUNK - 1) / KDA_CHUNK;
        slot0 = seq * nchunk;
    } else {
        nchunk = ((int64_t)cu[seq + 1] - cu[seq] + KDA_CHUNK - 1) / KDA_CHUNK;
        slot0 = chunk_off[seq];
    }
}

/* segments of a sequence of nchunk chunks (at least one, also when it is empty) */
__device__ __forceinline__ int64_t seq_segments(int64_t nchunk, int64_t segc)
{
    return nchunk > segc ? (nchunk + segc - 1) / segc : 1;
}

/* one wave per (chain, segment slot < G - 1, 16-column tile of [B | M]); the 16
   tiles of a segment run on one XCD and share its L2. Only segments that are
   not their sequence's last are mapped; they hold segc full chunks. */
extern "C" __global__ void __launch_bounds__(64)
kda_seg_map_kernel(const unsigned char *rec_base, const int32_t *__restrict__ cu,
                   const int32_t *__restrict__ chunk_off, int64_t nchain, int64_t T, int H, int64_t nslots,
                   int64_t nseg, int64_t segc, float *seg_area)
{
    const int l = threadIdx.x, g = l >> 4, n16 = l & 15;
    const int64_t b = blockIdx.x;
    const int64_t xcd = b & 7, qd = b >> 3;
    const int t16 = (int)(qd & 15);
    const int64_t grp = (qd >> 4) * 8 + xcd; /* chain * (nseg - 1) + segment */
    if (grp >= nchain * (nseg - 1)) return;
    const int64_t chain = grp / (nseg - 1), seg = grp - chain * (nseg - 1);
    const int64_t seq = chain / H;
    const int h = (int)(chain - seq * H);
    int64_t nchunk, slot0;
    seq_chunks(seq, cu, chunk_off, T, nchunk, slot0);
    if (seg >= seq_segments(nchunk, segc) - 1) return;
    const bool homog = t16 >= 8;
    const int nt = t16 & 7;
    const unsigned char *rec0 = rec_base + ((size_t)h * nslots + slot0 + seg * segc) * KDA_REC_BYTES;
    auto rec_of = [&](int64_t c) { return rec0 + (size_t)(c < segc ? c : segc - 1) * KDA_REC_BYTES; };
    const int ubase = KDA_REC_U + nt * 2048;

    /* [B | M] starts at [0 | I]: tile nt of M holds the identity's columns 16 nt .. 16 nt + 15 */
    f32x4 S[8];
#pragma unroll
    for (int mt = 0; mt < 8; mt++)
#pragma unroll
        for (int e = 0; e < 4; e++) S[mt][e] = (homog && 16 * mt + 4 * g + e == 16 * nt + n16) ? 1.f : 0.f;
    ScanSetS<4> X, Y;
    int64_t c = 0;
    if (segc & 1) {
        load_set<4, 8>(X, rec_of(0), ubase, l, g);
        map_step(X, Y, S, rec_of(1), ubase, l, g, homog);
        c = 1;
    } else {
        load_set<4, 8>(Y, rec_of(0), ubase, l, g);
    }
    for (; c < segc; c += 2) {
        map_step(Y, X, S, rec_of(c + 1), ubase, l, g, homog);
        map_step(X, Y, S, rec_of(c + 2), ubase, l, g, homog);
    }
    float *dst = seg_area + ((size_t)(homog ? nchain * (nseg - 1) : 0) + grp) * KDA_DK * KDA_DV;
#pragma unroll
    for (int mt = 0; mt < 8; mt++)
#pragma unroll
        for (int e = 0; e < 4; e++) dst[(16 * mt + 4 * g + e) * KDA_DV + 16 * nt + n16] = S[mt][e];
}

__device__ __forceinline__ f32x4 mfma_f32x4(float a, float b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

/* LDS slot of row R, column j of a 128 x 16 fp32 state tile (rows 32 apart are
   spread over the banks) */
__host__ __device__ constexpr int chain_lds(int R, int j) { return R * 16 + (R >> 5) * 8 + j; }

/* one workgroup of 4 waves per (chain, 16-column tile): S_0 = initial state,
   S_{s+1} = M_s S_s + B_s for s below the sequence's segment count - 1, in fp32
   (v_mfma_f32_16x16x4f32); wave w computes row tiles 2 w, 2 w + 1 of each
   product. Writes S_0 .. S_{segments - 1} of the chain's G slots. */
extern "C" __global__ void __launch_bounds__(256)
kda_seg_chain_kernel(float *seg_area, const void *init_state, int state_fp32, const int32_t *__restrict__ cu,
                     int64_t T, int H, int64_t nchain, int64_t nseg, int64_t segc)
{
    __shared__ float sS[chain_lds(127, 15) + 1];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gq = l >> 4, r16 = l & 15;
    const int64_t b = blockIdx.x;
    const int64_t xcd = b & 7, qd = b >> 3;
    const int nt = (int)(qd & 7);
    const int64_t chain = (qd >> 3) * 8 + xcd;
    if (chain >= nchain) return;
    const int64_t seq = chain / H;
    const int64_t nchunk = cu == nullptr ? (T + KDA_CHUNK - 1) / KDA_CHUNK
                                         : ((int64_t)cu[seq + 1] - cu[seq] + KDA_CHUNK - 1) / KDA_CHUNK;
    const int64_t nsteps = seq_segments(nchunk, segc) - 1;
    const float *segM = seg_area + (size_t)nchain * (nseg - 1) * KDA_DK * KDA_DV;
    const float *segB = seg_area;
    float *segS = seg_area + (size_t)2 * nchain * (nseg - 1) * KDA_DK * KDA_DV + (size_t)chain * nseg * KDA_DK * KDA_DV;

    for (int i = tid; i < KDA_DK * 16; i += 256) {
        const int R = i >> 4, j = i & 15;
        const size_t idx = ((size_t)chain * KDA_DK + R) * KDA_DV + 16 * nt + j;
        float v = 0.f;
        if (init_state) v = state_fp32 ? ((const float *)init_state)[idx] : bf2f(((const uint16_t *)init_state)[idx]);
        sS[chain_lds(R, j)] = v;
        segS[R * KDA_DV + 16 * nt + j] = v;
    }
    __syncthreads();
    for (int64_t s = 0; s < nsteps; s++) {
        const size_t mo = ((size_t)chain * (nseg - 1) + s) * KDA_DK * KDA_DV;
        f32x4 acc[2];
#pragma unroll
        for (int rr = 0; rr < 2; rr++) {
            const int rt = 2 * w + rr;
            /* accumulator starts at B_s (rows 16 rt + 4 gq + e, column n16) */
#pragma unroll
            for (int e = 0; e < 4; e++) acc[rr][e] = segB[mo + (size_t)(16 * rt + 4 * gq + e) * KDA_DV + 16 * nt + r16];
            /* A = rows 16 rt + r16 of M_s, contraction index 32 gq + k over the 4 lane groups */
            float4 a4[8];
            const float *mrow = segM + mo + (size_t)(16 * rt + r16) * KDA_DV + 32 * gq;
#pragma unroll
            for (int i = 0; i < 8; i++) a4[i] = *(const float4 *)(mrow + 4 * i);
#pragma unroll
            for (int k = 0; k < 32; k++) {
                const float a = k % 4 == 0 ? a4[k / 4].x : k % 4 == 1 ? a4[k / 4].y : k % 4 == 2 ? a4[k / 4].z : a4[k / 4].w;
                acc[rr] = mfma_f32x4(a, sS[chain_lds(32 * gq + k, r16)], acc[rr]);
            }
        }
        __syncthreads(); /* every wave has read S_s */
#pragma unroll
        for (int rr = 0; rr < 2; rr++) {
            const int rt = 2 * w + rr;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int R = 16 * rt + 4 * gq + e;
                sS[chain_lds(R, r16)] = acc[rr][e];
                segS[(size_t)(s + 1) * KDA_DK * KDA_DV + R * KDA_DV + 16 * nt + r16] = acc[rr][e];
            }
        }
        __syncthreads();
    }
}

/* ------------------------------------------------------------------------- */
/* many-chain scan: one workgroup of 8 waves per (sequence, head)              */
/* ------------------------------------------------------------------------- */
/*
 * The three-wave kernel above holds a whole CU (its waves need ~450 registers
 * each) to hide the latency of one long chain, and its eight value tiles each
 * read the whole record. When there are many chains (packed batches of short
 * sequences, per-sequence states in and out) the latency is hidden by running
 * many chains side by side instead, and the record is read once per chain:
 * the workgroup copies the shared part of each chunk's record (W, Q', K~, P,
 * e^{G_L}: the first KDA_REC_U bytes, in record layout) into LDS, and wave w
 * runs value tile w (state update and output) from there, with its own slice
 * of U read from memory. Waves are limited to 128 registers and the workgroup
 * to 55.8 KB of LDS, so two workgroups share a CU. The arithmetic, its order
 * and the operand layouts are those of the three-wave kernel, so both produce
 * the same bits.
 * The state slice is read and written through buffer descriptors whose range is
 * empty when the state pointer is null (loads return 0, stores are dropped).
 */
template <int DK, int DV>
__device__ __forceinline__ void state_io_rsrc(const void *state, int state_fp32, int64_t chain, const void *dummy,
                                              __amdgpu_buffer_rsrc_t &r)
{
    const uint32_t bytes = (uint32_t)(DK * DV * (state_fp32 ? 4 : 2));
    r = state ? buf_rsrc((const unsigned char *)state + (size_t)chain * bytes, bytes) : buf_rsrc(dummy, 0);
}

__device__ __forceinline__ bf16x8 ldsld(const unsigned char *base, int off)
{
    return *(const bf16x8 *)(base + off);
}

/* One workgroup of NVT waves per chain (wave = 16-column value tile), the
   chunk's shared operands in LDS; DK = 32 NKB key channels, DV = 16 NVT value
   columns (record layout RecLayout<NKB, NVT>). */
template <int NKB, int NVT>
__device__ __forceinline__ void scan_many_body(const unsigned char *rec_base, const int32_t *__restrict__ cu,
                                               const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H,
                                               int64_t nslots, uint16_t *out, const void *init_state,
                                               void *final_state, int state_fp32, int64_t max_chunks)
{
    using RL = RecLayout<NKB, NVT>;
    constexpr int DK = 32 * NKB, DV = 16 * NVT, NKT = 2 * NKB, NTH = 64 * NVT;
    constexpr int PIECES = RL::U / 16, FILL_ITERS = (PIECES + NTH - 1) / NTH; /* 16-byte pieces of the shared operands */
    __shared__ __attribute__((aligned(16))) unsigned char opnd[RL::U];
    const int tid = threadIdx.x;
    const int l = tid & 63, g = l >> 4, n16 = l & 15;
    const int nt = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t chain = blockIdx.x;
    const int64_t seq = chain / H;
    const int h = (int)(chain - seq * H);

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
    if (nchunk > max_chunks) return; /* left to the three-wave kernel (uniform over the workgroup) */
    const unsigned char *rec0 = rec_base + ((size_t)h * nslots + slot0) * RL::BYTES;
    const int ubase = RL::U + nt * 2048;
    const int row_bytes = H * DV * 2;

    /* element (16 mt + 4 g + e, 16 nt + n16) of the state */
    const int esz = state_fp32 ? 4 : 2;
    const int soff = ((4 * g) * DV + 16 * nt + n16) * esz;
    __amdgpu_buffer_rsrc_t ri, rf;
    state_io_rsrc<DK, DV>(init_state, state_fp32, chain, rec_base, ri);
    state_io_rsrc<DK, DV>(final_state, state_fp32, chain, rec_base, rf);
    f32x4 S[NKT];
    if (state_fp32) {
#pragma unroll
        for (int mt = 0; mt < NKT; mt++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                S[mt][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ri, soff, (16 * mt + e) * DV * 4, 0));
    } else {
#pragma unroll
        for (int mt = 0; mt < NKT; mt++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                S[mt][e] = bf2f(__builtin_amdgcn_raw_buffer_load_b16(ri, soff, (16 * mt + e) * DV * 2, 0));
    }

    for (int64_t c = 0; c < nchunk; c++) {
        const __amdgpu_buffer_rsrc_t r = buf_rsrc(rec0 + (size_t)c * RL::BYTES, RL::BYTES);
        const int64_t t0 = bos + c * KDA_CHUNK;
        const int64_t rem = eos - t0;
        const int L = (int)(rem < KDA_CHUNK ? rem : KDA_CHUNK);
        /* In a partial last chunk, the fragments of token tiles past its L tokens
           hold only the zeros of the prep's padded rows: W, Q' row tiles mt >=
           nmt, K~^T token blocks jb >= njb, P row tiles mt >= nmt, U rows >= 32
           when L <= 32. They are read through a descriptor of empty range, which
           loads the same zeros without a memory request. Piece p of the fill
           lies in fragment p / 64 = i NVT + nt, so the choice is wave-uniform. */
        const __amdgpu_buffer_rsrc_t rz = buf_rsrc(rec0, 0);
        /* this chunk's shared operands: loads issued before the barrier that
           frees the LDS copy of the previous chunk, stores after it */
        u32x4 stage[FILL_ITERS];
        /* lanes past the last piece read outside the record's range (zeros, no
           branch around the load); their LDS stores below are skipped */
        auto piece_off = [&](int i) {
            const int p = i * NTH + tid;
            return (i + 1) * NTH <= PIECES || p < PIECES ? p * 16 : RL::BYTES;
        };
        if (L == KDA_CHUNK) {
#pragma unroll
            for (int i = 0; i < FILL_ITERS; i++) stage[i] = __builtin_amdgcn_raw_buffer_load_b128(r, piece_off(i), 0, 0);
        } else {
            const int nmt = (L + 15) >> 4, njb = (L + 31) >> 5;
            const int lim_p = nmt <= 2 ? nmt : 2 * nmt - 2;
            static_assert(3 * RL::NFR + 6 < 64 && (PIECES + 63) / 64 <= 64, "fragment mask");
            const uint64_t nfr_bits = (1ull << RL::NFR) - 1;
            const uint64_t wq = (1ull << (nmt * NKB)) - 1; /* W, Q': index mt NKB + kb */
            const uint64_t kt = njb == 2 ? nfr_bits : nfr_bits & 0x5555555555555555ull; /* ct 2 + jb */
            const uint64_t need = wq | wq << RL::NFR | kt << (2 * RL::NFR) |
                                  ((1ull << lim_p) - 1) << (3 * RL::NFR) | ~0ull << (3 * RL::NFR + 6);
#pragma unroll
            for (int i = 0; i < FILL_ITERS; i++) {
                const uint32_t f = __builtin_amdgcn_readfirstlane(i * NVT + nt); /* = piece / 64 */
                stage[i] = __builtin_amdgcn_raw_buffer_load_b128((need >> f) & 1 ? r : rz, piece_off(i), 0, 0);
            }
        }
        bf16x8 U[2];
        U[0] = bufld(r, l * 32, ubase);
        U[1] = bufld(L > 32 ? r : rz, l * 32, ubase + 16);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FILL_ITERS; i++) {
            const int p = i * NTH + tid;
            if (p < PIECES) *(u32x4 *)(opnd + p * 16) = stage[i];
        }
        __syncthreads();

        bf16x8 sb[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; kb++) sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
        /* D = U - W S; LDS operands are read in groups of eight fragments */
        f32x4 D[4];
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            const int o = (mt & 1) * 4;
            const bf16x8 &u = U[mt >> 1];
            D[mt] = f32x4{(float)u[o], (float)u[o + 1], (float)u[o + 2], (float)u[o + 3]};
        }
        bf16x8 fr[8];
#pragma unroll
        for (int half = 0; half < NKB / 2; half++) {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int kb = 2 * half + (i >> 2), mt = i & 3;
                fr[i] = ldsld(opnd, RL::W + (mt * NKB + kb) * 1024 + l * 16);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int kb = 2 * half + (i >> 2), mt = i & 3;
                D[mt] = mfma(fr[i], sb[kb], D[mt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        /* out^T = S^T Q'^T + U^T P^T */
        f32x4 O[4];
#pragma unroll
        for (int mt = 0; mt < 4; mt++) O[mt] = zero4();
#pragma unroll
        for (int half = 0; half < NKB / 2; half++) {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int kb = 2 * half + (i >> 2), mt = i & 3;
                fr[i] = ldsld(opnd, RL::Q + (mt * NKB + kb) * 1024 + l * 16);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int kb = 2 * half + (i >> 2), mt = i & 3;
                O[mt] = mfma(sb[kb], fr[i], O[mt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int f = 0; f < 6; f++) fr[f] = ldsld(opnd, RL::P + f * 1024 + l * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
            for (int jb = 0; jb <= (mt >> 1); jb++) O[mt] = mfma(U[jb], fr[KDA_PIDX(mt, jb)], O[mt]);
        __builtin_amdgcn_sched_barrier(0);
        const __amdgpu_buffer_rsrc_t ro =
            buf_rsrc(out + ((size_t)t0 * H + h) * DV, (uint32_t)((L - 1) * row_bytes + DV * 2));
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            u32x2 u;
            u[0] = pack_bf16x2(O[mt][0], O[mt][1]);
            u[1] = pack_bf16x2(O[mt][2], O[mt][3]);
            __builtin_amdgcn_raw_buffer_store_b64(u, ro, (16 * mt + n16) * row_bytes + (16 * nt + 4 * g) * 2, 0, 0);
        }

        /* S <- diag(e^{G_L}) S + K~^T D */
#pragma unroll
        for (int mt = 0; mt < NKT; mt++) S[mt] *= *(const f32x4 *)(opnd + RL::GL + mt * 64 + g * 16);
        bf16x8 db[2];
        db[0] = pack8(D[0], D[1]);
        db[1] = pack8(D[2], D[3]);
#pragma unroll
        for (int jb = 0; jb < 2; jb++) {
#pragma unroll
            for (int mt = 0; mt < NKT; mt++) fr[mt] = ldsld(opnd, RL::KT + (mt * 2 + jb) * 1024 + l * 16);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < NKT; mt++) S[mt] = mfma(fr[mt], db[jb], S[mt]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (state_fp32) {
#pragma unroll
        for (int mt = 0; mt < NKT; mt++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[mt][e]), rf, soff, (16 * mt + e) * DV * 4, 0);
    } else {
#pragma unroll
        for (int mt = 0; mt < NKT; mt++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                __builtin_amdgcn_raw_buffer_store_b16(f2bf_bits(S[mt][e]), rf, soff, (16 * mt + e) * DV * 2, 0);
    }
}

extern "C" __global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
kda_scan_many_kernel(const unsigned char *rec_base, const int32_t *__restrict__ cu,
                     const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H, int64_t nslots,
                     uint16_t *out, const void *init_state, void *final_state, int state_fp32, int64_t max_chunks)
{
    scan_many_body<4, 8>(rec_base, cu, chunk_off, nseq, T, H, nslots, out, init_state, final_state, state_fp32,
                         max_chunks);
}

/* K = V = 64: four waves per chain, every chain of any length */
extern "C" __global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
kda_scan_many_k64_kernel(const unsigned char *rec_base, const int32_t *__restrict__ cu,
                         const int32_t *__restrict__ chunk_off, int64_t nseq, int64_t T, int H, int64_t nslots,
                         uint16_t *out, const void *init_state, void *final_state, int state_fp32)
{
    scan_many_body<2, 4>(rec_base, cu, chunk_off, nseq, T, H, nslots, out, init_state, final_state, state_fp32,
                         INT64_MAX);
}

/* ------------------------------------------------------------------------- */
/* launcher (called by kda_api.cpp after validation)                           */
/* ------------------------------------------------------------------------- */
/*
 * With fewer than KDA_MANY_CHAINS (sequence, head) chains the three-wave kernel
 * runs them all (a CU per value tile hides the latency of a long chain, about
 * 1 us per chunk, for 32 chains at a time). With more, the eight-wave kernel
 * runs up to 512 chains at once (about 3-6 us per chunk, bound by memory
 * traffic): in a fixed-length batch all of them; in a packed batch every chain
 * of at most KDA_MANY_MAX_CHUNKS chunks, and the three-wave kernel then runs the
 * longer ones (a few long prompts among many short ones) from the list of long
 * sequences the chunk-table kernel leaves after chunk_off.
 */
#define KDA_MANY_CHAINS 128
/* from this many chains up (and below KDA_MANY_CHAINS) the pair scan
   (kda_scan_pair.hip, four CUs per chain instead of eight): 32 chains fill the
   GPU with the three-wave kernel's 256 workgroups (one CU each), beyond that
   they run in two or more rounds, while the pair scan runs 64 chains in one
   (dense batch, 64 chains of 32 chunks: scan 0.053 ms against 0.063 ms). With
   32 chains or fewer the three-wave kernel is faster (long prefill: 1.05 ms
   against 1.31 ms). */
#ifndef KDA_PAIR_MIN_CHAINS
#define KDA_PAIR_MIN_CHAINS 33
#endif

extern "C" hipError_t kda_launch_scan_pair(const void *records, const int32_t *cu, const int32_t *chunk_off,
                                           int64_t nseq, int64_t T, int64_t H, int64_t nslots, void *out,
                                           const void *init_state, void *final_state, int state_fp32,
                                           int64_t max_chains, const int32_t *long_list, hipStream_t st);

/* The longest sequence, in chunks, that kda_launch_scan gives to the many-chain
   kernel for these sizes (0: that kernel does not run). The chunk preparation
   leaves the padded fragments of those sequences' partial chunks unwritten,
   since that kernel reads them as zeros without touching memory. */
extern "C" int64_t kda_scan_many_max_chunks(const int32_t *cu, int64_t nseq, int64_t H, int64_t K, int64_t V,
                                            int64_t segc)
{
    if (nseq * H < KDA_MANY_CHAINS) return 0;
    if (K == 64 && V == 64) return INT64_MAX;
    if (segc > 0) return 0;
    return cu == nullptr ? INT64_MAX : (int64_t)KDA_MANY_MAX_CHUNKS;
}

extern "C" hipError_t kda_launch_scan(const void *records, const int32_t *cu, const int32_t *chunk_off,
                                      int64_t nseq, int64_t T, int64_t H, int64_t nslots, int64_t K, int64_t V,
                                      void *out, const void *init_state, void *final_state, int state_fp32,
                                      int64_t segc, void *seg_area, hipStream_t st)
{
    const unsigned char *rec = (const unsigned char *)records;
    const int64_t nchain = nseq * H;
    if (K == 64 && V == 64) {
        /* K = V = 64: the three-wave form (four value tiles per chain) for fewer
           than KDA_MANY_CHAINS chains, the many-chain form for more; each takes
           every chain of any length */
        if (nchain < KDA_MANY_CHAINS)
            hipLaunchKernelGGL(kda_scan_k64_kernel, dim3((unsigned)((nchain + 7) / 8 * 32)), dim3(192), 0, st, rec,
                               cu, chunk_off, nseq, T, (int)H, nslots, (uint16_t *)out, init_state, final_state,
                               state_fp32);
        else
            hipLaunchKernelGGL(kda_scan_many_k64_kernel, dim3((unsigned)nchain), dim3(256), 0, st, rec, cu,
                               chunk_off, nseq, T, (int)H, nslots, (uint16_t *)out, init_state, final_state,
                               state_fp32);
        return hipGetLastError();
    }
    if (K != KDA_DK || V != KDA_DV) return hipErrorInvalidValue;
    if (segc > 0) { /* segment-parallel (few long chains) */
        const int64_t G = kda_seg_slots(T, segc);
        float *area = (float *)seg_area;
        const int64_t ngrp = nchain * (G - 1);
        hipLaunchKernelGGL(kda_seg_map_kernel, dim3((unsigned)((ngrp + 7) / 8 * 128)), dim3(64), 0, st, rec, cu,
                           chunk_off, nchain, T, (int)H, nslots, G, segc, area);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kda_seg_chain_kernel, dim3((unsigned)((nchain + 7) / 8 * 64)), dim3(256), 0, st, area,
                           init_state, state_fp32, cu, T, (int)H, nchain, G, segc);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kda_scan_seg_kernel, dim3((unsigned)((nchain * G + 7) / 8 * 64)), dim3(192), 0, st, rec,
                           cu, chunk_off, nseq, T, (int)H, nslots, (uint16_t *)out, final_state, state_fp32, G, segc,
                           (const float *)(area + (size_t)2 * ngrp * KDA_DK * KDA_DV));
        return hipGetLastError();
    }
    if (nchain < KDA_MANY_CHAINS) {
        if (nchain >= KDA_PAIR_MIN_CHAINS)
            return kda_launch_scan_pair(rec, cu, chunk_off, nseq, T, H, nslots, out, init_state, final_state,
                                        state_fp32, nchain, nullptr, st);
        hipLaunchKernelGGL(kda_scan_kernel, dim3((unsigned)((nchain + 7) / 8 * 64)), dim3(192), 0, st, rec, cu,
                           chunk_off, nseq, T, (int)H, nslots, (uint16_t *)out, init_state, final_state, state_fp32,
                           (const int32_t *)nullptr);
        return hipGetLastError();
    }
    const int64_t max_chunks = kda_scan_many_max_chunks(cu, nseq, H, K, V, segc);
    hipLaunchKernelGGL(kda_scan_many_kernel, dim3((unsigned)nchain), dim3(512), 0, st, rec, cu, chunk_off, nseq, T,
                       (int)H, nslots, (uint16_t *)out, init_state, final_state, state_fp32, max_chunks);
    const hipError_t e = hipGetLastError();
    const int64_t max_long = kda_max_long_seqs(T);
    if (e != hipSuccess || cu == nullptr || max_long == 0) return e;
    hipLaunchKernelGGL(kda_scan_kernel, dim3((unsigned)((max_long * H + 7) / 8 * 64)), dim3(192), 0, st, rec, cu,
                       chunk_off, nseq, T, (int)H, nslots, (uint16_t *)out, init_state, final_state, state_fp32,
                       chunk_off + nseq + 1);
    return hipGetLastError();
}
