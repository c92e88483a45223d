/*
 * kda_internal.h -- layouts shared by the libkda kernels and host launcher.
 * Not installed; the public interface is include/kda.h.
 *
 * Chunked evaluation (derived from the gated delta rule; the FlashKDA pages
 * describe a chunked kernel for it without formulas). Per sequence and head,
 * tokens are cut into chunks of 64 that restart at every sequence start. For a
 * chunk of L <= 64 tokens with state S entering it and G = inclusive cumsum of
 * log a over the chunk (per key channel):
 *   A_rj = beta_r sum_c k^_r k^_j e^{G_r - G_j}   (j < r),   T = (I + A)^-1
 *   W = T diag(beta) (K^ o e^G),   U = T diag(beta) V,   D = U - W S
 *   P_rj = scale sum_c q^_r k^_j e^{G_r - G_j}   (j <= r)
 *   Q' = scale (Q^ o e^G) - P W
 *   out = Q' S + P U                  (= scale [(Q^ o e^G) S + P_unscaled D])
 *   S  <- diag(e^{G_L}) S + (K^ o e^{G_L - G})^T D
 * A "prep" kernel forms everything that does not depend on S for all chunks in
 * parallel and stores it as a per-(chunk, head) record; a "scan" kernel walks
 * the chunks of each (sequence, head) in order, keeping S in registers.
 *
 * Record operands are stored in the exact register layout of the gfx950
 * v_mfma_f32_16x16x32_bf16 operands the scan issues, so every scan load is a
 * contiguous 16-byte (or 32-byte) read per lane:
 *   "fragment" = 64 lanes x 8 bf16 = 1 KiB. Lane l covers row (l % 16) of a
 *   16-row tile; its 8 values cover the 32-wide contraction block in the order
 *   kperm(g, i) = i < 4 ? 4g + i : 16 + 4g + (i - 4),  g = l / 16,
 *   which is the order in which a pair of 16x16 fp32 accumulator tiles holds
 *   rows (4g + e) -- so an accumulator pair converts to an operand in place.
 */
#ifndef KDA_INTERNAL_H
#define KDA_INTERNAL_H

#include <stddef.h>
#include <stdint.h>

#define KDA_CHUNK 64
#define KDA_DK 128
#define KDA_DV 128

/* byte offsets inside one (chunk, head) record */
#define KDA_REC_W 0          /* -W   : 16 fragments, index mt*4 + kb (mt: token tile, kb: key block) */
#define KDA_REC_Q 16384      /* Q'   : 16 fragments, index mt*4 + kb                                  */
#define KDA_REC_KT 32768     /* Kt^T : 16 fragments, index ct*2 + jb (ct: key tile, jb: token block) */
#define KDA_REC_P 49152      /* P    : 6 fragments (lower triangle), index kda_pidx(mt, jb)           */
#define KDA_REC_GL 55296     /* e^{G_L}: 128 fp32, key-channel order                               */
#define KDA_REC_U 55808      /* U    : [8 value tiles][64 lanes][4 token tiles][4] bf16              */
#define KDA_REC_BYTES 72192

/* The same layout for any head dims DK = 32 NKB key channels and DV = 16 NVT
 * value columns (K, V in {64, 128}): NKB key blocks of 32 channels, NVT value
 * tiles of 16 columns; W and Q' hold 4 NKB fragments (index mt * NKB + kb),
 * K~^T 4 NKB (index ct * 2 + jb over the 2 NKB key tiles ct), P 6, e^{G_L} DK
 * floats, U NVT x 64 lanes x 16 bf16. RecLayout<4, 8> is the layout above. */
template <int NKB, int NVT> struct RecLayout {
    static constexpr int NFR = 4 * NKB;
    static constexpr int W = 0, Q = NFR * 1024, KT = 2 * NFR * 1024, P = 3 * NFR * 1024;
    static constexpr int GL = P + 6 * 1024, U = GL + 128 * NKB, BYTES = U + NVT * 2048;
};
static_assert(RecLayout<4, 8>::Q == KDA_REC_Q && RecLayout<4, 8>::KT == KDA_REC_KT &&
                  RecLayout<4, 8>::P == KDA_REC_P && RecLayout<4, 8>::GL == KDA_REC_GL &&
                  RecLayout<4, 8>::U == KDA_REC_U && RecLayout<4, 8>::BYTES == KDA_REC_BYTES,
              "record layout");

/* record bytes for head dims K, V in {64, 128} (at most KDA_REC_BYTES) */
static inline size_t kda_rec_bytes(int64_t K, int64_t V)
{
    return (size_t)(3 * 4 * (K / 32) * 1024 + 6 * 1024 + 4 * K + (V / 16) * 2048);
}

/* fragment index of P(mt, jb); only jb <= mt / 2 exists */
#define KDA_PIDX(mt, jb) ((mt) < 2 ? (mt) : 2 + 2 * ((mt) - 2) + (jb))

/* In a packed (varlen) batch with many chains, sequences of more than
 * KDA_MANY_MAX_CHUNKS chunks are scanned by the three-wave kernel and the rest
 * by the eight-wave kernel. At most kda_max_long_seqs(T) of T packed tokens. */
#define KDA_MANY_MAX_CHUNKS 128
static inline int64_t kda_max_long_seqs(int64_t T) { return T / (KDA_MANY_MAX_CHUNKS * KDA_CHUNK + 1); }

/* workspace = [chunk table, padded to 256 B][records]
 * The chunk table (varlen only) is int32: chunk_off[N + 1], then the number of
 * long sequences and their indices in ascending order (kda_max_long_seqs slots).
 * Records are head-major, record(slot, h) at (h * nslots + slot) * KDA_REC_BYTES
 * with nslots = kda_max_chunks(...), so the chunks of one (sequence, head) that
 * the scan walks in order are adjacent in memory. */
static inline size_t kda_chunk_map_bytes(int64_t num_seqs, int64_t T)
{
    return num_seqs > 0 ? (size_t)(((num_seqs + 2 + kda_max_long_seqs(T)) * 4 + 255) / 256 * 256) : 0;
}

/* upper bound on the number of chunks: exact without cu_seqlens */
static inline int64_t kda_max_chunks(int64_t B, int64_t T, int64_t num_seqs)
{
    if (num_seqs > 0)
        return T / KDA_CHUNK + num_seqs;
    return B * ((T + KDA_CHUNK - 1) / KDA_CHUNK);
}

/* Segment-parallel scan (few, long chains: B * H or num_seqs * H <= 10). The
 * chunks of each chain are cut into segments of kda_seg_len chunks (about 32
 * segments over all chains, at least 16 chunks each; a sequence's last segment
 * takes the rest). The state after a segment is an affine function of the state
 * entering it, S -> M S + B; M and B of every segment are computed in parallel,
 * chained in a short pass, and each segment is then rescanned from its entering
 * state. kda_seg_len returns 0 (the plain scan) unless the longest possible
 * sequence has at least 3 segments. */
static inline int64_t kda_seg_len(int64_t B, int64_t T, int64_t H, int64_t num_seqs)
{
    if (B <= 0 || T <= 0 || H <= 0 || num_seqs < 0) return 0;
    const int64_t nchain = (num_seqs > 0 ? num_seqs : B) * H;
    if (nchain > 10) return 0;
    const int64_t maxc = (T + KDA_CHUNK - 1) / KDA_CHUNK;   /* chunks of the longest possible sequence */
    const int64_t total = num_seqs > 0 ? maxc : B * maxc;   /* chunks over all sequences (about) */
    int64_t segc = (total * H + 31) / 32;
    if (segc < 16) segc = 16;
    return (maxc + segc - 1) / segc >= 3 ? segc : 0;
}
/* segment slots per chain: the most segments a sequence of at most T tokens has */
static inline int64_t kda_seg_slots(int64_t T, int64_t segc)
{
    return ((T + KDA_CHUNK - 1) / KDA_CHUNK + segc - 1) / segc;
}
/* segment area after the records (fp32 128 x 128 blocks), G = kda_seg_slots:
 * M and B of segment slots 0 .. G-2, [chains][G - 1] each, then the entering
 * states of slots 0 .. G-1, [chains][G] (slot 0's is the initial state, copied) */
static inline size_t kda_seg_bytes(int64_t B, int64_t T, int64_t H, int64_t num_seqs)
{
    const int64_t segc = kda_seg_len(B, T, H, num_seqs);
    if (segc == 0) return 0;
    const int64_t G = kda_seg_slots(T, segc), nchain = (num_seqs > 0 ? num_seqs : B) * H;
    return (size_t)nchain * (size_t)(3 * G - 2) * KDA_DK * KDA_DV * 4;
}

/* ---- backward (kda_bwd) ----
 * Per (chunk, head) fp32 area written by the chunk kernel, offsets in floats,
 * rows are the chunk's 64 token positions (rows past the chunk's end are 0):
 *   W, U, Q' (scale included), K~ = k^ o e^{G_L - G}, q^, k^, G   [64][128] each,
 *   T = (I + A)^-1 and P (scale included, j <= i)                  [64][64] each,
 *   e^{G_L} [128], beta [64], |q| and |k| norms sqrt(|x|^2 + 1e-6) [64] each.
 * Areas are head-major like the forward records: (h * nslots + slot). */
#define KDA_BR_W 0
#define KDA_BR_U 8192
#define KDA_BR_QP 16384
#define KDA_BR_KT 24576
#define KDA_BR_QN 32768
#define KDA_BR_KN 40960
#define KDA_BR_G 49152
#define KDA_BR_T 57344
#define KDA_BR_P 61440
#define KDA_BR_GL 65536
#define KDA_BR_BETA 65664
#define KDA_BR_NQ 65728
#define KDA_BR_NK 65792
#define KDA_BR_FLOATS 66048
/* per (chunk, head) gate partials: d dt_bias [128], then d A_log */
#define KDA_BWD_PART_FLOATS 132
/* scratch of one gradient workgroup: 14 [64][128] and 3 [64][64] fp32 matrices */
#define KDA_BWD_SCR_FLOATS (14 * 8192 + 3 * 4096)
/* at most this many gradient workgroups (each loops over (chunk, head) items) */
#define KDA_BWD_GRAD_WGS 1024

/* backward workspace = [chunk table][chunk areas][S at each chunk start]
 * [dS at each chunk end][gate partials][gradient scratch]; every part is a
 * multiple of 256 bytes */
static inline size_t kda_bwd_grad_wgs(int64_t items)
{
    return (size_t)(items < KDA_BWD_GRAD_WGS ? items : KDA_BWD_GRAD_WGS);
}
static inline size_t kda_bwd_part_bytes(int64_t items)
{
    return ((size_t)items * KDA_BWD_PART_FLOATS * 4 + 255) / 256 * 256;
}

#endif
