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

/* Segment-parallel scan (fixed-length batches with few, long chains): the
 * chunks of each chain are cut into G segments of kda_seg_chunks chunks (the
 * last takes the rest). The state after a segment is an affine function of the
 * state entering it, S -> M S + B; M and B of every segment are computed in
 * parallel, chained in a short pass, and each segment is then rescanned from
 * its entering state. G = 1 means the plain scan. */
static inline int64_t kda_scan_segments(int64_t B, int64_t T, int64_t H, int64_t num_seqs)
{
    if (num_seqs > 0 || B <= 0 || T <= 0 || H <= 0) return 1;
    const int64_t nchain = B * H, nchunk = (T + KDA_CHUNK - 1) / KDA_CHUNK;
    if (nchain > 16) return 1;
    int64_t G = 32 / nchain;           /* about 256 workgroups in the rescan */
    if (G > nchunk / 16) G = nchunk / 16; /* segments of at least 16 chunks */
    while (G >= 3 && (G - 1) * ((nchunk + G - 1) / G) >= nchunk) G--; /* every segment non-empty */
    return G >= 3 ? G : 1;
}
static inline int64_t kda_seg_chunks(int64_t T, int64_t G)
{
    const int64_t nchunk = (T + KDA_CHUNK - 1) / KDA_CHUNK;
    return (nchunk + G - 1) / G;
}
/* segment area after the records (fp32 128 x 128 blocks): M and B of segments
 * 0 .. G-2, [B * H][G - 1] each, then the entering states of segments 0 .. G-1,
 * [B * H][G] (segment 0's is the initial state, copied) */
static inline size_t kda_seg_bytes(int64_t B, int64_t T, int64_t H, int64_t num_seqs)
{
    const int64_t G = kda_scan_segments(B, T, H, num_seqs);
    return G > 1 ? (size_t)(B * H) * (size_t)(3 * G - 2) * KDA_DK * KDA_DV * 4 : 0;
}

#endif
