/*
 * kda_device.h -- device helpers shared by the libkda kernels (gfx950 only).
 * Layout conventions are described in kda_internal.h.
 */
#ifndef KDA_DEVICE_H
#define KDA_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

namespace kda_dev {

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

/* position inside a 32-wide contraction block of operand slot i of lane group g */
__device__ __forceinline__ int kperm(int g, int i) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f2bf_bits(float x)
{
    __bf16 b = (__bf16)x; /* round to nearest even */
    return __builtin_bit_cast(uint16_t, b);
}

/* two floats -> a packed bf16 pair (a in the low half), round to nearest even; one
   v_cvt_pk_bf16_f32 */
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 pack8(const f32x4 &a, const f32x4 &b)
{
    bf16x8 r;
    r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
    r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
    return r;
}

__device__ __forceinline__ bf16x8 pack8f(const float *x)
{
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = (__bf16)x[i];
    return r;
}

#define KDA_BUF_FLAGS 0x00020000 /* raw buffer, 32-bit data format (gfx9 family) */

/* Buffer descriptor over [base, base + bytes): the base lives in SGPRs, lanes
   pass 32-bit byte offsets, loads past the end return 0 and stores past the end
   are dropped by the hardware range check. */
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, KDA_BUF_FLAGS);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

/* inclusive prefix sum over the 16 lanes of a DPP row */
__device__ __forceinline__ float row_scan16(float x)
{
    int v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true));
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true));
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

/* sequence / chunk of a chunk slot; returns false for slots past the end */
__device__ __forceinline__ bool locate_chunk(int64_t slot, const int32_t *cu, const int32_t *chunk_off,
                                             int64_t nseq, int64_t T, int64_t &t0, int &L, int64_t &seq)
{
    if (cu == nullptr) {
        const int64_t cps = (T + KDA_CHUNK - 1) / KDA_CHUNK;
        seq = slot / cps;
        const int64_t c = slot - seq * cps;
        t0 = seq * T + c * KDA_CHUNK;
        const int64_t rem = T - c * KDA_CHUNK;
        L = (int)(rem < KDA_CHUNK ? rem : KDA_CHUNK);
        return true;
    }
    if (slot >= chunk_off[nseq]) return false;
    int64_t lo = 0, hi = nseq - 1; /* largest n with chunk_off[n] <= slot */
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= slot) lo = mid; else hi = mid - 1;
    }
    seq = lo;
    const int64_t c = slot - chunk_off[lo];
    t0 = cu[lo] + c * KDA_CHUNK;
    const int64_t rem = cu[lo + 1] - t0;
    L = (int)(rem < KDA_CHUNK ? rem : KDA_CHUNK);
    return true;
}

} // namespace kda_dev
using namespace kda_dev;

#endif
