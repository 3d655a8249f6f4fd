// Device helpers shared by the gfx950 kernels: number formats, the tree mask,
// KV row addressing, wavefront reductions.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "sv_internal.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    __bf16 h = (__bf16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// two fp32 -> packed bf16 pair (lo in bits 0-15), round to nearest even, one
// v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t h = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Low (sel=0) or high (sel=1) 16-bit halves of a and b packed as (a_half, b_half).
__device__ __forceinline__ uint32_t pack_lo_halves(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi_halves(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Precondition reports (sv_check_device_errors): in a build with SV_DEBUG a
// kernel that meets a broken device-side input ORs its bit into the word;
// release builds compile the checks away.
#ifdef SV_DEBUG
#define SV_DEVCHECK(err, cond, bit)                                   \
    do {                                                              \
        if ((err) != nullptr && (cond)) atomicOr((err), (unsigned)(bit)); \
    } while (0)
#else
#define SV_DEVCHECK(err, cond, bit) \
    do {                            \
    } while (0)
#endif

// Ancestor-or-self bit set of every node of one tree, built from the parent
// array in LDS.  `par` holds parent[0..n-1]; a parent that is not an earlier
// node ends the walk (no out-of-range access, bounded by n steps).
__device__ __forceinline__ uint64_t ancestor_bits(const int *par, int i) {
    uint64_t a = 1ull << i;
    int j = i;
#pragma unroll 1
    for (int step = 0; step < 64 && j > 0; ++step) {
        const int pj = par[j];
        if (pj < 0 || pj >= j) break;
        a |= 1ull << pj;
        j = pj;
    }
    return a;
}

// Row number of KV row (b, h, pos) in the cache arrays (rows of any width); -1
// when the page id is outside the pool (the row is then read as zeros and
// never written).
__device__ __forceinline__ int64_t kv_row_index(const KvView &kv, int b, int Hkv, int h, int pos,
                                                unsigned int *err = nullptr) {
    if (kv.page_table == nullptr) {
        return ((int64_t)b * Hkv + h) * kv.capacity + pos;
    }
    const int ps = kv.page_size;
    const int page = kv.page_table[(int64_t)b * kv.max_pages + pos / ps];
    if (page < 0 || page >= kv.capacity) {
        SV_DEVCHECK(err, true, SV_DEVERR_PAGE);
        return -1;
    }
    return ((int64_t)page * Hkv + h) * ps + (pos % ps);
}

__device__ __forceinline__ int clamp_ctx(int c, int max_ctx) {
    return c < 0 ? 0 : (c > max_ctx ? max_ctx : c);
}

// ctx_lens[b], clamped to [0, max_ctx] (out-of-range values reported)
__device__ __forceinline__ int ctx_of(const int32_t *ctx_lens, int b, int max_ctx, unsigned int *err) {
    const int c = ctx_lens[b];
    SV_DEVCHECK(err, c < 0 || c > max_ctx, SV_DEVERR_CTX);
    return clamp_ctx(c, max_ctx);
}

// parent[b][i] (row pointer `par_row`); an entry of node i >= 1 outside
// [0, i) is reported (the walks treat it as the end of the path)
__device__ __forceinline__ int parent_of(const int32_t *par_row, int i, unsigned int *err) {
    const int v = par_row[i];
    SV_DEVCHECK(err, i >= 1 && (v < 0 || v >= i), SV_DEVERR_PARENT);
    return v;
}

// XOR lane exchange within a wavefront of 64
__device__ __forceinline__ float xor_shfl(float v, int m) {
    return __shfl_xor(v, m, 64);
}

}  // namespace sv
