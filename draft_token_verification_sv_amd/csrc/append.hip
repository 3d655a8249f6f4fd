// Writing the verify block's K/V rows into the cache, quantised at write time
// for a 4-bit cache.
//
// The rows are stored before attention reads the cache, and a 4-bit cache
// converts them as they are written [single-RTX-3090 DFlash note, "128K
// context in 24 GB": the KV cache kept in 4 bits, read by flash attention].
// Row i of sequence b lands at position ctx_b + i.  One wavefront per (row,
// KV head, K|V): lane l holds head-dim values 4l .. 4l+3 (16-byte fp32 or
// 8-byte bf16 loads).
//   fp32 cache: the values;  bf16 cache: round to nearest even;
//   4-bit cache: per 32-value block (8 lanes) d = half(max|x| / 7) with the
//   division in fp32 then round to nearest even into half precision; code =
//   clamp(rint(x / d), -8, 7) + 8 (fp32 division, ties to even), 8 when d = 0;
//   lane l writes bytes 2l and 2l+1 (value 2t in the low nibble of byte t),
//   the block's first lane its scale.
#include "device_common.h"

namespace sv {
namespace {

template <int SRC, int DST>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t rows = (int64_t)p.B * p.n * p.Hkv * 2;
    if (id >= rows) return;
    const int which = (int)(id & 1);                    // 0: K, 1: V
    int64_t rest = id >> 1;
    const int h = (int)(rest % p.Hkv);
    rest /= p.Hkv;
    const int i = (int)(rest % p.n);
    const int b = (int)(rest / p.n);
    const int D = p.D;
    if (4 * lane >= D) return;
    const int pos = ctx_of(p.ctx_lens, b, p.max_ctx, p.err) + i;
    const int64_t ri = kv_row_index(p.kv, b, p.Hkv, h, pos, p.err);
    if (ri < 0) return;

    // the lane's 4 source values
    const int64_t src_off = (((int64_t)b * p.n + i) * p.Hkv + h) * D + 4 * lane;
    const void *src = which ? p.v_new : p.k_new;
    float x[4];
    if constexpr (SRC == SV_F32) {
        const f32x4 v = *(const f32x4 *)((const float *)src + src_off);
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = v[k];
    } else {
        const u32x2 v = *(const u32x2 *)((const uint16_t *)src + src_off);
        x[0] = bf16_bits_to_f32(v[0] & 0xFFFFu);
        x[1] = bf16_bits_to_f32(v[0] >> 16);
        x[2] = bf16_bits_to_f32(v[1] & 0xFFFFu);
        x[3] = bf16_bits_to_f32(v[1] >> 16);
    }

    uint8_t *dst = (uint8_t *)(which ? p.kv.v : p.kv.k);
    if constexpr (DST == SV_F32) {
        *(f32x4 *)((float *)dst + ri * D + 4 * lane) = f32x4{x[0], x[1], x[2], x[3]};
    } else if constexpr (DST == SV_BF16) {
        const u32x2 o = {f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16),
                         f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16)};
        *(u32x2 *)((uint16_t *)dst + ri * D + 4 * lane) = o;
    } else {
        // block maximum over the block's 8 lanes (lane groups of 8 are aligned)
        float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        const _Float16 dh = (_Float16)(amax / 7.0f);     // fp32 divide, round to nearest even half
        const float d = (float)dh;
        uint32_t c[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float q = d == 0.f ? 0.f : fminf(fmaxf(rintf(x[k] / d), -8.f), 7.f);
            c[k] = (uint32_t)((int)q + 8);
        }
        const uint16_t bytes = (uint16_t)((c[0] | (c[1] << 4)) | ((c[2] | (c[3] << 4)) << 8));
        *(uint16_t *)(dst + ri * (D / 2) + 2 * lane) = bytes;
        if ((lane & 7) == 0) {
            uint8_t *sdst = (uint8_t *)(which ? p.kv.vs : p.kv.ks);
            *(uint16_t *)(sdst + ri * (D / 32) * 2 + (lane / 8) * 2) = __builtin_bit_cast(uint16_t, dh);
        }
    }
}

template <int SRC>
hipError_t launch_src(const AppendParams &p, int dst, hipStream_t st) {
    const int64_t rows = (int64_t)p.B * p.n * p.Hkv * 2;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (dst == SV_F32) hipLaunchKernelGGL((kv_append_kernel<SRC, SV_F32>), grid, dim3(256), 0, st, p);
    else if (dst == SV_BF16) hipLaunchKernelGGL((kv_append_kernel<SRC, SV_BF16>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((kv_append_kernel<SRC, SV_Q4>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendParams &p, int src_dtype, int dst_dtype, hipStream_t st) {
    return src_dtype == SV_F32 ? launch_src<SV_F32>(p, dst_dtype, st) : launch_src<SV_BF16>(p, dst_dtype, st);
}

}  // namespace sv
