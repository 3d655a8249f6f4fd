// Greedy acceptance: vocab argmax of every verify row, then the walk.
//
// Greedy verification [single-RTX-3090 DFlash note, "Architecture"] accepts a
// draft token iff it equals the target's argmax at the draft's parent; over a
// DDTree the longest accepted root path is kept and the target's argmax at its
// last node is the bonus token ["From autoregressive to DDTree"; the verifier
// reads budget+1 logits rows, "Key breakthroughs"].
//
// One launch.  Workgroup (row, chunk) streams `chunk` logits of one row with
// 16-byte loads (up to 8 per thread in flight at once) and reduces them to a
// 64-bit key
//     (order-preserving fp32 bits << 32) | (0xFFFFFFFF - index),
// whose maximum is the largest value at the lowest index (wavefront maxima by
// DPP lane moves).  Completion is tracked with device-scope atomics only (no
// cache flushes):
//   1. atomic max of the key into keys[row]; wait for its return;
//   2. add 1 to done[b]; the workgroup that brings it to N * chunks (the last
//      arrival of sequence b) sets it back to zero, takes every key of the
//      sequence with an atomic exchange against zero, runs the acceptance walk
//      for its <= 64 nodes in one wavefront and writes the outputs.
// Each step is issued only after the previous atomic has returned, and all of
// them act on the device-coherent copy, so the last workgroup sees every
// key.  Every call leaves the keys and counters it used at zero.
#include "device_common.h"

namespace sv {
namespace {

__device__ __forceinline__ unsigned long long make_key(float v, uint32_t idx) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;                      // -0 ties with +0
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

// one DPP step of a 64-bit running maximum: lanes outside the move's source
// range (and rows outside `rmask`) contribute the identity 0
#define SV_DPP_MAX64(k, ctrl, rmask)                                                                      \
    do {                                                                                               \
        const uint32_t lo_ = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k), ctrl, rmask, 0xf, false); \
        const uint32_t hi_ = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)((k) >> 32), ctrl, rmask, 0xf, false); \
        k = umax64(k, ((unsigned long long)hi_ << 32) | lo_);                                         \
    } while (0)

// maximum over the 64 lanes (row shifts 1, 2, 4, 8, then the broadcasts of
// lanes 15 and 31 leave the running maximum of all lanes in lane 63)
__device__ __forceinline__ unsigned long long wave_max64(unsigned long long k) {
    SV_DPP_MAX64(k, 0x111, 0xf);
    SV_DPP_MAX64(k, 0x112, 0xf);
    SV_DPP_MAX64(k, 0x114, 0xf);
    SV_DPP_MAX64(k, 0x118, 0xf);
    SV_DPP_MAX64(k, 0x142, 0xa);
    SV_DPP_MAX64(k, 0x143, 0xc);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 63);
    return ((unsigned long long)hi << 32) | lo;
}

// vmcnt(0): every vector memory operation of this wave (the atomics above
// included, their results returned) has completed
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <bool F32, bool VEC>
__global__ __launch_bounds__(256) void argmax_accept_kernel(AcceptParams p) {
    __shared__ unsigned long long red[4];
    __shared__ int last_s;
    __shared__ int am_s[64], dr_s[64], par_s[64];

    const int c = blockIdx.x % p.n_chunks;
    const int row = blockIdx.x / p.n_chunks;             // b * N + i
    const int b = row / p.N;
    const int tid = threadIdx.x;
    const int64_t V = p.V;
    const int64_t lo = (int64_t)c * p.chunk;
    const int64_t hi = min<int64_t>(V, lo + p.chunk);
    constexpr int EPL = F32 ? 4 : 8;                      // elements per 16-byte load
    constexpr int UNR = 8;                                // loads in flight per thread

    unsigned long long best = 0ull;
    if constexpr (VEC) {
        // full groups of UNR loads, then the rest one load at a time
        const void *base = F32 ? (const void *)((const float *)p.logits + (int64_t)row * V)
                               : (const void *)((const uint16_t *)p.logits + (int64_t)row * V);
        int64_t e = lo + (int64_t)tid * EPL;
        for (; e + (int64_t)(UNR - 1) * 256 * EPL < hi; e += (int64_t)UNR * 256 * EPL) {
            u32x4 v[UNR];
#pragma unroll
            for (int k = 0; k < UNR; ++k)
                v[k] = *(const u32x4 *)((const uint8_t *)base + (e + (int64_t)k * 256 * EPL) * (F32 ? 4 : 2));
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const uint32_t i0 = (uint32_t)(e + (int64_t)k * 256 * EPL);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if constexpr (F32) {
                        best = umax64(best, make_key(__uint_as_float(v[k][t]), i0 + t));
                    } else {
                        best = umax64(best, make_key(bf16_bits_to_f32(v[k][t] & 0xFFFFu), i0 + 2 * t));
                        best = umax64(best, make_key(bf16_bits_to_f32(v[k][t] >> 16), i0 + 2 * t + 1));
                    }
                }
            }
        }
        for (; e < hi; e += 256 * EPL) {
            const u32x4 v = *(const u32x4 *)((const uint8_t *)base + e * (F32 ? 4 : 2));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if constexpr (F32) {
                    best = umax64(best, make_key(__uint_as_float(v[t]), (uint32_t)(e + t)));
                } else {
                    best = umax64(best, make_key(bf16_bits_to_f32(v[t] & 0xFFFFu), (uint32_t)(e + 2 * t)));
                    best = umax64(best, make_key(bf16_bits_to_f32(v[t] >> 16), (uint32_t)(e + 2 * t + 1)));
                }
            }
        }
    } else if constexpr (F32) {
        const float *rowp = (const float *)p.logits + (int64_t)row * V;
        for (int64_t e = lo + tid; e < hi; e += 256) best = umax64(best, make_key(rowp[e], (uint32_t)e));
    } else {
        const uint16_t *rowp = (const uint16_t *)p.logits + (int64_t)row * V;
        for (int64_t e = lo + tid; e < hi; e += 256)
            best = umax64(best, make_key(bf16_bits_to_f32(rowp[e]), (uint32_t)e));
    }
    best = wave_max64(best);
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
        const unsigned long long k = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
        // consuming `was` keeps the returning form of the atomic, whose
        // result comes back only once it has been performed
        const unsigned long long was =
            __hip_atomic_fetch_max(&p.keys[row], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" : : "v"((uint32_t)was));
        wait_vm0();
        const unsigned int done =
            __hip_atomic_fetch_add(&p.seqs_done[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_s = done == (unsigned int)(p.N * p.n_chunks - 1);
    }
    __syncthreads();
    if (!last_s) return;

    // ---- the last arrival of sequence b: take keys, then walk -----------------
    const int N = p.N;
    const int wave = tid >> 6, lane = tid & 63;
    if (wave != 0) return;
    if (lane == 0) __hip_atomic_store(&p.seqs_done[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane < N) {
        const unsigned long long k =
            __hip_atomic_exchange(&p.keys[(int64_t)b * N + lane], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        am_s[lane] = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
        dr_s[lane] = p.draft[(int64_t)b * N + lane];
        par_s[lane] = p.parent[(int64_t)b * N + lane];
    }
    __builtin_amdgcn_s_waitcnt(0);           // the LDS writes of all lanes (one wave: no barrier)
    __builtin_amdgcn_wave_barrier();

    // node `lane`: accepted iff every edge of its root path is accepted
    int acc = 0, depth = 0;
    if (lane < N) {
        acc = 1;
        int j = lane;
#pragma unroll 1
        for (int step = 0; step < 64 && j > 0; ++step) {
            const int pj = par_s[j];
            if (pj < 0 || pj >= j) { acc = 0; break; }
            if (dr_s[j] != am_s[pj]) acc = 0;
            ++depth;
            j = pj;
        }
    }
    // deepest accepted node, ties to the smallest index (node 0 always qualifies)
    unsigned int key = acc ? (((unsigned)depth << 8) | (unsigned)(255 - lane)) : 0u;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) key = max(key, (unsigned)__shfl_xor((int)key, m, 64));
    const int best_node = 255 - (int)(key & 255u);
    const int a = (int)(key >> 8);

    int32_t *path = p.path + (int64_t)b * N;
    int32_t *tok = p.tokens + (int64_t)b * N;
    if (lane == 0) {
        int j = best_node;
        for (int d = a; d >= 0; --d) {
            path[d] = j;
            if (d > 0) tok[d - 1] = dr_s[j];
            j = (j > 0) ? par_s[j] : 0;
        }
        tok[a] = am_s[best_node];
        p.accept_len[b] = a;
    }
    if (lane < N && lane > a) {
        path[lane] = -1;
        tok[lane] = -1;
    }
    if (p.argmax != nullptr && lane < N) p.argmax[(int64_t)b * N + lane] = am_s[lane];
}

}  // namespace

hipError_t launch_accept(const AcceptParams &p, hipStream_t st) {
    const int grid = p.B * p.N * p.n_chunks;
    const int esize = p.logits_f32 ? 4 : 2;
    const bool vec = ((uintptr_t)p.logits % 16 == 0) && (((int64_t)p.V * esize) % 16 == 0) &&
                     ((int64_t)p.chunk * esize) % 16 == 0;
    if (p.logits_f32) {
        if (vec) hipLaunchKernelGGL((argmax_accept_kernel<true, true>), dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL((argmax_accept_kernel<true, false>), dim3(grid), dim3(256), 0, st, p);
    } else {
        if (vec) hipLaunchKernelGGL((argmax_accept_kernel<false, true>), dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL((argmax_accept_kernel<false, false>), dim3(grid), dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace sv
