// Greedy acceptance: vocab argmax of every verify row, then the walk.
//
// Greedy verification [single-RTX-3090 DFlash note, "Architecture"] accepts a
// draft token iff it equals the target's argmax at the draft's parent; over a
// DDTree the longest accepted root path is kept and the target's argmax at its
// last node is the bonus token ["From autoregressive to DDTree"; the verifier
// reads budget+1 logits rows, "Key breakthroughs"].
//
// One launch.  Workgroup (row, chunk) streams `chunk` logits of one row with
// 16-byte loads and reduces them to a 64-bit key
//     (order-preserving fp32 bits << 32) | (0xFFFFFFFF - index),
// whose maximum is the largest value at the lowest index.  The key is stored
// to the workspace, then a per-sequence counter is incremented; the workgroup
// that brings the counter to N * chunks (the last one of that sequence) reads
// all keys of the sequence, runs the acceptance walk for its <= 64 nodes in
// one wavefront, writes the outputs and sets its keys and counter back to
// zero, so the whole workspace is zero between calls of any shape.
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

__device__ __forceinline__ unsigned long long wave_max64(unsigned long long k) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, m, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), m, 64);
        k = umax64(k, ((unsigned long long)hi << 32) | lo);
    }
    return k;
}

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

    unsigned long long best = 0ull;
    if constexpr (F32) {
        const float *rowp = (const float *)p.logits + (int64_t)row * V;
        if constexpr (VEC) {
            for (int64_t e = lo + tid * 4; e < hi; e += 256 * 4) {
                const f32x4 v = *(const f32x4 *)(rowp + e);
#pragma unroll
                for (int t = 0; t < 4; ++t) best = umax64(best, make_key(v[t], (uint32_t)(e + t)));
            }
        } else {
            for (int64_t e = lo + tid; e < hi; e += 256) best = umax64(best, make_key(rowp[e], (uint32_t)e));
        }
    } else {
        const uint16_t *rowp = (const uint16_t *)p.logits + (int64_t)row * V;
        if constexpr (VEC) {
            for (int64_t e = lo + tid * 8; e < hi; e += 256 * 8) {
                const u32x4 v = *(const u32x4 *)(rowp + e);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    best = umax64(best, make_key(bf16_bits_to_f32(v[t] & 0xFFFFu), (uint32_t)(e + 2 * t)));
                    best = umax64(best, make_key(bf16_bits_to_f32(v[t] >> 16), (uint32_t)(e + 2 * t + 1)));
                }
            }
        } else {
            for (int64_t e = lo + tid; e < hi; e += 256)
                best = umax64(best, make_key(bf16_bits_to_f32(rowp[e]), (uint32_t)e));
        }
    }
    best = wave_max64(best);
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
        const unsigned long long k = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
        p.keys[(int64_t)row * p.n_chunks + c] = k;
        __threadfence();
        const unsigned int prev = atomicAdd(&p.counters[b], 1u);
        last_s = (prev == (unsigned int)(p.N * p.n_chunks - 1));
    }
    __syncthreads();
    if (!last_s) return;

    // ---- last workgroup of sequence b: reduce keys, then walk ----------------
    __threadfence();
    const int N = p.N;
    const int wave = tid >> 6, lane = tid & 63;
    for (int i = wave; i < N; i += 4) {
        const unsigned long long *kp = p.keys + ((int64_t)b * N + i) * p.n_chunks;
        unsigned long long k = 0ull;
        for (int cc = lane; cc < p.n_chunks; cc += 64)
            k = umax64(k, __hip_atomic_load(kp + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        k = wave_max64(k);
        if (lane == 0) am_s[i] = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
    }
    if (tid < N) {
        dr_s[tid] = p.draft[(int64_t)b * N + tid];
        par_s[tid] = p.parent[(int64_t)b * N + tid];
    }
    __syncthreads();
    if (wave != 0) return;

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
    // leave this sequence's part of the workspace zero again: its keys (a later
    // call with another shape may place its counters there) and its counter
    unsigned long long *kz = p.keys + (int64_t)b * N * p.n_chunks;
    for (int e = lane; e < N * p.n_chunks; e += 64) kz[e] = 0ull;
    if (lane == 0) __hip_atomic_store(&p.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
