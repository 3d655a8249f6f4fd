// Acceptance helpers shared by the argmax / sampling kernels: order-preserving
// 64-bit (value, index) keys, their wavefront maximum, and the acceptance walk
// of one sequence [single-RTX-3090 DFlash note, "From autoregressive to
// DDTree": the longest accepted root path plus the bonus token].
#pragma once

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

// The walk of sequence b by one wavefront (lane = node), once every row's
// key of the sequence is in p.keys: takes the keys (leaving zeros), decides
// which nodes are accepted, writes accept_len, path and tokens.  am_s / dr_s /
// par_s (and path_s when PATH_LDS) are LDS arrays of 64 entries; returns the
// accept length a.
template <bool PATH_LDS>
__device__ int walk_sequence(const AcceptParams &p, int b, int lane, int *am_s, int *dr_s, int *par_s,
                             int *path_s) {
    const int N = p.N;
    if (lane < N) {
        const unsigned long long k =
            __hip_atomic_exchange(&p.keys[(int64_t)b * N + lane], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        am_s[lane] = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
        dr_s[lane] = p.draft[(int64_t)b * N + lane];
        par_s[lane] = parent_of(p.parent + (int64_t)b * N, lane, p.err);
    }
    __builtin_amdgcn_s_waitcnt(0);           // the LDS writes of all lanes (one wave: no barrier)
    __builtin_amdgcn_wave_barrier();

    // node `lane`: accepted iff every edge of its root path is accepted (the
    // edge parent -> i: a valid parent, parent[i] < i, whose argmax is the
    // draft of i).  The root paths are combined by pointer doubling instead of
    // walked one step at a time: after round k each node knows the AND of its
    // edges' acceptance, its depth and its ancestor set over its first 2^k
    // ancestors; six rounds cover the 63 edges of the deepest tree.  An
    // invalid edge ends its node's path at the root and rejects the node.
    const bool node = lane < N;
    const int pj = node ? par_s[lane] : 0;
    const bool valid = node && lane > 0 && pj >= 0 && pj < lane;
    const int am_parent = __shfl(node ? am_s[lane] : 0, valid ? pj : 0, 64);
    int up = valid ? pj : 0;
    int acc = !node ? 0 : (lane == 0 ? 1 : (valid && dr_s[lane] == am_parent ? 1 : 0));
    int depth = valid ? 1 : 0;
    unsigned long long anc = node ? (1ull << lane) : 0ull;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        const int acc_u = __shfl(acc, up, 64);
        const int dep_u = __shfl(depth, up, 64);
        const unsigned long long anc_u = __shfl(anc, up, 64);
        const int up_u = __shfl(up, up, 64);
        acc &= acc_u;
        depth += dep_u;
        anc |= anc_u;
        up = up_u;
    }
    // deepest accepted node, ties to the smallest index (node 0 always qualifies)
    unsigned int key = acc ? (((unsigned)depth << 8) | (unsigned)(255 - lane)) : 0u;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) key = max(key, (unsigned)__shfl_xor((int)key, m, 64));
    const int best_node = 255 - (int)(key & 255u);
    const int a = (int)(key >> 8);

    // the path: the ancestors of the best node (itself included), each at its
    // depth; the tokens: their drafts, then the best node's argmax
    const unsigned long long on_path = __shfl(anc, best_node, 64);
    int32_t *path = p.path + (int64_t)b * N;
    int32_t *tok = p.tokens + (int64_t)b * N;
    if (node && ((on_path >> lane) & 1ull)) {
        path[depth] = lane;
        if constexpr (PATH_LDS) path_s[depth] = lane;
        if (depth > 0) tok[depth - 1] = dr_s[lane];
    }
    if (lane == 0) {
        tok[a] = am_s[best_node];
        p.accept_len[b] = a;
    }
    if (lane < N && lane > a) {
        path[lane] = -1;
        tok[lane] = -1;
    }
    return a;
}

}  // namespace
}  // namespace sv
