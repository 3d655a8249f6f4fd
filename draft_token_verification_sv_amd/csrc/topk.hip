// Top-k stochastic verification: every verify row samples among its k largest
// logits (Gumbel-max with the caller's noise, as for plain temperature
// sampling), then the acceptance walk runs on the samples [single-RTX-3090
// DFlash note, "Next steps": temperature and top-k sampling for the verify
// path].  The kept set is every token whose logit is at least the row's k-th
// largest (ties at the k-th value kept).
//
// One workgroup of 1024 threads per row, k <= 1024.  Logits are compared
// through their order-preserving 32-bit keys (-0 folded onto +0):
//   1. each thread's maximum over its slice of the row (16-byte loads, fp32
//      compares: two vector operations per logit);
//   2. the k-th largest of the 1024 maxima to 16 bits (two 8-bit radix
//      rounds in LDS): at least k logits reach it, so it bounds the k-th
//      largest logit from below;
//   3. a second pass appends every logit at or above the bound to an LDS
//      candidate list (one atomic per wavefront); the top-k set is inside it;
//   4. the exact k-th largest key of the candidates (four radix rounds), then
//      the Gumbel-max over the candidates at or above it (their noise
//      gathered);
//   If the list overflows (many logits tie at the bound) the k-th key and the
//   sample come from passes over the whole row instead.
// The sample's key goes to the sequence's slot, and the last row of each
// sequence to finish runs the acceptance walk.
#include "accept_walk.h"

namespace sv {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkCap = 4096;          // LDS candidates (key, index)

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;                      // -0 ties with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// the value of an order key; keys below that of -inf (a bound truncated from
// the maximum of a thread that saw no logit) read as -inf
__device__ __forceinline__ float key_value(uint32_t k) {
    if (k <= 0x007FFFFFu) return -INFINITY;
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The k-th largest (1-based) of the keys every thread passes to `visit`'s
// callback, to the top 8 * rounds bits (rounds = 4: exact).  All threads of
// the workgroup call it; `visit` must offer the same keys on every call.
template <class Visit>
__device__ uint32_t kth_largest(Visit visit, int k, int rounds, uint32_t *hist, int *sh) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0u, mask = 0u;
    int kk = k;
#pragma unroll 1
    for (int r = 0; r < rounds; ++r) {
        const int shift = 24 - 8 * r;
        if (tid < 256) hist[tid] = 0u;
        __syncthreads();
        visit([&](uint32_t key) {
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        if (tid < 64) {
            // lane l holds bins 255-4l .. 252-4l, highest first
            uint32_t c[4], sum = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = hist[255 - 4 * tid - j];
                sum += c[j];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t o = (uint32_t)__shfl_up((int)incl, d, 64);
                if (tid >= d) incl += o;
            }
            const uint32_t excl = incl - sum;
            if (excl < (uint32_t)kk && (uint32_t)kk <= incl) {
                uint32_t run = excl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (run < (uint32_t)kk && (uint32_t)kk <= run + c[j]) {
                        sh[0] = 255 - 4 * tid - j;
                        sh[1] = kk - (int)run;
                    }
                    run += c[j];
                }
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sh[0] << shift;
        mask |= 255u << shift;
        kk = sh[1];
        __syncthreads();
    }
    return prefix;
}

template <bool F32>
__global__ __launch_bounds__(kTopkThreads) void topk_sample_accept_kernel(AcceptParams p) {
    __shared__ uint32_t hist[256];
    __shared__ int sh[4];
    __shared__ uint32_t ckey[kTopkCap];
    __shared__ int cidx[kTopkCap];
    __shared__ unsigned long long red[kTopkThreads / 64];
    __shared__ int last_s;
    __shared__ int am_s[64], dr_s[64], par_s[64];

    const int row = blockIdx.x;                          // b * N + i
    const int b = row / p.N;
    const int tid = threadIdx.x;
    const int V = p.V;
    constexpr int EPL = F32 ? 4 : 8;                     // values per 16-byte load
    const uint8_t *base = (const uint8_t *)p.logits + (int64_t)row * V * (F32 ? 4 : 2);
    const float *grow = p.gumbel + (int64_t)row * V;
    const bool vec_ok = ((uintptr_t)p.logits % 16 == 0) && (((int64_t)V * (F32 ? 4 : 2)) % 16 == 0);
    const int nfull = vec_ok ? V / EPL : 0;              // whole 16-byte groups (else value by value)

    // every logit of this thread's slice: f(value, index)
    auto each_logit = [&](auto f) {
        // batches of 4 loads per thread, the next batch in flight while one is used
        auto load4 = [&](int gi, u32x4 (&v)[4]) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int g = min(gi + u * kTopkThreads, nfull - 1);
                v[u] = *(const u32x4 *)(base + (int64_t)g * 16);
            }
        };
        auto use4 = [&](int gi, const u32x4 (&v)[4]) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int g = gi + u * kTopkThreads;
                if (g < nfull) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if constexpr (F32) {
                            f(__uint_as_float(v[u][t]), g * 4 + t);
                        } else {
                            f(bf16_bits_to_f32(v[u][t] & 0xFFFFu), g * 8 + 2 * t);
                            f(bf16_bits_to_f32(v[u][t] >> 16), g * 8 + 2 * t + 1);
                        }
                    }
                }
            }
        };
        if (tid < nfull) {
            u32x4 va[4], vb[4];
            load4(tid, va);
            for (int gi = tid; gi < nfull; gi += 8 * kTopkThreads) {
                const int g2 = gi + 4 * kTopkThreads;
                if (g2 < nfull) load4(g2, vb);
                use4(gi, va);
                if (g2 >= nfull) break;
                if (g2 + 4 * kTopkThreads < nfull) load4(g2 + 4 * kTopkThreads, va);
                use4(g2, vb);
            }
        }
        for (int e = nfull * EPL + tid; e < V; e += kTopkThreads) {      // tail (V not a multiple of EPL)
            const float l = F32 ? ((const float *)base)[e] : bf16_bits_to_f32(((const uint16_t *)base)[e]);
            f(l, e);
        }
    };

    // 1. per-thread maxima; 2. a lower bound of the k-th largest logit
    float fmax_t = -INFINITY;
    each_logit([&](float l, int) { fmax_t = fmaxf(fmax_t, l); });
    const uint32_t tmax = order_key(fmax_t);
    const int k = p.top_k;
    const uint32_t bound = kth_largest([&](auto f) { f(tmax); }, k, 2, hist, sh);
    const float bound_f = key_value(bound);               // l >= bound_f  <=>  key(l) >= bound

    // 3. candidates: every logit at or above the bound
    if (tid == 0) sh[2] = 0;
    __syncthreads();
    each_logit([&](float l, int e) {
        const bool take = l >= bound_f;
        const uint64_t m = __ballot(take);
        if (m == 0ull) return;
        const int lane = tid & 63;
        int slot0 = 0;
        if (lane == (int)__builtin_ctzll(m)) slot0 = atomicAdd(&sh[2], __popcll(m));
        slot0 = __shfl(slot0, (int)__builtin_ctzll(m), 64);
        if (take) {
            const int s = slot0 + __popcll(m & ((1ull << lane) - 1ull));
            if (s < kTopkCap) {
                ckey[s] = order_key(l);
                cidx[s] = e;
            }
        }
    });
    __syncthreads();
    const int ncand = sh[2];
    const float T = p.temperature;                        // key = l / T + g
    unsigned long long best = 0ull;
    if (ncand <= kTopkCap) {
        // 4. the exact k-th largest among the candidates, then the sample
        const uint32_t kth = kth_largest(
            [&](auto f) {
                for (int s = tid; s < ncand; s += kTopkThreads) f(ckey[s]);
            },
            k, F32 ? 4 : 2, hist, sh);                  // bf16 logits: the keys' low 16 bits are zero
        for (int s = tid; s < ncand; s += kTopkThreads) {
            if (ckey[s] >= kth) {
                const int e = cidx[s];
                best = umax64(best, make_key(key_value(ckey[s]) / T + grow[e], (uint32_t)e));
            }
        }
    } else {
        // many logits tie at the bound: the k-th key and the sample from whole-row passes
        const uint32_t kth = kth_largest([&](auto f) { each_logit([&](float l, int) { f(order_key(l)); }); }, k, 4,
                                         hist, sh);
        each_logit([&](float l, int e) {
            if (order_key(l) >= kth) best = umax64(best, make_key(l / T + grow[e], (uint32_t)e));
        });
    }
    best = wave_max64(best);
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
        unsigned long long kb = 0ull;
#pragma unroll
        for (int w = 0; w < kTopkThreads / 64; ++w) kb = umax64(kb, red[w]);
        const unsigned long long was =
            __hip_atomic_fetch_max(&p.keys[row], kb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" : : "v"((uint32_t)was));
        wait_vm0();
        const unsigned int done =
            __hip_atomic_fetch_add(&p.seqs_done[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_s = done == (unsigned int)(p.N - 1);
    }
    __syncthreads();
    if (!last_s || tid >= 64) return;
    if (tid == 0) __hip_atomic_store(&p.seqs_done[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    walk_sequence<false>(p, b, tid, am_s, dr_s, par_s, nullptr);
    if (p.argmax != nullptr && tid < p.N) p.argmax[(int64_t)b * p.N + tid] = am_s[tid];
}

}  // namespace

hipError_t launch_topk_accept(const AcceptParams &p, hipStream_t st) {
    const dim3 grid((unsigned)(p.B * p.N));
    if (p.logits_f32) hipLaunchKernelGGL((topk_sample_accept_kernel<true>), grid, dim3(kTopkThreads), 0, st, p);
    else hipLaunchKernelGGL((topk_sample_accept_kernel<false>), grid, dim3(kTopkThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace sv
