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
//
// Fused form (acceptance + compaction): the last workgroup of sequence b then
// moves the accepted rows' KV itself with all of its threads, so the sequence
// needs no second launch (the standalone compaction kernel is compact.hip).
#include "accept_walk.h"

namespace sv {
namespace {

constexpr int kCompactLds = 32768;      // staging bytes of the fused compaction

// In-place compaction of sequence b by one workgroup of 256 threads: for
// every layer, KV head and K|V, row ctx + j <- row ctx + path[j] for the
// accepted nodes j in [1, a] with path[j] > j (the others stay).  Copies go in
// rounds that fill the staging buffer, each round reading all of its rows
// before writing any; rounds take the moving rows in increasing j, and since
// path[j] >= j a round's sources are never an earlier round's destinations.
// path_s / mov_s live in LDS; mov_s[0 .. n_mov) lists the moving j in order.
__device__ void compact_sequence(const CompactParams &cp, int b, int ctx, const int *path_s, const int *mov_s,
                                 int n_mov, uint8_t *stage) {
    if (n_mov == 0) return;
    const int tid = threadIdx.x;
    const int D = cp.D;
    const bool q4 = cp.dtype == SV_Q4;
    const int row_bytes = cp.dtype == SV_F32 ? D * 4 : (cp.dtype == SV_BF16 ? D * 2 : D / 2);
    const int srow_bytes = q4 ? (D / 32) * 2 : 0;
    const int vpieces = row_bytes / 16;                  // 16-byte pieces of a value row
    const int pieces = vpieces + srow_bytes / 4;         // + 4-byte pieces of its scale row
    const int unit_bytes = row_bytes + 16;               // staging room per (row, layer, head, K|V)
    const int per_row = cp.n_layers * cp.Hkv * 2;
    const int total = n_mov * per_row;
    const int cap = kCompactLds / unit_bytes;
    for (int u0 = 0; u0 < total; u0 += cap) {
        const int nu = min(cap, total - u0);
        for (int pass = 0; pass < 2; ++pass) {           // 0: sources -> LDS, 1: LDS -> destinations
            for (int e = tid; e < nu * pieces; e += 256) {
                const int ul = e / pieces, pc = e - ul * pieces;
                const int u = u0 + ul;
                const int m = u / per_row;
                int r = u - m * per_row;
                const int which = r & 1;
                r >>= 1;
                const int h = r % cp.Hkv, layer = r / cp.Hkv;
                const int j = mov_s[m];
                const int64_t ri = kv_row_index(cp.kv, b, cp.Hkv, h, ctx + (pass == 0 ? path_s[j] : j), cp.err);
                // a source whose page is outside the pool reads as a zero row; such
                // a destination is not written
                if (ri < 0 && pass == 1) continue;
                uint8_t *lds = stage + ul * unit_bytes;
                if (pc < vpieces) {
                    uint8_t *g = (uint8_t *)(which ? cp.kv.v : cp.kv.k) + (int64_t)layer * cp.layer_stride +
                                 ri * row_bytes + pc * 16;
                    const u32x4 zero = {0u, 0u, 0u, 0u};
                    if (pass == 0) *(u32x4 *)(lds + pc * 16) = ri < 0 ? zero : *(const u32x4 *)g;
                    else *(u32x4 *)g = *(const u32x4 *)(lds + pc * 16);
                } else {
                    const int w = pc - vpieces;
                    uint8_t *g = (uint8_t *)(which ? cp.kv.vs : cp.kv.ks) + (int64_t)layer * cp.scale_layer_stride +
                                 ri * srow_bytes + w * 4;
                    if (pass == 0) *(uint32_t *)(lds + row_bytes + w * 4) = ri < 0 ? 0u : *(const uint32_t *)g;
                    else *(uint32_t *)g = *(const uint32_t *)(lds + row_bytes + w * 4);
                }
            }
            __syncthreads();
        }
    }
}

// SAMPLE: stochastic verification at temperature T -- the row's key for
// token v is the fp32 sum l_v / T + g_v (Gumbel-max sampling with the given
// noise g; the division and the addition each round to nearest), its maximum
// (lowest index on ties) is the row's sample and replaces the argmax in the
// walk [single-RTX-3090 note, "Next steps": temperature sampling in verify].
template <bool F32, bool VEC, bool COMPACT, bool SAMPLE>
__global__ __launch_bounds__(256) void argmax_accept_kernel(AcceptParams p) {
    __shared__ unsigned long long red[4];
    __shared__ int last_s;
    __shared__ int am_s[64], dr_s[64], par_s[64];
    __shared__ int path_s[COMPACT ? 64 : 1], mov_s[COMPACT ? 64 : 1];
    __shared__ int cinfo_s[2];                             // ctx, moving rows
    __shared__ __attribute__((aligned(16))) uint8_t stage_s[COMPACT ? kCompactLds : 16];

    const int c = blockIdx.x % p.n_chunks;
    const int row = blockIdx.x / p.n_chunks;             // b * N + i
    const int b = row / p.N;
    const int tid = threadIdx.x;
    const int64_t V = p.V;
    const int64_t lo = (int64_t)c * p.chunk;
    const int64_t hi = min<int64_t>(V, lo + p.chunk);
    constexpr int EPL = F32 ? 4 : 8;                      // elements per 16-byte load
    constexpr int UNR = 8;                                // loads in flight per thread

    const float *grow = SAMPLE ? p.gumbel + (int64_t)row * V : nullptr;
    // the key value of token index e with logit l (g: its noise when sampling)
    auto keyv = [&](float l, float g) -> float {
        if constexpr (SAMPLE) return l / p.temperature + g;
        else return l;
    };
    unsigned long long best = 0ull;
    if constexpr (VEC) {
        // full groups of UNR loads, then the rest one load at a time
        const void *base = F32 ? (const void *)((const float *)p.logits + (int64_t)row * V)
                               : (const void *)((const uint16_t *)p.logits + (int64_t)row * V);
        // EPL consecutive values at e (their noise in gn when sampling)
        auto consume = [&](const u32x4 &v, const f32x4 (&gn)[2], int64_t e) {
            const uint32_t i0 = (uint32_t)e;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if constexpr (F32) {
                    best = umax64(best, make_key(keyv(__uint_as_float(v[t]), gn[0][t]), i0 + t));
                } else {
                    best = umax64(best, make_key(keyv(bf16_bits_to_f32(v[t] & 0xFFFFu), gn[(2 * t) / 4][(2 * t) % 4]),
                                                 i0 + 2 * t));
                    best = umax64(best, make_key(keyv(bf16_bits_to_f32(v[t] >> 16), gn[(2 * t + 1) / 4][(2 * t + 1) % 4]),
                                                 i0 + 2 * t + 1));
                }
            }
        };
        auto gload = [&](int64_t e, f32x4 (&gn)[2]) {
            if constexpr (SAMPLE) {
                gn[0] = *(const f32x4 *)(grow + e);
                if constexpr (!F32) gn[1] = *(const f32x4 *)(grow + e + 4);
            }
        };
        int64_t e = lo + (int64_t)tid * EPL;
        if constexpr (!F32 && !SAMPLE) {
            // bf16 greedy rows: each value becomes a 16-bit code with the
            // order of its 64-bit key (negatives 0x8000 - |x|, -0 and +0 both
            // 0x8000, positives 0x8000 + |x|), two per dword with packed 16-bit
            // ops; a code and 127 - slot (slot = 8 k + t over the group's 16
            // loads, in index order within the thread) make a 32-bit key whose
            // maximum is the group's largest value at its lowest index, which
            // then enters the 64-bit key: 3 to 4 vector ops per value instead of
            // ~10.  All 16 loads of a group go out together (the default chunk,
            // 32768 values, is one group); loads past the chunk's end reread its
            // last 8 values and are left out of the maximum (the vector path
            // has chunks and rows of whole 16-byte loads).
            typedef short s16x2 __attribute__((ext_vector_type(2)));
            typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
            constexpr int GL = 16;
            for (; e < hi; e += (int64_t)GL * 256 * EPL) {
                u32x4 v[GL];
#pragma unroll
                for (int k = 0; k < GL; ++k)
                    v[k] = *(const u32x4 *)((const uint8_t *)base + min(e + (int64_t)k * 256 * EPL, hi - EPL) * 2);
                uint32_t kb = 0u;
#pragma unroll
                for (int k = 0; k < GL; ++k) {
                    uint32_t kk = 0u;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint32_t w = v[k][t];
                        const uint32_t sg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, w) >> (short)15);
                        const uint32_t o = __builtin_bit_cast(
                            uint32_t, __builtin_bit_cast(u16x2, w ^ (sg | 0x80008000u)) - __builtin_bit_cast(u16x2, sg));
                        const uint32_t k0 = (o << 16) | (uint32_t)(8 * GL - 1 - (8 * k + 2 * t));
                        const uint32_t k1 = (o & 0xFFFF0000u) | (uint32_t)(8 * GL - 1 - (8 * k + 2 * t + 1));
                        kk = max(kk, max(k0, k1));
                    }
                    kb = e + (int64_t)k * 256 * EPL < hi ? max(kb, kk) : kb;
                }
                const uint32_t slot = (uint32_t)(8 * GL - 1) - (kb & 0xFFFFu);
                const uint32_t code = kb >> 16;
                const uint32_t bits = code >= 0x8000u ? code - 0x8000u : (0x8000u | (0x8000u - code));
                const uint32_t idx = (uint32_t)e + (slot >> 3) * (256u * EPL) + (slot & 7u);
                best = umax64(best, make_key(bf16_bits_to_f32(bits), idx));
            }
        }
        for (; e + (int64_t)(UNR - 1) * 256 * EPL < hi; e += (int64_t)UNR * 256 * EPL) {
            u32x4 v[UNR];
            f32x4 gv[UNR][2];
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                v[k] = *(const u32x4 *)((const uint8_t *)base + (e + (int64_t)k * 256 * EPL) * (F32 ? 4 : 2));
                gload(e + (int64_t)k * 256 * EPL, gv[k]);
            }
#pragma unroll
            for (int k = 0; k < UNR; ++k) consume(v[k], gv[k], e + (int64_t)k * 256 * EPL);
        }
        for (; e < hi; e += 256 * EPL) {
            const u32x4 v = *(const u32x4 *)((const uint8_t *)base + e * (F32 ? 4 : 2));
            f32x4 gv[2];
            gload(e, gv);
            consume(v, gv, e);
        }
    } else if constexpr (F32) {
        const float *rowp = (const float *)p.logits + (int64_t)row * V;
        for (int64_t e = lo + tid; e < hi; e += 256)
            best = umax64(best, make_key(keyv(rowp[e], SAMPLE ? grow[e] : 0.f), (uint32_t)e));
    } else {
        const uint16_t *rowp = (const uint16_t *)p.logits + (int64_t)row * V;
        for (int64_t e = lo + tid; e < hi; e += 256)
            best = umax64(best, make_key(keyv(bf16_bits_to_f32(rowp[e]), SAMPLE ? grow[e] : 0.f), (uint32_t)e));
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
    if constexpr (!COMPACT) {
        if (wave != 0) return;
    } else if (wave != 0) {
        __syncthreads();                                   // the walk's path in LDS
        compact_sequence(p.cp, b, cinfo_s[0], path_s, mov_s, cinfo_s[1], stage_s);
        return;
    }
    if (lane == 0) __hip_atomic_store(&p.seqs_done[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (COMPACT) {
        if (lane == 0) cinfo_s[0] = ctx_of(p.cp.ctx_lens, b, p.cp.max_ctx, p.err);
    }
    const int a = walk_sequence<COMPACT>(p, b, lane, am_s, dr_s, par_s, path_s);
    if (p.argmax != nullptr && lane < N) p.argmax[(int64_t)b * N + lane] = am_s[lane];
    if constexpr (COMPACT) {
        // the moving rows j in [1, a] (path[j] > j), in increasing order
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        const bool mv = lane >= 1 && lane <= a && path_s[lane] > lane;
        const uint64_t bal = __ballot(mv);
        if (mv) mov_s[__popcll(bal & ((1ull << lane) - 1ull))] = lane;
        if (lane == 0) {
            cinfo_s[1] = __popcll(bal);
            if (p.cp.new_lens != nullptr) p.cp.new_lens[b] = cinfo_s[0] + a + 1;
        }
        __syncthreads();
        compact_sequence(p.cp, b, cinfo_s[0], path_s, mov_s, cinfo_s[1], stage_s);
    }
}

template <bool COMPACT, bool SAMPLE>
void launch_accept_t(const AcceptParams &p, bool vec, int grid, hipStream_t st) {
    if (p.logits_f32) {
        if (vec) hipLaunchKernelGGL((argmax_accept_kernel<true, true, COMPACT, SAMPLE>), dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL((argmax_accept_kernel<true, false, COMPACT, SAMPLE>), dim3(grid), dim3(256), 0, st, p);
    } else {
        if (vec) hipLaunchKernelGGL((argmax_accept_kernel<false, true, COMPACT, SAMPLE>), dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL((argmax_accept_kernel<false, false, COMPACT, SAMPLE>), dim3(grid), dim3(256), 0, st, p);
    }
}

}  // namespace

hipError_t launch_accept(const AcceptParams &p, hipStream_t st) {
    const int grid = p.B * p.N * p.n_chunks;
    const int esize = p.logits_f32 ? 4 : 2;
    bool vec = ((uintptr_t)p.logits % 16 == 0) && (((int64_t)p.V * esize) % 16 == 0) &&
               ((int64_t)p.chunk * esize) % 16 == 0;
    if (p.gumbel != nullptr) vec = vec && ((uintptr_t)p.gumbel % 16 == 0) && (p.V % 4 == 0);
    if (p.compact) launch_accept_t<true, false>(p, vec, grid, st);
    else if (p.gumbel != nullptr) launch_accept_t<false, true>(p, vec, grid, st);
    else launch_accept_t<false, false>(p, vec, grid, st);
    return hipGetLastError();
}

}  // namespace sv
