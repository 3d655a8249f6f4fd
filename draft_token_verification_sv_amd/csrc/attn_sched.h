// Work units of the split-KV attention kernels.
//
// A unit is (sequence b, KV head, split s): positions [p0, p1) of the
// sequence's L = ctx + N keys.  Its partial results (O, m, l of every packed
// row) go to slot `part` of the workspace, which the merge kernel reads.
//
// Two schedules:
//   static   one split length for all sequences, chosen on the host from the
//            largest context; unit u = (b * Hkv + kvh) * n_splits + s.  Used
//            for a single sequence, where it is already balanced.
//   dynamic  for a batch, whose context lengths live only on the device.  Every
//            workgroup reads all lengths and derives the same plan: the
//            smallest split length (a multiple of split_q, within
//            [split_min, split_max]) for which the units
//                U(sl) = Hkv * sum_b ceil(L_b / sl)
//            fit the grid (units_max), so the work per unit is about the
//            average and short sequences do not leave most of the grid idle
//            while long ones finish.  Units are numbered sequence by sequence
//            (then KV head, then split), so unit u is also its partial slot.
//            The unit (b, head 0, split 0) of row block 0 records
//            (first unit, splits, split length) of sequence b for the merge.
#pragma once

#include "device_common.h"

namespace sv {

constexpr int kSchedSeqPerThread = 4;           // 256 threads: batch <= 1024
constexpr int kSchedMaxBatch = 256 * kSchedSeqPerThread;

struct AttnUnit {
    int b, kvh, s;
    int ctx, p0, p1;
    int64_t part;                 // partial slot
};

struct SchedLds {
    long long red[2][4];
    int pick[4];                  // b, first unit, splits, L of the chosen sequence
};

// Sum over the 256 threads of a block; `par` alternates the two reduction
// slots so that one barrier per call suffices.
__device__ __forceinline__ long long sched_block_sum(long long v, SchedLds &sm, int &par) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if ((threadIdx.x & 63) == 0) sm.red[par][threadIdx.x >> 6] = v;
    __syncthreads();
    const long long r = sm.red[par][0] + sm.red[par][1] + sm.red[par][2] + sm.red[par][3];
    par ^= 1;
    return r;
}

// Decodes unit u.  Must be called by all 256 threads of the block (the dynamic
// schedule synchronises); returns false, uniformly, when u holds no work.
// `record` marks the row block that writes the per-sequence table.
__device__ __forceinline__ bool attn_unit(const AttnParams &p, int u, bool record, SchedLds &sm,
                                          AttnUnit &w) {
    if (!p.dyn) {
        if (u >= p.B * p.Hkv * p.n_splits) return false;
        w.s = u % p.n_splits;
        const int bh = u / p.n_splits;
        w.kvh = bh % p.Hkv;
        w.b = bh / p.Hkv;
        w.ctx = clamp_ctx(p.ctx_lens[w.b], p.max_ctx);
        const int L = w.ctx + p.N;
        w.p0 = w.s * p.split_len;
        if (w.p0 >= L) return false;
        w.p1 = min(w.p0 + p.split_len, L);
        w.part = u;
        return true;
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t Lr[kSchedSeqPerThread];
    long long tl = 0;
#pragma unroll
    for (int k = 0; k < kSchedSeqPerThread; ++k) {
        const int b = tid * kSchedSeqPerThread + k;
        Lr[k] = b < p.B ? (uint32_t)(clamp_ctx(p.ctx_lens[b], p.max_ctx) + p.N) : 0u;
        tl += Lr[k];
    }
    if (tid == 0) sm.pick[0] = -1;
    int par = 0;
    const long long tot = sched_block_sum(tl, sm, par);

    const long long q = p.split_q, H = p.Hkv, U = p.units_max;
    const long long BH = (long long)p.B * H;
    auto rup = [&](long long x) { return (x + q - 1) / q * q; };
    // any feasible length is >= H * tot / U; with U > B * H the length
    // H * tot / (U - B * H) is feasible (each sequence adds < 1 unit per head
    // to H * L_b / sl); split_max is feasible by the host's choice of U
    long long lo = rup((H * tot + U - 1) / U);
    lo = lo > p.split_min ? lo : (long long)p.split_min;
    long long hi = p.split_max;
    if (U > BH) {
        const long long s0 = rup((H * tot + (U - BH) - 1) / (U - BH));
        hi = s0 < hi ? s0 : hi;
    }
    hi = hi > lo ? hi : lo;
    auto units_at = [&](long long sl) -> long long {
        long long c = 0;
#pragma unroll
        for (int k = 0; k < kSchedSeqPerThread; ++k) c += (Lr[k] + (uint32_t)sl - 1u) / (uint32_t)sl;
        return H * sched_block_sum(c, sm, par);
    };
    if (hi > lo) {
        if (units_at(lo) <= U) {
            hi = lo;
        } else {
#pragma unroll 1
            while (hi - lo > q) {                        // U(lo) > U_max >= U(hi)
                const long long mid = lo + (hi - lo) / q / 2 * q;
                if (units_at(mid) <= U) hi = mid;
                else lo = mid;
            }
        }
    }
    const int sl = (int)hi;

    // exclusive scan of the per-thread split counts -> first unit of each sequence
    int ns[kSchedSeqPerThread];
    int c = 0;
#pragma unroll
    for (int k = 0; k < kSchedSeqPerThread; ++k) {
        ns[k] = (int)((Lr[k] + (uint32_t)sl - 1u) / (uint32_t)sl);
        c += ns[k];
    }
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
    }
    if (lane == 63) sm.red[par][wave] = incl;
    __syncthreads();
    long long first = incl - c;
    for (int wv = 0; wv < wave; ++wv) first += sm.red[par][wv];
    first *= H;
#pragma unroll
    for (int k = 0; k < kSchedSeqPerThread; ++k) {
        const long long span = H * ns[k];
        if (u >= first && u < first + span) {
            sm.pick[0] = tid * kSchedSeqPerThread + k;
            sm.pick[1] = (int)first;
            sm.pick[2] = ns[k];
            sm.pick[3] = (int)Lr[k];
        }
        first += span;
    }
    __syncthreads();
    if (sm.pick[0] < 0) return false;
    w.b = sm.pick[0];
    const int rel = u - sm.pick[1];
    w.kvh = rel / sm.pick[2];
    w.s = rel % sm.pick[2];
    const int L = sm.pick[3];
    w.ctx = L - p.N;
    w.p0 = w.s * sl;
    w.p1 = min(w.p0 + sl, L);
    w.part = u;
    if (record && rel == 0 && tid == 0) p.seq_tab[w.b] = make_int4(sm.pick[1], sm.pick[2], sl, 0);
    return true;
}

}  // namespace sv
