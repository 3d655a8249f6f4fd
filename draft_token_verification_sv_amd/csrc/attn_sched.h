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
//            fit the grid (units_max); sequence b then takes
//            ns_b = ceil(L_b / sl) splits of about L_b / ns_b positions each
//            (rounded up to the quantum), so the work per unit is about the
//            average and short sequences do not leave most of the grid idle
//            while long ones finish.  Each sequence owns a contiguous range of
//            unit numbers (KV head major, then split); unit u is also its
//            partial slot.  The unit (b, head 0, split 0) of row block 0
//            records (first unit, splits, split length) of sequence b for the
//            merge.  Reductions and scans over the batch use DPP lane moves
//            within a wavefront and one LDS exchange between the 4 wavefronts.
#pragma once

#include "device_common.h"

namespace sv {

constexpr int kSchedRounds = 4;                 // sequences b = 256 * round + thread
constexpr int kSchedMaxBatch = 256 * kSchedRounds;

struct AttnUnit {
    int b, kvh, s;
    int ctx, p0, p1;
    int64_t part;                 // partial slot
};

struct SchedLds {
    double tot[4];
    uint32_t red[2][4];
    int pick[6];                  // b, first unit, splits, L, split length, ctx + N of the chosen sequence
};

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP moves (row
// shifts by 1, 2, 4, 8 within rows of 16 lanes, then the row broadcasts of
// lanes 15 and 31), no LDS traffic.
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

#define SV_DPP_ADD_F64(x, ctrl, rmask)                                                            \
    do {                                                                                       \
        const uint64_t u_ = __builtin_bit_cast(uint64_t, x);                                   \
        const uint32_t lo_ = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u_, ctrl, rmask, 0xf, false); \
        const uint32_t hi_ =                                                                   \
            (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u_ >> 32), ctrl, rmask, 0xf, false); \
        x += __builtin_bit_cast(double, ((uint64_t)hi_ << 32) | lo_);                          \
    } while (0)

// Wavefront sum of doubles holding integers (exact below 2^53), in every lane.
__device__ __forceinline__ double wave_sum_f64(double x) {
    SV_DPP_ADD_F64(x, 0x111, 0xf);
    SV_DPP_ADD_F64(x, 0x112, 0xf);
    SV_DPP_ADD_F64(x, 0x114, 0xf);
    SV_DPP_ADD_F64(x, 0x118, 0xf);
    SV_DPP_ADD_F64(x, 0x142, 0xa);
    SV_DPP_ADD_F64(x, 0x143, 0xc);
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Block (256 threads) sum of 32-bit counts; `par` alternates the two LDS slots
// so that one barrier per call suffices.
__device__ __forceinline__ uint32_t sched_block_sum(uint32_t v, SchedLds &sm, int &par) {
    v = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_u32(v), 63);
    if ((threadIdx.x & 63) == 0 && threadIdx.x < 256) sm.red[par][threadIdx.x >> 6] = v;
    __syncthreads();
    const uint32_t r = sm.red[par][0] + sm.red[par][1] + sm.red[par][2] + sm.red[par][3];
    par ^= 1;
    return r;
}

// Bounds of the split-length search.  Split lengths are multiples of the
// power of two q.  Any feasible length is >= H * tot / U; with U > B * H the
// length H * tot / (U - B * H) is feasible (each sequence adds < 1 unit per
// head to H * L_b / sl); split_max is feasible by the host's choice of U.  The
// quotients are worked out in double (exact for the integers involved, rounded
// up and padded) so that no 64-bit integer division is needed.
__device__ __forceinline__ void split_bounds(const AttnParams &p, double tot, int &lo, int &hi) {
    const int qm = p.split_q - 1;
    const double U = (double)p.units_max, BH = (double)p.B * p.Hkv, HT = (double)p.Hkv * tot;
    auto rup = [&](double x) -> int {
        const double c = ceil(x);
        return c >= (double)p.split_max ? p.split_max : (((int)c + qm) & ~qm);
    };
    lo = rup(HT / U);
    lo = lo > p.split_min ? lo : p.split_min;
    hi = p.split_max;
    if (U > BH) {
        const int s0 = rup(HT / (U - BH) + 1.0);
        hi = s0 < hi ? s0 : hi;
    }
    lo = lo < p.split_max ? lo : p.split_max;
    hi = hi > lo ? hi : lo;
}

// Smallest length in [lo, hi] whose unit count fits (hi fits); the caller's
// units_at(sl) must return the same value in every thread that calls it.
template <class F>
__device__ __forceinline__ uint32_t split_search(int lo, int hi, int qm, long long umax, F units_at) {
    if (hi > lo) {
        if (units_at((uint32_t)lo) <= umax) {
            hi = lo;
        } else {
#pragma unroll 1
            while (hi - lo > qm + 1) {                   // U(lo) > U_max >= U(hi)
                const int mid = lo + (((hi - lo) >> 1) & ~qm);
                if (units_at((uint32_t)mid) <= umax) hi = mid;
                else lo = mid;
            }
        }
    }
    return (uint32_t)hi;
}

// Records sequence b (length L, ns splits from unit `first`) as the owner of
// unit u when u falls in its range.
__device__ __forceinline__ void sched_pick(SchedLds &sm, int u, int b, uint32_t L, uint32_t full, uint32_t ns,
                                           long long first, int H, int qm) {
    if (ns > 0 && u >= first && u < first + (long long)H * ns) {
        sm.pick[0] = b;
        sm.pick[1] = (int)first;
        sm.pick[2] = (int)ns;
        sm.pick[3] = (int)L;
        sm.pick[5] = (int)full;
        // the sequence's own length: its ns splits made as even as the
        // quantum allows (<= sl, so the unit count is unchanged)
        const uint32_t even = (L + ns - 1u) / ns;
        sm.pick[4] = (int)((even + (uint32_t)qm) & ~(uint32_t)qm);
    }
}

// Length of the key range that sequence b's units cover: ctx + N, or its last
// `window` rows.
__device__ __forceinline__ uint32_t key_range(const AttnParams &p, int ctx) {
    const int L = ctx + p.N;
    return (uint32_t)(p.window > 0 && L > p.window ? p.window : L);
}

// Decodes unit u.  Must be called by all threads of the block (the dynamic
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
        w.ctx = ctx_of(p.ctx_lens, w.b, p.max_ctx, p.err);
        const int L = w.ctx + p.N;
        const int lo = L - (int)key_range(p, w.ctx);    // first key row (0 without a window)
        w.p0 = lo + w.s * p.split_len;
        if (w.p0 >= L) return false;
        // the last split also takes the keys past n_splits * split_len (a plan
        // may leave a short remainder on it instead of a unit of its own)
        w.p1 = w.s == p.n_splits - 1 ? L : min(w.p0 + p.split_len, L);
        w.part = u;
        return true;
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qm = p.split_q - 1;
    const int H = p.Hkv;
    const long long umax = p.units_max;
    if (p.B <= 64) {
        // one sequence per lane of wavefront 0: every reduction is a DPP scan,
        // no barrier until the result is published
        if (wave == 0) {
            const int cb = lane < p.B ? ctx_of(p.ctx_lens, lane, p.max_ctx, p.err) : 0;
            const uint32_t Lb = lane < p.B ? key_range(p, cb) : 0u;
            const double tot = wave_sum_f64((double)Lb);
            int lo, hi;
            split_bounds(p, tot, lo, hi);
            const uint32_t sl = split_search(lo, hi, qm, umax, [&](uint32_t x) -> long long {
                const uint32_t c = wave_scan_u32((Lb + x - 1u) / x);
                return (long long)H * (uint32_t)__builtin_amdgcn_readlane((int)c, 63);
            });
            uint32_t ns = (Lb + sl - 1u) / sl;
            // Fill the grid: while unit slots remain, give the sequence whose
            // units are the longest one more split (its units shrink toward
            // the average), so that the last workgroups to finish do not carry
            // units up to twice the average.  A split is taken only if it
            // shortens the units (after rounding to the quantum) and leaves no
            // unit empty; ties go to the lowest sequence.
            {
                const uint32_t budget = (uint32_t)(umax / H);
                uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_u32(ns), 63);
#pragma unroll 1
                for (int it = 0; it < 64 && total < budget; ++it) {
                    const uint32_t cur = ns ? (((Lb + ns - 1u) / ns + (uint32_t)qm) & ~(uint32_t)qm) : 0u;
                    const uint32_t n1 = ns + 1u;
                    const uint32_t nxt = ((Lb + n1 - 1u) / n1 + (uint32_t)qm) & ~(uint32_t)qm;
                    const bool can = ns > 0u && n1 <= (uint32_t)kMaxSplits && nxt < cur &&
                                     (uint64_t)ns * nxt < (uint64_t)Lb;
                    unsigned long long key = can ? (((unsigned long long)cur << 8) | (unsigned)(63 - lane)) : 0ull;
#pragma unroll
                    for (int m = 1; m < 64; m <<= 1) {
                        const unsigned long long o = __shfl_xor(key, m, 64);
                        key = o > key ? o : key;
                    }
                    if (key == 0ull) break;
                    if ((unsigned)(63 - lane) == (unsigned)(key & 255ull)) ns = n1;
                    ++total;
                }
            }
            const uint32_t before = wave_scan_u32(ns) - ns;
            if (lane == 0) sm.pick[0] = -1;           // same wavefront: ordered before the pick
            sched_pick(sm, u, lane, Lb, (uint32_t)(cb + p.N), ns, (long long)H * before, H, qm);
        }
        __syncthreads();
    } else {
        // the first 256 threads hold the sequences; threads beyond them (a
        // workgroup of 512) take part in the barriers with no sequence
        const bool act = tid < 256;
        const int rounds = (p.B + 255) >> 8;         // uniform, <= kSchedRounds
        uint32_t Lr[kSchedRounds], Fr[kSchedRounds];
        double tl = 0.0;
#pragma unroll
        for (int k = 0; k < kSchedRounds; ++k) {
            const int b = 256 * k + tid;
            const bool has = act && b < p.B;
            const int cb = has ? ctx_of(p.ctx_lens, b, p.max_ctx, p.err) : 0;
            Lr[k] = has ? key_range(p, cb) : 0u;
            Fr[k] = (uint32_t)(cb + p.N);
            tl += (double)Lr[k];
        }
        tl = wave_sum_f64(tl);
        if (lane == 0 && act) sm.tot[wave] = tl;
        if (tid == 0) sm.pick[0] = -1;
        __syncthreads();
        const double tot = (sm.tot[0] + sm.tot[1]) + (sm.tot[2] + sm.tot[3]);
        int lo, hi;
        split_bounds(p, tot, lo, hi);
        int par = 0;
        const uint32_t sl = split_search(lo, hi, qm, umax, [&](uint32_t x) -> long long {
            uint32_t c = 0;
#pragma unroll
            for (int k = 0; k < kSchedRounds; ++k)
                if (k < rounds) c += (Lr[k] + x - 1u) / x;
            return (long long)H * sched_block_sum(c, sm, par);
        });
        // units of sequence b: a contiguous range, assigned round by round in
        // thread order (any fixed order works: the merge reads the table)
        uint32_t first = 0;
#pragma unroll
        for (int k = 0; k < kSchedRounds; ++k) {
            if (k >= rounds) break;
            const uint32_t ns = (Lr[k] + sl - 1u) / sl;
            const uint32_t incl = wave_scan_u32(ns);
            if (lane == 63 && act) sm.red[par][wave] = incl;
            __syncthreads();
            uint32_t before = first + incl - ns;
            uint32_t all = 0;
#pragma unroll
            for (int wv = 0; wv < 4; ++wv) {
                const uint32_t t = sm.red[par][wv];
                before += wv < wave ? t : 0u;
                all += t;
            }
            par ^= 1;
            sched_pick(sm, u, 256 * k + tid, Lr[k], Fr[k], ns, (long long)H * before, H, qm);
            first += all;
        }
        __syncthreads();
    }
    if (sm.pick[0] < 0) return false;
    w.b = sm.pick[0];
    const int rel = u - sm.pick[1];
    w.kvh = rel / sm.pick[2];
    w.s = rel % sm.pick[2];
    const int L = sm.pick[3], slb = sm.pick[4], full = sm.pick[5];
    w.ctx = full - p.N;
    w.p0 = (full - L) + w.s * slb;                     // the key range starts at full - L
    w.p1 = min(w.p0 + slb, full);
    w.part = u;
    if (record && rel == 0 && tid == 0) p.seq_tab[w.b] = make_int4(sm.pick[1], sm.pick[2], slb, 0);
    return true;
}

}  // namespace sv
