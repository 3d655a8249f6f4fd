// Split-KV verify attention on gfx950 bf16 matrix cores.
//
// One workgroup (4 waves) handles one (sequence, KV head, row block, split).
// The packed query rows of a KV head are r = node * G + g (G query heads share
// the KV head): the DDTree / DFlash verify rows of every query head of the
// GQA group [single-RTX-3090 DFlash note: 24 Q / 4 KV heads of dim 256,
// "Why we ran this test"; 16-row blocks, "Architecture"; budget+1 tree rows,
// "Key breakthroughs"].  Each wave owns up to NT tiles of 16 rows; waves split
// the positions of a staged tile when a row block has fewer tiles than waves.
//
// Per staged tile of T positions (T * D = 16384 bf16 per K or V):
//   global -> registers (prefetched one tile ahead, 16-byte loads, a wave
//   covers whole 512-byte rows) -> LDS: K in its natural [pos][d] order with an
//   XOR swizzle of 16-byte chunks, V transposed to [d][pos] by an in-register
//   8x8 transpose (4-bit caches are dequantised on the way in).
// Scores are computed transposed, S^T = K Q^T (16x16x32 bf16 MFMA: positions
// are the M side, rows the N side), so each lane holds one row and 8 of the
// chunk's 32 positions; row max/sum need only two cross-lane steps.  The
// probabilities of a lane are already the B operand of O^T = V^T P^T, and the
// O accumulators keep the same row-per-lane layout, so no shuffles are needed
// between the two products.  Online softmax in log2 units with a stale
// maximum: the accumulators are rescaled only when a row's maximum grows by
// more than 2^8 (exact: numerator and denominator share the reference).
//
// The tree mask [DFN "From autoregressive to DDTree"; for chains, the causal
// mask aligned to the end of the keys, xdnf.cn notes section 5.3] is a 64-bit
// ancestor set per node built in LDS from the parent array, applied only on
// chunks that reach the draft rows.
//
// Output per workgroup: unnormalised partials (O, m, l) per row; the merge
// kernel combines the splits.
#include "attn_sched.h"

namespace sv {
namespace {

template <int D, bool Q4, int NT, int PG>
struct Cfg {
    static constexpr int T = kMfmaTileElems / D;      // staged positions per tile
    static constexpr int CR = D / 8;                  // 16-byte bf16 chunks per K row
    static constexpr int KCH_PT = (T * CR) / 256;     // K chunks per thread (bf16)
    static constexpr int RG = 4 / PG;                 // row groups
    static constexpr int TW = T / PG;                 // positions per wave per tile
    static constexpr int KS = D / 32;                 // k-steps of S^T
    static constexpr int DT = D / 16;                 // 16-wide d tiles of O^T
    static constexpr int LDS_K = T * D * 2;
    static constexpr int LDS_V = D * T * 2;
    static constexpr int Q4_KPAIRS_PT = (T * (D / 32)) / 256;   // (row, block) pairs per thread
    static_assert(T % PG == 0 && TW % 32 == 0, "a wave handles whole 32-position chunks");
    static_assert((T * CR) % 256 == 0 && (T / 8) * CR == 256, "tile / thread mapping");
};

__device__ __forceinline__ int kswz(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int vswz(int d) { return (d + (d >> 3)) & 7; }

template <int D, bool Q4, bool PAGED, int NT, int PG>
__global__ __launch_bounds__(256, 1) void attn_mfma_kernel(AttnParams p) {
    using C = Cfg<D, Q4, NT, PG>;
    constexpr int T = C::T;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_K + C::LDS_V];
    __shared__ int par_s[64];
    __shared__ uint64_t anc_s[64];
    uint8_t *const Kl = lds;
    uint8_t *const Vl = lds + C::LDS_K;

    __shared__ SchedLds sched_s;

    // ---- which unit: (b, kv head, row block, split) ------------------------
    // Row blocks of one (b, kv head, split) get ids 8 apart: the dispatcher
    // deals ids round-robin to the 8 XCDs, so they share an L2.
    const int id = blockIdx.x;
    const int xcd = id & 7, k8 = id >> 3;
    const int rb = k8 % p.n_rowblocks;
    AttnUnit wu;
    if (!attn_unit(p, (k8 / p.n_rowblocks) * 8 + xcd, rb == 0, sched_s, wu)) return;
    const int b = wu.b, kvh = wu.kvh;
    const int N = p.N, G = p.G, R = p.R;
    const int ctx = wu.ctx, p0 = wu.p0, p1 = wu.p1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = wave % C::RG, pg = wave / C::RG;
    const int l16 = lane & 15, qd = lane >> 4;

    if (p1 > ctx) {                     // this split reaches the draft rows
        if (tid < N) par_s[tid] = parent_of(p.parent + (int64_t)b * N, tid, p.err);
        __syncthreads();
        if (tid < N) anc_s[tid] = ancestor_bits(par_s, tid);
        // visible after the first barrier of the tile loop
    }

    // ---- this lane's rows and their query fragments -------------------------
    const int row0 = rb * p.rows_per_block;
    const int rows_here = min(p.rows_per_block, R - row0);
    bool tile_on[NT];
    int node_of[NT];
    bf16x8 qf[NT][C::KS];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int rt = rg + C::RG * i;
        tile_on[i] = rt * 16 < rows_here;
        const int r = row0 + rt * 16 + l16;
        const bool ok = tile_on[i] && (rt * 16 + l16) < rows_here;
        node_of[i] = ok ? r / G : -1;
        if (ok) {
            const int n = r / G, g = r % G;
            const __bf16 *qp = (const __bf16 *)p.q +
                               (((int64_t)b * N + n) * p.Hq + (int64_t)kvh * G + g) * D + qd * 8;
#pragma unroll
            for (int k = 0; k < C::KS; ++k) qf[i][k] = *(const bf16x8 *)(qp + 32 * k);
        } else {
#pragma unroll
            for (int k = 0; k < C::KS; ++k) {
                const bf16x8 z = {};
                qf[i][k] = z;
            }
        }
    }

    f32x4 o[NT][C::DT];
    float m_ref[NT], l_sum[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        m_ref[i] = -INFINITY;
        l_sum[i] = 0.f;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) o[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- staging registers ---------------------------------------------------
    const int64_t krow_bytes = Q4 ? D / 2 : D * 2;       // bytes per KV row (codes for 4-bit)
    const int64_t srow_bytes = (D / 32) * 2;             // 4-bit scale bytes per row
    const uint8_t *kbase = (const uint8_t *)p.kv.k;
    const uint8_t *vbase = (const uint8_t *)p.kv.v;
    const uint8_t *ksbase = (const uint8_t *)p.kv.ks;
    const uint8_t *vsbase = (const uint8_t *)p.kv.vs;

    // bf16: K chunks (row = c / CR, chunk = c % CR) and one 8x8 V block per thread
    u32x4 kreg[Q4 ? 1 : C::KCH_PT];
    u32x4 vreg[Q4 ? 1 : 8];
    // 4-bit: (row, block) K pairs and one 8x8 V block (8 code dwords + 8 scales)
    u32x4 kq[Q4 ? C::Q4_KPAIRS_PT : 1];
    uint32_t ksq[Q4 ? C::Q4_KPAIRS_PT : 1];
    uint32_t vq[Q4 ? 8 : 1];
    uint32_t vsq[Q4 ? 8 : 1];

    const int vdg = tid % C::CR, vpg = tid / C::CR;      // V block: d group, position group

    auto row_idx = [&](int pos) -> int64_t {
        if (!PAGED) return ((int64_t)b * p.Hkv + kvh) * p.kv.capacity + pos;
        return kv_row_index(p.kv, b, p.Hkv, kvh, pos, p.err);
    };

    auto load_tile = [&](int tp) {
        if constexpr (!Q4) {
#pragma unroll
            for (int i = 0; i < C::KCH_PT; ++i) {
                const int c = tid + 256 * i;
                const int row = c / C::CR, ch = c % C::CR;
                const int pos = tp + row;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (pos < p1) {
                    const int64_t ri = row_idx(pos);
                    if (ri >= 0) val = *(const u32x4 *)(kbase + ri * krow_bytes + ch * 16);
                }
                kreg[i] = val;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int pos = tp + vpg * 8 + j;
                u32x4 val = {0u, 0u, 0u, 0u};
                if (pos < p1) {
                    const int64_t ri = row_idx(pos);
                    if (ri >= 0) val = *(const u32x4 *)(vbase + ri * krow_bytes + vdg * 16);
                }
                vreg[j] = val;
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::Q4_KPAIRS_PT; ++i) {
                const int c = tid + 256 * i;
                const int row = c / (D / 32), blk = c % (D / 32);
                const int pos = tp + row;
                u32x4 val = {0u, 0u, 0u, 0u};
                uint32_t sc = 0;
                if (pos < p1) {
                    const int64_t ri = row_idx(pos);
                    if (ri >= 0) {
                        val = *(const u32x4 *)(kbase + ri * krow_bytes + blk * 16);
                        sc = *(const uint16_t *)(ksbase + ri * srow_bytes + blk * 2);
                    }
                }
                kq[i] = val;
                ksq[i] = sc;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int pos = tp + vpg * 8 + j;
                uint32_t val = 0, sc = 0;
                if (pos < p1) {
                    const int64_t ri = row_idx(pos);
                    if (ri >= 0) {
                        val = *(const uint32_t *)(vbase + ri * krow_bytes + vdg * 4);
                        sc = *(const uint16_t *)(vsbase + ri * srow_bytes + (vdg / 4) * 2);
                    }
                }
                vq[j] = val;
                vsq[j] = sc;
            }
        }
    };

    auto store_tile = [&]() {
        if constexpr (!Q4) {
#pragma unroll
            for (int i = 0; i < C::KCH_PT; ++i) {
                const int c = tid + 256 * i;
                const int row = c / C::CR, ch = c % C::CR;
                *(u32x4 *)(Kl + row * (D * 2) + ((ch ^ kswz(row)) * 16)) = kreg[i];
            }
            // 8x8 transpose: vreg[j] holds d = 8*vdg .. +7 of position 8*vpg + j
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x4 w;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const uint32_t a = vreg[2 * kk][e >> 1], c2 = vreg[2 * kk + 1][e >> 1];
                    w[kk] = (e & 1) ? pack_hi_halves(a, c2) : pack_lo_halves(a, c2);
                }
                const int d = 8 * vdg + e;
                *(u32x4 *)(Vl + d * (T * 2) + ((vpg ^ vswz(d)) * 16)) = w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::Q4_KPAIRS_PT; ++i) {
                const int c = tid + 256 * i;
                const int row = c / (D / 32), blk = c % (D / 32);
                const float sc = fp16_bits_to_f32(ksq[i]);
                const float off8 = -8.f * sc;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t cw = kq[i][w];
                    u32x4 outw;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float lo = __builtin_fmaf((float)((cw >> (8 * t)) & 15u), sc, off8);
                        const float hi = __builtin_fmaf((float)((cw >> (8 * t + 4)) & 15u), sc, off8);
                        outw[t] = pack_bf16x2(lo, hi);
                    }
                    const int ch = 4 * blk + w;
                    *(u32x4 *)(Kl + row * (D * 2) + ((ch ^ kswz(row)) * 16)) = outw;
                }
            }
            float vs[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) vs[j] = fp16_bits_to_f32(vsq[j]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x4 w;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int j0 = 2 * kk, j1 = 2 * kk + 1;
                    const float a = __builtin_fmaf((float)((vq[j0] >> (4 * e)) & 15u), vs[j0], -8.f * vs[j0]);
                    const float c2 = __builtin_fmaf((float)((vq[j1] >> (4 * e)) & 15u), vs[j1], -8.f * vs[j1]);
                    w[kk] = pack_bf16x2(a, c2);
                }
                const int d = 8 * vdg + e;
                *(u32x4 *)(Vl + d * (T * 2) + ((vpg ^ vswz(d)) * 16)) = w;
            }
        }
    };

    // ---- main loop over staged tiles -----------------------------------------
    load_tile(p0);
#pragma unroll 1
    for (int tp = p0; tp < p1; tp += T) {
        __syncthreads();                         // previous tile fully consumed
        store_tile();
        __syncthreads();
        if (tp + T < p1) load_tile(tp + T);      // in flight during this tile's math

#pragma unroll 1
        for (int c = 0; c < C::TW / 32; ++c) {
            const int cb = pg * C::TW + c * 32;   // chunk base within the tile
            const int abase = tp + cb;            // absolute position of the chunk
            if (abase >= p1) break;

            f32x4 sacc[NT][2];
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                sacc[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                sacc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int krow = cb + 8 * (l16 >> 2) + 4 * t + (l16 & 3);
                const uint8_t *kp = Kl + krow * (D * 2);
                const int sw = kswz(krow);
#pragma unroll
                for (int k = 0; k < C::KS; ++k) {
                    const bf16x8 a = *(const bf16x8 *)(kp + (((4 * k + qd) ^ sw) * 16));
#pragma unroll
                    for (int i = 0; i < NT; ++i)
                        if (tile_on[i])
                            sacc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[i][k], sacc[i][t], 0, 0, 0);
                }
            }

            const bool need_mask = (abase + 32 > ctx) || (abase + 32 > p1);
            bf16x8 pb[NT];
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                if (!tile_on[i]) continue;
                float sv[8];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) sv[4 * t + j] = sacc[i][t][j] * p.scale_log2;
                if (need_mask) {
                    const uint64_t anc = node_of[i] >= 0 ? anc_s[node_of[i]] : 0ull;
                    const int rel0 = abase + 8 * qd - ctx;      // draft index of value 0
                    const int lim = p1 - (abase + 8 * qd);      // values e < lim are in the split
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int rel = rel0 + e;
                        bool vis = e < lim;
                        if (rel >= 0) vis = vis && (((anc >> (rel & 63)) & 1ull) != 0ull);
                        sv[e] = vis ? sv[e] : -INFINITY;
                    }
                }
                float cm = sv[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) cm = fmaxf(cm, sv[e]);
                cm = fmaxf(cm, xor_shfl(cm, 16));
                cm = fmaxf(cm, xor_shfl(cm, 32));
                const bool need = cm > m_ref[i] + 8.f;
                if (__any(need)) {
                    const float mn = need ? cm : m_ref[i];
                    const float alpha = need ? exp2f(m_ref[i] - mn) : 1.f;
                    m_ref[i] = mn;
                    l_sum[i] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt) o[i][dt] *= alpha;
                }
                const float mu = (m_ref[i] == -INFINITY) ? 0.f : m_ref[i];
                float pr[8];
                float ls = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pr[e] = exp2f(sv[e] - mu);
                    ls += pr[e];
                }
                l_sum[i] += ls;
#pragma unroll
                for (int e = 0; e < 8; ++e) pb[i][e] = (__bf16)pr[e];
            }

            // O^T += V^T P^T over this chunk's 32 positions
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                const int vrow = 16 * dt + l16;
                const bf16x8 a = *(const bf16x8 *)(Vl + vrow * (T * 2) +
                                                   ((((cb >> 3) + qd) ^ vswz(vrow)) * 16));
#pragma unroll
                for (int i = 0; i < NT; ++i)
                    if (tile_on[i])
                        o[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[i], o[i][dt], 0, 0, 0);
            }
        }
    }

    // ---- combine the position groups of a row group (PG > 1) ------------------
    if constexpr (PG > 1) {
        __syncthreads();
        f32x4 *buf = (f32x4 *)lds;
        constexpr int SLOT = C::DT + 1;
        static_assert((PG - 1) * C::RG * NT * SLOT * 64 * 16 <= C::LDS_K + C::LDS_V, "combine buffer");
        if (pg > 0) {
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const int slot = ((pg - 1) * C::RG + rg) * NT + i;      // own slot per (group, row group)
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) buf[(slot * SLOT + dt) * 64 + lane] = o[i][dt];
                buf[(slot * SLOT + C::DT) * 64 + lane] = f32x4{m_ref[i], l_sum[i], 0.f, 0.f};
            }
        }
        __syncthreads();
        if (pg > 0) return;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            float mx = m_ref[i];
            for (int q2 = 1; q2 < PG; ++q2) {
                const int slot = ((q2 - 1) * C::RG + rg) * NT + i;
                mx = fmaxf(mx, buf[(slot * SLOT + C::DT) * 64 + lane][0]);
            }
            const float w0 = (m_ref[i] == -INFINITY) ? 0.f : exp2f(m_ref[i] - mx);
            l_sum[i] *= w0;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) o[i][dt] *= w0;
            for (int q2 = 1; q2 < PG; ++q2) {
                const int slot = ((q2 - 1) * C::RG + rg) * NT + i;
                const f32x4 ml = buf[(slot * SLOT + C::DT) * 64 + lane];
                const float w = (ml[0] == -INFINITY) ? 0.f : exp2f(ml[0] - mx);
                l_sum[i] += w * ml[1];
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) o[i][dt] += w * buf[(slot * SLOT + dt) * 64 + lane];
            }
            m_ref[i] = mx;
        }
    }

    // ---- write the partials of this split ---------------------------------------
    const int64_t part = wu.part;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if (!tile_on[i]) continue;
        float ls = l_sum[i];
        ls += xor_shfl(ls, 16);
        ls += xor_shfl(ls, 32);
        const int rt = rg + C::RG * i;
        const int rl = rt * 16 + l16;
        if (rl >= rows_here) continue;
        const int r = row0 + rl;
        float *op = p.part_o + (part * R + r) * D + qd * 4;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) *(f32x4 *)(op + 16 * dt) = o[i][dt];
        if (qd == 0) {
            p.part_ml[(part * R + r) * 2 + 0] = m_ref[i];
            p.part_ml[(part * R + r) * 2 + 1] = ls;
        }
    }
}

template <int D, bool Q4, bool PAGED, int NT, int PG>
hipError_t launch_one(const AttnParams &p, hipStream_t st) {
    const int grid = ((p.n_units + 7) / 8) * 8 * p.n_rowblocks;
    hipLaunchKernelGGL((attn_mfma_kernel<D, Q4, PAGED, NT, PG>), dim3(grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int D, bool Q4, bool PAGED>
hipError_t launch_shape(const AttnParams &p, int nt, int pg, hipStream_t st) {
    if (pg == 1) {
        if (nt == 1) return launch_one<D, Q4, PAGED, 1, 1>(p, st);
        if (nt == 2) return launch_one<D, Q4, PAGED, 2, 1>(p, st);
        if (nt == 3) return launch_one<D, Q4, PAGED, 3, 1>(p, st);
    } else if (pg == 2 && nt == 1) {
        return launch_one<D, Q4, PAGED, 1, 2>(p, st);
    } else if (pg == 4 && nt == 1 && D <= 128) {
        return launch_one<D, Q4, PAGED, 1, (D <= 128 ? 4 : 2)>(p, st);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_d(const AttnParams &p, int dtype, int nt, int pg, hipStream_t st) {
    const bool paged = p.kv.page_table != nullptr;
    if (dtype == SV_Q4)
        return paged ? launch_shape<D, true, true>(p, nt, pg, st) : launch_shape<D, true, false>(p, nt, pg, st);
    return paged ? launch_shape<D, false, true>(p, nt, pg, st) : launch_shape<D, false, false>(p, nt, pg, st);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams &p, int dtype, int D, int nt, int pg, hipStream_t st) {
    switch (D) {
        case 64: return launch_d<64>(p, dtype, nt, pg, st);
        case 128: return launch_d<128>(p, dtype, nt, pg, st);
        case 256: return launch_d<256>(p, dtype, nt, pg, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace sv
