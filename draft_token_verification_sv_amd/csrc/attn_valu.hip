// Vector-ALU verify attention (fp32 arithmetic) and the split merge.
//
// The VALU kernel serves packed row blocks of fewer than 16 rows with bf16
// queries (single-row decode, small GQA groups) and every fp32-query call.  It
// stages each KV tile in LDS as fp32 (4-bit rows dequantised as d * (n - 8)),
// keeps up to 16 query rows in LDS, and gives each row 16 threads: the
// threads of a row split the tile's positions for the scores and the head
// dimension for the output accumulation.  The tree mask is the ancestor-set
// mask built in LDS from the parent array [single-RTX-3090 DFlash note,
// "From autoregressive to DDTree"; causal mask aligned to the end of the keys,
// xdnf.cn notes section 5.3].  Partials use the same layout as the matrix-core
// kernel.
//
// The merge combines the splits of every row with the log-sum-exp rule
//   M = max_s m_s,  out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
//   lse = ln 2 * (M + log2 sum_s 2^(m_s - M) l_s)
// (m in log2 units), and writes the output in the query dtype.
#include "attn_sched.h"

namespace sv {
namespace {

constexpr int kRowsV = 16;

template <int KVT>
__device__ __forceinline__ void load_row_chunk_f32(float *dst, const uint8_t *base, const uint8_t *sbase,
                                                   int64_t ri, int chunk, int D) {
    // one 16-byte chunk of codes / values of row ri, widened to fp32 into dst
    if constexpr (KVT == SV_F32) {
        const f32x4 v = *(const f32x4 *)(base + ri * (D * 4) + chunk * 16);
        dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
    } else if constexpr (KVT == SV_BF16) {
        const u32x4 v = *(const u32x4 *)(base + ri * (D * 2) + chunk * 16);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            dst[2 * w] = bf16_bits_to_f32(v[w] & 0xFFFFu);
            dst[2 * w + 1] = bf16_bits_to_f32(v[w] >> 16);
        }
    } else {
        // a 16-byte chunk of codes is one 32-value block
        const u32x4 v = *(const u32x4 *)(base + ri * (D / 2) + chunk * 16);
        const float d = fp16_bits_to_f32(*(const uint16_t *)(sbase + ri * ((D / 32) * 2) + chunk * 2));
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                dst[8 * w + t] = (float)(int)((v[w] >> (4 * t)) & 15u) * d - 8.f * d;
    }
}

template <int D, int KVT, bool QF32>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnParams p) {
    constexpr int T = kValuTileElems / D;          // 32, 64 or 128 positions per tile
    constexpr int DP = D + 1;                      // padded K row (bank spread)
    constexpr int VPC = (KVT == SV_F32) ? 4 : (KVT == SV_BF16 ? 8 : 32);  // values per chunk
    constexpr int CPR = D / VPC;                   // chunks per row
    __shared__ float Ks[T * DP];
    __shared__ float Vs[T * D];
    __shared__ float Qs[kRowsV * D];
    __shared__ float Ps[kRowsV * T];
    __shared__ int par_s[64];
    __shared__ uint64_t anc_s[64];

    __shared__ SchedLds sched_s;

    const int id = blockIdx.x;
    const int xcd = id & 7, k8 = id >> 3;
    const int rb = k8 % p.n_rowblocks;
    AttnUnit wu;
    if (!attn_unit(p, (k8 / p.n_rowblocks) * 8 + xcd, rb == 0, sched_s, wu)) return;
    const int b = wu.b, kvh = wu.kvh;
    const int N = p.N, G = p.G, R = p.R;
    const int ctx = wu.ctx, p0 = wu.p0, p1 = wu.p1;

    const int tid = threadIdx.x;
    const int r = tid >> 4, j = tid & 15;           // row in block, thread in row
    const int rglob = rb * kRowsV + r;
    const bool row_ok = r < p.rows_per_block && rglob < R;

    if (tid < N) par_s[tid] = parent_of(p.parent + (int64_t)b * N, tid, p.err);
    __syncthreads();
    if (tid < N) anc_s[tid] = ancestor_bits(par_s, tid);

    // query rows -> LDS (fp32)
    for (int e = tid; e < kRowsV * D; e += 256) {
        const int rr = e / D, d = e % D;
        const int rg = rb * kRowsV + rr;
        float val = 0.f;
        if (rr < p.rows_per_block && rg < R) {
            const int n = rg / G, g = rg % G;
            const int64_t qi = (((int64_t)b * N + n) * p.Hq + (int64_t)kvh * G + g) * D + d;
            val = QF32 ? ((const float *)p.q)[qi] : bf16_bits_to_f32(((const uint16_t *)p.q)[qi]);
        }
        Qs[e] = val;
    }
    __syncthreads();
    const uint64_t anc = row_ok ? anc_s[rglob / G] : 0ull;

    float o[D / 16];
#pragma unroll
    for (int k = 0; k < D / 16; ++k) o[k] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const uint8_t *kb = (const uint8_t *)p.kv.k, *vb = (const uint8_t *)p.kv.v;
    const uint8_t *ksb = (const uint8_t *)p.kv.ks, *vsb = (const uint8_t *)p.kv.vs;

#pragma unroll 1
    for (int tp = p0; tp < p1; tp += T) {
        // the tile's positions in the split: the loops below stop there (a
        // short split costs what its positions cost, not a whole tile)
        const int nv = min(T, p1 - tp);
        // stage K and V rows [tp, tp + nv) as fp32
        for (int c = tid; c < nv * CPR; c += 256) {
            const int row = c / CPR, ch = c % CPR;
            const int pos = tp + row;
            float kv8[VPC], vv8[VPC];
            bool ok = false;
            if (pos < p1) {
                const int64_t ri = kv_row_index(p.kv, b, p.Hkv, kvh, pos, p.err);
                if (ri >= 0) {
                    load_row_chunk_f32<KVT>(kv8, kb, ksb, ri, ch, D);
                    load_row_chunk_f32<KVT>(vv8, vb, vsb, ri, ch, D);
                    ok = true;
                }
            }
#pragma unroll
            for (int e = 0; e < VPC; ++e) {
                Ks[row * DP + ch * VPC + e] = ok ? kv8[e] : 0.f;
                Vs[row * D + ch * VPC + e] = ok ? vv8[e] : 0.f;
            }
        }
        __syncthreads();

        // scores for this thread's positions j, j+16, ...
        float sc[T / 16];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < T / 16; ++i) {
            const int pt = j + 16 * i;
            const int pos = tp + pt;
            float acc = 0.f;
            if (pt < nv) {
#pragma unroll 8
                for (int d = 0; d < D; ++d) acc = __builtin_fmaf(Qs[r * D + d], Ks[pt * DP + d], acc);
            }
            const int rel = pos - ctx;          // draft index (negative: cache row)
            bool vis = row_ok && pos < p1;
            if (rel >= 0) vis = vis && (((anc >> (rel & 63)) & 1ull) != 0ull);
            sc[i] = vis ? acc * p.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, sc[i]);
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, m, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float mu = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - mu);
        float lt = 0.f;
#pragma unroll
        for (int i = 0; i < T / 16; ++i) {
            const float pr = exp2f(sc[i] - mu);
            Ps[r * T + j + 16 * i] = pr;
            lt += pr;
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) lt += __shfl_xor(lt, m, 64);
        l_run = l_run * alpha + lt;
        m_run = m_new;
        __syncthreads();

#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
            const int d = j + 16 * k;
            float acc = o[k] * alpha;
#pragma unroll 8
            for (int pt = 0; pt < nv; ++pt) acc = __builtin_fmaf(Ps[r * T + pt], Vs[pt * D + d], acc);
            o[k] = acc;
        }
        __syncthreads();
    }

    if (!row_ok) return;
    const int64_t part = wu.part;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) p.part_o[(part * R + rglob) * D + j + 16 * k] = o[k];
    if (j == 0) {
        p.part_ml[(part * R + rglob) * 2 + 0] = m_run;
        p.part_ml[(part * R + rglob) * 2 + 1] = l_run;
    }
}

// Split merge: one block of 256 threads per output row.  Thread t covers the 4
// columns 4 (t % (D/4)) .. +3 of the splits s = t / (D/4) (mod NSG), NSG =
// 1024 / D split groups, with 16-byte loads.  Each wavefront loads the (m, l)
// pairs of all splits, then the first OB partial rows of each thread; it finds
// M = max_s m_s and the weights 2^(m_s - M) (kept in its own LDS copy) by lane
// shuffles while the rows land, every thread accumulates its weighted
// partials, and the split groups add up through LDS (the one block barrier).
// Slots past the sequence's splits (not written by this call) are never used.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
    constexpr int CG = D / 4;               // column groups of one row
    constexpr int NSG = 256 / CG;           // split groups
    constexpr int OB = 16;                  // partial rows in flight per thread
    __shared__ float w_s[4][kMaxSplits];            // split weights, one copy per wavefront
    __shared__ f32x4 acc_s[NSG - 1][CG];
    const int tid = threadIdx.x;
    const int c = tid % CG, sg = tid / CG;
    const int lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x;
    const int h = row % p.Hq;
    const int n = (row / p.Hq) % p.N;
    const int b = row / (p.Hq * p.N);
    const int kvh = h / p.G, g = h % p.G;
    const int r = n * p.G + g;
    // first partial slot and split count of (b, kvh); the static schedule
    // knows the slots without the context length, so the loads start together
    // with the ctx_lens load
    int64_t base;
    int ns, ns_cap;
    if (p.dyn) {
        const int4 tb = p.seq_tab[b];
        base = tb.x + (int64_t)kvh * tb.y;
        ns = ns_cap = tb.y;
    } else {
        base = ((int64_t)b * p.Hkv + kvh) * p.n_splits;
        ns_cap = p.n_splits;
        const int L = (int)key_range(p, ctx_of(p.ctx_lens, b, p.max_ctx, p.err));
        ns = min(p.n_splits, (L + p.split_len - 1) / p.split_len);
    }
    // every wavefront reads all (m, l) pairs itself (one per lane up to 64
    // splits), before the partial rows: the maximum and the weights are then
    // formed while the rows are still in flight, with no workgroup barrier
    const float2 *ml = (const float2 *)p.part_ml + base * p.R + r;
    const float2 ml0 = lane < ns_cap ? ml[(int64_t)lane * p.R] : make_float2(-INFINITY, 0.f);
    const float *op = p.part_o + (base * p.R + r) * D + 4 * c;
    const int64_t sstride = (int64_t)p.R * D;
    f32x4 ov[OB];
#pragma unroll
    for (int k = 0; k < OB; ++k) {
        const int sp = sg + k * NSG;
        ov[k] = sp < ns_cap ? *(const f32x4 *)(op + sp * sstride) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float M = lane < ns ? ml0.x : -INFINITY;
    for (int j = 64 + lane; j < ns; j += 64) M = fmaxf(M, ml[(int64_t)j * p.R].x);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    float *w_w = w_s[wave];
    float ls = 0.f;
    if (lane < ns) {
        const float w = ml0.x == -INFINITY ? 0.f : exp2f(ml0.x - M);
        w_w[lane] = w;
        ls = w * ml0.y;
    }
    for (int j = 64 + lane; j < ns; j += 64) {
        const float2 t = ml[(int64_t)j * p.R];
        const float w = t.x == -INFINITY ? 0.f : exp2f(t.x - M);
        w_w[j] = w;
        ls += w * t.y;
    }
    float lsum = ls;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) lsum += __shfl_xor(lsum, m, 64);
    // the weights were written by other lanes of this wavefront
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < OB; ++k) {
        const int sp = sg + k * NSG;
        if (sp < ns) acc += w_w[sp] * ov[k];
    }
#pragma unroll 1
    for (int s0 = OB * NSG; s0 < ns; s0 += OB * NSG) {
#pragma unroll
        for (int k = 0; k < OB; ++k) {
            const int sp = s0 + sg + k * NSG;
            ov[k] = sp < ns ? *(const f32x4 *)(op + sp * sstride) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < OB; ++k) {
            const int sp = s0 + sg + k * NSG;
            if (sp < ns) acc += w_w[sp] * ov[k];
        }
    }
    if (sg > 0) acc_s[sg - 1][c] = acc;
    __syncthreads();
    if (sg > 0) return;
#pragma unroll
    for (int k = 0; k < NSG - 1; ++k) acc += acc_s[k][c];
    if (p.part_perm) {
        // slots 4c .. 4c + 3 hold head dims 8 (c / 2) + (0, 4, 2, 6) for even c,
        // (1, 5, 3, 7) for odd c: with the neighbour's four each lane has its
        // four consecutive dims 4c .. 4c + 3
        const f32x4 o = {__shfl_xor(acc[0], 1, 64), __shfl_xor(acc[1], 1, 64), __shfl_xor(acc[2], 1, 64),
                         __shfl_xor(acc[3], 1, 64)};
        acc = (c & 1) == 0 ? f32x4{acc[0], o[0], acc[2], o[2]} : f32x4{o[1], acc[1], o[3], acc[3]};
    }
    const float inv = 1.f / lsum;
    const int64_t oi = (((int64_t)b * p.N + n) * p.Hq + h) * D + 4 * c;
    if (p.q_f32) {
        *(f32x4 *)((float *)p.out + oi) = acc * inv;
    } else {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(acc[0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(acc[2] * inv) | ((uint32_t)f32_to_bf16_bits(acc[3] * inv) << 16);
        *(uint2 *)((uint16_t *)p.out + oi) = pk;
    }
    if (tid == 0 && p.lse != nullptr)
        p.lse[((int64_t)b * p.N + n) * p.Hq + h] = (M + log2f(lsum)) * 0.69314718055994530942f;
}

template <int D, int KVT>
hipError_t launch_valu_t(const AttnParams &p, hipStream_t st) {
    const int grid = ((p.n_units + 7) / 8) * 8 * p.n_rowblocks;
    if (p.q_f32)
        hipLaunchKernelGGL((attn_valu_kernel<D, KVT, true>), dim3(grid), dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((attn_valu_kernel<D, KVT, false>), dim3(grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_valu_d(const AttnParams &p, int dtype, hipStream_t st) {
    if (dtype == SV_F32) return launch_valu_t<D, SV_F32>(p, st);
    if (dtype == SV_BF16) return launch_valu_t<D, SV_BF16>(p, st);
    if (dtype == SV_Q4) return launch_valu_t<D, SV_Q4>(p, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_valu(const AttnParams &p, int dtype, int D, hipStream_t st) {
    switch (D) {
        case 64: return launch_valu_d<64>(p, dtype, st);
        case 128: return launch_valu_d<128>(p, dtype, st);
        case 256: return launch_valu_d<256>(p, dtype, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(const AttnParams &p, int D, hipStream_t st) {
    const int rows = p.B * p.N * p.Hq;
    switch (D) {
        case 64:
            hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(rows), dim3(256), 0, st, p);
            break;
        case 128:
            hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(rows), dim3(256), 0, st, p);
            break;
        case 256:
            hipLaunchKernelGGL(attn_merge_kernel<256>, dim3(rows), dim3(256), 0, st, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sv
