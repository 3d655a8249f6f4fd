// Tree-aware recurrent state of the hybrid target's Gated DeltaNet layers.
//
// The single-RTX-3090 DFlash note verifies DDTree trees on a target whose
// DeltaNet layers keep a recurrent state next to the KV cache ("Why we ran
// this test"); its "Key breakthroughs" section names the two tree kernels
// this file provides for gfx950, plus the commit that follows acceptance:
//
//   conv_tree_kernel    the short causal depthwise conv in front of the
//                       recurrence, each node's window gathered along its
//                       parent chain (past the root: the committed conv state);
//   delta_tree_kernel   the gated delta rule (Yang, Kautz, Hatamizadeh, Gated
//                       Delta Networks, ICLR 2025) over the tree, every node's
//                       state written straight to the per-node buffer (fp32
//                       or f16) in the same pass;
//   commit_kernel       the accepted node's state into the committed state and
//                       the accepted path's last K-1 inputs into the conv state.
//
// delta_tree_kernel: one workgroup of 4 waves per (sequence, value head, block
// of 32 value rows); lane (jr, rg) of a wave owns value row jr and 8*R/8 = R of
// the key columns, in chunks of VEC contiguous columns spaced 8*VEC apart (so
// the 8 lanes of a row store whole 128-byte lines of the per-node buffer).  The
// state never leaves registers between a node and its first child.  Nodes are
// visited in depth-first order with the children of each node sorted by
// subtree size (largest last): a node with two or more children parks its
// state in an LDS slot that its later children restore; along any root path a
// slot is live only below a child that is not its parent's largest, so at most
// floor(log2(N+1)) - 1 slots are ever live.  The order is computed per wave
// with one lane per node (ancestor sets by pointer doubling, subtree sizes,
// sibling ranks), no host work.
#include "device_common.h"

namespace sv {
namespace {

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// sum over the 8 lanes 8m .. 8m+7 (result in all 8)
__device__ __forceinline__ float sum8(float v) {
    v += dpp_f<0xB1>(v);      // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);      // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);     // row_half_mirror
    return v;
}

template <int DT>
__device__ __forceinline__ f32x4 load4(const void *base, int64_t off) {
    if constexpr (DT == SV_F32) {
        return *(const f32x4 *)((const float *)base + off);
    } else {
        const u32x2 u = *(const u32x2 *)((const uint16_t *)base + off);
        return f32x4{bf16_bits_to_f32(u[0] & 0xFFFFu), bf16_bits_to_f32(u[0] >> 16),
                     bf16_bits_to_f32(u[1] & 0xFFFFu), bf16_bits_to_f32(u[1] >> 16)};
    }
}

template <int DT>
__device__ __forceinline__ void store4(void *base, int64_t off, f32x4 v) {
    if constexpr (DT == SV_F32) {
        *(f32x4 *)((float *)base + off) = v;
    } else {
        *(u32x2 *)((uint16_t *)base + off) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const uint32_t l = __builtin_bit_cast(uint16_t, (_Float16)lo);   // round to nearest even
    const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)hi);
    return l | (h << 16);
}

// ---------------------------------------------------------------------------
// conv windows along parent chains
// ---------------------------------------------------------------------------

// One thread per (sequence, node, 4 channels); grid (C/1024 rounded up, N, B).
template <int DT, int K>
__global__ __launch_bounds__(256) void conv_tree_kernel(ConvTreeParams p) {
    const int b = blockIdx.z, i = blockIdx.y;
    const int c0 = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c0 >= p.C) return;
    const int N = p.N, C = p.C;
    float w[4 * K];                     // taps of channels c0 .. c0+3 (4K contiguous floats)
#pragma unroll
    for (int e = 0; e < K; ++e) {
        const f32x4 t = *(const f32x4 *)(p.w + (int64_t)c0 * K + 4 * e);
#pragma unroll
        for (int u = 0; u < 4; ++u) w[4 * e + u] = t[u];
    }
    f32x4 acc = p.bias ? *(const f32x4 *)(p.bias + c0) : f32x4{0.f, 0.f, 0.f, 0.f};
    // the window, newest first: node i, its parent, ... then the conv state
    int node = i;
    int back = 0;                       // conv-state rows used so far
#pragma unroll
    for (int m = 0; m < K; ++m) {
        f32x4 val;
        if (node >= 0) {
            val = load4<DT>(p.x, ((int64_t)b * N + node) * C + c0);
            int pn;
            if (p.parent == nullptr) {
                pn = node - 1;
            } else {
                pn = p.parent[(int64_t)b * N + node];
                if (pn < 0 || pn >= node) pn = -1;
            }
            node = pn;
        } else {
            ++back;
            val = load4<DT>(p.conv_state, ((int64_t)b * (K - 1) + (K - 1 - back)) * C + c0);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = fmaf(w[c * K + K - 1 - m], val[c], acc[c]);
    }
    if (p.silu) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = acc[c] / (1.0f + expf(-acc[c]));
    }
    store4<DT>(p.out, ((int64_t)b * N + i) * C + c0, acc);
}

// ---------------------------------------------------------------------------
// gated delta rule over the tree, every node's state persisted
// ---------------------------------------------------------------------------

template <int NMAX>
struct SlotCount {
    static constexpr int value = NMAX <= 16 ? 3 : (NMAX <= 32 ? 4 : 5);   // floor(log2(NMAX+1)) - 1
};

template <int R, int NMAX, bool TREE, int DT, int SDT>
__global__ __launch_bounds__(256) void delta_tree_kernel(DeltaParams p) {
    constexpr int DK = 8 * R;
    constexpr int VEC = SDT == SV_F16 ? 8 : 4;        // contiguous key columns per chunk
    constexpr int NCH = R / VEC;                      // chunks per lane
    constexpr int NSLOT = TREE ? SlotCount<NMAX>::value : 0;
    static_assert(R % VEC == 0, "chunking");

    __shared__ __attribute__((aligned(16))) float k_s[NMAX * DK];
    __shared__ __attribute__((aligned(16))) float q_s[NMAX * DK];
    __shared__ float v_s[NMAX * 32];
    __shared__ float a_s[NMAX], b_s[NMAX];
    __shared__ __attribute__((aligned(16))) f32x4 slot_s[NSLOT > 0 ? NSLOT * 4 * (R / 4) * 64 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int jb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int N = p.N, Hv = p.Hv, Dv = p.Dv;
    const int hk = h / (Hv / p.Hk);
    const int jr = lane >> 3, rg = lane & 7;
    const int jrow = jb * 32 + wave * 8 + jr;         // this lane's value row
    const int64_t bn = (int64_t)b * N;

    // ---- stage q, k (all nodes, this key head), v (32 rows), decay, beta ----
    // (all loads issued first; they land in LDS after the order is computed)
    constexpr int QK_IT = (NMAX * DK / 4 + 255) / 256;
    constexpr int V_IT = (NMAX * 8 + 255) / 256;
    f32x4 qv[QK_IT], kv[QK_IT], vv[V_IT];
    float gv = 0.f, bv = 0.f;
#pragma unroll
    for (int it = 0; it < QK_IT; ++it) {
        const int e = tid + it * 256;
        if (e < N * (DK / 4)) {
            const int i = e / (DK / 4), c4 = e - i * (DK / 4);
            const int64_t off = (bn + i) * p.qk_stride + (int64_t)hk * DK + 4 * c4;
            qv[it] = load4<DT>(p.q, off);
            kv[it] = load4<DT>(p.k, off);
        }
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
        const int e = tid + it * 256;
        if (e < N * 8) {
            const int i = e >> 3, c4 = e & 7;
            vv[it] = load4<DT>(p.v, (bn + i) * p.v_stride + (int64_t)h * Dv + jb * 32 + 4 * c4);
        }
    }
    if (tid < N) {
        gv = p.g[(bn + tid) * Hv + h];
        bv = p.beta[(bn + tid) * Hv + h];
    }

    // ---- committed state into registers ----
    float S[R];
    const float *s0 = p.state + (((int64_t)b * Hv + h) * Dv + jrow) * DK + rg * VEC;
    auto load_s0 = [&]() {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
#pragma unroll
            for (int u = 0; u < VEC / 4; ++u) {
                const f32x4 t = *(const f32x4 *)(s0 + c * 8 * VEC + 4 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e) S[c * VEC + 4 * u + e] = t[e];
            }
        }
    };
    load_s0();

    // ---- depth-first order, one lane per node ----
    int par = lane - 1, pos = lane, slot = 0, nch = 0;
    if constexpr (TREE) {
        const bool live = lane < N;
        par = -1;
        if (live) {
            const int pr = p.parent[bn + lane];
            par = (pr >= 0 && pr < lane) ? pr : -1;
        }
        // ancestor-or-self sets by pointer doubling (depth < 64)
        uint64_t anc = live ? (1ull << lane) : 0ull;
        int jp = par;
#pragma unroll 1
        for (int r = 0; r < 6; ++r) {
            if (__ballot(jp >= 0) == 0) break;
            const int src = jp >= 0 ? jp : lane;
            const uint32_t alo = (uint32_t)__shfl((int)(uint32_t)anc, src, 64);
            const uint32_t ahi = (uint32_t)__shfl((int)(uint32_t)(anc >> 32), src, 64);
            const int jp2 = __shfl(jp, src, 64);
            if (jp >= 0) {
                anc |= ((uint64_t)ahi << 32) | alo;
                jp = jp2;
            }
        }
        // subtree sizes and child counts
        int size = 0;
#pragma unroll 1
        for (int j = 0; j < N; ++j) {
            const uint32_t alo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)anc, j);
            const uint32_t ahi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(anc >> 32), j);
            const uint64_t aj = ((uint64_t)ahi << 32) | alo;
            size += (int)((aj >> lane) & 1ull);
            nch += __builtin_amdgcn_readlane(par, j) == lane ? 1 : 0;
        }
        // siblings ordered by (subtree size, index); the last one is the largest
        int pre = 0;
        bool last = true;
#pragma unroll 1
        for (int j = 0; j < N; ++j) {
            const int pj = __builtin_amdgcn_readlane(par, j);
            const int sj = __builtin_amdgcn_readlane(size, j);
            if (pj == par && j != lane) {
                if (sj < size || (sj == size && j < lane)) pre += sj;
                else last = false;
            }
        }
        const int light = (par >= 0 && !last) ? 1 : 0;
        // preorder position and slot index from the ancestors' ranks
        pos = -1;
#pragma unroll 1
        for (int j = 0; j < N; ++j) {
            const int pj = __builtin_amdgcn_readlane(pre, j);
            const int lj = __builtin_amdgcn_readlane(light, j);
            if ((anc >> j) & 1ull) {
                pos += 1 + pj;
                slot += lj;
            }
        }
        if (!live) pos = -1;
    }

#pragma unroll
    for (int it = 0; it < QK_IT; ++it) {
        const int e = tid + it * 256;
        if (e < N * (DK / 4)) {
            *(f32x4 *)&q_s[4 * e] = qv[it];          // node e / (DK/4), columns 4 (e % (DK/4)) ..
            *(f32x4 *)&k_s[4 * e] = kv[it];
        }
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
        const int e = tid + it * 256;
        if (e < N * 8) *(f32x4 *)&v_s[4 * e] = vv[it];
    }
    if (tid < N) {
        a_s[tid] = expf(gv);
        b_s[tid] = bv;
    }
    __syncthreads();

    // ---- the walk ----
    const float scale = p.scale;
    f32x4 *my_slot = slot_s + wave * (R / 4) * 64 + lane;           // + s * 4 * (R/4) * 64 + t * 64
    int prev = -1;
#pragma unroll 1
    for (int ks = 0; ks < N; ++ks) {
        int x = ks;
        if constexpr (TREE) {
            const uint64_t m = __ballot(pos == ks);
            if (m == 0ull) break;                                   // not reached for a valid order
            x = (int)__builtin_ctzll(m);
            const int px = __builtin_amdgcn_readlane(par, x);
            if (px != prev) {
                if (px < 0) {
                    load_s0();                                      // another root: the committed state
                } else {
                    const int sp = __builtin_amdgcn_readlane(slot, px);
                    if (sp < NSLOT) {
#pragma unroll
                        for (int t = 0; t < R / 4; ++t) {
                            const f32x4 v4 = my_slot[(sp * 4 * (R / 4) + t) * 64];
#pragma unroll
                            for (int e = 0; e < 4; ++e) S[4 * t + e] = v4[e];
                        }
                    }
                }
            }
        }
        const float a = a_s[x], bt = b_s[x];
        float kk[R], qq[R];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
#pragma unroll
            for (int u = 0; u < VEC / 4; ++u) {
                const int col = c * 8 * VEC + rg * VEC + 4 * u;
                const f32x4 k4 = *(const f32x4 *)&k_s[x * DK + col];
                const f32x4 q4 = *(const f32x4 *)&q_s[x * DK + col];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kk[c * VEC + 4 * u + e] = k4[e];
                    qq[c * VEC + 4 * u + e] = q4[e];
                }
            }
        }
        // u = beta (v - a S k);  S <- a S + u k^T;  o = scale S q
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int t = 0; t < R; t += 2) {
            d0 = fmaf(S[t], kk[t], d0);
            d1 = fmaf(S[t + 1], kk[t + 1], d1);
        }
        const float dot = sum8(d0 + d1);
        const float u = (v_s[x * 32 + wave * 8 + jr] - a * dot) * bt;
#pragma unroll
        for (int t = 0; t < R; ++t) S[t] = fmaf(S[t], a, u * kk[t]);
        float o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int t = 0; t < R; t += 2) {
            o0 = fmaf(S[t], qq[t], o0);
            o1 = fmaf(S[t + 1], qq[t + 1], o1);
        }
        const float o = sum8(o0 + o1) * scale;
        const int64_t orow = (bn + x) * Hv + h;
        if (rg == 0) {
            if constexpr (DT == SV_F32) {
                ((float *)p.out)[orow * Dv + jrow] = o;
            } else {
                ((uint16_t *)p.out)[orow * Dv + jrow] = (uint16_t)f32_to_bf16_bits(o);
            }
        }
        // persist this node's state
        const int64_t srow = (orow * Dv + jrow) * DK + rg * VEC;
        if constexpr (SDT == SV_F32) {
            float *dst = (float *)p.state_nodes + srow;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                *(f32x4 *)(dst + c * 32) = f32x4{S[4 * c], S[4 * c + 1], S[4 * c + 2], S[4 * c + 3]};
        } else {
            uint16_t *dst = (uint16_t *)p.state_nodes + srow;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const float *sc = &S[8 * c];
                *(u32x4 *)(dst + c * 64) = u32x4{pack_f16x2(sc[0], sc[1]), pack_f16x2(sc[2], sc[3]),
                                                 pack_f16x2(sc[4], sc[5]), pack_f16x2(sc[6], sc[7])};
            }
        }
        if constexpr (TREE) {
            if (__builtin_amdgcn_readlane(nch, x) >= 2) {
                const int sx = __builtin_amdgcn_readlane(slot, x);
                if (sx < NSLOT) {
#pragma unroll
                    for (int t = 0; t < R / 4; ++t)
                        my_slot[(sx * 4 * (R / 4) + t) * 64] = f32x4{S[4 * t], S[4 * t + 1], S[4 * t + 2], S[4 * t + 3]};
                }
            }
        }
        prev = x;
    }
}

// ---------------------------------------------------------------------------
// commit of the accepted node
// ---------------------------------------------------------------------------

// grid (state_blocks + conv blocks, B).  Workgroups below state_blocks copy 8
// state values per thread; the others move 4 conv channels per thread.
template <int SDT, int DT>
__global__ __launch_bounds__(256) void commit_kernel(CommitParams p) {
    __shared__ int ok_s;
    __shared__ int path_s[64];
    const int b = blockIdx.y, tid = threadIdx.x;
    const int N = p.N;
    if (tid < 64) {
        const int a = p.accept_len[b];
        const bool a_ok = a >= 0 && a <= N - 1;
        int pj = 0;
        bool good = true;
        if (a_ok && tid <= a) {
            pj = p.path[(int64_t)b * N + tid];
            good = pj >= tid && pj <= N - 1;
        }
        const uint64_t bad = __ballot(!good);
        if (tid < N) path_s[tid] = pj;
        if (tid == 0) ok_s = (a_ok && bad == 0ull) ? a : -1;
    }
    __syncthreads();
    const int a = ok_s;
    if (a < 0) return;
    if ((int)blockIdx.x < p.state_blocks) {
        const int64_t e = ((int64_t)blockIdx.x * 256 + tid) * 8;
        if (e >= p.state_elems) return;
        const int64_t src = ((int64_t)b * N + path_s[a]) * p.state_elems + e;
        float v[8];
        if constexpr (SDT == SV_F32) {
            const f32x4 x0 = *(const f32x4 *)((const float *)p.state_nodes + src);
            const f32x4 x1 = *(const f32x4 *)((const float *)p.state_nodes + src + 4);
#pragma unroll
            for (int t = 0; t < 4; ++t) { v[t] = x0[t]; v[4 + t] = x1[t]; }
        } else {
            const u32x4 h = *(const u32x4 *)((const uint16_t *)p.state_nodes + src);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v[2 * t] = fp16_bits_to_f32(h[t] & 0xFFFFu);
                v[2 * t + 1] = fp16_bits_to_f32(h[t] >> 16);
            }
        }
        float *dst = p.state + (int64_t)b * p.state_elems + e;
        *(f32x4 *)dst = f32x4{v[0], v[1], v[2], v[3]};
        *(f32x4 *)(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
        return;
    }
    const int c0 = ((blockIdx.x - p.state_blocks) * 256 + tid) * 4;
    if (c0 >= p.C) return;
    const int K1 = p.K - 1, C = p.C;
    // the last K-1 of (old conv state, x[path[0]], .., x[path[a]]): read all, then write
    constexpr int kMaxK1 = 7;
    f32x4 nv[kMaxK1];
    const int total = K1 + a + 1;
#pragma unroll
    for (int t = 0; t < kMaxK1; ++t) {
        if (t < K1) {
            const int s = total - K1 + t;
            nv[t] = s < K1 ? load4<DT>(p.conv_state, ((int64_t)b * K1 + s) * C + c0)
                           : load4<DT>(p.x, ((int64_t)b * N + path_s[s - K1]) * C + c0);
        }
    }
#pragma unroll
    for (int t = 0; t < kMaxK1; ++t) {
        if (t < K1) store4<DT>(p.conv_state, ((int64_t)b * K1 + t) * C + c0, nv[t]);
    }
}

template <int DT, int K>
hipError_t launch_conv_k(const ConvTreeParams &p, hipStream_t st) {
    const dim3 grid((unsigned)((p.C + 1023) / 1024), (unsigned)p.N, (unsigned)p.B);
    hipLaunchKernelGGL((conv_tree_kernel<DT, K>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int R, int NMAX, bool TREE, int DT>
hipError_t launch_delta_s(const DeltaParams &p, int sdt, hipStream_t st) {
    const dim3 grid((unsigned)(p.Dv / 32), (unsigned)p.Hv, (unsigned)p.B);
    if (sdt == SV_F16)
        hipLaunchKernelGGL((delta_tree_kernel<R, NMAX, TREE, DT, SV_F16>), grid, dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((delta_tree_kernel<R, NMAX, TREE, DT, SV_F32>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int R, int NMAX, bool TREE>
hipError_t launch_delta_d(const DeltaParams &p, int dt, int sdt, hipStream_t st) {
    return dt == SV_F32 ? launch_delta_s<R, NMAX, TREE, SV_F32>(p, sdt, st)
                        : launch_delta_s<R, NMAX, TREE, SV_BF16>(p, sdt, st);
}

template <int R>
hipError_t launch_delta_r(const DeltaParams &p, int dt, int sdt, hipStream_t st) {
    const bool tree = p.parent != nullptr;
    if (p.N <= 16) return tree ? launch_delta_d<R, 16, true>(p, dt, sdt, st) : launch_delta_d<R, 16, false>(p, dt, sdt, st);
    if (p.N <= 32) return tree ? launch_delta_d<R, 32, true>(p, dt, sdt, st) : launch_delta_d<R, 32, false>(p, dt, sdt, st);
    return tree ? launch_delta_d<R, 64, true>(p, dt, sdt, st) : launch_delta_d<R, 64, false>(p, dt, sdt, st);
}

}  // namespace

hipError_t launch_conv_tree(const ConvTreeParams &p, int dtype, hipStream_t st) {
    if (dtype == SV_F32) {
        return p.K == 2 ? launch_conv_k<SV_F32, 2>(p, st) : p.K == 3 ? launch_conv_k<SV_F32, 3>(p, st)
                                                                     : launch_conv_k<SV_F32, 4>(p, st);
    }
    return p.K == 2 ? launch_conv_k<SV_BF16, 2>(p, st) : p.K == 3 ? launch_conv_k<SV_BF16, 3>(p, st)
                                                                  : launch_conv_k<SV_BF16, 4>(p, st);
}

hipError_t launch_delta_tree(const DeltaParams &p, int dtype, int state_dtype, int Dk, hipStream_t st) {
    return Dk == 64 ? launch_delta_r<8>(p, dtype, state_dtype, st) : launch_delta_r<16>(p, dtype, state_dtype, st);
}

hipError_t launch_commit(const CommitParams &p, int state_dtype, int dtype, hipStream_t st) {
    const int conv_blocks = (p.C + 1023) / 1024;
    const dim3 grid((unsigned)(p.state_blocks + conv_blocks), (unsigned)p.B);
    if (state_dtype == SV_F16) {
        if (dtype == SV_F32) hipLaunchKernelGGL((commit_kernel<SV_F16, SV_F32>), grid, dim3(256), 0, st, p);
        else hipLaunchKernelGGL((commit_kernel<SV_F16, SV_BF16>), grid, dim3(256), 0, st, p);
    } else {
        if (dtype == SV_F32) hipLaunchKernelGGL((commit_kernel<SV_F32, SV_F32>), grid, dim3(256), 0, st, p);
        else hipLaunchKernelGGL((commit_kernel<SV_F32, SV_BF16>), grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace sv
