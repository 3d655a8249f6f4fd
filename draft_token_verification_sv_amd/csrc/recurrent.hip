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
// delta_tree_kernel: one workgroup of 8 waves (4 for trees of more than 32
// nodes) per (sequence, value head, block of 4 value rows per wave); lane
// (jr, rg) of a wave owns value row jr and R = Dk/16 of
// the key columns, in chunks of VEC contiguous columns spaced 16*VEC apart (so
// the 16 lanes of a row store the row's whole span of the per-node buffer), and
// the row sums are DPP reductions within a 16-lane row.  The state never leaves
// registers between a node and its first child.  Nodes are
// visited in depth-first order with the children of each node sorted by
// subtree size (largest last): a node with two or more children parks its
// state in an LDS slot that its later children restore; along any root path a
// slot is live only below a child that is not its parent's largest, so at most
// floor(log2(N+1)) - 1 slots are ever live.  The order is computed by one wave
// with one lane per node (ancestor sets by pointer doubling, subtree sizes,
// sibling ranks) into one word per step, no host work; a step reads the next
// node's operands and parked state from LDS while it computes.
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

// sum over the 16 lanes of a DPP row (result in all 16)
__device__ __forceinline__ float sum16(float v) {
    v += dpp_f<0xB1>(v);      // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);      // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);     // row_half_mirror
    v += dpp_f<0x140>(v);     // row_mirror
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

// two fp32 -> packed IEEE halves (lo in bits 0-15), round to nearest even
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
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

// wavefronts per workgroup (4 value rows each): 8, or 4 for trees of up to
// 64 nodes (whose q / k staging and parked states fill the LDS)
constexpr int delta_waves(int nmax) { return nmax <= 32 ? 8 : 4; }

template <int NMAX>
struct SlotCount {
    static constexpr int value = NMAX <= 16 ? 3 : (NMAX <= 32 ? 4 : 5);   // floor(log2(NMAX+1)) - 1
};

template <int DT>
struct Raw4 {
    using type = f32x4;                               // fp32: the 4 values
};
template <>
struct Raw4<SV_BF16> {
    using type = u32x2;                               // bf16: the 4 values' bits
};

template <int DT>
__device__ __forceinline__ typename Raw4<DT>::type load_raw4(const void *base, int64_t off) {
    if constexpr (DT == SV_F32) return *(const f32x4 *)((const float *)base + off);
    else return *(const u32x2 *)((const uint16_t *)base + off);
}

__device__ __forceinline__ f32x4 raw_f32(f32x4 r) { return r; }
__device__ __forceinline__ f32x4 raw_f32(u32x2 u) {
    return f32x4{bf16_bits_to_f32(u[0] & 0xFFFFu), bf16_bits_to_f32(u[0] >> 16),
                 bf16_bits_to_f32(u[1] & 0xFFFFu), bf16_bits_to_f32(u[1] >> 16)};
}

// The visiting order of one tree, one lane per node (par: this lane's valid
// parent or -1), by all `nw` wavefronts of the workgroup together (every
// thread calls it; the loops over nodes are split over the wavefronts):
// depth-first, each node's children by subtree size with the largest last.
// Wavefront 0 writes one word per preorder position into sched_s:
// node | restore << 8 | save << 16.  cnt_s: 64 ints, part_s: 64 * nw ints.
__device__ void tree_order(int par, int N, int *cnt_s, int *part_s, int *sched_s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const bool live = lane < N;
    int pos = lane, slot = 0, nch = lane < N - 1 ? 1 : 0, pre = 0;
    const bool is_chain = __ballot(live && par != lane - 1) == 0ull;   // the same in every wavefront
    if (!is_chain) {
        // ancestor-or-self sets by pointer doubling (depth < 64)
        uint64_t anc = live ? (1ull << lane) : 0ull;
        int jp = par;
#pragma unroll 1
        for (int r = 0; r < 6; ++r) {
            if (__ballot(jp >= 0) == 0ull) break;
            const int src = jp >= 0 ? jp : lane;
            const uint32_t alo = (uint32_t)__shfl((int)(uint32_t)anc, src, 64);
            const uint32_t ahi = (uint32_t)__shfl((int)(uint32_t)(anc >> 32), src, 64);
            const int jp2 = __shfl(jp, src, 64);
            if (jp >= 0) {
                anc |= ((uint64_t)ahi << 32) | alo;
                jp = jp2;
            }
        }
        // subtree sizes and child counts: column counts of the ancestor sets
#pragma unroll 1
        for (int i = wave; i < N; i += nw) {
            const int c1 = __popcll(__ballot(((anc >> i) & 1ull) != 0ull));
            const int c2 = __popcll(__ballot(par == i));
            if (lane == 0) cnt_s[i] = c1 | (c2 << 8);
        }
        __syncthreads();
        const int cw = cnt_s[min(lane, N - 1)];
        const int size = live ? (cw & 255) : 0;
        nch = live ? (cw >> 8) : 0;
        // siblings ordered by (subtree size, index), the largest last: the
        // sizes of the siblings before this node, and whether one comes after
        int prep = 0, later = 0;
#pragma unroll 1
        for (int j = wave; j < N; j += nw) {
            const int pj = __builtin_amdgcn_readlane(par, j);
            const int sj = __builtin_amdgcn_readlane(size, j);
            const bool sib = pj == par && j != lane;
            const bool before = sj < size || (sj == size && j < lane);
            prep += (sib && before) ? sj : 0;
            later |= (sib && !before) ? 1 : 0;
        }
        part_s[wave * 64 + lane] = prep | (later << 16);
        __syncthreads();
        int later_all = 0;
#pragma unroll
        for (int w2 = 0; w2 < nw; ++w2) {
            const int v = part_s[w2 * 64 + lane];
            pre += v & 0xFFFF;
            later_all |= v >> 16;
        }
        // preorder position = sum of (1 + pre) along the root path, slot =
        // number of non-largest children on it: path sums by pointer doubling
        int aw = live ? 1 + pre : 0, al = (par >= 0 && later_all) ? 1 : 0;
        jp = par;
#pragma unroll 1
        for (int r = 0; r < 6; ++r) {
            if (__ballot(jp >= 0) == 0ull) break;
            const int src = jp >= 0 ? jp : lane;
            const int aw2 = __shfl(aw, src, 64);
            const int al2 = __shfl(al, src, 64);
            const int jp2 = __shfl(jp, src, 64);
            if (jp >= 0) {
                aw += aw2;
                al += al2;
                jp = jp2;
            }
        }
        pos = live ? aw - 1 : -1;
        slot = al;
    }
    // one word per preorder position: node | restore << 8 | save << 16;
    // restore 0: the parent's state is in registers (a first child comes
    // right after its parent; the first top node starts from the committed
    // state already loaded), 1: the committed state, 2 + s: slot s;
    // save 1 + s: park the state in slot s
    if (wave == 0) {
        const int pslot = __shfl(slot, par >= 0 ? par : 0, 64);
        if (live) {
            const int rc = (pre == 0 && (par >= 0 || pos == 0)) ? 0 : (par < 0 ? 1 : 2 + pslot);
            const int sc = nch >= 2 ? 1 + slot : 0;
            sched_s[pos] = lane | (rc << 8) | (sc << 16);
        }
    }
}

template <int R, int NMAX, bool TREE, int DT, int SDT>
__global__ __launch_bounds__(64 * delta_waves(NMAX)) void delta_tree_kernel(DeltaParams p) {
    constexpr int DK = 16 * R;
    constexpr int VEC = (SDT == SV_F16 && R >= 8) ? 8 : 4;   // contiguous key columns per chunk
    constexpr int NCH = R / VEC;                             // chunks per lane
    constexpr int NSLOT = TREE ? SlotCount<NMAX>::value : 0;
    constexpr int WAVES = delta_waves(NMAX), NT = 64 * WAVES, RPB = 4 * WAVES;   // threads, value rows per workgroup
    constexpr int QK_IT = (NMAX * DK / 4 + NT - 1) / NT;
    constexpr int V_IT = (NMAX * RPB / 4 + NT - 1) / NT;
    static_assert(R % VEC == 0 && R % 4 == 0, "chunking");
    using Raw = typename Raw4<DT>::type;

    __shared__ __attribute__((aligned(16))) float k_s[NMAX * DK];
    __shared__ __attribute__((aligned(16))) float q_s[NMAX * DK];
    __shared__ __attribute__((aligned(16))) float v_s[NMAX * RPB];
    __shared__ float a_s[NMAX], b_s[NMAX];
    __shared__ int sched_s[TREE ? 64 : 1], cnt_s[TREE ? 64 : 1], part_s[TREE ? NT : 1];
    __shared__ float opart_s[NMAX * RPB * 4];           // [node][wave][row * 4 + quad]
    __shared__ __attribute__((aligned(16))) f32x4 slot_s[NSLOT > 0 ? NSLOT * WAVES * (R / 4) * 64 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int jb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int N = p.N, Hv = p.Hv, Dv = p.Dv;
    const int hk = h / (Hv / p.Hk);
    const int jr = lane >> 4, rg = lane & 15;
    const int jloc = wave * 4 + jr;                   // this lane's value row in the block
    const int jrow = jb * RPB + jloc;
    const int64_t bn = (int64_t)b * N;

    // ---- loads, in the order they are needed: the tree, the committed
    // state, then q, k (all nodes, this key head), v (16 rows), decay, beta
    // (indices clamped into range; converted once the order is known) ----
    int par = lane - 1, sched_g = lane;
    if constexpr (TREE) {
        par = -1;
        if (p.sched != nullptr) {
            sched_g = p.sched[(int64_t)b * 64 + min(lane, N - 1)];
        } else if (lane < N) {
            const int pr = p.parent[bn + lane];
            par = (pr >= 0 && pr < lane) ? pr : -1;
        }
    }
    float S[R];
    const float *s0 = p.state + (((int64_t)b * Hv + h) * Dv + jrow) * DK + rg * VEC;
    auto load_s0 = [&]() {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
#pragma unroll
            for (int u = 0; u < VEC / 4; ++u) {
                const f32x4 t = *(const f32x4 *)(s0 + c * 16 * VEC + 4 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e) S[c * VEC + 4 * u + e] = t[e];
            }
        }
    };
    load_s0();
    Raw qr[QK_IT], kr[QK_IT], vr[V_IT];
    const int nqk = N * (DK / 4);
#pragma unroll
    for (int it = 0; it < QK_IT; ++it) {
        const int e = min(tid + it * NT, nqk - 1);
        const int i = e / (DK / 4), c4 = e - i * (DK / 4);
        const int64_t off = (bn + i) * p.qk_stride + (int64_t)hk * DK + 4 * c4;
        qr[it] = load_raw4<DT>(p.q, off);
        kr[it] = load_raw4<DT>(p.k, off);
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
        const int e = min(tid + it * NT, N * (RPB / 4) - 1);
        const int i = e / (RPB / 4), c4 = e % (RPB / 4);
        vr[it] = load_raw4<DT>(p.v, (bn + i) * p.v_stride + (int64_t)h * Dv + jb * RPB + 4 * c4);
    }
    const int gi = min(tid, N - 1);
    const float gv = p.g[(bn + gi) * Hv + h];
    const float bv = p.beta[(bn + gi) * Hv + h];

    // ---- depth-first order: precomputed (one word per step), or computed
    // here by the 4 wavefronts ----
    if constexpr (TREE) {
        if (p.sched == nullptr) tree_order(par, N, cnt_s, part_s, sched_s);
    }

    // ---- operands into LDS ----
#pragma unroll
    for (int it = 0; it < QK_IT; ++it) {
        const int e = tid + it * NT;
        if (e < nqk) {
            *(f32x4 *)&q_s[4 * e] = raw_f32(qr[it]);      // node e / (DK/4), columns 4 (e % (DK/4)) ..
            *(f32x4 *)&k_s[4 * e] = raw_f32(kr[it]);
        }
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
        const int e = tid + it * NT;
        if (e < N * (RPB / 4)) *(f32x4 *)&v_s[4 * e] = raw_f32(vr[it]);
    }
    if (tid < N) {
        a_s[tid] = expf(gv);
        b_s[tid] = bv;
    }
    __syncthreads();
    int schedv = lane;                                 // word of preorder position `lane`
    if constexpr (TREE) schedv = p.sched != nullptr ? sched_g : sched_s[min(lane, N - 1)];

    // ---- the walk: the next node's operands (and parked parent state) are
    // read from LDS during the step before ----
    const float scale = p.scale;
    // node x's state row of this lane: st_base + x * node_elems + lane_off
    const int64_t st_base = (bn * Hv + h) * (int64_t)Dv * DK + (int64_t)jb * RPB * DK;
    const uint32_t node_elems = (uint32_t)Hv * (uint32_t)Dv * DK;
    const uint32_t lane_off = (uint32_t)jloc * DK + rg * VEC;
    f32x4 *my_slot = slot_s + wave * (R / 4) * 64 + lane;           // + (s * waves * (R/4) + t) * 64
    auto fetch = [&](int x, float (&kd)[R], float (&qd)[R], float &vd, float &ad, float &bd) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
#pragma unroll
            for (int u = 0; u < VEC / 4; ++u) {
                const int col = c * 16 * VEC + rg * VEC + 4 * u;
                const f32x4 k4 = *(const f32x4 *)&k_s[x * DK + col];
                const f32x4 q4 = *(const f32x4 *)&q_s[x * DK + col];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kd[c * VEC + 4 * u + e] = k4[e];
                    qd[c * VEC + 4 * u + e] = q4[e];
                }
            }
        }
        vd = v_s[x * RPB + jloc];
        ad = a_s[x];
        bd = b_s[x];
    };
    float Sr[R];                                        // a parked state read ahead
    auto step = [&](int ks, int word, const float (&kk)[R], const float (&qq)[R], float vx, float a, float bt,
                    float (&kn)[R], float (&qn)[R], float &vn, float &an, float &bn_) -> int {
        const int x = min(word & 63, N - 1);
        if constexpr (TREE) {
            const int rc = (word >> 8) & 255;
            if (rc == 1) {
                load_s0();                                  // another root: the committed state
            } else if (rc >= 2) {
#pragma unroll
                for (int t = 0; t < R; ++t) S[t] = Sr[t];
            }
        }
        const int wn = ks + 1 < N ? __builtin_amdgcn_readlane(schedv, ks + 1) : word;
        fetch(min(wn & 63, N - 1), kn, qn, vn, an, bn_);
        if constexpr (TREE) {
            const int rcn = (wn >> 8) & 255;
            // (a node followed by a restore is a leaf: it parks nothing)
            if (rcn >= 2 && rcn - 2 < NSLOT) {
#pragma unroll
                for (int t = 0; t < R / 4; ++t) {
                    const f32x4 v4 = my_slot[((rcn - 2) * WAVES * (R / 4) + t) * 64];
#pragma unroll
                    for (int e = 0; e < 4; ++e) Sr[4 * t + e] = v4[e];
                }
            }
        }
        // u = beta (v - a S k);  S <- a S + u k^T;  o = scale S q
        float d[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < R; ++t) d[t & 3] = fmaf(S[t], kk[t], d[t & 3]);
        const float dot = sum16((d[0] + d[1]) + (d[2] + d[3]));
        const float u = (vx - a * dot) * bt;
#pragma unroll
        for (int t = 0; t < R; ++t) S[t] = fmaf(S[t], a, u * kk[t]);
        float o4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < R; ++t) o4[t & 3] = fmaf(S[t], qq[t], o4[t & 3]);
        // quad sums of S q go to LDS; the 4 quads of a row are added after the walk
        float oq = (o4[0] + o4[1]) + (o4[2] + o4[3]);
        oq += dpp_f<0xB1>(oq);
        oq += dpp_f<0x4E>(oq);
        opart_s[(x * WAVES + wave) * 16 + (lane >> 2)] = oq;
        // persist this node's state (uniform node base + per-lane offset;
        // streaming stores: the buffer is read back at most once, by the commit)
        if constexpr (SDT == SV_F32) {
            float *dst = (float *)p.state_nodes + st_base + (uint32_t)x * node_elems;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                __builtin_nontemporal_store(f32x4{S[4 * c], S[4 * c + 1], S[4 * c + 2], S[4 * c + 3]},
                                            (f32x4 *)(dst + (lane_off + c * 64)));
        } else if constexpr (VEC == 8) {
            uint16_t *dst = (uint16_t *)p.state_nodes + st_base + (uint32_t)x * node_elems;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const float *sc = &S[8 * c];
                __builtin_nontemporal_store(u32x4{pack_f16x2(sc[0], sc[1]), pack_f16x2(sc[2], sc[3]),
                                                  pack_f16x2(sc[4], sc[5]), pack_f16x2(sc[6], sc[7])},
                                            (u32x4 *)(dst + (lane_off + c * 128)));
            }
        } else {
            uint16_t *dst = (uint16_t *)p.state_nodes + st_base + (uint32_t)x * node_elems;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const float *sc = &S[4 * c];
                __builtin_nontemporal_store(u32x2{pack_f16x2(sc[0], sc[1]), pack_f16x2(sc[2], sc[3])},
                                            (u32x2 *)(dst + (lane_off + c * 64)));
            }
        }
        if constexpr (TREE) {
            const int sc = word >> 16;
            if (sc >= 1 && sc - 1 < NSLOT) {
#pragma unroll
                for (int t = 0; t < R / 4; ++t)
                    my_slot[((sc - 1) * WAVES * (R / 4) + t) * 64] = f32x4{S[4 * t], S[4 * t + 1], S[4 * t + 2], S[4 * t + 3]};
            }
        }
        return wn;
    };
    float kA[R], qA[R], kB[R], qB[R];
    float vA = 0.f, aA = 0.f, bA = 0.f, vB = 0.f, aB = 0.f, bB = 0.f;
    int word = __builtin_amdgcn_readlane(schedv, 0);
    fetch(min(word & 63, N - 1), kA, qA, vA, aA, bA);
#pragma unroll 1
    for (int ks = 0; ks < N; ks += 2) {
        word = step(ks, word, kA, qA, vA, aA, bA, kB, qB, vB, aB, bB);
        if (ks + 1 >= N) break;
        word = step(ks + 1, word, kB, qB, vB, aB, bB, kA, qA, vA, aA, bA);
    }

    // ---- outputs: the 4 quad sums of each (node, row), coalesced rows of 16 ----
    __syncthreads();
    for (int e = tid; e < N * RPB; e += NT) {
        const int x = e / RPB, jl = e % RPB;
        const float *pq = &opart_s[(x * WAVES + (jl >> 2)) * 16 + (jl & 3) * 4];
        const float o = ((pq[0] + pq[1]) + (pq[2] + pq[3])) * scale;
        const int64_t oi = ((bn + x) * Hv + h) * Dv + jb * RPB + jl;
        if constexpr (DT == SV_F32) ((float *)p.out)[oi] = o;
        else ((uint16_t *)p.out)[oi] = (uint16_t)f32_to_bf16_bits(o);
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
        // the accepted node's state: 8 values per thread and round, 4 rounds in
        // flight, the sequence's workgroups striding over it
        const int64_t src0 = ((int64_t)b * N + path_s[a]) * p.state_elems;
        float *dst0 = p.state + (int64_t)b * p.state_elems;
        const int64_t stride = (int64_t)p.state_blocks * 256 * 8;
        for (int64_t e0 = ((int64_t)blockIdx.x * 256 + tid) * 8; e0 < p.state_elems; e0 += 4 * stride) {
            float v[4][8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t e = min(e0 + r * stride, p.state_elems - 8);
                if constexpr (SDT == SV_F32) {
                    const f32x4 x0 = *(const f32x4 *)((const float *)p.state_nodes + src0 + e);
                    const f32x4 x1 = *(const f32x4 *)((const float *)p.state_nodes + src0 + e + 4);
#pragma unroll
                    for (int t = 0; t < 4; ++t) { v[r][t] = x0[t]; v[r][4 + t] = x1[t]; }
                } else {
                    const u32x4 hv = *(const u32x4 *)((const uint16_t *)p.state_nodes + src0 + e);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        v[r][2 * t] = fp16_bits_to_f32(hv[t] & 0xFFFFu);
                        v[r][2 * t + 1] = fp16_bits_to_f32(hv[t] >> 16);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t e = e0 + r * stride;
                if (e < p.state_elems) {
                    *(f32x4 *)(dst0 + e) = f32x4{v[r][0], v[r][1], v[r][2], v[r][3]};
                    *(f32x4 *)(dst0 + e + 4) = f32x4{v[r][4], v[r][5], v[r][6], v[r][7]};
                }
            }
        }
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

// One workgroup of 4 wavefronts per sequence: the order words of its tree,
// for every recurrent layer of the verify step to share.
__global__ __launch_bounds__(256) void tree_schedule_kernel(const int32_t *parent, int N, int32_t *sched) {
    __shared__ int cnt_s[64], part_s[256], sched_s[64];
    const int b = blockIdx.x, lane = threadIdx.x & 63;
    int par = -1;
    if (lane < N) {
        const int pr = parent[(int64_t)b * N + lane];
        par = (pr >= 0 && pr < lane) ? pr : -1;
    }
    tree_order(par, N, cnt_s, part_s, sched_s);
    __syncthreads();
    if (threadIdx.x < 64) sched[(int64_t)b * 64 + lane] = lane < N ? sched_s[lane] : 0;
}

template <int DT, int K>
hipError_t launch_conv_k(const ConvTreeParams &p, hipStream_t st) {
    const dim3 grid((unsigned)((p.C + 1023) / 1024), (unsigned)p.N, (unsigned)p.B);
    hipLaunchKernelGGL((conv_tree_kernel<DT, K>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int R, int NMAX, bool TREE, int DT>
hipError_t launch_delta_s(const DeltaParams &p, int sdt, hipStream_t st) {
    constexpr int W = delta_waves(NMAX);
    const dim3 grid((unsigned)(p.Dv / (4 * W)), (unsigned)p.Hv, (unsigned)p.B);
    if (sdt == SV_F16)
        hipLaunchKernelGGL((delta_tree_kernel<R, NMAX, TREE, DT, SV_F16>), grid, dim3(64 * W), 0, st, p);
    else
        hipLaunchKernelGGL((delta_tree_kernel<R, NMAX, TREE, DT, SV_F32>), grid, dim3(64 * W), 0, st, p);
    return hipGetLastError();
}

template <int R, int NMAX, bool TREE>
hipError_t launch_delta_d(const DeltaParams &p, int dt, int sdt, hipStream_t st) {
    return dt == SV_F32 ? launch_delta_s<R, NMAX, TREE, SV_F32>(p, sdt, st)
                        : launch_delta_s<R, NMAX, TREE, SV_BF16>(p, sdt, st);
}

template <int R>
hipError_t launch_delta_r(const DeltaParams &p, int dt, int sdt, hipStream_t st) {
    const bool tree = p.parent != nullptr || p.sched != nullptr;
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

hipError_t launch_tree_schedule(const int32_t *parent, int B, int N, int32_t *sched, hipStream_t st) {
    hipLaunchKernelGGL(tree_schedule_kernel, dim3((unsigned)B), dim3(256), 0, st, parent, N, sched);
    return hipGetLastError();
}

hipError_t launch_delta_tree(const DeltaParams &p, int dtype, int state_dtype, int Dk, hipStream_t st) {
    return Dk == 64 ? launch_delta_r<4>(p, dtype, state_dtype, st) : launch_delta_r<8>(p, dtype, state_dtype, st);
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
