// Split-KV verify attention over a 4-bit KV cache of head dim 256 on gfx950:
// a cooperative four-wave schedule on fp16 matrix cores.
//
// The 4-bit cache [single-RTX-3090 DFlash note, "128K context in 24 GB": the
// KV cache kept in 4 bits so that 128K tokens of context fit] is read by the
// same direct-to-LDS stages as the bf16 pipeline: a stage is 128 positions of
// raw codes and fp16 scales (36 KB, 9 one-KB DMA instructions per wave).
//
// Work split.  One workgroup (4 waves) handles one (sequence, KV head, row
// block, key split); a row block is 2 * NTS tiles of 16 packed rows (r = node
// * G + g, the verify rows of every query head of the GQA group).  Per
// 32-position chunk:
//   S^T = K Q^T  wave w computes position tile w & 1 (16 positions) for row
//                tiles (w >> 1) * NTS .. + NTS - 1: every S tile is computed
//                once and the four waves carry equal matrix work;
//   O^T += V^T P^T  wave w owns head-dim slice [64 w, 64 w + 64) of every row
//                tile: again equal work, and every V element is read by one
//                wave.
// The probabilities cross waves through LDS (P is written by the wave that
// computed S and read by all four).  The online-softmax reference maximum of a
// row must be the same in every wave (each holds a slice of the row's O), so
// the waves publish their per-tile row maxima and all apply the same lazy
// rule: the reference moves only when a chunk's maximum exceeds it by more
// than 2^8 (numerator and denominator share it, so this is exact).
//
// Dequantisation.  value = d * (code - 8) with d the block's fp16 scale.  The
// 256 threads turn each staged chunk into fp16 rows in LDS with packed fp16
// arithmetic: the codes are placed in the mantissa of 1024.0 (code n at bits
// 0-3 gives 1024 + n, at bits 4-7 gives 1024 + 16 n), one packed add or fma
// makes n - 8 exactly, one packed multiply by d rounds d (n - 8) to nearest
// fp16.  The eight values of a 32-bit code word come out in the order
// (0, 4, 2, 6, 1, 5, 3, 7); the query fragments are permuted the same way
// (a permutation of the contraction index), and the output head-dim index is
// mapped back when the partials are stored.  The queries are converted to
// fp16 after scaling each row by a power of two that puts its largest
// magnitude in [2^14, 2^15) (exact for bf16 values in the normal range; the
// scale is folded back into the softmax exponent).
//
// Pipeline per chunk g (two barriers): after the first, every wave applies
// the published row maxima of S(g); then the matrix instructions of S(g + 1)
// run while the vector units take the exponentials of P(g) and dequantise
// V(g + 1); after the second, the matrix instructions of O += V^T P(g)^T run
// while the vector units take the row maxima of S(g + 1) and dequantise
// K(g + 2).  Each matrix instruction is followed by its share of the vector
// work, in that order (one wave per SIMD: the overlap comes from the
// instruction stream).  K and V staging and P are double-buffered by chunk
// parity; cross-lane row reductions use the permlane swaps.
//
// Tree mask [DFN "From autoregressive to DDTree"; for chains the causal mask
// aligned to the end of the keys, xdnf.cn notes section 5.3]: 64-bit ancestor
// sets in LDS, applied on chunks that reach the draft rows or the split end.
// Output: unnormalised partials (O, m, l) per row for the split merge.
#include "attn_q4_common.h"

namespace sv {
namespace {

constexpr int LPW = NKB / 4;                // DMA instructions per wave and stage
static_assert(NKB % 4 == 0, "stage split over four waves");


template <int NTS, bool PAGED>
__global__ __launch_bounds__(256, 1) void attn_q4c_kernel(AttnParams p) {
    constexpr int RB = 2 * NTS;                 // row tiles per block
    constexpr int ROWS = 16 * RB;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t kst[2 * FST];
    __shared__ __attribute__((aligned(1024))) uint8_t vst[2 * FST];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[2 * ROWS * PROW];
    __shared__ __attribute__((aligned(16))) float mxb[2 * ROWS * 2];
    __shared__ float lsx[ROWS];
    __shared__ int par_s[64];
    __shared__ uint64_t anc_s[64];
    __shared__ int pages_s[PAGED ? kMaxPages : 1];
    __shared__ SchedLds sched_s;

    // ---- unit: (b, kv head, row block, split); the row blocks of one unit get
    // ids 8 apart (same XCD, shared L2) ------------------------------------------
    const int id = blockIdx.x;
    const int xcd = id & 7, k8 = id >> 3;
    const int rb = k8 % p.n_rowblocks;
    AttnUnit wu;
    if (!attn_unit(p, (k8 / p.n_rowblocks) * 8 + xcd, rb == 0, sched_s, wu)) return;
    const int b = __builtin_amdgcn_readfirstlane(wu.b), kvh = __builtin_amdgcn_readfirstlane(wu.kvh);
    const int N = p.N, G = p.G, R = p.R;
    const int ctx = __builtin_amdgcn_readfirstlane(wu.ctx);
    const int p0 = __builtin_amdgcn_readfirstlane(wu.p0), p1 = __builtin_amdgcn_readfirstlane(wu.p1);
    const int n_st = (p1 - p0 + T - 1) / T;
    const int NCH = (p1 - p0 + 31) / 32;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pt = wave & 1, hh = wave >> 1;
    const int l16 = lane & 15, qd = lane >> 4;

    // ---- tree (splits that reach the draft rows) and page ids --------------
    const bool has_draft = p1 > ctx;
    if (has_draft && tid < N) par_s[tid] = parent_of(p.parent + (int64_t)b * N, tid, p.err);
    int first_page = 0;
    if constexpr (PAGED) {
        first_page = p0 / p.kv.page_size;
        const int last_page = (p1 - 1) / p.kv.page_size;
        for (int e = tid; e <= last_page - first_page; e += 256) {
            const int pgid = p.kv.page_table[(int64_t)b * p.kv.max_pages + first_page + e];
            const bool bad = pgid < 0 || pgid >= p.kv.capacity;
            SV_DEVCHECK(p.err, bad, SV_DEVERR_PAGE);
            pages_s[e] = bad ? -1 : pgid;
        }
    }
    __syncthreads();
    if (has_draft && tid < N) anc_s[tid] = ancestor_bits(par_s, tid);   // visible after the next barrier

    // ---- DMA issue ---------------------------------------------------------------
    // Instruction j of this wave covers 1 KB of the stage [K codes][V codes]
    // [K scales][V scales]: lane offset within the array's part of the stage,
    // the array (wave-uniform) and its log2 row bytes.
    const uint8_t *arr_base[4] = {(const uint8_t *)p.kv.k, (const uint8_t *)p.kv.v, (const uint8_t *)p.kv.ks,
                                  (const uint8_t *)p.kv.vs};
    uint32_t dma_off[LPW];
    const uint8_t *dma_gb[LPW];
    int dma_rsh[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int kbi = wave * LPW + j;
        const int arr = kbi < KCI ? 0 : (kbi < 2 * KCI ? 1 : (kbi < 2 * KCI + KSI ? 2 : 3));
        const int start = arr == 0 ? 0 : (arr == 1 ? KCI : (arr == 2 ? 2 * KCI : 2 * KCI + KSI));
        dma_off[j] = (uint32_t)((kbi - start) * 1024 + lane * 16);
        dma_gb[j] = arr_base[arr];
        dma_rsh[j] = arr < 2 ? 7 : 4;                  // 128 code bytes / 16 scale bytes per row
    }
    const int64_t head_row0 = ((int64_t)b * p.Hkv + kvh) * p.kv.capacity;
    const uint32_t ring_u32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)ring;

    // Stage st = positions p0 + 128 st .. + 127; rows past the split's end
    // repeat its last row (their scores are masked).  Paged rows whose page is
    // outside the pool fetch row 0 of the array (no out-of-range access) and
    // are replaced by zero rows when dequantised.
    auto issue = [&](int st) {
        const int tb = p0 + st * T;
        const uint32_t slot = ring_u32 + (uint32_t)((st & 1) * STAGE + wave * LPW * 1024);
        if constexpr (!PAGED) {
            if (tb + T <= p1) {
#pragma unroll
                for (int j = 0; j < LPW; ++j)
                    dma16s(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)),
                           dma_gb[j] + ((head_row0 + tb) << dma_rsh[j]), dma_off[j]);
            } else {
                const int lim = p1 - 1 - tb;
#pragma unroll
                for (int j = 0; j < LPW; ++j) {
                    const int rsh = dma_rsh[j];
                    const int row = (int)(dma_off[j] >> rsh);
                    const uint32_t col = dma_off[j] & ((1u << rsh) - 1u);
                    dma16s(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)),
                           dma_gb[j] + ((head_row0 + tb) << rsh), ((uint32_t)min(row, lim) << rsh) | col);
                }
            }
        } else {
            // all page-id reads first: each DMA statement orders memory, so a
            // read placed between two of them would be waited for alone
            const int ps = p.kv.page_size;
            const uint8_t *src[LPW];
#pragma unroll
            for (int j = 0; j < LPW; ++j) {
                const int rsh = dma_rsh[j];
                const int row = (int)(dma_off[j] >> rsh);
                const uint32_t col = dma_off[j] & ((1u << rsh) - 1u);
                const int pos = min(tb + row, p1 - 1);
                const int pq = pos / ps, pr = pos - pq * ps;
                const int pg = pages_s[pq - first_page];
                const int64_t ri = pg < 0 ? 0 : ((int64_t)pg * p.Hkv + kvh) * ps + pr;
                src[j] = dma_gb[j] + (ri << rsh) + col;
            }
#pragma unroll
            for (int j = 0; j < LPW; ++j) dma16(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)), src[j]);
        }
    };

    // DMA instruction j of this wave for full stage st of a contiguous cache
    // (the last stage and paged caches: the whole stage at once through issue)
    auto issue_one = [&](int st, int j) {
        const int tb = p0 + st * T;
        if constexpr (!PAGED) {
            if (tb + T <= p1) {
                const uint32_t slot = ring_u32 + (uint32_t)((st & 1) * STAGE + wave * LPW * 1024);
                dma16s(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)),
                       dma_gb[j] + ((head_row0 + tb) << dma_rsh[j]), dma_off[j]);
                return;
            }
        }
        if (j == 0) issue(st);
    };

    // ---- prologue: stage 0, the queries, stage 1 --------------------------------
    issue(0);

    const int row0 = rb * p.rows_per_block;
    const int rows_here = min(p.rows_per_block, R - row0);
    // S rows of this lane: tile hh * NTS + i, row l16
    h8 qf[NTS][8];
    float sl2[NTS];
    int node_of[NTS];
#pragma unroll
    for (int i = 0; i < NTS; ++i) {
        const int rl = 16 * (hh * NTS + i) + l16;
        const bool ok = rl < rows_here;
        const int r = row0 + rl;
        node_of[i] = ok ? r / G : -1;
        bf16x8 raw[8];
        if (ok) {
            const int n = r / G, g = r % G;
            const __bf16 *qp = (const __bf16 *)p.q + (((int64_t)b * N + n) * p.Hq + (int64_t)kvh * G + g) * D + qd * 8;
#pragma unroll
            for (int k = 0; k < 8; ++k) raw[k] = *(const bf16x8 *)(qp + 32 * k);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const bf16x8 z = {};
                raw[k] = z;
            }
        }
        // row maximum magnitude (the row's 256 values sit in the 4 lanes l16 + 16 qd)
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)raw[k][j]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        // 2^kq * amax in [2^14, 2^15): frexp gives amax = m 2^e, m in [0.5, 1)
        int kq = 0;
        if (amax > 0.f) {
            kq = 15 - __builtin_amdgcn_frexp_expf(amax);
            kq = kq > 100 ? 100 : (kq < -110 ? -110 : kq);
        }
        sl2[i] = ldexpf(p.scale_log2, -kq);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            // slot j holds value pi(j), pi = (0, 4, 2, 6, 1, 5, 3, 7)
            const int pi[8] = {0, 4, 2, 6, 1, 5, 3, 7};
            h8 v;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (_Float16)ldexpf((float)raw[k][pi[j]], kq);
            qf[i][k] = v;
        }
    }
    if (n_st > 1) issue(1);

    // O^T tile (row tile t, head-dim tile dt of this wave) = OTile<4 t + dt>
    static_for<0, 4 * RB>([&](auto ic) { OTile<decltype(ic)::value>::zero(); });
    float m_ref[RB], l_s[NTS], l_p[NTS];
#pragma unroll
    for (int t = 0; t < RB; ++t) m_ref[t] = -INFINITY;
#pragma unroll
    for (int i = 0; i < NTS; ++i) l_s[i] = 0.f;

    // ---- LDS layout of a staged fp16 chunk of K or V: the 16-byte unit of
    // logical head-dim chunk c (8 values) and position p sits at
    // c * 512 + (p ^ 4 (c & 1)) * 16.  With it the dequantisation writes, the K
    // fragment reads and the transposed V reads are free of bank conflicts.
    // K fragment, position tile pt, k-step k: chunk 4 k + qd, position 16 pt + l16
    const int k_lane = qd * 512 + ((16 * pt + l16) ^ (4 * (qd & 1))) * 16;          // + 2048 k
    // V^T fragment of 16-wide head-dim tile dg, half h: lane reads the 4-value
    // run r = l16 & 3 of position 8 qd + l16 / 4 + 4 h in chunk 2 dg + r / 2
    const int vsel = (l16 & 3) >> 1;
    const int va = 8 * qd + (l16 >> 2);
    const int v_lane0 = vsel * 512 + (va + 4 * vsel) * 16 + (l16 & 1) * 8;         // + 1024 dg
    const int v_lane1 = vsel * 512 + (va + 4 - 4 * vsel) * 16 + (l16 & 1) * 8;
    // P rows of this lane (PV operand): 8 positions 8 qd .. 8 qd + 7 of row 16 t + l16
    const int p_lane = l16 * PROW + 16 * qd;

    // Dequantisation: thread (row, 32-value block) of a chunk, laid out so that
    // the 8 threads of each LDS access group take 8 different rows (mod 8) and
    // 8 different blocks: their code reads and their fp16 writes both spread
    // over all banks.
    const int di = tid & 7, dj = tid >> 3;
    const int drow = 8 * (dj & 3) + di, dblk = (di + (dj >> 2)) & 7;
    const int dsrc = drow * CROW + dblk * 16, dssrc = drow * SROW + dblk * 2;
    const int ddst0 = (4 * dblk) * 512 + drow * 16;             // words m = 0, 2: + 1024 (m / 2)
    const int ddst1 = (4 * dblk + 1) * 512 + (drow ^ 4) * 16;   // words m = 1, 3
    const uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = 0x64006400u;
    struct Codes {
        u32x4 w;
        h2 s;
    };
    // codes and scale of chunk g of K (which = 0) or V (1) from the ring
    auto dq_load = [&](int which, int g) {
        const uint8_t *stg = ring + ((g / CPS) & 1) * STAGE + (g % CPS) * 32 * CROW;
        Codes c;
        c.w = *(const u32x4 *)(stg + which * T * CROW + dsrc);
        const uint32_t sb = *(const uint16_t *)(ring + ((g / CPS) & 1) * STAGE + 2 * T * CROW + which * T * SROW +
                                                (g % CPS) * 32 * SROW + dssrc);
        c.s = __builtin_bit_cast(h2, sb * 0x10001u);
        if constexpr (PAGED) {
            // a page outside the pool reads as a zero row
            const int pos = min(p0 + 32 * g + drow, p1 - 1);
            if (pages_s[pos / p.kv.page_size - first_page] < 0) c.s = h2{(_Float16)0.f, (_Float16)0.f};
        }
        return c;
    };
    auto dq_word = [&](int which, int g, const Codes &c, int m) {
        uint8_t *dst = (which ? vst : kst) + (g & 1) * FST + ((m & 1) ? ddst1 : ddst0) + (m >> 1) * 1024;
        *(u32x4 *)dst = dequant_word(c.w[m], c.s, m_lo, m_hi, magic);
    };
    auto kread = [&](int g, int k) { return *(const h8 *)(kst + (g & 1) * FST + k_lane + 2048 * k); };

    // row maxima of one S tile (log2 units) into the exchange buffer; the 4
    // lanes of a row all hold the row's value after the swaps and all store it
    auto xmax = [](float x, bool by32) {
        const auto r = by32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                            : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    // exchange buffer layout [row l16][row tile][position tile]: a lane's 2 RB
    // values are contiguous
    auto row_max = [&](const f32x4 &sc, int i, float *mxw) {
        float c = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        c = xmax(xmax(c, false), true);
        mxw[(l16 * RB + hh * NTS + i) * 2 + pt] = c * sl2[i];
    };
    // tree / split-end mask of chunk g on an S tile set (lane: positions pos0 .. pos0 + 3)
    auto apply_mask = [&](int g, f32x4 (&sc)[NTS]) {
        const int cb = p0 + 32 * g;
        if (cb + 32 > ctx || cb + 32 > p1) {
            const int pos0 = cb + 16 * pt + 4 * qd;
#pragma unroll
            for (int i = 0; i < NTS; ++i) {
                const uint64_t anc_r = anc_s[node_of[i] > 0 ? node_of[i] : 0];     // in bounds for every lane
                const uint64_t anc = node_of[i] >= 0 ? anc_r : 0ull;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int pos = pos0 + j;
                    bool vis = pos < p1;
                    // bitwise, not short-circuit: no branch per lane
                    vis &= (pos < ctx) | (((anc >> ((pos - ctx) & 63)) & 1ull) != 0ull);
                    sc[i][j] = vis ? sc[i][j] : -INFINITY;
                }
            }
        }
    };

    // ---- prologue: stage 0 landed (stage 1 may be in flight) -----------------
    if (n_st > 1) wait_vm<LPW>();
    else wait_vm<0>();
    __syncthreads();
    {
        const Codes k0 = dq_load(0, 0), v0 = dq_load(1, 0), k1 = dq_load(0, min(1, NCH - 1));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            dq_word(0, 0, k0, m);
            dq_word(1, 0, v0, m);
            dq_word(0, 1, k1, m);
        }
    }
    __syncthreads();

    f32x4 sacc[NTS];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const h8 kf = kread(0, k);
#pragma unroll
        for (int i = 0; i < NTS; ++i) {
            if (k == 0) sacc[i] = mfma_s_first(kf, qf[i][k]);
            else mfma_s_acc(sacc[i], kf, qf[i][k]);
        }
    }
    mfma_drain_s(sacc);
    apply_mask(0, sacc);
#pragma unroll
    for (int i = 0; i < NTS; ++i) row_max(sacc[i], i, mxb);

    auto vread = [&](int g, int dt) {
        const uint8_t *vp = vst + (g & 1) * FST;
        const int dg = 4 * wave + dt;                    // 16-wide head-dim tile
        const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(__attribute__((address_space(3))) uint8_t *)(
                vp + v_lane0 + 1024 * dg));
        const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(__attribute__((address_space(3))) uint8_t *)(
                vp + v_lane1 + 1024 * dg));
        const short __attribute__((ext_vector_type(8))) w8 = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        return __builtin_bit_cast(h8, w8);
    };

    // References from chunk 0's exact row maxima (every wave reads the same
    // published values), so that typical splits never move one afterwards.
    __syncthreads();
    {
        const float *mxr = mxb + l16 * RB * 2;
#pragma unroll
        for (int t = 0; t < RB; ++t) m_ref[t] = fmaxf(mxr[2 * t], mxr[2 * t + 1]);
    }

    // Vector and matrix instructions of a SIMD do not overlap on this hardware
    // (measured: a matrix instruction plus n vector instructions cost the sum
    // of both), so each phase is ordered for latency: its LDS reads go out
    // first, the vector work that needs only registers follows, and the
    // matrix instructions (whose operands have landed by then) come last,
    // with the vector work that needs late operands slotted between them.
    // Chunks past the last one are still dequantised and multiplied (into
    // buffers nobody reads afterwards; the ring reads stay in bounds), so the
    // streams have no branches.
    //
    // chunk(SLOW, g, first): one chunk.  The fast form (SLOW false) returns
    // true, before any matrix work, when a row maximum would move its
    // reference; the caller then finishes the split with the slow form, which
    // rescales in place.  Keeping the rescale out of the fast loop leaves its
    // matrix accumulators written by matrix instructions only, so they stay
    // in the accumulation registers without copies.  `first` skips barrier 1
    // (already passed by the chunk the fast loop left).
    auto chunk = [&](auto slow_c, int g, bool first) -> bool {
        constexpr bool SLOW = decltype(slow_c)::value;
        // ---- barrier 1: maxima of S(g) published, K(g + 1) staged; the ring
        // slot of stage s + 1 is free once every wave has dequantised chunk
        // 4 s + 3 (its loads go out between the matrix instructions below)
        if (!first) __syncthreads();
        const int st_issue = ((g + 1) & (CPS - 1)) == 0 ? (g + 1) / CPS + 1 : n_st;

        // ---- (c) loads: row maxima of S(g), K fragments of S(g + 1), codes of
        // V(g + 1) ----------------------------------------------------------------
        const float *mxr = mxb + (g & 1) * ROWS * 2 + l16 * RB * 2;
        float mxv[2 * RB];
#pragma unroll
        for (int t = 0; t < 2 * RB; ++t) mxv[t] = mxr[t];
        // K fragments of S(g + 1): a ring of KR, the first KR read now
        constexpr int KR = 3;
        const int gs = g + 1 < NCH ? g + 1 : g;
        h8 kf[KR];
#pragma unroll
        for (int k = 0; k < KR; ++k) kf[k] = kread(gs, k);
        const Codes cv = dq_load(1, g + 1);

        if constexpr (SLOW) {
            // ---- (b) the lazy rule, in place: a reference moves when the
            // chunk's maximum exceeds it by more than 2^8
            float alpha[RB];
            bool grow = false;
#pragma unroll
            for (int t = 0; t < RB; ++t) {
                const float cm = fmaxf(mxv[2 * t], mxv[2 * t + 1]);
                const bool need = cm > m_ref[t] + 8.f;
                alpha[t] = need ? __builtin_amdgcn_exp2f(m_ref[t] - cm) : 1.f;
                m_ref[t] = need ? cm : m_ref[t];
                grow |= need;
            }
            if (__any(grow)) {
                mfma_drain();
                static_for<0, 4 * RB>([&](auto ic) {
                    constexpr int I = decltype(ic)::value;
                    OTile<I>::scale(alpha[I / 4]);
                });
                asm volatile("s_nop 3");
#pragma unroll
                for (int i = 0; i < NTS; ++i) l_s[i] *= hh ? alpha[NTS + i] : alpha[i];
            }
        }

        // P(g) (the fast form checks the references after writing it)
        uint8_t *pw = pbuf + (g & 1) * ROWS * PROW;
#pragma unroll
        for (int t = 0; t < NTS; ++t) {
            const float mr = hh ? m_ref[NTS + t] : m_ref[t];
            const float mu = mr == -INFINITY ? 0.f : mr;
            float pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pr[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][j], sl2[t], -mu));
            l_p[t] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
            typedef float f32x2_t __attribute__((ext_vector_type(2)));
            u32x2 pk;
            pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){pr[0], pr[1]}, h2));
            pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){pr[2], pr[3]}, h2));
            *(u32x2 *)(pw + (16 * (hh * NTS + t) + l16) * PROW + (16 * pt + 4 * qd) * 2) = pk;
        }
        dq_word(1, g + 1, cv, 0);
        dq_word(1, g + 1, cv, 1);
        if constexpr (!SLOW) {
            bool grow = false;
#pragma unroll
            for (int t = 0; t < RB; ++t) grow |= fmaxf(mxv[2 * t], mxv[2 * t + 1]) > m_ref[t] + 8.f;
            if (__builtin_expect(__any(grow), 0)) return true;
        }

#pragma unroll
        for (int t = 0; t < NTS; ++t) l_s[t] += l_p[t];

        // ---- S(g + 1) on the matrix cores; V(g + 1) words 2, 3 and the loads of
        // a freed ring slot between them ------------------------------------------
        f32x4 sacc_n[NTS];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const h8 ka = kf[k % KR];
            if (k + KR < 8) kf[k % KR] = kread(gs, k + KR);
#pragma unroll
            for (int i = 0; i < NTS; ++i) {
                if (k == 0) sacc_n[i] = mfma_s_first(ka, qf[i][k]);
                else mfma_s_acc(sacc_n[i], ka, qf[i][k]);
            }
            if (k == 2) dq_word(1, g + 1, cv, 2);
            if (k == 5) dq_word(1, g + 1, cv, 3);
            if (k < LPW && st_issue < n_st) issue_one(st_issue, k);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (LPW > 8 && st_issue < n_st)
#pragma unroll
            for (int j = 8; j < LPW; ++j) issue_one(st_issue, j);
        mfma_drain_s(sacc_n);                               // S(g + 1) complete before vector reads

        // stage (g + 2) / 4 is needed from here on: this wave's part landed
        if (((g + 2) & (CPS - 1)) == 0 && g + 2 < NCH) wait_vm<0>();

        // ---- barrier 2: P(g) published; V(g + 1) staged; K(g + 2)'s stage landed
        __syncthreads();

        // ---- (e) loads: V^T fragments, codes of K(g + 2), P(g) fragments; then
        // the row maxima of S(g + 1), K(g + 2), and O^T += V^T P(g)^T -------------
        {
            h8 vf[4];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) vf[dt] = vread(g, dt);
            const int gk = g + 2 < NCH ? g + 2 : g;
            const Codes ck = dq_load(0, gk);
            const uint8_t *prd = pbuf + (g & 1) * ROWS * PROW + p_lane;
            // P fragments: a ring of 2
            h8 pf[2];
            pf[0] = *(const h8 *)prd;
            pf[1] = *(const h8 *)(prd + 16 * PROW);
            apply_mask(g + 1, sacc_n);
            float *mxw = mxb + ((g + 1) & 1) * ROWS * 2;
#pragma unroll
            for (int i = 0; i < NTS; ++i) row_max(sacc_n[i], i, mxw);
            dq_word(0, gk, ck, 0);
            dq_word(0, gk, ck, 1);
            static_for<0, RB>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                const h8 pa = pf[t & 1];
                if constexpr (t + 2 < RB) pf[t & 1] = *(const h8 *)(prd + 16 * (t + 2) * PROW);
                static_for<0, 4>([&](auto dc) {
                    constexpr int dt = decltype(dc)::value;
                    OTile<4 * t + dt>::mac(vf[dt], pa);
                });
                // K words 2 and 3 between the matrix instructions (both after the
                // first tile when there are only two)
                if constexpr (t == (RB >= 4 ? 1 : 0)) dq_word(0, gk, ck, 2);
                if constexpr (t == (RB >= 4 ? 3 : 1)) dq_word(0, gk, ck, 3);
                __builtin_amdgcn_sched_barrier(0);
            });
        }
#pragma unroll
        for (int i = 0; i < NTS; ++i) sacc[i] = sacc_n[i];
        return false;
    };

    using FastTag = std::integral_constant<bool, false>;
    using SlowTag = std::integral_constant<bool, true>;
    int g = 0;
#pragma unroll 1
    for (; g < NCH; ++g)
        if (chunk(FastTag{}, g, g == 0)) break;
    if (g < NCH) {
        chunk(SlowTag{}, g, true);
#pragma unroll 1
        for (++g; g < NCH; ++g) chunk(SlowTag{}, g, false);
    }

    mfma_drain();
    // ---- row sums: lanes of a row, then the two position-tile waves -----------
#pragma unroll
    for (int i = 0; i < NTS; ++i) {
        l_s[i] += __shfl_xor(l_s[i], 16, 64);
        l_s[i] += __shfl_xor(l_s[i], 32, 64);
        if (pt == 1 && qd == 0) lsx[16 * (hh * NTS + i) + l16] = l_s[i];
    }
    __syncthreads();

    // ---- partials of this split --------------------------------------------------
    const int64_t part = wu.part;
    static_for<0, RB>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        const int rl = 16 * t + l16;
        float *op = p.part_o + (part * R + row0 + rl) * D;
        static_for<0, 4>([&](auto dc) {
            constexpr int dt = decltype(dc)::value;
            const f32x4 o = OTile<4 * t + dt>::read();
            if (rl >= rows_here) return;
            // the four values of slots s0 .. s0 + 3 in one 16-byte store, the row
            // left in slot order (slot s holds head dim 8 (s / 8) + pi(s % 8),
            // pi = 0, 4, 2, 6, 1, 5, 3, 7; the merge restores the order): four
            // scattered 4-byte stores per value group kept every workgroup's
            // last ~5 us on issuing them
            const int s0 = 64 * wave + 16 * dt + 4 * qd;
            *(f32x4 *)(op + s0) = o;
        });
    });
    if (pt == 0 && qd == 0) {
#pragma unroll
        for (int i = 0; i < NTS; ++i) {
            const int rl = 16 * (hh * NTS + i) + l16;
            if (rl >= rows_here) continue;
            const float mr = hh ? m_ref[NTS + i] : m_ref[i];
            p.part_ml[(part * R + row0 + rl) * 2 + 0] = mr;
            p.part_ml[(part * R + row0 + rl) * 2 + 1] = l_s[i] + lsx[rl];
        }
    }
}

template <int NTS, bool PAGED>
hipError_t launch_t(const AttnParams &p, hipStream_t st) {
    const int grid = ((p.n_units + 7) / 8) * 8 * p.n_rowblocks;
    hipLaunchKernelGGL((attn_q4c_kernel<NTS, PAGED>), dim3(grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_p(const AttnParams &p, int nts, hipStream_t st) {
    if (nts == 1) return launch_t<1, PAGED>(p, st);
    if (nts == 2) return launch_t<2, PAGED>(p, st);
    if (nts == 3) return launch_t<3, PAGED>(p, st);
    return hipErrorInvalidValue;
}

}  // namespace

int attn_q4c_max_split_pages() { return kMaxPages; }

hipError_t launch_attn_q4c(const AttnParams &p, int nts, hipStream_t st) {
    return p.kv.page_table != nullptr ? launch_p<true>(p, nts, st) : launch_p<false>(p, nts, st);
}

}  // namespace sv
