// Split-KV verify attention over a 4-bit KV cache of head dim 256 on gfx950:
// eight waves per workgroup, two per SIMD.
//
// Same cache, stages, dequantisation, tree mask and partial outputs as the
// four-wave cooperative kernel [single-RTX-3090 DFlash note, "128K context in
// 24 GB": the 4-bit cache; DFN "From autoregressive to DDTree": the tree
// mask].  The difference is the occupancy.  A SIMD issues one instruction of
// a wave per turn; with one wave per SIMD every scalar instruction, hazard
// pad, barrier wait and exposed LDS latency of that wave is a turn in which
// the SIMD does nothing, and measured on gfx950 those cost about as much as
// the matrix and vector instructions themselves.  With two waves per SIMD the
// other wave issues in those turns.  Matrix and vector instructions of one
// SIMD still take turns, so the aim is a SIMD that is always busy with one or
// the other.
//
// Work split (wave w, 0..7; waves w and w + 4 share SIMD w & 3).  Per
// 32-position chunk:
//   S^T = K Q^T  wave w computes position tile w & 1, row tiles
//                ((w >> 1) & 1) * NTS .. + NTS - 1, over the head-dim half
//                w >> 2 (k-steps 4 (w >> 2) .. + 3).  The two halves of a
//                tile meet in LDS: each wave writes the two values of each
//                of its lanes' four that its partner finishes and reads the
//                partner's share of its own two, so that both waves of the
//                pair take half of the softmax (the second half reads each
//                group of four K rows in the order 2, 3, 0, 1, so that in both
//                waves a lane's values 0, 1 are its own).
//   O^T += V^T P^T  wave w owns head-dim slice [32 w, 32 w + 32) of every row
//                tile.
// The queries and O each take 48 registers at 96 rows (half of the
// four-wave kernel's), which is what lets two waves share a SIMD's register
// file.
//
// Buffers.  K and V are dequantised into one fp16 buffer each: K(g + 2) is
// written in the second phase of chunk g, after every wave has read K(g + 1)
// in the first; V(g) is written in the first phase of chunk g and read in the
// second.  P, the row maxima and the score halves are single buffers for the
// same reason (written before a barrier, read after it, rewritten only after
// the next).  A stage's ring slot is refilled from the first chunk of the
// stage after it, once the last codes read from it (V of its last chunk) are
// behind a barrier.
//
// Online softmax: the references follow the four-wave kernel's lazy rule
// (a reference moves only when a chunk's row maximum exceeds it by more than
// 2^8).  A wave that finds one of its rows past that bound raises a flag in
// LDS; the fast loop reads only the flag, the slow loop (which rescales O in
// place) the published maxima.
#include "attn_q4_common.h"

namespace sv {
namespace {

// Scale rows of pages outside the pool are copied from here: a zero scale
// makes every value of the row zero, with no check in the dequantisation.
__device__ __attribute__((aligned(16))) uint8_t zero_scales[SROW] = {};

constexpr int NW = 8;                       // waves per workgroup
// DMA instructions of a stage per wave: the first four waves 5, the others 4
constexpr int WL = 5;
static_assert(NKB == 4 * 5 + 4 * 4, "stage split over eight waves");

// Query fragments in the accumulation registers a48..a95 (fragment J = 4 i + k
// of row tile i, k-step k in a[48 + 4 J .. + 3]), next to the O tiles in
// a0..a47: at two waves per SIMD the compiler's own values get 128
// architectural registers, and with the queries out of them they fit.  The
// matrix instructions read them as their B operand; only the inline assembly
// here and in OTile names these registers (the compiler places nothing of its
// own in a0..a95: checked on the compiled code).
template <int J> struct QTile;
#define SV_QTILE(J, R0, R1, R2, R3)                                                                       \
    template <> struct QTile<J> {                                                                         \
        static __device__ __forceinline__ void load(h8 q) {                                               \
            const u32x4 w = __builtin_bit_cast(u32x4, q);                                                 \
            asm volatile("v_accvgpr_write_b32 a" #R0 ", %0\n\tv_accvgpr_write_b32 a" #R1                  \
                         ", %1\n\tv_accvgpr_write_b32 a" #R2 ", %2\n\tv_accvgpr_write_b32 a" #R3 ", %3"   \
                         ::"v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3])                                     \
                         : "a" #R0, "a" #R1, "a" #R2, "a" #R3);                                            \
        }                                                                                                 \
        static __device__ __forceinline__ f32x4 first(h8 k) {                                             \
            f32x4 d;                                                                                      \
            asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, a[" #R0 ":" #R3 "], 0"                \
                         : "=&v"(d)                                                                       \
                         : "v"(k));                                                                       \
            return d;                                                                                     \
        }                                                                                                 \
        static __device__ __forceinline__ void acc(f32x4 &c, h8 k) {                                      \
            asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, a[" #R0 ":" #R3 "], %0"               \
                         : "+v"(c)                                                                        \
                         : "v"(k));                                                                       \
        }                                                                                                 \
    };
SV_QTILE(0, 48, 49, 50, 51)
SV_QTILE(1, 52, 53, 54, 55)
SV_QTILE(2, 56, 57, 58, 59)
SV_QTILE(3, 60, 61, 62, 63)
SV_QTILE(4, 64, 65, 66, 67)
SV_QTILE(5, 68, 69, 70, 71)
SV_QTILE(6, 72, 73, 74, 75)
SV_QTILE(7, 76, 77, 78, 79)
SV_QTILE(8, 80, 81, 82, 83)
SV_QTILE(9, 84, 85, 86, 87)
SV_QTILE(10, 88, 89, 90, 91)
SV_QTILE(11, 92, 93, 94, 95)
#undef SV_QTILE

template <int NTS, bool PAGED>
__global__ __launch_bounds__(64 * NW, 1) void attn_q4w_kernel(AttnParams p) {
    constexpr int RB = 2 * NTS;                 // row tiles per block
    constexpr int ROWS = 16 * RB;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t kst[FST];
    __shared__ __attribute__((aligned(1024))) uint8_t vst[FST];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[ROWS * PROW];
    __shared__ __attribute__((aligned(16))) float mxb[ROWS * 4];
    __shared__ __attribute__((aligned(16))) float sxb[4 * 2 * NTS * 64 * 2];
    __shared__ float lsx[4 * ROWS];
    __shared__ int gflag[2];                    // a row maximum moved past its reference (by chunk parity)
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
    const int pt = wave & 1, hh = (wave >> 1) & 1, dh = wave >> 2;
    const int l16 = lane & 15, qd = lane >> 4;

    // ---- tree (splits that reach the draft rows) and page ids --------------
    const bool has_draft = p1 > ctx;
    if (has_draft && tid < N) par_s[tid] = parent_of(p.parent + (int64_t)b * N, tid, p.err);
    int first_page = 0;
    if constexpr (PAGED) {
        first_page = p0 / p.kv.page_size;
        const int last_page = (p1 - 1) / p.kv.page_size;
        for (int e = tid; e <= last_page - first_page; e += 64 * NW) {
            const int pgid = p.kv.page_table[(int64_t)b * p.kv.max_pages + first_page + e];
            const bool bad = pgid < 0 || pgid >= p.kv.capacity;
            SV_DEVCHECK(p.err, bad, SV_DEVERR_PAGE);
            pages_s[e] = bad ? -1 : pgid;
        }
    }
    __syncthreads();
    if (has_draft && tid < N) anc_s[tid] = ancestor_bits(par_s, tid);   // visible after the next barrier

    // ---- DMA issue ---------------------------------------------------------------
    // Instruction j (< n_dma) of this wave covers 1 KB kb0 + j of the stage
    // [K codes][V codes][K scales][V scales].
    const int n_dma = wave < 4 ? 5 : 4;
    const int kb0 = 4 * wave + (wave < 4 ? wave : 4);
    // byte offset of instruction j within its array's part of the stage:
    // dma_kb[j] * 1024 (wave-uniform) + 16 lane
    uint32_t dma_kb[WL];
    const uint8_t *dma_gb[WL];
    int dma_rsh[WL];
    const uint32_t lane16 = (uint32_t)lane * 16u;
#pragma unroll
    for (int j = 0; j < WL; ++j) {
        const int kbi = kb0 + j < NKB ? kb0 + j : NKB - 1;   // j < n_dma keeps kb0 + j < NKB
        const int arr = kbi < KCI ? 0 : (kbi < 2 * KCI ? 1 : (kbi < 2 * KCI + KSI ? 2 : 3));
        const int start = arr == 0 ? 0 : (arr == 1 ? KCI : (arr == 2 ? 2 * KCI : 2 * KCI + KSI));
        dma_kb[j] = (uint32_t)(kbi - start);
        dma_gb[j] = arr == 0 ? (const uint8_t *)p.kv.k
                             : (arr == 1 ? (const uint8_t *)p.kv.v
                                         : (arr == 2 ? (const uint8_t *)p.kv.ks : (const uint8_t *)p.kv.vs));
        dma_rsh[j] = arr < 2 ? 7 : 4;                  // 128 code bytes / 16 scale bytes per row
    }
    const int64_t head_row0 = ((int64_t)b * p.Hkv + kvh) * p.kv.capacity;
    const uint32_t ring_u32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)ring;

    // Stage st = positions p0 + 128 st .. + 127; rows past the split's end
    // repeat its last row (their scores are masked).  Paged rows whose page is
    // outside the pool fetch the codes of row 0 of the array (no out-of-range
    // access) and zero scales, so they dequantise to zero rows.
    auto dma_off = [&](int j) { return (dma_kb[j] << 10) + lane16; };
    auto issue = [&](int st) {
        const int tb = p0 + st * T;
        const uint32_t slot = ring_u32 + (uint32_t)((st & 1) * STAGE + kb0 * 1024);
        if constexpr (!PAGED) {
            if (tb + T <= p1) {
#pragma unroll
                for (int j = 0; j < WL; ++j)
                    if (j < n_dma)
                        dma16s(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)),
                               dma_gb[j] + ((head_row0 + tb) << dma_rsh[j]), dma_off(j));
            } else {
                const int lim = p1 - 1 - tb;
#pragma unroll
                for (int j = 0; j < WL; ++j) {
                    if (j >= n_dma) continue;
                    const int rsh = dma_rsh[j];
                    const int row = (int)(dma_off(j) >> rsh);
                    const uint32_t col = dma_off(j) & ((1u << rsh) - 1u);
                    dma16s(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)),
                           dma_gb[j] + ((head_row0 + tb) << rsh), ((uint32_t)min(row, lim) << rsh) | col);
                }
            }
        } else {
            // all page-id reads first: each DMA statement orders memory, so a
            // read placed between two of them would be waited for alone
            const int ps = p.kv.page_size;
            const uint8_t *src[WL];
#pragma unroll
            for (int j = 0; j < WL; ++j) {
                const int rsh = dma_rsh[j];
                const int row = (int)(dma_off(j) >> rsh);
                const uint32_t col = dma_off(j) & ((1u << rsh) - 1u);
                const int pos = min(tb + row, p1 - 1);
                const int pq = pos / ps, pr = pos - pq * ps;
                const int pg = j < n_dma ? pages_s[pq - first_page] : 0;
                const int64_t ri = pg < 0 ? 0 : ((int64_t)pg * p.Hkv + kvh) * ps + pr;
                src[j] = (pg < 0 && rsh == 4) ? zero_scales : dma_gb[j] + (ri << rsh) + col;
            }
#pragma unroll
            for (int j = 0; j < WL; ++j)
                if (j < n_dma) dma16(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)), src[j]);
        }
    };

    // DMA instruction j of this wave for full stage st of a contiguous cache
    // (the last stage and paged caches: the whole stage at once through issue)
    auto issue_one = [&](int st, int j) {
        const int tb = p0 + st * T;
        if constexpr (!PAGED) {
            if (tb + T <= p1) {
                if (j < n_dma) {
                    const uint32_t slot = ring_u32 + (uint32_t)((st & 1) * STAGE + kb0 * 1024);
                    dma16s(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)),
                           dma_gb[j] + ((head_row0 + tb) << dma_rsh[j]), dma_off(j));
                }
                return;
            }
        }
        if (j == 0) issue(st);
    };

    // ---- prologue: the queries, then stages 0 and 1 ---------------------------------
    // The query loads go out first (behind every workgroup's stage 0 they
    // landed ~6 us after issue on the 131072-key block).  A wave loads only
    // its head-dim half of its rows; the row's scale comes from both halves'
    // maxima, exchanged with the partner wave (w ^ 4) through the score-half
    // buffer, which is free until the first chunk.
    const int row0 = rb * p.rows_per_block;
    const int rows_here = min(p.rows_per_block, R - row0);
    // S rows of this lane: tile hh * NTS + i, row l16; query fragments of the
    // head-dim half dh go to QTile<4 i + k>
    float sl2[NTS];
    int node_of[NTS];
    bf16x8 raw[NTS][4];
    float amax[NTS];
#pragma unroll
    for (int i = 0; i < NTS; ++i) {
        const int rl = 16 * (hh * NTS + i) + l16;
        const bool ok = rl < rows_here;
        const int r = row0 + rl;
        node_of[i] = ok ? r / G : -1;
        if (ok) {
            const int n = r / G, g = r % G;
            const __bf16 *qp = (const __bf16 *)p.q + (((int64_t)b * N + n) * p.Hq + (int64_t)kvh * G + g) * D +
                               128 * dh + qd * 8;
#pragma unroll
            for (int k = 0; k < 4; ++k) raw[i][k] = *(const bf16x8 *)(qp + 32 * k);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bf16x8 z = {};
                raw[i][k] = z;
            }
        }
    }
    // row maximum magnitude over this half (the lanes l16 + 16 qd), then over
    // both halves
    float *qx = sxb;                                   // [wave][tile][row l16]
#pragma unroll
    for (int i = 0; i < NTS; ++i) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf((float)raw[i][k][j]));
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        amax[i] = a;
        if (qd == 0) qx[(wave * NTS + i) * 16 + l16] = a;
    }
    // stages 0 and 1 go out while the other waves' queries land
    issue(0);
    if (n_st > 1) issue(1);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NTS; ++i) {
        const float a = fmaxf(amax[i], qx[((wave ^ 4) * NTS + i) * 16 + l16]);
        // 2^kq * amax in [2^14, 2^15): frexp gives amax = m 2^e, m in [0.5, 1)
        int kq = 0;
        if (a > 0.f) {
            kq = 15 - __builtin_amdgcn_frexp_expf(a);
            kq = kq > 100 ? 100 : (kq < -110 ? -110 : kq);
        }
        sl2[i] = ldexpf(p.scale_log2, -kq);
        h8 qv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // slot j holds value pi(j), pi = (0, 4, 2, 6, 1, 5, 3, 7)
            const int pi[8] = {0, 4, 2, 6, 1, 5, 3, 7};
            const bf16x8 src = raw[i][k];
#pragma unroll
            for (int j = 0; j < 8; ++j) qv[k][j] = (_Float16)ldexpf((float)src[pi[j]], kq);
        }
        static_for<0, 4 * NTS>([&](auto jc) {
            constexpr int J = decltype(jc)::value;
            if (J / 4 == i) QTile<J>::load(qv[J % 4]);
        });
    }

    // O^T tile (row tile t, head-dim tile dt of this wave) = OTile<2 t + dt>
    static_for<0, 2 * RB>([&](auto ic) { OTile<decltype(ic)::value>::zero(); });
    float m_ref[RB], l_s[NTS], l_p[NTS];
#pragma unroll
    for (int t = 0; t < RB; ++t) m_ref[t] = -INFINITY;
#pragma unroll
    for (int i = 0; i < NTS; ++i) l_s[i] = 0.f;

    // ---- LDS layout of a staged fp16 chunk of K or V: the 16-byte unit of
    // logical head-dim chunk c (8 values) and position p sits at
    // c * 512 + (p ^ 4 (c & 1)) * 16 (conflict-free writes, K fragment reads
    // and transposed V reads).
    // K fragment, position tile pt, k-step k: chunk 4 k + qd, position
    // 16 pt + (l16 ^ 2 dh).  The second head-dim half takes the positions of
    // each group of 4 in the order (2, 3, 0, 1), so that in both waves of a
    // pair a lane's score values 0, 1 are the two it finishes (positions
    // 4 qd + 2 dh + 0, 1) and values 2, 3 the two its partner finishes.
    const int k_lane = qd * 512 + ((16 * pt + (l16 ^ (2 * dh))) ^ (4 * (qd & 1))) * 16;   // + 2048 k
    // V^T fragment of 16-wide head-dim tile dg, half h: lane reads the 4-value
    // run r = l16 & 3 of position 8 qd + l16 / 4 + 4 h in chunk 2 dg + r / 2
    const int vsel = (l16 & 3) >> 1;
    const int va = 8 * qd + (l16 >> 2);
    const int v_lane0 = vsel * 512 + (va + 4 * vsel) * 16 + (l16 & 1) * 8;         // + 1024 dg
    const int v_lane1 = vsel * 512 + (va + 4 - 4 * vsel) * 16 + (l16 & 1) * 8;
    // P rows of this lane (PV operand): 8 positions 8 qd .. 8 qd + 7 of row 16 t + l16
    const int p_lane = l16 * PROW + 16 * qd;

    // Dequantisation: thread (row, 32-value block, half) of a chunk; the 256
    // (row, block) items are laid out so that the 8 threads of each LDS access
    // group take 8 different rows (mod 8) and 8 different blocks, and the two
    // halves (code words 0-1 and 2-3 of the block) go to waves w and w + 4.
    const int it = tid & 255, half = tid >> 8;
    const int di = it & 7, dj = it >> 3;
    const int drow = 8 * (dj & 3) + di, dblk = (di + (dj >> 2)) & 7;
    const int dsrc = drow * CROW + dblk * 16 + 8 * half, dssrc = drow * SROW + dblk * 2;
    const int ddst0 = (4 * dblk) * 512 + drow * 16 + 1024 * half;           // word 2 half
    const int ddst1 = (4 * dblk + 1) * 512 + (drow ^ 4) * 16 + 1024 * half; // word 2 half + 1
    const uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = 0x64006400u;
    struct Codes {
        u32x2 w;
        h2 s;
    };
    // codes and scale of chunk g of K (which = 0) or V (1) from the ring
    auto dq_load = [&](int which, int g) {
        const uint8_t *stg = ring + ((g / CPS) & 1) * STAGE + (g % CPS) * 32 * CROW;
        Codes c;
        c.w = *(const u32x2 *)(stg + which * T * CROW + dsrc);
        const uint32_t sb = *(const uint16_t *)(ring + ((g / CPS) & 1) * STAGE + 2 * T * CROW + which * T * SROW +
                                                (g % CPS) * 32 * SROW + dssrc);
        c.s = __builtin_bit_cast(h2, sb * 0x10001u);
        return c;
    };
    auto dq_word = [&](int which, const Codes &c, int mm) {
        uint8_t *dst = (which ? vst : kst) + (mm ? ddst1 : ddst0);
        *(u32x4 *)dst = dequant_word(c.w[mm], c.s, m_lo, m_hi, magic);
    };
    auto kread = [&](int k) { return *(const h8 *)(kst + k_lane + 2048 * k); };

    // row maxima of one S tile (log2 units) into the exchange buffer
    auto xmax = [](float x, bool by32) {
        const auto r = by32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                            : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    // layout [row l16][row tile][position tile, head-dim half]
    auto row_max = [&](float s0, float s1, int i) {
        float c = fmaxf(s0, s1);
        c = xmax(xmax(c, false), true) * sl2[i];
        mxb[(l16 * RB + hh * NTS + i) * 4 + 2 * pt + dh] = c;
        return c;
    };
    // tree / split-end mask of chunk g on this lane's two positions of each tile
    auto apply_mask = [&](int g, float (&s)[NTS][2]) {
        const int cb = p0 + 32 * g;
        if (cb + 32 > ctx || cb + 32 > p1) {
            const int pos0 = cb + 16 * pt + 4 * qd + 2 * dh;
#pragma unroll
            for (int i = 0; i < NTS; ++i) {
                const uint64_t anc_r = anc_s[node_of[i] > 0 ? node_of[i] : 0];     // in bounds for every lane
                const uint64_t anc = node_of[i] >= 0 ? anc_r : 0ull;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int pos = pos0 + j;
                    bool vis = pos < p1;
                    vis &= (pos < ctx) | (((anc >> ((pos - ctx) & 63)) & 1ull) != 0ull);
                    s[i][j] = vis ? s[i][j] : -INFINITY;
                }
            }
        }
    };
    // score halves: wave (pair w & 3, half dh) writes values 2, 3 of each
    // lane (those its partner finishes) ...
    float2 *sx_w = (float2 *)sxb + ((wave & 3) * 2 + dh) * NTS * 64 + lane;
    const float2 *sx_r = (const float2 *)sxb + ((wave & 3) * 2 + (dh ^ 1)) * NTS * 64 + lane;
    auto sx_put = [&](const f32x4 (&sc)[NTS]) {
#pragma unroll
        for (int i = 0; i < NTS; ++i) sx_w[i * 64] = make_float2(sc[i][2], sc[i][3]);
    };
    // ... and adds the partner's share to its own values 0, 1
    auto sx_take = [&](const f32x4 (&sc)[NTS], const float2 (&o)[NTS], float (&s)[NTS][2]) {
#pragma unroll
        for (int i = 0; i < NTS; ++i) {
            s[i][0] = sc[i][0] + o[i].x;
            s[i][1] = sc[i][1] + o[i].y;
        }
    };
    auto sx_load = [&](float2 (&o)[NTS]) {
#pragma unroll
        for (int i = 0; i < NTS; ++i) o[i] = sx_r[i * 64];
    };
    // the halves of S over this wave's four k-steps; kf holds the fragments
    // of k-steps 0 and 1 on entry (a ring of two: each read goes out after the
    // instructions that free its slot)
    auto s_partial = [&](f32x4 (&sc)[NTS], h8 (&kf)[2], auto between) {
        static_for<0, 4>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            const h8 ka = kf[k & 1];
            if constexpr (k + 2 < 4) kf[k & 1] = kread(4 * dh + k + 2);
            static_for<0, NTS>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                if constexpr (k == 0) sc[i] = QTile<4 * i + k>::first(ka);
                else QTile<4 * i + k>::acc(sc[i], ka);
            });
            between(k);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- prologue: stage 0 landed (stage 1 may be in flight) -----------------
    if (n_st > 1) {
        if (n_dma == 5) wait_vm<5>();
        else wait_vm<4>();
    } else {
        wait_vm<0>();
    }
    __syncthreads();
    {
        const Codes k0 = dq_load(0, 0);
        dq_word(0, k0, 0);
        dq_word(0, k0, 1);
    }
    __syncthreads();
    f32x4 sacc[NTS];
    float s2[NTS][2];
    {
        h8 kf[2] = {kread(4 * dh), kread(4 * dh + 1)};
        s_partial(sacc, kf, [](int) {});
        mfma_drain_s(sacc);
        sx_put(sacc);
    }
    __syncthreads();
    {
        float2 o[NTS];
        sx_load(o);
        sx_take(sacc, o, s2);
    }
    apply_mask(0, s2);
#pragma unroll
    for (int i = 0; i < NTS; ++i) row_max(s2[i][0], s2[i][1], i);
    {
        const Codes k1 = dq_load(0, min(1, NCH - 1));
        dq_word(0, k1, 0);
        dq_word(0, k1, 1);
    }
    if (tid < 2) gflag[tid] = 0;
    // References from chunk 0's exact row maxima (every wave reads the same
    // published values), so that typical splits never move one afterwards.
    __syncthreads();
    {
        const float4 *mxr = (const float4 *)mxb + l16 * RB;
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            const float4 m4 = mxr[t];
            m_ref[t] = fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w));
        }
    }

    auto vread = [&](int dt) {
        const int dg = 2 * wave + dt;                    // 16-wide head-dim tile
        const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(__attribute__((address_space(3))) uint8_t *)(
                vst + v_lane0 + 1024 * dg));
        const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(__attribute__((address_space(3))) uint8_t *)(
                vst + v_lane1 + 1024 * dg));
        const short __attribute__((ext_vector_type(8))) w8 = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        return __builtin_bit_cast(h8, w8);
    };

    // chunk(SLOW, g, first): one chunk, in two phases between barriers.
    //   phase 1: P(g) from the published maxima of S(g); V(g) dequantised;
    //            the halves of S(g + 1) on the matrix cores; the score halves
    //            exchanged; the next stage's copies issued.
    //   phase 2: S(g + 1) finished, masked and its row maxima published;
    //            K(g + 2) dequantised; O^T += V(g)^T P(g)^T.
    // The fast form (SLOW false) returns true, before any matrix work, when a
    // row maximum would move its reference; the caller then finishes the split
    // with the slow form, which rescales in place.  Chunks past the last one
    // are still computed from in-bounds ring data into buffers nobody reads.
    auto chunk = [&](auto slow_c, int g, bool first) -> bool {
        constexpr bool SLOW = decltype(slow_c)::value;
        // ---- barrier 1: maxima of S(g) published, K(g + 1) staged; every
        // wave has read V(g - 1) and the codes of chunk g - 1, so the ring
        // slot of the stage before g's is free from chunk 4 s on
        if (!first) __syncthreads();
        const int st_issue = ((g & (CPS - 1)) == 0 && g > 0) ? g / CPS + 1 : n_st;

        // the fast form: one flag says whether any row maximum of S(g) moved
        // past its reference (set by the waves that found it); the caller then
        // restarts the chunk in the slow form
        const int moved = SLOW ? 0 : gflag[g & 1];     // checked once P(g) is written
        h8 kf[2] = {kread(4 * dh), kread(4 * dh + 1)};
        const Codes cv = dq_load(1, g);

        if constexpr (SLOW) {
            // the lazy rule, in place: a reference moves when the chunk's
            // maximum exceeds it by more than 2^8
            float cm[RB];
            const float4 *mxr = (const float4 *)mxb + l16 * RB;
#pragma unroll
            for (int t = 0; t < RB; ++t) {
                const float4 m4 = mxr[t];
                cm[t] = fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w));
            }
            float alpha[RB];
            bool grow = false;
#pragma unroll
            for (int t = 0; t < RB; ++t) {
                const bool need = cm[t] > m_ref[t] + 8.f;
                alpha[t] = need ? __builtin_amdgcn_exp2f(m_ref[t] - cm[t]) : 1.f;
                m_ref[t] = need ? cm[t] : m_ref[t];
                grow |= need;
            }
            if (__any(grow)) {
                mfma_drain();
                static_for<0, 2 * RB>([&](auto ic) {
                    constexpr int I = decltype(ic)::value;
                    OTile<I>::scale(alpha[I / 2]);
                });
                asm volatile("s_nop 3");
#pragma unroll
                for (int i = 0; i < NTS; ++i) l_s[i] *= hh ? alpha[NTS + i] : alpha[i];
            }
        }

        // P(g): this lane's two positions of each tile
#pragma unroll
        for (int t = 0; t < NTS; ++t) {
            const float mr = (hh ? m_ref[NTS + t] : m_ref[t]);
            const float mu = mr == -INFINITY ? 0.f : mr;
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[t][0], sl2[t], -mu));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[t][1], sl2[t], -mu));
            l_p[t] = e0 + e1;
            typedef float f32x2_t __attribute__((ext_vector_type(2)));
            *(uint32_t *)(pbuf + (16 * (hh * NTS + t) + l16) * PROW + (16 * pt + 4 * qd + 2 * dh) * 2) =
                __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){e0, e1}, h2));
        }
        dq_word(1, cv, 0);
        if constexpr (!SLOW) {
            if (__builtin_expect(moved != 0, 0)) return true;
        }
#pragma unroll
        for (int t = 0; t < NTS; ++t) l_s[t] += l_p[t];

        // ---- halves of S(g + 1); V(g) word 1 and the stage copies between the
        // matrix instructions ---------------------------------------------------------
        // (a paged stage goes out whole before them: its page lookups need
        // registers that the score halves hold during the matrix instructions)
        if constexpr (PAGED) {
            if (st_issue < n_st) issue(st_issue);
        }
        f32x4 sacc_n[NTS];
        s_partial(sacc_n, kf, [&](int k) {
            if (k == 1) dq_word(1, cv, 1);
            if constexpr (!PAGED) {
                if (st_issue < n_st) issue_one(st_issue, k);
            }
        });
        if constexpr (!PAGED) {
            if (st_issue < n_st) issue_one(st_issue, 4);
        }
        mfma_drain_s(sacc_n);                               // S(g + 1) halves complete before vector reads
        sx_put(sacc_n);

        // stage (g + 2) / 4 is needed from here on: this wave's part landed
        if (((g + 2) & (CPS - 1)) == 0 && g + 2 < NCH) wait_vm<0>();

        // ---- barrier 2: P(g), V(g) and the score halves published; every wave
        // has read K(g + 1) -------------------------------------------------------------
        __syncthreads();

        {
            // the score halves first (the row maxima wait on them), then the
            // operands of the P.V instructions and the codes of K(g + 2)
            float2 sxo[NTS];
            sx_load(sxo);
            __builtin_amdgcn_sched_barrier(0);
            h8 vf[2];
            vf[0] = vread(0);
            vf[1] = vread(1);
            const int gk = g + 2 < NCH ? g + 2 : g;
            const Codes ck = dq_load(0, gk);
            const uint8_t *prd = pbuf + p_lane;
            h8 pf[2];
            pf[0] = *(const h8 *)prd;
            pf[1] = *(const h8 *)(prd + 16 * PROW);
            float s2n[NTS][2];
            sx_take(sacc_n, sxo, s2n);
            apply_mask(g + 1, s2n);
            bool grow = false;
#pragma unroll
            for (int i = 0; i < NTS; ++i) {
                const float c = row_max(s2n[i][0], s2n[i][1], i);
                grow |= c > (hh ? m_ref[NTS + i] : m_ref[i]) + 8.f;
            }
            if constexpr (!SLOW) {
                // every wave read this chunk's flag before the second barrier
                if (tid == 0) gflag[g & 1] = 0;
                if (__any(grow) && lane == 0) gflag[(g + 1) & 1] = 1;
            }
            dq_word(0, ck, 0);
            static_for<0, RB>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                const h8 pa = pf[t & 1];
                if constexpr (t + 2 < RB) pf[t & 1] = *(const h8 *)(prd + 16 * (t + 2) * PROW);
                OTile<2 * t>::mac(vf[0], pa);
                OTile<2 * t + 1>::mac(vf[1], pa);
                if constexpr (t == RB / 2 - 1) dq_word(0, ck, 1);
                __builtin_amdgcn_sched_barrier(0);
            });
#pragma unroll
            for (int i = 0; i < NTS; ++i) {
                s2[i][0] = s2n[i][0];
                s2[i][1] = s2n[i][1];
            }
        }
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
    // ---- row sums: lanes of a row, then the four (position tile, head-dim
    // half) waves of a row tile ----------------------------------------------------
#pragma unroll
    for (int i = 0; i < NTS; ++i) {
        l_s[i] += __shfl_xor(l_s[i], 16, 64);
        l_s[i] += __shfl_xor(l_s[i], 32, 64);
        if (qd == 0) lsx[(2 * pt + dh) * ROWS + 16 * (hh * NTS + i) + l16] = l_s[i];
    }
    __syncthreads();

    // ---- partials of this split --------------------------------------------------
    const int64_t part = wu.part;
    static_for<0, RB>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        const int rl = 16 * t + l16;
        float *op = p.part_o + (part * R + row0 + rl) * D;
        static_for<0, 2>([&](auto dc) {
            constexpr int dt = decltype(dc)::value;
            const f32x4 o = OTile<2 * t + dt>::read();
            if (rl >= rows_here) return;
            // the four values of slots s0 .. s0 + 3 in one 16-byte store, the row
            // left in slot order (slot s holds head dim 8 (s / 8) + pi(s % 8),
            // pi = 0, 4, 2, 6, 1, 5, 3, 7; the merge restores the order): four
            // scattered 4-byte stores per value group kept every workgroup's
            // last ~5 us on issuing them
            const int s0 = 32 * wave + 16 * dt + 4 * qd;
            *(f32x4 *)(op + s0) = o;
        });
    });
    if (pt == 0 && dh == 0 && qd == 0) {
#pragma unroll
        for (int i = 0; i < NTS; ++i) {
            const int rl = 16 * (hh * NTS + i) + l16;
            if (rl >= rows_here) continue;
            const float mr = hh ? m_ref[NTS + i] : m_ref[i];
            const float ls = (lsx[rl] + lsx[ROWS + rl]) + (lsx[2 * ROWS + rl] + lsx[3 * ROWS + rl]);
            p.part_ml[(part * R + row0 + rl) * 2 + 0] = mr;
            p.part_ml[(part * R + row0 + rl) * 2 + 1] = ls;
        }
    }
}

template <int NTS, bool PAGED>
hipError_t launch_t(const AttnParams &p, hipStream_t st) {
    const int grid = ((p.n_units + 7) / 8) * 8 * p.n_rowblocks;
    hipLaunchKernelGGL((attn_q4w_kernel<NTS, PAGED>), dim3(grid), dim3(64 * NW), 0, st, p);
    return hipGetLastError();
}

}  // namespace

// Paged caches take blocks of up to 2 row tiles per wave pair: at 3 the page
// lookups push the compiler's values past its 128 registers into the
// accumulation registers that hold the queries (the planner sends those
// blocks to the four-wave kernel).
bool attn_q4w_supports(bool paged, int nts) { return nts >= 1 && nts <= (paged ? 2 : 3); }

hipError_t launch_attn_q4w(const AttnParams &p, int nts, hipStream_t st) {
    const bool paged = p.kv.page_table != nullptr;
    if (!attn_q4w_supports(paged, nts)) return hipErrorInvalidValue;
    if (paged) return nts == 1 ? launch_t<1, true>(p, st) : launch_t<2, true>(p, st);
    if (nts == 1) return launch_t<1, false>(p, st);
    if (nts == 2) return launch_t<2, false>(p, st);
    return launch_t<3, false>(p, st);
}

}  // namespace sv
