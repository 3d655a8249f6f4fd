// Split-KV verify attention over a bf16 KV cache on gfx950: direct-to-LDS
// multi-stage pipeline + bf16 matrix cores.
//
// One workgroup (4 waves) handles one (sequence, KV head, row block, split).
// Packed query rows of a KV head are r = node * G + g: the verify rows of all
// query heads of the GQA group [single-RTX-3090 DFlash note: 24 Q / 4 KV heads
// of dim 256, "Why we ran this test"; 16-row blocks, "Architecture"; budget+1
// tree rows, "Key breakthroughs"].  A wave owns up to NT tiles of 16 rows; when
// a block has a single row tile, PG waves split each stage's positions.
//
// Memory pipeline.  A stage is T = 32 * PG consecutive key positions: the K
// rows then the V rows, both in their natural [pos][d] order, 16-byte chunks
// XOR-swizzled per row.  Stages are fetched with global_load_lds_dwordx4 (each
// lane's 16 bytes land at M0 + 16 * lane), issued from inline assembly so the
// compiler does not drain them before every LDS read; an S-deep ring keeps
// S - 1 stages in flight and each wave waits on its own vmcnt for exactly the
// stage it is about to use.  No registers stage the data and nothing is
// transposed on the way in.
//
// Math per 32-position chunk (16x16x32 bf16 MFMA):
//   S^T = K Q^T    A = K rows from LDS (one ds_read_b128 per k-step),
//                  B = the wave's query fragments held in registers;
//   online softmax in log2 units, per lane one row and 8 positions; the
//   reference maximum is refreshed only when a row's maximum grows by more
//   than 2^8 (numerator and denominator share it, so this is exact);
//   O^T += V^T P^T  A = V^T fragments read with ds_read_b64_tr_b16 (within a
//                  16-lane group, lane i receives element i % 4 of the 4-value
//                  runs read by lanes 4k + i/4, k = 0..3: two such reads give a
//                  lane 8 positions of one head-dim column straight from the
//                  natural V layout), B = the probabilities already in place.
// Tree mask [DFN "From autoregressive to DDTree"; chains: causal mask aligned
// to the end of the keys, xdnf.cn notes section 5.3]: 64-bit ancestor sets in
// LDS, applied on chunks that reach the draft rows.
// Output: unnormalised partials (O, m, l) per row for the split merge.
#include "attn_sched.h"

#ifndef SV_SWZ_W
#define SV_SWZ_W 16
#endif

namespace sv {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D, int NT, int PG, bool Q4, int OCC>
struct DCfg {
    static constexpr int W = D >= 128 ? SV_SWZ_W : 8;          // swizzle width (chunks)
    // positions per stage: 32 per position group for bf16; for the 4-bit
    // cache 32768 / D, so a stage is 36 whole 1 KB loads (9 per wave)
    static constexpr int T = Q4 ? 32768 / D : 32 * PG;
    static constexpr int ROWB = D * 2;                // bytes per bf16 K / V row
    static constexpr int CROWB = D / 2;               // 4-bit codes per row
    static constexpr int SROWB = D / 16;              // fp16 scales per row
    static constexpr int KBYTES = Q4 ? T * CROWB : T * ROWB;   // K part of a stage
    static constexpr int STAGE = Q4 ? 2 * T * (CROWB + SROWB) : 2 * KBYTES;
    static constexpr int S_RAW = 131072 / OCC / STAGE;   // OCC workgroups share a CU's LDS
    static constexpr int S = Q4 ? 2 : (S_RAW < 2 ? 2 : (S_RAW > 8 ? 8 : S_RAW));   // ring depth
    static constexpr int NKB = STAGE / 1024;          // 1 KB DMA instructions per stage
    static constexpr int LPW = NKB / 4;               // per wave
    static constexpr int RPK = 1024 / ROWB;           // rows per DMA instruction (bf16)
    static constexpr int RG = 4 / PG;
    static constexpr int KS = D / 32;
    static constexpr int DT = D / 16;
    static constexpr int CH = Q4 ? T / 32 : 1;        // 32-position chunks per stage, in turn
    // bf16, several row tiles per wave, one DMA instruction per k-step: a full
    // stage's loads go out between the k-steps of the chunk before (with one
    // tile the chunk is short and the branch costs more than it saves)
    static constexpr bool SPREAD = !Q4 && LPW <= KS && NT >= 2;
    static constexpr int STAGING = Q4 ? 2 * 32 * ROWB : 0;   // dequantised K and V of one chunk (x2 buffers)
    static_assert(Q4 ? (NKB % 4 == 0) : (NKB % 8 == 0), "stage split evenly between waves (and K/V)");
    static_assert(!Q4 || (D == 256 && PG == 1), "4-bit stages: head dim 256, one position group");
    static_assert(LPW * (S - 2) < 64, "vmcnt range");
};

// Chunk swizzle shared by the K (16-byte) and V (transposed 8-byte) reads.  A
// K fragment read touches 16 rows {8a + b : a, b < 4} (+4t) at one logical
// chunk; a V transposed read touches rows 8q + 4h + b (b < 4) at two adjacent
// chunks.  W = 16 spreads the 16 K rows over 16 distinct 16-byte bank groups
// and each 8-row half of the V rows over 8 distinct pairs (head dims >= 128,
// i.e. >= 16 chunks per row); W = 8 is the 3-bit form for 8 chunks per row.
template <int W>
__device__ __forceinline__ int swz(int row) {
    if constexpr (W == 16) return ((row & 3) << 1) | (((row >> 3) & 1) << 3) | ((row >> 4) & 1);
    return ((row & 3) << 1) | ((row >> 3) & 1);
}

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int STEP, int K>
__device__ __forceinline__ void wait_vm_dyn(int k) {
    if constexpr (K < 0) {
        wait_vm<0>();
    } else {
        if (k >= K) wait_vm<STEP * K>();
        else wait_vm_dyn<STEP, K - 1>(k);
    }
}

__device__ __forceinline__ void dma16(uint32_t lds_base, const void *gptr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(gptr)
                 : "memory", "m0");
}

// the same with a wave-uniform 64-bit base (scalar registers) and a 32-bit
// lane offset
__device__ __forceinline__ void dma16s(uint32_t lds_base, const void *sbase, uint32_t voff) {
    // (the builtin returns int: widen each half as unsigned, never sign-extend)
    const uint64_t a = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(u)
                 : "memory", "m0");
}

constexpr int kMaxSplitPages = 512;

// the source of every DMA of a row whose page lies outside the pool: one row
// of zeros as wide as the widest row (bf16, head dim 256)
__device__ __attribute__((aligned(16))) uint8_t zero_row[512] = {};

template <int D, int NT, int PG, bool PAGED, bool Q4, int OCC>
__global__ __launch_bounds__(256, OCC) void attn_dma_kernel(AttnParams p) {
    using C = DCfg<D, NT, PG, Q4, OCC>;
    constexpr int T = C::T, S = C::S;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[S * C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t staging[Q4 ? 2 * C::STAGING : 16];
    __shared__ int par_s[64];
    __shared__ uint64_t anc_s[64];
    __shared__ int pages_s[PAGED ? kMaxSplitPages : 1];

    __shared__ SchedLds sched_s;

    // ---- unit: (b, kv head, row block, split); row blocks of one (b, head,
    // split) get ids 8 apart, i.e. the same XCD and L2 ---------------------
    const int id = blockIdx.x;
    const int xcd = id & 7, k8 = id >> 3;
    const int rb = k8 % p.n_rowblocks;
    AttnUnit wu;
    if (!attn_unit(p, (k8 / p.n_rowblocks) * 8 + xcd, rb == 0, sched_s, wu)) return;
    // the unit is the same for the whole block: keep it in scalar registers
    const int b = __builtin_amdgcn_readfirstlane(wu.b), kvh = __builtin_amdgcn_readfirstlane(wu.kvh);
    const int N = p.N, G = p.G, R = p.R;
    const int ctx = __builtin_amdgcn_readfirstlane(wu.ctx);
    const int p0 = __builtin_amdgcn_readfirstlane(wu.p0), p1 = __builtin_amdgcn_readfirstlane(wu.p1);
    const int n_st = (p1 - p0 + T - 1) / T;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave-uniform
    const int rg = wave % C::RG, pg = wave / C::RG;
    const int l16 = lane & 15, qd = lane >> 4;

    // ---- tree (only splits that reach the draft rows) and page ids ---------
    const bool has_draft = p1 > ctx;
    if (has_draft && tid < N) par_s[tid] = parent_of(p.parent + (int64_t)b * N, tid, p.err);
    int first_page = 0;
    const int ps_shift = (p.kv.page_size > 0 && (p.kv.page_size & (p.kv.page_size - 1)) == 0)
                             ? __builtin_ctz((unsigned)p.kv.page_size) : -1;
    if constexpr (PAGED) {
        first_page = p0 / p.kv.page_size;
        const int last_page = (p1 - 1) / p.kv.page_size;
        for (int e = tid; e <= last_page - first_page; e += 256) {
            const int pgid = p.kv.page_table[(int64_t)b * p.kv.max_pages + first_page + e];
            const bool bad = pgid < 0 || pgid >= p.kv.capacity;
            SV_DEVCHECK(p.err, bad, SV_DEVERR_PAGE);
            pages_s[e] = bad ? -1 : pgid;                  // -1: a zero row
        }
    }
    __syncthreads();
    if (has_draft && tid < N) anc_s[tid] = ancestor_bits(par_s, tid);   // visible after the loop's first barrier

    // ---- DMA issue: instruction j of this wave covers 1 KB of the stage ------
    const uint8_t *kbase = (const uint8_t *)p.kv.k;
    const uint8_t *vbase = (const uint8_t *)p.kv.v;
    const uint8_t *ksbase = (const uint8_t *)p.kv.ks;
    const uint8_t *vsbase = (const uint8_t *)p.kv.vs;
    const int64_t head_row0 = ((int64_t)b * p.Hkv + kvh) * p.kv.capacity;   // contiguous
    const uint32_t ring_u32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)ring;

    // Lane constants of DMA instruction j: the byte offset of the lane's 16
    // bytes within the array's part of a stage (row * row bytes + column, rows
    // in order) and (4-bit cache) the array it reads: a 4-bit stage is
    // [K codes][V codes][K scales][V scales].  bf16 rows are swizzled in
    // 16-byte chunks as they land: the lane fetches the chunk whose swizzled
    // place is its own slot of the 1 KB the instruction writes.
    uint32_t dma_off[C::LPW];
    int dma_arr[C::LPW];                    // wave-uniform
    // the array's base and log2 row bytes (wave-uniform; a bf16 wave reads
    // one array only: waves 0-1 K, waves 2-3 V)
    const uint8_t *dma_gb[Q4 ? C::LPW : 1];
    int dma_rsh[Q4 ? C::LPW : 1];
    static_assert(Q4 || (2 * C::LPW) % (C::NKB / 2) == 0 || C::NKB / 2 % C::LPW == 0, "one array per bf16 wave");
    if constexpr (!Q4) {
        dma_gb[0] = wave * C::LPW >= C::NKB / 2 ? vbase : kbase;
        dma_rsh[0] = __builtin_ctz(C::ROWB);
    }
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) {
        const int kbi = wave * C::LPW + j;
        if constexpr (Q4) {
            constexpr int KCI = C::T * C::CROWB / 1024, KSI = C::T * C::SROWB / 1024;
            const int arr = kbi < KCI ? 0 : (kbi < 2 * KCI ? 1 : (kbi < 2 * KCI + KSI ? 2 : 3));
            const int start = arr == 0 ? 0 : (arr == 1 ? KCI : (arr == 2 ? 2 * KCI : 2 * KCI + KSI));
            dma_arr[j] = arr;
            dma_off[j] = (uint32_t)((kbi - start) * 1024 + lane * 16);
            dma_gb[j] = arr == 0 ? kbase : (arr == 1 ? vbase : (arr == 2 ? ksbase : vsbase));
            dma_rsh[j] = arr < 2 ? __builtin_ctz(C::CROWB) : __builtin_ctz(C::SROWB);
        } else {
            const int kb_in = kbi >= C::NKB / 2 ? kbi - C::NKB / 2 : kbi;
            const int row = kb_in * C::RPK + (lane * 16) / C::ROWB;
            const int chunk = ((lane * 16) % C::ROWB / 16) ^ swz<C::W>(row);
            dma_arr[j] = kbi >= C::NKB / 2;
            dma_off[j] = (uint32_t)(row * C::ROWB + chunk * 16);
        }
    }

    // Stage st = positions tb .. tb + T - 1 of the split; rows past the
    // split's end (last stage) repeat its last row.  Contiguous cache: one
    // uniform base per array and stage, lane offsets fixed for full stages.
    // This wave's DMA instructions for stage st: contiguous cache, a uniform
    // base per array and a lane offset (rows past the split's end, last stage
    // only, repeat its last row); paged cache, the lane addresses.
    auto issue = [&](int st) {
        const int tb = p0 + st * T;
        const uint32_t slot = ring_u32 + (uint32_t)((st % S) * C::STAGE + wave * C::LPW * 1024);
        if constexpr (!PAGED) {
            if (tb + T <= p1) {                                  // full stage (uniform)
#pragma unroll
                for (int j = 0; j < C::LPW; ++j) {
                    const int jj = Q4 ? j : 0;
                    dma16s(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)),
                           dma_gb[jj] + ((head_row0 + tb) << dma_rsh[jj]), dma_off[j]);
                }
            } else {
                const int lim = p1 - 1 - tb;                     // last row of the split in this stage
#pragma unroll
                for (int j = 0; j < C::LPW; ++j) {
                    const int jj = Q4 ? j : 0;
                    const int rsh = dma_rsh[jj];
                    const int row = (int)(dma_off[j] >> rsh);
                    const uint32_t col = dma_off[j] & ((1u << rsh) - 1u);
                    dma16s(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)),
                           dma_gb[jj] + ((head_row0 + tb) << rsh), ((uint32_t)min(row, lim) << rsh) | col);
                }
            }
        } else {
            // all page-id reads first: each DMA statement orders memory, so a
            // read placed between two of them would be waited for alone
            const int ps = p.kv.page_size;
            const uint8_t *src[C::LPW];
#pragma unroll
            for (int j = 0; j < C::LPW; ++j) {
                const int jj = Q4 ? j : 0;
                const int rsh = dma_rsh[jj];
                const int row = (int)(dma_off[j] >> rsh);
                const uint32_t col = dma_off[j] & ((1u << rsh) - 1u);
                const int pos = min(tb + row, p1 - 1);
                int pq, pr;
                if (ps_shift >= 0) {
                    pq = pos >> ps_shift;
                    pr = pos & (ps - 1);
                } else {
                    pq = pos / ps;
                    pr = pos - pq * ps;
                }
                const int pg = pages_s[pq - first_page];
                const int64_t ri = ((int64_t)pg * p.Hkv + kvh) * ps + pr;
                // a page outside the pool reads the zero row
                src[j] = pg < 0 ? zero_row + col : dma_gb[jj] + (ri << rsh) + col;
            }
#pragma unroll
            for (int j = 0; j < C::LPW; ++j) dma16(__builtin_amdgcn_readfirstlane(slot + (uint32_t)(j * 1024)), src[j]);
        }
    };
    // instruction j of full stage st of a contiguous cache
    auto issue_full = [&](int st, int j) {
        const int jj = Q4 ? j : 0;
        dma16s(__builtin_amdgcn_readfirstlane(ring_u32 + (uint32_t)((st % S) * C::STAGE + (wave * C::LPW + j) * 1024)),
               dma_gb[jj] + ((head_row0 + p0 + st * T) << dma_rsh[jj]), dma_off[j]);
    };

    // ---- pipeline prologue: the first stages go out before the query loads, so
    // their latencies overlap ----------------------------------------------------
    const int pro = min(S - 1, n_st);
    for (int st = 0; st < pro; ++st) issue(st);

    // ---- query fragments and accumulators ------------------------------------
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

    // Lane constants of the LDS fragment reads.  K rows read by a lane are
    // 8 * (l16 / 4) + (l16 % 4) (+ 4t); V rows 8 * qd + l16 / 4 (+ 4hh); with a
    // chunk base that is a multiple of 32 rows their swizzle does not depend on
    // the chunk, t or hh, so each read is a lane constant plus an immediate.
    constexpr int W = C::W;
    const int ksz = swz<W>(8 * (l16 >> 2) + (l16 & 3));
    const int k_lane = (8 * (l16 >> 2) + (l16 & 3)) * C::ROWB;
    int k_off[W / 4];                       // K chunk 4k + qd: k % (W/4) varies the XOR
#pragma unroll
    for (int kk = 0; kk < W / 4; ++kk) k_off[kk] = ((4 * kk + qd) ^ ksz) * 16;
    const int vsz = swz<W>(8 * qd + (l16 >> 2));
    const int vch = (l16 & 3) >> 1;
    const int v_lane = (8 * qd + (l16 >> 2)) * C::ROWB + (l16 & 1) * 8;
    int v_off[W / 2];                       // V chunk 2dt + vch: dt % (W/2) varies the XOR
#pragma unroll
    for (int dd = 0; dd < W / 2; ++dd) v_off[dd] = ((2 * dd + vch) ^ vsz) * 16;

    // The query loads were issued after the prologue stages; waiting for them
    // (the compiler would insert the same wait before their first use) also
    // waits for those stages.
    wait_vm<0>();

    // ---- 4-bit cache: the 256 threads turn chunk c of ring slot `slot` into
    // bf16 rows in staging buffer `buf` (thread: one row, one 32-value block of
    // K and of V; value = d * (code - 8) exactly in fp32, rounded to
    // nearest-even bf16) --------------------------------------------------------
    auto dequant = [&](int slot, int c, int buf) {
        if constexpr (Q4) {
            const uint8_t *stg = ring + slot * C::STAGE;
            const int row = tid >> 3, blk = tid & 7;
#pragma unroll
            for (int which = 0; which < 2; ++which) {
                const u32x4 w = *(const u32x4 *)(stg + which * C::T * C::CROWB + (c * 32 + row) * C::CROWB + blk * 16);
                const float sc = fp16_bits_to_f32(*(const uint16_t *)(stg + 2 * C::T * C::CROWB +
                                                                    which * C::T * C::SROWB +
                                                                    (c * 32 + row) * C::SROWB + blk * 2));
                const float off = -8.f * sc;
                uint8_t *dst = staging + buf * C::STAGING + which * 32 * C::ROWB + row * C::ROWB;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    // byte t of the row holds values 2t (low nibble) and 2t + 1
                    const uint32_t lo = w[m] & 0x0F0F0F0Fu, hi = (w[m] >> 4) & 0x0F0F0F0Fu;
                    u32x4 out;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        out[k] = pack_bf16x2(__builtin_fmaf((float)((lo >> (8 * k)) & 0xFFu), sc, off),
                                             __builtin_fmaf((float)((hi >> (8 * k)) & 0xFFu), sc, off));
                    *(u32x4 *)(dst + ((4 * blk + m) ^ swz<C::W>(row)) * 16) = out;
                }
            }
        }
    };

    // ---- one 32-position chunk of K / V rows in LDS (natural order, 16-byte
    // chunks swizzled): scores, masks, online softmax, O^T += V^T P^T ----------
    // (4-bit cache: the next chunk's dequantisation runs between this chunk's
    // Q K^T matrix instructions)
    // ist >= 0: this wave's DMA instructions of full stage ist (contiguous
    // cache) go out between the k-steps (a wave that sends a whole stage at
    // once stalls until the memory pipeline has taken them all)
    auto compute = [&](const int ist, const uint8_t *Kl, const uint8_t *Vl, const int cb, const int abase,
                       int n_slot, int n_c, int n_buf) {
        // Every wave runs all NT tile slots: a slot without rows holds zero
        // queries, gives finite scores and is never written back, and no
        // branch breaks the stream of matrix instructions (the waves meet at
        // the next barrier anyway).
        //
        // Order within a stage (one wavefront, so overlap comes from the
        // instruction order): the K fragment reads, then the Q K^T matrix
        // instructions with the V^T fragment reads of this stage slotted
        // between them; the masks and lane-local maxima; then per tile the
        // exponentials of tile i+1 slotted between the V^T P^T matrix
        // instructions of tile i.
        const uint8_t *kp = Kl + cb * C::ROWB + k_lane;
        const uint8_t *vp = Vl + cb * C::ROWB + v_lane;
        f32x4 sacc[NT][2];
        bf16x8 vf[C::DT];
        {
            // K fragment (t, k) sits at k_lane + 4t rows + (k / (W/4)) * 16W bytes
            // + a lane constant that depends only on k % (W/4); V^T fragment
            // (dt, hh) at v_lane + 4hh rows + (dt / (W/2)) * 16W bytes + a lane
            // constant that depends only on dt % (W/2)
            auto kread = [&](int t, int k) {
                return *(const bf16x8 *)(kp + 4 * t * C::ROWB + (k / (W / 4)) * (W * 16) + k_off[k % (W / 4)]);
            };
            auto vread = [&](int dt) {
                s16x4 h[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4 *)(__attribute__((address_space(3))) uint8_t *)(
                            vp + 4 * hh * C::ROWB + (dt / (W / 2)) * (W * 16) + v_off[dt % (W / 2)]));
                const short __attribute__((ext_vector_type(8))) w8 = {h[0][0], h[0][1], h[0][2], h[0][3],
                                                                      h[1][0], h[1][1], h[1][2], h[1][3]};
                return __builtin_bit_cast(bf16x8, w8);
            };
            // k-step by k-step: the K fragments of step k+1 and a share of the
            // V^T fragments are read while the matrix instructions of step k run
            constexpr int VPK = (C::DT + C::KS - 1) / C::KS;     // V^T fragments per k-step
            bf16x8 kc[2] = {kread(0, 0), kread(1, 0)};
#pragma unroll
            for (int k = 0; k < C::KS; ++k) {
                bf16x8 kn[2];
                if (k + 1 < C::KS) {
                    kn[0] = kread(0, k + 1);
                    kn[1] = kread(1, k + 1);
                }
                if constexpr (C::SPREAD && !PAGED) {
                    if (ist >= 0 && k < C::LPW) issue_full(ist, k);
                }
#pragma unroll
                for (int v = 0; v < VPK; ++v)
                    if (k * VPK + v < C::DT) vf[k * VPK + v] = vread(k * VPK + v);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < NT; ++i)
                        sacc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            kc[t], qf[i][k], k == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[i][t], 0, 0, 0);
                if (k + 1 < C::KS) {
                    kc[0] = kn[0];
                    kc[1] = kn[1];
                }
            }
            if constexpr (Q4) {
                dequant(n_slot, n_c, n_buf);

            }
        }

        // raw scores; the softmax scale (log2 units) is applied inside the
        // exponent, so the maxima below are raw too
        float sv[NT][8];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) sv[i][4 * t + j] = sacc[i][t][j];
        if ((abase + 32 > ctx) || (abase + 32 > p1)) {
            const int rel0 = abase + 8 * qd - ctx;          // draft index of value 0
            const int lim = p1 - (abase + 8 * qd);          // values e < lim are in the split
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const uint64_t anc = node_of[i] >= 0 ? anc_s[node_of[i]] : 0ull;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int rel = rel0 + e;
                    bool vis = e < lim;
                    if (rel >= 0) vis = vis && (((anc >> (rel & 63)) & 1ull) != 0ull);
                    sv[i][e] = vis ? sv[i][e] : -INFINITY;
                }
            }
        }
        // lazy rescale: the reference m_ref (log2 units) moves only when some
        // score exceeds it by more than 8; a lane's own 8 values decide
        // whether the wave looks at row maxima at all
        float cm[NT];
        bool grow = false;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            cm[i] = sv[i][0];
#pragma unroll
            for (int e = 1; e < 8; ++e) cm[i] = fmaxf(cm[i], sv[i][e]);
            grow = grow || (cm[i] * p.scale_log2 > m_ref[i] + 8.f);
        }
        if (__any(grow)) {
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                float c = fmaxf(cm[i], xor_shfl(cm[i], 16));
                c = fmaxf(c, xor_shfl(c, 32));
                const float cms = c * p.scale_log2;
                const bool need = cms > m_ref[i] + 8.f;
                const float mn = need ? cms : m_ref[i];
                const float alpha = need ? exp2f(m_ref[i] - mn) : 1.f;
                m_ref[i] = mn;
                l_sum[i] *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) o[i][dt] *= alpha;
            }
        }

        // P = 2^(s * scale - m) (v_exp_f32; results below 2^-126 flush to 0)
        bf16x8 pb[NT];
        auto softmax_tile = [&](int i) {
            const float mu = (m_ref[i] == -INFINITY) ? 0.f : m_ref[i];
            float ls = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i][e], p.scale_log2, -mu));
                ls += pr;
                pb[i][e] = (__bf16)pr;
            }
            l_sum[i] += ls;
        };
        // O^T += V^T P^T, the exponentials of the next tile between the
        // matrix instructions of this one
        softmax_tile(0);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
                o[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pb[i], o[i][dt], 0, 0, 0);
            if (i + 1 < NT) {
                softmax_tile(i + 1);
#pragma unroll
                for (int k = 0; k < C::DT; ++k) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 1);
                }
            }
        }
    };

    // ---- main loop ---------------------------------------------------------
    if constexpr (Q4) {
        // chunks g = 0 .. G-1 of 32 positions, CH per stage.  Staging buffer
        // g % 2 holds chunk g, dequantised during chunk g - 1; one barrier per
        // chunk.  Stage st + 1 is loaded while stage st is consumed.
        const int G = (p1 - p0 + 31) / 32;
        __syncthreads();                                   // stage 0 (waited above) landed everywhere
        dequant(0, 0, 0);
        __syncthreads();
#pragma unroll 1
        for (int g = 0; g < G; ++g) {
            const int st = g / C::CH, c = g % C::CH;
            if (c == 0 && st + 1 < n_st) issue(st + 1);    // slot of stage st - 1: fully dequantised
            if (c == C::CH - 1 && st + 1 < n_st) {
                wait_vm<0>();                              // stage st + 1, dequantised during this chunk
                __syncthreads();
            }
            // the chunk after this one (past the end: this one again, into the idle buffer)
            const int gn = g + 1 < G ? g + 1 : g;
            const uint8_t *Kl = staging + (g & 1) * C::STAGING;
            if (tile_on[0]) {
                compute(-1, Kl, Kl + 32 * C::ROWB, 0, p0 + g * 32, (gn / C::CH) % S, gn % C::CH, (g + 1) & 1);
            } else {
                dequant((gn / C::CH) % S, gn % C::CH, (g + 1) & 1);
            }
            __syncthreads();
        }
    } else {
#pragma unroll 1
        for (int it = 0; it < n_st; ++it) {
            wait_vm_dyn<C::LPW, S - 2>(min(S - 2, n_st - 1 - it));   // this wave's part of stage `it` landed
            __syncthreads();                                           // everyone's part landed; slot it-1 free
            const int ist = it + S - 1 < n_st ? it + S - 1 : -1;   // stage to load into slot it-1
            const uint8_t *Kl = ring + (it % S) * C::STAGE;
            const int cb = pg * 32;
            const int abase = p0 + it * T + cb;
            // a wavefront whose row group has no rows (fewer row tiles than
            // wavefronts) only issues its share of the loads
            if (abase >= p1 || !tile_on[0]) {
                if (ist >= 0) issue(ist);
                continue;
            }
            // a full stage of a contiguous cache goes out over the k-steps;
            // the last stage and paged caches at once
            const bool spread = C::SPREAD && !PAGED && ist >= 0 && p0 + ist * T + T <= p1;
            if (ist >= 0 && !spread) issue(ist);
            compute(spread ? ist : -1, Kl, Kl + C::KBYTES, cb, abase, 0, 0, 0);
        }
    }

    // ---- combine position groups (PG > 1) through LDS --------------------------
    if constexpr (PG > 1) {
        __syncthreads();
        f32x4 *buf = (f32x4 *)ring;
        constexpr int SLOT = C::DT + 1;
        static_assert((PG - 1) * C::RG * NT * SLOT * 64 * 16 <= S * C::STAGE, "combine buffer");
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
            for (int q2 = 1; q2 < PG; ++q2)
                mx = fmaxf(mx, buf[((((q2 - 1) * C::RG + rg) * NT + i) * SLOT + C::DT) * 64 + lane][0]);
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

    // ---- partials of this split --------------------------------------------------
    const int64_t part = wu.part;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if (!tile_on[i]) continue;
        float ls = l_sum[i];
        ls += xor_shfl(ls, 16);
        ls += xor_shfl(ls, 32);
        const int rl = (rg + C::RG * i) * 16 + l16;
        if (rl >= rows_here) continue;
        const int r = row0 + rl;
        float *op = p.part_o + (part * R + r) * D + qd * 4;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            if (p.part_nt) __builtin_nontemporal_store(o[i][dt], (f32x4 *)(op + 16 * dt));
            else *(f32x4 *)(op + 16 * dt) = o[i][dt];
        }
        if (qd == 0) {
            p.part_ml[(part * R + r) * 2 + 0] = m_ref[i];
            p.part_ml[(part * R + r) * 2 + 1] = ls;
        }
    }
}

template <int D, int NT, int PG, bool PAGED, bool Q4, int OCC = 1>
hipError_t launch_one(const AttnParams &p, hipStream_t st) {
    const int grid = ((p.n_units + 7) / 8) * 8 * p.n_rowblocks;
    hipLaunchKernelGGL((attn_dma_kernel<D, NT, PG, PAGED, Q4, OCC>), dim3(grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_shape(const AttnParams &p, int nt, int pg, bool q4, int occ, hipStream_t st) {
    if (occ == 2) {
        // two workgroups per CU (half-size rings): one row tile, stages of <= 16 KB
        if (q4 || nt != 1) return hipErrorInvalidValue;
        if (pg == 1) return launch_one<D, 1, 1, PAGED, false, 2>(p, st);
        if constexpr (D <= 128) {
            if (pg == 2) return launch_one<D, 1, 2, PAGED, false, 2>(p, st);
        }
        return hipErrorInvalidValue;
    }
    if (occ != 1) return hipErrorInvalidValue;
    if (q4) {
        if constexpr (D == 256) {
            if (pg != 1) return hipErrorInvalidValue;
            if (nt == 1) return launch_one<D, 1, 1, PAGED, true>(p, st);
            if (nt == 2) return launch_one<D, 2, 1, PAGED, true>(p, st);
            if (nt == 3) return launch_one<D, 3, 1, PAGED, true>(p, st);
        }
        return hipErrorInvalidValue;
    }
    if (pg == 1) {
        if (nt == 1) return launch_one<D, 1, 1, PAGED, false>(p, st);
        if (nt == 2) return launch_one<D, 2, 1, PAGED, false>(p, st);
        if (nt == 3) return launch_one<D, 3, 1, PAGED, false>(p, st);
    } else if (nt == 1 && pg == 2) {
        return launch_one<D, 1, 2, PAGED, false>(p, st);
    } else if (nt == 1 && pg == 4 && D <= 128) {
        return launch_one<D, 1, (D <= 128 ? 4 : 2), PAGED, false>(p, st);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_d(const AttnParams &p, int nt, int pg, bool q4, int occ, hipStream_t st) {
    return p.kv.page_table != nullptr ? launch_shape<D, true>(p, nt, pg, q4, occ, st)
                                      : launch_shape<D, false>(p, nt, pg, q4, occ, st);
}

}  // namespace

int attn_dma_max_split_pages() { return kMaxSplitPages; }

hipError_t launch_attn_dma(const AttnParams &p, int D, int nt, int pg, bool q4, int occ, hipStream_t st) {
    switch (D) {
        case 64: return launch_d<64>(p, nt, pg, q4, occ, st);
        case 128: return launch_d<128>(p, nt, pg, q4, occ, st);
        case 256: return launch_d<256>(p, nt, pg, q4, occ, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace sv
