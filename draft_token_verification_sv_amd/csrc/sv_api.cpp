// Host side of the C ABI declared in include/sv.h: argument validation, launch
// planning and error mapping.  Nothing here allocates device memory or
// synchronises; every kernel goes to the caller's stream.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "attn_sched.h"

namespace sv {
namespace {

thread_local int g_last_hip_error = 0;

// One call's tuning (sv_tuning), validated, zeros meaning the library's choice.
struct Tuning {
    int attn_target_wgs = 0;   // 0: choose by kernel (see plan_attn)
    int attn_rowblocks = 0;    // 0: planner's choice
    int attn_posgroups = 0;    // 0: planner's choice
    int attn_occupancy = 0;    // 0: planner's choice
    int attn_q4_pipelined = 0; // 1: 4-bit head-dim-256 caches on the pipelined bf16-staging kernel
    int attn_q4_four_wave = 0; // 1: 4-bit head-dim-256 caches on the four-wave cooperative kernel
    int argmax_chunk = 0;      // 0: by kernel (see accept_params)
};

// sv_tuning -> Tuning; false for a value out of range
bool read_tuning(const sv_tuning *t, Tuning &out) {
    out = Tuning{};
    if (t == nullptr) return true;
    if (t->attn_target_wgs < 0 || t->attn_rowblocks < 0) return false;
    if (t->attn_posgroups != 0 && t->attn_posgroups != 1 && t->attn_posgroups != 2 && t->attn_posgroups != 4)
        return false;
    if (t->attn_occupancy < 0 || t->attn_occupancy > 2) return false;
    if (t->attn_q4_kernel < 0 || t->attn_q4_kernel > 3) return false;
    if (t->argmax_chunk < 0 || t->argmax_chunk % 8 != 0) return false;
    out.attn_target_wgs = t->attn_target_wgs;
    out.attn_rowblocks = t->attn_rowblocks;
    out.attn_posgroups = t->attn_posgroups;
    out.attn_occupancy = t->attn_occupancy;
    out.attn_q4_pipelined = t->attn_q4_kernel == 2;
    out.attn_q4_four_wave = t->attn_q4_kernel == 1;
    if (t->argmax_chunk > 0) out.argmax_chunk = t->argmax_chunk;
    return true;
}


int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t m) { return ceil_div(a, m) * m; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Validates the cache descriptor against a call touching positions
// [0, max_ctx + n_nodes) of sequences [0, batch).
int check_kv(const sv_kv_cache *kv, int batch, int n_nodes, int max_ctx) {
    if (kv == nullptr) return SV_EINVAL;
    if (kv->dtype != SV_F32 && kv->dtype != SV_BF16 && kv->dtype != SV_Q4) return SV_EINVAL;
    if (kv->n_kv_heads < 1) return SV_EINVAL;
    if (kv->head_dim != 64 && kv->head_dim != 128 && kv->head_dim != 256) return SV_EINVAL;
    if (kv->k == nullptr || kv->v == nullptr) return SV_EINVAL;
    if (!aligned(kv->k, 16) || !aligned(kv->v, 16)) return SV_EINVAL;
    if (kv->dtype == SV_Q4) {
        if (kv->k_scale == nullptr || kv->v_scale == nullptr) return SV_EINVAL;
        if (!aligned(kv->k_scale, 4) || !aligned(kv->v_scale, 4)) return SV_EINVAL;
    }
    if (kv->capacity < 1) return SV_EINVAL;
    const int64_t need = (int64_t)max_ctx + n_nodes;
    if (kv->page_size == 0) {
        if (kv->page_table != nullptr) return SV_EINVAL;
        if (kv->n_seqs < batch) return SV_EINVAL;
        if (kv->capacity < need) return SV_EINVAL;
    } else {
        if (kv->page_size < 0 || kv->page_size % 8 != 0 || kv->page_size > (1 << 20)) return SV_EINVAL;
        if (kv->page_table == nullptr) return SV_EINVAL;
        if (kv->max_pages_per_seq < 1) return SV_EINVAL;
        if ((int64_t)kv->max_pages_per_seq * kv->page_size < need) return SV_EINVAL;
    }
    return SV_OK;
}

KvView view_of(const sv_kv_cache *kv) {
    KvView v;
    v.k = kv->k;
    v.v = kv->v;
    v.ks = kv->k_scale;
    v.vs = kv->v_scale;
    v.page_table = kv->page_size ? kv->page_table : nullptr;
    v.capacity = kv->capacity;
    v.page_size = kv->page_size;
    v.max_pages = kv->max_pages_per_seq;
    return v;
}

enum AttnKind { kValu = 0, kMfmaStaged = 1, kMfmaDma = 2, kQ4Coop = 3 };

struct AttnPlan {
    int kind;
    int nt, pg;
    int occ;                                  // pipelined kernel: workgroups per CU
    int wide;                                 // 4-bit fp16 kernel: eight waves per workgroup
    int rows_per_block, n_rowblocks;
    int n_splits, split_len;                  // static schedule
    int dyn, units, split_q, split_min, split_max;
    size_t o_off, ml_off, tab_off, ws_bytes;
};

// Launch plan for sv_verify_attn.  Work units are (sequence, KV head, row
// block, split of the key positions); the grid holds about `target`
// workgroups (one per CU for the pipelined kernel, whose ring fills most of
// the LDS; two for the others).  A single sequence is split evenly on the host
// (static schedule); a batch, whose lengths are known only on the device,
// gets the dynamic schedule (split length chosen by the kernel from the
// actual lengths, see attn_sched.h).  Row blocks are added while the split
// partials would exceed ~15% of the KV bytes.
//   bf16 queries, >= 16 packed rows:  bf16 KV, 4-bit KV of head dim 256 ->
//                                     direct-to-LDS pipelined kernel
//                                     other 4-bit KV -> register-staged kernel
//   otherwise                         vector-ALU kernel
AttnPlan plan_attn(int kv_dtype, int q_dtype, int D, int B, int N, int Hq, int Hkv, int max_ctx,
                   int page_size, int window, const Tuning &tu) {
    AttnPlan pl{};
    const int G = Hq / Hkv;
    const int R = G * N;
    // the key range of the longest sequence (its last `window` rows with a window)
    const int64_t L = window > 0 ? std::min<int64_t>((int64_t)max_ctx + N, window) : (int64_t)max_ctx + N;
    const bool mfma = (q_dtype == SV_BF16) && (kv_dtype == SV_BF16 || kv_dtype == SV_Q4) && R >= 16;
    // the pipelined kernel takes bf16 caches of any head dim and 4-bit caches of
    // head dim 256; other 4-bit caches go to the register-staged kernel
    const bool q4 = kv_dtype == SV_Q4;
    pl.kind = !mfma ? kValu : ((kv_dtype == SV_BF16 || (q4 && D == 256)) ? kMfmaDma : kMfmaStaged);
    if (pl.kind == kMfmaDma && q4 && !tu.attn_q4_pipelined) pl.kind = kQ4Coop;
    pl.wide = pl.kind == kQ4Coop && !tu.attn_q4_four_wave;
    int target = tu.attn_target_wgs > 0 ? tu.attn_target_wgs : ((pl.kind == kMfmaDma || pl.kind == kQ4Coop) ? 256 : 512);
    pl.occ = 1;
    const double pos_bytes = kv_dtype == SV_F32 ? D * 8.0 : (kv_dtype == SV_BF16 ? D * 4.0 : D * 1.125);
    // the pipelined kernel keeps a split's page ids in LDS
    const int64_t max_split = (pl.kind == kMfmaDma && page_size > 0)
                                  ? (int64_t)(attn_dma_max_split_pages() - 1) * page_size
                                  : ((pl.kind == kQ4Coop && page_size > 0)
                                         ? (int64_t)(attn_q4c_max_split_pages() - 1) * page_size
                                         : ((int64_t)1 << 40));

    // static split lengths: multiples of 8 positions, of the 128-position stage
    // for the pipelined kernel's 4-bit cache
    const int64_t squant = ((pl.kind == kMfmaDma && q4) || pl.kind == kQ4Coop) ? 128 : 8;
    auto splits_for = [&](int units, int &split_len, int &n_splits) {
        const int64_t want = std::max<int64_t>(1, target / std::max(units, 1));
        int64_t sl = round_up(std::max<int64_t>(ceil_div(L, want), 8), squant);
        sl = std::max<int64_t>(sl, round_up(ceil_div(L, kMaxSplits), squant));   // merge keeps <= kMaxSplits weights
        sl = std::min(sl, max_split / squant * squant);
        split_len = (int)sl;
        n_splits = (int)ceil_div(L, split_len);
    };

    // Two workgroups per CU on the pipelined kernel (half-size rings, stages of
    // <= 32 KB, one row tile per wavefront): twice the units balance uneven
    // sequences better and each workgroup's start overlaps the other's work.
    // Default for batches (8 paged sequences of 1K-16K positions: -3 %), for
    // single sequences regrouped into one-tile-per-wavefront blocks (below),
    // and for single sequences of <= 6K keys at the one-per-CU grid (the
    // shallower ring lets the first chunk start once one stage has landed:
    // 24/4 heads, dim 256, 8-row chain at 1K-4K keys -2 to -4 %; at 8K-32K
    // within the spread, at 128K +3.5 %).
    auto occupancy2 = [&](bool single_pair, bool single_short) {
        const bool planned = tu.attn_occupancy == 0 && (B > 1 || single_pair || single_short);
        if (!(planned || tu.attn_occupancy == 2) || pl.kind != kMfmaDma || q4 || pl.nt != 1) return;
        pl.occ = 2;
        pl.pg = std::min(pl.pg, std::max(1, std::min(2, 32768 / (128 * D))));
        // a batch and the regrouped blocks fill two workgroups per CU; a short
        // single sequence keeps the one-per-CU grid (regrouped blocks too:
        // 24/4 heads, dim 256, 16-row chain at 4K keys 22.5 -> 18.8 us)
        const bool keep_grid = planned && B == 1 && (!single_pair || single_short);
        if (tu.attn_target_wgs == 0 && !keep_grid) target = 512;
    };

    // Pipelined bf16 kernel, one sequence (static splits): a split of 4.25
    // stages runs a fifth, nearly empty one; when less than half of the last
    // stage is used, the split is cut to whole stages if the grid still fits
    // the CUs' workgroup slots (256 per workgroup per CU).  Chain of 8 at 4K
    // keys: 136-position splits 16.9 us, 128 16.1-16.4 us.
    auto whole_stages = [&](int groups) {
        if (pl.kind != kMfmaDma || q4 || B != 1) return;
        const int64_t st = 32 * pl.pg;
        const int64_t lo = (int64_t)pl.split_len / st * st;
        if (lo < st || pl.split_len - lo == 0 || pl.split_len - lo >= st / 2) return;
        if (lo < ceil_div(L, kMaxSplits) || (int64_t)groups * ceil_div(L, lo) > 256LL * pl.occ) return;
        pl.split_len = (int)lo;
        pl.n_splits = (int)ceil_div(L, lo);
    };

    if (pl.kind == kQ4Coop) {
        // cooperative 4-bit kernel: blocks of 2 * nts row tiles (nts <= 3),
        // one workgroup per CU
        const int RT = (R + 15) / 16;
        const int nts = RT <= 2 ? 1 : (RT <= 4 ? 2 : 3);
        pl.nt = nts;
        pl.pg = 1;
        pl.rows_per_block = 32 * nts;
        pl.n_rowblocks = (RT + 2 * nts - 1) / (2 * nts);
        if (tu.attn_rowblocks > 0) {
            pl.n_rowblocks = std::max(pl.n_rowblocks, std::min(tu.attn_rowblocks, (RT + 1) / 2));
            const int per = (RT + pl.n_rowblocks - 1) / pl.n_rowblocks;     // tiles per block
            pl.nt = (per + 1) / 2;
            pl.rows_per_block = 32 * pl.nt;
            pl.n_rowblocks = (R + pl.rows_per_block - 1) / pl.rows_per_block;
        }
        // the eight-wave kernel where it takes the block (else the four-wave
        // one): 131072 4-bit keys, 96 rows, 1.3 % faster (129.7 us vs 131.4)
        pl.wide = pl.wide && attn_q4w_supports(page_size > 0, pl.nt);
        splits_for(B * Hkv * pl.n_rowblocks, pl.split_len, pl.n_splits);
    } else if (mfma) {
        const int RT = (R + 15) / 16;
        // row tiles per wave: up to 3 on the pipelined kernel, 2 on the
        // register-staged one
        const int max_tiles = pl.kind == kMfmaDma ? 12 : 8;
        if (RT == 1) {
            pl.pg = pl.kind == kMfmaDma ? (q4 ? 1 : std::min(4, 65536 / (128 * D)))
                                        : std::min(4, (kMfmaTileElems / D) / 32);
            if (tu.attn_posgroups > 0 && pl.kind == kMfmaDma && !q4)
                pl.pg = std::min(tu.attn_posgroups, std::min(4, 65536 / (128 * D)));
            pl.nt = 1;
            pl.rows_per_block = 16;
            pl.n_rowblocks = 1;
            occupancy2(false, false);
            splits_for(B * Hkv, pl.split_len, pl.n_splits);
            whole_stages(B * Hkv);
        } else {
            pl.pg = 1;
            int nrb = (RT + max_tiles - 1) / max_tiles;
            if (tu.attn_rowblocks > 0) nrb = std::max(nrb, std::min(tu.attn_rowblocks, RT));
            // One sequence with more row tiles than wavefronts, 4K-64K keys:
            // blocks of <= 4 tiles (one per wavefront) at two workgroups
            // per CU, so each SIMD runs two wavefronts whose matrix and vector
            // instructions interleave; each block reads the split's KV rows
            // (from L2 after the first).  Measured on the 24/4-head, dim-256
            // tree at 32K: 9 tiles in one block 52.9 us, in 3 blocks 47.9 us;
            // at 8K 38.1 -> 25.8 us; at 128K it loses (135 -> 147 us), where
            // the prologue is amortised and the single block reads KV once,
            // and below 4K too (2K: 18.6 -> 22.7 us), where the splits are few
            // positions long and the extra row blocks only add prologues.
            const bool single_pair = pl.kind == kMfmaDma && !q4 && B == 1 && RT > 4 && L > 4096 && L <= 65536 &&
                                     tu.attn_rowblocks == 0 && tu.attn_occupancy != 1;
            if (single_pair) nrb = (RT + 3) / 4;
            // One short sequence (<= 5K keys) of at most four row tiles: one
            // tile per block, so each block's wavefront runs alone on its
            // SIMD with the split's stages to itself and the splits stay long
            // (24/4 heads, dim 256, 8-row chain: 1K 12.7 -> 11.4 us, 4K 15.2
            // -> 14.8 us, but 6K 16.0 -> 16.3 us; 4-row chain at 4K 15.7 ->
            // 12.7 us)
            const bool single_short = B == 1 && L <= 6144;
            if (pl.kind == kMfmaDma && !q4 && B == 1 && L <= 5120 && RT <= 4 && tu.attn_rowblocks == 0 &&
                tu.attn_occupancy != 1)
                nrb = RT;
            // More row blocks (each reads the same KV tiles, from L2 after the
            // first) shorten the per-split work but multiply the splits, whose
            // fp32 partials the merge reads back.  Added while the partials
            // exceed a fraction of the KV bytes: 35% on the pipelined kernel
            // (whose per-stage cost grows with the tiles per wave), 15% on the
            // register-staged one (measured on the workloads of the bench).
            const double max_part = pl.kind == kMfmaDma ? 0.35 : 0.15;
            for (; tu.attn_rowblocks == 0 && !single_pair;) {
                const int tpb = (RT + nrb - 1) / nrb;
                splits_for(B * Hkv * nrb, pl.split_len, pl.n_splits);
                const double part = (double)pl.n_splits * R * (D + 2) * 4.0;
                const double kvb = (double)L * pos_bytes;
                if (part <= max_part * kvb || tpb <= 2) break;
                ++nrb;
            }
            const int tpb = (RT + nrb - 1) / nrb;
            pl.n_rowblocks = (RT + tpb - 1) / tpb;
            pl.rows_per_block = tpb * 16;
            pl.nt = (tpb + 3) / 4;
            // a block of one or two row tiles leaves wavefronts without rows:
            // they take other positions of a longer stage instead (bf16 cache)
            if (pl.kind == kMfmaDma && !q4 && pl.nt == 1 && tu.attn_posgroups > 0) {
                const int pg_rows = tpb == 1 ? 4 : (tpb == 2 ? 2 : 1);
                pl.pg = std::min(std::min(tu.attn_posgroups, pg_rows), std::min(4, 65536 / (128 * D)));
            }
            occupancy2(single_pair, single_short);
            splits_for(B * Hkv * pl.n_rowblocks, pl.split_len, pl.n_splits);
            whole_stages(B * Hkv * pl.n_rowblocks);
        }
    } else {
        pl.nt = 1;
        pl.pg = 1;
        pl.rows_per_block = 16;
        pl.n_rowblocks = (R + 15) / 16;
        splits_for(B * Hkv * pl.n_rowblocks, pl.split_len, pl.n_splits);
    }

    // One sequence: a key range a little over a multiple of the split length
    // (ctx + N = 64 * 2048 + 16 for 16 draft rows after a 128K context) is
    // rounded up to longer splits, or leaves a nearly empty last one.  For n
    // splits from the planned count up to what the grid holds, splits of
    // floor(L / n) (in whole quanta) whose last one also takes the remainder
    // are used instead when that last split runs fewer chunks than the planned
    // splits (the last split of a plan ends at the key range's end,
    // attn_sched.h).  4-bit 16-row block at 131072 keys: 61 splits of 2176 ->
    // 64 of 2048, the last 2064.
    if (B == 1) {
        const int64_t groups = (int64_t)Hkv * pl.n_rowblocks;
        const int64_t n_cap = std::min<int64_t>(std::max<int64_t>(groups * pl.n_splits, target) / groups, kMaxSplits);
        const int64_t chunk = (pl.kind == kMfmaDma && !q4) ? 32 * pl.pg : 32;
        auto chunks = [&](int64_t len) { return ceil_div(len, chunk); };
        // at least two stages per split: the per-split costs (prologue,
        // partials, merge) outweigh one stage (4-bit, 8 rows at 8K: 36 -> 39 us)
        const int64_t min_sl = 2 * std::max(squant, chunk);
        int64_t best = chunks(pl.split_len), best_sl = 0, best_n = 0;
        for (int64_t n = pl.n_splits; n <= n_cap; ++n) {
            const int64_t sl = L / n / squant * squant;
            if (sl < min_sl) break;
            const int64_t last = L - (n - 1) * sl;           // >= sl
            if (last > max_split || chunks(last) >= best) continue;
            best = chunks(last);
            best_sl = sl;
            best_n = n;
        }
        if (best_n > 0) {
            pl.split_len = (int)best_sl;
            pl.n_splits = (int)best_n;
        }
    }

    int64_t units = (int64_t)B * Hkv * pl.n_splits;
    pl.dyn = B > 1;
    if (pl.dyn) {
        // split lengths: multiples of the kernel's stage (8 positions for the
        // others), at most kMaxSplits splits per sequence, page ids of a split
        // within the pipelined kernel's LDS table
        const int64_t q = pl.kind == kQ4Coop ? 128 : (pl.kind == kMfmaDma ? (q4 ? 128 : 32 * pl.pg) : 8);   // a power of two
        const int64_t smax = std::min(round_up(L, q), max_split / q * q);
        const int64_t smin = std::max<int64_t>(q, round_up(ceil_div(L, kMaxSplits), q));
        pl.split_q = (int)q;
        pl.split_min = (int)smin;
        pl.split_max = (int)std::max(smax, smin);    // smax < smin is rejected by the caller
        units = std::max<int64_t>(target / pl.n_rowblocks, 2 * (int64_t)B * Hkv);
        units = std::max<int64_t>(units, (int64_t)B * Hkv * ceil_div(L, pl.split_max));
        if (smax < smin) pl.split_max = -1;
    }
    pl.units = (int)std::min<int64_t>(units, INT32_MAX / 2);
    const size_t o_bytes = (size_t)units * R * D * 4;
    const size_t ml_bytes = (size_t)units * R * 2 * 4;
    pl.o_off = 0;
    pl.ml_off = (size_t)round_up((int64_t)o_bytes, 256);
    pl.tab_off = pl.ml_off + (size_t)round_up((int64_t)ml_bytes, 256);
    pl.ws_bytes = pl.tab_off + (pl.dyn ? (size_t)round_up((int64_t)B * 16, 256) : 0);
    return pl;
}

int check_attn_shape(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads, int max_ctx) {
    if (batch < 1 || n_nodes < 1 || n_nodes > 64 || n_q_heads < 1 || max_ctx < 0) return SV_EINVAL;
    if (max_ctx > (1 << 30)) return SV_EINVAL;
    if (kv == nullptr || kv->n_kv_heads < 1 || n_q_heads % kv->n_kv_heads != 0) return SV_EINVAL;
    const int64_t rows = (int64_t)(n_q_heads / kv->n_kv_heads) * n_nodes;
    if (rows > 4096) return SV_EUNSUPPORTED;
    return check_kv(kv, batch, n_nodes, max_ctx);
}

}  // namespace
}  // namespace sv

int sv::hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return SV_EHIP;
}

using namespace sv;

extern "C" {

const char *sv_error_string(int code) {
    switch (code) {
        case SV_OK: return "ok";
        case SV_EINVAL: return "invalid argument";
        case SV_EUNSUPPORTED: return "unsupported combination";
        case SV_EWORKSPACE: return "workspace missing or too small";
        case SV_EHIP: return "HIP error";
    }
    return "unknown error code";
}

int sv_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

namespace {

size_t attn_workspace_size(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads, int max_ctx, int window,
                           const sv_tuning *tuning) {
    Tuning tu;
    if (!read_tuning(tuning, tu)) return 0;
    if (check_attn_shape(kv, batch, n_nodes, n_q_heads, max_ctx) != SV_OK) return 0;
    if (window < 0 || (window > 0 && window < n_nodes)) return 0;
    const AttnPlan pl = plan_attn(kv->dtype, SV_BF16, kv->head_dim, batch, n_nodes, n_q_heads,
                                  kv->n_kv_heads, max_ctx, kv->page_size, window, tu);
    const AttnPlan pf = plan_attn(kv->dtype, SV_F32, kv->head_dim, batch, n_nodes, n_q_heads,
                                  kv->n_kv_heads, max_ctx, kv->page_size, window, tu);
    return std::max(pl.ws_bytes, pf.ws_bytes);
}

int verify_attn(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads, const int32_t *ctx_lens, int max_ctx,
                const void *q, int q_dtype, const int32_t *parent, float sm_scale, int window,
                const sv_tuning *tuning, void *out, float *lse, void *workspace, size_t workspace_bytes,
                void *stream) {
    Tuning tu;
    if (!read_tuning(tuning, tu)) return SV_EINVAL;
    int rc = check_attn_shape(kv, batch, n_nodes, n_q_heads, max_ctx);
    if (rc != SV_OK) return rc;
    if (window < 0 || (window > 0 && window < n_nodes)) return SV_EINVAL;
    if (q == nullptr || out == nullptr || ctx_lens == nullptr || parent == nullptr) return SV_EINVAL;
    if (q_dtype != SV_F32 && q_dtype != SV_BF16) return SV_EINVAL;
    if (!aligned(q, 16) || !aligned(out, 16)) return SV_EINVAL;
    if (!isfinite(sm_scale)) return SV_EINVAL;
    if (q_dtype == SV_BF16 && kv->dtype == SV_F32) return SV_EUNSUPPORTED;
    const int D = kv->head_dim;
    const AttnPlan pl = plan_attn(kv->dtype, q_dtype, D, batch, n_nodes, n_q_heads, kv->n_kv_heads, max_ctx,
                                  kv->page_size, window, tu);
    if (pl.dyn ? (batch > kSchedMaxBatch || pl.split_max < 0) : pl.n_splits > kMaxSplits)
        return SV_EUNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < pl.ws_bytes) return SV_EWORKSPACE;
    if (!aligned(workspace, 16)) return SV_EINVAL;

    AttnParams p{};
    p.kv = view_of(kv);
    p.q = q;
    p.ctx_lens = ctx_lens;
    p.parent = parent;
    p.part_o = (float *)((char *)workspace + pl.o_off);
    p.part_ml = (float *)((char *)workspace + pl.ml_off);
    p.seq_tab = pl.dyn ? (int4 *)((char *)workspace + pl.tab_off) : nullptr;
    p.out = out;
    p.lse = lse;
    p.B = batch;
    p.N = n_nodes;
    p.Hq = n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.G = n_q_heads / kv->n_kv_heads;
    p.R = p.G * n_nodes;
    p.max_ctx = max_ctx;
    p.window = window;
    p.n_splits = pl.n_splits;
    p.split_len = pl.split_len;
    p.dyn = pl.dyn;
    p.units_max = pl.units;
    p.split_q = pl.split_q;
    p.split_min = pl.split_min;
    p.split_max = pl.split_max;
    p.rows_per_block = pl.rows_per_block;
    p.n_rowblocks = pl.n_rowblocks;
    p.n_units = pl.units;
    const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)D);
    p.scale_log2 = scale * 1.4426950408889634f;
    p.q_f32 = q_dtype == SV_F32;
    // Small partial sets (a few MB) are written with streaming stores: less to
    // write back from L2 when the split kernel ends, which the merge waits for.
    // Large ones stay cached for the merge (measured: 6 MB -1 us, 34 MB +3 us).
    p.part_nt = pl.ml_off <= ((size_t)8 << 20);
    p.part_perm = pl.kind == kQ4Coop;
    p.err = device_error_word();

    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (pl.kind == kQ4Coop) e = pl.wide ? launch_attn_q4w(p, pl.nt, st) : launch_attn_q4c(p, pl.nt, st);
    else if (pl.kind == kMfmaDma) e = launch_attn_dma(p, D, pl.nt, pl.pg, kv->dtype == SV_Q4, pl.occ, st);
    else if (pl.kind == kMfmaStaged) e = launch_attn_mfma(p, kv->dtype, D, pl.nt, pl.pg, st);
    else e = launch_attn_valu(p, kv->dtype, D, st);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_attn_merge(p, D, st);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

}  // namespace

namespace {

// Split partials of sv_verify_attn_noalloc: a static buffer in device memory,
// one copy per GPU (each device that loads the library holds it until the
// process ends).  In host code `scratch` is only a stand-in for the symbol;
// its device address on each GPU comes from hipGetSymbolAddress, looked up
// once per device with that device current and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = (size_t)SV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's copy of `scratch`, or nullptr (HIP error recorded).
void *device_scratch() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        hip_fail(e);
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxScratchDevices) {
        hip_fail(hipErrorInvalidDevice);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int sv_verify_attn_noalloc(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                           const int32_t *ctx_lens, int max_ctx,
                           const void *q, int q_dtype, const int32_t *parent, float sm_scale, int window,
                           void *out, float *lse, void *stream) {
    // argument and size checks first: a call that cannot run touches no device
    int rc = check_attn_shape(kv, batch, n_nodes, n_q_heads, max_ctx);
    if (rc != SV_OK) return rc;
    if (window < 0 || (window > 0 && window < n_nodes)) return SV_EINVAL;
    if (q_dtype != SV_F32 && q_dtype != SV_BF16) return SV_EINVAL;
    const AttnPlan pl = plan_attn(kv->dtype, q_dtype, kv->head_dim, batch, n_nodes, n_q_heads, kv->n_kv_heads,
                                  max_ctx, kv->page_size, window, Tuning{});
    if (pl.ws_bytes > kScratchBytes) return SV_EWORKSPACE;
    void *ws = device_scratch();
    if (ws == nullptr) return SV_EHIP;
    return verify_attn(kv, batch, n_nodes, n_q_heads, ctx_lens, max_ctx, q, q_dtype, parent, sm_scale, window,
                       nullptr, out, lse, ws, kScratchBytes, stream);
}

size_t sv_verify_attn_workspace_size(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                                     int max_ctx) {
    return attn_workspace_size(kv, batch, n_nodes, n_q_heads, max_ctx, 0, nullptr);
}

int sv_verify_attn(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                   const int32_t *ctx_lens, int max_ctx,
                   const void *q, int q_dtype, const int32_t *parent, float sm_scale,
                   void *out, float *lse,
                   void *workspace, size_t workspace_bytes, void *stream) {
    return verify_attn(kv, batch, n_nodes, n_q_heads, ctx_lens, max_ctx, q, q_dtype, parent, sm_scale, 0, nullptr,
                       out, lse, workspace, workspace_bytes, stream);
}

size_t sv_verify_attn_window_workspace_size(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                                            int max_ctx, int window) {
    return attn_workspace_size(kv, batch, n_nodes, n_q_heads, max_ctx, window, nullptr);
}

int sv_verify_attn_window(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                          const int32_t *ctx_lens, int max_ctx,
                          const void *q, int q_dtype, const int32_t *parent, float sm_scale, int window,
                          void *out, float *lse,
                          void *workspace, size_t workspace_bytes, void *stream) {
    return verify_attn(kv, batch, n_nodes, n_q_heads, ctx_lens, max_ctx, q, q_dtype, parent, sm_scale, window,
                       nullptr, out, lse, workspace, workspace_bytes, stream);
}

size_t sv_verify_attn_tuned_workspace_size(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                                           int max_ctx, int window, const sv_tuning *tuning) {
    return attn_workspace_size(kv, batch, n_nodes, n_q_heads, max_ctx, window, tuning);
}

int sv_verify_attn_tuned(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                         const int32_t *ctx_lens, int max_ctx,
                         const void *q, int q_dtype, const int32_t *parent, float sm_scale, int window,
                         const sv_tuning *tuning, void *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream) {
    return verify_attn(kv, batch, n_nodes, n_q_heads, ctx_lens, max_ctx, q, q_dtype, parent, sm_scale, window,
                       tuning, out, lse, workspace, workspace_bytes, stream);
}

size_t sv_greedy_accept_workspace_size(int batch, int n_nodes, int vocab) {
    if (batch < 1 || n_nodes < 1 || n_nodes > 64 || vocab < 1) return 0;
    const int64_t rows = (int64_t)batch * n_nodes;
    return (size_t)(round_up(rows * 8, 256) + round_up((int64_t)batch * 4, 256));
}

}  // extern "C"

namespace {

// argument checks and parameters of an acceptance launch
int accept_params(int batch, int n_nodes, int vocab, const void *logits, int logits_dtype,
                  const int32_t *draft_ids, const int32_t *parent, int32_t *accept_len, int32_t *path,
                  int32_t *tokens, int32_t *argmax, void *workspace, size_t workspace_bytes, AcceptParams &p,
                  bool sampled, const sv_tuning *tuning = nullptr) {
    Tuning tu;
    if (!read_tuning(tuning, tu)) return SV_EINVAL;
    // logits per workgroup: greedy bf16 rows 32768 (one group of 16 loads per
    // thread; 16 rows of 151936: 9.0 -> 7.5 us with the 16-bit codes),
    // otherwise 16384
    if (tu.argmax_chunk == 0) tu.argmax_chunk = (!sampled && logits_dtype == SV_BF16) ? 32768 : 16384;
    if (batch < 1 || n_nodes < 1 || n_nodes > 64 || vocab < 1) return SV_EINVAL;
    if (logits == nullptr || draft_ids == nullptr || parent == nullptr || accept_len == nullptr ||
        path == nullptr || tokens == nullptr)
        return SV_EINVAL;
    if (logits_dtype != SV_F32 && logits_dtype != SV_BF16) return SV_EINVAL;
    const int64_t chunks = ceil_div(vocab, tu.argmax_chunk);
    if ((int64_t)batch * n_nodes * chunks > (int64_t)INT32_MAX) return SV_EUNSUPPORTED;
    const size_t need = sv_greedy_accept_workspace_size(batch, n_nodes, vocab);
    if (workspace == nullptr || workspace_bytes < need) return SV_EWORKSPACE;
    if (!aligned(workspace, 16)) return SV_EINVAL;
    p = AcceptParams{};
    p.logits = logits;
    p.draft = draft_ids;
    p.parent = parent;
    p.accept_len = accept_len;
    p.path = path;
    p.tokens = tokens;
    p.argmax = argmax;
    const int64_t rows = (int64_t)batch * n_nodes;
    p.keys = (unsigned long long *)workspace;
    p.seqs_done = (unsigned int *)((char *)workspace + round_up(rows * 8, 256));
    p.B = batch;
    p.N = n_nodes;
    p.V = vocab;
    p.chunk = tu.argmax_chunk;
    p.err = device_error_word();
    p.n_chunks = (int)chunks;
    p.logits_f32 = logits_dtype == SV_F32;
    return SV_OK;
}

// argument checks and parameters of a compaction (path / accept_len may be
// null when the fused call produces them)
int compact_params(const sv_kv_cache *kv, int n_layers, int batch, int n_nodes, const int32_t *ctx_lens,
                   int max_ctx, const int32_t *path, const int32_t *accept_len, int32_t *new_lens, bool fused,
                   CompactParams &p) {
    if (n_layers < 1 || batch < 1 || n_nodes < 1 || n_nodes > 64 || max_ctx < 0) return SV_EINVAL;
    if (max_ctx > (1 << 30)) return SV_EINVAL;
    const int rc = check_kv(kv, batch, n_nodes, max_ctx);
    if (rc != SV_OK) return rc;
    if (ctx_lens == nullptr || (!fused && (path == nullptr || accept_len == nullptr))) return SV_EINVAL;
    if (n_layers > 1 && (kv->layer_stride == 0 ||
                         (kv->dtype == SV_Q4 && kv->scale_layer_stride == 0)))
        return SV_EINVAL;
    if (kv->layer_stride % 16 != 0 || kv->scale_layer_stride % 4 != 0) return SV_EINVAL;
    if ((int64_t)batch * n_layers * kv->n_kv_heads * 2 > (int64_t)INT32_MAX) return SV_EUNSUPPORTED;
    p = CompactParams{};
    p.kv = view_of(kv);
    p.layer_stride = kv->layer_stride;
    p.scale_layer_stride = kv->scale_layer_stride;
    p.ctx_lens = ctx_lens;
    p.path = path;
    p.accept_len = accept_len;
    p.new_lens = new_lens;
    p.B = batch;
    p.N = n_nodes;
    p.Hkv = kv->n_kv_heads;
    p.D = kv->head_dim;
    p.n_layers = n_layers;
    p.max_ctx = max_ctx;
    p.dtype = kv->dtype;
    p.err = device_error_word();
    return SV_OK;
}

}  // namespace

extern "C" {

int sv_greedy_accept(int batch, int n_nodes, int vocab,
                     const void *logits, int logits_dtype,
                     const int32_t *draft_ids, const int32_t *parent,
                     int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *argmax,
                     void *workspace, size_t workspace_bytes, void *stream) {
    AcceptParams p;
    const int rc = accept_params(batch, n_nodes, vocab, logits, logits_dtype, draft_ids, parent, accept_len, path,
                                 tokens, argmax, workspace, workspace_bytes, p, false);
    if (rc != SV_OK) return rc;
    const hipError_t e = launch_accept(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_greedy_accept_tuned(int batch, int n_nodes, int vocab,
                           const void *logits, int logits_dtype,
                           const int32_t *draft_ids, const int32_t *parent,
                           int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *argmax,
                           const sv_tuning *tuning, void *workspace, size_t workspace_bytes, void *stream) {
    AcceptParams p;
    const int rc = accept_params(batch, n_nodes, vocab, logits, logits_dtype, draft_ids, parent, accept_len, path,
                                 tokens, argmax, workspace, workspace_bytes, p, false, tuning);
    if (rc != SV_OK) return rc;
    const hipError_t e = launch_accept(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_kv_compact(const sv_kv_cache *kv, int n_layers, int batch, int n_nodes,
                  const int32_t *ctx_lens, int max_ctx,
                  const int32_t *path, const int32_t *accept_len,
                  int32_t *new_lens, void *stream) {
    CompactParams p;
    const int rc = compact_params(kv, n_layers, batch, n_nodes, ctx_lens, max_ctx, path, accept_len, new_lens,
                                  false, p);
    if (rc != SV_OK) return rc;
    const hipError_t e = launch_compact(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_kv_append(const sv_kv_cache *kv, int batch, int n_rows, const int32_t *ctx_lens, int max_ctx,
                 const void *k_new, const void *v_new, int src_dtype, void *stream) {
    if (batch < 1 || n_rows < 1 || n_rows > 64 || max_ctx < 0 || max_ctx > (1 << 30)) return SV_EINVAL;
    const int rc = check_kv(kv, batch, n_rows, max_ctx);
    if (rc != SV_OK) return rc;
    if (ctx_lens == nullptr || k_new == nullptr || v_new == nullptr) return SV_EINVAL;
    if (src_dtype != SV_F32 && src_dtype != SV_BF16) return SV_EINVAL;
    if (!aligned(k_new, 16) || !aligned(v_new, 16)) return SV_EINVAL;
    if ((int64_t)batch * n_rows * kv->n_kv_heads * 2 / 4 + 1 > (int64_t)INT32_MAX) return SV_EUNSUPPORTED;
    AppendParams p{};
    p.kv = view_of(kv);
    p.ctx_lens = ctx_lens;
    p.k_new = k_new;
    p.v_new = v_new;
    p.B = batch;
    p.n = n_rows;
    p.Hkv = kv->n_kv_heads;
    p.D = kv->head_dim;
    p.max_ctx = max_ctx;
    p.err = device_error_word();
    const hipError_t e = launch_append(p, src_dtype, kv->dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_sample_accept(int batch, int n_nodes, int vocab,
                     const void *logits, int logits_dtype, const float *gumbel, float temperature,
                     const int32_t *draft_ids, const int32_t *parent,
                     int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *sampled,
                     void *workspace, size_t workspace_bytes, void *stream) {
    AcceptParams p;
    const int rc = accept_params(batch, n_nodes, vocab, logits, logits_dtype, draft_ids, parent, accept_len, path,
                                 tokens, sampled, workspace, workspace_bytes, p, true);
    if (rc != SV_OK) return rc;
    if (gumbel == nullptr || !aligned(gumbel, 4)) return SV_EINVAL;
    if (!(temperature > 0.f) || !isfinite(temperature)) return SV_EINVAL;
    p.gumbel = gumbel;
    p.temperature = temperature;
    const hipError_t e = launch_accept(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_sample_accept_topk(int batch, int n_nodes, int vocab,
                          const void *logits, int logits_dtype, const float *gumbel, float temperature, int top_k,
                          const int32_t *draft_ids, const int32_t *parent,
                          int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *sampled,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if (top_k <= 0 || top_k >= vocab)
        return sv_sample_accept(batch, n_nodes, vocab, logits, logits_dtype, gumbel, temperature, draft_ids, parent,
                                accept_len, path, tokens, sampled, workspace, workspace_bytes, stream);
    AcceptParams p;
    const int rc = accept_params(batch, n_nodes, vocab, logits, logits_dtype, draft_ids, parent, accept_len, path,
                                 tokens, sampled, workspace, workspace_bytes, p, true);
    if (rc != SV_OK) return rc;
    if (gumbel == nullptr || !aligned(gumbel, 4)) return SV_EINVAL;
    if (!(temperature > 0.f) || !isfinite(temperature)) return SV_EINVAL;
    if (top_k > 1024) return SV_EUNSUPPORTED;
    p.gumbel = gumbel;
    p.temperature = temperature;
    p.top_k = top_k;
    const hipError_t e = launch_topk_accept(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_greedy_accept_compact(int batch, int n_nodes, int vocab,
                             const void *logits, int logits_dtype,
                             const int32_t *draft_ids, const int32_t *parent,
                             int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *argmax,
                             const sv_kv_cache *kv, int n_layers, const int32_t *ctx_lens, int max_ctx,
                             int32_t *new_lens, void *workspace, size_t workspace_bytes, void *stream) {
    AcceptParams p;
    int rc = accept_params(batch, n_nodes, vocab, logits, logits_dtype, draft_ids, parent, accept_len, path, tokens,
                           argmax, workspace, workspace_bytes, p, false);
    if (rc != SV_OK) return rc;
    rc = compact_params(kv, n_layers, batch, n_nodes, ctx_lens, max_ctx, nullptr, nullptr, new_lens, true, p.cp);
    if (rc != SV_OK) return rc;
    p.compact = 1;
    const hipError_t e = launch_accept(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_ssm_conv_tree(int batch, int n_nodes, int channels, int kernel_width,
                     const void *x, const void *conv_state, int dtype,
                     const float *weight, const float *bias, const int32_t *parent,
                     int activation, void *out, void *stream) {
    if (batch < 1 || batch > 65535 || n_nodes < 1 || n_nodes > 64) return SV_EINVAL;
    if (channels < 4 || channels % 4 != 0 || kernel_width < 2 || kernel_width > 4) return SV_EINVAL;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EINVAL;
    if (activation != 0 && activation != 1) return SV_EINVAL;
    if (x == nullptr || conv_state == nullptr || weight == nullptr || out == nullptr) return SV_EINVAL;
    if (!aligned(x, 16) || !aligned(conv_state, 16) || !aligned(out, 16) || !aligned(weight, 16)) return SV_EINVAL;
    if (bias != nullptr && !aligned(bias, 16)) return SV_EINVAL;
    if (parent != nullptr && !aligned(parent, 4)) return SV_EINVAL;
    ConvTreeParams p{};
    p.x = x;
    p.conv_state = conv_state;
    p.w = weight;
    p.bias = bias;
    p.parent = parent;
    p.out = out;
    p.B = batch;
    p.N = n_nodes;
    p.C = channels;
    p.K = kernel_width;
    p.silu = activation;
    const hipError_t e = launch_conv_tree(p, dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_tree_schedule(int batch, int n_nodes, const int32_t *parent, int32_t *schedule, void *stream) {
    if (batch < 1 || batch > 65535 || n_nodes < 1 || n_nodes > 64) return SV_EINVAL;
    if (parent == nullptr || schedule == nullptr || !aligned(parent, 4) || !aligned(schedule, 4)) return SV_EINVAL;
    const hipError_t e = launch_tree_schedule(parent, batch, n_nodes, schedule, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_gated_delta_net_tree(int batch, int n_nodes, int n_k_heads, int n_v_heads, int k_dim, int v_dim,
                            const void *q, const void *k, const void *v, int64_t qk_stride, int64_t v_stride,
                            int dtype, const float *g, const float *beta, const float *state,
                            const int32_t *parent, const int32_t *schedule, float scale, void *out,
                            void *state_nodes, int state_dtype, void *stream) {
    if (batch < 1 || batch > 65535 || n_nodes < 1 || n_nodes > 64) return SV_EINVAL;
    if (n_k_heads < 1 || n_v_heads < 1 || n_v_heads > 65535 || n_v_heads % n_k_heads != 0) return SV_EINVAL;
    if (k_dim != 64 && k_dim != 128) return SV_EUNSUPPORTED;
    if (v_dim < 32 || v_dim % 32 != 0 || v_dim > 32 * 65535) return SV_EINVAL;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EINVAL;
    if (state_dtype != SV_F32 && state_dtype != SV_F16) return SV_EINVAL;
    if (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr || state == nullptr ||
        out == nullptr || state_nodes == nullptr)
        return SV_EINVAL;
    const int64_t qk_min = (int64_t)n_k_heads * k_dim, v_min = (int64_t)n_v_heads * v_dim;
    if (qk_stride == 0) qk_stride = qk_min;
    if (v_stride == 0) v_stride = v_min;
    if (qk_stride < qk_min || v_stride < v_min || qk_stride % 8 != 0 || v_stride % 8 != 0) return SV_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16) ||
        !aligned(state_nodes, 16) || !aligned(g, 4) || !aligned(beta, 4) || !aligned(out, 4))
        return SV_EINVAL;
    if (parent != nullptr && !aligned(parent, 4)) return SV_EINVAL;
    if (schedule != nullptr && !aligned(schedule, 4)) return SV_EINVAL;
    if (!isfinite(scale)) return SV_EINVAL;
    if ((uint64_t)n_nodes * n_v_heads * v_dim * k_dim > 0xFFFFFFFFull) return SV_EUNSUPPORTED;
    DeltaParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.qk_stride = qk_stride;
    p.v_stride = v_stride;
    p.g = g;
    p.beta = beta;
    p.state = state;
    p.parent = parent;
    p.sched = schedule;
    p.out = out;
    p.state_nodes = state_nodes;
    p.B = batch;
    p.N = n_nodes;
    p.Hk = n_k_heads;
    p.Hv = n_v_heads;
    p.Dv = v_dim;
    p.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)k_dim);
    const hipError_t e = launch_delta_tree(p, dtype, state_dtype, k_dim, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

int sv_recurrent_commit(int batch, int n_nodes, int n_v_heads, int k_dim, int v_dim,
                        const void *state_nodes, int state_dtype, float *state,
                        int channels, int kernel_width, const void *x, void *conv_state, int dtype,
                        const int32_t *path, const int32_t *accept_len, void *stream) {
    if (batch < 1 || batch > 65535 || n_nodes < 1 || n_nodes > 64) return SV_EINVAL;
    if (n_v_heads < 1 || (k_dim != 64 && k_dim != 128) || v_dim < 32 || v_dim % 32 != 0) return SV_EINVAL;
    if (state_dtype != SV_F32 && state_dtype != SV_F16) return SV_EINVAL;
    if (channels < 4 || channels % 4 != 0 || kernel_width < 2 || kernel_width > 4) return SV_EINVAL;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EINVAL;
    if (state_nodes == nullptr || state == nullptr || x == nullptr || conv_state == nullptr || path == nullptr ||
        accept_len == nullptr)
        return SV_EINVAL;
    if (!aligned(state_nodes, 16) || !aligned(state, 16) || !aligned(x, 16) || !aligned(conv_state, 16) ||
        !aligned(path, 4) || !aligned(accept_len, 4))
        return SV_EINVAL;
    const int64_t elems = (int64_t)n_v_heads * v_dim * k_dim;
    // workgroups per sequence on the state copy: about 1024 in all, each copying
    // at least 2048 values
    const int64_t blocks = std::min<int64_t>((elems / 8 + 255) / 256, std::max(8, 1024 / batch));
    if (blocks + (channels + 1023) / 1024 > (int64_t)INT32_MAX) return SV_EUNSUPPORTED;
    CommitParams p{};
    p.state_nodes = state_nodes;
    p.state = state;
    p.x = x;
    p.conv_state = conv_state;
    p.path = path;
    p.accept_len = accept_len;
    p.state_elems = elems;
    p.B = batch;
    p.N = n_nodes;
    p.C = channels;
    p.K = kernel_width;
    p.state_blocks = (int)blocks;
    const hipError_t e = launch_commit(p, state_dtype, dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SV_OK;
}

}  // extern "C"
