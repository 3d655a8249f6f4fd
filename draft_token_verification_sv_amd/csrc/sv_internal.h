// Internal launch parameters shared by the host API (sv_api.cpp) and the HIP
// kernels.  Plain C++ structs passed by value as kernel arguments.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/sv.h"

namespace sv {

// Where one layer of the KV cache lives (see sv_kv_cache in sv.h).
struct KvView {
    const void *k, *v;            // codes / values, layer 0 of this call
    const void *ks, *vs;          // 4-bit scales or nullptr
    const int32_t *page_table;    // nullptr: contiguous
    int64_t capacity;             // positions per (seq, head) or pages in the pool
    int32_t page_size;            // 0: contiguous
    int32_t max_pages;            // page-table row length
};

struct AttnParams {
    KvView kv;
    const void *q;                // [B][N][Hq][D]
    const int32_t *ctx_lens;      // [B]
    const int32_t *parent;        // [B][N]
    float *part_o;                // [unit][R][D]  (unnormalised, scaled to 2^-m)
    float *part_ml;               // [unit][R][2]  (m in log2 units, l)
    void *out;                    // [B][N][Hq][D]
    float *lse;                   // [B][N][Hq] or nullptr
    int B, N, Hq, Hkv, G, R;      // R = G * N packed rows per (b, kv head)
    int max_ctx;
    int n_splits, split_len;      // static schedule: splits per sequence, positions per split
    int dyn;                      // 1: dynamic schedule (split length chosen on the device)
    int units_max;                // dynamic: units the grid covers (= partial slots)
    int split_q, split_min, split_max;   // dynamic: split length quantum and bounds
    int4 *seq_tab;                // dynamic: [B] (first unit, splits, split length, 0)
    int rows_per_block, n_rowblocks;
    int n_units;                  // units the grid covers (without row blocks)
    float scale_log2;             // sm_scale * log2(e)
    int q_f32;                    // 1: q/out are fp32, 0: bf16
    int part_nt;                  // 1: streaming (non-temporal) stores for the partial O
    int part_perm;                // 1: partial O in the 4-bit kernels' slot order: slot s of a
                                  // row holds head dim 8 (s / 8) + pi(s % 8), pi = 0,4,2,6,1,5,3,7
    int window;                   // > 0: only the last `window` key rows of each sequence
    unsigned int *err;            // precondition word (SV_DEBUG builds), else nullptr
};

struct CompactParams {
    KvView kv;
    int64_t layer_stride, scale_layer_stride;   // bytes
    const int32_t *ctx_lens, *path, *accept_len;
    int32_t *new_lens;
    int B, N, Hkv, D, n_layers, max_ctx, dtype;
    unsigned int *err;            // precondition word (SV_DEBUG builds), else nullptr
};

struct AcceptParams {
    const void *logits;           // [B][N][V]
    const int32_t *draft;         // [B][N]
    const int32_t *parent;        // [B][N]
    int32_t *accept_len, *path, *tokens, *argmax;
    unsigned long long *keys;     // [B][N] packed (value, index) maxima  (zero between calls)
    unsigned int *seqs_done;      // [B]    (row, chunk) workgroups done (zero between calls)
    int B, N, V, chunk, n_chunks;
    int logits_f32;
    int compact;                  // also compact the KV of each sequence (cp; path / accept_len unused)
    CompactParams cp;
    const float *gumbel;          // [B][N][V] noise: sample at `temperature` instead of the argmax (or null)
    float temperature;
    int top_k;                    // > 0: sample among each row's top_k logits (launch_topk_accept)
    unsigned int *err;            // precondition word (SV_DEBUG builds), else nullptr
};

struct AppendParams {
    KvView kv;                    // layer 0; k / v (and ks / vs) are written
    const int32_t *ctx_lens;      // [B]
    const void *k_new, *v_new;    // [B][n][Hkv][D], fp32 or bf16
    int B, n, Hkv, D, max_ctx;
    unsigned int *err;            // precondition word (SV_DEBUG builds), else nullptr
};

struct ConvTreeParams {
    const void *x;                // [B][N][C]
    const void *conv_state;       // [B][K-1][C]
    const float *w;               // [C][K]
    const float *bias;            // [C] or nullptr
    const int32_t *parent;        // [B][N] or nullptr (chains)
    void *out;                    // [B][N][C]
    int B, N, C, K, silu;
};

struct DeltaParams {
    const void *q, *k, *v;        // token (b, i) rows at (b * N + i) * stride
    int64_t qk_stride, v_stride;  // elements
    const float *g, *beta;        // [B][N][Hv]
    const float *state;           // [B][Hv][Dv][Dk]
    const int32_t *parent;        // [B][N] or nullptr (chains)
    const int32_t *sched;         // [B][64] order words from tree_schedule_kernel, or nullptr
    void *out;                    // [B][N][Hv][Dv]
    void *state_nodes;            // [B][N][Hv][Dv][Dk]
    int B, N, Hk, Hv, Dv;
    float scale;
};

struct CommitParams {
    const void *state_nodes;      // [B][N][Hv][Dv][Dk], fp32 or f16
    float *state;                 // [B][Hv][Dv][Dk]
    const void *x;                // [B][N][C]
    void *conv_state;             // [B][K-1][C]
    const int32_t *path, *accept_len;
    int64_t state_elems;          // Hv * Dv * Dk
    int B, N, C, K;
    int state_blocks;             // workgroups per sequence on the state copy
};

// Kernel-side tile sizes (positions staged per iteration) -----------------
constexpr int kMfmaTileElems = 16384;          // T * D bf16 elements per K (or V) tile
constexpr int kValuTileElems = 8192;           // T * D fp32 elements per K (or V) tile
constexpr int kMaxSplits = 1024;               // splits per (sequence, KV head, row block)

// Records e as the calling thread's last HIP error; returns SV_EHIP.
int hip_fail(hipError_t e);

// The current device's precondition word (sv_check_device_errors): its
// device address in a build with SV_DEBUG, nullptr otherwise.
unsigned int *device_error_word();

// launchers (return the hipError_t of the launch) -------------------------
hipError_t launch_attn_mfma(const AttnParams &p, int dtype, int D, int nt, int pg, hipStream_t s);
hipError_t launch_attn_dma(const AttnParams &p, int D, int nt, int pg, bool q4, int occ, hipStream_t s);
int attn_dma_max_split_pages();
hipError_t launch_attn_q4c(const AttnParams &p, int nts, hipStream_t s);
hipError_t launch_attn_q4w(const AttnParams &p, int nts, hipStream_t s);
bool attn_q4w_supports(bool paged, int nts);
int attn_q4c_max_split_pages();
hipError_t launch_attn_valu(const AttnParams &p, int dtype, int D, hipStream_t s);
hipError_t launch_attn_merge(const AttnParams &p, int D, hipStream_t s);
hipError_t launch_accept(const AcceptParams &p, hipStream_t s);
hipError_t launch_topk_accept(const AcceptParams &p, hipStream_t s);
hipError_t launch_compact(const CompactParams &p, hipStream_t s);
hipError_t launch_append(const AppendParams &p, int src_dtype, int dst_dtype, hipStream_t s);
hipError_t launch_conv_tree(const ConvTreeParams &p, int dtype, hipStream_t s);
hipError_t launch_delta_tree(const DeltaParams &p, int dtype, int state_dtype, int Dk, hipStream_t s);
hipError_t launch_commit(const CommitParams &p, int state_dtype, int dtype, hipStream_t s);
hipError_t launch_tree_schedule(const int32_t *parent, int B, int N, int32_t *sched, hipStream_t s);

}  // namespace sv
