/*
 * sv.h -- the verify step of speculative decoding on one AMD MI355X (gfx950).
 *
 * Three calls verify a draft (a chain or a token tree) against the target
 * model, for one layer's KV cache at a time:
 *
 *   sv_verify_attn    tree- or chain-masked GQA attention of the N verify rows
 *                     over the KV cache (contiguous, paged or 4-bit);
 *   sv_greedy_accept  per-row argmax of the target logits, greedy acceptance of
 *                     the longest root path whose drafts equal their parent's
 *                     argmax, plus the bonus token;
 *   sv_kv_compact     in-place compaction of the accepted rows' KV so that only
 *                     the accepted path remains;
 *   sv_greedy_accept_compact  the last two in one launch;
 *   sv_kv_append      the verify block's K/V rows written into the cache
 *                     (quantised at write time for a 4-bit cache);
 *   sv_verify_attn_window  the attention over a sliding window of keys;
 *   sv_sample_accept  stochastic verification at a temperature (and
 *                     sv_sample_accept_topk over each row's top-k tokens);
 *   sv_ssm_conv_tree, sv_gated_delta_net_tree, sv_recurrent_commit
 *                     the tree-aware recurrent state of a hybrid target's
 *                     Gated DeltaNet layers.
 *
 * Sources (web pages on speculative decoding; citations name page and section):
 *   [DFN]  "Making Qwen3.5-27B token generation 6x faster on one RTX 3090"
 *          (blog.xiaohack.org): greedy verify of 16-row DFlash blocks
 *          ("Architecture"), DDTree verification of budget+1 rows ("From
 *          autoregressive to DDTree", "Key breakthroughs"), compaction after
 *          a sibling branch is accepted ("Key breakthroughs"), flash attention
 *          reading a 4-bit KV cache at 128K context ("128K context in 24 GB").
 *   [XDN]  xdnf.cn notes on Qwen3.8-27B speculative decoding: 16-token KV pages
 *          (section 2); the draft block's causal mask must be aligned to the
 *          end of the keys (section 5.3).
 *   [KWK]  kwkr.cn RTX-4080 notes: rolling back rejected draft KV (section 3.3).
 *
 * Conventions used by every call
 * ------------------------------
 *  - Pointers named "device" point to GPU memory owned by the caller; the
 *    library keeps no pointer after a call returns.  Host pointers are read
 *    during the call only.
 *  - N (n_nodes) is the number of verify rows INCLUDING the root: row 0 is the
 *    last committed token, rows 1..N-1 are drafts.  1 <= N <= 64.
 *  - parent[b][i] (device int32 [batch][N]): parent[b][0] = -1 and
 *    0 <= parent[b][i] < i for i >= 1 (a chain has parent[i] = i - 1).  An
 *    entry that breaks this rule is treated as the end of the node's path
 *    (never read out of bounds, result unspecified).
 *  - ctx_lens[b] (device int32 [batch]) counts the cached tokens before the
 *    verify block.  The N verify rows' K/V are already in the cache at logical
 *    positions ctx .. ctx+N-1 in node order (written by the caller, quantised
 *    for a 4-bit cache).  Values above max_ctx are clamped to max_ctx, negative
 *    ones to 0.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream); outputs are valid once the stream has been synchronised.  The
 *    library never synchronises and never allocates device memory.
 *  - Return codes: SV_OK, or a negative SV_E* code; on SV_EHIP the HIP error is
 *    available from sv_last_hip_error() (per thread).  Argument errors are
 *    detected on the host before anything is launched.
 */
#ifndef SV_H
#define SV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_OK            0
#define SV_EINVAL       -1   /* bad argument (null pointer, size, dtype, layout) */
#define SV_EUNSUPPORTED -2   /* valid but not implemented combination            */
#define SV_EWORKSPACE   -3   /* workspace missing or smaller than required      */
#define SV_EHIP         -4   /* a HIP call or kernel launch failed              */

#define SV_F32  0            /* IEEE binary32                                     */
#define SV_BF16 1            /* bfloat16                                          */
#define SV_Q4   2            /* 4-bit KV blocks: see sv_kv_cache                  */
#define SV_F16  3            /* IEEE binary16 (per-node recurrent states)         */

/*
 * KV cache descriptor (one layer is read by sv_verify_attn; sv_kv_compact walks
 * n_layers layers spaced layer_stride bytes apart).
 *
 * Row = one (sequence, KV head, position): head_dim values.
 *   SV_F32 / SV_BF16: k, v hold the values, head_dim per row.
 *   SV_Q4 [DFN "128K context in 24 GB"]: k, v hold 4-bit codes, head_dim/2
 *     bytes per row; value 2t of a row is the low nibble of byte t, value 2t+1
 *     the high nibble.  k_scale, v_scale hold one IEEE-half scale per 32
 *     consecutive values (head_dim/32 per row).  Value i of a row is
 *     scale[i/32] * (code_i - 8).
 * Layout (page_size == 0, contiguous): row (b, h, p) is row number
 *     (b * n_kv_heads + h) * capacity + p   of each array.
 * Layout (page_size > 0, paged) [XDN section 2]: page_table[b][p / page_size]
 *     names the physical page of logical position p of sequence b; row
 *     (b, h, p) is row number (page * n_kv_heads + h) * page_size + p % page_size.
 *     Page ids outside [0, capacity) are read as zero rows and never written.
 */
typedef struct sv_kv_cache {
    int32_t dtype;              /* SV_F32, SV_BF16 or SV_Q4                         */
    int32_t n_kv_heads;         /* >= 1                                             */
    int32_t head_dim;           /* 64, 128 or 256                                   */
    int32_t page_size;          /* 0: contiguous; else tokens per page (multiple of 8) */
    int64_t capacity;           /* contiguous: positions per (seq, head); paged: pages in the pool */
    int32_t n_seqs;             /* contiguous: sequences held (>= batch); paged: unused */
    int32_t max_pages_per_seq;  /* paged: row length of page_table                  */
    void *k;                    /* device, layer 0                                  */
    void *v;                    /* device, layer 0                                  */
    void *k_scale;              /* device, SV_Q4 only (else NULL)                   */
    void *v_scale;              /* device, SV_Q4 only (else NULL)                   */
    const int32_t *page_table;  /* device int32 [batch][max_pages_per_seq], paged only */
    int64_t layer_stride;       /* bytes between layers in k and v                  */
    int64_t scale_layer_stride; /* bytes between layers in k_scale and v_scale      */
} sv_kv_cache;

/*
 * sv_verify_attn -- masked GQA attention of the verify rows.
 *
 * For sequence b, query head h (KV head h / (n_q_heads / n_kv_heads)) and
 * verify row i, with keys/values at logical positions j in [0, ctx + N):
 *   visible(i, j)  = j < ctx, or j - ctx is node i or one of its ancestors
 *                    (for a chain: row i sees ctx + 0..i, the causal mask
 *                    aligned to the end of the keys [XDN section 5.3]; for a
 *                    DDTree the ancestor mask [DFN "From autoregressive to
 *                    DDTree"]);
 *   out[b][i][h]   = sum_j softmax_visible(sm_scale * q . k_j) v_j;
 *   lse[b][i][h]   = ln sum_visible exp(sm_scale * q . k_j).
 *
 * q    device [batch][N][n_q_heads][head_dim], q_dtype SV_F32 or SV_BF16.
 * out  device, same shape and dtype as q (bf16 rounded to nearest even).
 * lse  device float [batch][N][n_q_heads], or NULL.
 * sm_scale  <= 0 selects 1/sqrt(head_dim).
 * max_ctx   host int >= every ctx_lens[b]; sizes the launch.  The cache must
 *           hold max_ctx + N positions per sequence (contiguous: capacity;
 *           paged: max_pages_per_seq * page_size).
 * workspace device scratch of at least sv_verify_attn_workspace_size() bytes
 *           (any contents; 256-byte aligned).  One workspace serves one
 *           stream at a time.
 * batch     at most 1024 (SV_EUNSUPPORTED beyond).  For batch > 1 the kernels
 *           choose the key-split length on the device from ctx_lens, so the
 *           work per workgroup follows the actual lengths rather than max_ctx.
 * Supported: q SV_BF16 with KV SV_BF16 or SV_Q4 (matrix cores when
 * (n_q_heads/n_kv_heads) * N >= 16 rows -- bf16, or fp16 for a 4-bit cache of
 * head dim 256, whose values d * (n - 8) are then rounded to fp16 and whose
 * query rows are scaled by a power of two into fp16's range; vector ALU
 * otherwise); q SV_F32 with KV SV_F32, SV_BF16 or SV_Q4 (vector ALU, fp32
 * arithmetic).
 */
size_t sv_verify_attn_workspace_size(const sv_kv_cache *kv, int batch, int n_nodes,
                                     int n_q_heads, int max_ctx);
int sv_verify_attn(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                   const int32_t *ctx_lens, int max_ctx,
                   const void *q, int q_dtype, const int32_t *parent, float sm_scale,
                   void *out, float *lse,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_verify_attn_window -- sv_verify_attn over a sliding window [DFN, the
 * 60K-context addendum: flash attention over only the most recent 2,048 KV
 * positions instead of the whole context].  The key range of sequence b is
 * cut to its last `window` rows, [max(0, ctx_b + N - window), ctx_b + N), for
 * every verify row of the block alike; the tree mask applies as before.
 * N <= window (the draft rows always stay inside); window = 0 is
 * sv_verify_attn.  Anything else as sv_verify_attn, with the workspace sized
 * by sv_verify_attn_window_workspace_size (0 for invalid arguments).
 */
size_t sv_verify_attn_window_workspace_size(const sv_kv_cache *kv, int batch, int n_nodes,
                                            int n_q_heads, int max_ctx, int window);
int sv_verify_attn_window(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                          const int32_t *ctx_lens, int max_ctx,
                          const void *q, int q_dtype, const int32_t *parent, float sm_scale, int window,
                          void *out, float *lse,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_verify_attn_noalloc -- sv_verify_attn_window (window 0 = the whole key
 * range) with no workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid allocation.  The split partials go to a static buffer of
 * SV_NOALLOC_SCRATCH_BYTES (32 MiB) in device memory, one per GPU, that the
 * library holds from its first use on that GPU until the process ends; the
 * call allocates and frees nothing.  A call whose launch plan needs more than
 * that (sv_verify_attn_window_workspace_size tells in advance) returns
 * SV_EWORKSPACE before touching the device.  The buffer needs no clearing
 * (the partials are written before they are read within each call), but
 * every call on one GPU shares it: calls that may overlap on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * Arguments, results and errors otherwise as sv_verify_attn_window.
 */
#define SV_NOALLOC_SCRATCH_BYTES (32u << 20)
int sv_verify_attn_noalloc(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                           const int32_t *ctx_lens, int max_ctx,
                           const void *q, int q_dtype, const int32_t *parent, float sm_scale, int window,
                           void *out, float *lse, void *stream);

/*
 * sv_greedy_accept -- greedy acceptance [DFN "Architecture": greedy verify;
 * "From autoregressive to DDTree": longest accepted root path].
 *
 * logits    device [batch][N][vocab], SV_F32 or SV_BF16 (finite values).  Row i
 *           holds the target's logits after node i (N = budget + 1 rows for a
 *           DDTree [DFN "Key breakthroughs"]).
 * draft_ids device int32 [batch][N]; entry 0 (the committed token) is ignored.
 * am[b][i]  = lowest index of the maximum of row (b, i), compared in fp32.
 * Node i is accepted iff its parent is accepted and draft_ids[b][i] ==
 * am[b][parent[b][i]] (node 0 always).  The deepest accepted node wins, ties
 * to the smallest node index; path = its root path (node 0 first).
 * Outputs (device int32):
 *   accept_len [batch]     a = accepted drafts (0 .. N-1); a + 1 tokens commit;
 *   path       [batch][N]  path[0..a] node indices, then -1;
 *   tokens     [batch][N]  draft ids of path[1..a], then the bonus am[path[a]],
 *                          then -1;
 *   argmax     [batch][N]  am, or NULL.
 * workspace device scratch of sv_greedy_accept_workspace_size() bytes.  It must
 *           be zero-filled before its first use; every completed call leaves
 *           all of it zero-filled again (whatever the shape of the next call).  One workspace serves one stream at a
 *           time (concurrent calls sharing it race).
 */
size_t sv_greedy_accept_workspace_size(int batch, int n_nodes, int vocab);
int sv_greedy_accept(int batch, int n_nodes, int vocab,
                     const void *logits, int logits_dtype,
                     const int32_t *draft_ids, const int32_t *parent,
                     int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *argmax,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_kv_compact -- keep only the accepted rows [DFN "Key breakthroughs";
 * KWK section 3.3].  In place, for every layer l < n_layers, KV head, K and V
 * (and the 4-bit scale rows):
 *     row ctx + j  <-  row ctx + path[b][j]      for j = 0 .. accept_len[b],
 * with every source read before any destination is written.  Rows where
 * path[j] == j are not touched (a chain moves nothing); rows past
 * ctx + accept_len are left as they were.
 * new_lens  device int32 [batch] = ctx + accept_len + 1, or NULL.
 * path / accept_len are sv_greedy_accept's outputs (device).  Entries that are
 * out of range (accept_len outside [0, N-1], path[j] outside [j, N-1]) skip the
 * affected rows.
 */
int sv_kv_compact(const sv_kv_cache *kv, int n_layers, int batch, int n_nodes,
                  const int32_t *ctx_lens, int max_ctx,
                  const int32_t *path, const int32_t *accept_len,
                  int32_t *new_lens, void *stream);

/*
 * sv_sample_accept -- stochastic verification at temperature T [DFN "Next
 * steps": temperature sampling planned for the verify path].  Every row (b, i)
 * is sampled instead of maximised: y = the lowest index of the maximum of the
 * fp32 key  logits[b][i][v] / T + gumbel[b][i][v]  (Gumbel-max sampling of
 * softmax(logits / T) with the caller's standard-Gumbel noise; the division
 * and the addition each round to nearest).  The acceptance walk then runs as
 * in sv_greedy_accept with y in place of the argmax: a draft is accepted iff
 * it equals its parent's sample, the bonus token is the sample at the last
 * accepted node.  With a deterministic drafter this commits tokens
 * distributed as sampling from the target one token at a time.
 *   gumbel   device float [batch][N][vocab], 4-byte aligned (16-byte aligned
 *            with vocab % 4 == 0 for the vectorised loads).
 *   temperature  > 0 and finite.
 *   sampled  device int32 [batch][N]: y, or NULL.
 * Other arguments, outputs, workspace and errors as sv_greedy_accept.
 */
int sv_sample_accept(int batch, int n_nodes, int vocab,
                     const void *logits, int logits_dtype, const float *gumbel, float temperature,
                     const int32_t *draft_ids, const int32_t *parent,
                     int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *sampled,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_sample_accept_topk -- sv_sample_accept restricted to each row's top-k
 * tokens [DFN "Next steps": temperature and top-k sampling planned for the
 * verify path].  Token v of row (b, i) competes in the Gumbel-max sample only
 * if its logit is >= the row's k-th largest logit (values compared as fp32,
 * -0 == +0; ties at the k-th value stay in).  top_k <= 0 or >= vocab is
 * sv_sample_accept; 1 <= top_k <= 1024 runs one workgroup per row (k-th
 * largest by radix selection over LDS candidates); larger k: SV_EUNSUPPORTED.
 * Arguments, outputs, workspace and errors as sv_sample_accept (the gumbel
 * rows are read only at the candidate tokens).
 */
int sv_sample_accept_topk(int batch, int n_nodes, int vocab,
                          const void *logits, int logits_dtype, const float *gumbel, float temperature, int top_k,
                          const int32_t *draft_ids, const int32_t *parent,
                          int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *sampled,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_kv_append -- write the verify block's K/V rows into the cache, quantising
 * them for a 4-bit cache [DFN "128K context in 24 GB": the KV cache is kept in
 * 4 bits and converted as rows are written].  The step just before
 * sv_verify_attn: row i of sequence b goes to position ctx_b + i (ctx clamped
 * to [0, max_ctx]) of every KV head, layer 0 of `kv`.
 *   k_new, v_new  device [batch][n_rows][n_kv_heads][head_dim], src_dtype
 *                 SV_F32 or SV_BF16, 16-byte aligned (bf16 sources are
 *                 widened exactly to fp32).
 *   SV_F32 cache: the values; SV_BF16 cache: round to nearest even;
 *   SV_Q4 cache:  per 32-value block d = half(max|x| / 7) (fp32 division, then
 *                 round to nearest even into IEEE half), code =
 *                 clamp(round_half_even(x / d), -8, 7) + 8 (fp32 division),
 *                 8 for every value of a block with d = 0; layout as above.
 * Paged: positions whose page id lies outside the pool are skipped.
 * 1 <= n_rows <= 64; the capacity checks of sv_verify_attn apply with
 * n_nodes = n_rows.  Non-finite inputs give unspecified codes.
 */
int sv_kv_append(const sv_kv_cache *kv, int batch, int n_rows, const int32_t *ctx_lens, int max_ctx,
                 const void *k_new, const void *v_new, int src_dtype, void *stream);

/*
 * sv_greedy_accept_compact -- sv_greedy_accept followed by sv_kv_compact on
 * the same stream, in one launch: the workgroup that finishes a sequence's
 * acceptance walk moves that sequence's accepted KV rows itself (every layer,
 * KV head, K and V, scale rows of a 4-bit cache), in rounds of at most 32 KB
 * that each read all their rows before writing any.  Arguments, outputs,
 * workspace rules and errors are those of the two calls (accept_len and path
 * are outputs here, not inputs); results are identical to the two calls'.
 * Sized for few moving rows per sequence (a tree's accepted branch): with many
 * layers the single workgroup per sequence is slower than sv_kv_compact.
 */
int sv_greedy_accept_compact(int batch, int n_nodes, int vocab,
                             const void *logits, int logits_dtype,
                             const int32_t *draft_ids, const int32_t *parent,
                             int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *argmax,
                             const sv_kv_cache *kv, int n_layers, const int32_t *ctx_lens, int max_ctx,
                             int32_t *new_lens, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Recurrent layers of a hybrid target (tree-aware state)
 * ------------------------------------------------------
 * [DFN "Why we ran this test"]: 48 of the target's 64 layers are Gated
 * DeltaNet layers, each keeping a recurrent state beside the KV cache.  [DFN
 * "Key breakthroughs"]: verifying a tree needs every node's state after its
 * root path; the conv windows follow parent chains, not the row order, and the
 * per-node states are written straight into a persistent buffer (optionally
 * f16) from which the accepted node's state is taken.  The rows are the N
 * verify rows, parent[] as above (an entry outside [0, i) starts a new path
 * from the committed state); parent NULL means a chain.
 */

/*
 * sv_ssm_conv_tree -- the short causal depthwise convolution, per node.
 *   out[b][i][c] = act(bias[c] + sum_{m=0}^{K-1} weight[c][K-1-m] * X_m[c])
 * where X_0 = x[b][i], X_m = x[b][m-th ancestor of i] while the path lasts,
 * then conv_state[b][K-2], conv_state[b][K-3], ... (the inputs before the
 * block, oldest first).  act = identity (activation 0) or SiLU (1).
 * x, out      device [batch][N][channels], dtype SV_F32 or SV_BF16 (out
 *             rounded to nearest even); out must not overlap x or conv_state.
 * conv_state  device [batch][kernel_width-1][channels], same dtype.
 * weight      device float [channels][kernel_width]; bias device float
 *             [channels] or NULL.  kernel_width 2, 3 or 4; channels a
 *             multiple of 4; all arrays 16-byte aligned.
 */
int sv_ssm_conv_tree(int batch, int n_nodes, int channels, int kernel_width,
                     const void *x, const void *conv_state, int dtype,
                     const float *weight, const float *bias, const int32_t *parent,
                     int activation, void *out, void *stream);

/*
 * sv_gated_delta_net_tree -- the gated delta rule over the tree, every node's
 * state persisted.  The rule is that of Gated DeltaNet (Yang, Kautz,
 * Hatamizadeh, ICLR 2025); per value head h (key head h / (Hv/Hk)) with state
 * S (v_dim x k_dim, row-major), node i continues from its parent's state (the
 * committed state S0 at the top of a path):
 *   a = exp(g), S_i = a S_p + beta (v - a S_p k) k^T,  out_i = scale S_i q.
 * q, k        device, token (b, i) at element (b*N + i) * qk_stride, key head
 *             hk at + hk * k_dim; v likewise with v_stride and v_dim (strides
 *             0 = packed; else >= heads * dim and a multiple of 8, so that q, k,
 *             v may point into one packed conv output).  dtype SV_F32 or
 *             SV_BF16; 16-byte aligned.
 * g, beta     device float [batch][N][n_v_heads] (g the log decay).
 * state       device float [batch][n_v_heads][v_dim][k_dim]: S0 (read only).
 * out         device [batch][N][n_v_heads][v_dim] in dtype.
 * state_nodes device [batch][N][n_v_heads][v_dim][k_dim] in state_dtype
 *             (SV_F32, or SV_F16 rounded to nearest even): every node's state.
 * schedule    device int32 [batch][64] from sv_tree_schedule for the same
 *             parent array, or NULL (the kernel then derives the visiting
 *             order from parent itself; with a schedule, parent is not read).
 * scale <= 0 selects 1/sqrt(k_dim).  k_dim 64 or 128, and N * n_v_heads * v_dim *
 * k_dim below 2^32 (else SV_EUNSUPPORTED);
 * v_dim a multiple of 32.  Arithmetic in fp32.
 */
int sv_gated_delta_net_tree(int batch, int n_nodes, int n_k_heads, int n_v_heads, int k_dim, int v_dim,
                            const void *q, const void *k, const void *v, int64_t qk_stride, int64_t v_stride,
                            int dtype, const float *g, const float *beta, const float *state,
                            const int32_t *parent, const int32_t *schedule, float scale, void *out,
                            void *state_nodes, int state_dtype, void *stream);

/*
 * sv_tree_schedule -- the visiting order sv_gated_delta_net_tree uses for a
 * tree, computed once per verify step and shared by every recurrent layer
 * (the tree is the same in all of them).  schedule: device int32
 * [batch][64]; entry t of a sequence is the t-th node of a depth-first walk
 * (children by subtree size, the largest last) | (where its parent's state
 * is: 0 registers, 1 the committed state, 2 + s parked slot s) << 8 | (the
 * slot to park its own state in, plus 1, or 0) << 16.  parent as above.
 */
int sv_tree_schedule(int batch, int n_nodes, const int32_t *parent, int32_t *schedule, void *stream);

/*
 * sv_recurrent_commit -- after acceptance: state[b] <- state_nodes[b][path[b][a]]
 * (widened to fp32) and conv_state[b] <- the last kernel_width-1 entries of
 * (conv_state[b], x[b][path[b][0]], ..., x[b][path[b][a]]), a = accept_len[b].
 * path / accept_len are sv_greedy_accept's outputs (device); a sequence whose
 * entries are out of range (a outside [0, N-1], path[j] outside [j, N-1] for
 * j <= a) keeps its state and conv state.  Shapes and dtypes as in the two
 * calls above (x is the conv input of the block).
 */
int sv_recurrent_commit(int batch, int n_nodes, int n_v_heads, int k_dim, int v_dim,
                        const void *state_nodes, int state_dtype, float *state,
                        int channels, int kernel_width, const void *x, void *conv_state, int dtype,
                        const int32_t *path, const int32_t *accept_len, void *stream);

/* Static text for a return code. */
const char *sv_error_string(int code);
/* The hipError_t of this thread's last SV_EHIP return (0 if none). */
int sv_last_hip_error(void);

/*
 * Per-call launch tuning (benchmarks and sweeps; the defaults need none).
 * Passed by pointer to the *_tuned calls below; NULL, or a zero field, keeps
 * the library's choice.  The library keeps no tuning state between calls.
 *   attn_target_wgs  workgroups the attention launch aims for (>= 0); default
 *                    256 on the pipelined and cooperative kernels, 512 on the
 *                    others
 *   attn_rowblocks   packed-row blocks per (sequence, KV head) on the
 *                    matrix-core kernels (>= 0)
 *   attn_posgroups   waves sharing one 16-row tile on the pipelined bf16
 *                    kernel: 1, 2 or 4 (each takes 32 positions of a stage)
 *   attn_occupancy   workgroups per CU on the pipelined bf16 kernel for one
 *                    row tile per wave: 1 or 2 (half-size LDS rings, twice the
 *                    work units)
 *   attn_q4_kernel   4-bit caches of head dim 256 with >= 16 packed rows:
 *                    1 the cooperative fp16 matrix-core kernel with four
 *                    waves per workgroup, 2 the pipelined kernel with bf16
 *                    staging, 3 the cooperative fp16 kernel with eight waves
 *                    per workgroup (two per SIMD); 0 (default) and 3 take the
 *                    eight-wave kernel where it applies (contiguous caches,
 *                    and paged caches with up to 64 packed rows per block)
 *                    and the four-wave one otherwise
 *   argmax_chunk     logits per argmax workgroup, a positive multiple of 8
 *                    (0, the default: 32768 for greedy acceptance of bf16
 *                    logits, 16384 otherwise)
 * A value out of range makes the call return SV_EINVAL (the workspace-size
 * query returns 0).  A workspace sized under one tuning may be too small
 * under another (the call then returns SV_EWORKSPACE).
 */
typedef struct sv_tuning {
    int32_t attn_target_wgs;
    int32_t attn_rowblocks;
    int32_t attn_posgroups;
    int32_t attn_occupancy;
    int32_t attn_q4_kernel;
    int32_t argmax_chunk;
} sv_tuning;

/* sv_verify_attn_window with a tuning (window 0 = the whole key range). */
size_t sv_verify_attn_tuned_workspace_size(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                                           int max_ctx, int window, const sv_tuning *tuning);
int sv_verify_attn_tuned(const sv_kv_cache *kv, int batch, int n_nodes, int n_q_heads,
                         const int32_t *ctx_lens, int max_ctx,
                         const void *q, int q_dtype, const int32_t *parent, float sm_scale, int window,
                         const sv_tuning *tuning, void *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream);
/* sv_greedy_accept with a tuning (argmax_chunk). */
int sv_greedy_accept_tuned(int batch, int n_nodes, int vocab,
                           const void *logits, int logits_dtype,
                           const int32_t *draft_ids, const int32_t *parent,
                           int32_t *accept_len, int32_t *path, int32_t *tokens, int32_t *argmax,
                           const sv_tuning *tuning, void *workspace, size_t workspace_bytes, void *stream);

/*
 * sv_check_device_errors -- the device-side precondition word.
 *
 * The calls above treat broken device-side inputs as documented (a parent
 * that is not an earlier node ends the node's path; a page id outside the
 * pool reads as zero rows; ctx_lens are clamped to [0, max_ctx]; out-of-range
 * path / accept_len entries skip rows) and say nothing.  A library built with
 * SV_DEBUG (libsv_debug.so) also records each such input when a kernel meets
 * it, with an atomic OR into a word in device memory (one word per GPU):
 *   SV_DEVERR_PARENT  parent[b][i] outside [0, i) for some i >= 1
 *                     (attention, acceptance);
 *   SV_DEVERR_PAGE    a page id outside [0, capacity) for a position the call
 *                     reads or writes (attention, compaction, append);
 *   SV_DEVERR_CTX     ctx_lens[b] < 0 or > max_ctx (attention, compaction,
 *                     append);
 *   SV_DEVERR_PATH    accept_len[b] outside [0, N-1] or path[b][j] outside
 *                     [j, N-1] for j <= accept_len[b] (compaction).
 * This call waits for `stream` (the one exception to "never synchronises"),
 * returns the bits recorded on the current device since the previous call,
 * and clears them.  A release build records nothing and returns 0 without
 * touching the device.  Negative return: SV_EHIP.
 */
#define SV_DEVERR_PARENT 1
#define SV_DEVERR_PAGE   2
#define SV_DEVERR_CTX    4
#define SV_DEVERR_PATH   8
int sv_check_device_errors(void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SV_H */
