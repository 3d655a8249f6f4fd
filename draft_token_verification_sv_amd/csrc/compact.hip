// In-place KV compaction after acceptance.
//
// Only the accepted nodes' state may stay [single-RTX-3090 DFlash note, "Key
// breakthroughs": features of an accepted sibling branch must be compacted;
// kwkr.cn RTX-4080 notes section 3.3: rejected draft KV is rolled back].  The
// verify rows sit at ctx + node; the accepted path path[0..a] moves to
// ctx + 0..a:  row ctx + j <- row ctx + path[j].  Because path[j] >= j, a
// destination can be the source of a later move, so one workgroup per
// (sequence, layer, KV head, K|V) first reads every moving row into LDS, then
// writes them all.  Rows with path[j] == j are skipped (a chain moves nothing).
#include "device_common.h"

namespace sv {
namespace {

constexpr int kMaxRowBytes = 1024;      // fp32 x 256

__global__ __launch_bounds__(256) void compact_kernel(CompactParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t buf[64 * kMaxRowBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sbuf[64 * 16];
    __shared__ int src_s[64];
    __shared__ int nmov_s;

    const int which = blockIdx.x & 1;                    // 0: K, 1: V
    int rest = blockIdx.x >> 1;
    const int h = rest % p.Hkv;
    rest /= p.Hkv;
    const int layer = rest % p.n_layers;
    const int b = rest / p.n_layers;
    const int tid = threadIdx.x;
    const int N = p.N;

    // the length, the accept count and this thread's path entry load together
    const int ctx = ctx_of(p.ctx_lens, b, p.max_ctx, p.err);
    const int a = p.accept_len[b];
    const int pj = (tid >= 1 && tid < N) ? p.path[(int64_t)b * N + tid] : -1;
    const bool a_ok = a >= 0 && a < N;
    if (p.new_lens != nullptr && which == 0 && h == 0 && layer == 0 && tid == 0)
        p.new_lens[b] = a_ok ? ctx + a + 1 : ctx;
    SV_DEVCHECK(p.err, tid == 0 && !a_ok, SV_DEVERR_PATH);
    if (!a_ok) return;
    SV_DEVCHECK(p.err, tid >= 1 && tid <= a && (pj < tid || pj >= N), SV_DEVERR_PATH);

    // moving rows: j in [1, a] with j < path[j] < N
    if (tid < 64) src_s[tid] = (tid >= 1 && tid <= a && pj > tid && pj < N) ? pj : -1;
    __syncthreads();

    const int D = p.D;
    const int64_t row_bytes = p.dtype == SV_F32 ? D * 4 : (p.dtype == SV_BF16 ? D * 2 : D / 2);
    const int64_t srow_bytes = (D / 32) * 2;
    const int chunks = (int)(row_bytes / 16);
    const int schunks = (int)(srow_bytes / 4);          // 4-byte words of scales
    uint8_t *base = (uint8_t *)(which ? p.kv.v : p.kv.k) + (int64_t)layer * p.layer_stride;
    uint8_t *sbase = (p.dtype == SV_Q4)
                         ? (uint8_t *)(which ? p.kv.vs : p.kv.ks) + (int64_t)layer * p.scale_layer_stride
                         : nullptr;

    // gather every source row (a source whose page is outside the pool reads
    // as a zero row) ...
    for (int e = tid; e < 64 * chunks; e += 256) {
        const int jj = e / chunks, ch = e % chunks;
        const int src = src_s[jj];
        if (src < 0) continue;
        const int64_t ri = kv_row_index(p.kv, b, p.Hkv, h, ctx + src, p.err);
        const u32x4 zero = {0u, 0u, 0u, 0u};
        *(u32x4 *)(buf + jj * kMaxRowBytes + ch * 16) = ri < 0 ? zero : *(const u32x4 *)(base + ri * row_bytes + ch * 16);
    }
    if (sbase != nullptr) {
        for (int e = tid; e < 64 * schunks; e += 256) {
            const int jj = e / schunks, w = e % schunks;
            const int src = src_s[jj];
            if (src < 0) continue;
            const int64_t ri = kv_row_index(p.kv, b, p.Hkv, h, ctx + src);
            *(uint32_t *)(sbuf + jj * 16 + w * 4) = ri < 0 ? 0u : *(const uint32_t *)(sbase + ri * srow_bytes + w * 4);
        }
    }
    __syncthreads();
    // ... then write them to ctx + j
    for (int e = tid; e < 64 * chunks; e += 256) {
        const int jj = e / chunks, ch = e % chunks;
        if (src_s[jj] < 0) continue;
        const int64_t ri = kv_row_index(p.kv, b, p.Hkv, h, ctx + jj, p.err);
        if (ri < 0) continue;
        *(u32x4 *)(base + ri * row_bytes + ch * 16) = *(const u32x4 *)(buf + jj * kMaxRowBytes + ch * 16);
    }
    if (sbase != nullptr) {
        for (int e = tid; e < 64 * schunks; e += 256) {
            const int jj = e / schunks, w = e % schunks;
            if (src_s[jj] < 0) continue;
            const int64_t ri = kv_row_index(p.kv, b, p.Hkv, h, ctx + jj);
            if (ri < 0) continue;
            *(uint32_t *)(sbase + ri * srow_bytes + w * 4) = *(const uint32_t *)(sbuf + jj * 16 + w * 4);
        }
    }
}

}  // namespace

hipError_t launch_compact(const CompactParams &p, hipStream_t st) {
    const int grid = p.B * p.n_layers * p.Hkv * 2;
    hipLaunchKernelGGL(compact_kernel, dim3(grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace sv
