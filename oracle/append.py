"""Writing the verify block's K/V rows into the cache (oracle side).

TEST INFRASTRUCTURE ONLY: used by the tests, never by the product path.

The verify rows' keys and values are written into the cache before attention
reads it, and a 4-bit cache quantises them at write time: the single-RTX-3090
DFlash note keeps the KV cache in 4 bits so 128K of context fits ("128K
context in 24 GB"), converting as the rows are stored and reading the
quantised cache in flash attention.  The pages name the block format but give
neither its layout nor its rounding; the reading used here:

* blocks of 32 consecutive head-dim values share one IEEE-half scale
  ``d = half(max|x| / 7)`` (the division in fp32, then round to nearest even
  into half precision);
* the code of a value is ``clamp(round_half_even(x / d), -8, 7) + 8`` with the
  division in fp32, and 8 for every value of a block whose scale is 0;
* value 2t of a row sits in the low nibble of byte t, value 2t + 1 in the high
  nibble (so a stored value decodes to ``d * (code - 8)``).

bf16 caches store the round-to-nearest-even bf16 of the value; fp32 caches the
value itself.  Source rows in bf16 are widened exactly to fp32 first.
"""
import numpy as np

from .formats import widen_bf16


def bf16_round(x32: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest, ties to even.

    The 16 bits kept are the top half of the fp32 pattern; the discarded low
    half decides: above 0x8000 rounds up, below truncates, exactly 0x8000
    rounds to the even kept pattern.  (NaN inputs are not used.)
    """
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    top = u >> 16
    low = u & 0xFFFF
    up = (low > 0x8000) | ((low == 0x8000) & ((top & 1) == 1))
    return (top + up.astype(np.uint32)).astype(np.uint16)


def q4_quantise(x32: np.ndarray):
    """fp32 rows ``[..., D]`` -> (codes uint8 ``[..., D/2]``, scales uint16 ``[..., D/32]``)."""
    x32 = np.asarray(x32, dtype=np.float32)
    D = x32.shape[-1]
    assert D % 32 == 0
    out_codes = np.empty(x32.shape[:-1] + (D // 2,), dtype=np.uint8)
    out_scales = np.empty(x32.shape[:-1] + (D // 32,), dtype=np.uint16)
    flat = x32.reshape(-1, D)
    fc = out_codes.reshape(-1, D // 2)
    fs = out_scales.reshape(-1, D // 32)
    for r in range(flat.shape[0]):
        for blk in range(D // 32):
            vals = flat[r, 32 * blk:32 * blk + 32]
            amax = np.float32(0.0)
            for v in vals:
                amax = max(amax, np.float32(abs(v)))
            d_half = np.float16(np.float32(amax) / np.float32(7.0))     # fp32 divide, then RNE to half
            d = np.float32(d_half)
            codes = []
            for v in vals:
                if d == 0:
                    codes.append(8)
                else:
                    q = np.rint(np.float32(v) / d)                       # fp32 divide, ties to even
                    codes.append(int(min(max(q, -8.0), 7.0)) + 8)
            for t in range(16):
                fc[r, 16 * blk + t] = codes[2 * t] | (codes[2 * t + 1] << 4)
            fs[r, blk] = d_half.view(np.uint16)
    return out_codes, out_scales


def _rows_f32(new, src_dtype):
    if src_dtype == "f32":
        return np.asarray(new, dtype=np.float32)
    if src_dtype == "bf16":
        return widen_bf16(new).astype(np.float32)                      # exact
    raise ValueError(src_dtype)


def kv_append(arrays, new_k, new_v, *, ctx_lens, dtype, src_dtype, max_ctx=None, page_table=None, page_size=0):
    """The cache after writing the verify block.

    ``arrays``: cache arrays as stored (k, v; plus k_scale, v_scale for 4-bit),
    one layer: contiguous ``[B][H][capacity][...]`` or paged
    ``[pages][H][page_size][...]``.  ``new_k`` / ``new_v``: ``[B][n][H][D]`` in
    ``src_dtype`` ("f32" values or "bf16" bit patterns).  Row i of sequence b
    goes to position ctx_b + i (ctx clamped to [0, max_ctx]); a paged position
    whose page id is outside the pool is skipped.  Returns new arrays.
    """
    out = [np.array(a, copy=True) for a in arrays]
    B, n, H, D = np.asarray(new_k).shape
    kf = _rows_f32(new_k, src_dtype)
    vf = _rows_f32(new_v, src_dtype)
    for b in range(B):
        ctx = int(ctx_lens[b])
        if max_ctx is not None:
            ctx = min(max(ctx, 0), int(max_ctx))
        for i in range(n):
            pos = ctx + i
            for h in range(H):
                if page_table is None:
                    where = (b, h, pos)
                else:
                    page = int(page_table[b][pos // page_size])
                    if page < 0 or page >= out[0].shape[0]:
                        continue
                    where = (page, h, pos % page_size)
                for which, rows in ((0, kf), (1, vf)):
                    x = rows[b, i, h]
                    if dtype == "f32":
                        out[which][where] = x
                    elif dtype == "bf16":
                        out[which][where] = bf16_round(x)
                    elif dtype == "q4":
                        c, s = q4_quantise(x)
                        out[which][where] = c
                        out[2 + which][where] = s
                    else:
                        raise ValueError(dtype)
    return out
