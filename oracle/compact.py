"""KV compaction after acceptance (oracle side).

After a verify step only the accepted nodes' KV rows may stay in the cache:
the single-RTX-3090 DFlash note has to compact the state of an accepted
sibling branch (section "Key breakthroughs", the stale-feature fix), and the
kwkr.cn RTX-4080 notes roll rejected draft KV back (section 3.3).  With the
draft rows written at positions ``ctx .. ctx + N - 1`` in node order, the
accepted path ``path[0..a]`` (root first) is compacted to ``ctx .. ctx + a``:

    new[ctx + j] = old[ctx + path[j]]   for j = 0 .. a,

for every layer, KV head, K and V (and 4-bit scale rows), all sources read
before any destination is written.  Rows past ``ctx + a`` are left as they
were; the sequence's new length is ``ctx + a + 1``.
"""
import numpy as np


def compact_cache(arrays, *, ctx_lens, path, accept_len, page_table=None, page_size=0):
    """Snapshot copy.

    ``arrays``: list of storage arrays, each ``[layers][seq|page][head][pos|slot][...]``
    (a leading layer axis is required; pass ``a[None]`` for one layer).
    Returns ``(new_arrays, new_lens, dst_src)`` where ``dst_src[b]`` lists the
    ``(dst, src)`` logical positions moved for sequence b.
    """
    snaps = [np.array(a, copy=True) for a in arrays]
    outs = [np.array(a, copy=True) for a in arrays]
    B = len(ctx_lens)
    new_lens = np.empty(B, dtype=np.int32)
    dst_src = []
    for b in range(B):
        ctx = int(ctx_lens[b])
        a = int(accept_len[b])
        moves = [(ctx + j, ctx + int(path[b][j])) for j in range(a + 1)]
        dst_src.append(moves)
        new_lens[b] = ctx + a + 1
        for snap, out in zip(snaps, outs):
            for dst, src in moves:
                if page_table is None:
                    out[:, b, :, dst] = snap[:, b, :, src]
                else:
                    pd, od = page_table[b][dst // page_size], dst % page_size
                    pss, os_ = page_table[b][src // page_size], src % page_size
                    out[:, pd, :, od] = snap[:, pss, :, os_]
    return outs, new_lens, dst_src
