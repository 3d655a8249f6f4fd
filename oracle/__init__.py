"""CPU oracle of the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import, call or link anything here; only the tests, the
``smoke()`` check of the repository entry module and the benchmark's CPU
baseline leg use it.  It shares no code with the GPU path.

What it computes, plainly and slowly, in float64 from the exact widening of
the stored inputs:

* ``attention``: masked GQA softmax attention of the verify rows over the KV
  cache, with an explicit boolean mask matrix built from the token tree
  (the cache is visible to every row, the draft block only along each node's
  root path);
* ``accept``: per-row argmax (lowest index wins ties), the greedy acceptance
  walk (longest accepted root path, plus the bonus token), and an
  independent brute-force version of the walk; the sampled variant (each
  row's Gumbel-max sample at temperature T, optionally over its top-k
  tokens, in place of its argmax);
* ``compact``: the post-acceptance KV compaction as a snapshot copy;
* ``append``: writing the verify block's K/V rows into the cache, with the
  4-bit quantisation at write time;
* ``recurrent``: the tree-aware recurrent state of the hybrid target's Gated
  DeltaNet layers: the short causal conv with each node's window along its
  parent chain, the gated delta rule over the tree keeping every node's
  state, and the commit of the accepted node's state and conv window.

Sources: the single-RTX-3090 DFlash + DDTree note ("Making Qwen3.5-27B token
generation 6x faster on one RTX 3090", blog.xiaohack.org): greedy verify and
16-row blocks (section "Architecture"), DDTree verification of budget+1 rows
(section "Key breakthroughs", logits buffer fix), compaction of accepted
sibling branches (same section), the 4-bit KV cache read by flash attention
(section "128K context in 24 GB"); the xdnf.cn notes on Qwen3.8-27B
speculative decoding, section 5.3 (the draft block's causal mask must be
aligned to the end of the key range).

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` against closed forms, library routines
(``torch.nn.functional.scaled_dot_product_attention`` in float64,
``numpy.argmax``), brute force on small inputs and hand-worked fixtures in
``tests/golden/``.
"""
from .formats import widen_bf16, widen_fp16, widen_f32, q4_decode
from .attention import ancestor_matrix, verify_mask, verify_attention_seq, verify_attention
from .accept import (argmax_first, accept_walk, accept_bruteforce, greedy_accept, sample_row, sample_accept,
                     topk_threshold, sample_row_topk)
from .compact import compact_cache
from .append import bf16_round, q4_quantise, kv_append
from .recurrent import tree_parent, root_path, conv_tree, delta_rule_step, delta_net_tree, recurrent_commit

__all__ = [
    "widen_bf16", "widen_fp16", "widen_f32", "q4_decode",
    "ancestor_matrix", "verify_mask", "verify_attention_seq", "verify_attention",
    "argmax_first", "accept_walk", "accept_bruteforce", "greedy_accept", "sample_row", "sample_accept",
    "topk_threshold", "sample_row_topk",
    "compact_cache", "bf16_round", "q4_quantise", "kv_append",
    "tree_parent", "root_path", "conv_tree", "delta_rule_step", "delta_net_tree", "recurrent_commit",
]
