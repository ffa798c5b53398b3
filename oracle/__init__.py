"""CPU fp64 oracle for selection-based sparse attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy (float64) restatement of what the sparse-attention path computes.  Only
the test-suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the library and its Python binding never do, and it shares no code with
them (its only common ground with the GPU side is the seeded input generator in
``workloads``, which holds none of the method's arithmetic).

Sources (web summaries of five papers; cited by page title and section):

* "Full Attention Strikes Back" summary (RTPurbo) - Methodology items 1-3 and 5:
  retrieval/local head split, a 16-dim pre-RoPE low-rank indexer, the dynamic
  top-p selector, sort-free histogram thresholding, sparse decode.
* "Atencao Global Hierarquica (HGA)" summary - Core mechanism items 1-4:
  64-token chunks split into groups, two-level routing, always-visible sink,
  local and current chunks, RoPE-aware mixed summaries, exact token attention;
  Memory architecture: hot / warm (LRU) / cold (host RAM) K/V tiers.
* "Lighthouse Attention" summary - Methodology 2A-2C: symmetric mean pyramid,
  parameter-free l2 scoring with max inheritance, joint top-K across levels,
  dense attention on the gathered subsequence and scatter back (coarse query
  entries attend too, their outputs returned to their own slots); the backward
  pass through the gather, the attention and the scatter (2B: the selection
  itself gets no gradient).
* "Autonomia de Cabecas (AoH)" summary - Methodology item 4: head scores are
  averaged to the GQA group; sinks plus a recent window for streaming heads.
* "S2O" summary - Methodology 2-3: candidates visited in descending
  estimated importance after a dense first pass, stopping on the marginal
  gain of attention mass (monotone-gain early stop).
* Head-split prefill (RTPurbo, Methodology item 1): local heads window their
  prefill, retrieval heads attend densely; per-query-head selection as the
  group rule applied to a group of one head.

Readings of points the pages leave open are listed, one per line, in the
design notes next to this package and are restated where each is used.

Parity pins: every public function here is checked in ``tests/`` against
something other than itself (a library routine, a closed form, brute force on
tiny inputs, or a hand-worked fixture).  The parts fixed only by a stated
reading and not by the pages (the l2 score combination of q and k, the
high/low frequency cutoff, the index logit scale 1/sqrt(r), the tie-break)
are pinned to that reading alone: "parity unpinned" by the pages, pinned to
the stated reading.
"""
from .numerics import round_bf16, round_fp32, round_store, bf16_ulp
from .attention import attend, attend_heads, dense_causal
from .rope import rope_rotate, rope_angles
from .lowrank import (index_keys, index_query, index_logits, order, select_prefix,
                      select_topp, select_topk, topp_margin, cut_gap)
from .local import local_set
from .hga import (high_freq_pairs, chunk_summary, chunk_summaries, group_summaries,
                  route_token_list, route_scores, route_prefill_block, route_prefill_rows)
from .lighthouse import (pyramid_levels, pyramid_scores, visible_entries,
                         block_select, prefill_block, prefill, coarse_block, prefill_coarse)
from .lighthouse_bwd import block_grads, pyramid_backward, prefill_grads, n_entries
from .decode import decode_step, decode_token_sets, decode_token_sets_per_head
from .prefill_heads import prefill_visible, head_prefill_rows, visible_pairs
from .s2o import s2o_order, s2o_head
from .tier import WarmCache, split_positions, tier_rows, needed_groups

__all__ = [n for n in dir() if not n.startswith("_")]
