"""Plain fp64 CPU oracle for one Orthrus dual-view decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``dual_view_block_amd``) never imports it and shares no code,
header, table or helper with it; the oracle in turn imports nothing from the
product path.

What is computed follows the Orthrus pages:

* block attention of the diffusion view and of the AR verify pass over one
  shared KV cache -- ``oracle.attention``;
* greedy and T>0 (rejection-sampling) consensus -- ``oracle.consensus``;
* the commit that closes a decode cycle (verified rows into the cache, new
  lengths, emitted tokens, next anchor) and whole synthetic decode cycles --
  ``oracle.cycle``;
* the training objective's forward KL(P_AR || P_Diff) over the vocabulary and
  its draft-logit gradient -- ``oracle.kl``;
* the training-time dual-pass block-mask attention, forward and the backward
  of the diffusion rows -- ``oracle.train_attn``;
* tree verification (draft trees from top-M marginals, ancestor masks, greedy
  consensus along the tree, path commit) -- ``oracle.tree``;
* dynamic block sizes (a block length per sequence, the consensus and commit
  over it, and the rule that picks the next length from acceptance) --
  ``oracle.dynamic``.

Every function is the plain definition written out in float64 (or exact
integers), one sequence / head at a time, with explicit masks.  Library
primitives used as single steps: ``numpy.matmul``, ``numpy.exp``,
``numpy.cumsum``, ``numpy.searchsorted``.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library routines (``torch`` SDPA in float64), brute
force on tiny inputs, invariants the pages fix, and exact enumeration of the
sampler's uniforms.  No function is "parity unpinned".
"""
from .attention import (MASK_DIFF_BIDIR, MASK_EXPLICIT, MASK_VERIFY_CAUSAL, block_attention,
                        block_attention_rows, transient_kv_bytes)
from .consensus import (greedy_consensus, row_argmax, sample_consensus,
                        accept_prefix, accepts, residual_weights, inverse_cdf_pick,
                        fixed_point_weight, uniform_to_grid_int,
                        tokens_committed)
from .cycle import bits_to_bf16, commit_block, decode_cycles
from .kl import forward_kl, forward_kl_rows
from .train_attn import dual_pass_backward, dual_pass_forward, training_attention_flops
from .tree import (ancestor_masks, build_tree, commit_path, masks_to_bits, topk_logprobs,
                   tree_greedy_consensus)
from .dynamic import (block_attention_dyn, block_len_from_stat, commit_block_dyn, decode_cycles_dyn,
                      greedy_consensus_dyn, live_lengths, sample_consensus_dyn, update_accept_stat)

__all__ = [
    "MASK_DIFF_BIDIR", "MASK_VERIFY_CAUSAL", "block_attention",
    "block_attention_rows", "transient_kv_bytes", "greedy_consensus",
    "row_argmax", "sample_consensus", "accept_prefix", "accepts", "residual_weights",
    "inverse_cdf_pick", "fixed_point_weight", "uniform_to_grid_int",
    "tokens_committed", "bits_to_bf16", "commit_block", "decode_cycles", "forward_kl",
    "forward_kl_rows", "dual_pass_forward", "dual_pass_backward", "training_attention_flops",
    "MASK_EXPLICIT", "ancestor_masks", "build_tree", "commit_path", "masks_to_bits", "topk_logprobs",
    "tree_greedy_consensus", "block_attention_dyn", "commit_block_dyn", "greedy_consensus_dyn",
    "live_lengths", "sample_consensus_dyn", "decode_cycles_dyn", "update_accept_stat",
    "block_len_from_stat",
]
