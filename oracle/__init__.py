"""CPU fp64 oracle for masked scaled-dot-product attention with online softmax.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package: only the
tests, the smoke check and the benchmark's CPU-baseline leg may call it. It shares no
code with the HIP kernels.

Sources (web pages, cited by title and section):
  [FDMA]  "Optimize Flash Dynamic Mask Attention Kernel Configurations"
          (flash-sparse-attention pull request 148): split-KV with 1/2/4/8/16 splits,
          deterministic backward, softcap, windowed variants.
  [2CTA]  "Enable 2CTA for SM100 block-sparse backward" (flash-attention pull request
          2661): the fuzz tester's forward/backward call signatures (softmax scale
          1/sqrt(headdim), causal, softcap, window, score_mod, mask_mod,
          block_sparse_tensors, return_lse), its mask names (causal, sliding_window,
          block_diagonal, prefix_lm) and its window rule.
  [SDPA]  POPCORNBENCH transcript "Kimi-K2.6 l1 p97" (custom fp32 SDPA kernel): the
          math-backend definition softmax(Q K^T * scale) V and the two-chunk
          online-softmax merge rule (running max, rescaled sums and outputs).

Modules:
  masks      element mask predicates and the block-sparse tile semantics
  attention  materialised fp64 forward / backward / split-KV partial + combine
  blockmask  tile classification and index lists, by element enumeration
  scalar     a pure-Python scalar brute force for tiny shapes (cross-check)

Every function computes the plain definition with the full score matrix; there is no
tiling, fusion or reordering beyond what the definition states.
"""
from .masks import MaskSpec, allowed, block_sparse_allowed  # noqa: F401
from .attention import (  # noqa: F401
    forward, forward_bh, forward_varlen, backward, backward_bh, backward_varlen, scores_bh, kv_head,
    split_partials, combine_partials, streaming_forward_bh,
)
from .blockmask import classify_tiles, build_lists, BlockLists  # noqa: F401
