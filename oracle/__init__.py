"""Oracle for block-sparse masked attention: a plain, slow CPU implementation
of what the GPU path computes, written from the pages' definitions.

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check in __graft_entry__ and
the benchmark's CPU-baseline leg may import or run anything in this package.
It shares no code with the HIP library and never imports it.

Modules:
  predicate   -- the mask predicate for every (b, q, kv) pair
  block_mask  -- per-tile visible-pair counts (brute force, C with a numpy
                 check path), tile classes and the compacted tile lists
  attention   -- fp64 softmax attention forward and backward, per row and per
                 key column, with the ALiBi and soft-cap score modifications,
                 and the gradient with respect to the ALiBi slopes
"""
from .predicate import visible  # noqa: F401
from .block_mask import (  # noqa: F401
    tile_counts,
    tile_counts_dense_numpy,
    classify,
    block_mask_lists,
    spec_block_mask_lists,
    kv_block,
    EMPTY, PARTIAL, FULL, TILE,
)
from .attention import (  # noqa: F401
    forward_rows,
    forward_dense,
    backward_dense,
    backward_dq_rows,
    backward_dkdv_cols,
    slope_grad_dense,
    bias_grad_dense,
    bias_index,
    bias_radius,
)
