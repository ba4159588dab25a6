"""Mask predicate, evaluated per (b, q, kv) pair.  Oracle; test
infrastructure only.

Follows:
  * speedrun notes "FlexAttention", code listing: a position may attend to
    another when it is causal (q >= kv), in the same document
    (docs[q] == docs[kv]) and inside the window (q - kv < window);
  * tutorial "FlexAttention in PyTorch", Pattern 1 (document mask, causal and
    same document) and Pattern 2 (causal AND (in window OR sink), sink being
    kv < SINKS);
  * prefix-LM masking, which the tutorial's introduction lists among the
    variants: the keys of a prefix are seen by every query (bidirectional
    inside the prefix), the rest causally.

Readings taken where the pages leave it open: the sink term only widens the
window term (without a window there is nothing for it to widen), and it is
AND-ed with causality and the document term like every other term.  The
prefix term kv < PREFIX likewise only widens the causal term (q >= kv OR
kv < PREFIX; without causality every key is already allowed) and is AND-ed
with the document and window terms.
"""
from __future__ import annotations

import numpy as np


def visible(spec, b, q_idx, kv_idx) -> np.ndarray:
    """Boolean array, broadcast over q_idx and kv_idx (integer arrays).

    spec: workloads.MaskSpecData (causal, document, doc_ids [mask_b, T],
          window, sinks).
    b:    batch element; the mask row used is doc_ids[b] (or doc_ids[0] when
          the mask is shared across the batch).
    """
    q = np.asarray(q_idx, dtype=np.int64)
    kv = np.asarray(kv_idx, dtype=np.int64)
    ok = np.ones(np.broadcast_shapes(q.shape, kv.shape), dtype=bool)
    if spec.causal:
        causal_ok = q >= kv
        if getattr(spec, "prefix", 0):
            causal_ok = causal_ok | (kv < spec.prefix)
        ok &= causal_ok
    if spec.document:
        docs = spec.doc_ids[b if spec.doc_ids.shape[0] > 1 else 0].astype(np.int64)
        ok &= docs[q] == docs[kv]
    if spec.window is not None:
        in_window = (q - kv) < spec.window
        if spec.sinks:
            in_window = in_window | (kv < spec.sinks)
        ok &= in_window
    return ok
