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
    inside the prefix), the rest causally;
  * the same tutorial, Pattern 3, last paragraph: masks are composed with
    and_masks / or_masks rather than written as one predicate -- here any
    and / or / not composition of the five terms, given as its truth table;
  * the quick start: a block mask is built for given query and key lengths
    (Q_LEN, KV_LEN), which need not be equal.

Readings taken where the pages leave it open: the sink term only widens the
window term (without a window there is nothing for it to widen), and it is
AND-ed with causality and the document term like every other term.  The
prefix term kv < PREFIX likewise only widens the causal term (q >= kv OR
kv < PREFIX; without causality every key is already allowed) and is AND-ed
with the document and window terms.  With Q_LEN != KV_LEN, query i sits at
absolute position q_offset + i (0 by default) and every term compares
absolute positions; document ids are indexed by absolute position for
queries and keys alike.
"""
from __future__ import annotations

import numpy as np

# bit of each term in a truth-table index
C_BIT, D_BIT, W_BIT, S_BIT, P_BIT = 1, 2, 4, 8, 16


def terms(spec, b, q_idx, kv_idx):
    """The five terms as boolean arrays broadcast over q_idx (query indices)
    and kv_idx: causal, same document, window, sink, prefix.  A term whose
    data the spec lacks (no document ids, no window) is False."""
    qa = np.asarray(q_idx, dtype=np.int64) + int(getattr(spec, "q_offset", 0))
    kv = np.asarray(kv_idx, dtype=np.int64)
    shape = np.broadcast_shapes(qa.shape, kv.shape)
    false = np.zeros(shape, dtype=bool)
    causal = np.broadcast_to(qa >= kv, shape)
    if spec.document:
        docs = spec.doc_ids[b if spec.doc_ids.shape[0] > 1 else 0].astype(np.int64)
        same = np.broadcast_to(docs[qa] == docs[kv], shape)
    else:
        same = false
    window = np.broadcast_to((qa - kv) < spec.window, shape) if spec.window is not None else false
    sink = np.broadcast_to(kv < spec.sinks, shape) if spec.sinks else false
    prefix = np.broadcast_to(kv < spec.prefix, shape) if getattr(spec, "prefix", 0) else false
    return causal, same, window, sink, prefix


def visible(spec, b, q_idx, kv_idx) -> np.ndarray:
    """Boolean array, broadcast over q_idx and kv_idx (integer arrays of query
    indices and key positions).

    spec: workloads.MaskSpecData (causal, document, doc_ids, window, sinks,
          prefix, q_offset, table).
    b:    batch element; the mask row used is doc_ids[b] (or doc_ids[0] when
          the mask is shared across the batch).
    """
    c, d, w, s, p = terms(spec, b, q_idx, kv_idx)
    table = getattr(spec, "table", None)
    if table is not None:
        idx = c * C_BIT + d * D_BIT + w * W_BIT + s * S_BIT + p * P_BIT
        return ((int(table) >> idx) & 1).astype(bool)
    ok = np.ones(c.shape, dtype=bool)
    if spec.causal:
        ok &= c | p
    if spec.document:
        ok &= d
    if spec.window is not None:
        ok &= w | s
    return ok
