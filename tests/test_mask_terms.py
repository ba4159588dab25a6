"""The binding's mask composition (CPU only): CAUSAL, SAME_DOC, IN_WINDOW,
SINK and PREFIX and the and_masks / or_masks / ~ operators (tutorial
"FlexAttention in PyTorch", Pattern 3) produce truth tables that, looked up
with the oracle's five terms, give the same pairs as the boolean expression
evaluated directly on those terms.  A wrong term constant or a swapped
operator fails here."""
import itertools

import numpy as np

import oracle.predicate as pred
from workloads import MaskSpecData


def _api():
    from block_sparse_masked_build_amd import api
    return api


def _terms():
    rng = np.random.default_rng(5)
    T = 300
    docs = np.cumsum(rng.random(T) < 1 / 40).astype(np.int32)[None]
    spec = MaskSpecData(T, causal=False, document=True, doc_ids=docs, window=37, sinks=5, prefix=11)
    q = np.arange(T)[:, None]
    kv = np.arange(T)[None, :]
    return spec, q, kv, pred.terms(spec, 0, q, kv)


def _lookup(spec, q, kv, table):
    import dataclasses
    return pred.visible(dataclasses.replace(spec, table=table), 0, q, kv)


def test_single_terms():
    api = _api()
    spec, q, kv, (c, d, w, s, p) = _terms()
    for term, ref in ((api.CAUSAL, c), (api.SAME_DOC, d), (api.IN_WINDOW, w), (api.SINK, s), (api.PREFIX, p)):
        assert np.array_equal(_lookup(spec, q, kv, term.table), ref), term
        assert np.array_equal(_lookup(spec, q, kv, (~term).table), ~ref), term


def test_compositions():
    api = _api()
    spec, q, kv, (c, d, w, s, p) = _terms()
    named = {"C": (api.CAUSAL, c), "D": (api.SAME_DOC, d), "W": (api.IN_WINDOW, w), "S": (api.SINK, s),
             "P": (api.PREFIX, p)}
    for (na, (ta, ra)), (nb, (tb, rb)), (nc, (tc, rc)) in itertools.permutations(named.items(), 3):
        e1 = api.and_masks(api.or_masks(ta, tb), ~tc)
        assert np.array_equal(_lookup(spec, q, kv, e1.table), (ra | rb) & ~rc), (na, nb, nc)
        e2 = api.or_masks(ta & tb, tc)
        assert np.array_equal(_lookup(spec, q, kv, e2.table), (ra & rb) | rc), (na, nb, nc)


def test_pattern_2_spelled_out_is_the_standard_combination():
    """causal-or-prefix AND same document AND (window OR sink) as a table
    gives the standard combination's pairs."""
    import dataclasses
    api = _api()
    spec, q, kv, _ = _terms()
    std = dataclasses.replace(spec, causal=True)
    expr = api.and_masks(api.or_masks(api.CAUSAL, api.PREFIX), api.SAME_DOC, api.or_masks(api.IN_WINDOW, api.SINK))
    assert np.array_equal(_lookup(spec, q, kv, expr.table), pred.visible(std, 0, q, kv))


def test_empty_and_full():
    api = _api()
    assert api.and_masks().table == 0xFFFFFFFF
    assert api.or_masks().table == 0
    assert (api.CAUSAL & ~api.CAUSAL).table == 0
    assert (api.CAUSAL | ~api.CAUSAL).table == 0xFFFFFFFF
