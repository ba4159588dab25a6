"""Pins for the oracle's tile counter and tile lists (CPU only).

Each test checks the oracle against something other than itself: numbers the
pages print, closed forms derived from the predicate, brute force over pairs
in pure Python, or an independent dense-mask reduction.
"""
import os

import numpy as np
import pytest

import oracle
from workloads import MaskSpecData, doc_ids_chunks, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _spec_by_name(name, T):
    if name == "causal":
        return MaskSpecData(T, causal=True)
    if name == "causal_window_1024":
        return MaskSpecData(T, causal=True, window=1024)
    if name == "causal_chunks_1024":
        return MaskSpecData(T, causal=True, document=True, doc_ids=doc_ids_chunks(T, 1024)[None])
    raise KeyError(name)


def _visible_tiles(spec):
    return int((oracle.classify(oracle.tile_counts(spec)) > 0).sum())


def test_printed_tile_counts_64k():
    """Speedrun notes, tile-summary paragraph: 131,328 / 4,572 / 2,304."""
    for name, T, expected in _read_golden("tile_counts_64k.txt"):
        assert _visible_tiles(_spec_by_name(name, int(T))) == int(expected), name


def test_printed_work_ratios_64k():
    """Speedrun notes, Record #12: ~2x the chunked work; dense causal 57x."""
    for num, den, ratio, tol in _read_golden("work_ratios_64k.txt"):
        r = _visible_tiles(_spec_by_name(num, 65536)) / _visible_tiles(_spec_by_name(den, 65536))
        assert abs(r - float(ratio)) <= float(tol) * float(ratio), (num, den, r)


def _window_closed_form(T, w):
    """causal AND q-kv<w, no documents, n = T/128 tiles per side.

    Tile (i, j) on diagonal d = i - j >= 0 holds differences q - kv from
    128 d - 127 to 128 d + 127.  It has a visible pair iff its smallest
    difference is < w, i.e. d <= floor((w + 126) / 128); it is full iff its
    largest difference is < w and it lies strictly below the diagonal
    (the diagonal tile has q < kv pairs), i.e. 1 <= d <= floor(w/128) - 1.
    Diagonal d holds n - d tiles.
    """
    n = T // 128
    dv = min((w + 126) // 128, n - 1)
    visible = sum(n - d for d in range(0, dv + 1))
    df = min(w // 128 - 1, n - 1)
    full = sum(n - d for d in range(1, df + 1)) if df >= 1 else 0
    return visible, full


@pytest.mark.parametrize("w", list(range(64, 1792 + 1, 64)))
def test_window_sweep_closed_form(w):
    """The 28-step window schedule (speedrun notes, Record #13) on one
    65,536-token sequence without documents, against the closed form."""
    T = 65536
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(T, causal=True, window=w)))
    vis, full = _window_closed_form(T, w)
    assert int((cls > 0).sum()) == vis
    assert int((cls == oracle.FULL).sum()) == full


def test_dense_causal_8k_closed_form():
    """Tutorial quick start shape (S = 8192): 64 tile rows, causal -> the
    lower triangle with its diagonal: 64*65/2 tiles, 64 of them partial."""
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(8192, causal=True)))
    assert int((cls > 0).sum()) == 64 * 65 // 2
    assert int((cls == oracle.PARTIAL).sum()) == 64


def test_sinks_32k_closed_form():
    """Tutorial Pattern 2 (1024 window, 4 sinks) at 32,768 positions.

    Band tiles: diagonals 0..8 (256 - d tiles each); full: diagonals 1..7.
    Sinks (kv < 4) add tile column 0 for every row beyond the band
    (i = 9..255), each partial.  ~96.2 % of the full grid is skipped
    (the tutorial rounds it to ~97 %)."""
    T = 32768
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(T, causal=True, window=1024, sinks=4)))
    band = sum(256 - d for d in range(9))
    full = sum(256 - d for d in range(1, 8))
    sink_extra = 256 - 9
    assert int((cls > 0).sum()) == band + sink_extra == 2515
    assert int((cls == oracle.FULL).sum()) == full == 1764
    sparsity = 1.0 - (band + sink_extra) / 256 ** 2
    assert 0.955 < sparsity < 0.975


def _pairs_python(spec):
    """Pure-Python loops over every pair and every tile (tiny T)."""
    T = spec.T
    nt = T // 128
    res = np.zeros((spec.mask_b, nt, nt), dtype=np.int64)
    for b in range(spec.mask_b):
        docs = None if spec.doc_ids is None else [int(x) for x in spec.doc_ids[b]]
        for q in range(T):
            for kv in range(T):
                ok = True
                if spec.causal and not (q >= kv or (spec.prefix and kv < spec.prefix)):
                    ok = False
                if ok and spec.document and docs[q] != docs[kv]:
                    ok = False
                if ok and spec.window is not None:
                    if not ((q - kv) < spec.window or (spec.sinks and kv < spec.sinks)):
                        ok = False
                if ok:
                    res[b, q // 128, kv // 128] += 1
    return res


def _random_spec(rng, T, allow_nonmono=True):
    causal = bool(rng.integers(0, 2))
    document = bool(rng.integers(0, 2))
    mb = int(rng.integers(1, 3))
    docs = None
    if document:
        if allow_nonmono and rng.integers(0, 3) == 0:
            docs = rng.integers(0, 3, size=(mb, T)).astype(np.int32)
        else:
            docs = np.stack([np.cumsum(rng.random(T) < 1.0 / rng.integers(8, 300)).astype(np.int32)
                             for _ in range(mb)])
    window = None
    sinks = 0
    if rng.integers(0, 3) > 0:
        window = int(rng.choice([-3, 0, 1, 2, 64, 127, 128, 129, 200, 255, 256, 257, 700, 5000]))
        if rng.integers(0, 2):
            sinks = int(rng.choice([1, 4, 127, 128, 129, 300]))
    return MaskSpecData(T, causal=causal, document=document, doc_ids=docs,
                        window=window, sinks=sinks)


def test_brute_force_python_tiny():
    """C counter == pure-Python per-pair loops on tiny random specs."""
    rng = np.random.default_rng(11)
    for _ in range(6):
        spec = _random_spec(rng, 256)
        assert np.array_equal(oracle.tile_counts(spec), _pairs_python(spec)), spec


def test_brute_force_dense_numpy_random():
    """C counter == dense [T, T] boolean mask reduced per tile, random specs
    (monotone and non-monotone document ids, windows, sinks, T up to 2048)."""
    rng = np.random.default_rng(12)
    for T in (128, 256, 384, 1024, 2048):
        for _ in range(8):
            spec = _random_spec(rng, T)
            assert np.array_equal(oracle.tile_counts(spec), oracle.tile_counts_dense_numpy(spec)), spec


def test_lists_from_counts():
    """Lists: ascending, -1 padded, partial/full split, transposed view."""
    counts = np.array([[[0, 16384, 5], [16384, 0, 16384], [1, 2, 0]]], dtype=np.int32)
    bm = oracle.block_mask_lists(counts)
    assert bm["kv_num_blocks"].tolist() == [[[1, 0, 2]]]
    assert bm["kv_indices"].tolist() == [[[[2, -1, -1], [-1, -1, -1], [0, 1, -1]]]]
    assert bm["full_kv_num_blocks"].tolist() == [[[1, 2, 0]]]
    assert bm["full_kv_indices"].tolist() == [[[[1, -1, -1], [0, 2, -1], [-1, -1, -1]]]]
    assert bm["q_num_blocks"].tolist() == [[[1, 1, 1]]]
    assert bm["q_indices"].tolist() == [[[[2, -1, -1], [2, -1, -1], [0, -1, -1]]]]
    assert bm["full_q_num_blocks"].tolist() == [[[1, 1, 1]]]
    assert bm["full_q_indices"].tolist() == [[[[1, -1, -1], [0, -1, -1], [1, -1, -1]]]]


def test_config_masks_bounded_by_nodoc():
    """Adding the document term can only remove pairs: per tile the count with
    documents never exceeds the count without (configs 1, 2 shape at 8K)."""
    for key, T in ((1, None), (2, 8192)):
        w = make_config(key, T=T)
        c_doc = oracle.tile_counts(w.spec)
        nodoc = MaskSpecData(w.T, causal=True, window=w.spec.window)
        c_nodoc = oracle.tile_counts(nodoc)
        assert np.all(c_doc <= c_nodoc)
        assert int((c_doc > 0).sum()) < int((c_nodoc > 0).sum())


@pytest.mark.parametrize("P", [0, 1, 640, 677, 8192])
def test_prefix_lm_closed_form(P):
    """Causal with a prefix of P = 128 p + r positions every query sees
    (prefix-LM masking, tutorial introduction), T = 8192: the causal triangle
    plus, above the diagonal, the p (p - 1) / 2 tiles inside the prefix
    (full) and, when r > 0, tile column p for the rows before it (partial).
    The diagonal tiles inside the prefix are full."""
    T = 8192
    nt, p, r = T // 128, P // 128, P % 128
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(T, causal=True, prefix=P)))
    visible = nt * (nt + 1) // 2 + p * (p - 1) // 2 + (p if r else 0)
    full = nt * (nt - 1) // 2 + p * (p + 1) // 2
    assert int((cls > 0).sum()) == visible
    assert int((cls == oracle.FULL).sum()) == full


def _random_prefix_spec(rng, T):
    spec = _random_spec(rng, T)
    spec.prefix = int(rng.choice([1, 37, 128, 129, 300, T]))
    return spec


def test_prefix_brute_force():
    """With the prefix term: C counter == pure-Python per-pair loops (T = 256)
    and == the dense [T, T] mask reduction (T up to 1024), random specs."""
    rng = np.random.default_rng(13)
    for _ in range(4):
        spec = _random_prefix_spec(rng, 256)
        assert np.array_equal(oracle.tile_counts(spec), _pairs_python(spec)), spec
    for T in (128, 384, 1024):
        for _ in range(6):
            spec = _random_prefix_spec(rng, T)
            assert np.array_equal(oracle.tile_counts(spec), oracle.tile_counts_dense_numpy(spec)), spec


# ---------------------------------------------------------- Q_LEN != KV_LEN,
# lengths that are not multiples of 128, composed masks

# Truth tables of the five terms alone: bit `idx` of a term's table is set
# when the term's own bit is set in idx (C 1, Dc 2, W 4, S 8, P 16).
T_C, T_D, T_W, T_S, T_P = 0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0, 0xFF00FF00, 0xFFFF0000
ALL = 0xFFFFFFFF


def _pairs_python_general(spec):
    """Pure-Python loops over every (query index, key) pair (tiny sizes),
    with absolute query positions and, when given, the truth table."""
    kv_len, q_len, off = spec.T, spec.Q, spec.q_offset
    nq, nk = -(-q_len // 128), -(-kv_len // 128)
    res = np.zeros((spec.mask_b, nq, nk), dtype=np.int64)
    for b in range(spec.mask_b):
        docs = None if spec.doc_ids is None else [int(x) for x in spec.doc_ids[b]]
        for qi in range(q_len):
            q = off + qi
            for kv in range(kv_len):
                c = q >= kv
                d = spec.document and docs[q] == docs[kv]
                w = spec.window is not None and (q - kv) < spec.window
                s = bool(spec.sinks) and kv < spec.sinks
                p = bool(spec.prefix) and kv < spec.prefix
                if spec.table is not None:
                    ok = (spec.table >> (c + 2 * d + 4 * w + 8 * s + 16 * p)) & 1
                else:
                    ok = ((not spec.causal) or c or p) and ((not spec.document) or d) and \
                         (spec.window is None or w or s)
                if ok:
                    res[b, qi // 128, kv // 128] += 1
    return res


@pytest.mark.parametrize("T", [1000, 129, 383, 65535])
def test_ragged_causal_closed_form(T):
    """Causal with T = 128 n + r, 0 < r < 128: ceil(T/128) = n + 1 tiles per
    side; the (n+1)(n+2)/2 tiles on or below the diagonal are visible; full
    are only the n(n-1)/2 strictly below it among whole tiles -- the last
    row and column hold r < 128 positions, so no tile of theirs is full."""
    n = T // 128
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(T, causal=True)))
    assert cls.shape == (1, n + 1, n + 1)
    assert int((cls > 0).sum()) == (n + 1) * (n + 2) // 2
    assert int((cls == oracle.FULL).sum()) == n * (n - 1) // 2


@pytest.mark.parametrize("a,c", [(2, 6), (1, 0), (3, 5), (8, 504)])
def test_rectangular_bottom_right_causal_closed_form(a, c):
    """Q_LEN = 128 a queries at the end of KV_LEN = 128 (c + a) keys
    (q_offset = 128 c), causal: query-tile row i sees key tiles 0 .. c + i,
    all full but the diagonal one, so c a + a (a + 1) / 2 visible and
    c a + a (a - 1) / 2 full."""
    spec = MaskSpecData(128 * (c + a), causal=True, q_len=128 * a, q_offset=128 * c)
    cls = oracle.classify(oracle.tile_counts(spec))
    assert cls.shape == (1, a, c + a)
    assert int((cls > 0).sum()) == c * a + a * (a + 1) // 2
    assert int((cls == oracle.FULL).sum()) == c * a + a * (a - 1) // 2


def test_single_query_rows_are_partial():
    """One query (the decoding shape: Q_LEN 1 at position KV_LEN - 1), causal:
    every key tile holds a visible pair and none can be full."""
    for L in (1, 127, 128, 129, 1000, 4096):
        cls = oracle.classify(oracle.tile_counts(MaskSpecData(L, causal=True, q_len=1, q_offset=L - 1)))
        assert cls.shape == (1, 1, -(-L // 128))
        assert np.all(cls == oracle.PARTIAL)


def test_composed_closed_forms_64k():
    """Truth tables at T = 65,536 (512 tiles per side):
      * NOT causal (kv > q): the 130,816 tiles above the diagonal, full, and
        the 512 diagonal tiles, partial;
      * the window alone, no causal term (q - kv < 1024): every tile on or
        above the diagonal is full (q - kv <= 127 < 1024 there) and below it
        diagonal d holds differences 128 d - 127 .. 128 d + 127, so diagonals
        1..8 are visible and 1..7 full (128 * 7 + 127 = 1023 < 1024);
      * causal AND (window OR sink) written as a table equals Pattern 2 at
        32K (2,515 tiles, 1,764 full)."""
    T, n = 65536, 512
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(T, table=ALL ^ T_C)))
    assert int((cls > 0).sum()) == n * (n + 1) // 2 and int((cls == oracle.FULL).sum()) == n * (n - 1) // 2
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(T, window=1024, table=T_W)))
    upper = n * (n + 1) // 2
    assert int((cls > 0).sum()) == upper + sum(n - d for d in range(1, 9))
    assert int((cls == oracle.FULL).sum()) == upper + sum(n - d for d in range(1, 8))
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(32768, window=1024, sinks=4, table=T_C & (T_W | T_S))))
    assert int((cls > 0).sum()) == 2515 and int((cls == oracle.FULL).sum()) == 1764


def _equivalent_table(spec):
    """The standard combination of the spec's terms as a truth table,
    enumerated over the 32 term combinations."""
    t = 0
    for idx in range(32):
        c, d, w, s, p = (bool(idx & k) for k in (1, 2, 4, 8, 16))
        ok = ((not spec.causal) or c or p) and ((not spec.document) or d) and (spec.window is None or w or s)
        t |= int(ok) << idx
    return t


def _random_general_spec(rng, table=False):
    kv_len = int(rng.choice([1, 77, 128, 129, 300, 384, 700]))
    q_len = int(rng.choice([1, 5, 128, 200, kv_len]))
    q_off = int(rng.choice([0, max(0, kv_len - q_len), 3, 130]))
    npos = max(kv_len, q_off + q_len)
    spec = _random_spec(rng, npos)
    spec.T, spec.q_len, spec.q_offset = kv_len, q_len, q_off
    spec.prefix = int(rng.choice([0, 0, 40, 129]))
    if table:
        spec.table = int(rng.integers(0, 2 ** 32))
    return spec


def test_general_brute_force_python_tiny():
    """C counter == pure-Python per-pair loops on random rectangular, ragged
    and composed specs."""
    rng = np.random.default_rng(21)
    for it in range(10):
        spec = _random_general_spec(rng, table=bool(it % 2))
        assert np.array_equal(oracle.tile_counts(spec), _pairs_python_general(spec)), spec


def test_general_brute_force_dense_numpy():
    """C counter == the dense-mask reduction (numpy predicate) on random
    rectangular, ragged and composed specs."""
    rng = np.random.default_rng(22)
    for it in range(40):
        spec = _random_general_spec(rng, table=bool(it % 2))
        assert np.array_equal(oracle.tile_counts(spec), oracle.tile_counts_dense_numpy(spec)), spec


def test_table_of_the_standard_combination_gives_the_same_counts():
    """A truth table written out from the standard combination (causal OR
    prefix) AND document AND (window OR sink) classifies every tile as the
    standard path does, on random square and rectangular specs."""
    rng = np.random.default_rng(23)
    for it in range(30):
        spec = _random_general_spec(rng) if it % 2 else _random_spec(rng, int(rng.choice([256, 384, 1024])))
        ref = oracle.tile_counts(spec)
        spec.table = _equivalent_table(spec)
        assert np.array_equal(oracle.tile_counts(spec), ref), spec


# ------------------------------------------------ 64-key blocks (tutorial,
# "What to expect, and the sharp edges", item 4: block size is a tunable)

def _pairs_python_blocks(spec, tq, tk):
    """Pure-Python loops over every pair of a standard-combination spec,
    counted into tq x tk blocks (tiny sizes)."""
    kv_len, q_len, off = spec.T, spec.Q, spec.q_offset
    res = np.zeros((spec.mask_b, -(-q_len // tq), -(-kv_len // tk)), dtype=np.int64)
    for b in range(spec.mask_b):
        docs = None if spec.doc_ids is None else [int(x) for x in spec.doc_ids[b]]
        for qi in range(q_len):
            q = off + qi
            for kv in range(kv_len):
                ok = ((not spec.causal) or q >= kv or (bool(spec.prefix) and kv < spec.prefix)) and \
                     ((not spec.document) or docs[q] == docs[kv]) and \
                     (spec.window is None or (q - kv) < spec.window or (bool(spec.sinks) and kv < spec.sinks))
                if ok:
                    res[b, qi // tq, kv // tk] += 1
    return res


def test_64_key_blocks_brute_force_python():
    rng = np.random.default_rng(640)
    for it in range(6):
        T = int(rng.choice([64, 100, 200, 300]))
        Q = int(rng.choice([T, 1, 77, 150]))
        off = int(rng.integers(0, T + 1))
        docs = np.cumsum(rng.random(max(T, off + Q)) < 1 / 30).astype(np.int32)[None]
        spec = MaskSpecData(T, causal=bool(it % 3), document=bool(it % 2), doc_ids=docs,
                            window=int(rng.choice([5, 40, 90])) if it % 2 else None, sinks=3 if it == 3 else 0,
                            prefix=20 if it == 4 else 0, q_len=Q, q_offset=off)
        got = oracle.tile_counts(spec, 128, 64)
        assert np.array_equal(got, _pairs_python_blocks(spec, 128, 64)), it
        assert np.array_equal(got, oracle.tile_counts_dense_numpy(spec, 128, 64)), it


@pytest.mark.parametrize("T", [1024, 8192, 8192 + 77])
def test_64_key_blocks_causal_closed_form(T):
    """Causal, 128 x 64 blocks, n = T // 128 whole query tiles: row i sees
    key blocks 0 .. 2i + 1, of which the first 2i are full (every key below
    the row's first query).  A cut-short last row (T = 128 n + r) sees
    every key block, ceil(T/64) of them, and holds r < 128 queries, so none
    of its blocks is full."""
    n, r = divmod(T, 128)
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(T, causal=True), 128, 64), 128, 64)
    vis = n * (n + 1)
    full = n * (n - 1)
    if r:
        vis += -(-T // 64)  # the last row sees every key block
    assert int((cls > 0).sum()) == vis
    assert int((cls == oracle.FULL).sum()) == full


def _window_blocks_closed_form(n, w, tk):
    """Causal + window w at 128 x tk blocks, T = 128 n: block (i, j) holds
    differences q - k from 128 i - tk j - tk + 1 to 128 i + 127 - tk j; it
    is visible iff the largest is >= 0 and the smallest < w, full iff the
    smallest is >= 0 and the largest < w.  Arithmetic per block, no pairs."""
    vis = full = 0
    for i in range(n):
        for j in range(n * 128 // tk):
            lo, hi = 128 * i - tk * j - tk + 1, 128 * i + 127 - tk * j
            if hi >= 0 and lo < w:
                vis += 1
                if lo >= 0 and hi < w:
                    full += 1
    return vis, full


@pytest.mark.parametrize("w", [1, 64, 100, 640, 1024, 1792])
def test_64_key_blocks_window_closed_form(w):
    T = 8192
    cls = oracle.classify(oracle.tile_counts(MaskSpecData(T, causal=True, window=w), 128, 64), 128, 64)
    vis, full = _window_blocks_closed_form(T // 128, w, 64)
    assert int((cls > 0).sum()) == vis
    assert int((cls == oracle.FULL).sum()) == full
    # and the same arithmetic gives the 128 x 128 counts
    cls128 = oracle.classify(oracle.tile_counts(MaskSpecData(T, causal=True, window=w)))
    assert (int((cls128 > 0).sum()), int((cls128 == oracle.FULL).sum())) == _window_blocks_closed_form(T // 128, w, 128)


def test_64_key_blocks_refine_128_tiles():
    """Counts of the two 64-key halves add up to the 128 x 128 tile's; a
    tile is full iff both halves are, empty iff both are.  Row lists of a
    kv_block = 64 spec index 64-key blocks, column lists 128 x 128 tiles."""
    rng = np.random.default_rng(641)
    T = 1000
    docs = np.cumsum(rng.random(T) < 1 / 150).astype(np.int32)[None]
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs, window=300, sinks=4, kv_block=64)
    c64 = oracle.tile_counts(spec, 128, 64)
    c128 = oracle.tile_counts(spec)
    pad = np.zeros(c64.shape[:2] + (2 * c128.shape[2],), dtype=np.int64)
    pad[..., :c64.shape[2]] = c64
    assert np.array_equal(pad.reshape(c64.shape[0], c64.shape[1], -1, 2).sum(axis=3), c128)
    k64 = oracle.classify(c64, 128, 64)
    k128 = oracle.classify(c128)
    for j in range(c128.shape[2]):
        halves = k64[..., 2 * j:2 * j + 2]
        both_full = np.all(halves == oracle.FULL, axis=-1) & (halves.shape[-1] == 2)
        assert np.array_equal(k128[..., j] == oracle.FULL, both_full)
        assert np.array_equal(k128[..., j] == oracle.EMPTY, np.all(halves == oracle.EMPTY, axis=-1))
    lists = oracle.spec_block_mask_lists(spec)
    assert lists["kv_indices"].shape == (1, 1, 8, 16)
    assert lists["q_indices"].shape == (1, 1, 8, 8)
    ref128 = oracle.block_mask_lists(c128)
    for n in ("q_num_blocks", "q_indices", "full_q_num_blocks", "full_q_indices"):
        assert np.array_equal(lists[n], ref128[n]), n
