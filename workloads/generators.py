"""Seeded generators for the five synthetic workloads of block-sparse masked
attention (FlexAttention-style document, window and sink masks).

Sources of the shapes and distributions:
  * document ids as the running count of end-of-text flags -- speedrun notes
    "FlexAttention", code listing (docs = cumsum(tokens == EOT));
  * 65,536-token packed sequences with a 1024 window -- same page, Record #12;
  * window swept 64..1792 in steps of 64 -- same page, Record #13;
  * B=4, H=16, S=8192, D=64 causal and the 4-sink / 1024-window pattern --
    tutorial "FlexAttention in PyTorch", quick start and Pattern 2;
  * ALiBi and 30*tanh(s/30) soft-cap -- same tutorial, Pattern 3.

The token stream behind the speedrun is not available, so document lengths are
drawn from the stated distributions instead (Geometric via i.i.d. end-of-text
flags, or log-normal with median 500 and sigma 1.0, clipped to [16, 65,536]).

Random values: numpy.random.default_rng(seed) for document structure, and
torch.Generator('cpu').manual_seed(seed) for q, k, v, dO in that order, each
drawn as float32 N(0,1) and rounded to bfloat16 (round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass
class MaskSpecData:
    """Plain description of a mask predicate.

    T           -- number of key positions (KV_LEN)
    q_len       -- number of queries (Q_LEN; None: T); query i sits at
                   absolute position q_offset + i
    causal      -- q >= kv
    document    -- doc_ids[b, q] == doc_ids[b, kv]; doc_ids has shape
                   [mask_b, positions], positions = max(T, q_offset + q_len)
    window      -- q - kv < window   (None: no window term)
    sinks       -- kv < sinks, OR-ed with the window term (0: none)
    prefix      -- kv < prefix, OR-ed with the causal term (prefix-LM: the
                   first `prefix` positions are seen by every query; 0: none)
    kv_block    -- key-block width of the block mask's row lists: 128, or 64
                   for finer blocks (128 queries x 64 keys)
    table       -- None: the terms combine as above.  Otherwise a 32-bit truth
                   table over the five terms: the pair is visible iff bit
                   (C + 2 Dc + 4 W + 8 S + 16 P) of it is set, with C = q >= kv,
                   Dc = same document, W = q - kv < window, S = kv < sinks,
                   P = kv < prefix (a term whose data is absent -- no document
                   ids, no window -- is 0; the flags above are then unused
                   except to say which data exist)
    """
    T: int
    causal: bool = True
    document: bool = False
    doc_ids: Optional[np.ndarray] = None  # int32 [mask_b, positions]
    window: Optional[int] = None
    sinks: int = 0
    prefix: int = 0
    q_len: Optional[int] = None
    q_offset: int = 0
    table: Optional[int] = None
    kv_block: int = 128

    @property
    def mask_b(self) -> int:
        return 1 if self.doc_ids is None else int(self.doc_ids.shape[0])

    @property
    def Q(self) -> int:
        """Number of queries."""
        return self.T if self.q_len is None else int(self.q_len)

    @property
    def positions(self) -> int:
        """Positions covered by the document ids: keys and queries."""
        return max(self.T, self.q_offset + self.Q)


@dataclasses.dataclass
class ScoreModData:
    """ALiBi slopes (float32 [H]), a soft-cap value (None: off) and a
    relative-position bias table (float32 [H, 2R + 1], entry R + d for the
    query-key distance d in [-R, R]; None: off)."""
    alibi_slopes: Optional[np.ndarray] = None
    softcap: Optional[float] = None
    bias_table: Optional[np.ndarray] = None


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H: int
    T: int
    D: int
    spec: MaskSpecData
    mod: ScoreModData
    seed: int
    backward: bool = False
    windows: Optional[list] = None  # window sweep (config 3)
    dtype: str = "bf16"             # element type of q, k, v, dout: "bf16" or "f16"

    def tensors(self, with_dout: Optional[bool] = None) -> dict:
        """q, k, v (and dout) as CPU tensors [B, H, T, D] of the workload's
        element type (bfloat16 unless dtype says float16)."""
        if with_dout is None:
            with_dout = self.backward
        g = torch.Generator("cpu").manual_seed(self.seed)
        names = ["q", "k", "v"] + (["dout"] if with_dout else [])
        rand = random_f16 if self.dtype == "f16" else random_bf16
        return {n: rand((self.B, self.H, self.T, self.D), g) for n in names}


def random_bf16(shape, generator: torch.Generator) -> torch.Tensor:
    return torch.randn(shape, generator=generator, dtype=torch.float32).to(torch.bfloat16)


def random_f16(shape, generator: torch.Generator) -> torch.Tensor:
    """The same N(0, 1) draws rounded to fp16 (round-to-nearest-even)."""
    return torch.randn(shape, generator=generator, dtype=torch.float32).to(torch.float16)


def doc_ids_from_eot_flags(flags: np.ndarray) -> np.ndarray:
    """Document id of every position: the running count of end-of-text flags
    (the flagged position opens the next document)."""
    return np.cumsum(flags.astype(np.int64)).astype(np.int32)


def doc_ids_geometric(T: int, mean: float, rng: np.random.Generator) -> np.ndarray:
    """i.i.d. Bernoulli(1/mean) end-of-text flags; gaps are Geometric(mean)."""
    flags = rng.random(T) < (1.0 / mean)
    return doc_ids_from_eot_flags(flags)


def doc_ids_lognormal(T: int, median: float, sigma: float, lo: int, hi: int,
                      rng: np.random.Generator) -> np.ndarray:
    """Concatenate documents of log-normal length (rounded, clipped to
    [lo, hi]) until T positions are covered; the last one is truncated."""
    ids = np.empty(T, dtype=np.int32)
    pos, d = 0, 0
    mu = np.log(median)
    while pos < T:
        n = int(np.clip(np.rint(rng.lognormal(mu, sigma)), lo, hi))
        n = min(n, T - pos)
        ids[pos:pos + n] = d
        pos += n
        d += 1
    return ids


def doc_ids_chunks(T: int, chunk: int) -> np.ndarray:
    """Independent fixed-size chunks: position i belongs to chunk i // chunk."""
    return (np.arange(T, dtype=np.int64) // chunk).astype(np.int32)


def bias_table(H: int, R: int, seed: int, sd: float = 1.0) -> np.ndarray:
    """A synthetic learned relative-position bias: float32 [H, 2R + 1] of
    N(0, sd^2) draws from numpy's default_rng(seed)."""
    return (np.random.default_rng(seed).standard_normal((H, 2 * R + 1)) * sd).astype(np.float32)


def alibi_slopes(H: int) -> np.ndarray:
    """slope[h] = 2^(-8 (h+1) / H), h = 0..H-1."""
    h = np.arange(H, dtype=np.float64)
    return np.power(2.0, -8.0 * (h + 1.0) / H).astype(np.float32)


CONFIG_NAMES = {
    1: "tiny: B1 H2 T1024 D64 causal+document(Geometric 256)",
    2: "packed 64K: B1 H6 T65536 D128 causal+document(log-normal 500)+window 1024",
    "2-causal": "B1 H6 T65536 D128 causal",
    "2-window": "B1 H6 T65536 D128 causal+window 1024",
    "2-chunks": "B1 H6 T65536 D128 causal within 1024-token chunks",
    3: "window sweep 64..1792 on the 64K packed-document shape",
    "4a": "B4 H16 S8192 D64 causal",
    "4b": "B1 H16 S32768 D64 causal+(window 1024 | 4 sinks)",
    5: "B2 H16 S16384 D128 causal+document(Geometric 1024) ALiBi+softcap 30, fwd+bwd",
    "decode": "decoding step: B8 H32 cache 32768 D128 causal, one query per (b, h)",
    "decode-docs": "decoding step: B8 H32 cache 32768 D128 causal+document(log-normal 500) with the block mask",
}


def make_config(key, *, seed: Optional[int] = None, T: Optional[int] = None,
                B: Optional[int] = None, H: Optional[int] = None) -> Workload:
    """Build one of the named workloads. T, B, H may be overridden to get a
    smaller instance with the same structure (used by tests)."""
    k = str(key)
    base_seed = {"1": 1, "2": 2, "2-causal": 2, "2-window": 2, "2-chunks": 2,
                 "3": 3, "4a": 4, "4b": 4, "5": 5, "decode": 6, "decode-docs": 6}[k]
    seed = base_seed if seed is None else seed
    rng = np.random.default_rng(seed)
    if k == "1":
        B_, H_, T_, D = 1, 2, 1024, 64
        T_ = T or T_
        spec = MaskSpecData(T_, causal=True, document=True,
                            doc_ids=doc_ids_geometric(T_, 256, rng)[None, :])
        return Workload(CONFIG_NAMES[1], B or B_, H or H_, T_, D, spec, ScoreModData(), seed)
    if k in ("2", "3"):
        B_, H_, T_, D = 1, 6, 65536, 128
        T_ = T or T_
        docs = doc_ids_lognormal(T_, 500.0, 1.0, 16, 65536, rng)[None, :]
        spec = MaskSpecData(T_, causal=True, document=True, doc_ids=docs, window=1024)
        w = Workload(CONFIG_NAMES[int(k)], B or B_, H or H_, T_, D, spec, ScoreModData(), seed)
        if k == "3":
            w.windows = list(range(64, 1792 + 1, 64))
        return w
    if k == "2-causal":
        T_ = T or 65536
        return Workload(CONFIG_NAMES[k], B or 1, H or 6, T_, 128,
                        MaskSpecData(T_, causal=True), ScoreModData(), seed)
    if k == "2-window":
        T_ = T or 65536
        return Workload(CONFIG_NAMES[k], B or 1, H or 6, T_, 128,
                        MaskSpecData(T_, causal=True, window=1024), ScoreModData(), seed)
    if k == "2-chunks":
        T_ = T or 65536
        spec = MaskSpecData(T_, causal=True, document=True,
                            doc_ids=doc_ids_chunks(T_, 1024)[None, :])
        return Workload(CONFIG_NAMES[k], B or 1, H or 6, T_, 128, spec, ScoreModData(), seed)
    if k == "4a":
        T_ = T or 8192
        return Workload(CONFIG_NAMES[k], B or 4, H or 16, T_, 64,
                        MaskSpecData(T_, causal=True), ScoreModData(), seed)
    if k == "4b":
        T_ = T or 32768
        return Workload(CONFIG_NAMES[k], B or 1, H or 16, T_, 64,
                        MaskSpecData(T_, causal=True, window=1024, sinks=4),
                        ScoreModData(), seed)
    if k == "decode":
        T_ = T or 32768
        return Workload(CONFIG_NAMES[k], B or 8, H or 32, T_, 128, MaskSpecData(T_, causal=True),
                        ScoreModData(), seed)
    if k == "decode-docs":
        B_, T_ = B or 8, T or 32768
        docs = np.stack([doc_ids_lognormal(T_, 500.0, 1.0, 16, 65536, rng) for _ in range(B_)])
        return Workload(CONFIG_NAMES[k], B_, H or 32, T_, 128,
                        MaskSpecData(T_, causal=True, document=True, doc_ids=docs), ScoreModData(), seed)
    if k == "5":
        B_, H_, T_, D = 2, 16, 16384, 128
        B_ = B or B_
        H_ = H or H_
        T_ = T or T_
        docs = np.stack([doc_ids_geometric(T_, 1024, rng) for _ in range(B_)])
        spec = MaskSpecData(T_, causal=True, document=True, doc_ids=docs)
        mod = ScoreModData(alibi_slopes=alibi_slopes(H_), softcap=30.0)
        return Workload(CONFIG_NAMES[5], B_, H_, T_, D, spec, mod, seed, backward=True)
    raise KeyError(key)
