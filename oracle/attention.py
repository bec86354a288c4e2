"""Decode attention, attention states and their merge, in float64 (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (pages are cited by title and section):

* [KANTHI] "Flash-Decoding: Split-KV Attention for Long-Context Decode"
  (kanthi.in book chapter): §1 defines the scores and the output; §2 defines
  the attention state (o(I), LSE(I)), the merge for disjoint key sets and its
  max-subtracted stable form; §3 splits with uneven ``linspace`` boundaries;
  §4 splits by ``chunk = cdiv(T_max, S)`` and gives the empty-split rule.
* [XUUJII] "Decode 专项 Attention：把长KV拆开算，再正确合并" (xuujii KB):
  §04 keeps per block the state (m, ℓ, u) = (max score, Σexp(s−m),
  Σexp(s−m)·v) and merges by rebasing to the common max; §06 says a fully
  masked block contributes zero and exp(−∞−(−∞)) must never be formed.
* [AIFETCHLY] "FlashDecoding: Fast Long-Context Generation Guide": the fixed
  chunk C (1024) partition.

Readings where the pages are silent:

* A query row whose sequence has no visible key (seq_len = 0) returns
  o = 0 and LSE = −∞, the same convention as an empty split ([KANTHI] §4;
  [XUUJII] §06 leaves the choice to the backend).
* GQA maps query head ``hq`` to KV head ``hq // g`` with g = Hq / Hkv
  ([KANTHI] §1 GQA note says only that a group of query heads shares one KV
  head; contiguous groups are the plainest reading).
* The LSE is a natural logarithm ([KANTHI] §2 writes log; §8 asks that the
  base be stated).
* Paged pools are ``[num_pages, page_size, Hkv, D]`` and token t of sequence
  b is row ``t % page_size`` of page ``block_table[b, t // page_size]``
  ([KANTHI] §7 and §9 name a pool plus block table but no layout).
* A short query block (speculative decode, [KANTHI] §7 "Short query blocks"
  and §9 item 1: q is [B, q_len, Hq, D]) holds the last q_len positions of
  the sequence, whose keys are already in the cache; row i sees the first
  seq_len − (q_len − 1 − i) tokens ([XUUJII] §06: every query keeps its own
  visibility). Rows that see no token follow the empty-row convention.

Every stored input (fp16, bf16 or fp32) is upcast exactly to float64; all
arithmetic below is float64.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# Input handling
# ---------------------------------------------------------------------------

def f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (any float dtype, any device) or array to float64."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64)
    import torch  # local: the oracle also works on plain arrays

    return x.detach().to("cpu").to(torch.float64).numpy()


def ints(x) -> np.ndarray:
    if isinstance(x, (list, tuple)):
        return np.asarray(x, dtype=np.int64)
    if isinstance(x, np.ndarray):
        return x.astype(np.int64)
    return x.detach().to("cpu").to(dtype=__import__("torch").int64).numpy()


def default_scale(head_dim: int) -> float:
    """1/sqrt(d), the score scale of [KANTHI] §1."""
    return 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------
# The definition ([KANTHI] §1 and §2)
# ---------------------------------------------------------------------------

def scores(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """s_i = scale · qᵀk_i for every key row of ``K`` ([KANTHI] §1 equation)."""
    return (K @ q) * scale


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Tuple[np.ndarray, float]:
    """Full softmax attention of one query row over the keys of ``K``/``V``.

    o = Σ_i softmax(s)_i v_i and LSE = log Σ_i e^{s_i} ([KANTHI] §1 and the
    definition of LSE(I) in §2). Written with the maximum factored out, which
    changes nothing mathematically. No keys: (0, −∞).
    """
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), NEG_INF
    s = scores(q, K, scale)
    m = float(s.max())
    p = np.exp(s - m)
    den = float(p.sum())
    return (p @ V) / den, m + math.log(den)


def segment_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float
                  ) -> Tuple[float, float, np.ndarray]:
    """The (m, ℓ, u) state of one KV segment ([XUUJII] §04):
    m = max_i s_i, ℓ = Σ_i e^{s_i − m}, u = Σ_i e^{s_i − m} v_i.
    An empty segment is (−∞, 0, 0) ([KANTHI] §4 empty-split rule)."""
    if K.shape[0] == 0:
        return NEG_INF, 0.0, np.zeros(V.shape[1])
    s = scores(q, K, scale)
    m = float(s.max())
    p = np.exp(s - m)
    return m, float(p.sum()), p @ V


def state_to_olse(m: float, l: float, u: np.ndarray) -> Tuple[np.ndarray, float]:
    """(m, ℓ, u) -> (o, LSE): o = u/ℓ and LSE = m + log ℓ ([XUUJII] §04 notes
    u = ℓ·o; [KANTHI] §2 defines LSE). Empty -> (0, −∞)."""
    if m == NEG_INF or l == 0.0:
        return np.zeros_like(u), NEG_INF
    return u / l, m + math.log(l)


def merge_uml(states: Sequence[Tuple[float, float, np.ndarray]]) -> Tuple[float, float, np.ndarray]:
    """Merge (m, ℓ, u) states by rebasing to the common maximum ([XUUJII] §04):
    m = max_j m_j, α_j = e^{m_j − m}, ℓ = Σ α_j ℓ_j, u = Σ α_j u_j.
    A state with m_j = −∞ gets weight 0 explicitly ([XUUJII] §06: never form
    e^{−∞−(−∞)}); if every state is empty the result is (−∞, 0, 0)."""
    d = len(states[0][2])
    m = max(st[0] for st in states)
    if m == NEG_INF:
        return NEG_INF, 0.0, np.zeros(d)
    l = 0.0
    u = np.zeros(d)
    for mj, lj, uj in states:
        if mj == NEG_INF:
            continue
        a = math.exp(mj - m)
        l += a * lj
        u = u + a * uj
    return m, l, u


def merge_olse(states: Sequence[Tuple[np.ndarray, float]]) -> Tuple[np.ndarray, float]:
    """Merge (o, LSE) states with the stable form of [KANTHI] §2:
    m = max_j LSE_j, w_j = e^{LSE_j − m}, o = Σ w_j o_j / Σ w_j,
    LSE = m + log Σ w_j. Empty states (LSE = −∞) weigh 0; all empty -> (0, −∞)."""
    d = len(states[0][0])
    m = max(st[1] for st in states)
    if m == NEG_INF:
        return np.zeros(d), NEG_INF
    num = np.zeros(d)
    den = 0.0
    for oj, lj in states:
        if lj == NEG_INF:
            continue
        w = math.exp(lj - m)
        num = num + w * oj
        den += w
    return num / den, m + math.log(den)


# ---------------------------------------------------------------------------
# Split partitions
# ---------------------------------------------------------------------------

def chunk_bounds(seq_len: int, chunk: int, num_splits: int) -> List[Tuple[int, int]]:
    """Split s covers [s·chunk, min(s·chunk + chunk, seq_len)) ([KANTHI] §4
    split kernel; with chunk = C this is the fixed-chunk partition of
    [AIFETCHLY] "The Two-Stage Execution Model"). A split starting at or past
    seq_len is empty and is returned as (start, start)."""
    out = []
    for s in range(num_splits):
        a = s * chunk
        b = min(a + chunk, seq_len)
        out.append((a, max(a, b)))
    return out


def alternating_bounds(seq_len: int, even_chunk: int, odd_chunk: int, num_splits: int) -> List[Tuple[int, int]]:
    """The partition of chunk_bounds with two alternating lengths: split s
    holds even_chunk tokens for even s and odd_chunk for odd s, starting where
    split s - 1 ends, clipped at seq_len; a split starting at or past seq_len
    is empty and is returned as (start, start). Any contiguous partition
    merges to the same result ([KANTHI] §2); this one lets the splits that
    run on slower hardware units hold fewer tokens."""
    out = []
    a = 0
    for s in range(num_splits):
        n = even_chunk if s % 2 == 0 else odd_chunk
        out.append((a, max(a, min(a + n, seq_len))))
        a += n
    return out


def linspace_bounds(total: int, num_splits: int) -> List[int]:
    """Uneven boundaries ``linspace(0, T, S+1)`` truncated to int ([KANTHI] §3)."""
    return np.linspace(0, total, num_splits + 1).astype(int).tolist()


# ---------------------------------------------------------------------------
# Cache access (layouts)
# ---------------------------------------------------------------------------

class Cache:
    """Read-only view of a decode step's inputs in float64.

    ``k``/``v`` are contiguous ``[B, Hkv, T, D]`` or, with ``block_table``,
    pools ``[P, page, Hkv, D]``. Rows are fetched per (b, kv head) on demand so
    sampled checks at full size never upcast the whole cache.
    """

    def __init__(self, q, k, v, seq_lens, block_table=None, scale: Optional[float] = None):
        self.q = f64(q)
        self._k = k
        self._v = v
        self.seq_lens = ints(seq_lens)
        self.block_table = None if block_table is None else ints(block_table)
        self.B, self.Hq, self.D = self.q.shape
        if self.block_table is None:
            self.Hkv = k.shape[1]
            self.page = 0
        else:
            self.Hkv = k.shape[2]
            self.page = k.shape[1]
        if self.Hq % self.Hkv:
            raise ValueError("query heads must be a multiple of KV heads")
        self.g = self.Hq // self.Hkv
        self.scale = default_scale(self.D) if not scale else float(scale)

    def kv_head(self, hq: int) -> int:
        """GQA head mapping: contiguous groups, hkv = hq // g."""
        return hq // self.g

    def rows(self, b: int, hkv: int, lo: int, hi: int) -> Tuple[np.ndarray, np.ndarray]:
        """K and V rows of tokens [lo, hi) of sequence b, kv head hkv, as float64."""
        if hi <= lo:
            return np.zeros((0, self.D)), np.zeros((0, self.D))
        if self.block_table is None:
            return f64(self._k[b, hkv, lo:hi]), f64(self._v[b, hkv, lo:hi])
        t = np.arange(lo, hi)
        pages = self.block_table[b, t // self.page]
        slots = t % self.page
        import torch

        pi = torch.as_tensor(pages)
        si = torch.as_tensor(slots)
        return f64(self._k[pi, si, hkv]), f64(self._v[pi, si, hkv])


# ---------------------------------------------------------------------------
# Whole decode step
# ---------------------------------------------------------------------------

def attention_one(cache: Cache, b: int, hq: int) -> Tuple[np.ndarray, float]:
    """Output and LSE of one (sequence, query head) by the definition."""
    L = int(max(0, cache.seq_lens[b]))
    K, V = cache.rows(b, cache.kv_head(hq), 0, L)
    return attend(cache.q[b, hq], K, V, cache.scale)


def decode_attention(cache: Cache, pairs: Optional[Iterable[Tuple[int, int]]] = None):
    """O [B, Hq, D] and LSE [B, Hq] in float64 by the definition, one query head
    at a time (no GQA packing). With ``pairs`` only those (b, hq) are computed and
    the rest are NaN."""
    O = np.full((cache.B, cache.Hq, cache.D), np.nan)
    LSE = np.full((cache.B, cache.Hq), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(cache.B) for h in range(cache.Hq)]
    for b, hq in todo:
        O[b, hq], LSE[b, hq] = attention_one(cache, b, hq)
    return O, LSE


def block_row_cache(q_block, k, v, seq_lens, i: int, block_table=None, scale: Optional[float] = None) -> Cache:
    """Row i of a short query block as a single-query decode step: query
    q_block[:, i] over the first seq_len − (q_len − 1 − i) tokens (clamped at 0)."""
    q_len = q_block.shape[1]
    lens = ints(seq_lens) - (q_len - 1 - i)
    return Cache(q_block[:, i], k, v, np.maximum(lens, 0), block_table, scale)


def decode_attention_block(q_block, k, v, seq_lens, block_table=None, scale: Optional[float] = None,
                           rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """O [B, q_len, Hq, D] and LSE [B, q_len, Hq] of a short query block, by the
    definition: each (b, i, hq) attends to its visible prefix. With ``rows``
    only those (b, i, hq) are computed and the rest are NaN."""
    B, q_len, Hq, D = q_block.shape
    O = np.full((B, q_len, Hq, D), np.nan)
    LSE = np.full((B, q_len, Hq), np.nan)
    want = None if rows is None else sorted(set(rows))
    for i in range(q_len):
        pairs = None if want is None else [(b, h) for b, ii, h in want if ii == i]
        if pairs == []:
            continue
        O[:, i], LSE[:, i] = decode_attention(block_row_cache(q_block, k, v, seq_lens, i, block_table, scale), pairs)
    return O, LSE


def split_states(cache: Cache, num_splits: int, chunk: int,
                 pairs: Optional[Iterable[Tuple[int, int]]] = None, bounds=None):
    """Per-split (m, ℓ, u) of every (b, hq) for the partition ``chunk_bounds``,
    or, with ``bounds(b, hkv) -> [(lo, hi), ...]`` (at most S entries; missing
    ones are empty splits), for that partition instead.
    Returns m [B, Hq, S], l [B, Hq, S], u [B, Hq, S, D] (NaN where not computed).
    m is the largest natural-log score of the split."""
    S = num_splits
    M = np.full((cache.B, cache.Hq, S), np.nan)
    Lw = np.full((cache.B, cache.Hq, S), np.nan)
    U = np.full((cache.B, cache.Hq, S, cache.D), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(cache.B) for h in range(cache.Hq)]
    for b, hq in todo:
        L = int(max(0, cache.seq_lens[b]))
        if bounds is None:
            parts = chunk_bounds(L, chunk, S)
        else:
            parts = list(bounds(b, cache.kv_head(hq)))
            assert len(parts) <= S
            parts += [(L, L)] * (S - len(parts))
        for s, (lo, hi) in enumerate(parts):
            K, V = cache.rows(b, cache.kv_head(hq), lo, hi)
            M[b, hq, s], Lw[b, hq, s], U[b, hq, s] = segment_state(cache.q[b, hq], K, V, cache.scale)
    return M, Lw, U


def split_then_merge(cache: Cache, bounds_for_len, pairs=None, form: str = "uml"):
    """The independent split-and-merge path: for each (b, hq), cut [0, L) with
    ``bounds_for_len(L) -> [(lo, hi), ...]``, take each segment's state and merge
    them with ``merge_uml`` (form "uml") or ``merge_olse`` (form "olse").
    Returns O [B, Hq, D] and LSE [B, Hq]."""
    O = np.full((cache.B, cache.Hq, cache.D), np.nan)
    LSE = np.full((cache.B, cache.Hq), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(cache.B) for h in range(cache.Hq)]
    for b, hq in todo:
        L = int(max(0, cache.seq_lens[b]))
        hkv = cache.kv_head(hq)
        sts = []
        for lo, hi in bounds_for_len(L):
            K, V = cache.rows(b, hkv, lo, hi)
            sts.append(segment_state(cache.q[b, hq], K, V, cache.scale))
        if form == "uml":
            O[b, hq], LSE[b, hq] = state_to_olse(*merge_uml(sts))
        else:
            O[b, hq], LSE[b, hq] = merge_olse([state_to_olse(*st) for st in sts])
    return O, LSE
