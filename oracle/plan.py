"""Split-count rules (oracle). TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "Flash-Decoding: Split-KV Attention for Long-Context Decode" (kanthi.in)
§6 "How many splits?" -- the wave-efficiency rule of the FlashAttention-2
dispatcher -- and the same rule as explained in the FA3 comment quoted in the
vatshank blog "Benchmarking split-KV against vanilla FA" (48 work items on 108
SMs: 2 splits give efficiency 0.89, 3 splits 0.67).

The rule, in words: launch W·S workgroups onto ``slots`` resident slots; a
split count S fills a fraction W·S/slots of the machine, and the last wave of
that launch is busy for frac(W·S/slots) of its length; S = 1 when W alone
already fills 80 % of the slots; otherwise among the split counts up to
min(max_splits, slots, n_blocks) that change the number of blocks per split,
take the smallest one whose efficiency is at least 85 % of the best.

``num_splits_fa2`` is that rule as the page states it (pinned by the page's
printed table and by the FA3 comment's two efficiencies). ``num_splits_traffic``
adds the overhead check at the end of §6 -- the fp32 workspace written and read
back, relative to the KV bytes, must stay under a budget -- generalised to g
query heads per KV head and (D + 2) floats per state; it is what the library's
planner runs with the MI355X slot count. Its choices on MI355X are
"parity unpinned": the pages give no MI355X numbers; measured split sweeps
justify the defaults instead.
"""
from __future__ import annotations

import math


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def wave_efficiency(work: int, splits: int, slots: int) -> float:
    """Busy fraction of the last wave: w / ceil(w) with w = work·splits/slots."""
    w = work * splits / slots
    return w / math.ceil(w)


def _eligible(s: int, n_blocks: int) -> bool:
    """A split count is worth trying only if it changes the blocks per split."""
    return s == 1 or cdiv(n_blocks, s) != cdiv(n_blocks, s - 1)


def num_splits_fa2(work: int, slots: int, n_blocks: int, max_splits: int = 128) -> int:
    """The §6 wave-efficiency rule."""
    if work >= 0.8 * slots:
        return 1
    cap = min(max_splits, slots, n_blocks)
    if cap <= 1:
        return 1
    cands = [s for s in range(1, cap + 1) if _eligible(s, n_blocks)]
    eff = {s: wave_efficiency(work, s, slots) for s in cands}
    best = max(eff.values())
    return min(s for s in cands if eff[s] >= 0.85 * best)


def workspace_ratio(splits: int, group: int, head_dim: int, kv_elt: int, max_len: int) -> float:
    """Workspace bytes (written by the split kernel, read by the merge) per KV byte
    for one (sequence, KV head): 2·S·g·(D+2)·4 / (2·L·D·elt). With g = 1, elt = 2
    and the (D+2) taken as D this is the 2S/t of the §6 overhead check."""
    if max_len <= 0:
        return math.inf
    return (2.0 * splits * group * (head_dim + 2) * 4.0) / (2.0 * max_len * head_dim * kv_elt)


def num_splits_traffic(work: int, slots: int, n_blocks: int, max_splits: int, group: int,
                       head_dim: int, kv_elt: int, max_len: int, budget: float,
                       threshold: float = 0.85) -> int:
    """The §6 rule restricted to split counts whose workspace traffic stays within
    ``budget`` of the KV bytes (S = 1 is always allowed), taking the smallest
    split count whose efficiency reaches ``threshold`` of the best (the page
    uses 0.85). Parity unpinned."""
    if work >= 0.8 * slots:
        return 1
    cap = min(max_splits, slots, n_blocks)
    if cap <= 1:
        return 1
    cands = [s for s in range(1, cap + 1) if _eligible(s, n_blocks)
             and (s == 1 or workspace_ratio(s, group, head_dim, kv_elt, max_len) <= budget)]
    eff = {s: wave_efficiency(work, s, slots) for s in cands}
    best = max(eff.values())
    return min(s for s in cands if eff[s] >= threshold * best)


def chunk_for(max_len: int, splits: int, align: int) -> int:
    """Tokens per split: cdiv(max_len, S) (the §4 wrapper of the kanthi.in chapter)
    rounded up to a multiple of ``align`` (KV page and/or tile; §7 aligns split
    boundaries to KV pages)."""
    c = max(1, cdiv(max(max_len, 1), splits))
    return cdiv(c, align) * align


def chunk_from_lengths(lengths, max_len: int, kv_heads: int, slots: int, align: int, max_splits: int,
                       group: int, head_dim: int, kv_elt: int, budget: float) -> int:
    """Tokens per split for a batch whose lengths are known on the host: no
    split longer than one slot's share of the total work, i.e. chunk =
    cdiv(Hkv * sum(len), slots) rounded up to ``align``, then enlarged until
    S = cdiv(max_len, chunk) respects ``max_splits`` and the workspace-traffic
    budget of the §6 overhead check (kanthi.in). ``max_len`` is the problem's
    bound on the lengths (the split grid spans it). With equal lengths this is
    the split count at which the wave-efficiency rule fills one wave exactly.
    Parity unpinned (derived from MI355X measurements)."""
    if max_len <= 0:
        return align
    total = kv_heads * sum(max(0, int(x)) for x in lengths)
    chunk = max(align, cdiv(cdiv(total, slots), align) * align)
    while True:
        s = cdiv(max_len, chunk)
        if s <= max(1, max_splits) and (s == 1 or workspace_ratio(s, group, head_dim, kv_elt, max_len) <= budget):
            return chunk
        chunk += align


def balanced_schedule(lengths, kv_heads: int, granule: int, slots: int, min_granules: int = 4, cost: int = 0,
                      odd_permille: int = 0):
    """The balanced split schedule, from its definition: segment (b, h) is
    cdiv(len_b, G) token granules followed by ``cost`` granules that hold no
    tokens (a piece's start-up cost; none for an empty segment); the
    segments, in (b, h) order, form one line of T granules; N = min(slots,
    cdiv(T, min_granules)) workgroups (1 if T = 0) take the ranges
    [floor(w T / N), floor((w + 1) T / N)); with ``odd_permille`` = x > 0
    range w instead holds 1000 + x parts (w even) or 1000 - x parts (w odd),
    its start being floor(T * (parts of ranges before w) / (all parts)), so
    that odd workgroups, which the hardware places on the slower odd XCDs,
    get less of the line. Every non-empty intersection of a
    range with a segment's token granules is one piece. Returns (N, S,
    pieces, T) with pieces[(b, h)] = [(w, token_lo, token_hi), ...] in
    workgroup order and S = the largest number of pieces of one segment (at
    least 1). It is a Stream-K-style partition of the kind kanthi.in §7 lists
    (LeanAttention), one that gives every workgroup the same bytes plus
    start-up costs. Parity unpinned as a performance choice; its partition is
    checked exhaustively in tests."""
    lens = [max(0, int(n)) for n in lengths]
    plens = [cdiv(n, granule) for n in lens]
    seg = [p + cost if p > 0 else 0 for p in plens]
    T = kv_heads * sum(seg)
    N = min(slots, cdiv(T, min_granules)) if T > 0 else 1
    parts = [1000 + odd_permille if w % 2 == 0 else 1000 - odd_permille for w in range(N)]
    before = [sum(parts[:w]) for w in range(N + 1)]
    cuts = [T * c // before[N] for c in before]
    ranges = list(zip(cuts[:-1], cuts[1:]))
    pieces = {}
    x = 0
    for b, (n, plen, sl) in enumerate(zip(lens, plens, seg)):
        for h in range(kv_heads):
            ss = x + h * sl
            se = ss + plen
            lst = []
            for w, (gs, ge) in enumerate(ranges):
                lo, hi = max(ss, gs), min(se, ge)
                if lo < hi:
                    lst.append((w, (lo - ss) * granule, min((hi - ss) * granule, n)))
            pieces[(b, h)] = lst
        x += kv_heads * sl
    S = max([1] + [len(v) for v in pieces.values()])
    return N, S, pieces, T
