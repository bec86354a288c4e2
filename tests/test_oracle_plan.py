"""Pins of the oracle's split-count rules (kanthi.in §6; vatshank FA3 comment)."""
import math
import pytest

from oracle import plan as P
from tests.conftest import golden


def test_page_split_table():
    g = golden("split_table.json")
    for row in g["rows"]:
        work = row["batch"] * row["heads"]
        assert work == row["work"]
        n_blocks = math.ceil(row["context"] / g["block_n"])
        s = P.num_splits_fa2(work, g["slots"], n_blocks, g["max_splits"])
        assert s == row["splits"], row
        assert work * s == row["ctas"]


def test_fa3_comment_efficiencies():
    g = golden("fa3_efficiency.json")
    for s, e in g["efficiency"].items():
        assert round(P.wave_efficiency(g["work"], int(s), g["sms"]), g["printed_precision"]) == e


def test_overhead_ratio_matches_page():
    g = golden("split_table.json")["overhead_check"]
    # g = 1, fp16, D large: 4 S g (D+2) / (L D elt) -> 2S/t as D grows
    r = P.workspace_ratio(g["splits"], 1, 1 << 20, 2, g["tokens"])
    assert abs(100 * r - g["ratio_percent_approx"]) < 0.01
    assert abs(r - 2 * g["splits"] / g["tokens"]) < 1e-9


def test_traffic_rule_reduces_to_page_rule():
    for work in (1, 3, 8, 32, 128, 500):
        for n_blocks in (1, 2, 3, 7, 100, 1000):
            a = P.num_splits_fa2(work, 264, n_blocks, 128)
            b = P.num_splits_traffic(work, 264, n_blocks, 128, 8, 128, 2, 10**9, 1e9)
            assert a == b


def test_rule_invariants():
    for work in (1, 2, 8, 64, 409, 410, 512, 4096):
        for n_blocks in (0, 1, 5, 64, 1000):
            for slots in (264, 512, 768):
                s = P.num_splits_traffic(work, slots, n_blocks, 128, 4, 128, 2, 128 * max(n_blocks, 1), 0.05)
                assert s >= 1
                if work >= 0.8 * slots or n_blocks <= 1:
                    assert s == 1
                assert s <= max(1, min(128, slots, n_blocks))
                if s > 1:
                    assert math.ceil(n_blocks / s) != math.ceil(n_blocks / (s - 1))
                    assert P.workspace_ratio(s, 4, 128, 2, 128 * n_blocks) <= 0.05


def test_chunk_for():
    assert P.chunk_for(1000, 8, 1) == 125
    assert P.chunk_for(1000, 3, 1) == 334
    assert P.chunk_for(128000, 56, 128) == 2304
    assert P.chunk_for(0, 4, 16) == 16


def test_balanced_schedule_partitions_every_segment():
    """Pieces tile each segment exactly, in order; every workgroup's share of
    the line differs from the others' by at most one granule; a workgroup
    meets a segment at most once; zero-length rows get no pieces."""
    import numpy as np
    rng = np.random.default_rng(3)
    for trial in range(200):
        B = int(rng.integers(1, 12))
        hkv = int(rng.choice([1, 2, 8]))
        G = int(rng.choice([16, 32, 64]))
        lens = [int(x) if rng.random() > 0.2 else 0 for x in rng.integers(0, int(rng.choice([5, 300, 5000])), B)]
        slots = int(rng.choice([1, 3, 7, 64, 256]))
        N, S, pieces, T = P.balanced_schedule(lens, hkv, G, slots)
        assert T == hkv * sum(-(-n // G) for n in lens)
        assert 1 <= N <= max(1, min(slots, T))
        share = [0] * N
        for (b, h), lst in pieces.items():
            n = lens[b]
            assert len(lst) <= S
            if n == 0:
                assert lst == []
                continue
            assert lst[0][1] == 0 and lst[-1][2] == n
            for (w0, _, hi0), (w1, lo1, _) in zip(lst, lst[1:]):
                assert hi0 == lo1 and w1 == w0 + 1 and lo1 % G == 0
            for w, lo, hi in lst:
                assert lo < hi
                share[w] += -(-hi // G) - lo // G
        assert sum(share) == T
        if T:
            assert max(share) - min(share) <= 1


def test_balanced_schedule_with_piece_cost():
    """With start-up cost granules on the line, pieces still tile every
    segment exactly; the line holds the cost of every non-empty segment; and
    a workgroup whose range covers many short segments receives fewer tokens
    than one covering a single long segment."""
    import numpy as np
    rng = np.random.default_rng(4)
    for trial in range(100):
        B = int(rng.integers(1, 20))
        hkv, G, cost = int(rng.choice([1, 4])), 32, int(rng.choice([1, 4, 8]))
        lens = [int(x) if rng.random() > 0.2 else 0 for x in rng.integers(0, 3000, B)]
        N, S, pieces, T = P.balanced_schedule(lens, hkv, G, int(rng.choice([3, 64, 256])), cost=cost)
        assert T == hkv * sum(-(-n // G) + cost for n in lens if n > 0)
        for (b, h), lst in pieces.items():
            n = lens[b]
            if n == 0:
                assert lst == []
                continue
            assert lst[0][1] == 0 and lst[-1][2] == n
            for (w0, _, hi0), (w1, lo1, _) in zip(lst, lst[1:]):
                assert hi0 == lo1 and w1 > w0
    lens = [32] * 12 + [32 * 120]                # twelve 1-granule rows, then a long one
    N, S, pieces, T = P.balanced_schedule(lens, 1, 32, 2, cost=4)
    assert N == 2
    tokens = [0, 0]
    for lst in pieces.values():
        for w, lo, hi in lst:
            tokens[w] += hi - lo
    assert tokens[0] < tokens[1]


def test_balanced_schedule_worked_example():
    """A partition worked out by hand from the definition. Lengths [96, 40],
    two KV heads, 32-token granules, no cost granules, four slots, ranges of
    at least one granule: segments (0,0), (0,1) hold 3 granules each and
    (1,0), (1,1) hold 2, so the line has T = 10 granules, in (b, h) order at
    [0,3), [3,6), [6,8), [8,10). N = 4 ranges: [0,2), [2,5), [5,7), [7,10)
    (floor(w * 10 / 4)). Each segment's pieces are its intersections with the
    ranges, in tokens; the last granule of sequence 1 holds tokens 32..39 only."""
    N, S, pieces, T = P.balanced_schedule([96, 40], 2, 32, 4, min_granules=1)
    assert (N, S, T) == (4, 2, 10)
    assert pieces == {
        (0, 0): [(0, 0, 64), (1, 64, 96)],
        (0, 1): [(1, 0, 64), (2, 64, 96)],
        (1, 0): [(2, 0, 32), (3, 32, 40)],
        (1, 1): [(3, 0, 40)],
    }
    # with one cost granule per segment the line grows to 14 and the cuts move:
    # segments at [0,4), [4,8), [8,11), [11,14) (token granules first, then the
    # cost granule); ranges [0,3), [3,7), [7,10), [10,14) now each hold one
    # segment's token granules whole, so every segment is one piece (S = 1)
    N, S, pieces, T = P.balanced_schedule([96, 40], 2, 32, 4, min_granules=1, cost=1)
    assert (N, S, T) == (4, 1, 14)
    assert pieces == {
        (0, 0): [(0, 0, 96)],
        (0, 1): [(1, 0, 96)],
        (1, 0): [(2, 0, 40)],
        (1, 1): [(3, 0, 40)],
    }


def test_balanced_schedule_odd_ranges_worked_example():
    """The same line of T = 10 granules (segments at [0,3), [3,6), [6,8),
    [8,10)) cut into four ranges of alternating size, x = 500: parts 1500,
    500, 1500, 500 of 4000, so the ranges start at floor(10 * c / 4000) for
    c = 0, 1500, 2000, 3500: granules 0, 3, 5, 8, i.e. [0,3), [3,5), [5,8),
    [8,10). Segment (0,1) is cut after its second granule (token 64)."""
    N, S, pieces, T = P.balanced_schedule([96, 40], 2, 32, 4, min_granules=1, odd_permille=500)
    assert (N, S, T) == (4, 2, 10)
    assert pieces == {
        (0, 0): [(0, 0, 96)],
        (0, 1): [(1, 0, 64), (2, 64, 96)],
        (1, 0): [(2, 0, 40)],
        (1, 1): [(3, 0, 40)],
    }
    assert P.balanced_schedule([96, 40], 2, 32, 4, min_granules=1, odd_permille=0) == \
        P.balanced_schedule([96, 40], 2, 32, 4, min_granules=1)


def test_balanced_schedule_odd_ranges_shares():
    """With alternating range sizes every range holds its exact share of the
    line, T (1000 +- x) / (1000 N) granules, to within one granule; pieces
    still tile every segment in order; and x = 0 gives the equal cut."""
    import numpy as np
    rng = np.random.default_rng(5)
    for trial in range(150):
        B = int(rng.integers(1, 16))
        hkv, G, cost = int(rng.choice([1, 2, 8])), int(rng.choice([16, 32])), int(rng.choice([0, 2, 16]))
        x = int(rng.choice([0, 1, 45, 300, 999]))
        lens = [int(n) if rng.random() > 0.2 else 0 for n in rng.integers(0, int(rng.choice([300, 5000])), B)]
        slots = int(rng.choice([2, 8, 64, 256]))
        N, S, pieces, T = P.balanced_schedule(lens, hkv, G, slots, cost=cost, odd_permille=x)
        parts = [1000 + x if w % 2 == 0 else 1000 - x for w in range(N)]
        tokens_of = [0] * N
        for (b, h), lst in pieces.items():
            n = lens[b]
            if n == 0:
                assert lst == []
                continue
            assert lst[0][1] == 0 and lst[-1][2] == n and len(lst) <= S
            for (w0, _, hi0), (w1, lo1, _) in zip(lst, lst[1:]):
                assert hi0 == lo1 and w1 > w0 and lo1 % G == 0
            for w, lo, hi in lst:
                tokens_of[w] += -(-hi // G) - lo // G
        if T == 0:
            continue
        # a range's token granules plus the cost granules it covers; recount the latter from the line
        seg = [(-(-n // G) + cost) if n > 0 else 0 for n in lens]
        line = []
        for b in range(B):
            for h in range(hkv):
                line += [1] * (-(-lens[b] // G)) + [0] * (cost if lens[b] > 0 else 0)
        assert len(line) == T == hkv * sum(seg)
        share = []
        pos = 0
        M = sum(parts)
        for w in range(N):
            exact = T * parts[w] / M
            end = (T * sum(parts[:w + 1])) // M
            share.append(end - pos)
            assert sum(line[pos:end]) == tokens_of[w]
            assert abs(share[-1] - exact) < 1 + 1e-9
            pos = end
        assert pos == T
        if x == 0:
            assert P.balanced_schedule(lens, hkv, G, slots, cost=cost) == (N, S, pieces, T)


def test_length_aware_chunk_worked_example():
    """By hand: lengths [1000, 3000] over 8 KV heads are 32 000 token-heads of
    work; one slot's share on 256 slots is cdiv(32000, 256) = 125 tokens,
    rounded up to the 32-token tile: 128, i.e. S = cdiv(3000, 128) = 24 splits.
    The workspace check (g = 4, D = 128, fp16) puts 2*24*4*130*4 bytes of
    states against 2*3000*128*2 of K/V per (sequence, KV head): 0.065 > 0.02.
    The chunk grows by whole tiles until the ratio fits: 416 tokens still
    gives S = 8 (0.0217), 448 gives S = 7 (0.0190)."""
    assert P.workspace_ratio(24, 4, 128, 2, 3000) == pytest.approx(2 * 24 * 4 * 130 * 4 / (2 * 3000 * 128 * 2))
    assert P.workspace_ratio(24, 4, 128, 2, 3000) > 0.02
    assert P.workspace_ratio(8, 4, 128, 2, 3000) > 0.02 >= P.workspace_ratio(7, 4, 128, 2, 3000)
    assert P.chunk_from_lengths([1000, 3000], 3000, 8, 256, 32, 128, 4, 128, 2, 0.02) == 448
    # without the budget the share alone decides
    assert P.chunk_from_lengths([1000, 3000], 3000, 8, 256, 32, 128, 4, 128, 2, 1.0) == 128
