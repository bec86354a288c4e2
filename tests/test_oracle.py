"""Pins of the float64 oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own formulas: printed values
from the pages (tests/golden), closed forms, scipy's softmax/logsumexp, and
brute-force loops. ``test_planted_mistakes_are_caught`` plants plausible
mistakes in the oracle (on the CPU) and shows that a pin fails for each.
"""
import itertools
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import attention as A
from tests.conftest import golden

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# Worked example (xuujii KB §03/§04)
# ---------------------------------------------------------------------------

def _worked():
    g = golden("worked_example.json")
    s = np.log(np.array(g["score_weights"], dtype=np.float64))
    K = s.reshape(-1, 1)                 # D = 1, q = 1, scale = 1  ->  scores = s
    V = np.array(g["values"], dtype=np.float64).reshape(-1, 1)
    q = np.ones(1)
    return g, q, K, V


def check_worked_example():
    g, q, K, V = _worked()
    o, lse = A.attend(q, K, V, 1.0)
    num, den = g["output_fraction"]
    assert abs(o[0] - num / den) < 1e-14 and abs(o[0] - g["output"]) < 1e-14
    # LSE = ln(1+2+3+4) = ln 10: closed form of the same example.
    assert abs(lse - math.log(sum(g["score_weights"]))) < 1e-14

    states = []
    for blk in g["blocks"]:
        lo, hi = blk["positions"][0], blk["positions"][-1] + 1
        m, l, u = A.segment_state(q, K[lo:hi], V[lo:hi], 1.0)
        assert abs(m - math.log(blk["m_log_of"])) < 1e-14
        assert abs(l - blk["l"]) < 1e-14 and abs(u[0] - blk["u"]) < 1e-13
        n, d = blk["local_output_fraction"]
        assert abs(u[0] / l - n / d) < 1e-14
        states.append((m, l, u))
    m, l, u = A.merge_uml(states)
    rb = g["rebased_to_common_max"]
    assert abs(m - math.log(rb["m_log_of"])) < 1e-14
    assert abs(l - rb["l"]) < 1e-14 and abs(u[0] - rb["u"]) < 1e-13
    assert abs(u[0] / l - rb["output"]) < 1e-14
    # Global shares and contributions of the two blocks.
    tot = sum(math.exp(st[0]) * st[1] for st in states)
    for blk, st in zip(g["blocks"], states):
        share = math.exp(st[0]) * st[1] / tot
        assert abs(share - blk["share"]) < 1e-14
        assert abs(share * st[2][0] / st[1] - blk["contribution"]) < 1e-13
    # (o, LSE) form gives the same answer.
    o2, lse2 = A.merge_olse([A.state_to_olse(*st) for st in states])
    assert abs(o2[0] - 4.9) < 1e-14 and abs(lse2 - math.log(10.0)) < 1e-14
    return states


def test_worked_example():
    check_worked_example()


def test_naive_average_is_wrong():
    g = golden("worked_example.json")
    states = check_worked_example()
    local = [st[2][0] / st[1] for st in states]
    naive = sum(local) / len(local)
    # The page prints ~3.976 for equal-weight averaging.
    assert abs(naive - g["naive_average_printed"]) < 5e-4
    assert abs(naive - 167.0 / 42.0) < 1e-14
    # A merge that averages local outputs fails the 4.9 pin; the oracle's does not.
    assert abs(naive - g["output"]) > 0.9
    o, _ = A.merge_olse([A.state_to_olse(*st) for st in states])
    assert abs(o[0] - g["output"]) < 1e-14


# ---------------------------------------------------------------------------
# Merge trap (kanthi §3)
# ---------------------------------------------------------------------------

def check_merge_trap():
    g = golden("merge_trap.json")
    lse = np.array(g["lse_f32"], dtype=np.float32).astype(np.float64)
    o = np.array(g["o_f32"], dtype=np.float32).astype(np.float64)
    out, lse_out = A.merge_olse(list(zip(o, lse)))
    pr = g["printed"]
    np.testing.assert_allclose(out, pr["stable_merge"], rtol=0, atol=1e-7)
    assert abs(lse_out - pr["merged_lse"]) < 1e-5
    # weights implied by the merge: w_j = exp(lse_j - max)
    w = np.exp(lse - lse.max())
    np.testing.assert_allclose(w, pr["stable_weights"], rtol=0, atol=1e-7)  # printed to 7-8 decimals
    # uml form of the same states agrees
    m, l, u = A.merge_uml([(lj, 1.0, oj) for oj, lj in zip(o, lse)])
    np.testing.assert_allclose(u / l, out, rtol=0, atol=1e-15)
    assert abs(m + math.log(l) - lse_out) < 1e-13


def test_merge_trap_stable():
    check_merge_trap()


def test_merge_trap_naive_overflows_in_f32():
    g = golden("merge_trap.json")
    lse = np.array(g["lse_f32"], dtype=np.float32)
    o = np.array(g["o_f32"], dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.exp(lse)
        merged = (w[:, None] * o).sum(0) / w.sum()
    assert np.all(np.isinf(w)) and np.all(np.isnan(merged))


# ---------------------------------------------------------------------------
# Library routines and brute force
# ---------------------------------------------------------------------------

def _rand(seed, L, D):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(D), rng.standard_normal((L, D)), rng.standard_normal((L, D))


def check_against_scipy(seed=1, L=37, D=12, gain=3.0):
    q, K, V = _rand(seed, L, D)
    q = q * gain
    scale = 1.0 / math.sqrt(D)
    s = np.array([scale * sum(q[d] * K[i, d] for d in range(D)) for i in range(L)])  # brute force
    o, lse = A.attend(q, K, V, scale)
    np.testing.assert_allclose(o, softmax(s) @ V, rtol=0, atol=1e-13)
    assert abs(lse - logsumexp(s)) < 1e-12


def test_against_scipy_softmax_logsumexp():
    for seed in range(5):
        check_against_scipy(seed=seed)


def test_brute_force_tiny():
    # direct softmax without max subtraction, explicit loops, small logits
    for seed, (L, D) in enumerate([(1, 1), (2, 3), (5, 8), (16, 4)]):
        q, K, V = _rand(100 + seed, L, D)
        scale = 0.7
        e = [math.exp(scale * sum(q[d] * K[i, d] for d in range(D))) for i in range(L)]
        tot = sum(e)
        ref = [sum(e[i] * V[i, d] for i in range(L)) / tot for d in range(D)]
        o, lse = A.attend(q, K, V, scale)
        np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-14)
        assert abs(lse - math.log(tot)) < 1e-13


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_single_key():
    q, K, V = _rand(7, 1, 16)
    o, lse = A.attend(q, K, V, 0.25)
    np.testing.assert_array_equal(o, V[0])
    assert abs(lse - 0.25 * float(q @ K[0])) < 1e-15


def test_equal_keys_give_mean():
    rng = np.random.default_rng(3)
    D, L = 8, 50
    q = rng.standard_normal(D)
    K = np.tile(rng.standard_normal(D), (L, 1))
    V = rng.standard_normal((L, D))
    o, lse = A.attend(q, K, V, 0.5)
    np.testing.assert_allclose(o, V.mean(0), rtol=0, atol=1e-14)
    assert abs(lse - (0.5 * float(q @ K[0]) + math.log(L))) < 1e-13


def test_dominant_key():
    rng = np.random.default_rng(4)
    D, L = 8, 30
    q = np.zeros(D)
    q[0] = 1.0
    K = rng.standard_normal((L, D)) * 0.1
    K[17, 0] = 1000.0                    # s_17 exceeds all others by ~1000
    V = rng.standard_normal((L, D))
    o, lse = A.attend(q, K, V, 1.0)
    np.testing.assert_allclose(o, V[17], rtol=0, atol=1e-12)
    assert abs(lse - 1000.0) < 1e-9


def test_empty_row():
    o, lse = A.attend(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert lse == NEG_INF and np.all(o == 0)


# ---------------------------------------------------------------------------
# Merge invariance (kanthi §2/§3 "Try this" 1; xuujii §07)
# ---------------------------------------------------------------------------

def test_split_partitions_and_orders():
    q, K, V = _rand(11, 1000, 16)
    q *= 4.0
    scale = 0.25
    o_ref, lse_ref = A.attend(q, K, V, scale)
    rng = np.random.default_rng(12)
    partitions = []
    for S in range(1, 9):
        c = -(-1000 // S)
        partitions.append(A.chunk_bounds(1000, c, S))
        b = A.linspace_bounds(1000, S)
        partitions.append(list(zip(b[:-1], b[1:])))
    for _ in range(5):
        cuts = sorted(rng.integers(0, 1001, size=rng.integers(1, 12)).tolist())
        edges = [0] + cuts + [1000]
        partitions.append(list(zip(edges[:-1], edges[1:])))   # may contain empty segments
    for part in partitions:
        states = [A.segment_state(q, K[a:b], V[a:b], scale) for a, b in part]
        for _ in range(3):
            perm = rng.permutation(len(states))
            o, lse = A.state_to_olse(*A.merge_uml([states[i] for i in perm]))
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
            assert abs(lse - lse_ref) < 1e-12
        o2, lse2 = A.merge_olse([A.state_to_olse(*states[i]) for i in rng.permutation(len(states))])
        np.testing.assert_allclose(o2, o_ref, rtol=0, atol=1e-12)
        assert abs(lse2 - lse_ref) < 1e-12


def test_random_order_100_times_and_trees():
    q, K, V = _rand(21, 700, 8)
    scale = 0.3
    b = A.linspace_bounds(700, 7)
    states = [A.state_to_olse(*A.segment_state(q, K[x:y], V[x:y], scale)) for x, y in zip(b[:-1], b[1:])]
    o_ref, lse_ref = A.attend(q, K, V, scale)
    rng = np.random.default_rng(0)
    for _ in range(100):
        perm = rng.permutation(len(states))
        o, lse = A.merge_olse([states[i] for i in perm])
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        assert abs(lse - lse_ref) < 1e-12
    tree = A.merge_olse([A.merge_olse(states[:3]), A.merge_olse(states[3:])])
    np.testing.assert_allclose(tree[0], o_ref, rtol=0, atol=1e-12)
    nested = A.merge_olse([A.merge_olse([states[0], A.merge_olse(states[1:4])]), A.merge_olse(states[4:])])
    np.testing.assert_allclose(nested[0], o_ref, rtol=0, atol=1e-12)


def test_pages_split_reference_in_f64():
    g = golden("split_reference.json")["linspace"]
    rng = np.random.default_rng(0)
    D, T, S = g["D"], g["T"], g["S"]
    q = rng.standard_normal(D).astype(np.float32).astype(np.float64)
    K = rng.standard_normal((T, D)).astype(np.float32).astype(np.float64)
    V = rng.standard_normal((T, D)).astype(np.float32).astype(np.float64)
    b = A.linspace_bounds(T, S)
    assert b == g["boundaries"]
    o_full, lse_full = A.attend(q, K, V, 1.0 / math.sqrt(D))
    parts = [A.state_to_olse(*A.segment_state(q, K[x:y], V[x:y], 1.0 / math.sqrt(D))) for x, y in zip(b[:-1], b[1:])]
    o, lse = A.merge_olse(parts)
    # the page's float32 run printed ~1e-10; float64 agrees far tighter
    assert np.abs(o - o_full).max() < 1e-13 and abs(lse - lse_full) < 1e-12


# ---------------------------------------------------------------------------
# Empty / fully masked splits (kanthi §4; xuujii §06)
# ---------------------------------------------------------------------------

def test_alternating_bounds_by_hand_and_against_chunk_bounds():
    """By hand: 10 tokens in four splits of 4, 2, 4, 2 tokens end at 4, 6, 10 and
    start the fourth at 10 (empty); 7 tokens clip the third split to [6, 7).
    Equal lengths give chunk_bounds' partition; any lengths tile [0, len)
    in order."""
    assert A.alternating_bounds(10, 4, 2, 4) == [(0, 4), (4, 6), (6, 10), (10, 10)]
    assert A.alternating_bounds(7, 4, 2, 4) == [(0, 4), (4, 6), (6, 7), (10, 10)]
    assert A.alternating_bounds(0, 3, 5, 2) == [(0, 0), (3, 3)]
    for L in (0, 1, 37, 999, 1000, 1001):
        for S, c in ((3, 334), (8, 125), (32, 40)):
            assert A.alternating_bounds(L, c, c, S) == A.chunk_bounds(L, c, S)
    rng = np.random.default_rng(5)
    for _ in range(200):
        S = int(rng.integers(1, 20))
        ce, co = int(rng.integers(1, 50)), int(rng.integers(1, 50))
        L = int(rng.integers(0, (S // 2) * (ce + co) + (S % 2) * ce + 1))
        b = A.alternating_bounds(L, ce, co, S)
        covered = [t for lo, hi in b for t in range(lo, hi)]
        assert covered == list(range(L))


def test_chunk_bounds_ragged_table():
    g = golden("split_reference.json")["ragged"]
    assert -(-g["T_max"] // g["num_splits"]) == g["chunk"]
    for L, n_empty in zip(g["seq_lens"], g["empty_splits"]):
        bounds = A.chunk_bounds(L, g["chunk"], g["num_splits"])
        assert sum(1 for a, b in bounds if b <= a) == n_empty
        assert sum(b - a for a, b in bounds) == L
    assert A.chunk_bounds(1, 125, 8)[0] == (0, 1)


def test_empty_splits_contribute_nothing():
    q, K, V = _rand(31, 200, 8)
    scale = 0.4
    b = A.linspace_bounds(200, 4)
    states = [A.segment_state(q, K[x:y], V[x:y], scale) for x, y in zip(b[:-1], b[1:])]
    empty = A.segment_state(q, K[:0], V[:0], scale)
    assert empty[0] == NEG_INF and empty[1] == 0.0 and np.all(empty[2] == 0)
    base = A.merge_uml(states)
    with_empty = A.merge_uml(states + [empty] * 5)
    assert base[0] == with_empty[0] and base[1] == with_empty[1]
    np.testing.assert_array_equal(base[2], with_empty[2])
    base_o = A.merge_olse([A.state_to_olse(*s) for s in states])
    with_o = A.merge_olse([A.state_to_olse(*s) for s in [empty] + states + [empty]])
    np.testing.assert_array_equal(base_o[0], with_o[0])
    # all-empty: no NaN, the neutral state
    m, l, u = A.merge_uml([empty, empty])
    assert m == NEG_INF and l == 0 and not np.any(np.isnan(u))
    o, lse = A.merge_olse([A.state_to_olse(*empty)] * 3)
    assert lse == NEG_INF and np.all(o == 0)


def test_large_logits_no_overflow():
    q, K, V = _rand(41, 300, 16)
    q *= 400.0                            # logits in the hundreds/thousands
    o_ref, lse_ref = A.attend(q, K, V, 0.25)
    assert np.all(np.isfinite(o_ref)) and math.isfinite(lse_ref) and lse_ref > 88.7
    states = [A.segment_state(q, K[x:x + 50], V[x:x + 50], 0.25) for x in range(0, 300, 50)]
    o, lse = A.state_to_olse(*A.merge_uml(states))
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    assert abs(lse - lse_ref) < 1e-9


# ---------------------------------------------------------------------------
# Layouts and head mapping
# ---------------------------------------------------------------------------

def test_gqa_mapping_and_scipy():
    gen = torch.Generator().manual_seed(5)
    B, Hq, Hkv, T, D = 2, 8, 2, 40, 16
    q = torch.randn(B, Hq, D, generator=gen).half()
    k = torch.randn(B, Hkv, T, D, generator=gen).half()
    v = torch.randn(B, Hkv, T, D, generator=gen).half()
    lens = torch.tensor([40, 13], dtype=torch.int32)
    c = A.Cache(q, k, v, lens)
    O, LSE = A.decode_attention(c)
    for b in range(B):
        for hq in range(Hq):
            hk = hq // 4
            L = int(lens[b])
            s = (k[b, hk, :L].double().numpy() @ q[b, hq].double().numpy()) / math.sqrt(D)
            np.testing.assert_allclose(O[b, hq], softmax(s) @ v[b, hk, :L].double().numpy(), atol=1e-13, rtol=0)
            assert abs(LSE[b, hq] - logsumexp(s)) < 1e-12
    # a wrong head mapping (hq % Hkv) would give a different answer
    hk_wrong = 1 % Hkv
    s = (k[0, hk_wrong].double().numpy() @ q[0, 1].double().numpy()) / math.sqrt(D)
    assert np.abs(O[0, 1] - softmax(s) @ v[0, hk_wrong].double().numpy()).max() > 1e-3


def test_paged_equals_contiguous():
    gen = torch.Generator().manual_seed(6)
    B, Hq, Hkv, D, page = 3, 4, 2, 8, 16
    lens = [45, 16, 1]
    T = 48
    q = torch.randn(B, Hq, D, generator=gen).to(torch.bfloat16)
    k = torch.randn(B, Hkv, T, D, generator=gen).to(torch.bfloat16)
    v = torch.randn(B, Hkv, T, D, generator=gen).to(torch.bfloat16)
    n_pages = sum(-(-L // page) for L in lens) + 2
    perm = torch.randperm(n_pages, generator=gen)
    kp = torch.zeros(n_pages, page, Hkv, D, dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    table = torch.zeros(B, 3, dtype=torch.int32)
    cur = 0
    for b, L in enumerate(lens):
        for p in range(-(-L // page)):
            pid = int(perm[cur])
            cur += 1
            table[b, p] = pid
            n = min(page, L - p * page)
            kp[pid, :n] = k[b, :, p * page:p * page + n].transpose(0, 1)
            vp[pid, :n] = v[b, :, p * page:p * page + n].transpose(0, 1)
    sl = torch.tensor(lens, dtype=torch.int32)
    Oc, Lc = A.decode_attention(A.Cache(q, k, v, sl))
    Op, Lp = A.decode_attention(A.Cache(q, kp, vp, sl, block_table=table))
    np.testing.assert_array_equal(Oc, Op)
    np.testing.assert_array_equal(Lc, Lp)


def test_split_states_match_definition():
    gen = torch.Generator().manual_seed(8)
    q = torch.randn(2, 4, 16, generator=gen)
    k = torch.randn(2, 2, 100, 16, generator=gen)
    v = torch.randn(2, 2, 100, 16, generator=gen)
    lens = torch.tensor([100, 30], dtype=torch.int32)
    c = A.Cache(q, k, v, lens)
    M, L, U = A.split_states(c, 4, 25)
    O, LSE = A.decode_attention(c)
    for b in range(2):
        for h in range(4):
            sts = [(M[b, h, s], L[b, h, s], U[b, h, s]) for s in range(4)]
            o, lse = A.state_to_olse(*A.merge_uml(sts))
            np.testing.assert_allclose(o, O[b, h], atol=1e-13, rtol=0)
            assert abs(lse - LSE[b, h]) < 1e-12
    assert M[1, 0, 2] == NEG_INF and L[1, 0, 3] == 0.0      # 30 tokens: splits 2, 3 empty
    Os, Ls = A.split_then_merge(c, lambda n: A.chunk_bounds(n, 25, 4), form="olse")
    np.testing.assert_allclose(Os, O, atol=1e-13, rtol=0)


def test_seq_len_zero_row():
    q = torch.randn(1, 2, 4)
    k = torch.randn(1, 2, 5, 4)
    c = A.Cache(q, k, k, torch.tensor([0], dtype=torch.int32))
    O, LSE = A.decode_attention(c)
    assert np.all(O == 0) and np.all(LSE == NEG_INF)


# ---------------------------------------------------------------------------
# Planted mistakes: each one must be caught by at least one pin above.
# ---------------------------------------------------------------------------

def _all_pins():
    check_worked_example()
    check_merge_trap()
    for seed in range(3):
        check_against_scipy(seed=seed)


def _mut_scores_no_scale(q, K, scale):
    return K @ q


def _mut_scores_sign(q, K, scale):
    return -(K @ q) * scale


def _mut_attend_no_norm(q, K, V, scale):
    s = (K @ q) * scale
    m = float(s.max())
    p = np.exp(s - m)
    return p @ V, m + math.log(p.sum())


def _mut_attend_lse_log2(q, K, V, scale):
    s = (K @ q) * scale
    m = float(s.max())
    p = np.exp(s - m)
    return (p @ V) / p.sum(), m + math.log2(p.sum())


def _mut_merge_uml_no_rebase(states):
    m = max(st[0] for st in states)
    return m, sum(st[1] for st in states), sum(st[2] for st in states)


def _mut_merge_olse_average(states):
    return sum(st[0] for st in states) / len(states), max(st[1] for st in states)


@pytest.mark.parametrize("name,fn", [
    ("scores", _mut_scores_no_scale),
    ("scores", _mut_scores_sign),
    ("attend", _mut_attend_no_norm),
    ("attend", _mut_attend_lse_log2),
    ("merge_uml", _mut_merge_uml_no_rebase),
    ("merge_olse", _mut_merge_olse_average),
])
def test_planted_mistakes_are_caught(monkeypatch, name, fn):
    _all_pins()                                    # the real oracle passes
    monkeypatch.setattr(A, name, fn)
    with pytest.raises(AssertionError):
        _all_pins()


# ---------------------------------------------------------------------------
# Short query blocks (speculative decode)
# ---------------------------------------------------------------------------

def _masked_softmax_block(q, K, V, L, scale):
    """Brute force, written independently: scores of every (row i, token t) for
    t < L, with the bottom-right causal mask t > L - q_len + i set to -inf."""
    q_len = q.shape[0]
    s = (q @ K[:L].T) * scale
    t = np.arange(L)[None, :]
    i = np.arange(q_len)[:, None]
    s = np.where(t > L - q_len + i, -np.inf, s)
    out = np.zeros((q_len, V.shape[1]))
    lse = np.full(q_len, -np.inf)
    for r in range(q_len):
        if np.all(np.isneginf(s[r])):
            continue
        m = s[r].max()
        e = np.exp(s[r] - m)
        out[r] = e @ V[:L] / e.sum()
        lse[r] = m + np.log(e.sum())
    return out, lse


def test_block_rows_against_brute_force():
    rng = np.random.default_rng(11)
    for q_len in (1, 2, 4, 8):
        for L in (0, 1, 3, q_len, q_len + 1, 40):
            B, Hq, Hkv, D = 2, 4, 2, 8
            q = rng.standard_normal((B, q_len, Hq, D))
            k = rng.standard_normal((B, Hkv, 48, D))
            v = rng.standard_normal((B, Hkv, 48, D))
            lens = np.array([L, max(0, L - 1)])
            O, LSE = A.decode_attention_block(q, k, v, lens, scale=0.5)
            for b in range(B):
                for h in range(Hq):
                    ro, rl = _masked_softmax_block(q[b, :, h], k[b, h // 2], v[b, h // 2], int(lens[b]), 0.5)
                    assert np.allclose(O[b, :, h], ro, atol=1e-12)
                    assert np.array_equal(np.isneginf(LSE[b, :, h]), np.isneginf(rl))
                    fin = np.isfinite(rl)
                    assert np.allclose(LSE[b, fin, h], rl[fin], atol=1e-12)


def test_block_last_row_is_single_query_decode():
    """The last row of a block sees the whole cache: it equals single-query
    decode over seq_len; row i equals it over seq_len - (q_len - 1 - i)."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 4, 2, 16))
    k = rng.standard_normal((1, 2, 30, 16))
    v = rng.standard_normal((1, 2, 30, 16))
    O, LSE = A.decode_attention_block(q, k, v, [30])
    for i in range(4):
        o1, l1 = A.decode_attention(A.Cache(q[:, i], k, v, [30 - (3 - i)]))
        assert np.array_equal(O[:, i], o1) and np.array_equal(LSE[:, i], l1)
