"""GPU parity of the balanced split schedule: the batch's (sequence, KV head)
segments laid end to end and cut into equal ranges, one per workgroup. Final
outputs against the float64 oracle; partial states against the oracle's
states over the pieces of oracle.plan.balanced_schedule."""
import numpy as np
import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W
from oracle import attention as A
from oracle import plan as OP
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

BAL = fd.SCHEDULES["balanced"]


def case(name):
    if name == "gqa8_f16_ragged":
        return W.contiguous(name, seed=90, batch=6, q_heads=64, kv_heads=8, head_dim=128, capacity=6000,
                            seq_lens=[6000, 1, 0, 2500, 33, 4097], dtype="f16")
    if name == "gqa4_bf16_d64":
        return W.contiguous(name, seed=91, batch=5, q_heads=16, kv_heads=4, head_dim=64, capacity=3000,
                            seq_lens=[3000, 64, 2999, 0, 700], dtype="bf16")
    if name == "gqa2_f16_many_tiny":
        lens = [int(x) for x in np.random.default_rng(92).integers(0, 41, 300)]
        return W.contiguous(name, seed=92, batch=300, q_heads=4, kv_heads=2, head_dim=128, capacity=40,
                            seq_lens=lens, dtype="f16")
    if name == "all_empty":
        return W.contiguous(name, seed=93, batch=3, q_heads=16, kv_heads=2, head_dim=128, capacity=64,
                            seq_lens=[0, 0, 0], dtype="f16")
    if name == "one_long":
        return W.contiguous(name, seed=94, batch=1, q_heads=32, kv_heads=4, head_dim=128, capacity=20000,
                            seq_lens=[20000], dtype="bf16")
    if name == "mha_f16_ragged":                 # VALU kernel (g = 1)
        return W.contiguous(name, seed=99, batch=6, q_heads=8, kv_heads=8, head_dim=128, capacity=5000,
                            seq_lens=[5000, 0, 17, 3100, 1, 900], dtype="f16")
    if name == "mha_bf16_d64_qblock":            # VALU kernel, short query block (R = 2)
        return W.contiguous(name, seed=100, batch=4, q_heads=4, kv_heads=4, head_dim=64, capacity=2500,
                            seq_lens=[2500, 3, 0, 1200], dtype="bf16", q_len=2)
    if name == "f32_g2":                         # VALU kernel, fp32 cache, g = 2
        return W.contiguous(name, seed=101, batch=3, q_heads=8, kv_heads=4, head_dim=64, capacity=1500,
                            seq_lens=[1500, 40, 700], dtype="f32")
    if name == "gqa8_f16_long_ragged":           # over 4096 K/V rows per range on 256 CUs: alternating ranges
        return W.contiguous(name, seed=103, batch=8, q_heads=32, kv_heads=8, head_dim=128, capacity=40000,
                            seq_lens=[30000, 5000, 20000, 1, 40000, 12000, 25000, 0], dtype="f16")
    if name == "mha_f16_long_ragged":            # VALU kernel with alternating ranges on 256 CUs
        return W.contiguous(name, seed=105, batch=4, q_heads=8, kv_heads=8, head_dim=128, capacity=50000,
                            seq_lens=[40000, 30000, 50000, 20001], dtype="f16")
    if name == "gqa4_bf16_long_qblock2":         # two-row query block with alternating ranges on 256 CUs
        return W.contiguous(name, seed=106, batch=4, q_heads=32, kv_heads=8, head_dim=128, capacity=50000,
                            seq_lens=[50000, 33, 45000, 41000], dtype="bf16", q_len=2)
    if name == "paged_long_ragged":
        return W.paged(name, seed=104, batch=6, q_heads=32, kv_heads=8, head_dim=128,
                       seq_lens=[40000, 900, 33000, 0, 29000, 30000], page_size=16, dtype="f16")
    if name == "paged_mha":
        return W.paged(name, seed=102, batch=4, q_heads=8, kv_heads=8, head_dim=128,
                       seq_lens=[3000, 16, 0, 1700], page_size=32, dtype="f16")
    if name.startswith("paged"):
        _, page, layout = name.split("_")
        return W.paged(name, seed=95, batch=5, q_heads=32, kv_heads=8, head_dim=128,
                       seq_lens=[5000, 17, 0, 1200, 3333], page_size=int(page), dtype="f16",
                       pool_layout=layout, extra_pages=2)
    raise KeyError(name)


# batches with over 4096 K/V rows per range on 256 CUs: ranges of alternating size there
ALTERNATING = {"gqa8_f16_long_ragged", "paged_long_ragged", "mha_f16_long_ragged", "gqa4_bf16_long_qblock2"}

CASES = ["gqa8_f16_ragged", "gqa4_bf16_d64", "gqa2_f16_many_tiny", "all_empty", "one_long",
         "paged_16_hnd", "paged_64_nhd", "mha_f16_ragged", "mha_bf16_d64_qblock", "f32_g2", "paged_mha",
         "mha_f16_long_ragged", "gqa4_bf16_long_qblock2"]


@pytest.mark.parametrize("cus", [256, 5])
@pytest.mark.parametrize("name", CASES)
def test_balanced_matches_oracle(name, cus):
    w = case(name)
    plan, out, lse, ws_o, ws_stats = H.run(w, num_cus=cus, schedule="balanced")
    assert plan.schedule == BAL
    if name in ALTERNATING:                     # alternating ranges on 256 CUs only
        assert plan.odd_range_permille == (45 if cus == 256 else 0)
    H.check_against_oracle(w, out, lse)


@pytest.mark.parametrize("ws_format", ["uml", "olse"])
@pytest.mark.parametrize("name,cus", [("gqa8_f16_ragged", 7), ("paged_16_hnd", 7), ("mha_f16_ragged", 7),
                                      ("gqa8_f16_long_ragged", 256), ("paged_long_ragged", 256)])
def test_balanced_partial_states(name, cus, ws_format):
    """Slot i of segment (b, h) holds the state of its i-th piece; slots past
    the segment's piece count hold the neutral state. On 256 CUs the long
    batches get ranges of alternating size (odd ranges smaller), and the
    pieces are those of the oracle's alternating cut."""
    w = case(name)
    plan, out, lse, ws_o, ws_stats = H.run(w, num_cus=cus, ws_format=ws_format, schedule="balanced")
    assert plan.schedule == BAL
    assert plan.odd_range_permille == (45 if cus == 256 else 0)
    H.say(f"{name}: N={plan.grid_x} S={plan.num_splits} odd_range_permille={plan.odd_range_permille}")
    lens = w.seq_lens.tolist()
    N, S, pieces, _ = OP.balanced_schedule(lens, w.num_kv_heads, plan.chunk_tokens, plan.slots, cost=plan.piece_cost,
                                           odd_permille=plan.odd_range_permille)
    assert (plan.grid_x, plan.num_splits) == (N, S)
    B, Hq = w.batch, w.num_q_heads
    M, Lw, U = A.split_states(H.cache_of(w), S, plan.chunk_tokens,
                              bounds=lambda b, h: [(lo, hi) for _, lo, hi in pieces[(b, h)]])
    ws_o = ws_o.view(B, Hq, S, -1)
    ws_stats = ws_stats.view(B, Hq, S, -1)
    o, lse_s, m, l = H.split_states_of(plan, ws_o, ws_stats)
    with np.errstate(divide="ignore", invalid="ignore"):
        ref_o = np.where(Lw[..., None] > 0, U / Lw[..., None], 0.0)
        ref_lse = np.where(Lw > 0, M + np.log(np.where(Lw > 0, Lw, 1.0)), -np.inf)
    assert np.array_equal(np.isneginf(lse_s), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert np.max(np.abs(lse_s[fin] - ref_lse[fin]) / np.maximum(1, np.abs(ref_lse[fin]))) <= H.LSE_REL
    assert np.max(np.abs(o - ref_o)) <= H.MAX_ABS
    assert np.all(o[~fin] == 0)
    if m is not None:
        assert np.all(l[~fin] == 0) and np.all(np.isneginf(m[~fin]))


@pytest.mark.parametrize("cus", [256, 5])
@pytest.mark.parametrize("name", ["gqa8_f16_ragged", "gqa2_f16_many_tiny", "all_empty", "paged_16_hnd",
                                  "mha_f16_ragged", "f32_g2", "gqa8_f16_long_ragged", "paged_long_ragged",
                                  "mha_f16_long_ragged", "gqa4_bf16_long_qblock2"])
def test_balanced_fused(name, cus):
    w = case(name)
    plan, out, lse, ctr = H.run_fused(w, num_cus=cus, schedule="balanced")
    assert plan.schedule == BAL
    assert torch.all(ctr == 0).item(), "counters must be back at zero"
    H.check_against_oracle(w, out, lse)


def test_balanced_equals_uniform_bitwise_when_pieces_coincide():
    """B = 1 and a range per 4000-token split: the balanced pieces are exactly
    the uniform splits, so the two schedules give identical bits."""
    w = W.contiguous("coincide", seed=96, batch=1, q_heads=64, kv_heads=8, head_dim=128, capacity=32000,
                     seq_lens=[32000], dtype="f16")
    p1, o1, l1, _, _ = H.run(w, num_cus=64, wgs_per_cu=1, schedule="balanced", piece_cost_tokens=-1)
    p2, o2, l2, _, _ = H.run(w, num_cus=64, schedule="uniform", host_seq_lens=None, force_chunk_tokens=4000)
    assert (p1.grid_x, p1.num_splits) == (64, 8) and p2.num_splits == 8
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_balanced_fused_mixes_direct_and_merged_groups():
    """Three ranges over [2, 0, 1, 3]-granule rows (two KV heads): most groups
    are one piece and are written directly, one crosses a range boundary and
    goes through the counter and the merge."""
    w = W.contiguous("mixed_direct", seed=98, batch=4, q_heads=8, kv_heads=2, head_dim=128, capacity=96,
                     seq_lens=[64, 0, 32, 96], dtype="f16")
    plan, out, lse, ctr = H.run_fused(w, num_cus=3, wgs_per_cu=1, schedule="balanced")
    assert plan.schedule == BAL and plan.grid_x == 3 and plan.num_splits == 2
    assert torch.all(ctr == 0).item()
    H.check_against_oracle(w, out, lse)
