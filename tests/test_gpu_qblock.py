"""GPU parity of short query blocks (speculative decode): q [B, q_len, Hq, D],
row i of the block sees the first seq_len - (q_len - 1 - i) tokens. Against
the oracle's block attention, over both kernels, forced and planned splits,
both schedules, paged pools and the fused merge."""
import numpy as np
import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W
from oracle import attention as A
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

LENS = [700, 1, 0, 5, 33, 3, 64, 65]


def block(g, q_len, dtype, lens=LENS, seed=0, paged=False, D=128):
    name = f"qblock_g{g}_q{q_len}_{dtype}_{'paged' if paged else 'contig'}"
    if paged:
        return W.paged(name, seed=200 + seed, batch=len(lens), q_heads=2 * g, kv_heads=2, head_dim=D,
                       seq_lens=lens, page_size=16, dtype=dtype, q_len=q_len)
    return W.contiguous(name, seed=300 + seed, batch=len(lens), q_heads=2 * g, kv_heads=2, head_dim=D,
                        capacity=max(lens), seq_lens=lens, dtype=dtype, q_len=q_len)


MFMA_CASES = [(1, 2, "f16"), (1, 8, "bf16"), (2, 4, "f16"), (4, 2, "bf16"), (2, 3, "f16"), (8, 1, "f16"),
              (8, 2, "f16"), (4, 3, "bf16"), (3, 3, "f16"), (2, 8, "bf16")]     # last four: two column tiles
VALU_CASES = [(1, 4, "f32"), (2, 2, "bf16"), (1, 3, "f16"), (4, 1, "f32")]


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("g,q_len,dtype", MFMA_CASES)
def test_mfma_block(g, q_len, dtype, splits):
    w = block(g, q_len, dtype)
    opts = {"kernel": "mfma"}
    if splits:
        opts["force_splits"] = splits
    plan, out, lse, _, _ = H.run(w, **opts)
    assert plan.kernel == fd.KERNELS["mfma"]
    assert tuple(out.shape) == tuple(w.q.shape)
    H.check_against_oracle(w, out, lse)


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("g,q_len,dtype", VALU_CASES)
def test_valu_block(g, q_len, dtype, splits):
    w = block(g, q_len, dtype, D=64 if dtype == "f32" else 128)
    plan, out, lse, _, _ = H.run(w, kernel="valu", force_splits=splits)
    assert plan.kernel == fd.KERNELS["valu"]
    H.check_against_oracle(w, out, lse)


def test_split_edge_inside_the_block():
    """A split boundary two tokens before the end: the last split holds fewer
    tokens than the block has rows, so some rows see nothing in it."""
    lens = [4098, 4100]
    w = block(2, 4, "f16", lens=lens)
    plan, out, lse, ws_o, ws_stats = H.run(w, force_chunk_tokens=2048)
    assert plan.num_splits == 3
    H.check_against_oracle(w, out, lse)
    # the workspace of the last split against the oracle's per-row split states
    o_s, lse_s, m_s, l_s = H.split_states_of(plan, ws_o, ws_stats)
    for i in range(4):
        cache = A.block_row_cache(w.q, w.k, w.v, w.seq_lens, i)
        M, Lw, U = A.split_states(cache, 3, 2048, pairs=[(0, 0), (1, 3)])
        for b, h in ((0, 0), (1, 3)):
            s = 2
            if Lw[b, h, s] == 0:
                assert np.isneginf(m_s[b, i, h, s]) and l_s[b, i, h, s] == 0
            else:
                o_ref, l_ref = A.state_to_olse(M[b, h, s], Lw[b, h, s], U[b, h, s])
                assert np.abs(o_s[b, i, h, s] - o_ref).max() < 2e-3
                assert abs(lse_s[b, i, h, s] - l_ref) <= 1e-5 * max(1, abs(l_ref))


@pytest.mark.parametrize("paged", [False, True])
def test_balanced_block(paged):
    w = block(2, 4, "f16", lens=[3000, 7, 0, 2000, 1, 1500], paged=paged, seed=5)
    plan, out, lse, _, _ = H.run(w, num_cus=5, schedule="balanced")
    assert plan.schedule == fd.SCHEDULES["balanced"]
    H.check_against_oracle(w, out, lse)


@pytest.mark.parametrize("schedule", ["uniform", "balanced"])
def test_fused_block(schedule):
    w = block(4, 2, "bf16", lens=[2500, 3, 0, 900], seed=6)
    opts = {"num_cus": 7, "schedule": schedule}
    if schedule == "uniform":
        opts.update(host_seq_lens=None, force_splits=4)
    plan, out, lse, ctr = H.run_fused(w, **opts)
    assert torch.all(ctr == 0).item()
    H.check_against_oracle(w, out, lse)


def test_block_of_one_equals_single_query():
    """q_len = 1 given as [B, 1, Hq, D] runs the same path as [B, Hq, D]."""
    w = block(4, 1, "f16", seed=7)
    w4 = W.Workload(**{**w.__dict__, "q": w.q.unsqueeze(1).contiguous()})
    p1, o1, l1, _, _ = H.run(w, force_splits=3)
    p2, o2, l2, _, _ = H.run(w4, force_splits=3)
    assert torch.equal(o1, o2.squeeze(1)) and torch.equal(l1, l2.squeeze(1))


@pytest.mark.parametrize("D", [64, 128])
def test_two_column_tiles_fused_and_balanced(D):
    """g = 8 with a 2-row block (16 rows per KV head, two MFMA column tiles)
    through the fused merge and the balanced schedule."""
    w = block(8, 2, "bf16", lens=[2600, 1, 0, 1800], seed=8, D=D)
    plan, out, lse, ctr = H.run_fused(w, num_cus=7, schedule="balanced")
    assert plan.schedule == fd.SCHEDULES["balanced"] and torch.all(ctr == 0).item()
    H.check_against_oracle(w, out, lse)
    plan, out, lse, ctr = H.run_fused(w, force_splits=4, host_seq_lens=None)
    assert torch.all(ctr == 0).item()
    H.check_against_oracle(w, out, lse)
