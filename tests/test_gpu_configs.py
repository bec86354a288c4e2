"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (plan defaults unless the workload forces splits/chunks).
Every (sequence, query head) output of every workload is compared with the
oracle, element by element; properties that hold at any size (finite,
NaN-free, neutral empty splits) are checked too. Grids larger than the
workloads' (thousands of rows or splits) are checked on sampled rows."""
import numpy as np
import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W
from oracle import attention as A
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

_BUILDERS = {
    "gqa64x8_f16_L128000": W.long_gqa_f16,
    "mha32_bf16_L65536_C1024": W.mha_bf16_chunked,
    "paged_gqa32x8_f16_B16": W.paged_ragged_f16,
    "edge_gqa32x8_f16_B64": W.edge_gqa_f16,
    "tiny_mha_f32_L1000": lambda: W.tiny_mha_f32(num_splits=3),
}
_CACHE = {}


def _workload(name):
    """The full-size workload and its whole oracle output, computed once per
    process (the oracle takes seconds on the largest ones, 20 s on the paged batch)."""
    if name not in _CACHE:
        w = _BUILDERS[name]()
        H.say(f"oracle: every row of {name}")
        _CACHE[name] = (w, A.decode_attention(H.cache_of(w)))
    return _CACHE[name]


def _check_all_rows(name, w, out, lse):
    O, LSE = _workload(name)[1]
    return H.compare(out, lse, O, LSE, None, label=f"{name} (all {w.batch * w.num_q_heads} rows)")


def _finite_everywhere(out, lse, seq_lens):
    assert torch.all(torch.isfinite(out))
    nonempty = seq_lens > 0
    assert torch.all(torch.isfinite(lse[nonempty]))


@pytest.mark.parametrize("splits", [3, 1, 2, 4, 5, 6, 7, 8])
def test_tiny_mha_f32_config(splits):
    w = W.tiny_mha_f32(num_splits=splits)
    plan, out, lse, _, _ = H.run(w)
    H.check_against_oracle(w, out, lse)


def test_long_gqa_f16_128k():
    name = "gqa64x8_f16_L128000"
    w = _workload(name)[0]
    plan, out, lse, _, _ = H.run(w)
    H.say(f"long GQA plan: S={plan.num_splits} chunk={plan.chunk_tokens} slots={plan.slots}")
    assert plan.kernel == fd.KERNELS["mfma"] and plan.num_splits > 1
    _finite_everywhere(out, lse, w.seq_lens)
    _check_all_rows(name, w, out, lse)                      # all 64 heads, all 8 KV groups


def test_mha_bf16_fixed_chunks():
    name = "mha32_bf16_L65536_C1024"
    w = _workload(name)[0]
    plan, out, lse, ws_o, ws_stats = H.run(w)
    assert plan.num_splits == 64 and plan.chunk_tokens == 1024 and plan.ws_format == fd.WS_FORMATS["olse"]
    _finite_everywhere(out, lse, w.seq_lens)
    _check_all_rows(name, w, out, lse)                      # all 32 heads
    # the (o, lse) workspace against the oracle's split states: all 64 splits of every head
    M, L, U = A.split_states(H.cache_of(w), 64, 1024)
    o_s, lse_s = ws_o[0].double().numpy(), ws_stats[0, :, :, 0].double().numpy()
    worst_o, worst_l = 0.0, 0.0
    for h in range(32):
        for s in range(64):
            o_ref, l_ref = A.state_to_olse(M[0, h, s], L[0, h, s], U[0, h, s])
            worst_o = max(worst_o, float(np.abs(o_s[h, s] - o_ref).max()))
            worst_l = max(worst_l, abs(lse_s[h, s] - l_ref) / max(1, abs(l_ref)))
    H.say(f"64 split states x 32 heads: max |do| {worst_o:.2e}, max rel dlse {worst_l:.2e}")
    assert worst_o < 2e-3 and worst_l < 1e-5


def test_paged_ragged_f16():
    name = "paged_gqa32x8_f16_B16"
    w = _workload(name)[0]
    plan, out, lse, _, _ = H.run(w)
    H.say(f"paged plan: S={plan.num_splits} chunk={plan.chunk_tokens}")
    _finite_everywhere(out, lse, w.seq_lens)
    _check_all_rows(name, w, out, lse)                      # all 16 x 32 rows


@pytest.mark.parametrize("schedule", ["auto", "uniform"])
def test_edge_gqa_plan_splits(schedule):
    w = W.edge_gqa_f16()
    plan, out, lse, _, _ = H.run(w, schedule=schedule)
    H.say(f"edge plan: S={plan.num_splits} schedule={plan.schedule}")
    if schedule == "uniform":
        assert plan.num_splits == 1                     # 512 work units fill the machine
    H.check_against_oracle(w, out, lse)                 # every (b, hq)


def test_edge_gqa_forced_masked_splits():
    w = W.edge_gqa_f16(forced_splits=8)
    plan, out, lse, ws_o, ws_stats = H.run(w)
    assert plan.num_splits == 8 and plan.chunk_tokens == 256
    H.check_against_oracle(w, out, lse)
    o_s, lse_s, m_s, l_s = H.split_states_of(plan, ws_o, ws_stats)
    n_masked = 0
    for b, L in enumerate(w.seq_lens.tolist()):
        for s in range(8):
            if s * 256 >= L:
                n_masked += 1
                assert np.all(ws_o[b, :, s].numpy() == 0)
                assert np.all(np.isneginf(m_s[b, :, s])) and np.all(l_s[b, :, s] == 0)
    assert n_masked > 0
    # one-token splits exist (lengths chunk*k + 1) and match the oracle's split state
    rows = [b for b, L in enumerate(w.seq_lens.tolist()) if L % 256 == 1 and L > 1]
    assert rows
    b = rows[0]
    s = w.seq_lens[b].item() // 256
    M, Lw, U = A.split_states(H.cache_of(w), 8, 256, pairs=[(b, 0)])
    assert abs(m_s[b, 0, s] - M[b, 0, s]) < 1e-5 * max(1, abs(M[b, 0, s]))
    assert abs(l_s[b, 0, s] - 1.0) < 1e-6


def test_max_length_single_sequence():
    """One sequence of 2^20 tokens (one KV head, 8 query heads, D=128, fp16:
    512 MiB of K/V) through the planner's default plan."""
    L = 1 << 20
    w = W.contiguous("max_len_1M", seed=7, batch=1, q_heads=8, kv_heads=1, head_dim=128, capacity=L,
                     seq_lens=[L], dtype="f16")
    plan, out, lse, _, _ = H.run(w)
    H.say(f"1M-token plan: S={plan.num_splits} chunk={plan.chunk_tokens} schedule={plan.schedule}")
    _finite_everywhere(out, lse, w.seq_lens)
    H.check_against_oracle(w, out, lse, [(0, 0), (0, 5)])


@pytest.mark.parametrize("name", list(_BUILDERS))
def test_bench_launch_configuration(name):
    """The benchmark's own plan options and path choice (bench.plan_options,
    bench.choose_path) at full size, every row against the oracle."""
    import bench

    w = _workload(name)[0]
    opts = bench.plan_options(w)
    dev = torch.device("cuda", 0)
    prob = fd.problem_for(w.q.to(dev), w.k.to(dev), w.v.to(dev), w.seq_lens.to(dev),
                          None if w.block_table is None else w.block_table.to(dev), max_seq_len=w.max_seq_len)
    plan = fd.fd_plan(prob, **opts)
    path = bench.choose_path(plan)
    H.say(f"{name}: S={plan.num_splits} schedule={plan.schedule} kernel={plan.kernel} path={path}")
    if path == "fused":
        plan2, out, lse, ctr = H.run_fused(w, **opts)
        assert torch.all(ctr == 0).item()
    else:
        plan2, out, lse, _, _ = H.run(w, **opts)
    assert (plan2.num_splits, plan2.chunk_tokens, plan2.schedule) == (plan.num_splits, plan.chunk_tokens, plan.schedule)
    _finite_everywhere(out, lse, w.seq_lens)
    _check_all_rows(name, w, out, lse)


@pytest.mark.parametrize("case", ["rows_4096", "splits_1024", "balanced_rows_1000", "balanced_fused_rows_1000"])
def test_large_grids(case):
    """Grids far larger than the workloads': 4096 sequences of short ragged
    lengths (a (1, 2, 4096) uniform grid), one sequence forced into 1024 mostly
    short or empty splits, and the balanced schedule over 1000 sequences (four
    rows per thread in its scan, lengths read back from memory in its walk),
    split + merge and fused; sampled rows against the oracle, every row finite."""
    rng = np.random.default_rng(3000)
    if case == "rows_4096":
        lens = [int(x) for x in rng.integers(0, 80, 4096)]
        w = W.contiguous(case, seed=3001, batch=4096, q_heads=8, kv_heads=2, head_dim=64, capacity=80,
                         seq_lens=lens, dtype="f16")
        plan, out, lse, _, _ = H.run(w)
    elif case == "splits_1024":
        w = W.contiguous(case, seed=3002, batch=1, q_heads=16, kv_heads=2, head_dim=128, capacity=40000,
                         seq_lens=[40000], dtype="bf16")
        plan, out, lse, _, _ = H.run(w, force_splits=1024)
        assert plan.num_splits == 1024
    else:
        lens = [int(x) for x in rng.integers(0, 600, 1000)]
        lens[::97] = [0] * len(lens[::97])
        w = W.contiguous(case, seed=3003, batch=1000, q_heads=8, kv_heads=2, head_dim=128, capacity=600,
                         seq_lens=lens, dtype="f16")
        opts = dict(schedule="balanced", host_seq_lens=lens)
        if case == "balanced_fused_rows_1000":
            plan, out, lse, ctr = H.run_fused(w, **opts)
            assert torch.all(ctr == 0).item()
        else:
            plan, out, lse, _, _ = H.run(w, **opts)
        assert plan.schedule == fd.SCHEDULES["balanced"]
    H.say(f"{case}: S={plan.num_splits} grid=({plan.grid_x}, {plan.grid_y}, {plan.grid_z}) schedule={plan.schedule}")
    _finite_everywhere(out, lse, w.seq_lens)
    H.check_against_oracle(w, out, lse, H.sample_pairs(w.batch, w.num_q_heads, 24, seed=3004))


@pytest.mark.parametrize("name", ["gqa64x8_f16_L128000", "mha32_bf16_L65536_C1024", "paged_gqa32x8_f16_B16"])
def test_fused_full_size(name):
    """The fused call at full size, every row against the oracle: 32 splits of
    4000 tokens for 8 GQA groups and 64 splits of 1024 tokens for 32 MHA heads
    (the last workgroup of each group merges all of its states), and the
    paged batch on its balanced plan."""
    w = _workload(name)[0]
    plan, out, lse, ctr = H.run_fused(w)
    H.say(f"fused {name}: S={plan.num_splits} schedule={plan.schedule}")
    if name != "paged_gqa32x8_f16_B16":
        assert plan.num_splits in (32, 64)
    assert torch.all(ctr == 0).item()
    _finite_everywhere(out, lse, w.seq_lens)
    _check_all_rows(name, w, out, lse)
