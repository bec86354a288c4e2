"""The no-allocation entry point (fd_decode_fused_noalloc) through the C ABI
against fd_decode_fused with caller buffers: two calls in a row, the second on
a smaller problem, each equal to the caller-buffer call bit for bit and within
the parity tolerances of the oracle."""
import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _both(w, **opts):
    dev = torch.device("cuda", 0)
    q, k, v, sl = w.q.to(dev), w.k.to(dev), w.v.to(dev), w.seq_lens.to(dev)
    bt = None if w.block_table is None else w.block_table.to(dev)
    plan = fd.fd_plan(fd.problem_for(q, k, v, sl, bt, max_seq_len=w.max_seq_len), **opts)
    H.say(f"noalloc {w.name}: S={plan.num_splits} schedule={plan.schedule} grid={plan.grid_x}")
    out_n = torch.full(q.shape, float("nan"), device=dev)
    lse_n = torch.full(q.shape[:-1], float("nan"), device=dev)
    fd.fd_decode_fused_noalloc(plan, q, k, v, sl, out_n, lse_n, bt)
    torch.cuda.synchronize()
    ws_o, ws_stats = fd.workspace(plan, dev)
    ctr = fd.counters(plan, dev)
    out_f = torch.empty(q.shape, device=dev)
    lse_f = torch.empty(q.shape[:-1], device=dev)
    fd.fd_decode_fused(plan, q, k, v, sl, ws_o, ws_stats, ctr, out_f, lse_f, bt)
    torch.cuda.synchronize()
    return plan, out_n.cpu(), lse_n.cpu(), out_f.cpu(), lse_f.cpu()


@pytest.mark.parametrize("case", ["uniform", "balanced_paged"])
def test_noalloc_matches_fused_twice_second_smaller(case):
    if case == "uniform":
        first = W.contiguous("noalloc_big", seed=500, batch=2, q_heads=64, kv_heads=8, head_dim=128, capacity=20000,
                             seq_lens=[20000, 13001], dtype="f16")
        second = W.contiguous("noalloc_small", seed=501, batch=1, q_heads=32, kv_heads=8, head_dim=128,
                              capacity=3000, seq_lens=[2999], dtype="bf16")
        opts = ({"force_splits": 24}, {"force_splits": 5})
    else:
        first = W.paged("noalloc_paged_big", seed=502, batch=6, q_heads=32, kv_heads=8, head_dim=128,
                        seq_lens=[9000, 17, 0, 4000, 7000, 2500], page_size=16, dtype="f16")
        second = W.paged("noalloc_paged_small", seed=503, batch=3, q_heads=16, kv_heads=4, head_dim=128,
                         seq_lens=[1200, 3000, 5], page_size=16, dtype="f16")
        opts = tuple({"schedule": "balanced", "host_seq_lens": w.seq_lens.tolist()} for w in (first, second))
    for w, o in zip((first, second), opts):
        plan, out_n, lse_n, out_f, lse_f = _both(w, **o)
        assert plan.num_splits > 1
        assert torch.equal(out_n, out_f) and torch.equal(lse_n, lse_f), "noalloc differs from fd_decode_fused"
        H.check_against_oracle(w, out_n, lse_n)


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    w = W.contiguous("noalloc_too_big", seed=504, batch=256, q_heads=64, kv_heads=8, head_dim=128, capacity=64,
                     seq_lens=[64] * 256, dtype="f16")
    dev = torch.device("cuda", 0)
    q, k, v, sl = w.q.to(dev), w.k.to(dev), w.v.to(dev), w.seq_lens.to(dev)
    plan = fd.fd_plan(fd.problem_for(q, k, v, sl), force_splits=128, force_chunk_tokens=1)
    assert plan.ws_o_bytes >= fd.NOALLOC_SCRATCH_BYTES
    out = torch.empty(q.shape, device=dev)
    with pytest.raises(fd.FdError) as e:
        fd.fd_decode_fused_noalloc(plan, q, k, v, sl, out)
    assert e.value.status == fd.FD_ERR_WORKSPACE
