"""HIP graph capture of the decode step. The library launches only on the
caller's stream, allocates nothing and keeps the fused call's counters at zero
from inside its kernels, so a captured step can be replayed. Each replay runs
on new K/V contents copied into the captured tensors, with eager work and
synchronisations between replays, and is checked against the eager result of
the same inputs and against the oracle."""
import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _workloads(kind):
    if kind == "gqa":
        base = W.contiguous("graph_gqa", seed=60, batch=2, q_heads=32, kv_heads=4, head_dim=128, capacity=6000,
                            seq_lens=[6000, 2500], dtype="f16")
    elif kind == "paged_balanced":
        base = W.paged("graph_paged", seed=61, batch=4, q_heads=16, kv_heads=4, head_dim=128,
                       seq_lens=[3000, 17, 0, 2200], page_size=16, dtype="bf16")
    else:
        base = W.contiguous("graph_mha", seed=62, batch=2, q_heads=8, kv_heads=8, head_dim=64, capacity=4000,
                            seq_lens=[4000, 1500], dtype="f32")
    return [base] + [W.redraw_kv(base, 900 + i) for i in range(1, REPLAYS)]


@pytest.mark.parametrize("path", ["split", "fused"])
@pytest.mark.parametrize("kind", ["gqa", "paged_balanced", "mha"])
def test_graph_replays_match_eager(kind, path):
    dev = torch.device("cuda", 0)
    ws_cpu = _workloads(kind)
    w0 = ws_cpu[0].to(dev)
    opts = {"host_seq_lens": ws_cpu[0].seq_lens.tolist()}
    if kind == "paged_balanced":
        opts["schedule"] = "balanced"
        opts["num_cus"] = 5                    # several pieces per segment
    else:
        opts["force_splits"] = 6
        del opts["host_seq_lens"]
    plan = fd.fd_plan(fd.problem_for(w0.q, w0.k, w0.v, w0.seq_lens, w0.block_table, max_seq_len=w0.max_seq_len),
                      **opts)
    H.say(f"graph {kind} {path}: S={plan.num_splits} schedule={plan.schedule} kernel={plan.kernel}")
    ws_o, ws_stats = fd.workspace(plan, dev)
    ctr = fd.counters(plan, dev)
    out = torch.empty(*w0.q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(*w0.q.shape[:-1], dtype=torch.float32, device=dev)

    def step():
        if path == "fused":
            fd.fd_decode_fused(plan, w0.q, w0.k, w0.v, w0.seq_lens, ws_o, ws_stats, ctr, out, lse, w0.block_table)
        else:
            fd.fd_decode_split(plan, w0.q, w0.k, w0.v, w0.seq_lens, ws_o, ws_stats, w0.block_table)
            fd.fd_merge(plan, ws_o, ws_stats, out, lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # warm-up off the capture, as torch asks
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i, wc in enumerate(ws_cpu):
        w0.k.copy_(wc.k.to(dev))
        w0.v.copy_(wc.v.to(dev))
        torch.cuda.synchronize()
        step()                                 # eager result of the same inputs
        torch.cuda.synchronize()
        ref_o, ref_l = out.clone(), lse.clone()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {i}: output differs from the eager call"
        assert torch.equal(lse, ref_l), f"replay {i}: LSE differs from the eager call"
        assert torch.all(ctr == 0).item()
        H.check_against_oracle(wc, out.cpu(), lse.cpu())
