"""Race check: the build with extra synchronisation around every hand-over of
LDS (FD_DEBUG_BARRIERS; workgroup barriers where every thread arrives, a full
memory wait and a wave barrier inside the per-wave streaming loops) must give
the release build's results bit for bit. A missing barrier in the release
kernels (a wave reading an LDS tile before it is written, a slice reused
while another wave still reads it) would make the two differ. Both libraries
run the same plans on the same inputs through the C ABI; the workspace, the
outputs and the LSE are compared bitwise."""
import ctypes
import os

import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W

DEBUG_LIB = os.path.join(os.path.dirname(os.path.abspath(fd.__file__)), "variants", "libfd_debug_barriers.so")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not os.path.exists(DEBUG_LIB),
                       reason="race-check build missing: python -m decode_attention_fd_amd.build --debug-barriers"),
]


def _case(name):
    if name == "gqa_uniform":
        return W.contiguous(name, seed=600, batch=2, q_heads=64, kv_heads=8, head_dim=128, capacity=12000,
                            seq_lens=[12000, 7001], dtype="f16"), {"force_splits": 24}
    if name == "mha_valu":
        return W.contiguous(name, seed=601, batch=3, q_heads=8, kv_heads=8, head_dim=128, capacity=5000,
                            seq_lens=[5000, 17, 3333], dtype="bf16"), {"force_splits": 7, "ws_format": "olse"}
    if name == "paged_balanced":
        w = W.paged(name, seed=602, batch=6, q_heads=32, kv_heads=8, head_dim=128,
                    seq_lens=[9000, 40, 0, 3000, 7000, 2500], page_size=16, dtype="f16")
        return w, {"schedule": "balanced", "host_seq_lens": w.seq_lens.tolist()}
    if name == "qblock_two_tiles":
        return W.contiguous(name, seed=603, batch=2, q_heads=64, kv_heads=8, head_dim=128, capacity=4000,
                            seq_lens=[4000, 1500], dtype="bf16", q_len=2), {"force_splits": 9}
    if name == "d64_f32_valu":
        return W.contiguous(name, seed=604, batch=2, q_heads=8, kv_heads=4, head_dim=64, capacity=3000,
                            seq_lens=[3000, 999], dtype="f32"), {"force_splits": 5}
    if name == "gqa_shifted":                  # uniform splits of two lengths (256 CUs)
        w = W.contiguous(name, seed=605, batch=2, q_heads=64, kv_heads=8, head_dim=128, capacity=48000,
                         seq_lens=[48000, 30001], dtype="f16")
        return w, {"num_cus": 256, "schedule": "uniform", "host_seq_lens": w.seq_lens.tolist()}
    if name == "paged_alternating":            # balanced ranges of alternating size (256 CUs)
        w = W.paged(name, seed=606, batch=6, q_heads=32, kv_heads=8, head_dim=128,
                    seq_lens=[40000, 900, 33000, 0, 29000, 30000], page_size=16, dtype="f16")
        return w, {"num_cus": 256, "schedule": "balanced", "host_seq_lens": w.seq_lens.tolist()}
    if name == "edge_batch":
        w = W.edge_gqa_f16()
        return w, {"host_seq_lens": w.seq_lens.tolist()}
    raise KeyError(name)


def _launch(L, plan, w, dev, fused):
    """One call of the library L; returns (out, lse, ws_o, ws_stats) on the CPU."""
    q, k, v, sl = w.q.to(dev), w.k.to(dev), w.v.to(dev), w.seq_lens.to(dev)
    bt = None if w.block_table is None else w.block_table.to(dev)
    ws_o, ws_stats = fd.workspace(plan, dev)
    ws_o.fill_(float("nan"))
    ws_stats.fill_(float("nan"))
    ctr = fd.counters(plan, dev)
    out = torch.full(q.shape, float("nan"), device=dev)
    lse = torch.full(q.shape[:-1], float("nan"), device=dev)
    args = fd.Args(q.data_ptr(), k.data_ptr(), v.data_ptr(), sl.data_ptr(), None if bt is None else bt.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = lambda t: t.numel() * t.element_size()
    if fused:
        st = L.fd_decode_fused(ctypes.byref(plan), ctypes.byref(args), ws_o.data_ptr(), nbytes(ws_o),
                               ws_stats.data_ptr(), nbytes(ws_stats), ctr.data_ptr(), nbytes(ctr), out.data_ptr(),
                               lse.data_ptr(), stream)
    else:
        st = L.fd_decode_split(ctypes.byref(plan), ctypes.byref(args), ws_o.data_ptr(), nbytes(ws_o),
                               ws_stats.data_ptr(), nbytes(ws_stats), stream)
        assert st == fd.FD_OK
        st = L.fd_merge(ctypes.byref(plan), ws_o.data_ptr(), nbytes(ws_o), ws_stats.data_ptr(), nbytes(ws_stats),
                        out.data_ptr(), lse.data_ptr(), stream)
    assert st == fd.FD_OK, fd.status_str(st)
    torch.cuda.synchronize()
    assert torch.all(ctr == 0).item()
    return out.cpu(), lse.cpu(), ws_o.cpu(), ws_stats.cpu()


def _same_bits(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", ["gqa_uniform", "mha_valu", "paged_balanced", "qblock_two_tiles", "d64_f32_valu",
                                  "edge_batch", "gqa_shifted", "paged_alternating"])
def test_debug_barrier_build_equals_release_bitwise(name, fused):
    w, opts = _case(name)
    dev = torch.device("cuda", 0)
    prob = fd.problem_for(w.q, w.k, w.v, w.seq_lens, w.block_table, max_seq_len=w.max_seq_len)
    plan = fd.fd_plan(prob, **opts)
    print(f"[race] {name} fused={fused} S={plan.num_splits} kernel={plan.kernel} schedule={plan.schedule} "
          f"chunks {plan.chunk_tokens}/{plan.odd_chunk_tokens} odd_range={plan.odd_range_permille}", flush=True)
    if name == "gqa_shifted":
        assert plan.chunk_tokens > plan.odd_chunk_tokens
    if name == "paged_alternating":
        assert plan.odd_range_permille > 0
    release = _launch(fd.lib(), plan, w, dev, fused)
    debug = _launch(fd.load(DEBUG_LIB), plan, w, dev, fused)
    for what, a, b in zip(("out", "lse"), release[:2], debug[:2]):
        assert _same_bits(a, b), f"{name}: {what} differs between the release and the debug-barrier build"
    if not fused:                       # every workspace slot is written by the split kernel
        for what, a, b in zip(("ws_o", "ws_stats"), release[2:], debug[2:]):
            assert _same_bits(a, b), f"{name}: {what} differs between the release and the debug-barrier build"
