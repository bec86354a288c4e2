"""GPU parity of fd_merge_states, the merge operator on caller-built states:
the worked overflow example of the pages, cascade attention over two halves
of a cache, and random states (with empty ones) against the oracle's merges."""
import numpy as np
import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W
from oracle import attention as A
from tests import gpu_helpers as H
from tests.conftest import golden

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def test_merge_trap_values():
    """kanthi.in §3: three (o, lse) states with LSEs near 95 merge to the printed
    output and LSE (the naive exp would overflow)."""
    g = golden("merge_trap.json")
    D = 64
    states = torch.zeros(1, 3, D)
    states[0, :, :2] = torch.tensor(g["o_f32"])
    stats = torch.tensor([g["lse_f32"]], dtype=torch.float32)
    out, lse = fd.fd_merge_states(states.to(DEV), stats.to(DEV))
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert np.allclose(out[0, :2].numpy(), g["printed"]["stable_merge"], atol=1e-7)
    assert torch.all(out[0, 2:] == 0)
    assert abs(lse[0].item() - g["printed"]["merged_lse"]) <= 1e-5 * abs(g["printed"]["merged_lse"])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 3, 17, 300])
@pytest.mark.parametrize("fmt", ["olse", "uml"])
def test_random_states_against_oracle(fmt, S, D):
    rng = np.random.default_rng(S * 1000 + D)
    rows = 37
    o = rng.standard_normal((rows, S, D))
    lse = rng.uniform(-30, 90, (rows, S))
    lse[rng.random((rows, S)) < 0.2] = -np.inf          # empty states
    lse[5] = -np.inf                                     # a row with nothing to merge
    if fmt == "olse":
        states, stats = o.astype(np.float32), lse.astype(np.float32)
    else:                                                # u = l * o, m = lse - ln l
        l = rng.uniform(0.5, 40, (rows, S))
        l[np.isneginf(lse)] = 0.0
        with np.errstate(divide="ignore"):
            m = np.where(np.isneginf(lse), -np.inf, lse - np.log(np.where(l > 0, l, 1.0)))
        states = (o * l[..., None]).astype(np.float32)
        stats = np.stack([m, l], axis=-1).astype(np.float32)
    out, lse_out = fd.fd_merge_states(torch.from_numpy(states).to(DEV), torch.from_numpy(stats).to(DEV),
                                      ws_format=fmt)
    torch.cuda.synchronize()
    out, lse_out = out.cpu().double().numpy(), lse_out.cpu().double().numpy()
    s64, st64 = states.astype(np.float64), stats.astype(np.float64)
    for r in range(rows):
        if fmt == "olse":
            ref_o, ref_l = A.merge_olse([(s64[r, s], st64[r, s]) for s in range(S)])
        else:
            ref_o, ref_l = A.state_to_olse(*A.merge_uml([(st64[r, s, 0], st64[r, s, 1], s64[r, s])
                                                          for s in range(S)]))
        assert np.isneginf(lse_out[r]) == np.isneginf(ref_l), r
        assert np.max(np.abs(out[r] - ref_o)) <= 5e-5 * max(1.0, np.max(np.abs(ref_o))), r
        if np.isfinite(ref_l):
            assert abs(lse_out[r] - ref_l) <= 1e-5 * max(1.0, abs(ref_l)), r


@pytest.mark.parametrize("cut", [1, 2048, 4999])
def test_cascade_two_halves(cut):
    """Attention over [0, L) = merge of the attention over [0, cut) and over
    [cut, L), each computed by the split + merge path with its LSE."""
    L = 5000
    w = W.contiguous("cascade", seed=97, batch=2, q_heads=32, kv_heads=4, head_dim=128, capacity=L,
                     seq_lens=[L, L], dtype="f16")
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    parts = []
    for lo, hi in ((0, cut), (cut, L)):
        kk, vv = k[:, :, lo:hi], v[:, :, lo:hi]
        sl = torch.full((2,), hi - lo, dtype=torch.int32, device=DEV)
        parts.append(fd.flash_decode(q, kk, vv, sl, max_seq_len=hi - lo))
    states = torch.stack([parts[0][0], parts[1][0]], dim=2).contiguous()     # [B, Hq, 2, D]
    stats = torch.stack([parts[0][1], parts[1][1]], dim=2).contiguous()      # [B, Hq, 2]
    out, lse = fd.fd_merge_states(states, stats)
    torch.cuda.synchronize()
    H.check_against_oracle(w, out.cpu(), lse.cpu())
