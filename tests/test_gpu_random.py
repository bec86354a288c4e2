"""Seeded random configurations across the whole surface (dtype, head dim,
group size, query-block rows, layout and pool storage, lengths with empty
rows and tile/page edges, schedule, forced or planned splits, workspace form,
fused or two-launch path), each checked against the float64 oracle."""
import numpy as np
import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

N_CASES = 120


def config(i):
    rng = np.random.default_rng(1000 + i)
    dtype = str(rng.choice(["f16", "bf16", "f32"]))
    D = int(rng.choice([64, 128]))
    half = dtype != "f32"
    while True:
        g = int(rng.choice([1, 2, 3, 4, 8]))
        q_len = int(rng.choice([1, 1, 2, 3, 4]))
        R = g * q_len
        if (half and R <= 16) or R <= 4:
            break
    Hkv = int(rng.choice([1, 2, 3]))
    B = int(rng.choice([1, 2, 5]))
    hi = int(rng.choice([40, 700, 3000]))
    edges = [0, 1, 31, 32, 33, 63, 64, 65]
    lens = [int(rng.choice(edges)) if rng.random() < 0.3 else int(rng.integers(0, hi + 1)) for _ in range(B)]
    paged = bool(rng.random() < 0.4)
    opts = {}
    r = rng.random()
    if r < 0.3:
        opts["force_splits"] = int(rng.integers(1, 9))
    elif r < 0.5:
        opts["schedule"] = "balanced"
        opts["num_cus"] = int(rng.choice([3, 17, 256]))
    opts["ws_format"] = str(rng.choice(["uml", "olse"]))
    fused = bool(rng.random() < 0.35)
    kw = dict(seed=2000 + i, batch=B, q_heads=Hkv * g, kv_heads=Hkv, head_dim=D, seq_lens=lens, dtype=dtype,
              q_len=q_len)
    if paged:
        w = W.paged(f"rand{i}", page_size=int(rng.choice([16, 32, 64])),
                    pool_layout=str(rng.choice(["hnd", "nhd"])), extra_pages=int(rng.integers(0, 3)), **kw)
    else:
        w = W.contiguous(f"rand{i}", capacity=max(lens + [1]) + int(rng.integers(0, 40)), **kw)
    return w, opts, fused


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    w, opts, fused = config(i)
    H.say(f"case {i}: B={w.batch} q={tuple(w.q.shape)} k={tuple(w.k.shape)} lens={w.seq_lens.tolist()} "
          f"paged={w.paged} opts={opts} fused={fused}")
    if fused:
        plan, out, lse, ctr = H.run_fused(w, **opts)
        assert torch.all(ctr == 0).item()
    else:
        plan, out, lse, _, _ = H.run(w, **opts)
    H.check_against_oracle(w, out, lse)


N_LONG_CASES = 12


def long_config(i):
    """Long, ragged or equal lengths on a 256-CU plan, where the MI355X rule
    shifts tokens toward the even XCDs (uniform splits of at least 1536
    tokens, balanced ranges of at least 4096 K/V rows)."""
    rng = np.random.default_rng(3000 + i)
    dtype = str(rng.choice(["f16", "bf16"]))
    D = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 4, 8]))
    q_len = int(rng.choice([1, 1, 2]))
    schedule = str(rng.choice(["auto", "uniform", "balanced"]))
    if schedule == "balanced":        # over 4096 K/V rows per range: ranges of alternating size
        Hkv, B, hi, equal = 8, 6, 48000, False
    else:
        Hkv = int(rng.choice([4, 8]))
        B = int(rng.choice([1, 2, 4]))
        hi = int(rng.choice([20000, 48000]))
        equal = bool(rng.random() < 0.4)
    lens = [hi] * B if equal else [int(rng.integers(hi // 4, hi + 1)) for _ in range(B)]
    paged = bool(rng.random() < 0.3)
    opts = {"num_cus": 256, "schedule": schedule, "ws_format": str(rng.choice(["uml", "olse"]))}
    fused = bool(rng.random() < 0.3)
    kw = dict(seed=4000 + i, batch=B, q_heads=Hkv * g, kv_heads=Hkv, head_dim=D, seq_lens=lens, dtype=dtype,
              q_len=q_len)
    if paged:
        w = W.paged(f"long{i}", page_size=int(rng.choice([16, 64])), pool_layout="hnd", **kw)
    else:
        w = W.contiguous(f"long{i}", capacity=hi, **kw)
    return w, opts, fused


@pytest.mark.parametrize("i", range(N_LONG_CASES))
def test_random_long_configuration(i):
    w, opts, fused = long_config(i)
    H.say(f"long case {i}: B={w.batch} q={tuple(w.q.shape)} lens={w.seq_lens.tolist()} paged={w.paged} "
          f"opts={opts} fused={fused}")
    if fused:
        plan, out, lse, ctr = H.run_fused(w, **opts)
        assert torch.all(ctr == 0).item()
    else:
        plan, out, lse, _, _ = H.run(w, **opts)
    H.say(f"long case {i}: S={plan.num_splits} chunks {plan.chunk_tokens}/{plan.odd_chunk_tokens} "
          f"schedule={plan.schedule} odd_range={plan.odd_range_permille}")
    H.check_against_oracle(w, out, lse)
