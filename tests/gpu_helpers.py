"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare it with the float64 oracle.

Tolerances (fp32 accumulation over fp16/bf16/fp32 caches): max |O - O_ref| <=
2e-3 and mean |O - O_ref| <= 1e-3; LSE: |LSE - LSE_ref| <= 1e-5 * max(1,
|LSE_ref|), and -inf must be returned exactly where the reference is -inf.
"""
from __future__ import annotations

import math
import sys
from typing import Iterable, Optional, Tuple

import numpy as np
import torch

import decode_attention_fd_amd as fd
from oracle import attention as A

MAX_ABS = 2e-3
MEAN_ABS = 1e-3
LSE_REL = 1e-5


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def plan_opts_for(w, **over):
    """The plan options the benchmark uses: forced splits/chunk where the workload
    fixes them, else the length-aware planner fed the host copy of the lengths."""
    opts = {"ws_format": w.ws_format}
    if w.num_splits:
        opts["force_splits"] = w.num_splits
    if w.chunk_tokens:
        opts["force_chunk_tokens"] = w.chunk_tokens
    if not w.num_splits and not w.chunk_tokens:
        opts["host_seq_lens"] = w.seq_lens.cpu().tolist()
    opts.update(over)
    return opts


def run(w, stream=None, **over):
    """Plan + split + merge on cuda:0. Returns (plan, out, lse, ws_o, ws_stats) on the CPU."""
    dev = torch.device("cuda", 0)
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    sl = w.seq_lens.to(dev)
    bt = None if w.block_table is None else w.block_table.to(dev)
    opts = plan_opts_for(w, **over)
    say(f"run {w.name} opts={ {k_: v_ for k_, v_ in opts.items() if k_ != 'host_seq_lens'} }")
    prob = fd.problem_for(q, k, v, sl, bt, max_seq_len=w.max_seq_len, scale=w.scale)
    plan = fd.fd_plan(prob, **opts)
    ws_o, ws_stats = fd.workspace(plan, dev)
    out = torch.empty(*q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(*q.shape[:-1], dtype=torch.float32, device=dev)
    fd.fd_decode_split(plan, q, k, v, sl, ws_o, ws_stats, bt, stream)
    fd.fd_merge(plan, ws_o, ws_stats, out, lse, stream)
    torch.cuda.synchronize()
    say(f"done {w.name} S={plan.num_splits} chunk={plan.chunk_tokens} kernel={plan.kernel} "
        f"schedule={plan.schedule} grid={plan.grid_x}")
    return plan, out.cpu(), lse.cpu(), ws_o.cpu(), ws_stats.cpu()


def run_fused(w, ctr=None, **over):
    """Plan + fused split/merge on cuda:0. Returns (plan, out, lse, counters)."""
    dev = torch.device("cuda", 0)
    q, k, v, sl = w.q.to(dev), w.k.to(dev), w.v.to(dev), w.seq_lens.to(dev)
    bt = None if w.block_table is None else w.block_table.to(dev)
    opts = plan_opts_for(w, **over)
    say(f"fused {w.name} opts={ {k_: v_ for k_, v_ in opts.items() if k_ != 'host_seq_lens'} }")
    plan = fd.fd_plan(fd.problem_for(q, k, v, sl, bt, max_seq_len=w.max_seq_len, scale=w.scale), **opts)
    ws_o, ws_stats = fd.workspace(plan, dev)
    ctr = fd.counters(plan, dev) if ctr is None else ctr
    out = torch.empty(*q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(*q.shape[:-1], dtype=torch.float32, device=dev)
    fd.fd_decode_fused(plan, q, k, v, sl, ws_o, ws_stats, ctr, out, lse, bt)
    torch.cuda.synchronize()
    return plan, out.cpu(), lse.cpu(), ctr


def cache_of(w) -> A.Cache:
    return A.Cache(w.q, w.k, w.v, w.seq_lens, w.block_table, scale=w.scale or None)


def compare(out: torch.Tensor, lse: torch.Tensor, O: np.ndarray, LSE: np.ndarray,
            pairs: Optional[Iterable[Tuple[int, int]]] = None, max_abs=MAX_ABS, mean_abs=MEAN_ABS,
            label="") -> dict:
    """Element-wise comparison at the given (b, hq) pairs (all if None)."""
    o = out.double().numpy()
    l = lse.double().numpy()
    if pairs is None:
        sel = (slice(None), slice(None))
        go, ro, gl, rl = o, O, l, LSE
    else:
        bs, hs = zip(*pairs)
        go, ro, gl, rl = o[list(bs), list(hs)], O[list(bs), list(hs)], l[list(bs), list(hs)], LSE[list(bs), list(hs)]
    assert np.all(np.isfinite(go)), f"{label}: non-finite output"
    err = np.abs(go - ro)
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean())}
    neg = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), neg), f"{label}: -inf LSE mismatch"
    fin = ~neg
    if fin.any():
        lerr = np.abs(gl[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin]))
        stats["lse_rel"] = float(lerr.max())
        assert stats["lse_rel"] <= LSE_REL, f"{label}: LSE error {stats}"
    assert not np.any(np.isnan(gl)), f"{label}: NaN LSE"
    say(f"{label} {stats}")
    assert stats["max_abs"] <= max_abs and stats["mean_abs"] <= mean_abs, f"{label}: {stats}"
    return stats


def check_against_oracle(w, out, lse, pairs=None, **tol):
    if w.q.dim() == 4:                       # short query block: rows (b, i) flattened
        B, q_len, Hq, D = w.q.shape
        rows = None if pairs is None else [(b, i, h) for b, h in pairs for i in range(q_len)]
        O, LSE = A.decode_attention_block(w.q, w.k, w.v, w.seq_lens, w.block_table, w.scale or None, rows)
        flat = None if pairs is None else [(b * q_len + i, h) for b, h in pairs for i in range(q_len)]
        return compare(out.reshape(B * q_len, Hq, D), lse.reshape(B * q_len, Hq), O.reshape(B * q_len, Hq, D),
                       LSE.reshape(B * q_len, Hq), flat, label=w.name, **tol)
    O, LSE = A.decode_attention(cache_of(w), pairs)
    return compare(out, lse, O, LSE, pairs, label=w.name, **tol)


def split_states_of(plan, ws_o, ws_stats):
    """Workspace -> (o_s, lse_s) per split, in float64, whatever its format."""
    u = ws_o.double().numpy()
    st = ws_stats.double().numpy()
    if plan.ws_format == fd.WS_FORMATS["uml"]:
        m, l = st[..., 0], st[..., 1]
        with np.errstate(divide="ignore", invalid="ignore"):
            o = np.where(l[..., None] > 0, u / l[..., None], 0.0)
            lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
        return o, lse, m, l
    return u, st[..., 0], None, None


def sample_pairs(B, Hq, n, seed=0):
    rng = np.random.default_rng(seed)
    pairs = {(b, int(rng.integers(Hq))) for b in range(B)}
    while len(pairs) < min(n, B * Hq):
        pairs.add((int(rng.integers(B)), int(rng.integers(Hq))))
    return sorted(pairs)
