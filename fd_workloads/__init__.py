"""Seeded synthetic decode-attention workloads.

This module only draws random tensors and lays them out; it holds none of the
attention arithmetic. Both the float64 oracle (through the tests) and the HIP
path read the tensors it returns, so the two sides always see the same bytes.

Every workload follows the shapes and value distributions of the pages:
q, K, V ~ N(0, 1) drawn in float32 from a seeded ``torch.Generator`` and then
rounded once to the cache dtype (the "Worked numbers" of "Flash-Decoding:
Split-KV Attention for Long-Context Decode" §1, the Triton test of §4 and the
PyTorch simulation of "FlashDecoding: Fast Long-Context Generation Guide" all
use standard-normal synthetic tensors). No dataset or trained weight is used.

Layouts
-------
contiguous : K, V are ``[B, Hkv, T_cap, D]`` with ``d`` contiguous.
paged      : K, V pools are indexed ``[num_pages, page_size, Hkv, D]``;
             ``block_table`` is int32 ``[B, max_pages_per_seq]``; token ``t``
             of sequence ``b`` lives in page ``block_table[b, t // page_size]``
             at row ``t % page_size``. Unused block-table entries are filled
             with a valid page id (0) so that any read stays inside the pool.
             The pool's storage order is either head-major ("hnd": memory
             ``[page, head, token, D]``, one head's page contiguous, the
             default) or token-major ("nhd": memory ``[page, token, head, D]``);
             both are handed over as the same ``[P, page, Hkv, D]`` index
             order and differ only in strides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Workload:
    """One decode step's inputs. Tensors live on ``device``."""

    name: str
    q: torch.Tensor                 # [B, Hq, D], or [B, q_len, Hq, D] for a short query block
    k: torch.Tensor                 # contiguous [B, Hkv, T, D] or pool [P, page, Hkv, D]
    v: torch.Tensor
    seq_lens: torch.Tensor          # int32 [B]
    block_table: Optional[torch.Tensor] = None   # int32 [B, max_pages] (paged only)
    page_size: int = 0
    num_splits: int = 0             # 0 = let the planner choose
    chunk_tokens: int = 0           # 0 = derived from num_splits
    ws_format: str = "uml"          # "uml" (u, m, l) or "olse" (o, lse)
    scale: float = 0.0              # 0 = 1/sqrt(D)
    k_gain: float = 1.0             # K was drawn as k_gain * N(0, 1)
    pool_layout: str = ""           # paged only: "hnd" or "nhd" storage order

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[-2]

    @property
    def q_len(self) -> int:
        return self.q.shape[1] if self.q.dim() == 4 else 1

    @property
    def head_dim(self) -> int:
        return self.q.shape[-1]

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[2] if self.paged else self.k.shape[1]

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max().item()) if self.seq_lens.numel() else 0

    def kv_bytes(self) -> int:
        """K+V bytes a decode step must read: sum_b len_b * Hkv * 2 * D * elt."""
        elt = self.k.element_size()
        tokens = int(self.seq_lens.to(torch.int64).sum().item())
        return tokens * self.num_kv_heads * 2 * self.head_dim * elt

    def to(self, device) -> "Workload":
        """Copy to ``device`` keeping every tensor's strides (pool storage order)."""
        moved = dataclasses.replace(self)
        for f in ("q", "k", "v", "seq_lens", "block_table"):
            t = getattr(self, f)
            if t is not None:
                c = torch.empty_strided(tuple(t.shape), t.stride(), dtype=t.dtype, device=device)
                setattr(moved, f, c.copy_(t))
        return moved


def _randn(gen: torch.Generator, shape, dtype, device, gain: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    if gain != 1.0:
        x.mul_(gain)
    return x.to(dtype)


def contiguous(name: str, *, seed: int, batch: int, q_heads: int, kv_heads: int,
               head_dim: int, capacity: int, seq_lens, dtype: str = "f16",
               q_gain: float = 1.0, k_gain: float = 1.0, device="cpu",
               num_splits: int = 0, chunk_tokens: int = 0, ws_format: str = "uml", q_len: int = 1) -> Workload:
    """Contiguous-cache workload. ``seq_lens`` is a list or int32 tensor of length B.
    ``q_len`` > 1 draws a short query block q [B, q_len, Hq, D]."""
    dt = DTYPES[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    qshape = (batch, q_len, q_heads, head_dim) if q_len > 1 else (batch, q_heads, head_dim)
    q = _randn(gen, qshape, dt, device, q_gain)
    k = _randn(gen, (batch, kv_heads, capacity, head_dim), dt, device, k_gain)
    v = _randn(gen, (batch, kv_heads, capacity, head_dim), dt, device)
    sl = torch.as_tensor(seq_lens, dtype=torch.int32).to(device)
    assert sl.shape == (batch,) and int(sl.max()) <= capacity
    return Workload(name, q, k, v, sl, num_splits=num_splits, chunk_tokens=chunk_tokens,
                    ws_format=ws_format, k_gain=k_gain)


def _pool(gen, num_pages, page_size, kv_heads, head_dim, dt, device, layout, gain=1.0):
    """A K or V pool indexed [P, page, Hkv, D], drawn in its storage order."""
    if layout == "hnd":
        return _randn(gen, (num_pages, kv_heads, page_size, head_dim), dt, device, gain).permute(0, 2, 1, 3)
    if layout == "nhd":
        return _randn(gen, (num_pages, page_size, kv_heads, head_dim), dt, device, gain)
    raise ValueError(f"unknown pool layout {layout!r}")


def paged(name: str, *, seed: int, batch: int, q_heads: int, kv_heads: int, head_dim: int,
          seq_lens, page_size: int = 16, dtype: str = "f16", device="cpu",
          num_splits: int = 0, chunk_tokens: int = 0, extra_pages: int = 0,
          pool_layout: str = "hnd", q_len: int = 1) -> Workload:
    """Paged-pool workload: the pool holds exactly sum_b cdiv(len_b, page) pages
    (+ ``extra_pages`` unused ones); a seeded ``randperm`` of the pool is dealt
    out to the sequences in order, so each sequence's pages are scattered."""
    dt = DTYPES[dtype]
    sl = torch.as_tensor(seq_lens, dtype=torch.int32)
    pages_per_seq = [max(1, math.ceil(int(n) / page_size)) for n in sl.tolist()]
    num_pages = sum(pages_per_seq) + extra_pages
    max_pages = max(pages_per_seq)
    gen_cpu = torch.Generator()
    gen_cpu.manual_seed(seed)
    perm = torch.randperm(num_pages, generator=gen_cpu)
    table = torch.zeros(batch, max_pages, dtype=torch.int32)
    cursor = 0
    for b, n in enumerate(pages_per_seq):
        table[b, :n] = perm[cursor:cursor + n].to(torch.int32)
        cursor += n
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1000)
    q = _randn(gen, (batch, q_len, q_heads, head_dim) if q_len > 1 else (batch, q_heads, head_dim), dt, device)
    k = _pool(gen, num_pages, page_size, kv_heads, head_dim, dt, device, pool_layout)
    v = _pool(gen, num_pages, page_size, kv_heads, head_dim, dt, device, pool_layout)
    return Workload(name, q, k, v, sl.to(device), block_table=table.to(device),
                    page_size=page_size, num_splits=num_splits, chunk_tokens=chunk_tokens,
                    pool_layout=pool_layout)


def redraw_kv(w: Workload, seed: int) -> Workload:
    """A copy of ``w`` with K and V drawn again (same shapes, dtype, device, gain
    and lengths; q and block table shared): extra cache copies for a benchmark
    that must not find one step's K/V in cache from the previous step."""
    gen = torch.Generator(device=w.k.device)
    gen.manual_seed(seed)
    if w.paged:
        P, page, hkv, d = w.k.shape
        k = _pool(gen, P, page, hkv, d, w.k.dtype, w.k.device, w.pool_layout, w.k_gain)
        v = _pool(gen, P, page, hkv, d, w.v.dtype, w.v.device, w.pool_layout)
    else:
        k = _randn(gen, tuple(w.k.shape), w.k.dtype, w.k.device, w.k_gain)
        v = _randn(gen, tuple(w.v.shape), w.v.dtype, w.v.device)
    return dataclasses.replace(w, k=k, v=v)


def uniform_lengths(seed: int, batch: int, lo: int, hi: int) -> torch.Tensor:
    """Seeded integer lengths uniform on [lo, hi] (inclusive)."""
    gen = torch.Generator()
    gen.manual_seed(seed)
    return torch.randint(lo, hi + 1, (batch,), generator=gen, dtype=torch.int64).to(torch.int32)


def boundary_lengths(seed: int, lengths: torch.Tensor, chunk: int, num_splits: int) -> torch.Tensor:
    """Move a seeded third of ``lengths`` onto split edges: chunk*k or chunk*k+1 for
    k in 1..num_splits-1, so trailing splits of those rows are fully masked and
    some splits hold exactly one token (the ``chunk·k ± 1`` rows of the
    verification table in §8 of the kanthi.in chapter)."""
    gen = torch.Generator()
    gen.manual_seed(seed)
    out = lengths.clone()
    n = out.numel()
    idx = torch.randperm(n, generator=gen)[: max(1, n // 3)]
    for j, i in enumerate(idx.tolist()):
        k = 1 + (j % max(1, num_splits - 1))
        out[i] = chunk * k + (j // max(1, num_splits - 1)) % 2
    return out


# ---------------------------------------------------------------------------
# The five workloads, by what they are.
# ---------------------------------------------------------------------------

def tiny_mha_f32(num_splits: int = 3, q_gain: float = 1.0, device="cpu") -> Workload:
    """B=1, 4 query heads = 4 KV heads, D=64, L=1000 (not a tile multiple), fp32."""
    return contiguous(f"tiny_mha_f32_L1000_S{num_splits}", seed=0, batch=1, q_heads=4,
                      kv_heads=4, head_dim=64, capacity=1000, seq_lens=[1000], dtype="f32",
                      q_gain=q_gain, device=device, num_splits=num_splits)


def ragged_mha_f32(num_splits: int = 8, q_gain: float = 1.0, device="cpu") -> Workload:
    """The ragged batch of the Triton test in §4: B=3, H=4, D=64, T=1000,
    seq_lens [1000, 37, 1]; with 8 splits of 125 tokens the 37-token row has
    seven empty splits and the last row a one-token cache."""
    return contiguous(f"ragged_mha_f32_S{num_splits}", seed=0, batch=3, q_heads=4, kv_heads=4,
                      head_dim=64, capacity=1000, seq_lens=[1000, 37, 1], dtype="f32",
                      q_gain=q_gain, device=device, num_splits=num_splits)


def long_gqa_f16(length: int = 128000, device="cpu", num_splits: int = 0) -> Workload:
    """B=1, 64 query heads over 8 KV heads, D=128, L=128000, fp16 (~524 MB K+V)."""
    return contiguous(f"gqa64x8_f16_L{length}", seed=2, batch=1, q_heads=64, kv_heads=8,
                      head_dim=128, capacity=length, seq_lens=[length], dtype="f16",
                      device=device, num_splits=num_splits)


def mha_bf16_chunked(length: int = 65536, chunk: int = 1024, device="cpu") -> Workload:
    """B=1, 32 = 32 heads, D=128, L=65536, bf16, fixed 1024-token chunks (64 splits),
    fp32 partial O + LSE workspace."""
    return contiguous(f"mha32_bf16_L{length}_C{chunk}", seed=3, batch=1, q_heads=32,
                      kv_heads=32, head_dim=128, capacity=length, seq_lens=[length],
                      dtype="bf16", device=device, chunk_tokens=chunk, ws_format="olse")


def paged_ragged_f16(batch: int = 16, lo: int = 1024, hi: int = 32768, device="cpu",
                     pool_layout: str = "hnd") -> Workload:
    """B=16, 32 query heads over 8 KV heads, D=128, lengths U[1024, 32768], fp16 pool of
    16-token pages (head-major storage by default) dealt out by a seeded permutation."""
    lens = uniform_lengths(4, batch, lo, hi)
    suffix = "" if pool_layout == "hnd" else f"_{pool_layout}"
    return paged(f"paged_gqa32x8_f16_B{batch}{suffix}", seed=4, batch=batch, q_heads=32, kv_heads=8,
                 head_dim=128, seq_lens=lens, page_size=16, dtype="f16", device=device,
                 pool_layout=pool_layout)


def edge_gqa_f16(batch: int = 64, hi: int = 2048, device="cpu", forced_splits: int = 0,
                 chunk: int = 256) -> Workload:
    """B=64, 32 query heads over 8 KV heads, D=128, lengths U[1, 2048], fp16 with K scaled
    x8 (logits of tens). With ``forced_splits`` the lengths of a seeded third of the rows
    sit on split edges so some splits are fully masked."""
    lens = uniform_lengths(5, batch, 1, hi)
    name = f"edge_gqa32x8_f16_B{batch}"
    if forced_splits:
        lens = boundary_lengths(55, lens, chunk, forced_splits)
        name += f"_S{forced_splits}"
    return contiguous(name, seed=5, batch=batch, q_heads=32, kv_heads=8, head_dim=128,
                      capacity=hi, seq_lens=lens, dtype="f16", k_gain=8.0, device=device,
                      num_splits=forced_splits, chunk_tokens=chunk if forced_splits else 0)
