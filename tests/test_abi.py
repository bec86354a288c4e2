"""Host-side tests of the C ABI (no GPU): symbols, struct layouts, planner and
argument validation. Nothing here launches a kernel."""
import ctypes
import math
import os
import re

import numpy as np

import pytest
import torch

import decode_attention_fd_amd as fd
from oracle import plan as OP
from tests.conftest import ROOT, golden

HEADER = os.path.join(ROOT, "include", "fd.h")


def _declared_functions():
    src = open(HEADER).read()
    return re.findall(r"FD_API\s+[\w\s\*]+?\b(fd_\w+)\s*\(", src)


def test_library_exports_every_declared_symbol():
    L = fd.lib()
    names = _declared_functions()
    assert set(names) >= {"fd_plan", "fd_decode_split", "fd_merge", "fd_status_str", "fd_version"}
    for n in names:
        assert hasattr(L, n), n
    assert fd.version() == re.search(r'FD_VERSION_STRING "([^"]+)"', open(HEADER).read()).group(1)


def test_struct_sizes_match_header():
    L = fd.lib()
    for i, cls in enumerate((fd.Problem, fd.PlanOpts, fd.Plan, fd.Args)):
        assert L.fd_struct_size(i) == ctypes.sizeof(cls)
    assert L.fd_struct_size(99) == 0


def test_status_strings():
    for s in range(7):
        assert fd.status_str(s)
    assert fd.status_str(12345) == "unknown status"


# ---------------------------------------------------------------------------
# Planner
# ---------------------------------------------------------------------------

def contiguous_problem(B=1, Hq=8, Hkv=8, D=128, L=1000, dtype=1, cap=None, **kw):
    p = fd.Problem()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim = B, Hq, Hkv, D
    p.q_dtype = p.kv_dtype = dtype
    p.layout = fd.LAYOUT_CONTIGUOUS
    p.max_seq_len = L
    cap = L if cap is None else cap
    p.q_stride_h = D
    p.q_stride_b = Hq * D
    p.kv_stride_t = D
    p.kv_stride_h = cap * D
    p.kv_stride_b = Hkv * cap * D
    p.kv_capacity = cap
    for k_, v_ in kw.items():
        setattr(p, k_, v_)
    return p


def paged_problem(B=2, Hq=32, Hkv=8, D=128, L=1000, page=16, dtype=1, **kw):
    p = fd.Problem()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim = B, Hq, Hkv, D
    p.q_dtype = p.kv_dtype = dtype
    p.layout = fd.LAYOUT_PAGED
    p.max_seq_len = L
    p.q_stride_h = D
    p.q_stride_b = Hq * D
    p.page_size = page
    p.max_pages_per_seq = -(-L // page)
    p.num_pages = B * p.max_pages_per_seq
    p.bt_stride_b = p.max_pages_per_seq
    p.pool_stride_h = D
    p.pool_stride_t = Hkv * D
    p.pool_stride_page = page * Hkv * D
    for k_, v_ in kw.items():
        setattr(p, k_, v_)
    return p


def test_fa2_heuristic_reproduces_page_table():
    g = golden("split_table.json")
    for row in g["rows"]:
        prob = contiguous_problem(B=row["batch"], Hq=row["heads"], Hkv=row["heads"], L=row["context"])
        plan = fd.fd_plan(prob, num_cus=g["sms"], wgs_per_cu=2, heuristic="fa2")
        assert plan.num_splits == row["splits"], row
        assert plan.grid_x * plan.grid_y * plan.grid_z == row["ctas"]
        assert plan.slots == g["slots"]


def base_chunk(plan, paged=False, cus=256):
    """The split rule's chunk of a uniform plan, after checking the odd-XCD
    shift: with an even split count on a 256-CU device (contiguous cache) and
    splits of at least FD_XCD_SHIFT_MIN_SPLIT_TOKENS (1536), even-numbered
    splits hold chunk + shift and odd ones chunk - shift tokens, shift =
    chunk * FD_DEFAULT_ODD_XCD_PERMILLE // 1000; else both chunk."""
    c, c_odd, S = plan.chunk_tokens, plan.odd_chunk_tokens, plan.num_splits
    assert (c + c_odd) % 2 == 0
    base = (c + c_odd) // 2
    shift = base * 45 // 1000
    if not paged and S % 2 == 0 and cus == 256 and base >= 1536 and 0 < shift < base:
        assert (c, c_odd) == (base + shift, base - shift), (S, c, c_odd)
    else:
        assert c == c_odd, (S, c, c_odd)
    return base


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
@pytest.mark.parametrize("wgs", [1, 2])
def test_mi355x_heuristic_matches_oracle_rule(kernel, wgs):
    cus = 256
    budget = 0.25                                   # the MI355X default
    for B in (1, 2, 4, 16, 64):
        for Hkv, g in ((8, 8), (8, 4), (32, 1), (2, 2)):
            if (kernel == "mfma" and g == 1) or (kernel == "valu" and g > 4):
                continue
            for L in (1, 100, 1000, 4096, 32768, 128000):
                prob = contiguous_problem(B=B, Hq=Hkv * g, Hkv=Hkv, L=L)
                plan = fd.fd_plan(prob, num_cus=cus, wgs_per_cu=wgs, kernel=kernel)
                block = plan.tile_tokens * plan.waves_per_wg
                s = OP.num_splits_traffic(B * Hkv, cus * wgs, math.ceil(L / block), 128, g, 128, 2, L, budget,
                                          threshold=1.0)
                chunk = OP.chunk_for(L, s, 1)              # contiguous: cdiv(L, S), no tile rounding
                assert base_chunk(plan) == chunk, (B, Hkv, g, L)
                assert plan.num_splits == math.ceil(L / chunk), (B, Hkv, g, L)
                assert plan.num_splits <= s


def test_mi355x_choices_for_the_workloads():
    """The planner's picks for the four large workloads (256 CUs, defaults)."""
    assert fd.fd_plan(contiguous_problem(Hq=64, Hkv=8, L=128000), num_cus=256).num_splits == 32
    p = fd.fd_plan(contiguous_problem(Hq=64, Hkv=8, L=128000), num_cus=256)
    assert base_chunk(p) == 4000 and p.slots == 256
    assert (p.chunk_tokens, p.odd_chunk_tokens) == (4180, 3820)     # 4.5 % from odd-XCD splits to even ones
    p = fd.fd_plan(contiguous_problem(Hq=64, Hkv=8, L=128000), num_cus=256, odd_xcd_permille=-1)
    assert (p.num_splits, p.chunk_tokens, p.odd_chunk_tokens) == (32, 4000, 4000)
    p = fd.fd_plan(contiguous_problem(Hq=64, Hkv=8, L=128000), num_cus=256, odd_xcd_permille=100)
    assert (p.chunk_tokens, p.odd_chunk_tokens) == (4400, 3600)
    p = fd.fd_plan(contiguous_problem(Hq=64, Hkv=8, L=128000), num_cus=128)
    assert p.chunk_tokens == p.odd_chunk_tokens                      # not the 256-CU device
    p = fd.fd_plan(contiguous_problem(Hq=64, Hkv=8, L=128000), num_cus=256, force_splits=32)
    assert p.chunk_tokens == p.odd_chunk_tokens == 4000               # forced plans keep equal splits
    for L, chunk in ((16000, 500), (32000, 1000), (48000, 1500)):  # short splits stay equal
        p = fd.fd_plan(contiguous_problem(B=1, Hq=64, Hkv=8, L=L), num_cus=256)
        assert (p.num_splits, p.chunk_tokens, p.odd_chunk_tokens) == (32, chunk, chunk), L
    p = fd.fd_plan(contiguous_problem(B=1, Hq=64, Hkv=8, L=64000), num_cus=256)
    assert (p.chunk_tokens, p.odd_chunk_tokens) == (2090, 1910)
    assert _status(contiguous_problem(), odd_xcd_permille=1000) == fd.FD_ERR_INVALID_ARG
    assert _status(contiguous_problem(), odd_xcd_permille=-2) == fd.FD_ERR_INVALID_ARG
    assert fd.fd_plan(contiguous_problem(B=64, Hq=32, Hkv=8, L=2048), num_cus=256).num_splits == 1
    assert fd.fd_plan(contiguous_problem(Hq=32, Hkv=32, L=65536, dtype=2), num_cus=256).num_splits == 8


@pytest.mark.parametrize("paged", [False, True])
def test_length_aware_rule_matches_oracle(paged):
    """With host lengths the MI355X planner caps a split at one slot's share of
    the batch's total work (oracle.plan.chunk_from_lengths)."""
    rng = np.random.default_rng(17)
    for trial in range(60):
        B = int(rng.choice([1, 2, 3, 16, 64]))
        Hkv, g = ((8, 8), (8, 4), (2, 2), (32, 1))[trial % 4]
        kernel = "valu" if g == 1 else "auto"
        hi = int(rng.choice([1, 40, 1000, 32768, 131072]))
        lens = rng.integers(0, hi + 1, size=B)
        L = max(int(lens.max()), 1) + int(rng.integers(0, 64))
        mk = paged_problem if paged else contiguous_problem
        prob = mk(B=B, Hq=Hkv * g, Hkv=Hkv, L=L)
        plan = fd.fd_plan(prob, num_cus=256, kernel=kernel, host_seq_lens=lens.tolist(), schedule="uniform")
        align = max(plan.tile_tokens, 16) if paged else 1
        chunk = OP.chunk_from_lengths(lens.tolist(), L, Hkv, 256, align, 128, g, 128, 2, 0.25)
        assert base_chunk(plan, paged) == chunk, (B, Hkv, g, L, lens.tolist()[:4])
        assert plan.num_splits == math.ceil(L / chunk)


def test_length_aware_choices():
    """Equal lengths reproduce the wave-filling choice; a ragged batch splits by
    its total work, not by its longest row."""
    p = fd.fd_plan(contiguous_problem(Hq=64, Hkv=8, L=128000), num_cus=256, host_seq_lens=[128000],
                   schedule="uniform")
    assert (p.num_splits, base_chunk(p)) == (32, 4000)
    lens = [32768] + [1024] * 15
    p = fd.fd_plan(paged_problem(B=16, L=32768), num_cus=256, host_seq_lens=lens, schedule="uniform")
    assert p.chunk_tokens == OP.cdiv(OP.cdiv(8 * sum(lens), 256), 32) * 32
    with pytest.raises(fd.FdError):
        fd.fd_plan(paged_problem(B=16, L=32768), num_cus=256, host_seq_lens=lens[:15])
    with pytest.raises(fd.FdError):
        fd.fd_plan(paged_problem(B=16, L=1000), num_cus=256, host_seq_lens=lens)


@pytest.mark.parametrize("paged", [False, True])
def test_balanced_schedule_matches_oracle(paged):
    """Grid size, granule and slot count of the balanced plan equal the
    oracle's schedule from its definition."""
    rng = np.random.default_rng(29)
    for trial in range(80):
        B = int(rng.choice([1, 2, 5, 16, 64]))
        Hkv, g = ((8, 8), (8, 4), (2, 2), (4, 2), (8, 1))[trial % 5]
        lens = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(0, int(rng.choice([40, 2048, 40000])), B)]
        L = max(lens + [1])
        cus = int(rng.choice([7, 64, 256]))
        mk = paged_problem if paged else contiguous_problem
        page = int(rng.choice([16, 64])) if paged else 0
        prob = mk(B=B, Hq=Hkv * g, Hkv=Hkv, L=L, **({"page": page} if paged else {}))
        plan = fd.fd_plan(prob, num_cus=cus, host_seq_lens=lens, schedule="balanced")
        assert plan.schedule == fd.SCHEDULES["balanced"]
        G = max(32, page)
        assert plan.slots == cus                       # one range per CU by default
        assert plan.piece_cost == -(-512 // G)           # default start-up cost: 512 tokens
        N, S, _, _ = OP.balanced_schedule(lens, Hkv, G, plan.slots, cost=plan.piece_cost,
                                          odd_permille=plan.odd_range_permille)
        assert (plan.grid_x, plan.grid_y, plan.grid_z) == (N, 1, 1), (lens, cus)
        assert plan.num_splits == S and plan.chunk_tokens == G
        assert plan.ws_o_bytes == B * Hkv * g * S * 128 * 4


@pytest.mark.parametrize("paged", [False, True])
def test_balanced_odd_ranges_match_oracle(paged):
    """Ranges of alternating size: the planner turns them on exactly when the
    MI355X rule runs on 256 CUs with a multiple of 8 ranges averaging at least
    FD_XCD_SHIFT_MIN_RANGE_TOKENS of K/V rows and every odd range keeps a
    granule, with the default 45 per mille or the caller's x; its split count
    S then equals the oracle's for the same alternating cut."""
    rng = np.random.default_rng(31)
    seen = set()
    for trial in range(120):
        B = int(rng.choice([3, 8, 16, 64]))
        Hkv, g = ((8, 4), (2, 2), (4, 1), (8, 8))[trial % 4]
        lens = [int(n) if rng.random() > 0.1 else 0 for n in rng.integers(0, int(rng.choice([3000, 60000])), B)]
        L = max(lens + [1])
        x = int(rng.choice([0, 1, 45, 250, 999]))
        wpc = int(rng.choice([1, 2]))
        mk = paged_problem if paged else contiguous_problem
        page = int(rng.choice([16, 64])) if paged else 0
        prob = mk(B=B, Hq=Hkv * g, Hkv=Hkv, L=L, **({"page": page} if paged else {}))
        plan = fd.fd_plan(prob, num_cus=256, wgs_per_cu=wpc, host_seq_lens=lens, schedule="balanced",
                          odd_xcd_permille=x)
        N = plan.grid_x
        T = OP.balanced_schedule(lens, Hkv, plan.chunk_tokens, plan.slots, cost=plan.piece_cost)[3]
        on = N % 8 == 0 and Hkv * sum(lens) >= 4096 * N and (1000 - (x or 45)) * T >= 1000 * N
        assert plan.odd_range_permille == ((x or 45) if on else 0), (lens, x, N)
        seen.add((on, x))
        N2, S, _, _ = OP.balanced_schedule(lens, Hkv, plan.chunk_tokens, plan.slots, cost=plan.piece_cost,
                                           odd_permille=plan.odd_range_permille)
        assert (N, plan.num_splits) == (N2, S), (lens, x)
        off = fd.fd_plan(prob, num_cus=256, wgs_per_cu=wpc, host_seq_lens=lens, schedule="balanced",
                         odd_xcd_permille=-1)
        assert off.odd_range_permille == 0 and off.grid_x == N
        assert fd.fd_plan(prob, num_cus=255, host_seq_lens=lens, schedule="balanced").odd_range_permille == 0
        assert fd.fd_plan(prob, num_cus=256, host_seq_lens=lens, schedule="balanced",
                          heuristic="fa2").odd_range_permille == 0
    assert {on for on, _ in seen} == {False, True} and (True, 250) in seen


def test_prefers_fused_rule():
    """The default path: one launch for one split, or for a balanced plan of at
    least FUSED_MIN_ROWS output rows (B * q_len * Hq); split + merge otherwise."""
    one = fd.fd_plan(contiguous_problem(B=64, Hq=32, Hkv=8, L=2048), num_cus=256)
    assert one.num_splits == 1 and fd.prefers_fused(one)
    uni = fd.fd_plan(contiguous_problem(B=1, Hq=64, Hkv=8, L=128000), num_cus=256)
    assert uni.num_splits == 32 and not fd.prefers_fused(uni)
    for B, fused in ((64, False), (127, False), (128, True), (256, True)):    # 32 query heads: rows = 32 B
        lens = [1 + (37 * i) % 2048 for i in range(B)]
        p = fd.fd_plan(contiguous_problem(B=B, Hq=32, Hkv=8, L=2048), num_cus=256, host_seq_lens=lens,
                       schedule="balanced")
        assert p.schedule == fd.SCHEDULES["balanced"] and p.num_splits > 1, B
        assert fd.prefers_fused(p) == fused, B
    assert fd.FUSED_MIN_ROWS == 4096


def test_schedule_selection():
    lens = [30000, 10, 0]                        # 8 * 30010 / 256 = 937 tokens per range
    prob = contiguous_problem(B=3, Hq=32, Hkv=8, L=30000)
    assert fd.fd_plan(prob, num_cus=256, host_seq_lens=lens).schedule == fd.SCHEDULES["balanced"]
    # too little work per range (8 heads x 24 576 tokens over 256 ranges = 768; one token less: 767.97)
    few = contiguous_problem(B=4, Hq=64, Hkv=8, L=8192)
    assert fd.fd_plan(few, num_cus=256, host_seq_lens=[8192, 8192, 8191, 1]).schedule == fd.SCHEDULES["balanced"]
    assert fd.fd_plan(few, num_cus=256, host_seq_lens=[8192, 8192, 8191, 0]).schedule == fd.SCHEDULES["uniform"]
    assert fd.fd_plan(few, num_cus=256, host_seq_lens=[8192, 8192, 8191, 0],
                      schedule="balanced").schedule == fd.SCHEDULES["balanced"]
    assert fd.fd_plan(prob, num_cus=256).schedule == fd.SCHEDULES["uniform"]
    assert fd.fd_plan(prob, num_cus=256, host_seq_lens=lens, schedule="uniform").schedule == fd.SCHEDULES["uniform"]
    assert fd.fd_plan(prob, num_cus=256, host_seq_lens=lens, force_splits=4).schedule == fd.SCHEDULES["uniform"]
    assert fd.fd_plan(prob, num_cus=256, host_seq_lens=lens, heuristic="fa2").schedule == fd.SCHEDULES["uniform"]
    # equal lengths, or short ones on average: uniform
    assert fd.fd_plan(prob, num_cus=256, host_seq_lens=[3000] * 3).schedule == fd.SCHEDULES["uniform"]
    many = contiguous_problem(B=40, Hq=32, Hkv=8, L=3000)                   # 320 segments, more than the slots
    many_lens = [3000 - (i % 7) for i in range(40)]
    assert fd.fd_plan(many, num_cus=256, host_seq_lens=many_lens).schedule == fd.SCHEDULES["balanced"]
    short = [767 + (i % 2) * 2 for i in range(40)]                           # mean 768
    assert fd.fd_plan(many, num_cus=256, host_seq_lens=short).schedule == fd.SCHEDULES["balanced"]
    short = [766 + (i % 2) * 2 for i in range(40)]                           # mean 767
    assert fd.fd_plan(many, num_cus=256, host_seq_lens=short).schedule == fd.SCHEDULES["uniform"]
    assert fd.fd_plan(many, num_cus=256, host_seq_lens=short,
                      schedule="balanced").schedule == fd.SCHEDULES["balanced"]
    # the VALU kernel (MHA) has its balanced variant too
    mha = contiguous_problem(B=3, Hq=8, Hkv=8, L=30000)
    p = fd.fd_plan(mha, num_cus=256, host_seq_lens=lens)
    assert p.kernel == fd.KERNELS["valu"] and p.schedule == fd.SCHEDULES["balanced"]
    assert p.slots == 256                               # one range per CU by default
    p2 = fd.fd_plan(mha, num_cus=256, host_seq_lens=lens, wgs_per_cu=4, schedule="balanced")
    assert p2.slots == 512                              # two resident balanced workgroups per CU at most
    # AUTO counts the work per range over those 512 ranges: 469 tokens, too few
    assert fd.fd_plan(mha, num_cus=256, host_seq_lens=lens, wgs_per_cu=4).schedule == fd.SCHEDULES["uniform"]
    with pytest.raises(fd.FdError):
        fd.fd_plan(prob, num_cus=256, schedule="balanced")            # needs host lengths
    with pytest.raises(fd.FdError):
        fd.fd_plan(prob, num_cus=256, host_seq_lens=lens, schedule="balanced", force_splits=2)


def test_forced_splits_and_chunk():
    p = fd.fd_plan(contiguous_problem(Hq=4, Hkv=4, D=64, L=1000, dtype=0), num_cus=256, force_splits=3)
    assert (p.num_splits, p.chunk_tokens) == (3, 334)
    p = fd.fd_plan(contiguous_problem(Hq=4, Hkv=4, D=64, L=1000, dtype=0), num_cus=256, force_splits=8)
    assert (p.num_splits, p.chunk_tokens) == (8, 125)
    p = fd.fd_plan(contiguous_problem(Hq=32, Hkv=32, L=65536, dtype=2), num_cus=256, force_chunk_tokens=1024,
                   ws_format="olse")
    assert (p.num_splits, p.chunk_tokens, p.ws_format) == (64, 1024, 1)
    assert p.ws_stats_bytes == 32 * 64 * 4 and p.ws_o_bytes == 32 * 64 * 128 * 4
    # paged: chunks are page- and tile-aligned
    p = fd.fd_plan(paged_problem(L=1000), num_cus=256, force_splits=3)
    assert p.chunk_tokens % 32 == 0 and p.num_splits * p.chunk_tokens >= 1000


def test_kernel_choice():
    assert fd.fd_plan(contiguous_problem(Hq=64, Hkv=8), num_cus=256).kernel == fd.KERNELS["mfma"]
    assert fd.fd_plan(contiguous_problem(Hq=8, Hkv=8), num_cus=256).kernel == fd.KERNELS["valu"]
    assert fd.fd_plan(contiguous_problem(Hq=16, Hkv=8, dtype=0), num_cus=256).kernel == fd.KERNELS["valu"]
    assert fd.fd_plan(contiguous_problem(Hq=8, Hkv=8), num_cus=256, kernel="mfma").kernel == fd.KERNELS["mfma"]


def _status(prob, **opts):
    try:
        fd.fd_plan(prob, num_cus=256, **opts)
        return fd.FD_OK
    except fd.FdError as e:
        return e.status


def test_problem_validation():
    assert _status(contiguous_problem(Hq=12, Hkv=8)) == fd.FD_ERR_INVALID_ARG
    assert _status(contiguous_problem(D=96)) == fd.FD_ERR_UNSUPPORTED
    assert _status(contiguous_problem(q_dtype=0)) == fd.FD_ERR_UNSUPPORTED
    assert _status(contiguous_problem(kv_dtype=7, q_dtype=7)) == fd.FD_ERR_INVALID_ARG
    assert _status(contiguous_problem(L=1000, cap=999)) == fd.FD_ERR_INVALID_ARG
    assert _status(contiguous_problem(kv_stride_t=132)) == fd.FD_ERR_ALIGNMENT
    assert _status(contiguous_problem(q_stride_h=129)) == fd.FD_ERR_ALIGNMENT
    assert _status(contiguous_problem(batch=0)) == fd.FD_ERR_INVALID_ARG
    assert _status(contiguous_problem(layout=5)) == fd.FD_ERR_INVALID_ARG
    assert _status(paged_problem(page=8)) == fd.FD_ERR_UNSUPPORTED
    assert _status(paged_problem(page=24)) == fd.FD_ERR_UNSUPPORTED
    assert _status(paged_problem(L=1000, max_pages_per_seq=10)) == fd.FD_ERR_INVALID_ARG
    assert _status(paged_problem(), force_chunk_tokens=40) == fd.FD_ERR_INVALID_ARG
    assert _status(contiguous_problem(Hq=64, Hkv=8, dtype=0)) == fd.FD_ERR_UNSUPPORTED    # fp32, g = 8
    assert _status(contiguous_problem(Hq=256, Hkv=8)) == fd.FD_ERR_UNSUPPORTED            # g = 32
    assert _status(contiguous_problem(dtype=0), kernel="mfma") == fd.FD_ERR_UNSUPPORTED


def test_strides_are_bounded_before_use():
    """A stride above FD_MAX_STRIDE elements is rejected instead of overflowing
    the byte products of the alignment checks; strides the layout does not use
    are not looked at."""
    import re

    hdr = open(HEADER).read()
    m = re.search(r"#define FD_MAX_STRIDE \(\(int64_t\)1 << (\d+)\)", hdr)
    assert m
    cap = 1 << int(m.group(1))
    huge = (1 << 63) - 1
    assert _status(contiguous_problem(q_stride_b=cap)) == fd.FD_OK
    assert _status(contiguous_problem(q_stride_b=cap + 8)) == fd.FD_ERR_INVALID_ARG
    for field in ("q_stride_b", "q_stride_h", "kv_stride_b", "kv_stride_h", "kv_stride_t"):
        assert _status(contiguous_problem(**{field: huge})) == fd.FD_ERR_INVALID_ARG, field
    for field in ("bt_stride_b", "pool_stride_page", "pool_stride_t", "pool_stride_h"):
        assert _status(paged_problem(**{field: huge})) == fd.FD_ERR_INVALID_ARG, field
        assert _status(contiguous_problem(**{field: huge})) == fd.FD_OK, field
    assert _status(contiguous_problem(q_stride_q=huge)) == fd.FD_OK                  # single query
    assert _status(contiguous_problem(q_len=2, q_stride_q=huge)) == fd.FD_ERR_INVALID_ARG
    assert _status(contiguous_problem(L=1000), force_chunk_tokens=100, force_splits=5) == fd.FD_ERR_INVALID_ARG
    assert _status(contiguous_problem(scale=float("nan"))) == fd.FD_ERR_INVALID_ARG
    assert _status(contiguous_problem(L=0)) == fd.FD_OK


def test_split_boundaries_fit_32_bits():
    """Uniform split s starts at token s * chunk, a 32-bit index on the device:
    a forced split count times a forced (or page-rounded) chunk past 2^31 - 1
    is refused, and the largest plan that fits is accepted."""
    big = contiguous_problem(Hq=8, Hkv=8, L=1000)
    assert _status(big, force_splits=65535, force_chunk_tokens=65536) == fd.FD_ERR_UNSUPPORTED
    assert _status(big, force_splits=32768, force_chunk_tokens=65536) == fd.FD_ERR_UNSUPPORTED   # 2^31 exactly
    p = fd.fd_plan(big, num_cus=256, force_splits=32767, force_chunk_tokens=65536)
    assert p.num_splits * p.chunk_tokens == 32767 * 65536 <= (1 << 31) - 1
    # paged: 2^20-token pages round every chunk up to a page
    paged = paged_problem(L=1 << 20, page=1 << 20, max_pages_per_seq=1)
    assert _status(paged, force_splits=4096) == fd.FD_ERR_UNSUPPORTED
    assert _status(paged, force_splits=2047) == fd.FD_OK


def test_output_rows_are_bounded():
    """B * q_len * Hq output rows index 32-bit merge grids: more than FD_MAX_ROWS
    is refused by the planner."""
    import re

    hdr = open(HEADER).read()
    m = re.search(r"#define FD_MAX_ROWS \(\(int64_t\)0x7fffffff - (\d+)\)", hdr)
    assert m
    max_rows = 0x7FFFFFFF - int(m.group(1))
    # 4096 KV heads x 16 query heads each: 65536 rows per sequence
    p = contiguous_problem(B=max_rows // 65536 + 1, Hq=65536, Hkv=4096, L=64)
    assert _status(p) == fd.FD_ERR_UNSUPPORTED
    p.batch = max_rows // 65536
    assert _status(p) == fd.FD_OK
    p = contiguous_problem(B=max_rows // (8 * 8192) + 1, Hq=8192, Hkv=4096, L=64, q_len=8,
                           q_stride_q=8192 * 128, q_stride_b=8 * 8192 * 128)
    assert _status(p) == fd.FD_ERR_UNSUPPORTED                         # g * q_len = 16, rows include q_len


def test_plan_resolves_scale_and_workspace():
    p = fd.fd_plan(contiguous_problem(B=2, Hq=16, Hkv=8, D=64, L=500), num_cus=256)
    assert abs(p.scale - 1 / 8) < 1e-7
    assert p.ws_o_bytes == 2 * 16 * p.num_splits * 64 * 4
    assert p.ws_stats_bytes == 2 * 16 * p.num_splits * 2 * 4
    p = fd.fd_plan(contiguous_problem(scale=0.3), num_cus=256)
    assert abs(p.scale - 0.3) < 1e-7


# ---------------------------------------------------------------------------
# Decode/merge argument validation: every case fails before any HIP call.
# ---------------------------------------------------------------------------

def _split_status(plan, args, ws_o=4096, ws_o_bytes=1 << 40, ws_st=8192, ws_st_bytes=1 << 40):
    return fd.lib().fd_decode_split(ctypes.byref(plan), ctypes.byref(args) if args is not None else None,
                                    ws_o, ws_o_bytes, ws_st, ws_st_bytes, None)


def test_decode_and_merge_validation_without_gpu():
    plan = fd.fd_plan(contiguous_problem(Hq=64, Hkv=8), num_cus=256)
    good = fd.Args(0x10000, 0x20000, 0x30000, 0x40000, None)
    assert _split_status(plan, None) == fd.FD_ERR_INVALID_ARG
    assert _split_status(plan, fd.Args(0, 0x20000, 0x30000, 0x40000, None)) == fd.FD_ERR_INVALID_ARG
    assert _split_status(plan, fd.Args(0x10008, 0x20000, 0x30000, 0x40000, None)) == fd.FD_ERR_ALIGNMENT
    assert _split_status(plan, good, ws_o=4100) == fd.FD_ERR_ALIGNMENT
    assert _split_status(plan, good, ws_o_bytes=plan.ws_o_bytes - 4) == fd.FD_ERR_WORKSPACE
    assert _split_status(plan, good, ws_st_bytes=plan.ws_stats_bytes - 4) == fd.FD_ERR_WORKSPACE
    bad = fd.Plan.from_buffer_copy(plan)
    bad.num_splits += 1
    assert _split_status(bad, good) == fd.FD_ERR_BAD_PLAN
    bad = fd.Plan.from_buffer_copy(plan)
    bad.magic = 0
    assert _split_status(bad, good) == fd.FD_ERR_BAD_PLAN
    L = fd.lib()
    big = 1 << 40

    def merge(pl, ws_o=4096, ws_o_bytes=big, ws_st=8192, ws_st_bytes=big, out=4096):
        return L.fd_merge(ctypes.byref(pl), ws_o, ws_o_bytes, ws_st, ws_st_bytes, out, None, None)

    assert merge(bad) == fd.FD_ERR_BAD_PLAN
    assert merge(plan, ws_o=None) == fd.FD_ERR_INVALID_ARG
    assert merge(plan, out=None) == fd.FD_ERR_INVALID_ARG
    assert merge(plan, out=4100) == fd.FD_ERR_ALIGNMENT
    # a workspace shorter than the plan's is refused before any launch
    assert merge(plan, ws_o_bytes=plan.ws_o_bytes - 4) == fd.FD_ERR_WORKSPACE
    assert merge(plan, ws_st_bytes=plan.ws_stats_bytes - 4) == fd.FD_ERR_WORKSPACE
    assert merge(plan, ws_o_bytes=0, ws_st_bytes=0) == fd.FD_ERR_WORKSPACE
    paged = fd.fd_plan(paged_problem(), num_cus=256)
    assert _split_status(paged, good) == fd.FD_ERR_INVALID_ARG          # no block table


def test_binding_checks_tensors_against_the_plan():
    """The Python launch wrappers refuse, before any C call, tensors that do not
    match the plan: host tensors, int64 lengths (read as int32 pairs they would
    give wrong lengths), a missing or short block table, K/V of another shape,
    and outputs or workspaces of the wrong size or type."""
    B, Hq, Hkv, D, T = 2, 8, 2, 128, 64
    q = torch.zeros(B, Hq, D, dtype=torch.float16)
    k = torch.zeros(B, Hkv, T, D, dtype=torch.float16)
    sl = torch.tensor([64, 5], dtype=torch.int32)
    plan = fd.fd_plan(fd.problem_for(q, k, k, sl), num_cus=256)
    ws_o, ws_st = torch.zeros(1), torch.zeros(1)

    def msg(fn):
        with pytest.raises(ValueError) as e:
            fn()
        return str(e.value)

    assert "GPU" in msg(lambda: fd.fd_decode_split(plan, q, k, k, sl, ws_o, ws_st))
    assert "seq_lens" in msg(lambda: fd.fd_decode_split(plan, q, k, k, sl.to(torch.int64), ws_o, ws_st))
    assert "seq_lens" in msg(lambda: fd.fd_decode_split(plan, q, k, k, sl[:1], ws_o, ws_st))
    assert "K shape" in msg(lambda: fd.fd_decode_split(plan, q, k[:, :, :32], k, sl, ws_o, ws_st))
    assert "dtypes" in msg(lambda: fd.fd_decode_split(plan, q.float(), k, k, sl, ws_o, ws_st))
    assert "q shape" in msg(lambda: fd.fd_decode_split(plan, q[:1], k, k, sl, ws_o, ws_st))
    assert "block_table" in msg(lambda: fd.fd_decode_split(plan, q, k, k, sl, ws_o, ws_st,
                                                           torch.zeros(B, 4, dtype=torch.int32)))
    pool = torch.zeros(8, 16, Hkv, D, dtype=torch.float16)
    bt = torch.zeros(B, 4, dtype=torch.int32)
    paged = fd.fd_plan(fd.problem_for(q, pool, pool, sl, bt), num_cus=256)
    assert "block_table" in msg(lambda: fd.fd_decode_split(paged, q, pool, pool, sl, ws_o, ws_st))
    assert "block_table" in msg(lambda: fd.fd_decode_split(paged, q, pool, pool, sl, ws_o, ws_st, bt[:1]))
    assert "block_table" in msg(lambda: fd.fd_decode_split(paged, q, pool, pool, sl, ws_o, ws_st, bt.long()))
    out = torch.zeros(B, Hq, D)
    lse = torch.zeros(B, Hq)
    fd._check_outputs(plan, out, lse)
    assert "out" in msg(lambda: fd._check_outputs(plan, out[:1], lse))
    assert "lse" in msg(lambda: fd._check_outputs(plan, out, lse.double()))
    assert "out" in msg(lambda: fd._check_outputs(plan, out.transpose(0, 1), lse))
    assert "ws_o" in msg(lambda: fd.fd_merge(plan, ws_o.double(), ws_st, out, lse))


def test_noalloc_validation_without_gpu():
    """fd_decode_fused_noalloc checks everything on the host before any HIP
    call: a plan whose workspace and counters exceed the static scratch, a
    tampered plan, missing arguments and misaligned outputs."""
    L = fd.lib()
    hdr = open(HEADER).read()
    m = re.search(r"#define FD_NOALLOC_SCRATCH_BYTES \((\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == fd.NOALLOC_SCRATCH_BYTES
    good = fd.Args(0x10000, 0x20000, 0x30000, 0x40000, None)
    plan = fd.fd_plan(contiguous_problem(B=2, Hq=64, Hkv=8, L=20000), num_cus=256)

    def call(pl, args=good, out=0x50000, lse=None):
        return L.fd_decode_fused_noalloc(ctypes.byref(pl), ctypes.byref(args) if args is not None else None,
                                         out, lse, None)

    assert call(plan, args=None) == fd.FD_ERR_INVALID_ARG
    assert call(plan, out=None) == fd.FD_ERR_INVALID_ARG
    assert call(plan, out=0x50004) == fd.FD_ERR_ALIGNMENT
    assert call(plan, args=fd.Args(0x10008, 0x20000, 0x30000, 0x40000, None)) == fd.FD_ERR_ALIGNMENT
    bad = fd.Plan.from_buffer_copy(plan)
    bad.num_splits += 1
    assert call(bad) == fd.FD_ERR_BAD_PLAN
    # 256 sequences x 64 query heads x 128 splits of fp32 states: 32 MiB of ws_o alone
    big = fd.fd_plan(contiguous_problem(B=256, Hq=64, Hkv=8, L=100000), num_cus=256, force_splits=128)
    assert big.ws_o_bytes >= fd.NOALLOC_SCRATCH_BYTES
    assert call(big) == fd.FD_ERR_WORKSPACE


def test_merge_states_validation_without_gpu():
    """Every argument error of fd_merge_states is caught on the host, before
    any launch (so none of these calls touches a device)."""
    L = fd.lib()
    olse, uml = fd.WS_FORMATS["olse"], fd.WS_FORMATS["uml"]
    ok = (0x10000, 0x20000, 8, 4, 128, 0x30000, 0x40000, None)

    def st(fmt, *a):
        return L.fd_merge_states(fmt, *a)
    assert st(7, *ok) == fd.FD_ERR_INVALID_ARG                             # format
    assert st(olse, 0x10000, 0x20000, -1, 4, 128, 0x30000, None, None) == fd.FD_ERR_INVALID_ARG
    assert st(olse, 0x10000, 0x20000, 1 << 31, 4, 128, 0x30000, None, None) == fd.FD_ERR_INVALID_ARG
    assert st(olse, 0x10000, 0x20000, (1 << 31) - 4096, 4, 128, 0x30000, None, None) == fd.FD_ERR_INVALID_ARG
    assert st(olse, 0x10000, 0x20000, 8, 0, 128, 0x30000, None, None) == fd.FD_ERR_INVALID_ARG
    assert st(olse, 0x10000, 0x20000, 8, 65536, 128, 0x30000, None, None) == fd.FD_ERR_INVALID_ARG
    assert st(olse, 0x10000, 0x20000, 8, 4, 96, 0x30000, None, None) == fd.FD_ERR_UNSUPPORTED
    assert st(olse, None, 0x20000, 8, 4, 128, 0x30000, None, None) == fd.FD_ERR_INVALID_ARG
    assert st(olse, 0x10000, None, 8, 4, 128, 0x30000, None, None) == fd.FD_ERR_INVALID_ARG
    assert st(olse, 0x10000, 0x20000, 8, 4, 128, None, None, None) == fd.FD_ERR_INVALID_ARG
    assert st(olse, 0x10004, 0x20000, 8, 4, 128, 0x30000, None, None) == fd.FD_ERR_ALIGNMENT
    assert st(olse, 0x10000, 0x20002, 8, 4, 128, 0x30000, None, None) == fd.FD_ERR_ALIGNMENT
    assert st(uml, 0x10000, 0x20004, 8, 4, 128, 0x30000, None, None) == fd.FD_ERR_ALIGNMENT
    assert st(olse, 0x10000, 0x20000, 8, 4, 128, 0x30008, None, None) == fd.FD_ERR_ALIGNMENT
    assert st(olse, 0x10000, 0x20000, 8, 4, 128, 0x30000, 0x40002, None) == fd.FD_ERR_ALIGNMENT
    assert st(olse, None, None, 0, 4, 128, None, None, None) == fd.FD_OK  # zero rows: nothing to do
    with pytest.raises(ValueError):
        fd.fd_merge_states(torch.zeros(3, 4, 128), torch.zeros(3, 5))
    with pytest.raises(ValueError):
        fd.fd_merge_states(torch.zeros(3, 4, 128), torch.zeros(3, 4), ws_format="uml")


def test_query_block_problems():
    """Short query blocks: validation, kernel choice by rows per KV head
    (g * q_len), workspace rows and the q_len = 1 equivalence."""
    def qb(q_len, Hq=8, Hkv=4, dtype=1, stride_q=None):
        p = contiguous_problem(Hq=Hq, Hkv=Hkv, L=500, dtype=dtype)
        p.q_len = q_len
        p.q_stride_q = Hq * 128 if stride_q is None else stride_q
        p.q_stride_b = q_len * Hq * 128
        return p
    assert fd.fd_plan(qb(4), num_cus=256).kernel == fd.KERNELS["mfma"]          # g=2, R=8
    assert fd.fd_plan(qb(8), num_cus=256).kernel == fd.KERNELS["mfma"]          # R=16: two column tiles
    with pytest.raises(fd.FdError):
        fd.fd_plan(qb(5, Hq=16, Hkv=4), num_cus=256)                             # g=4, R=20 > 16
    assert fd.fd_plan(qb(8, Hq=4, Hkv=4), num_cus=256, kernel="mfma").kernel == fd.KERNELS["mfma"]
    assert fd.fd_plan(qb(2, Hq=4, Hkv=4, dtype=0), num_cus=256).kernel == fd.KERNELS["valu"]   # fp32: VALU
    with pytest.raises(fd.FdError):
        fd.fd_plan(qb(8, Hq=4, Hkv=4, dtype=0), num_cus=256)                   # fp32, R=8 > 4
    with pytest.raises(fd.FdError):
        fd.fd_plan(qb(9, Hq=4, Hkv=4), num_cus=256)                             # q_len > 8
    with pytest.raises(fd.FdError):
        fd.fd_plan(qb(2, stride_q=1028), num_cus=256)                           # misaligned row stride
    p = fd.fd_plan(qb(3), num_cus=256, force_splits=2)
    assert p.ws_o_bytes == 3 * 8 * 2 * 128 * 4 and p.ws_stats_bytes == 3 * 8 * 2 * 2 * 4
    a = fd.fd_plan(qb(1), num_cus=256)
    b = fd.fd_plan(qb(0), num_cus=256)
    assert (a.num_splits, a.chunk_tokens, a.ws_o_bytes) == (b.num_splits, b.chunk_tokens, b.ws_o_bytes)
    q = torch.zeros(2, 3, 8, 128, dtype=torch.float16)
    k = torch.zeros(2, 4, 300, 128, dtype=torch.float16)
    pr = fd.problem_for(q, k, k, torch.tensor([300, 2], dtype=torch.int32))
    assert (pr.q_len, pr.q_stride_q, pr.q_stride_h, pr.q_stride_b) == (3, 8 * 128, 128, 3 * 8 * 128)


def test_read_probe_validation_without_gpu():
    L = fd.lib()
    n = fd.READ_PROBE_SINK_BYTES
    assert L.fd_read_probe(None, 1 << 20, 0x20000, n, None) == fd.FD_ERR_INVALID_ARG
    assert L.fd_read_probe(0x10000, 1 << 20, None, n, None) == fd.FD_ERR_INVALID_ARG
    assert L.fd_read_probe(0x10000, 8, 0x20000, n, None) == fd.FD_ERR_INVALID_ARG
    assert L.fd_read_probe(0x10000, (1 << 20) + 4, 0x20000, n, None) == fd.FD_ERR_INVALID_ARG
    assert L.fd_read_probe(0x10008, 1 << 20, 0x20000, n, None) == fd.FD_ERR_ALIGNMENT
    assert L.fd_read_probe(0x10000, 1 << 20, 0x20000, n - 4, None) == fd.FD_ERR_WORKSPACE


def test_wg_stamps_only_in_the_stamp_build():
    """The release library records no per-workgroup stamps: fd_wg_stamps
    refuses before touching the device, whatever it is given."""
    L = fd.lib()
    assert L.fd_wg_stamps(0x10000, fd.WG_STAMP_RECORDS * 32, None) == fd.FD_ERR_UNSUPPORTED
    assert L.fd_wg_stamps(None, 0, None) == fd.FD_ERR_UNSUPPORTED


def test_problem_for_tensors():
    q = torch.zeros(2, 16, 128, dtype=torch.float16)
    k = torch.zeros(2, 4, 300, 128, dtype=torch.float16)
    sl = torch.tensor([300, 5], dtype=torch.int32)
    p = fd.problem_for(q, k, k, sl)
    assert (p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.max_seq_len) == (2, 16, 4, 128, 300)
    assert (p.kv_stride_b, p.kv_stride_h, p.kv_stride_t, p.kv_capacity) == (4 * 300 * 128, 300 * 128, 128, 300)
    pool = torch.zeros(10, 16, 4, 128, dtype=torch.bfloat16)
    bt = torch.zeros(2, 5, dtype=torch.int32)
    p = fd.problem_for(q.to(torch.bfloat16), pool, pool, torch.tensor([70, 3], dtype=torch.int32), bt)
    assert (p.layout, p.page_size, p.num_pages, p.max_pages_per_seq, p.pool_stride_t) == (1, 16, 10, 5, 512)
    with pytest.raises(ValueError):
        fd.problem_for(q, k, k[:, :, :200], sl)


def test_every_entry_point_is_documented_with_its_source():
    """Each declaration in fd.h sits under its own comment; the decode calls'
    comments cite the page passage that defines the operation."""
    src = open(HEADER).read()
    decls = list(re.finditer(r"FD_API\s+[\w\s\*]+?\b(fd_\w+)\s*\(", src))
    prev_end = 0
    for m in decls:
        before = src[prev_end:m.start()]
        comment = before[before.rfind("/*"):] if "/*" in before else ""
        assert comment.strip(), f"{m.group(1)} has no comment above it"
        if m.group(1) in ("fd_plan", "fd_decode_split", "fd_merge", "fd_decode_fused", "fd_merge_states"):
            assert re.search(r"kanthi\.in|xuujii|tinyvolt", comment), f"{m.group(1)} cites no page"
        prev_end = src.index(";", m.end()) + 1


def test_balanced_plan_worked_example():
    """The planner on a partition worked out by hand: lengths [320, 96], one KV
    head, four CUs, no cost granules. Segments hold 10 and 3 granules of 32
    tokens (T = 13); N = min(4 slots, cdiv(13, 4)) = 4 ranges
    [0,3), [3,6), [6,9), [9,13). Sequence 0's granules [0,10) meet all four
    ranges (four pieces), sequence 1's [10,13) only the last: S = 4."""
    prob = contiguous_problem(B=2, Hq=4, Hkv=1, L=320)
    plan = fd.fd_plan(prob, num_cus=4, host_seq_lens=[320, 96], schedule="balanced", piece_cost_tokens=-1)
    assert plan.schedule == fd.SCHEDULES["balanced"] and plan.piece_cost == 0
    assert (plan.grid_x, plan.grid_y, plan.grid_z) == (4, 1, 1)
    assert plan.num_splits == 4 and plan.chunk_tokens == 32
