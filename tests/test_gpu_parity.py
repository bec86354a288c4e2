"""GPU parity: the HIP split + merge path (through the C ABI) against the
float64 oracle, element by element. Needs an MI355X and the built libfd.so."""
import math

import numpy as np
import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W
from oracle import attention as A
from tests import gpu_helpers as H
from tests.conftest import golden

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# Tiny MHA, fp32 (VALU path): every split count, both workspace forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("splits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("q_gain", [1.0, 40.0])
def test_tiny_mha_f32_every_split_count(splits, q_gain):
    w = W.tiny_mha_f32(num_splits=splits, q_gain=q_gain)
    plan, out, lse, _, _ = H.run(w)
    assert plan.num_splits == splits and plan.kernel == fd.KERNELS["valu"]
    st = H.check_against_oracle(w, out, lse)
    assert st["max_abs"] <= 1e-4          # fp32 cache: far inside the 2e-3 bar


@pytest.mark.parametrize("fmt", ["uml", "olse"])
def test_tiny_partial_states_match_oracle_splits(fmt):
    w = W.tiny_mha_f32(num_splits=3)
    plan, out, lse, ws_o, ws_stats = H.run(w, ws_format=fmt)
    o_s, lse_s, m_s, l_s = H.split_states_of(plan, ws_o, ws_stats)
    M, L, U = A.split_states(H.cache_of(w), plan.num_splits, plan.chunk_tokens)
    for s in range(plan.num_splits):
        for h in range(w.num_q_heads):
            o_ref, lse_ref = A.state_to_olse(M[0, h, s], L[0, h, s], U[0, h, s])
            assert np.abs(o_s[0, h, s] - o_ref).max() < 1e-5
            assert abs(lse_s[0, h, s] - lse_ref) < 1e-5 * max(1, abs(lse_ref))
            if fmt == "uml":           # m is the split's largest score, l its sum of e^(s - m)
                assert abs(m_s[0, h, s] - M[0, h, s]) < 1e-5 * max(1, abs(M[0, h, s]))
                assert abs(l_s[0, h, s] - L[0, h, s]) < 1e-5 * L[0, h, s]


@pytest.mark.parametrize("fmt", ["uml", "olse"])
def test_odd_xcd_shifted_plan_states(fmt):
    """A uniform plan the MI355X rule shifts (even split count, contiguous cache,
    256 CUs, splits of at least 1536 tokens; here S = 20 of 2547 / 2329):
    even-numbered splits hold chunk_tokens tokens and odd-numbered ones
    odd_chunk_tokens. Every split state of sampled rows against the oracle's
    states over the same alternating partition, and every output."""
    w = W.contiguous("xcd_shift", seed=120, batch=2, q_heads=64, kv_heads=8, head_dim=128, capacity=48000,
                     seq_lens=[48000, 30001], dtype="f16")
    plan, out, lse, ws_o, ws_stats = H.run(w, ws_format=fmt, schedule="uniform")
    H.say(f"shifted plan: S={plan.num_splits} chunks {plan.chunk_tokens}/{plan.odd_chunk_tokens}")
    assert plan.num_splits % 2 == 0 and plan.chunk_tokens > plan.odd_chunk_tokens
    H.check_against_oracle(w, out, lse)
    pairs = [(0, 0), (0, 37), (1, 5), (1, 63)]
    bounds = lambda b, h: A.alternating_bounds(int(w.seq_lens[b]), plan.chunk_tokens, plan.odd_chunk_tokens,
                                               plan.num_splits)
    M, L, U = A.split_states(H.cache_of(w), plan.num_splits, 0, pairs=pairs, bounds=bounds)
    o_s, lse_s, m_s, l_s = H.split_states_of(plan, ws_o, ws_stats)
    for b, h in pairs:
        for s in range(plan.num_splits):
            if L[b, h, s] == 0:
                assert np.isneginf(lse_s[b, h, s]) and np.all(o_s[b, h, s] == 0)
                continue
            o_ref, lse_ref = A.state_to_olse(M[b, h, s], L[b, h, s], U[b, h, s])
            assert np.abs(o_s[b, h, s] - o_ref).max() < 2e-3, (b, h, s)
            assert abs(lse_s[b, h, s] - lse_ref) < 1e-5 * max(1, abs(lse_ref)), (b, h, s)


SHIFTED_CASES = {
    # name: (workload arguments, odd_xcd_permille, fused)
    "mha_bf16_valu": (dict(batch=1, q_heads=8, kv_heads=8, head_dim=128, capacity=50000, seq_lens=[50000],
                           dtype="bf16"), 0, False),
    "gqa4_f16_d64_qblock2": (dict(batch=2, q_heads=16, kv_heads=4, head_dim=64, capacity=60000,
                                  seq_lens=[60000, 41000], dtype="f16", q_len=2), 300, False),
    "gqa2_f32_d64_valu": (dict(batch=1, q_heads=8, kv_heads=4, head_dim=64, capacity=120000, seq_lens=[120000],
                               dtype="f32"), 100, False),
    "gqa8_bf16_fused": (dict(batch=1, q_heads=64, kv_heads=8, head_dim=128, capacity=50000, seq_lens=[50000],
                             dtype="bf16"), 0, True),
}


@pytest.mark.parametrize("name", sorted(SHIFTED_CASES))
def test_odd_xcd_shifted_plan_variants(name):
    """Shifted uniform plans on both kernels (VALU for g = 1 and fp32 caches),
    a two-row query block, a large shift (300 per mille) and the fused call:
    every output row against the oracle."""
    kw, x, fused = SHIFTED_CASES[name]
    w = W.contiguous(name, seed=130, **kw)
    opts = dict(num_cus=256, schedule="uniform", odd_xcd_permille=x)
    if fused:
        plan, out, lse, ctr = H.run_fused(w, **opts)
        assert torch.all(ctr == 0).item()
    else:
        plan, out, lse, _, _ = H.run(w, **opts)
    H.say(f"{name}: S={plan.num_splits} chunks {plan.chunk_tokens}/{plan.odd_chunk_tokens} kernel={plan.kernel}")
    assert plan.num_splits % 2 == 0 and plan.chunk_tokens > plan.odd_chunk_tokens
    H.check_against_oracle(w, out, lse)


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("q_gain", [1.0, 40.0])
def test_ragged_batch_with_empty_splits(splits, q_gain):
    w = W.ragged_mha_f32(num_splits=splits, q_gain=q_gain)
    plan, out, lse, ws_o, ws_stats = H.run(w)
    H.check_against_oracle(w, out, lse)
    o_s, lse_s, m_s, l_s = H.split_states_of(plan, ws_o, ws_stats)
    # with 8 splits of 125 tokens the 37-token row has 7 empty splits: neutral states, exactly
    for b, L in enumerate(w.seq_lens.tolist()):
        for s in range(plan.num_splits):
            if s * plan.chunk_tokens >= L:
                assert np.all(ws_o[b, :, s].numpy() == 0)
                assert np.all(np.isneginf(m_s[b, :, s])) and np.all(l_s[b, :, s] == 0)


# ---------------------------------------------------------------------------
# Packed GQA on MFMA, fp16 / bf16, several tiles and a ragged tail
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("g", [2, 4, 8])
@pytest.mark.parametrize("D", [64, 128])
def test_gqa_mfma_small(dtype, g, D):
    w = W.contiguous(f"gqa_g{g}_D{D}_{dtype}", seed=10 + g, batch=2, q_heads=4 * g, kv_heads=4, head_dim=D,
                     capacity=3001, seq_lens=[3001, 1234], dtype=dtype)
    for splits in (0, 1, 3, 7):
        plan, out, lse, _, _ = H.run(w, force_splits=splits) if splits else H.run(w)
        assert plan.kernel == fd.KERNELS["mfma"]
        H.check_against_oracle(w, out, lse)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("g", [1, 2, 4])
def test_valu_small_groups(dtype, g):
    w = W.contiguous(f"valu_g{g}_{dtype}", seed=20 + g, batch=2, q_heads=2 * g, kv_heads=2, head_dim=128,
                     capacity=2500, seq_lens=[2500, 77], dtype=dtype)
    for splits in (1, 4):
        plan, out, lse, _, _ = H.run(w, force_splits=splits, kernel="valu")
        H.check_against_oracle(w, out, lse)


def test_mfma_forced_for_mha():
    w = W.contiguous("mha_mfma_bf16", seed=31, batch=2, q_heads=4, kv_heads=4, head_dim=128, capacity=1500,
                     seq_lens=[1500, 700], dtype="bf16")
    plan, out, lse, _, _ = H.run(w, kernel="mfma", force_splits=5)
    assert plan.kernel == fd.KERNELS["mfma"]
    H.check_against_oracle(w, out, lse)


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513])
def test_sequence_edges(L):
    """seq_len at 1, tile - 1, tile, tile + 1 and chunk*k +- 1 (chunk 128)."""
    w = W.contiguous(f"edge_L{L}", seed=40, batch=1, q_heads=16, kv_heads=2, head_dim=128, capacity=600,
                     seq_lens=[L], dtype="f16")
    plan, out, lse, _, _ = H.run(w, force_chunk_tokens=128, force_splits=5)
    H.check_against_oracle(w, out, lse)
    w2 = W.contiguous(f"edge_valu_L{L}", seed=41, batch=1, q_heads=2, kv_heads=2, head_dim=64, capacity=600,
                      seq_lens=[L], dtype="bf16")
    plan, out, lse, _, _ = H.run(w2, force_chunk_tokens=128, force_splits=5)
    H.check_against_oracle(w2, out, lse)


def test_zero_length_rows():
    w = W.contiguous("zero_rows", seed=42, batch=3, q_heads=8, kv_heads=2, head_dim=128, capacity=300,
                     seq_lens=[0, 300, 0], dtype="f16")
    plan, out, lse, _, _ = H.run(w, force_splits=2)
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
    assert torch.all(torch.isneginf(lse[0])) and torch.all(torch.isneginf(lse[2]))
    H.check_against_oracle(w, out, lse)


# ---------------------------------------------------------------------------
# Paged layout
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["hnd", "nhd"])
@pytest.mark.parametrize("page", [16, 32, 64])
@pytest.mark.parametrize("g", [1, 4])
def test_paged_small(page, g, layout):
    lens = [1000, 17, 333, 16]
    w = W.paged(f"paged_p{page}_g{g}_{layout}", seed=50 + page, batch=4, q_heads=4 * g, kv_heads=4,
                head_dim=128, seq_lens=lens, page_size=page, dtype="f16", extra_pages=3, pool_layout=layout)
    for splits in (1, 3):
        plan, out, lse, _, _ = H.run(w, force_splits=splits)
        H.check_against_oracle(w, out, lse)


@pytest.mark.parametrize("paged", [False, True])
def test_length_aware_plan(paged):
    """A ragged batch planned from its host lengths (splits sized by total work)
    and without them (by the longest row): both match the oracle."""
    lens = [3000, 40, 1, 0, 2500, 700]
    if paged:
        w = W.paged("lenaware_paged", seed=56, batch=6, q_heads=16, kv_heads=2, head_dim=128, seq_lens=lens,
                    page_size=16, dtype="f16")
    else:
        w = W.contiguous("lenaware", seed=57, batch=6, q_heads=16, kv_heads=2, head_dim=128, capacity=3000,
                         seq_lens=lens, dtype="bf16")
    seen = set()
    for opts in ({"host_seq_lens": lens}, {"host_seq_lens": None}, {"host_seq_lens": lens, "num_cus": 7}):
        plan, out, lse, _, _ = H.run(w, **opts)
        seen.add(plan.num_splits)
        H.check_against_oracle(w, out, lse)
    assert len(seen) >= 2, seen


# ---------------------------------------------------------------------------
# LSE checks: base and scale (merge two halves outside the library)
# ---------------------------------------------------------------------------

def test_external_merge_of_two_halves():
    w = W.contiguous("halves", seed=60, batch=1, q_heads=16, kv_heads=2, head_dim=128, capacity=4000,
                     seq_lens=[4000], dtype="f16", q_gain=3.0)
    _, out, lse, _, _ = H.run(w)
    parts = []
    for lo, hi in ((0, 1700), (1700, 4000)):
        wh = W.Workload("half", w.q, w.k[:, :, lo:hi].contiguous(), w.v[:, :, lo:hi].contiguous(),
                        torch.tensor([hi - lo], dtype=torch.int32))
        _, o_h, l_h, _, _ = H.run(wh)
        parts.append((o_h.double().numpy(), l_h.double().numpy()))
    O, LSE = A.decode_attention(H.cache_of(w))
    for h in range(16):
        om, lm = A.merge_olse([(p[0][0, h], p[1][0, h]) for p in parts])
        assert np.abs(om - O[0, h]).max() < 2e-3
        assert abs(lm - LSE[0, h]) < 1e-5 * max(1, abs(LSE[0, h]))
        assert abs(lm - lse[0, h].item()) < 1e-5 * max(1, abs(LSE[0, h]))


# ---------------------------------------------------------------------------
# Merge kernel alone: the merge-trap states of the kanthi.in chapter §3
# ---------------------------------------------------------------------------

def test_merge_trap_states_through_fd_merge():
    g = golden("merge_trap.json")
    prob = fd.Problem()
    prob.batch, prob.num_q_heads, prob.num_kv_heads, prob.head_dim = 1, 1, 1, 64
    prob.q_dtype = prob.kv_dtype = 1
    prob.max_seq_len = 3
    prob.q_stride_h = prob.q_stride_b = 64
    prob.kv_stride_t, prob.kv_stride_h, prob.kv_stride_b, prob.kv_capacity = 64, 192, 192, 3
    plan = fd.fd_plan(prob, num_cus=256, force_splits=3, force_chunk_tokens=1, ws_format="olse")
    ws_o = torch.zeros(1, 1, 3, 64, dtype=torch.float32)
    ws_o[0, 0, :, :2] = torch.tensor(g["o_f32"])
    ws_st = torch.tensor(g["lse_f32"], dtype=torch.float32).reshape(1, 1, 3, 1)
    out = torch.empty(1, 1, 64, device="cuda")
    lse = torch.empty(1, 1, device="cuda")
    fd.fd_merge(plan, ws_o.cuda(), ws_st.cuda(), out, lse)
    torch.cuda.synchronize()
    pr = g["printed"]
    np.testing.assert_allclose(out[0, 0, :2].cpu().numpy(), pr["stable_merge"], rtol=0, atol=1e-6)
    assert torch.all(out[0, 0, 2:] == 0)
    assert abs(lse.item() - pr["merged_lse"]) < 1e-4
    # same states in the (u, m, l) form: u = o, m = lse, l = 1
    plan_u = fd.fd_plan(prob, num_cus=256, force_splits=3, force_chunk_tokens=1, ws_format="uml")
    ws_su = torch.stack([ws_st[..., 0], torch.ones_like(ws_st[..., 0])], -1)
    fd.fd_merge(plan_u, ws_o.cuda(), ws_su.cuda(), out, lse)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out[0, 0, :2].cpu().numpy(), pr["stable_merge"], rtol=0, atol=1e-6)


def test_merge_all_empty_and_worked_example():
    # worked example of the xuujii page as two (m, l, u) states with D = 64 (value in dim 0)
    ex = golden("worked_example.json")
    prob = fd.Problem()
    prob.batch, prob.num_q_heads, prob.num_kv_heads, prob.head_dim = 2, 1, 1, 64
    prob.q_dtype = prob.kv_dtype = 1
    prob.max_seq_len = 4
    prob.q_stride_h, prob.q_stride_b = 64, 64
    prob.kv_stride_t, prob.kv_stride_h, prob.kv_stride_b, prob.kv_capacity = 64, 256, 256, 4
    plan = fd.fd_plan(prob, num_cus=256, force_splits=2, force_chunk_tokens=2)
    ws_o = torch.zeros(2, 1, 2, 64)
    ws_st = torch.zeros(2, 1, 2, 2)
    for s, blk in enumerate(ex["blocks"]):
        ws_o[0, 0, s, 0] = blk["u"]
        ws_st[0, 0, s] = torch.tensor([math.log(blk["m_log_of"]), blk["l"]])
    ws_st[1, 0, :, 0] = -math.inf         # row 1: every split empty
    out = torch.empty(2, 1, 64, device="cuda")
    lse = torch.empty(2, 1, device="cuda")
    fd.fd_merge(plan, ws_o.cuda(), ws_st.cuda(), out, lse)
    torch.cuda.synchronize()
    assert abs(out[0, 0, 0].item() - ex["output"]) < 1e-6
    assert abs(lse[0, 0].item() - math.log(10.0)) < 1e-6
    assert torch.all(out[1] == 0) and math.isinf(lse[1, 0].item()) and lse[1, 0].item() < 0


# ---------------------------------------------------------------------------
# Determinism and streams
# ---------------------------------------------------------------------------

def test_bitwise_deterministic_for_fixed_plan():
    w = W.contiguous("det", seed=70, batch=2, q_heads=32, kv_heads=4, head_dim=128, capacity=5000,
                     seq_lens=[5000, 4321], dtype="f16")
    a = H.run(w, force_splits=6)
    b = H.run(w, force_splits=6)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]) and torch.equal(a[3], b[3])


def test_runs_on_a_side_stream():
    w = W.contiguous("stream", seed=71, batch=1, q_heads=8, kv_heads=1, head_dim=128, capacity=2000,
                     seq_lens=[2000], dtype="bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        plan, out, lse, _, _ = H.run(w, stream=s)
    H.check_against_oracle(w, out, lse)


def test_occupancy_table_matches_device():
    """The built-in resident-workgroup table the planner uses without a device
    equals what the device reports for the same kernels."""
    props = torch.cuda.get_device_properties(0)
    cases = [(64, 8, 128, torch.float16, None), (32, 8, 64, torch.bfloat16, None), (32, 32, 128, torch.bfloat16, None),
             (4, 4, 64, torch.float32, None), (32, 8, 128, torch.float16, 16), (8, 4, 128, torch.float16, None)]
    for hq, hkv, d, dt, page in cases:
        q = torch.zeros(1, hq, d, dtype=dt, device="cuda")
        sl = torch.tensor([100], dtype=torch.int32, device="cuda")
        if page:
            k = torch.zeros(8, page, hkv, d, dtype=dt, device="cuda")
            bt = torch.zeros(1, 8, dtype=torch.int32, device="cuda")
        else:
            k = torch.zeros(1, hkv, 100, d, dtype=dt, device="cuda")
            bt = None
        prob = fd.problem_for(q, k, k, sl, bt)
        dev_plan = fd.fd_plan(prob)                                   # num_cus = 0: ask the device
        host_plan = fd.fd_plan(prob, num_cus=props.multi_processor_count)
        H.say(f"{hq}/{hkv} D{d} {dt} page={page}: CUs {props.multi_processor_count} device slots "
              f"{dev_plan.slots} table slots {host_plan.slots}")
        assert dev_plan.slots == host_plan.slots


# ---------------------------------------------------------------------------
# Fused merge (one launch): last workgroup per (sequence, KV head) merges
# ---------------------------------------------------------------------------

_run_fused = H.run_fused


@pytest.mark.parametrize("case", ["gqa_f16", "mha_bf16_valu", "paged", "tiny_f32", "zero_rows"])
def test_fused_matches_oracle(case):
    if case == "gqa_f16":
        w, opts = W.contiguous("fused_gqa", seed=80, batch=2, q_heads=32, kv_heads=4, head_dim=128, capacity=5000,
                               seq_lens=[5000, 1111], dtype="f16"), {}
    elif case == "mha_bf16_valu":
        w, opts = W.contiguous("fused_mha", seed=81, batch=2, q_heads=4, kv_heads=4, head_dim=128, capacity=3000,
                               seq_lens=[3000, 5], dtype="bf16"), {"force_splits": 7, "ws_format": "olse"}
    elif case == "paged":
        w, opts = W.paged("fused_paged", seed=82, batch=3, q_heads=16, kv_heads=4, head_dim=128,
                          seq_lens=[2000, 17, 700], page_size=16, dtype="f16"), {"force_splits": 5}
    elif case == "tiny_f32":
        w, opts = W.ragged_mha_f32(num_splits=8), {}
    else:
        w, opts = W.contiguous("fused_zero", seed=83, batch=3, q_heads=8, kv_heads=2, head_dim=64, capacity=300,
                               seq_lens=[0, 300, 0], dtype="f16"), {"force_splits": 3}
    plan, out, lse, ctr = _run_fused(w, **opts)
    assert torch.all(ctr == 0).item(), "counters must be back at zero"
    H.check_against_oracle(w, out, lse)


# The fused tail folds each row in batches of splits per lane (16 in the MFMA
# kernel, 8 in the VALU one) over one to four waves per row: split counts
# beyond one batch, every waves-per-row choice and both workspace forms.
FUSED_TAIL_CASES = [
    # (kernel, g, q_len, D, dtype, splits, ws_format)
    ("mfma", 8, 1, 128, "f16", 33, "uml"),      # 8 rows, two batches per lane group
    ("mfma", 8, 2, 128, "bf16", 65, "olse"),    # 16 rows (two column tiles), three batches
    ("mfma", 2, 1, 128, "f16", 70, "uml"),      # 2 rows: two waves per row
    ("mfma", 3, 1, 64, "bf16", 70, "olse"),     # 3 rows, D=64 (four lane groups per wave)
    ("mfma", 1, 2, 64, "f16", 129, "uml"),      # 2 rows of a query block, 129 splits
    ("valu", 1, 1, 128, "bf16", 70, "olse"),    # 1 row: four waves per row, batches of 8
    ("valu", 2, 1, 128, "f32", 37, "uml"),
    ("valu", 3, 1, 64, "f16", 50, "uml"),
]


@pytest.mark.parametrize("kernel,g,q_len,D,dtype,splits,ws_format", FUSED_TAIL_CASES)
def test_fused_tail_batches(kernel, g, q_len, D, dtype, splits, ws_format):
    lens = [splits * 64, 1, 0, splits * 40 + 3]        # full, one token, empty, trailing splits empty
    w = W.contiguous(f"fused_tail_{kernel}_g{g}_q{q_len}_S{splits}", seed=90 + splits, batch=len(lens),
                     q_heads=2 * g, kv_heads=2, head_dim=D, capacity=max(lens), seq_lens=lens, dtype=dtype,
                     q_len=q_len)
    plan, out, lse, ctr = _run_fused(w, kernel=kernel, force_splits=splits, ws_format=ws_format,
                                     host_seq_lens=None)
    assert plan.num_splits == splits and plan.kernel == fd.KERNELS[kernel]
    assert torch.all(ctr == 0).item(), "counters must be back at zero"
    H.check_against_oracle(w, out, lse)


def test_fused_repeated_calls_reset_counters():
    w1 = W.contiguous("fused_rep1", seed=84, batch=2, q_heads=16, kv_heads=2, head_dim=128, capacity=4000,
                      seq_lens=[4000, 2500], dtype="f16")
    w2 = W.contiguous("fused_rep2", seed=85, batch=2, q_heads=16, kv_heads=2, head_dim=128, capacity=4000,
                      seq_lens=[3333, 4000], dtype="f16")
    plan, out1, lse1, ctr = _run_fused(w1, force_splits=9)
    _, out2, lse2, ctr = _run_fused(w2, ctr=ctr, force_splits=9)
    _, out3, lse3, ctr = _run_fused(w1, ctr=ctr, force_splits=9)
    H.check_against_oracle(w1, out1, lse1)
    H.check_against_oracle(w2, out2, lse2)
    assert torch.equal(out1, out3) and torch.equal(lse1, lse3)


@pytest.mark.parametrize("case", ["mfma_uniform", "mfma_balanced_paged", "valu_olse"])
def test_fused_never_reads_stale_states(case):
    """The last workgroup of a group must read the states its group published
    in this call, never what the workspace held before. The workspace is first
    filled with states that would dominate any merge they entered (max 1e4,
    vectors 1e6), then left holding a previous call's states on other inputs;
    each fused call must still match the oracle."""
    if case == "mfma_uniform":
        mk = lambda i, lens: W.contiguous(f"stale_{case}_{i}", seed=400 + i, batch=2, q_heads=64, kv_heads=8,
                                          head_dim=128, capacity=12000, seq_lens=lens, dtype="f16")
        lens_seq, opts = ([12000, 9000], [7001, 12000], [12000, 12000]), {"force_splits": 32}
    elif case == "mfma_balanced_paged":
        mk = lambda i, lens: W.paged(f"stale_{case}_{i}", seed=410 + i, batch=5, q_heads=32, kv_heads=8,
                                     head_dim=128, seq_lens=lens, page_size=16, dtype="bf16")
        lens_seq = ([9000, 40, 3000, 0, 7000], [8000, 2999, 6000, 700, 1], [9000, 9000, 9000, 9000, 9000])
        opts = {"schedule": "balanced"}
    else:
        mk = lambda i, lens: W.contiguous(f"stale_{case}_{i}", seed=420 + i, batch=3, q_heads=8, kv_heads=8,
                                          head_dim=128, capacity=6000, seq_lens=lens, dtype="bf16")
        lens_seq, opts = ([6000, 5, 3000], [4000, 6000, 1]), {"force_splits": 12, "ws_format": "olse"}
    dev = torch.device("cuda", 0)
    ws = None
    for i, lens in enumerate(lens_seq):
        w = mk(i, lens)
        q, k, v, sl = w.q.to(dev), w.k.to(dev), w.v.to(dev), w.seq_lens.to(dev)
        bt = None if w.block_table is None else w.block_table.to(dev)
        o = dict(opts)
        if o.get("schedule") == "balanced":
            o["host_seq_lens"] = lens
        plan = fd.fd_plan(fd.problem_for(q, k, v, sl, bt, max_seq_len=w.max_seq_len), **o)
        if ws is None:                               # sized for the largest plan of the sequence
            big = max(plan.ws_o_bytes, 1 << 22) // 4 * 2
            ws = (torch.full((big,), 1e6, device=dev), torch.full((big // 64,), 1e4, device=dev),
                  torch.zeros(4096, dtype=torch.int32, device=dev))
        ws_o, ws_stats, ctr = ws
        assert ws_o.numel() * 4 >= plan.ws_o_bytes and ws_stats.numel() * 4 >= plan.ws_stats_bytes
        out = torch.empty(*q.shape, dtype=torch.float32, device=dev)
        lse = torch.empty(*q.shape[:-1], dtype=torch.float32, device=dev)
        H.say(f"stale {case} call {i}: S={plan.num_splits} schedule={plan.schedule}")
        fd.fd_decode_fused(plan, q, k, v, sl, ws_o, ws_stats, ctr, out, lse, bt)
        torch.cuda.synchronize()
        assert torch.all(ctr == 0).item()
        H.check_against_oracle(w, out.cpu(), lse.cpu())


def test_fused_agrees_with_two_launch_path():
    w = W.contiguous("fused_vs_split", seed=86, batch=1, q_heads=64, kv_heads=8, head_dim=128, capacity=20000,
                     seq_lens=[20000], dtype="f16")
    _, out_f, lse_f, _ = _run_fused(w)
    _, out_s, lse_s, _, _ = H.run(w)
    assert (out_f - out_s).abs().max().item() < 1e-5
    assert (lse_f - lse_s).abs().max().item() < 1e-5


@pytest.mark.parametrize("case", ["mfma", "valu", "qblock", "zero_rows"])
def test_fused_single_split_writes_rows_directly(case):
    """A fused call whose plan has one split writes out/lse from the split
    kernel's epilogue: the workspace is never touched (it stays NaN) and the
    counters stay zero."""
    if case == "mfma":
        w = W.contiguous("direct_mfma", seed=85, batch=3, q_heads=32, kv_heads=4, head_dim=128, capacity=900,
                         seq_lens=[900, 31, 400], dtype="bf16")
    elif case == "valu":
        w = W.contiguous("direct_valu", seed=86, batch=3, q_heads=4, kv_heads=4, head_dim=64, capacity=700,
                         seq_lens=[700, 1, 65], dtype="f32")
    elif case == "qblock":
        w = W.contiguous("direct_qblock", seed=87, batch=3, q_heads=8, kv_heads=4, head_dim=128, capacity=500,
                         seq_lens=[500, 2, 1], dtype="f16", q_len=3)
    else:
        w = W.contiguous("direct_zero", seed=88, batch=3, q_heads=16, kv_heads=2, head_dim=128, capacity=300,
                         seq_lens=[0, 300, 0], dtype="f16")
    dev = torch.device("cuda", 0)
    q, k, v, sl = w.q.to(dev), w.k.to(dev), w.v.to(dev), w.seq_lens.to(dev)
    plan = fd.fd_plan(fd.problem_for(q, k, v, sl), force_splits=1)
    assert plan.num_splits == 1
    ws_o, ws_stats = fd.workspace(plan, dev)
    ws_o.fill_(float("nan"))
    ws_stats.fill_(float("nan"))
    ctr = fd.counters(plan, dev)
    out = torch.empty(*q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(*q.shape[:-1], dtype=torch.float32, device=dev)
    fd.fd_decode_fused(plan, q, k, v, sl, ws_o, ws_stats, ctr, out, lse)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(ws_o)).item() and torch.all(torch.isnan(ws_stats)).item()
    assert torch.all(ctr == 0).item()
    H.check_against_oracle(w, out.cpu(), lse.cpu())


def test_read_probe_reads_every_byte():
    """The streaming-read probe's per-thread digests equal the XOR of the
    16-byte words each thread is assigned (so every byte was read)."""
    n16 = 70001                                   # not a multiple of the grid
    g = torch.Generator().manual_seed(99)
    host = torch.randint(0, 2**31 - 1, (n16, 4), generator=g, dtype=torch.int64).to(torch.int32)
    buf = host.to("cuda")
    sink = torch.zeros(fd.READ_PROBE_SINK_BYTES // 4, dtype=torch.int32, device="cuda")
    fd.fd_read_probe(buf, sink)
    torch.cuda.synchronize()
    words = host.numpy().view(np.uint32)
    grid, pt = fd.READ_PROBE_SINK_BYTES // (256 * 4), 256
    per = -(-n16 // grid)
    want = np.zeros(grid * pt, dtype=np.uint32)
    for w in range(grid):
        lo, hi = w * per, min(n16, w * per + per)
        for t in range(pt):
            idx = np.arange(lo + t, hi, pt)
            if idx.size:
                x = np.bitwise_xor.reduce(words[idx], axis=0)
                want[w * pt + t] = x[0] ^ x[1] ^ x[2] ^ x[3]
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
