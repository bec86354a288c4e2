"""GPU parity for caller layouts other than the generators' defaults: the
ABI takes element strides, so token-major caches, padded rows, strided q and
padded paged pools must all give the oracle's result."""
import pytest
import torch

import decode_attention_fd_amd as fd
import fd_workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _randn(shape, seed, dtype):
    """Seeded N(0, 1) drawn on the host and moved whole to the device, so the
    views taken afterwards keep their strides there."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype).to("cuda")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("g", [1, 4])
def test_token_major_contiguous_cache(dtype, g):
    """K/V stored [B, T, Hkv, D] (token-major) and handed over as the
    [B, Hkv, T, D] view: kv_stride_t = Hkv * D, kv_stride_h = D."""
    B, Hkv, T, D = 3, 4, 1500, 128
    k = _randn((B, T, Hkv, D), 1, dtype).permute(0, 2, 1, 3)
    v = _randn((B, T, Hkv, D), 2, dtype).permute(0, 2, 1, 3)
    q = _randn((B, Hkv * g, D), 3, dtype)
    w = W.Workload("token_major", q, k, v, torch.tensor([1500, 77, 1024], dtype=torch.int32))
    assert k.stride(2) == Hkv * D and k.stride(1) == D
    for splits in (1, 5):
        plan, out, lse, _, _ = H.run(w, force_splits=splits)
        H.check_against_oracle(w, out, lse)


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_padded_rows_and_strided_q(kernel):
    """Rows of K/V padded to 192 elements, q rows padded to 256 elements."""
    B, Hkv, g, T, D = 2, 2, 2, 900, 128
    kf = _randn((B, Hkv, T, 192), 4, torch.float16)
    vf = _randn((B, Hkv, T, 192), 5, torch.float16)
    qf = _randn((B, Hkv * g, 256), 6, torch.float16)
    w = W.Workload("padded", qf[..., :D], kf[..., :D], vf[..., :D], torch.tensor([900, 333], dtype=torch.int32))
    assert w.k.stride(2) == 192 and w.q.stride(1) == 256
    plan, out, lse, _, _ = H.run(w, kernel=kernel, force_splits=3)
    assert plan.kernel == fd.KERNELS[kernel]
    H.check_against_oracle(w, out, lse)


def test_paged_pool_with_padded_heads():
    """A paged pool whose head slices are padded (pool_stride_h = D + 64)."""
    base = W.paged("padded_pool", seed=7, batch=3, q_heads=16, kv_heads=4, head_dim=128,
                   seq_lens=[700, 20, 1300], page_size=32, dtype="f16", pool_layout="nhd")
    P, page, Hkv, D = base.k.shape
    kf = torch.zeros(P, page, Hkv, D + 64, dtype=base.k.dtype)
    vf = torch.zeros(P, page, Hkv, D + 64, dtype=base.v.dtype)
    kf[..., :D] = base.k
    vf[..., :D] = base.v
    kf, vf = kf.to("cuda"), vf.to("cuda")
    w = W.Workload("padded_pool", base.q.to("cuda"), kf[..., :D], vf[..., :D], base.seq_lens,
                   base.block_table.to("cuda"), page_size=page)
    assert w.k.stride(2) == D + 64
    for opts in ({"force_splits": 2}, {"host_seq_lens": base.seq_lens.tolist(), "schedule": "balanced"}):
        plan, out, lse, _, _ = H.run(w, **opts)
        H.check_against_oracle(w, out, lse)
