"""Python binding of the split-KV decode-attention library ``libfd.so``.

Argument marshalling only: every step of the decode runs in the HIP kernels
behind the C ABI of ``include/fd.h``. The entry points keep the C names:

    plan = fd_plan(problem_for(q, k, v, seq_lens, ...), **options)
    ws_o, ws_stats = workspace(plan, device)
    fd_decode_split(plan, q, k, v, seq_lens, ws_o, ws_stats, block_table=None)
    fd_merge(plan, ws_o, ws_stats, out, lse)

``flash_decode`` chains the three for convenience. PyTorch provides device
memory and the stream (``torch.cuda.current_stream()``); nothing here computes.
If ``libfd.so`` is missing every entry point raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FD_LIB_PATH names another build of the library (a measurement variant built
# with decode_attention_fd_amd/build.py --waves N --out PATH).
LIB_PATH = os.environ.get("FD_LIB_PATH") or os.path.join(_HERE, "libfd.so")

FD_OK, FD_ERR_INVALID_ARG, FD_ERR_UNSUPPORTED, FD_ERR_ALIGNMENT, FD_ERR_WORKSPACE, FD_ERR_HIP, FD_ERR_BAD_PLAN = range(7)
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
LAYOUT_CONTIGUOUS, LAYOUT_PAGED = 0, 1
WS_FORMATS = {"uml": 0, "olse": 1}
KERNELS = {"auto": 0, "mfma": 1, "valu": 2}
HEURISTICS = {"mi355x": 0, "fa2": 1}
SCHEDULES = {"auto": 0, "uniform": 1, "balanced": 2}
PLAN_MAGIC = 0x46445031


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("q_stride_b", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("kv_stride_b", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64), ("kv_stride_t", ctypes.c_int64),
        ("kv_capacity", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("bt_stride_b", ctypes.c_int64),
        ("pool_stride_page", ctypes.c_int64), ("pool_stride_t", ctypes.c_int64), ("pool_stride_h", ctypes.c_int64),
        ("scale", ctypes.c_float), ("q_len", ctypes.c_int32), ("q_stride_q", ctypes.c_int64),
    ]


class PlanOpts(ctypes.Structure):
    _fields_ = [
        ("num_cus", ctypes.c_int32), ("wgs_per_cu", ctypes.c_int32), ("force_splits", ctypes.c_int32),
        ("force_chunk_tokens", ctypes.c_int32), ("ws_format", ctypes.c_int32), ("kernel", ctypes.c_int32),
        ("heuristic", ctypes.c_int32), ("max_splits", ctypes.c_int32), ("overhead_budget", ctypes.c_float),
        ("num_host_seq_lens", ctypes.c_int32), ("schedule", ctypes.c_int32), ("piece_cost_tokens", ctypes.c_int32),
        ("odd_xcd_permille", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3),
        ("host_seq_lens", ctypes.POINTER(ctypes.c_int32)),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32), ("num_splits", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
        ("kernel", ctypes.c_int32), ("ws_format", ctypes.c_int32), ("group", ctypes.c_int32),
        ("tile_tokens", ctypes.c_int32), ("waves_per_wg", ctypes.c_int32), ("slots", ctypes.c_int32),
        ("grid_x", ctypes.c_int32), ("grid_y", ctypes.c_int32), ("grid_z", ctypes.c_int32),
        ("scale", ctypes.c_float), ("schedule", ctypes.c_int32),
        ("piece_cost", ctypes.c_int32), ("odd_chunk_tokens", ctypes.c_int32),
        ("odd_range_permille", ctypes.c_int32), ("reserved3", ctypes.c_int32),
        ("ws_o_bytes", ctypes.c_int64), ("ws_stats_bytes", ctypes.c_int64), ("ws_counter_bytes", ctypes.c_int64),
        ("prob", Problem), ("checksum", ctypes.c_uint64),
    ]


class Args(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p)]


class FdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_str(status)} (status {status})"
        if status == FD_ERR_HIP:
            msg += f" [{lib().fd_last_hip_error().decode()}]"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded ``libfd.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def load(path: str) -> ctypes.CDLL:
    """Open a build of the library at ``path`` with the C signatures set (the
    race-check build is opened beside libfd.so this way); raises if missing or
    if its struct layouts differ from this binding's."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m decode_attention_fd_amd.build`")
    L = ctypes.CDLL(path)
    L.fd_plan.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(PlanOpts), ctypes.POINTER(Plan)]
    L.fd_plan.restype = ctypes.c_int
    L.fd_decode_split.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args), ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.fd_decode_split.restype = ctypes.c_int
    L.fd_decode_fused.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args), ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.fd_decode_fused.restype = ctypes.c_int
    L.fd_merge.argtypes = [ctypes.POINTER(Plan), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                           ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.fd_merge.restype = ctypes.c_int
    L.fd_decode_fused_noalloc.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args), ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    L.fd_decode_fused_noalloc.restype = ctypes.c_int
    L.fd_merge_states.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.fd_merge_states.restype = ctypes.c_int
    L.fd_wg_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.fd_wg_stamps.restype = ctypes.c_int
    L.fd_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                ctypes.c_void_p]
    L.fd_read_probe.restype = ctypes.c_int
    L.fd_status_str.argtypes = [ctypes.c_int]
    L.fd_status_str.restype = ctypes.c_char_p
    L.fd_last_hip_error.argtypes = []
    L.fd_last_hip_error.restype = ctypes.c_char_p
    L.fd_version.argtypes = []
    L.fd_version.restype = ctypes.c_char_p
    L.fd_struct_size.argtypes = [ctypes.c_int]
    L.fd_struct_size.restype = ctypes.c_size_t
    for i, cls in enumerate((Problem, PlanOpts, Plan, Args)):
        if L.fd_struct_size(i) != ctypes.sizeof(cls):
            raise RuntimeError(f"ABI mismatch for {cls.__name__}: C {L.fd_struct_size(i)} vs {ctypes.sizeof(cls)}")
    return L


def status_str(status: int) -> str:
    return lib().fd_status_str(status).decode()


def version() -> str:
    return lib().fd_version().decode()


def _check(status: int, where: str) -> None:
    if status != FD_OK:
        raise FdError(status, where)


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def problem_for(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                block_table: Optional[torch.Tensor] = None, max_seq_len: Optional[int] = None,
                scale: float = 0.0) -> Problem:
    """Describe a decode step from its tensors (shapes and strides only).

    q [B, Hq, D], or [B, q_len, Hq, D] for a short query block (row i of the
    block sees the first seq_len - (q_len - 1 - i) tokens); contiguous K/V
    [B, Hkv, T, D] or paged pools [P, page, Hkv, D] with ``block_table`` int32
    [B, max_pages]. ``max_seq_len`` defaults to ``seq_lens.max()`` (a device
    sync if seq_lens lives on the GPU)."""
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("K and V must have the same shape and strides")
    if k.dtype not in DTYPES or q.dtype not in DTYPES:
        raise ValueError(f"unsupported dtype {k.dtype}/{q.dtype}")
    p = Problem()
    if q.dim() == 4:
        p.batch, p.q_len, p.num_q_heads, p.head_dim = q.shape
        p.q_stride_b, p.q_stride_q, p.q_stride_h = q.stride(0), q.stride(1), q.stride(2)
    else:
        p.batch, p.num_q_heads, p.head_dim = q.shape
        p.q_stride_b, p.q_stride_h = q.stride(0), q.stride(1)
    p.q_dtype = DTYPES[q.dtype]
    p.kv_dtype = DTYPES[k.dtype]
    if q.stride(-1) != 1 or k.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if seq_lens.numel() else 0
    p.max_seq_len = int(max_seq_len)
    p.scale = float(scale)
    if block_table is None:
        p.layout = LAYOUT_CONTIGUOUS
        p.num_kv_heads = k.shape[1]
        p.kv_stride_b, p.kv_stride_h, p.kv_stride_t = k.stride(0), k.stride(1), k.stride(2)
        p.kv_capacity = k.shape[2]
    else:
        p.layout = LAYOUT_PAGED
        p.num_kv_heads = k.shape[2]
        p.num_pages, p.page_size = k.shape[0], k.shape[1]
        p.pool_stride_page, p.pool_stride_t, p.pool_stride_h = k.stride(0), k.stride(1), k.stride(2)
        p.max_pages_per_seq = block_table.shape[1]
        p.bt_stride_b = block_table.stride(0)
        if block_table.dtype != torch.int32 or block_table.stride(1) != 1:
            raise ValueError("block_table must be int32 with contiguous rows")
    return p


def fd_plan(problem: Problem, *, num_cus: int = 0, wgs_per_cu: int = 0, force_splits: int = 0,
            force_chunk_tokens: int = 0, ws_format: str = "uml", kernel: str = "auto",
            heuristic: str = "mi355x", max_splits: int = 0, overhead_budget: float = 0.0,
            host_seq_lens=None, schedule: str = "auto", piece_cost_tokens: int = 0,
            odd_xcd_permille: int = 0) -> Plan:
    """Call ``fd_plan``. ``num_cus=0`` asks the current device. ``host_seq_lens``
    (a host list / CPU tensor of the batch's lengths) enables length-aware
    splits and the balanced schedule."""
    o = PlanOpts()
    keep = None
    if host_seq_lens is not None:
        keep = (ctypes.c_int32 * len(host_seq_lens))(*[int(x) for x in host_seq_lens])
        o.num_host_seq_lens = len(host_seq_lens)
        o.host_seq_lens = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
    o.num_cus, o.wgs_per_cu = num_cus, wgs_per_cu
    o.force_splits, o.force_chunk_tokens = force_splits, force_chunk_tokens
    o.ws_format = WS_FORMATS[ws_format]
    o.kernel = KERNELS[kernel]
    o.heuristic = HEURISTICS[heuristic]
    o.max_splits = max_splits
    o.overhead_budget = overhead_budget
    o.schedule = SCHEDULES[schedule]
    o.piece_cost_tokens = piece_cost_tokens
    o.odd_xcd_permille = odd_xcd_permille
    plan = Plan()
    _check(lib().fd_plan(ctypes.byref(problem), ctypes.byref(o), ctypes.byref(plan)), "fd_plan")
    del keep
    return plan


def _rows(plan: Plan) -> int:
    pr = plan.prob
    return pr.batch * (pr.q_len if pr.q_len > 1 else 1) * pr.num_q_heads


def _device_of(tensors) -> torch.device:
    """The one GPU every given tensor lives on; raises otherwise (the kernels
    dereference every pointer on that device)."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one GPU, got {sorted(str(d) for d in devs)}")
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError(f"tensors must be GPU tensors, got {dev}")
    return dev


def _check_f32(t: torch.Tensor, name: str, numel: Optional[int] = None, at_least: bool = False) -> None:
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor")
    if numel is not None and (t.numel() < numel if at_least else t.numel() != numel):
        raise ValueError(f"{name} holds {t.numel()} elements, the plan needs {'at least ' if at_least else ''}{numel}")


def _check_inputs(plan: Plan, q, k, v, seq_lens, block_table) -> None:
    """The launch's tensors against the plan's problem: dtypes, shapes and
    strides as planned, seq_lens int32 with an entry per sequence, the block
    table present exactly for paged problems and wide enough."""
    pr = plan.prob
    dtype_of = {c: t for t, c in DTYPES.items()}
    if q.dtype != dtype_of.get(pr.q_dtype) or k.dtype != dtype_of.get(pr.kv_dtype) or v.dtype != k.dtype:
        raise ValueError("q/K/V dtypes differ from the plan's problem")
    if q.dim() == 4:
        ql = pr.q_len if pr.q_len > 1 else 1
        want_q = ((pr.batch, ql, pr.num_q_heads, pr.head_dim), (pr.q_stride_b, pr.q_stride_q, pr.q_stride_h))
        got_q = (tuple(q.shape), tuple(q.stride()[:3]))
    else:
        want_q = ((pr.batch, pr.num_q_heads, pr.head_dim), (pr.q_stride_b, pr.q_stride_h))
        got_q = (tuple(q.shape), tuple(q.stride()[:2]))
    if got_q != want_q or q.stride(-1) != 1:
        raise ValueError(f"q shape/strides {got_q} differ from the plan's {want_q}")
    if pr.layout == LAYOUT_PAGED:
        want_kv = ((pr.num_pages, pr.page_size, pr.num_kv_heads, pr.head_dim),
                   (pr.pool_stride_page, pr.pool_stride_t, pr.pool_stride_h, 1))
        if block_table is None:
            raise ValueError("a paged plan needs block_table")
        if (block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] < pr.batch
                or block_table.shape[1] < pr.max_pages_per_seq or block_table.stride(1) != 1
                or block_table.stride(0) != pr.bt_stride_b):
            raise ValueError("block_table must be int32 [>= B, >= max_pages_per_seq] with the planned row stride")
    else:
        want_kv = ((pr.batch, pr.num_kv_heads, pr.kv_capacity, pr.head_dim),
                   (pr.kv_stride_b, pr.kv_stride_h, pr.kv_stride_t, 1))
        if block_table is not None:
            raise ValueError("a contiguous plan takes no block_table")
    for name, t in (("K", k), ("V", v)):
        if (tuple(t.shape), tuple(t.stride())) != want_kv:
            raise ValueError(f"{name} shape/strides {(tuple(t.shape), tuple(t.stride()))} differ from the plan's {want_kv}")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or seq_lens.stride(0) != 1 or seq_lens.numel() < pr.batch:
        raise ValueError("seq_lens must be a contiguous int32 vector with one entry per sequence")
    _device_of([q, k, v, seq_lens, block_table])


def _check_outputs(plan: Plan, out, lse) -> None:
    rows = _rows(plan)
    _check_f32(out, "out", rows * plan.prob.head_dim)
    if lse is not None:
        _check_f32(lse, "lse", rows)


def workspace(plan: Plan, device) -> Tuple[torch.Tensor, torch.Tensor]:
    """Allocate the fp32 workspace the plan asks for: (ws_o [B,(q_len,)Hq,S,D], ws_stats)."""
    pr = plan.prob
    S, D = plan.num_splits, pr.head_dim
    rows = (pr.batch, pr.q_len, pr.num_q_heads) if pr.q_len > 1 else (pr.batch, pr.num_q_heads)
    ws_o = torch.empty(*rows, S, D, dtype=torch.float32, device=device)
    last = 2 if plan.ws_format == WS_FORMATS["uml"] else 1
    ws_stats = torch.empty(*rows, S, last, dtype=torch.float32, device=device)
    return ws_o, ws_stats


def fd_decode_split(plan: Plan, q, k, v, seq_lens, ws_o, ws_stats, block_table=None, stream=None) -> None:
    """Launch the split kernel on ``stream`` (default: torch's current stream)."""
    _check_inputs(plan, q, k, v, seq_lens, block_table)
    _device_of([q, ws_o, ws_stats])
    _check_f32(ws_o, "ws_o")
    _check_f32(ws_stats, "ws_stats")
    a = Args(_ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(block_table))
    st = lib().fd_decode_split(ctypes.byref(plan), ctypes.byref(a), _ptr(ws_o), ws_o.numel() * ws_o.element_size(),
                               _ptr(ws_stats), ws_stats.numel() * ws_stats.element_size(), _stream_handle(stream))
    _check(st, "fd_decode_split")


def counters(plan: Plan, device) -> torch.Tensor:
    """Zeroed arrival counters for fd_decode_fused (uint32 [B * Hkv]; kept zero by every call)."""
    return torch.zeros(plan.ws_counter_bytes // 4, dtype=torch.int32, device=device)


def fd_decode_fused(plan: Plan, q, k, v, seq_lens, ws_o, ws_stats, ctr, out, lse=None, block_table=None,
                    stream=None) -> None:
    """Split kernel with the merge fused in: writes out (and lse) in one launch."""
    _check_inputs(plan, q, k, v, seq_lens, block_table)
    _device_of([q, ws_o, ws_stats, ctr, out, lse])
    _check_f32(ws_o, "ws_o")
    _check_f32(ws_stats, "ws_stats")
    _check_outputs(plan, out, lse)
    if ctr.dtype not in (torch.int32, torch.uint32) or not ctr.is_contiguous():
        raise ValueError("counters must be a contiguous 32-bit integer tensor")
    a = Args(_ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(block_table))
    st = lib().fd_decode_fused(ctypes.byref(plan), ctypes.byref(a), _ptr(ws_o), ws_o.numel() * ws_o.element_size(),
                               _ptr(ws_stats), ws_stats.numel() * ws_stats.element_size(), _ptr(ctr),
                               ctr.numel() * ctr.element_size(), _ptr(out), _ptr(lse), _stream_handle(stream))
    _check(st, "fd_decode_fused")


NOALLOC_SCRATCH_BYTES = 32 << 20


def fd_decode_fused_noalloc(plan: Plan, q, k, v, seq_lens, out, lse=None, block_table=None, stream=None) -> None:
    """fd_decode_fused with the library's static device scratch as workspace and
    counters: nothing is allocated (for graph capture and allocation-free loops).
    Calls on one GPU share that scratch and must not overlap in time."""
    _check_inputs(plan, q, k, v, seq_lens, block_table)
    _check_outputs(plan, out, lse)
    _device_of([q, out, lse])
    a = Args(_ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(block_table))
    st = lib().fd_decode_fused_noalloc(ctypes.byref(plan), ctypes.byref(a), _ptr(out), _ptr(lse),
                                       _stream_handle(stream))
    _check(st, "fd_decode_fused_noalloc")


def fd_merge(plan: Plan, ws_o, ws_stats, out, lse=None, stream=None) -> None:
    """Launch the merge kernel: out [B,Hq,D] fp32 (contiguous), lse [B,Hq] fp32 or None."""
    _check_f32(ws_o, "ws_o")
    _check_f32(ws_stats, "ws_stats")
    _check_outputs(plan, out, lse)
    _device_of([ws_o, ws_stats, out, lse])
    st = lib().fd_merge(ctypes.byref(plan), _ptr(ws_o), ws_o.numel() * 4, _ptr(ws_stats), ws_stats.numel() * 4,
                        _ptr(out), _ptr(lse), _stream_handle(stream))
    _check(st, "fd_merge")


def fd_merge_states(states, stats, out=None, lse_out=None, *, ws_format: str = "olse", stream=None):
    """Merge external attention states per row (the library's merge operator on
    caller-built states). states float32 [..., S, D]; stats float32 [..., S]
    (olse: natural-log LSE) or [..., S, 2] (uml: m, l). Returns (out [..., D],
    lse_out [...]), allocating them when not given."""
    fmt = WS_FORMATS[ws_format]
    _device_of([states, stats, out, lse_out])
    if states.dtype != torch.float32 or stats.dtype != torch.float32:
        raise ValueError("states and stats must be float32")
    if not states.is_contiguous() or not stats.is_contiguous():
        raise ValueError("states and stats must be contiguous")
    *lead, S, D = states.shape
    want = (*lead, S, 2) if fmt == WS_FORMATS["uml"] else (*lead, S)
    if tuple(stats.shape) != tuple(want):
        raise ValueError(f"stats shape {tuple(stats.shape)} != {tuple(want)}")
    rows = 1
    for n in lead:
        rows *= n
    if out is None:
        out = torch.empty(*lead, D, dtype=torch.float32, device=states.device)
    if lse_out is None:
        lse_out = torch.empty(*lead, dtype=torch.float32, device=states.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != rows * D:
        raise ValueError("out must be a contiguous float32 tensor of rows x D")
    if lse_out.dtype != torch.float32 or not lse_out.is_contiguous() or lse_out.numel() != rows:
        raise ValueError("lse_out must be a contiguous float32 tensor of rows")
    st = lib().fd_merge_states(fmt, _ptr(states), _ptr(stats), rows, S, D, _ptr(out), _ptr(lse_out),
                               _stream_handle(stream))
    _check(st, "fd_merge_states")
    return out, lse_out


READ_PROBE_SINK_BYTES = 512 * 256 * 4
WG_STAMP_RECORDS = 65536


def fd_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Launch the streaming-read probe over ``buf`` (device, bytes a multiple of
    16); ``sink`` is an int32/uint32 device tensor of READ_PROBE_SINK_BYTES."""
    _device_of([buf, sink])
    if not buf.is_contiguous() or not sink.is_contiguous():
        raise ValueError("buf and sink must be contiguous")
    st = lib().fd_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                             sink.numel() * sink.element_size(), _stream_handle(stream))
    _check(st, "fd_read_probe")


# Output rows (B * q_len * Hq) from which a balanced plan is faster as one fused
# launch than as split + merge on MI355X. Twelve ragged batches (lengths
# U[1, hi], 32 or 64 query heads over 8 or 32 KV heads): at 256-2048 rows split +
# merge was 0.3-6 us faster (B=4 up to 64k tokens: 64.0 vs 70.1 us), at 4096 and
# 8192 rows the fused call was (B=128: 101.5 vs 102.9 us; B=256: 180-186 vs
# 189-194 us), where most segments are one piece written directly and a merge
# kernel over that many rows costs more than the merges done inside.
FUSED_MIN_ROWS = 4096


def prefers_fused(plan: Plan) -> bool:
    """Whether one fused launch is the faster path for this plan: one split
    (its rows are written directly), or a balanced plan of at least
    FUSED_MIN_ROWS output rows; otherwise split + merge."""
    rows = plan.prob.batch * max(1, plan.prob.q_len) * plan.prob.num_q_heads
    return plan.num_splits == 1 or (plan.schedule == SCHEDULES["balanced"] and rows >= FUSED_MIN_ROWS)


def flash_decode(q, k, v, seq_lens, block_table=None, *, max_seq_len=None, scale: float = 0.0,
                 return_lse: bool = True, fused: Optional[bool] = None, stream=None, **plan_options):
    """Plan, split and merge (two launches, or one with ``fused=True``; by
    default the faster of the two for the plan, ``prefers_fused``); returns
    (out, lse) fp32 (lse None if not asked)."""
    plan = fd_plan(problem_for(q, k, v, seq_lens, block_table, max_seq_len, scale), **plan_options)
    ws_o, ws_stats = workspace(plan, q.device)
    out = torch.empty(*q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(*q.shape[:-1], dtype=torch.float32, device=q.device) if return_lse else None
    if fused is None:
        fused = prefers_fused(plan)
    if fused:
        fd_decode_fused(plan, q, k, v, seq_lens, ws_o, ws_stats, counters(plan, q.device), out, lse, block_table,
                        stream)
    else:
        fd_decode_split(plan, q, k, v, seq_lens, ws_o, ws_stats, block_table, stream)
        fd_merge(plan, ws_o, ws_stats, out, lse, stream)
    return out, lse
