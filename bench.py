"""Decode-attention benchmark: one layer-step of split-KV decode on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--splits S]

A step is the whole hot path for one batch: fd_decode_split (split kernel)
then fd_merge (merge kernel), back to back on one stream, inputs already
resident in HBM (the plan is made once, outside the timed region). K/V live in
several seeded copies that the steps rotate through, together larger than
twice the 256 MB Infinity Cache, so no step is served from the previous one.

Prints ONE JSON line: value = achieved K/V bandwidth in TB/s (algorithmic
K+V bytes of the step / wall time per step), the microseconds per layer-step,
a roofline object for the split kernel (its average duration from two HIP
events on the launch stream around back-to-back launches of that kernel
alone) and the float64 CPU oracle timed on the host over a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MALL_BYTES = 256 << 20      # Infinity Cache

WORKLOADS = {
    # name: (builder kwargs, description)
    "gqa64x8_f16_L128000": "B=1, 64 query heads over 8 KV heads, D=128, L=128000, fp16, planner's split count",
    "mha32_bf16_L65536_C1024": "B=1, 32 = 32 heads, D=128, L=65536, bf16, 1024-token chunks, (o, LSE) workspace",
    "paged_gqa32x8_f16_B16": "B=16, 32 query heads over 8 KV heads, D=128, L ~ U[1024, 32768], fp16, 16-token pages",
    "edge_gqa32x8_f16_B64": "B=64, 32 query heads over 8 KV heads, D=128, L ~ U[1, 2048], fp16, K x 8",
    "tiny_mha_f32_L1000": "B=1, 4 = 4 heads, D=64, L=1000, fp32, 3 splits",
}


def make_workload(name: str, device):
    import fd_workloads as W

    builders = {
        "gqa64x8_f16_L128000": lambda: W.long_gqa_f16(device=device),
        "mha32_bf16_L65536_C1024": lambda: W.mha_bf16_chunked(device=device),
        "paged_gqa32x8_f16_B16": lambda: W.paged_ragged_f16(device=device),
        "edge_gqa32x8_f16_B64": lambda: W.edge_gqa_f16(device=device),
        "tiny_mha_f32_L1000": lambda: W.tiny_mha_f32(num_splits=3, device=device),
    }
    if name not in builders:
        raise SystemExit(f"unknown workload {name}; choose from {sorted(builders)}")
    return builders[name]()


def plan_options(w, splits: int = 0, schedule: str = "auto", wgs_per_cu: int = 0, kernel: str = "auto",
                 piece_cost: int = 0, odd_xcd_permille: int = 0) -> dict:
    """fd_plan options of a benchmark run: the workload's forced splits or
    chunk if it has them, else the planner fed the host copy of the lengths."""
    opts = {"ws_format": w.ws_format}
    if splits:
        opts["force_splits"] = splits
    elif w.num_splits:
        opts["force_splits"] = w.num_splits
    if w.chunk_tokens and not splits:
        opts["force_chunk_tokens"] = w.chunk_tokens
    if "force_splits" not in opts and "force_chunk_tokens" not in opts:
        opts["host_seq_lens"] = w.seq_lens.cpu().tolist()   # length-aware split plan
        opts["schedule"] = schedule
    if wgs_per_cu:
        opts["wgs_per_cu"] = wgs_per_cu
    if kernel != "auto":
        opts["kernel"] = kernel
    if piece_cost:
        opts["piece_cost_tokens"] = piece_cost
    if odd_xcd_permille:
        opts["odd_xcd_permille"] = odd_xcd_permille
    return opts


def choose_path(plan, path: str = "auto") -> str:
    """auto: the library's choice (decode_attention_fd_amd.prefers_fused): the
    fused call when the plan has one split or is balanced with at least 4096
    output rows, else split + merge."""
    import decode_attention_fd_amd as fd

    if path != "auto":
        return path
    return "fused" if fd.prefers_fused(plan) else "split"


def kernel_source_hash(kernel: str = "mfma") -> str:
    """Hash of the sources a split kernel ("mfma" or "valu") is compiled from
    (the kernel the roofline and the traffic record describe)."""
    h = hashlib.sha256()
    for rel in (f"decode_attention_fd_amd/csrc/split_{kernel}.hip", "decode_attention_fd_amd/csrc/balance.h",
                "decode_attention_fd_amd/csrc/merge_rows.h", "decode_attention_fd_amd/csrc/fd_internal.h",
                "decode_attention_fd_amd/csrc/geometry.h",
                "include/fd.h"):
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(rel.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, kernel_hash: str):
    """HBM bytes per split-kernel launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_split_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_hash:
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 256 << 20


def _pmc_rows(d: str, counter: str):
    """(kernel name, counter value) per dispatch from a rocprofv3 --pmc CSV directory."""
    import csv
    import glob

    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def pmc_summary(workload: str, fetch_dir: str, write_dir: str, out_path: str = "") -> None:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the split kernel, scaled by the
    same counters on the calibration copy (COPY_BYTES read and written). Writes
    profiles/traffic_split_<workload>.json (or out_path; "-": print only)."""
    names = [n for n, _ in _pmc_rows(fetch_dir, "FETCH_SIZE") if "split_" in n and "kernel" in n]
    kernel = "valu" if names and all("split_valu" in n for n in names) else "mfma"
    out = {"workload": workload, "kernel": kernel, "kernel_source_hash": kernel_source_hash(kernel),
           "copy_bytes": COPY_BYTES}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _pmc_rows(d, counter)
        split = [v for n, v in rows if "split_" in n and "kernel" in n]
        copy = [v for n, v in rows if "copyBuffer" in n]     # the runtime's device-to-device copy kernel
        if not split or not copy:
            raise SystemExit(f"{counter}: no split-kernel or copy dispatches in {d}")
        split_kib = sum(split) / len(split)
        copy_kib = max(copy)                     # the 256 MiB calibration copy is the largest one
        factor = COPY_BYTES / (copy_kib * 1024.0)
        out[key] = {"counter": counter, "split_kib_per_dispatch": split_kib, "split_dispatches": len(split),
                    "copy_kib_per_dispatch": copy_kib, "scale": factor,
                    "bytes_per_launch": split_kib * 1024.0 * factor}
    out["bytes_per_launch"] = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    path = out_path or os.path.join(ROOT, "profiles", f"traffic_split_{workload}.json")
    if path != "-":
        with open(path, "w") as f:
            json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def pmc_dump(dirs) -> None:
    """Average of every counter per kernel over the dispatches in rocprofv3
    --pmc CSV directories (one JSON line per directory and kernel), and the
    average duration per kernel from --kernel-trace directories."""
    import csv
    import glob

    for d in dirs:
        acc = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    k = (r["Kernel_Name"], r["Counter_Name"])
                    acc.setdefault(k, []).append(float(r["Counter_Value"]))
        for path in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    acc[(r["Name"], "average_ns")] = [float(r["AverageNs"])]
                    acc[(r["Name"], "calls")] = [float(r["Calls"])]
        kernels = sorted({k for k, _ in acc})
        for kern in kernels:
            row = {c: sum(v) / len(v) for (k, c), v in acc.items() if k == kern}
            row["dispatches"] = max(len(v) for (k, c), v in acc.items() if k == kern)
            print(json.dumps({"dir": d, "kernel": kern[:120], **row}))


def wg_stamp_report(plan, launch, launches: int, torch, fd, stream) -> dict:
    """Per-workgroup stamps of `launches` launches of the split kernel (the
    per-workgroup stamp build, loaded through FD_LIB_PATH): each workgroup's
    end and duration relative to the launch's first start, its tokens, pieces
    and XCD, summarised by piece count and by XCD."""
    import numpy as np

    nwg = plan.grid_x * plan.grid_y * plan.grid_z
    buf = torch.zeros(fd.WG_STAMP_RECORDS * 4, dtype=torch.int64, device=stream.device)
    recs = []
    for i in range(launches):
        launch(i)
        st = fd.lib().fd_wg_stamps(ctypes_void_p(buf.data_ptr()), buf.numel() * 8, ctypes_void_p(stream.cuda_stream))
        if st != 0:
            raise SystemExit(f"fd_wg_stamps: {fd.status_str(st)} (run with FD_LIB_PATH naming the --wg-stamps build)")
        torch.cuda.synchronize()
        r = buf[:4 * nwg].view(nwg, 4).cpu().numpy().astype(np.int64)
        t0 = r[:, 0].min()
        recs.append(np.stack([r[:, 0] - t0, r[:, 1] - t0, r[:, 2], r[:, 3] & 0xFFFFFFFF, (r[:, 3] >> 32) & 0xFF,
                              (r[:, 3] >> 40) & 0xFF], 1))
    a = np.stack(recs)                          # [launch, wg, (start, end, tokens, pieces, xcc, place)]; 10 ns ticks
    start_us, end_us = a[..., 0] / 100.0, a[..., 1] / 100.0
    dur_us = end_us - start_us
    tokens, pieces, xcc = a[..., 2], a[..., 3], a[..., 4]
    cu = xcc * 256 + a[..., 5]                  # one id per CU of the device
    q = lambda x: [round(float(v), 2) for v in np.percentile(x, [0, 10, 50, 90, 100])]
    out = {"workgroups": int(nwg), "launches": int(launches),
           "end_us_min_p10_p50_p90_max": q(end_us), "duration_us_min_p10_p50_p90_max": q(dur_us),
           "start_us_max": round(float(start_us.max()), 2),
           "tokens_per_wg_min_p50_max": [int(tokens.min()), int(np.median(tokens)), int(tokens.max())]}
    byp = {}
    for n in sorted(set(pieces.ravel().tolist())):
        m = pieces == n
        byp[int(n)] = {"workgroups_per_launch": round(float(m.sum()) / launches, 1),
                       "mean_end_us": round(float(end_us[m].mean()), 2),
                       "mean_tokens": round(float(tokens[m].mean()), 1),
                       "us_per_1k_tokens": round(float(dur_us[m].sum() / max(1, tokens[m].sum()) * 1e3), 3)}
    out["by_pieces"] = byp
    byx = {}
    for x in sorted(set(xcc.ravel().tolist())):
        m = xcc == x
        byx[int(x)] = {"mean_end_us": round(float(end_us[m].mean()), 2), "max_end_us": round(float(end_us[m].max()), 2),
                       "mean_tokens": round(float(tokens[m].mean()), 1)}
    out["by_xcd"] = byx
    # the launch's end against its busiest workgroups: a least-squares fit of duration on tokens and pieces
    A = np.stack([tokens.ravel() / 1000.0, pieces.ravel(), np.ones(tokens.size)], 1)
    coef, *_ = np.linalg.lstsq(A, dur_us.ravel(), rcond=None)
    pred = A @ coef
    resid = dur_us.ravel() - pred
    out["fit_duration_us"] = {"per_1k_tokens": round(float(coef[0]), 3), "per_piece": round(float(coef[1]), 3),
                              "constant": round(float(coef[2]), 3),
                              "r2": round(float(1 - resid.var() / max(dur_us.var(), 1e-12)), 3)}
    # per launch: how far the last workgroup ends past the mean end
    spread = [float(end_us[i].max() - end_us[i].mean()) for i in range(launches)]
    out["last_end_minus_mean_end_us"] = round(float(np.mean(spread)), 2)
    # workgroups go to XCDs round-robin by linear index? and the odd / even XCDs' mean end per launch
    lin = np.arange(nwg)
    out["xcd_is_index_mod_8"] = round(float(np.mean(xcc == (lin % 8)[None, :])), 4)
    odd = (xcc % 2) == 1
    out["per_launch_mean_end_us_even_odd"] = [[round(float(end_us[i][~odd[i]].mean()), 2),
                                               round(float(end_us[i][odd[i]].mean()), 2)] for i in range(launches)]
    out["per_launch_max_end_us_even_odd"] = [[round(float(end_us[i][~odd[i]].max()), 2),
                                              round(float(end_us[i][odd[i]].max()), 2)] for i in range(launches)]
    # Does a workgroup's lateness follow its range (the data it reads) or its
    # CU? Lateness = end minus the launch's mean end. Mean lateness per range
    # and per CU over the even launches against the odd launches: a Pearson r
    # near 1 means it repeats from launch to launch.
    late = end_us - end_us.mean(axis=1, keepdims=True)
    out["same_cu_as_first_launch"] = round(float(np.mean(cu == cu[:1])), 4)
    out["distinct_cus"] = int(len(set(cu.ravel().tolist())))

    def repeat(key):
        halves = []
        for sel in (slice(0, None, 2), slice(1, None, 2)):
            k, v = key[sel].ravel(), late[sel].ravel()
            sums, counts = {}, {}
            for kk, vv in zip(k.tolist(), v.tolist()):
                sums[kk] = sums.get(kk, 0.0) + vv
                counts[kk] = counts.get(kk, 0) + 1
            halves.append({kk: sums[kk] / counts[kk] for kk in sums})
        common = sorted(set(halves[0]) & set(halves[1]))
        x = np.array([halves[0][kk] for kk in common])
        y = np.array([halves[1][kk] for kk in common])
        r = float(np.corrcoef(x, y)[0, 1]) if len(common) > 2 and x.std() > 0 and y.std() > 0 else float("nan")
        return {"pearson_r_even_vs_odd_launches": round(r, 3), "keys": len(common),
                "lateness_sd_us": round(float(np.concatenate([x, y]).std()), 2)}

    out["lateness_repeats_by_range"] = repeat(np.broadcast_to(lin[None, :], end_us.shape))
    out["lateness_repeats_by_cu"] = repeat(cu)
    out["lateness_sd_us_within_launch"] = round(float(late.std()), 2)
    if launches >= 2 and nwg <= 4096:
        keys = sorted(set(cu.ravel().tolist()))
        out["mean_lateness_us_by_cu"] = {int(k): round(float(late[cu == k].mean()), 2) for k in keys}
        out["cu_of_workgroup_first_launch"] = [int(c) for c in cu[0]]
    return out


def trace_follow(trace_dir: str) -> None:
    """Durations of the kernels in a rocprofv3 kernel trace, keyed by the kernel
    that ran before each on the same queue: a kernel starts when the one
    before it ends, so its traced duration includes its own dispatch (what a
    dependent launch costs). Prints one JSON line."""
    import csv
    import glob

    import numpy as np

    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    rows = []
    for path in paths:
        with open(path) as f:
            rows += list(csv.DictReader(f))
    rows.sort(key=lambda r: (r["Queue_Id"], int(r["Start_Timestamp"])))

    def short(name):
        for key in ("split_mfma", "split_valu", "merge_kernel", "stream_read_kernel", "elementwise", "copyBuffer"):
            if key in name:
                return key
        return name[:40]

    pairs = {}
    for a, b in zip(rows, rows[1:]):
        if a["Queue_Id"] != b["Queue_Id"]:
            continue
        key = f"{short(b['Kernel_Name'])} after {short(a['Kernel_Name'])}"
        pairs.setdefault(key, []).append(((int(b["End_Timestamp"]) - int(b["Start_Timestamp"])) / 1e3,
                                          (int(b["Start_Timestamp"]) - int(a["End_Timestamp"])) / 1e3))
    out = {}
    for key, v in sorted(pairs.items()):
        a = np.array(v)
        out[key] = {"n": len(v), "us_p10_p50_p90": [round(float(x), 2) for x in np.percentile(a[:, 0], [10, 50, 90])],
                    "gap_us_p50": round(float(np.median(a[:, 1])), 2)}
    print(json.dumps(out), flush=True)


def ctypes_void_p(x):
    import ctypes

    return ctypes.c_void_p(x)


def cpu_baseline(w, max_heads: int):
    """Time the float64 oracle on the host over the first `max_heads` (b, hq)
    pairs of copy 0 and scale to the whole step; returns the JSON object."""
    import numpy as np
    import threadpoolctl
    import torch

    from oracle import attention as A

    cpu = w.to("cpu")
    cache = A.Cache(cpu.q, cpu.k, cpu.v, cpu.seq_lens, cpu.block_table)
    pairs = [(b, h) for b in range(cache.B) for h in range(cache.Hq)][:max_heads]
    A.attention_one(cache, *pairs[0])                       # warm the allocator
    # passes over the sample until about 10 s of CPU work (at most 8 passes or
    # 30 s); the median pass is the sample's time
    passes = []
    while True:
        t0 = time.perf_counter()
        res = [A.attention_one(cache, b, h) for b, h in pairs]
        passes.append(time.perf_counter() - t0)
        if len(passes) == 1:
            out = res
        if sum(passes) >= 10.0 or len(passes) >= 8 or sum(passes) + passes[-1] > 30.0:
            break
    dt = sorted(passes)[len(passes) // 2]
    # KV bytes the sampled heads stand for, out of the step's total
    lens = cpu.seq_lens.to(torch.int64).tolist()
    per_head_bytes = [lens[b] * 2 * cache.D * cpu.k.element_size() for b, _ in pairs]
    sampled_fraction = sum(per_head_bytes) / (sum(lens) * cache.Hq * 2 * cache.D * cpu.k.element_size())
    step_s = dt / max(sampled_fraction, 1e-12)
    kv_bytes = w.kv_bytes()
    # host CPUs this process may run on, and the threads the oracle's NumPy/BLAS
    # calls actually use (capped by the environment's thread limits)
    cpus = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [torch.get_num_threads()])
    return {
        "value": kv_bytes / step_s / 1e12, "unit": "TB/s", "us_per_step": step_s * 1e6,
        "cores": min(cpus, threads), "host_cpus": cpus, "os_cpu_count": os.cpu_count(), "kind": "oracle",
        "sample": f"{len(pairs)} of {cache.B * cache.Hq} (sequence, query head) outputs of copy 0 in float64, "
                  f"{len(passes)} passes in {sum(passes):.1f} s (median pass {dt:.2f} s), scaled by their share of "
                  f"the step's KV bytes ({sampled_fraction:.3f})",
    }, out, pairs


SWEEP_BATCHES = (1, 4, 16, 64)
SWEEP_CONTEXTS = (1024, 4096, 16384, 65536, 131072)
SWEEP_MAX_TOKENS = 1 << 20          # B x L per point (4 GiB of fp16 K/V at 8 KV heads, D = 128)


def sweep_speedup(q_heads: int = 64, kv_heads: int = 8, min_ms: float = 20.0) -> None:
    """Speedup of split-KV decode over one split per (sequence, KV head), the
    performance check of the kanthi.in chapter's section 8 ("speedup vs
    num_splits = 1 across a (batch, context) sweep"): for every (B, L) with
    B x L <= SWEEP_MAX_TOKENS, GQA q_heads/kv_heads, D = 128, fp16, equal
    lengths L, the step of the planner's plan (split + merge, or the fused call
    where bench.choose_path takes it) against force_splits = 1 (the fused call,
    which then writes its rows directly, one launch). K/V copies rotate so
    that together they exceed twice the 256 MB Infinity Cache; each plan is
    timed by wall clock over enough steps for min_ms (eager launches through
    the binding: small steps then measure the host's launch rate) and by
    events around the replay of a HIP graph holding the same steps (device
    time alone; the graph has no memset node, the fused counters return to
    zero inside the kernels). One JSON line per point."""
    import torch

    import decode_attention_fd_amd as fd
    import fd_workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    for B in SWEEP_BATCHES:
        for L in SWEEP_CONTEXTS:
            if B * L > SWEEP_MAX_TOKENS:
                continue
            w0 = W.contiguous(f"sweep_B{B}_L{L}", seed=B * 1000003 + L, batch=B, q_heads=q_heads, kv_heads=kv_heads,
                              head_dim=128, capacity=L, seq_lens=[L] * B, dtype="f16", device=dev)
            kv = w0.kv_bytes()
            copies = min(128, max(2, math.ceil(2 * MALL_BYTES / kv) + 1))
            ws = [w0] + [W.redraw_kv(w0, 9000 + i) for i in range(1, copies)]
            prob = fd.problem_for(w0.q, w0.k, w0.v, w0.seq_lens, max_seq_len=L)
            row = {"batch": B, "context": L, "q_heads": q_heads, "kv_heads": kv_heads, "kv_bytes": kv,
                   "kv_copies": copies}
            for tag, opts in (("plan", {"host_seq_lens": [L] * B}), ("one_split", {"force_splits": 1})):
                plan = fd.fd_plan(prob, **opts)
                path = choose_path(plan) if tag == "plan" else "fused"
                ws_o, ws_stats = fd.workspace(plan, dev)
                ctr = fd.counters(plan, dev)
                out = torch.empty(B, q_heads, 128, dtype=torch.float32, device=dev)
                lse = torch.empty(B, q_heads, dtype=torch.float32, device=dev)

                def step(i):
                    w = ws[i % copies]
                    if path == "fused":
                        fd.fd_decode_fused(plan, w.q, w.k, w.v, w.seq_lens, ws_o, ws_stats, ctr, out, lse, None,
                                           stream)
                    else:
                        fd.fd_decode_split(plan, w.q, w.k, w.v, w.seq_lens, ws_o, ws_stats, None, stream)
                        fd.fd_merge(plan, ws_o, ws_stats, out, lse, stream)

                for i in range(3):
                    step(i)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                step(0)
                torch.cuda.synchronize()
                once = time.perf_counter() - t0
                n = int(min(400, max(5, min_ms * 1e-3 / max(once, 1e-6))))
                t0 = time.perf_counter()
                for i in range(n):
                    step(i)
                torch.cuda.synchronize()
                us = (time.perf_counter() - t0) / n * 1e6
                # the same steps from a HIP graph
                ng = min(n, 64)
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.stream(side):
                    with torch.cuda.graph(graph, stream=side):
                        stream = torch.cuda.current_stream()
                        for i in range(ng):
                            step(i)
                stream = torch.cuda.current_stream()
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = max(1, n // ng)
                e0.record(stream)
                for _ in range(reps):
                    graph.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                gus = e0.elapsed_time(e1) * 1e3 / (reps * ng)
                del graph
                row[tag] = {"us": round(us, 2), "tbps": round(kv / (us * 1e-6) / 1e12, 3), "graph_us": round(gus, 2),
                            "graph_tbps": round(kv / (gus * 1e-6) / 1e12, 3), "num_splits": plan.num_splits,
                            "schedule": {1: "uniform", 2: "balanced"}[plan.schedule], "path": path, "steps": n}
            row["speedup"] = round(row["one_split"]["us"] / row["plan"]["us"], 2)
            row["graph_speedup"] = round(row["one_split"]["graph_us"] / row["plan"]["graph_us"], 2)
            print(json.dumps(row), flush=True)
            del ws, w0


def build_parser() -> argparse.ArgumentParser:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa64x8_f16_L128000", choices=sorted(WORKLOADS))
    ap.add_argument("--splits", type=int, default=0, help="force the split count (0 = planner)")
    ap.add_argument("--copies", type=int, default=0, help="K/V copies to rotate (0 = enough for 2x the MALL)")
    ap.add_argument("--cpu-heads", type=int, default=64, help="(b, head) outputs the CPU oracle times")
    ap.add_argument("--path", choices=["auto", "fused", "split"], default="auto",
                    help="fused: one launch (last workgroup per group merges); split: split + merge kernels; "
                         "auto: fused when the plan has one split or is balanced, else split")
    ap.add_argument("--schedule", choices=["auto", "uniform", "balanced"], default="auto",
                    help="split schedule (auto: balanced when the planner gets the host lengths and can use it)")
    ap.add_argument("--wgs-per-cu", type=int, default=0, help="planner slots per CU (0 = library default)")
    ap.add_argument("--kernel", choices=["auto", "mfma", "valu"], default="auto", help="split kernel (auto: planner)")
    ap.add_argument("--piece-cost", type=int, default=0,
                    help="balanced schedule: start-up cost of one piece in KV tokens (0 = library default, -1 = none)")
    ap.add_argument("--odd-xcd-permille", type=int, default=0,
                    help="uniform plans: tokens shifted from odd-XCD to even-XCD splits, per mille "
                         "(0 = library default, -1 = equal splits)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain 256 MiB device copy (known bytes) to scale PMC counters")
    ap.add_argument("--sweep-speedup", action="store_true",
                    help="time the planner's plan against one split per (sequence, KV head) over a (batch, context) "
                         "sweep of 64/8 GQA fp16 steps; one JSON line per point, then exit")
    ap.add_argument("--wg-stamps", type=int, default=0, metavar="LAUNCHES",
                    help="with FD_LIB_PATH naming the per-workgroup stamp build (build.py --wg-stamps): run the "
                         "workload's split (or fused) kernel LAUNCHES times, print a summary of the workgroups' "
                         "start/end stamps, tokens, pieces and XCDs as JSON, and exit")
    ap.add_argument("--pmc-dump", nargs="+", metavar="DIR",
                    help="print per-kernel counter averages (and kernel-trace durations) of rocprofv3 CSV "
                         "directories, one JSON line per directory and kernel, and exit")
    ap.add_argument("--launch-floor", type=int, default=0, metavar="ROUNDS",
                    help="after each split kernel launch, in turn, the merge kernel, two 64-float fills and the "
                         "read probe over 1 MiB, ROUNDS times each (run under rocprofv3 --kernel-trace; read the "
                         "trace with --trace-follow)")
    ap.add_argument("--trace-follow", metavar="DIR",
                    help="durations of the kernels in a rocprofv3 kernel trace, by the kernel before each")
    ap.add_argument("--pmc-out", default="",
                    help="--pmc-summary: where to write the record (default profiles/traffic_split_<workload>.json; "
                         "'-': print only)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench into "
                         "profiles/traffic_split_<workload>.json and exit")
    return ap


def main():
    args = build_parser().parse_args()
    if args.pmc_dump:
        pmc_dump(args.pmc_dump)
        return
    if args.pmc_summary:
        pmc_summary(args.workload, *args.pmc_summary, out_path=args.pmc_out)
        return
    if args.trace_follow:
        trace_follow(args.trace_follow)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs the decode on a single device "
              "(sharding across GPUs is a design note, not built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.sweep_speedup:
        sweep_speedup()
        return

    import torch

    import decode_attention_fd_amd as fd

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] workload {args.workload}: {WORKLOADS[args.workload]}", file=sys.stderr, flush=True)

    w0 = make_workload(args.workload, dev)
    step_kv = w0.kv_bytes()
    alloc = w0.k.numel() * w0.k.element_size() * 2
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / step_kv) + 1)
    import fd_workloads as W

    ws = [w0] + [W.redraw_kv(w0, 7000 + i) for i in range(1, copies)]
    torch.cuda.synchronize()

    opts = plan_options(w0, args.splits, args.schedule, args.wgs_per_cu, args.kernel, args.piece_cost,
                        args.odd_xcd_permille)
    prob = fd.problem_for(w0.q, w0.k, w0.v, w0.seq_lens, w0.block_table, max_seq_len=w0.max_seq_len)
    t0 = time.perf_counter()
    plan = fd.fd_plan(prob, **opts)
    plan_first_us = (time.perf_counter() - t0) * 1e6   # includes the one-time device and occupancy query
    plan_times = []
    for _ in range(200):                               # a serving loop plans again every step
        t0 = time.perf_counter()
        fd.fd_plan(prob, **opts)
        plan_times.append((time.perf_counter() - t0) * 1e6)
    plan_us = statistics.median(plan_times)
    ws_o, ws_stats = fd.workspace(plan, dev)
    ctr = fd.counters(plan, dev)
    out = torch.empty(w0.batch, w0.num_q_heads, w0.head_dim, dtype=torch.float32, device=dev)
    lse = torch.empty(w0.batch, w0.num_q_heads, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    path = choose_path(plan, args.path)

    def step(i, evs=None):
        w = ws[i % copies]
        if evs is not None:
            evs[0].record(stream)
        if path == "fused":
            fd.fd_decode_fused(plan, w.q, w.k, w.v, w.seq_lens, ws_o, ws_stats, ctr, out, lse, w.block_table, stream)
            if evs is not None:
                evs[1].record(stream)
        else:
            fd.fd_decode_split(plan, w.q, w.k, w.v, w.seq_lens, ws_o, ws_stats, w.block_table, stream)
            if evs is not None:
                evs[1].record(stream)
            fd.fd_merge(plan, ws_o, ws_stats, out, lse, stream)
        if evs is not None:
            evs[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    if args.launch_floor:
        # after each split kernel, in turn: the merge kernel; two trivial fills
        # of 64 floats; the read probe over 1 MiB (about the merge's input)
        small = torch.empty(64, device=dev)
        pbuf = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        sink = torch.empty(fd.READ_PROBE_SINK_BYTES // 4, dtype=torch.int32, device=dev)
        for i in range(3 * args.launch_floor):
            w = ws[i % copies]
            fd.fd_decode_split(plan, w.q, w.k, w.v, w.seq_lens, ws_o, ws_stats, w.block_table, stream)
            if i % 3 == 0:
                fd.fd_merge(plan, ws_o, ws_stats, out, lse, stream)
            elif i % 3 == 1:
                small.zero_()
                small.zero_()
            else:
                fd.fd_read_probe(pbuf, sink, stream)
        torch.cuda.synchronize()
        print(json.dumps({"launch_floor_rounds": args.launch_floor, "workload": args.workload}), flush=True)
        return

    if args.wg_stamps:
        def launch(i):
            w = ws[i % copies]
            if path == "fused":
                fd.fd_decode_fused(plan, w.q, w.k, w.v, w.seq_lens, ws_o, ws_stats, ctr, out, lse, w.block_table,
                                   stream)
            else:
                fd.fd_decode_split(plan, w.q, w.k, w.v, w.seq_lens, ws_o, ws_stats, w.block_table, stream)

        rep = wg_stamp_report(plan, launch, args.wg_stamps, torch, fd, stream)
        rep.update({"workload": args.workload, "path": path, "num_splits": plan.num_splits,
                    "schedule": {1: "uniform", 2: "balanced"}[plan.schedule], "lib": fd.LIB_PATH})
        print(json.dumps(rep), flush=True)
        return

    # timed region: exactly K steps, wall clock between synchronisations
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us_step = wall / args.steps * 1e6

    # Per-kernel durations, each kernel alone: two events on the launch stream
    # bracket K back-to-back launches (rotating the same K/V copies), so the
    # average is the kernel's own duration without per-launch event overhead
    # (the basis of roofline.achieved; it is what a rocprofv3 kernel trace of
    # the same command averages).
    def bracket(launch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(min(args.warmup, 5)):
            launch(i)
        e0.record(stream)
        for i in range(args.steps):
            launch(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    def split_only(i):
        w = ws[i % copies]
        if path == "fused":
            fd.fd_decode_fused(plan, w.q, w.k, w.v, w.seq_lens, ws_o, ws_stats, ctr, out, lse, w.block_table, stream)
        else:
            fd.fd_decode_split(plan, w.q, w.k, w.v, w.seq_lens, ws_o, ws_stats, w.block_table, stream)

    split_us = bracket(split_only)

    # the step's distribution and per-launch event durations (events between the
    # kernels of every step; these include the events' own overhead). The merge
    # kernel is timed this way: a few microseconds long, back-to-back launches
    # of it would measure the host's launch rate instead.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    split_ev_us = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs) * 1e3
    merge_us = 0.0 if path == "fused" else sum(e[1].elapsed_time(e[2]) for e in evs) / len(evs) * 1e3
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)

    def pct(xs, q):
        return round(xs[min(len(xs) - 1, int(q * (len(xs) - 1) + 0.5))] * 1e3, 2)

    # same-run streaming-read probe: two 512 MiB buffers in turn (each twice the MALL)
    probe_bytes = 512 << 20
    pbufs = [torch.empty(probe_bytes, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(2)]
    sink = torch.empty(fd.READ_PROBE_SINK_BYTES // 4, dtype=torch.int32, device=dev)
    for i in range(4):
        fd.fd_read_probe(pbufs[i % 2], sink, stream)
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    probe_iters = 20
    pe[0].record(stream)
    for i in range(probe_iters):
        fd.fd_read_probe(pbufs[i % 2], sink, stream)
    pe[1].record(stream)
    torch.cuda.synchronize()
    probe_us = pe[0].elapsed_time(pe[1]) * 1e3 / probe_iters
    probe_gbps = probe_bytes / (probe_us * 1e-6) / 1e9
    del pbufs

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # every byte a step moves, beside the K/V bytes the metric counts
    if w0.paged:
        page = w0.k.shape[1]
        bt_bytes = sum(-(-int(n) // page) for n in w0.seq_lens.tolist()) * 4
    else:
        bt_bytes = 0
    moved = {
        "kv": step_kv,
        "q": w0.q.numel() * w0.q.element_size(),
        "out_lse": (out.numel() + lse.numel()) * 4,
        "workspace_rw": 2 * (plan.ws_o_bytes + plan.ws_stats_bytes),   # written by the split, read by the merge
        "block_table": bt_bytes,
        "seq_lens": w0.seq_lens.numel() * 4,
    }
    moved["total"] = sum(moved.values())
    tbps = step_kv / (us_step * 1e-6) / 1e12
    achieved = step_kv / (split_us * 1e-6) / 1e9
    khash = kernel_source_hash({1: "mfma", 2: "valu"}[plan.kernel])
    traffic = traffic_from_profile(args.workload, khash)
    result = {
        "metric": "decode-attention µs/layer-step and achieved HBM TB/s (% of peak), B=1 L=128k GQA",
        "value": round(tbps, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 5),
        "us_per_layer_step": round(us_step, 2),
        "pct_of_peak": round(100 * tbps * 1e3 / PEAK_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}[w0.k.dtype],
        "data": "synthetic: seeded N(0,1) q/K/V",
        "config": {
            "workload": args.workload, "batch": w0.batch, "q_heads": w0.num_q_heads, "kv_heads": w0.num_kv_heads,
            "head_dim": w0.head_dim, "max_seq_len": w0.max_seq_len, "kv_bytes_per_step": step_kv,
            "kv_bytes_allocated": alloc, "kv_copies": copies, "layout": "paged" if w0.paged else "contiguous",
            "num_splits": plan.num_splits, "chunk_tokens": plan.chunk_tokens,
            "odd_chunk_tokens": plan.odd_chunk_tokens,
            "odd_range_permille": plan.odd_range_permille,
            "kernel": {1: "mfma", 2: "valu"}[plan.kernel], "ws_format": {0: "uml", 1: "olse"}[plan.ws_format],
            "slots": plan.slots, "plan_us": round(plan_us, 1), "plan_first_us": round(plan_first_us, 1), "path": path,
            "schedule": {1: "uniform", 2: "balanced"}[plan.schedule], "grid": plan.grid_x * plan.grid_y * plan.grid_z,
        },
        "step_event_us": {"p10": pct(step_ms, 0.1), "p50": pct(step_ms, 0.5), "p90": pct(step_ms, 0.9)},
        "split_kernel_us": round(split_us, 2),
        "merge_kernel_event_us": round(merge_us, 2),
        "split_kernel_event_us": round(split_ev_us, 2),
        "merge_share": round(merge_us / max(split_us + merge_us, 1e-9), 4),
        "bytes_per_step": moved,
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
            "kernel": "fused split" if path == "fused" else "split", "bytes_per_launch": step_kv,
            "kernel_source_hash": khash,
            "basis": f"HIP events on the launch stream around {args.steps} back-to-back launches of the kernel alone",
        },
        "read_probe": {"value": round(probe_gbps, 1), "unit": "GB/s", "bytes": probe_bytes,
                       "us": round(probe_us, 2), "split_kernel_frac_of_probe": round(achieved / probe_gbps, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the float64 oracle on the host", file=sys.stderr, flush=True)
        cb, ref, pairs = cpu_baseline(w0, args.cpu_heads)
        # the GPU output of copy 0 on the sampled pairs, against the oracle (sanity)
        step(0)
        torch.cuda.synchronize()
        import numpy as np

        o = out.cpu().double().numpy()
        err = max(float(np.abs(o[b, h] - r[0]).max()) for (b, h), r in zip(pairs, ref))
        cb["gpu_max_abs_err_on_sample"] = err
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
