"""The boundary from plain C (no GPU): a C99 program that includes only
include/fd.h, links libfd.so and plans the 128k-token GQA step, an invalid
problem and a balanced ragged batch. Its output must equal what the Python
binding gets from the same calls, and the struct sizes it sees must equal the
library's own."""
import ctypes
import os
import shutil
import subprocess

import pytest
import torch

import decode_attention_fd_amd as fd
from tests.conftest import ROOT

PROGRAM = r"""
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fd.h"

static void contiguous(fd_problem* p, int B, int hq, int hkv, int D, int T) {
  memset(p, 0, sizeof *p);
  p->batch = B;
  p->num_q_heads = hq;
  p->num_kv_heads = hkv;
  p->head_dim = D;
  p->q_dtype = FD_DTYPE_F16;
  p->kv_dtype = FD_DTYPE_F16;
  p->layout = FD_LAYOUT_CONTIGUOUS;
  p->max_seq_len = T;
  p->q_stride_b = (int64_t)hq * D;
  p->q_stride_h = D;
  p->kv_stride_b = (int64_t)hkv * T * D;
  p->kv_stride_h = (int64_t)T * D;
  p->kv_stride_t = D;
  p->kv_capacity = T;
}

static void show(const char* tag, int st, const fd_plan_t* pl) {
  if (st != FD_OK) {
    printf("%s status %d %s\n", tag, st, fd_status_str(st));
    return;
  }
  printf("%s status 0 S %d chunk %d/%d kernel %d schedule %d grid %d %d %d odd %d ws %lld %lld\n", tag,
         pl->num_splits, pl->chunk_tokens, pl->odd_chunk_tokens, pl->kernel, pl->schedule, pl->grid_x, pl->grid_y,
         pl->grid_z, pl->odd_range_permille, (long long)pl->ws_o_bytes, (long long)pl->ws_stats_bytes);
}

int main(void) {
  fd_problem p;
  fd_plan_opts o;
  fd_plan_t pl;
  int32_t lens[6] = {3000, 17, 0, 2200, 5000, 900};
  int32_t long_lens[8] = {40000, 30000, 35000, 20000, 38000, 25000, 39000, 31000};

  printf("version %s\n", fd_version());
  printf("sizes %zu %zu %zu %zu\n", sizeof(fd_problem), sizeof(fd_plan_opts), sizeof(fd_plan_t), sizeof(fd_args));

  contiguous(&p, 1, 64, 8, 128, 128000);
  memset(&o, 0, sizeof o);
  o.num_cus = 256;
  show("gqa", fd_plan(&p, &o, &pl), &pl);

  contiguous(&p, 1, 64, 7, 128, 1000);     /* 64 query heads do not share 7 KV heads evenly */
  show("bad", fd_plan(&p, &o, &pl), &pl);

  contiguous(&p, 6, 32, 8, 128, 5000);
  o.schedule = FD_SCHEDULE_BALANCED;
  o.host_seq_lens = lens;
  o.num_host_seq_lens = 6;
  show("balanced", fd_plan(&p, &o, &pl), &pl);

  /* over 4096 K/V rows per range on 256 CUs: ranges of alternating size */
  contiguous(&p, 8, 32, 8, 128, 40000);
  o.host_seq_lens = long_lens;
  o.num_host_seq_lens = 8;
  show("balanced_long", fd_plan(&p, &o, &pl), &pl);
  o.odd_xcd_permille = -1;
  show("balanced_long_equal", fd_plan(&p, &o, &pl), &pl);

  /* a workspace one float short of the plan's: refused before any launch */
  contiguous(&p, 1, 64, 8, 128, 128000);
  memset(&o, 0, sizeof o);
  o.num_cus = 256;
  fd_plan(&p, &o, &pl);
  {
    int st = fd_merge(&pl, (const float*)(uintptr_t)4096, (size_t)pl.ws_o_bytes - 4,
                      (const float*)(uintptr_t)8192, (size_t)pl.ws_stats_bytes, (float*)(uintptr_t)4096, NULL, NULL);
    printf("merge_short status %d %s\n", st, fd_status_str(st));
  }

  /* split boundaries past 2^31 - 1 tokens */
  contiguous(&p, 1, 8, 8, 128, 1000);
  o.force_splits = 65535;
  o.force_chunk_tokens = 65536;
  show("overflow", fd_plan(&p, &o, &pl), &pl);
  return 0;
}
"""


def _python_side() -> list:
    def contiguous(B, hq, hkv, D, T):
        p = fd.Problem()
        p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim = B, hq, hkv, D
        p.q_dtype = p.kv_dtype = fd.DTYPES[torch.float16]
        p.layout = 0
        p.max_seq_len = T
        p.q_stride_b, p.q_stride_h = hq * D, D
        p.kv_stride_b, p.kv_stride_h, p.kv_stride_t = hkv * T * D, T * D, D
        p.kv_capacity = T
        return p

    def show(tag, fn):
        try:
            pl = fn()
        except fd.FdError as e:
            return f"{tag} status {e.status} {fd.status_str(e.status)}"
        return (f"{tag} status 0 S {pl.num_splits} chunk {pl.chunk_tokens}/{pl.odd_chunk_tokens} kernel {pl.kernel} "
                f"schedule {pl.schedule} grid {pl.grid_x} {pl.grid_y} {pl.grid_z} odd {pl.odd_range_permille} "
                f"ws {pl.ws_o_bytes} {pl.ws_stats_bytes}")

    L = fd.lib()
    lines = [f"version {fd.version()}",
             "sizes " + " ".join(str(L.fd_struct_size(i)) for i in range(4))]
    lines.append(show("gqa", lambda: fd.fd_plan(contiguous(1, 64, 8, 128, 128000), num_cus=256)))
    lines.append(show("bad", lambda: fd.fd_plan(contiguous(1, 64, 7, 128, 1000), num_cus=256)))
    lines.append(show("balanced", lambda: fd.fd_plan(contiguous(6, 32, 8, 128, 5000), num_cus=256,
                                                     schedule="balanced",
                                                     host_seq_lens=[3000, 17, 0, 2200, 5000, 900])))
    long_lens = [40000, 30000, 35000, 20000, 38000, 25000, 39000, 31000]
    for tag, x in (("balanced_long", 0), ("balanced_long_equal", -1)):
        lines.append(show(tag, lambda x=x: fd.fd_plan(contiguous(8, 32, 8, 128, 40000), num_cus=256,
                                                      schedule="balanced", host_seq_lens=long_lens,
                                                      odd_xcd_permille=x)))
    pl = fd.fd_plan(contiguous(1, 64, 8, 128, 128000), num_cus=256)
    st = L.fd_merge(ctypes.byref(pl), 4096, pl.ws_o_bytes - 4, 8192, pl.ws_stats_bytes, 4096, None, None)
    lines.append(f"merge_short status {st} {fd.status_str(st)}")
    lines.append(show("overflow", lambda: fd.fd_plan(contiguous(1, 8, 8, 128, 1000), num_cus=256,
                                                     force_splits=65535, force_chunk_tokens=65536)))
    return lines


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_plain_c_program_sees_the_same_library(tmp_path):
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(fd.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
                    str(src), "-o", str(exe), f"-L{libdir}", "-lfd", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.strip().splitlines()
    assert out == _python_side()
    assert out[2].startswith("gqa status 0 S 32 chunk 4180/3820 ") and out[3].startswith("bad status 1 ")
    assert " schedule 2 " in out[4] and " odd 0 " in out[4]
    assert " schedule 2 " in out[5] and " odd 45 " in out[5]          # alternating ranges
    assert " schedule 2 " in out[6] and " odd 0 " in out[6]           # turned off
    assert out[7] == f"merge_short status {fd.FD_ERR_WORKSPACE} {fd.status_str(fd.FD_ERR_WORKSPACE)}"
    assert out[8].startswith(f"overflow status {fd.FD_ERR_UNSUPPORTED} ")
