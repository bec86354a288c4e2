// Random and hostile fd_problem / fd_plan_opts values through fd_plan, built
// with the host sanitizers (address, undefined behaviour) by
// tests/test_plan_fuzz.py. Half the problems have consistent strides and
// options so the planner's rules run (a quarter of them with one stride set
// to an edge value); the rest mix edge values (0, -1,
// INT32_MAX, INT64_MAX, ...) into every field. Every plan that is accepted
// must be well formed; the sanitizers catch overflow and out-of-bounds reads.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>
#include "fd.h"
static std::mt19937_64 rng(12345);
static int32_t pick32() {
  static const int32_t edge[] = {0, 1, -1, 2, 7, 8, 16, 31, 32, 64, 100, 128, 1000, 4096, 65536, 128000,
                                 1 << 20, 1 << 24, INT32_MAX, INT32_MIN, INT32_MAX - 1};
  if (rng() % 3 == 0) return edge[rng() % (sizeof edge / sizeof *edge)];
  return (int32_t)(rng() % 200000) - (rng() % 10 == 0 ? 100000 : 0);
}
static int64_t pick64() {
  static const int64_t edge[] = {0, 1, -1, 128, 1 << 20, (int64_t)1 << 40, INT64_MAX, INT64_MIN};
  if (rng() % 3 == 0) return edge[rng() % 8];
  return (int64_t)(rng() % 100000000);
}
int main(int argc, char** argv) {
  long iters = argc > 1 ? atol(argv[1]) : 200000;
  long ok = 0, bad = 0;
  std::vector<int32_t> lens;
  for (long it = 0; it < iters; ++it) {
    fd_problem p; memset(&p, 0, sizeof p);
    fd_plan_opts o; memset(&o, 0, sizeof o);
    bool sane = rng() % 2;
    p.batch = sane ? 1 + rng() % 300 : pick32();
    p.num_kv_heads = sane ? 1 + rng() % 16 : pick32();
    p.num_q_heads = sane ? p.num_kv_heads * (1 + rng() % 16) : pick32();
    p.head_dim = sane ? (rng() % 2 ? 64 : 128) : pick32();
    p.q_dtype = p.kv_dtype = sane ? rng() % 3 : pick32();
    if (!sane && rng() % 2) p.kv_dtype = pick32();
    p.layout = (!sane && rng() % 3 == 0) ? pick32() : rng() % 2;
    p.max_seq_len = sane ? rng() % 300000 : pick32();
    p.q_stride_b = pick64(); p.q_stride_h = pick64(); p.q_stride_q = pick64();
    p.kv_stride_b = pick64(); p.kv_stride_h = pick64(); p.kv_stride_t = pick64();
    p.kv_capacity = sane ? p.max_seq_len : pick32();
    p.page_size = sane ? 16 << (rng() % 4) : pick32();
    p.num_pages = pick32(); p.max_pages_per_seq = pick32();
    p.bt_stride_b = pick64(); p.pool_stride_page = pick64(); p.pool_stride_t = pick64(); p.pool_stride_h = pick64();
    p.scale = rng() % 4 == 0 ? -1.0f : 0.0f;
    p.q_len = sane ? rng() % 10 : pick32();
    o.num_cus = rng() % 8 == 0 ? pick32() : 256;
    if (o.num_cus == 0) o.num_cus = 256;      // no device here
    o.wgs_per_cu = rng() % 4 == 0 ? pick32() : rng() % 3;
    o.force_splits = rng() % 5 == 0 ? pick32() : 0;
    o.force_chunk_tokens = rng() % 5 == 0 ? pick32() : 0;
    o.ws_format = rng() % 6 == 0 ? pick32() : rng() % 2;
    o.kernel = rng() % 6 == 0 ? pick32() : rng() % 3;
    o.heuristic = rng() % 6 == 0 ? pick32() : rng() % 3;
    o.max_splits = rng() % 4 == 0 ? pick32() : 0;
    o.overhead_budget = rng() % 4 == 0 ? (float)((int64_t)pick32()) * 1e-3f : 0.0f;
    o.schedule = rng() % 6 == 0 ? pick32() : rng() % 3;
    o.piece_cost_tokens = rng() % 4 == 0 ? pick32() : 0;
    if (rng() % 2 && p.batch > 0 && p.batch < 5000) {
      lens.resize(p.batch);
      for (auto& l : lens) l = rng() % 5 == 0 ? pick32() : (int32_t)(rng() % ((uint32_t)(p.max_seq_len > 0 ? p.max_seq_len : 1) + 1));
      o.host_seq_lens = lens.data();
      o.num_host_seq_lens = rng() % 10 == 0 ? pick32() : p.batch;
    }
    if (sane) {
      const int64_t D = p.head_dim, Hq = p.num_q_heads, Hkv = p.num_kv_heads;
      p.q_len = rng() % 3 == 0 ? 1 + rng() % 4 : 0;
      const int64_t ql = p.q_len > 1 ? p.q_len : 1;
      p.q_stride_h = D; p.q_stride_q = Hq * D; p.q_stride_b = ql * Hq * D;
      if (p.layout == FD_LAYOUT_PAGED) {
        p.max_pages_per_seq = (p.max_seq_len + p.page_size - 1) / p.page_size + (int32_t)(rng() % 3);
        if (p.max_pages_per_seq < 1) p.max_pages_per_seq = 1;
        p.num_pages = p.max_pages_per_seq * 2;
        p.bt_stride_b = p.max_pages_per_seq;
        p.pool_stride_t = D; p.pool_stride_h = p.page_size * D; p.pool_stride_page = Hkv * p.page_size * D;
      } else {
        p.kv_capacity = p.max_seq_len + (int32_t)(rng() % 100);
        p.kv_stride_t = D; p.kv_stride_h = (int64_t)p.kv_capacity * D; p.kv_stride_b = Hkv * p.kv_stride_h;
      }
      p.scale = 0.0f;
      if (rng() % 4 == 0) {          // one stride of a valid problem set to an edge value
        int64_t* f[] = {&p.q_stride_b, &p.q_stride_h, &p.q_stride_q, &p.kv_stride_b, &p.kv_stride_h,
                        &p.kv_stride_t, &p.bt_stride_b, &p.pool_stride_page, &p.pool_stride_t,
                        &p.pool_stride_h};
        static const int64_t edge[] = {-1, -16, (int64_t)1 << 40, ((int64_t)1 << 40) + 8, (int64_t)1 << 61,
                                       INT64_MAX, INT64_MAX - 7, INT64_MIN};
        *f[rng() % 10] = edge[rng() % 8];
      }
    }
    if (sane && rng() % 4 != 0) {
      o.num_cus = rng() % 4 == 0 ? 1 + rng() % 512 : 256;
      o.wgs_per_cu = rng() % 3;
      o.force_splits = rng() % 4 == 0 ? 1 + rng() % 300 : 0;
      o.force_chunk_tokens = rng() % 6 == 0 ? 1 + rng() % 9000 : 0;
      if (rng() % 16 == 0) {                 // forced pairs near the 32-bit token bound
        o.force_splits = 1 + (int32_t)(rng() % 65535);
        o.force_chunk_tokens = 1 << (10 + rng() % 11);
        if (p.layout == FD_LAYOUT_PAGED) o.force_chunk_tokens = 0;
      }
      o.ws_format = rng() % 2; o.kernel = 0; o.heuristic = rng() % 3;
      o.max_splits = rng() % 4 == 0 ? 1 + rng() % 300 : 0;
      o.overhead_budget = rng() % 4 == 0 ? (float)(rng() % 2000) * 1e-3f : 0.0f;
      o.schedule = rng() % 3;
      o.piece_cost_tokens = rng() % 3 == 0 ? -1 : (rng() % 3 == 0 ? (int32_t)(rng() % 4096) : 0);
      o.odd_xcd_permille = rng() % 4 == 0 ? (int32_t)(rng() % 1001) - 1 : 0;
      if (o.host_seq_lens) o.num_host_seq_lens = p.batch;
    }
    fd_plan_t pl;
    int st = fd_plan(&p, &o, &pl);
    if (st == FD_OK) {
      ++ok;
      if (pl.num_splits < 1 || pl.grid_x < 1 || pl.ws_o_bytes < 0 || pl.ws_stats_bytes < 0) {
        printf("iter %ld: odd plan S=%d grid=%d\n", it, pl.num_splits, pl.grid_x);
        return 1;
      }
      // uniform split s starts at token s * chunk, a 32-bit index on the device
      if (pl.schedule == FD_SCHEDULE_UNIFORM && (int64_t)pl.num_splits * pl.chunk_tokens > INT32_MAX) {
        printf("iter %ld: split boundaries overflow: S=%d chunk=%d\n", it, pl.num_splits, pl.chunk_tokens);
        return 1;
      }
      // weighted balanced cuts multiply granule positions by up to 1000 (N + 2)
      if (pl.schedule == FD_SCHEDULE_BALANCED && pl.odd_range_permille > 0) {
        const fd_problem& q = pl.prob;
        const int64_t cap = q.layout == FD_LAYOUT_PAGED ? (int64_t)q.max_pages_per_seq * q.page_size : q.kv_capacity;
        const int64_t G = pl.chunk_tokens;
        const int64_t t_max = (int64_t)q.batch * q.num_kv_heads * ((cap + G - 1) / G + pl.piece_cost);
        if ((__int128)t_max * (1000 * ((__int128)pl.grid_x + 2)) > ((__int128)1 << 62)) {
          printf("iter %ld: weighted cut overflows: t_max=%ld N=%d\n", it, (long)t_max, pl.grid_x);
          return 1;
        }
      }
      if (pl.odd_range_permille < 0 || pl.odd_range_permille > 999 ||
          (pl.schedule != FD_SCHEDULE_BALANCED && pl.odd_range_permille != 0)) {
        printf("iter %ld: bad odd_range_permille %d\n", it, pl.odd_range_permille);
        return 1;
      }
    } else ++bad;
  }
  printf("ok %ld rejected %ld\n", ok, bad);
  return 0;
}
