// Host-side planning and validation under AddressSanitizer and
// UndefinedBehaviorSanitizer: a seeded sweep of parameter sets, valid and
// hostile (zero, negative, INT32/INT64 extremes, sizes near the limits), fed
// to every planner and to the host checks of the C ABI. Built with g++ by
// tests/test_host_sanitizers.py; no GPU code is involved. Any sanitizer
// report aborts the process; the sweep prints "ok" and the number of
// accepted sets at the end.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "gsa.h"
#include "gsa_plan.hpp"

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;

uint64_t next_u64() {   // splitmix64
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

int64_t below(int64_t n) { return n <= 0 ? 0 : (int64_t)(next_u64() % (uint64_t)n); }

// a value that is usually one of `usual`, sometimes an extreme
int64_t pick(std::initializer_list<int64_t> usual, bool wide = false) {
  static const int64_t extremes[] = {0, -1, 1, 2, 3, 63, 64, 65, 4095, 4096, 4097, INT32_MAX, INT32_MIN,
                                     (int64_t)INT32_MAX + 1, INT64_MAX / 2, INT64_MAX, INT64_MIN, 1ll << 31,
                                     1ll << 40};
  if (below(100) < 94) return *(usual.begin() + below((int64_t)usual.size()));
  if (below(4) == 0) return wide ? (int64_t)next_u64() : (int32_t)next_u64();
  int64_t v = extremes[below(sizeof(extremes) / sizeof(extremes[0]))];
  return wide ? v : (int64_t)(int32_t)v;
}

int32_t p32(std::initializer_list<int64_t> usual) { return (int32_t)pick(usual); }

gsa_decode_params decode_params() {
  gsa_decode_params p;
  memset(&p, 0, sizeof(p));
  p.batch = p32({1, 2, 4, 8, 32, 64});
  p.n_kv_heads = p32({1, 2, 8});
  p.n_q_heads = (int32_t)((int64_t)p.n_kv_heads * p32({1, 2, 4, 8}));
  p.head_dim = p32({64, 128});
  p.chunk = p32({1, 4, 8, 16, 32});
  const int64_t C = p.chunk > 0 && p.chunk < 4096 ? p.chunk : 16;
  p.n_gist = pick({1, 7, 64, 640, 2048, 4096, 8192, 65536, 1 << 20}, true);
  const int64_t M = p.n_gist > 0 && p.n_gist < (1ll << 24) ? p.n_gist : 64;
  p.n_raw = below(5) == 0 ? pick({0, 1, 4096}, true) : M * C + below(C + 1);
  p.topk = p32({0, 1, 8, 16, 64, 65, 80});
  p.tail = p32({0, 16, 64, (int64_t)C, 100});
  p.scale = below(8) == 0 ? -1.0f : 0.0f;
  p.dtype = p32({GSA_BF16, GSA_F32});
  p.gist_set = p32({0, 1, 2});
  p.row_capacity = below(4) == 0 ? pick({0, 1, 1ll << 40}, true) : 0;
  return p;
}

gsa_prefill_params prefill_params() {
  gsa_prefill_params p;
  memset(&p, 0, sizeof(p));
  p.n_kv_heads = p32({1, 2, 8});
  p.n_q_heads = (int32_t)((int64_t)p.n_kv_heads * p32({1, 2, 4, 8}));
  p.head_dim = p32({64, 128});
  p.chunk = p32({4, 8, 16});
  p.topk = p32({0, 8, 16, 32, 64});
  p.window = p32({0, 16, 64, 128});
  const int64_t C = p.chunk > 0 && p.chunk < 4096 ? p.chunk : 16;
  p.n_gist = pick({1, 64, 4096, 65536}, true);
  const int64_t M = p.n_gist > 0 && p.n_gist < (1ll << 24) ? p.n_gist : 64;
  p.n_raw = below(5) == 0 ? pick({0, 1}, true) : M * C + below(C + 1);
  p.q_start = below(3) == 0 ? pick({0, -1, 1ll << 40}, true) : below(p.n_raw > 0 ? p.n_raw : 1);
  p.n_q = below(3) == 0 ? pick({0, 1, 4096}, true) : below(4097);
  p.scale = 0.0f;
  p.dtype = p32({GSA_BF16, GSA_F32});
  p.row_capacity = below(4) == 0 ? pick({0, 1}, true) : 0;
  return p;
}

template <class T>
void need(bool c, const char* what, const T& unused) {
  (void)unused;
  if (!c) {
    fprintf(stderr, "invariant broken: %s\n", what);
    abort();
  }
}

int g_accepted = 0;

void decode_case() {
  gsa_decode_params p = decode_params();
  gsa::DecodePlan d;
  int32_t n = 0;
  const gsa_status_t s = gsa::plan_decode(&p, &d);
  const gsa_status_t sl = gsa_decode_launches(&p, &n);
  need(s == sl, "gsa_decode_launches validates like the planner", 0);
  if (s == GSA_OK) {
    ++g_accepted;
    need(n >= 1 && n <= 3, "decode launch count", 0);
    need(d.total > 0 && d.off_part <= d.total && d.off_sel <= d.total, "decode workspace layout", 0);
    if (p.batch <= 64) {
      std::vector<int32_t> sn(p.batch), sm(p.batch);
      for (int b = 0; b < p.batch; ++b) {
        sn[b] = (int32_t)pick({1, 16, 4096, p.n_raw}, false);
        sm[b] = (int32_t)pick({0, 1, 256, p.n_gist}, false);
      }
      gsa_check_seq_lens(&p, sn.data(), sm.data());
    }
  }
  gsa_check_seq_lens(&p, nullptr, nullptr);

  gsa_hier_params h;
  h.base = p;
  h.fanout = p32({1, 4, 8, 16});
  h.topk2 = p32({0, 2, 8, 16, 64});
  gsa::HierPlan hp;
  if (gsa::plan_hier(&h, &hp) == GSA_OK) {
    need(gsa_decode_hier_launches(&h, &n) == GSA_OK && n >= 1 && n <= 5, "hier launch count", 0);
    need(hp.total > 0 && hp.off_part <= hp.total, "hier workspace layout", 0);
    if (p.batch <= 64) {
      std::vector<int32_t> sn(p.batch, (int32_t)p.n_raw), sm(p.batch, (int32_t)p.n_gist);
      gsa_check_hier_seq_lens(&h, sn.data(), sm.data());
    }
  }

  gsa_levels_params l;
  memset(&l, 0, sizeof(l));
  l.base = p;
  l.n_levels = p32({2, 3, 4, 6, 7});
  l.fanout = p32({2, 3, 4, 16});
  for (int i = 0; i < GSA_MAX_LEVELS - 1; ++i) l.topk_up[i] = p32({0, 1, 4, 8, 1025});
  gsa::LevelsPlan lp;
  if (gsa::plan_levels(&l, &lp) == GSA_OK) {
    need(gsa_decode_levels_launches(&l, &n) == GSA_OK && n >= 1 && n <= GSA_MAX_LEVELS + 1,
         "levels launch count", 0);
    if (p.batch <= 64) {
      std::vector<int32_t> sn(p.batch, (int32_t)p.n_raw), sm(p.batch, (int32_t)p.n_gist);
      gsa_check_levels_seq_lens(&l, sn.data(), sm.data());
    }
  }

  gsa_paged_params g;
  memset(&g, 0, sizeof(g));
  g.base = p;
  g.base.row_capacity = 0;
  g.page_chunks = p32({1, 2, 16, 64, 65});
  g.max_pages = p32({1, 16, 2048, 2049});
  g.n_pages = pick({1, 64, 4096}, true);
  g.max_extra = p32({0, 4, 64, 65});
  gsa::DecodePlan pp;
  if (gsa::plan_paged(&g, &pp) == GSA_OK && p.batch <= 8 && g.max_pages <= 2048 && g.max_extra <= 64) {
    std::vector<int32_t> table((size_t)p.batch * g.max_pages), extra((size_t)p.batch * (g.max_extra + 1) * 2);
    for (auto& t : table) t = (int32_t)below(g.n_pages + 1) - (below(50) == 0 ? 1 : 0);
    for (auto& e : extra) e = (int32_t)below(300) - 1;
    std::vector<int32_t> sn(p.batch, (int32_t)p.n_raw), sm(p.batch, (int32_t)p.n_gist);
    gsa_check_pages(&g, table.data(), sn.data(), sm.data(), extra.data());
  }
}

void prefill_case() {
  gsa_prefill_params p = prefill_params();
  gsa::PrefillPlan d;
  int32_t n = 0;
  const gsa_status_t s = gsa::plan_prefill(&p, &d);
  need(gsa_prefill_launches(&p, &n) == s, "gsa_prefill_launches validates like the planner", 0);
  if (s == GSA_OK) {
    ++g_accepted;
    need(n >= 0 && n <= 2, "prefill launch count", 0);
  }
  gsa_prefill_varlen_params v;
  v.base = p;
  v.batch = p32({1, 3, 16});
  gsa::PrefillPlan dv;
  if (gsa::plan_prefill_varlen(&v, &dv) == GSA_OK && v.batch <= 64) {
    std::vector<int32_t> seqs((size_t)v.batch * 4);
    for (auto& x : seqs) x = (int32_t)pick({0, 1, 16, 17, 512, 4096});
    gsa_check_prefill_seqs(&v, seqs.data());
  }
  gsa_gist_params gp;
  memset(&gp, 0, sizeof(gp));
  gp.n_kv_heads = p.n_kv_heads;
  gp.n_q_heads = p.n_q_heads;
  gp.head_dim = p.head_dim;
  gp.chunk = p.chunk;
  gp.n_raw = p.n_raw;
  gp.n_gist = p.n_gist;
  gp.m_start = below(3) == 0 ? pick({-1, 0, 1ll << 40}, true) : below(p.n_gist > 0 ? p.n_gist : 1);
  gp.n_q = pick({0, 1, 64, 4096}, true);
  gp.dtype = p.dtype;
  gsa::PrefillPlan g;
  (void)gsa::plan_gist(&gp, &g);
  gsa_append_params a;
  memset(&a, 0, sizeof(a));
  a.batch = p32({1, 4, 32});
  a.n_kv_heads = p.n_kv_heads;
  a.head_dim = p.head_dim;
  a.chunk = p.chunk;
  a.n_raw = p.n_raw;
  a.n_gist = p.n_gist;
  a.raw_new = pick({0, 1, 16, 4096}, true);
  a.gist_new = pick({0, 1, 256}, true);
  a.row_capacity = pick({0, 1ll << 20}, true);
  a.dtype = p.dtype;
  gsa::AppendPlan ap;
  (void)gsa::plan_append(&a, &ap);
}

void misc_case() {
  int32_t k = 0;
  gsa_topk_for_budget(pick({0, 100, 4096, 1ll << 40}, true), pick({0, 10, 2048}, true), p32({0, 1, 16}),
                      p32({0, 64, -1}), p32({0, 1, 2, 3}), below(20) == 0 ? nullptr : &k);
  need(gsa_status_string((gsa_status_t)(int32_t)pick({0, 1, 2, 3, 4, 5})) != nullptr, "status string", 0);
  need(gsa_last_error() != nullptr, "last error", 0);
  gsa_decode_launches(nullptr, &k);
  gsa_decode_hier_launches(nullptr, &k);
  gsa_decode_levels_launches(nullptr, &k);
  gsa_prefill_launches(nullptr, &k);
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 100000;
  if (argc > 2) g_state = strtoull(argv[2], nullptr, 0);
  for (long i = 0; i < iters; ++i) {
    decode_case();
    prefill_case();
    misc_case();
  }
  printf("ok %ld sets, %d accepted\n", iters, g_accepted);
  return 0;
}
