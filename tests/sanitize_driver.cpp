// Exercises the library's host-only code (host.cpp: composite-table checks,
// rank allocations; sched.cpp: the slot pool and the batch choice) under the
// address and undefined-behaviour sanitizers, built with the host compiler
// alone: valid inputs, every error path, and seeded random tables, pools and
// request sets.  Exits 0 when every call returned the status the input
// earns; a sanitizer report aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "tcl.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "line %d: %s\n", __LINE__, #cond);          \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

struct Table {
  std::vector<int32_t> gt, gp, pa;
  std::vector<float> pw;
  tcl_composites c{};
  void bind(int32_t T, int32_t N, int32_t cap) {
    c.n_tokens = T;
    c.n_groups = int32_t(gt.size()) - 1;
    c.n_pairs = int32_t(pa.size());
    c.n_adapters = N;
    c.max_tuples = cap;
    c.group_tok_ptr = gt.data();
    c.group_pair_ptr = gp.data();
    c.pair_adapter = pa.empty() ? nullptr : pa.data();
    c.pair_alpha = pw.empty() ? nullptr : pw.data();
  }
};

// one token per group, n pairs each, distinct ids
static Table simple(int T, int n, int N) {
  Table t;
  for (int g = 0; g <= T; ++g) {
    t.gt.push_back(g);
    t.gp.push_back(g * n);
  }
  for (int g = 0; g < T; ++g)
    for (int i = 0; i < n; ++i) {
      t.pa.push_back((g + i) % N);
      t.pw.push_back(0.5f);
    }
  t.bind(T, N, 1 << 20);
  return t;
}

static void composites() {
  int32_t P = 0, U = 0;
  Table t = simple(5, 3, 7);
  EXPECT(tcl_composites_validate(&t.c, &P, &U) == TCL_OK && P == 15);
  EXPECT(tcl_composites_validate(nullptr, &P, &U) == TCL_EINVAL);
  Table a = simple(5, 3, 7);
  a.pa[4] = 7;
  EXPECT(tcl_composites_validate(&a.c, &P, &U) == TCL_EINVAL);     // id out of range
  Table b = simple(5, 3, 7);
  b.pw[2] = std::nanf("");
  EXPECT(tcl_composites_validate(&b.c, &P, &U) == TCL_EINVAL);     // NaN alpha
  Table d = simple(5, 3, 7);
  d.pa[1] = d.pa[0];
  EXPECT(tcl_composites_validate(&d.c, &P, &U) == TCL_EINVAL);     // duplicate
  Table e = simple(5, 3, 7);
  e.gp[2] = 1;
  EXPECT(tcl_composites_validate(&e.c, &P, &U) == TCL_EINVAL);     // decreasing
  Table f = simple(2, 65, 100);
  EXPECT(tcl_composites_validate(&f.c, &P, &U) == TCL_EUNSUPPORTED);  // 65 pairs
  Table g = simple(5, 3, 7);
  g.c.max_tuples = 14;
  EXPECT(tcl_composites_validate(&g.c, &P, &U) == TCL_ENOSPC);
  Table h = simple(0, 0, 3);
  EXPECT(tcl_composites_validate(&h.c, &P, &U) == TCL_OK && P == 0);
  // random tables: CSR pointers that may decrease or overrun, ids that may
  // be out of range; the check must stay inside the arrays and return a code
  std::mt19937 rng(7);
  for (int it = 0; it < 4000; ++it) {
    Table r;
    const int G = int(rng() % 12), N = 1 + int(rng() % 10);
    int tok = 0, pr = 0;
    r.gt.push_back(0);
    r.gp.push_back(0);
    for (int gg = 0; gg < G; ++gg) {
      tok += int(rng() % 4) - (rng() % 17 == 0 ? 2 : 0);
      pr += int(rng() % 5) - (rng() % 19 == 0 ? 3 : 0);
      r.gt.push_back(tok);
      r.gp.push_back(pr);
    }
    const int NP = std::max(0, pr + (rng() % 23 == 0 ? 1 : 0));
    for (int q = 0; q < NP; ++q) {
      r.pa.push_back(int(rng() % (N + 2)) - (rng() % 29 == 0 ? 1 : 0));
      r.pw.push_back(rng() % 31 == 0 ? INFINITY : float(rng() % 100) / 100.f);
    }
    r.bind(std::max(0, tok) + (rng() % 13 == 0 ? 1 : 0), N, int(rng() % 64));
    const int rc = tcl_composites_validate(&r.c, &P, &U);
    EXPECT(rc == TCL_OK || rc == TCL_EINVAL || rc == TCL_EUNSUPPORTED || rc == TCL_ENOSPC);
    EXPECT(tcl_last_error() != nullptr);
  }
}

static void bam() {
  tcl_bam *b = nullptr;
  EXPECT(tcl_bam_create(0, &b) == TCL_EINVAL);
  EXPECT(tcl_bam_create(4, nullptr) == TCL_EINVAL);
  EXPECT(tcl_bam_create(6, &b) == TCL_OK && b);
  std::mt19937 rng(11);
  std::vector<int32_t> slot_of(16), ls(16), la(16), le(16), slots(6);
  for (int it = 0; it < 3000; ++it) {
    const int n = int(rng() % 9);
    std::vector<int32_t> ads(n);
    for (auto &a : ads) a = int(rng() % 14);
    int32_t nl = -1;
    const int rc = tcl_bam_acquire(b, ads.data(), n, slot_of.data(), ls.data(), la.data(),
                                   le.data(), &nl);
    EXPECT(rc == TCL_OK || rc == TCL_ENOSPC);
    EXPECT(nl >= 0 && nl <= n);
    EXPECT(tcl_bam_slots(b, slots.data()) == TCL_OK);
  }
  int32_t bad = -3, nl = 0;
  EXPECT(tcl_bam_acquire(b, &bad, 1, slot_of.data(), ls.data(), la.data(), le.data(), &nl) ==
         TCL_EINVAL);
  EXPECT(tcl_bam_acquire(b, nullptr, 1, slot_of.data(), ls.data(), la.data(), le.data(), &nl) ==
         TCL_EINVAL);
  tcl_bam_free(b);
  tcl_bam_free(nullptr);
}

static void lag() {
  std::mt19937 rng(13);
  for (int it = 0; it < 2000; ++it) {
    const int R = int(rng() % 20);
    std::vector<double> arr(R);
    std::vector<int32_t> ptr(1, 0), ads, res, chosen(R + 1);
    for (int i = 0; i < R; ++i) {
      arr[i] = double(rng() % 50);
      const int n = int(rng() % 4);
      for (int j = 0; j < n; ++j) ads.push_back(int(rng() % 12));
      ptr.push_back(int32_t(ads.size()));
    }
    for (int j = 0; j < int(rng() % 6); ++j) res.push_back(int(rng() % 12));
    int32_t nc = -1;
    const int rc = tcl_lag_select(arr.data(), ptr.data(), ads.empty() ? nullptr : ads.data(), R,
                                  res.empty() ? nullptr : res.data(), int32_t(res.size()), 60.0,
                                  double(rng() % 30), 1 + int(rng() % 6), 1 + int(rng() % 8),
                                  chosen.data(), &nc);
    EXPECT(rc == TCL_OK || rc == TCL_EINVAL);
    if (rc == TCL_OK) EXPECT(nc >= 0 && nc <= R);
  }
  double nan_t = std::nan("");
  int32_t ptr[2] = {0, 1}, ad = 0, ch = 0, nc = 0;
  EXPECT(tcl_lag_select(&nan_t, ptr, &ad, 1, nullptr, 0, 1.0, 1.0, 1, 1, &ch, &nc) ==
         TCL_EINVAL);
}

static void ranks() {
  std::mt19937 rng(17);
  for (int it = 0; it < 2000; ++it) {
    const int M = int(rng() % 8), L = 1 + int(rng() % 6);
    std::vector<int32_t> r(M), fl(M), u(M), k(M);
    std::vector<int64_t> cost(M);
    std::vector<double> sg(size_t(M) * L);
    for (int m = 0; m < M; ++m) {
      r[m] = int(rng() % (L + 1)) - (rng() % 37 == 0 ? L + 2 : 0);
      cost[m] = 1 + int64_t(rng() % 5);
      fl[m] = int(rng() % 3);
    }
    for (auto &s : sg) s = rng() % 41 == 0 ? -1.0 : double(rng() % 100) / 10.0;
    int64_t budget = 0;
    const int rc1 = tcl_rank_uniform(r.data(), cost.data(), M, 1 + int(rng() % 4), u.data(),
                                     &budget);
    EXPECT(rc1 == TCL_OK || rc1 == TCL_EINVAL);
    const int rc2 = tcl_rank_spectral(sg.data(), L, r.data(), cost.data(), fl.data(), M,
                                      int64_t(rng() % 40), k.data());
    EXPECT(rc2 == TCL_OK || rc2 == TCL_EINVAL);
  }
  int64_t b = 0;
  EXPECT(tcl_rank_uniform(nullptr, nullptr, 1, 1, nullptr, &b) == TCL_EINVAL);
}

int main() {
  composites();
  bam();
  lag();
  ranks();
  std::printf("sanitize driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
