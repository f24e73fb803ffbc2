// Host-only parts of the library: error reporting, the host-side check of a
// composite table, and the two rank allocations of the retained-rank
// producer.  Plain C++ with no device code and no HIP call, so that it also
// builds with the host compiler alone (the library's sanitizer build).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "tcl_internal.hpp"

namespace tcl {

static thread_local std::string g_err;

bool log_enabled() {
  static int on = [] {
    const char *s = std::getenv("TCL_LOG");
    return (s && *s && *s != '0') ? 1 : 0;
  }();
  return on != 0;
}

void logf(const char *fmt, ...) {
  if (!log_enabled()) return;
  va_list ap;
  va_start(ap, fmt);
  std::fprintf(stderr, "[tcl] ");
  std::vfprintf(stderr, fmt, ap);
  std::fprintf(stderr, "\n");
  va_end(ap);
}

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  logf("error %d: %s", code, buf);
  return code;
}

int check_composites(const tcl_composites *c) {
  if (!c) return fail(TCL_EINVAL, "composites is NULL");
  if (!c->group_tok_ptr || !c->group_pair_ptr)
    return fail(TCL_EINVAL, "group pointer arrays must not be NULL");
  if (c->n_pairs > 0 && (!c->pair_adapter || !c->pair_alpha))
    return fail(TCL_EINVAL, "pair arrays must not be NULL when n_pairs > 0");
  return TCL_OK;
}

// A host-resident composite table, checked on the host by the rules of the
// mapping stage (DyMerge-LoRA section 4.3: the tuples are built from the
// composites; the table's rules are the library's), with its codes and their
// precedence: TCL_EINVAL (CSR pointers that do not start at 0, end at the
// token count, end beyond the pair arrays or decrease; an adapter id outside
// [0, N) among the table's pairs; a
// non-finite alpha; an adapter twice in a composite of at most
// TCL_MAX_PAIRS_PER_GROUP pairs) before TCL_EUNSUPPORTED (a larger
// composite) before TCL_ENOSPC (more tuples than max_tuples).  Counts the
// tuples and the adapters that own at least one tuple.  No GPU is touched.
int validate_host(const tcl_composites *c, int64_t *P_out, int32_t *U_out) {
  const int32_t G = c->n_groups, NP = c->n_pairs, T = c->n_tokens, N = c->n_adapters;
  if (G < 0 || NP < 0 || T < 0 || c->max_tuples < 0)
    return fail(TCL_EINVAL, "negative size (tokens %d, groups %d, pairs %d, max_tuples %d)", T,
                G, NP, c->max_tuples);
  if (N < 1) return fail(TCL_EINVAL, "n_adapters must be >= 1 (got %d)", N);
  const int32_t *gt = c->group_tok_ptr, *gp = c->group_pair_ptr, *pa = c->pair_adapter;
  const float *pw = c->pair_alpha;
  if (gt[0] != 0 || gt[G] != T)
    return fail(TCL_EINVAL, "group_tok_ptr must run from 0 to n_tokens (%d .. %d, want 0 .. %d)",
                gt[0], gt[G], T);
  // the pair arrays hold n_pairs entries; the table's pairs end at gp[G],
  // and entries beyond it are unused capacity, never read
  if (gp[0] != 0 || gp[G] > NP)
    return fail(TCL_EINVAL,
                "group_pair_ptr must run from 0 to at most n_pairs (%d .. %d, n_pairs %d)",
                gp[0], gp[G], NP);
  for (int32_t g = 0; g < G; ++g)
    if (gt[g + 1] < gt[g] || gp[g + 1] < gp[g])
      return fail(TCL_EINVAL, "group pointers decrease at group %d", g);
  const int32_t NPe = gp[G];
  for (int32_t q = 0; q < NPe; ++q) {
    if (pa[q] < 0 || pa[q] >= N)
      return fail(TCL_EINVAL, "pair %d: adapter id %d outside [0, %d)", q, pa[q], N);
    if (!std::isfinite(pw[q])) return fail(TCL_EINVAL, "pair %d: alpha is not finite", q);
  }
  std::vector<int32_t> last(size_t(N), -1);
  for (int32_t g = 0; g < G; ++g) {
    if (gp[g + 1] - gp[g] > TCL_MAX_PAIRS_PER_GROUP) continue;  // not searched (too large)
    for (int32_t q = gp[g]; q < gp[g + 1]; ++q) {
      if (last[size_t(pa[q])] == g)
        return fail(TCL_EINVAL, "group %d holds adapter %d twice", g, pa[q]);
      last[size_t(pa[q])] = g;
    }
  }
  for (int32_t g = 0; g < G; ++g)
    if (gp[g + 1] - gp[g] > TCL_MAX_PAIRS_PER_GROUP)
      return fail(TCL_EUNSUPPORTED, "group %d holds %d pairs (at most %d)", g, gp[g + 1] - gp[g],
                  TCL_MAX_PAIRS_PER_GROUP);
  int64_t P = 0;
  std::vector<char> used(size_t(N), 0);
  int32_t U = 0;
  for (int32_t g = 0; g < G; ++g) {
    const int64_t nt = gt[g + 1] - gt[g];
    P += nt * (gp[g + 1] - gp[g]);
    if (nt > 0)
      for (int32_t q = gp[g]; q < gp[g + 1]; ++q)
        if (!used[size_t(pa[q])]) {
          used[size_t(pa[q])] = 1;
          ++U;
        }
  }
  if (P > c->max_tuples)
    return fail(TCL_ENOSPC, "the table expands to %lld tuples, max_tuples is %d", (long long)P,
                c->max_tuples);
  *P_out = P;
  *U_out = U;
  return TCL_OK;
}

}  // namespace tcl

using namespace tcl;

extern "C" {

const char *tcl_last_error(void) { return g_err.c_str(); }

int tcl_composites_validate(const tcl_composites *c, int32_t *n_tuples, int32_t *n_segments) {
  int rc = check_composites(c);
  if (rc) return rc;
  int64_t P = 0;
  int32_t U = 0;
  if ((rc = validate_host(c, &P, &U))) return rc;
  if (n_tuples) *n_tuples = int32_t(P);
  if (n_segments) *n_segments = U;
  return TCL_OK;
}

}  // extern "C"

extern "C" int tcl_rank_uniform(const int32_t *ranks, const int64_t *costs, int32_t n_modules,
                                int32_t denominator, int32_t *u_out, int64_t *budget_out) {
  if (n_modules < 0 || denominator < 1) return fail(TCL_EINVAL, "rank_uniform: bad sizes");
  if (n_modules > 0 && (!ranks || !costs || !u_out)) return fail(TCL_EINVAL, "rank_uniform: NULL pointer");
  if (!budget_out) return fail(TCL_EINVAL, "rank_uniform: budget_out is NULL");
  int64_t budget = 0;
  for (int m = 0; m < n_modules; ++m) {
    if (ranks[m] < 0 || costs[m] < 1) return fail(TCL_EINVAL, "rank_uniform: module %d: rank < 0 or cost < 1", m);
    u_out[m] = std::max(1, ranks[m] / denominator);
    budget += int64_t(u_out[m]) * costs[m];
  }
  *budget_out = budget;
  return TCL_OK;
}

extern "C" int tcl_rank_spectral(const double *sigma, int64_t ld_sigma, const int32_t *ranks,
                                 const int64_t *costs, const int32_t *floors, int32_t n_modules,
                                 int64_t budget, int32_t *k_out) {
  if (n_modules < 0) return fail(TCL_EINVAL, "rank_spectral: n_modules < 0");
  if (n_modules > 0 && (!sigma || !ranks || !costs || !floors || !k_out))
    return fail(TCL_EINVAL, "rank_spectral: NULL pointer");
  struct Item {
    double eta;
    int32_t m, j;
  };
  std::vector<Item> items;
  int64_t left = budget;
  for (int m = 0; m < n_modules; ++m) {
    if (ranks[m] < 0 || ranks[m] > ld_sigma || costs[m] < 1 || floors[m] < 0)
      return fail(TCL_EINVAL, "rank_spectral: module %d: bad rank, cost or floor", m);
    k_out[m] = std::min(floors[m], ranks[m]);
    left -= int64_t(k_out[m]) * costs[m];
    for (int j = 0; j < ranks[m]; ++j) {
      const double s = sigma[int64_t(m) * ld_sigma + j];
      if (!(s >= 0.0) || !std::isfinite(s)) return fail(TCL_EINVAL, "rank_spectral: sigma[%d][%d] not finite and >= 0", m, j);
      if (j >= k_out[m]) items.push_back({s * s / double(costs[m]), m, j});
    }
  }
  std::sort(items.begin(), items.end(), [](const Item &x, const Item &y) {
    if (x.eta != y.eta) return x.eta > y.eta;
    return x.m != y.m ? x.m < y.m : x.j < y.j;
  });
  for (const Item &it : items)
    if (it.j == k_out[it.m] && costs[it.m] <= left) {
      ++k_out[it.m];
      left -= costs[it.m];
    }
  return TCL_OK;
}
