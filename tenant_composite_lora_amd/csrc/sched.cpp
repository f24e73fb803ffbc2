// Adapter residency and batch choice on the host (DyMerge-LoRA, section 4:
// BAM keeps the raw adapter factors in GPU slots, pins the adapters of the
// running batch and lets the others go least recently used first; the LAG
// scheduler batches the requests that need the fewest adapters not already
// resident, serving requests that have waited too long first, in arrival
// order).  Plain C++: the decisions are a few thousand integer operations
// per batch; the GPU work they steer is the copy of each loaded adapter into
// its slot and the apply over the slot pool.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "tcl_internal.hpp"

struct tcl_bam {
  int32_t n_slots = 0;
  int64_t time = 0;                 // one tick per acquire call
  std::vector<int32_t> slot_adapter;  // -1: empty
  std::vector<int64_t> last_use;
  std::unordered_map<int32_t, int32_t> slot_of;  // resident adapter -> slot
};

using tcl::fail;

extern "C" int tcl_bam_create(int32_t n_slots, tcl_bam **out) {
  if (!out) return fail(TCL_EINVAL, "bam: out is NULL");
  if (n_slots < 1) return fail(TCL_EINVAL, "bam: n_slots %d < 1", n_slots);
  tcl_bam *b = new tcl_bam;
  b->n_slots = n_slots;
  b->slot_adapter.assign(n_slots, -1);
  b->last_use.assign(n_slots, -1);
  *out = b;
  return TCL_OK;
}

extern "C" void tcl_bam_free(tcl_bam *b) { delete b; }

extern "C" int tcl_bam_slots(const tcl_bam *b, int32_t *slot_adapter) {
  if (!b || !slot_adapter) return fail(TCL_EINVAL, "bam: NULL pointer");
  std::copy(b->slot_adapter.begin(), b->slot_adapter.end(), slot_adapter);
  return TCL_OK;
}

extern "C" int tcl_bam_acquire(tcl_bam *b, const int32_t *adapters, int32_t n, int32_t *slot_of,
                               int32_t *load_slot, int32_t *load_adapter, int32_t *load_evicted,
                               int32_t *n_loads) {
  if (!b || !n_loads || (n > 0 && (!adapters || !slot_of || !load_slot || !load_adapter ||
                                   !load_evicted)))
    return fail(TCL_EINVAL, "bam: NULL pointer");
  if (n < 0) return fail(TCL_EINVAL, "bam: n %d < 0", n);
  for (int i = 0; i < n; ++i)
    if (adapters[i] < 0) return fail(TCL_EINVAL, "bam: adapter id %d < 0", adapters[i]);
  const int64_t t = b->time++;
  *n_loads = 0;
  // the batch's distinct adapters in order of first appearance
  std::vector<int32_t> distinct;
  std::unordered_map<int32_t, int32_t> where;
  for (int i = 0; i < n; ++i)
    if (where.emplace(adapters[i], -1).second) distinct.push_back(adapters[i]);
  if (int64_t(distinct.size()) > b->n_slots)
    return fail(TCL_ENOSPC, "bam: %zu adapters in the batch, %d slots", distinct.size(), b->n_slots);
  std::vector<int32_t> sa = b->slot_adapter;
  std::vector<int64_t> last = b->last_use;
  std::vector<char> pinned(b->n_slots, 0);
  // hits first: pinned before any load can evict them
  for (int32_t a : distinct) {
    auto it = b->slot_of.find(a);
    if (it != b->slot_of.end()) {
      pinned[it->second] = 1;
      last[it->second] = t;
      where[a] = it->second;
    }
  }
  int nl = 0;
  for (int32_t a : distinct) {
    if (where[a] >= 0) continue;
    int s = -1;
    for (int q = 0; q < b->n_slots; ++q)
      if (sa[q] == -1) {
        s = q;
        break;
      }
    if (s < 0)
      for (int q = 0; q < b->n_slots; ++q)
        if (!pinned[q] && (s < 0 || last[q] < last[s])) s = q;
    // at most n_slots distinct adapters, so an unpinned slot exists
    load_slot[nl] = s;
    load_adapter[nl] = a;
    load_evicted[nl] = sa[s];
    ++nl;
    sa[s] = a;
    last[s] = t;
    pinned[s] = 1;
    where[a] = s;
  }
  for (int i = 0; i < nl; ++i) {
    if (load_evicted[i] >= 0) b->slot_of.erase(load_evicted[i]);
    b->slot_of[load_adapter[i]] = load_slot[i];
  }
  b->slot_adapter.swap(sa);
  b->last_use.swap(last);
  for (int i = 0; i < n; ++i) slot_of[i] = where[adapters[i]];
  *n_loads = nl;
  return TCL_OK;
}

extern "C" int tcl_lag_select(const double *arrival, const int32_t *req_ptr,
                              const int32_t *req_adapters, int32_t n_requests,
                              const int32_t *resident, int32_t n_resident, double now, double theta,
                              int32_t max_batch, int32_t n_slots, int32_t *chosen,
                              int32_t *n_chosen) {
  if (!n_chosen || n_requests < 0 || n_resident < 0 || max_batch < 0 || n_slots < 0)
    return fail(TCL_EINVAL, "lag: bad sizes or NULL n_chosen");
  if (n_requests > 0 && (!arrival || !req_ptr || !chosen))
    return fail(TCL_EINVAL, "lag: NULL pointer");
  if (n_resident > 0 && !resident) return fail(TCL_EINVAL, "lag: resident is NULL");
  if (std::isnan(now) || std::isnan(theta)) return fail(TCL_EINVAL, "lag: now or theta is NaN");
  *n_chosen = 0;
  int32_t max_id = -1;
  if (n_requests > 0) {
    if (req_ptr[0] != 0) return fail(TCL_EINVAL, "lag: req_ptr[0] != 0");
    for (int i = 0; i < n_requests; ++i) {
      if (req_ptr[i + 1] < req_ptr[i]) return fail(TCL_EINVAL, "lag: req_ptr decreasing");
      if (std::isnan(arrival[i])) return fail(TCL_EINVAL, "lag: arrival %d is NaN", i);
    }
    if (req_ptr[n_requests] > 0 && !req_adapters) return fail(TCL_EINVAL, "lag: req_adapters is NULL");
    for (int e = 0; e < req_ptr[n_requests]; ++e) {
      if (req_adapters[e] < 0) return fail(TCL_EINVAL, "lag: adapter id < 0");
      max_id = std::max(max_id, req_adapters[e]);
    }
  }
  for (int i = 0; i < n_resident; ++i) {
    if (resident[i] < 0) return fail(TCL_EINVAL, "lag: resident id < 0");
    max_id = std::max(max_id, resident[i]);
  }
  const size_t A = size_t(max_id) + 1;
  std::vector<char> res(A, 0), in_batch(A, 0), taken(n_requests, 0);
  for (int i = 0; i < n_resident; ++i) res[resident[i]] = 1;
  // a request's distinct adapters
  std::vector<std::vector<int32_t>> L(n_requests);
  {
    std::vector<int32_t> seen(A, -1);
    for (int i = 0; i < n_requests; ++i)
      for (int e = req_ptr[i]; e < req_ptr[i + 1]; ++e)
        if (seen[req_adapters[e]] != i) {
          seen[req_adapters[e]] = i;
          L[i].push_back(req_adapters[e]);
        }
  }
  int64_t batch_adapters = 0;
  auto extra = [&](int i) {  // adapters of i not yet in the batch
    int64_t c = 0;
    for (int32_t a : L[i]) c += !in_batch[a];
    return c;
  };
  auto take = [&](int i) {
    taken[i] = 1;
    chosen[(*n_chosen)++] = i;
    for (int32_t a : L[i])
      if (!in_batch[a]) {
        in_batch[a] = 1;
        ++batch_adapters;
      }
  };
  std::vector<int32_t> old;
  for (int i = 0; i < n_requests; ++i)
    if (now - arrival[i] > theta) old.push_back(i);
  std::sort(old.begin(), old.end(), [&](int x, int y) {
    return arrival[x] != arrival[y] ? arrival[x] < arrival[y] : x < y;
  });
  for (int i : old)
    if (*n_chosen < max_batch && batch_adapters + extra(i) <= n_slots) take(i);
  while (*n_chosen < max_batch) {
    int best = -1;
    int64_t best_new = 0;
    for (int i = 0; i < n_requests; ++i) {
      if (taken[i] || batch_adapters + extra(i) > n_slots) continue;
      int64_t nw = 0;
      for (int32_t a : L[i]) nw += !res[a] && !in_batch[a];
      if (best < 0 || nw < best_new ||
          (nw == best_new && (arrival[i] < arrival[best] || (arrival[i] == arrival[best] && i < best)))) {
        best = i;
        best_new = nw;
      }
    }
    if (best < 0) break;
    take(best);
  }
  return TCL_OK;
}
