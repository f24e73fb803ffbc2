// Mapping stage of the composite multi-LoRA apply: composites -> tuples
// reordered by adapter id (DyMerge-LoRA summary page, section 4.3, the
// mapping step of the MAF-MVM kernel; the reorder by LoRA id is what lets one
// workgroup stream one adapter's factors over a contiguous token run).
//
// The stage validates the composite table, fixes each pair's slot (its
// position in its composite ordered by adapter id), expands the groups into
// (token, adapter, alpha, slot) tuples and sorts them stably by adapter id,
// then writes the segment table, the per-token tuple index (also as packed
// slot records for the expand), the shrink work items and, for batches with
// token tiles, the token order of the prefill expand's tiles.  Three
// algorithms give the same output bit for bit:
//   - direct (tables of at most 512 pairs, one workgroup, table in LDS):
//     every pair takes a ticket in its adapter's bucket through an LDS
//     atomic, and its rank within the adapter is then counted from the
//     bucket (the tokens of the bucket's pairs with a smaller pair index), so
//     the order of the tickets does not reach the output;
//   - multi-workgroup (larger tables): each workgroup counts and ranks the
//     pairs of 64 consecutive groups the same way, one scan over the
//     (adapter, workgroup) counts gives every workgroup its first position
//     per adapter, and a scatter writes the tuples;
//   - chunked counting sort (tables beyond the multi path's limits, one
//     workgroup): per-(adapter, chunk) histograms, one exclusive scan in
//     adapter-major order, then each chunk walks its pairs in order.
// Within an adapter, tuples therefore follow token order, which is the
// (adapter, token, slot) order because a token holds an adapter at most
// once.  The LDS atomics only hand out counts and tickets; no output depends
// on the order in which they land.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "plan_core.hpp"
#include "tcl_internal.hpp"

namespace tcl {

int hip_fail(hipError_t e, const char *what) {
  return fail(TCL_EHIP, "%s failed: %s", what, hipGetErrorString(e));
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// multi-workgroup mapping: groups per workgroup, pair capacity per workgroup
// (a valid table has at most TCL_MAX_PAIRS_PER_GROUP pairs per group), and
// the limits within which it is used
constexpr int kMgGroups = 64;
constexpr int kMgPairs = kMgGroups * TCL_MAX_PAIRS_PER_GROUP;
constexpr int kMgThreads = 256;
constexpr int kMultiMaxN = 4096;
constexpr int kMultiMaxBlocks = 128;
static_assert(kMultiMaxBlocks <= 4 * 32, "plan_m_scan: at most 32 workgroups a lane when G >= 4");


int plan_layout(int32_t T, int32_t G, int32_t NP, int32_t N, int32_t cap, PlanLayout *L) {
  const int64_t kLim = int64_t(1) << 24;
  if (T < 0 || G < 0 || NP < 0 || cap < 0)
    return fail(TCL_EINVAL, "negative size (tokens %d, groups %d, pairs %d, max_tuples %d)", T,
                G, NP, cap);
  if (N < 1) return fail(TCL_EINVAL, "n_adapters must be >= 1 (got %d)", N);
  if (T > kLim || G > kLim || NP > kLim || N > (1 << 20) || cap > (1 << 28))
    return fail(TCL_EINVAL, "size beyond 32-bit indexing limits");
  PlanLayout l{};
  l.T = T;
  l.G = G;
  l.NP = NP;
  l.N = N;
  l.cap = cap;
  l.items_cap = (cap < N ? cap : N) + cap / kTile + 1;

  // Direct path in LDS: gtp, gpp (G+1 each), group tuple base (G); adapter,
  // alpha, slot, group, tokens, ticket, bucket pair and bucket tokens (NP
  // each); tuple count, pair count, segment start, item base, segment index
  // and bucket start (N each).
  const int64_t direct_ints = 3 * int64_t(G) + 2 + 8 * int64_t(NP) + 6 * int64_t(N) + 16;
  // Counting path in LDS: the same without the last two pair arrays, plus
  // the (adapter, chunk) histogram.
  const int64_t fixed = 3 * int64_t(G) + 2 + 5 * int64_t(NP);
  const int64_t mblocks = (int64_t(G) + kMgGroups - 1) / kMgGroups;
  if (NP <= kDirectMaxPairs && direct_ints <= kPlanLdsInts) {
    l.mode = PLAN_DIRECT;
    l.threads = NP <= 256 ? 256 : kPlanThreads;
    l.chunks = 1;
  } else if (N <= kMultiMaxN && mblocks <= kMultiMaxBlocks) {
    l.mode = PLAN_MULTI;
    l.threads = kMgThreads;
    l.chunks = 1;
    l.blocks = int32_t(mblocks < 1 ? 1 : mblocks);
  } else {
    l.threads = kPlanThreads;
    int64_t c = (NP + 7) / 8;
    if (c > kPlanThreads) c = kPlanThreads;
    if (c < 1) c = 1;
    if (fixed + int64_t(N) * c <= kPlanLdsInts) {
      l.mode = PLAN_COUNT_LDS;
    } else {
      int64_t room = kPlanLdsInts - fixed;
      int64_t cl = room > 0 ? room / N : 0;
      if (cl >= 16 || (cl >= 1 && cl >= c)) {
        l.mode = PLAN_COUNT_LDS;
        c = cl < c ? cl : c;
      } else {
        l.mode = PLAN_COUNT_GLOBAL;
        int64_t cmax = 65536 / N;
        if (c > cmax) c = cmax;
        if (c < 1) c = 1;
      }
    }
    l.chunks = int32_t(c);
  }

  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  l.o_status = take(ST_WORDS * 4);
  l.o_tok = take(size_t(cap) * 4);
  l.o_ad = take(size_t(cap) * 4);
  l.o_slot = take(size_t(cap) * 4);
  l.o_alpha = take(size_t(cap) * 4);
  l.o_toktuple = take(size_t(cap) * 4);
  l.o_tokrec = take(size_t(T) * kSlotPad * 16);
  l.o_tokn = take(size_t(T) * 4);
  l.o_tokptr = take(size_t(T + 1) * 4);
  l.o_segad = take(size_t(N) * 4);
  l.o_segbeg = take(size_t(N + 1) * 4);
  l.o_items = take(size_t(l.items_cap) * sizeof(Item));
  l.o_sslot = take(size_t(NP) * 4);
  l.o_sgroup = take(size_t(NP) * 4);
  l.o_spos = take(size_t(NP) * 4);
  l.o_sgbase = take(size_t(G) * 4);
  l.o_shist = take(l.mode == PLAN_COUNT_GLOBAL ? size_t(N) * size_t(l.chunks) * 4 : 4);
  l.o_sseg = take(l.mode == PLAN_DIRECT ? 4 : size_t(N) * 4);
  const bool multi = l.mode == PLAN_MULTI;
  l.o_mhist = take(multi ? size_t(N) * size_t(l.blocks) * 4 : 4);
  l.o_mblk = take(multi ? size_t(l.blocks) * 16 : 4);
  l.o_msst = take(multi ? size_t(N) * 4 : 4);
  l.o_msib = take(multi ? size_t(N) * 4 : 4);
  l.tiles = T >= kMfmaMinTokens ? (T + kXTok - 1) / kXTok : 0;
  // tile order: per workgroup of its flagging launch the count of flagged
  // tokens, and a slice of kOrdThreads entries listing them
  const size_t ob = size_t(ord_blocks(cap));
  l.o_ocnt = take(l.tiles ? ob * 4 : 4);
  l.o_oitem = take(l.tiles ? ob * kOrdThreads * 4 : 4);
  // device copy of a host-resident composite table: group_tok_ptr,
  // group_pair_ptr (G + 1 each), pair_adapter, pair_alpha (NP each)
  l.o_tab = take((2 * size_t(G) + 2 + 2 * size_t(NP)) * 4);
  l.total = o;
  *L = l;
  return TCL_OK;
}

// Token order of the prefill expand's 64-token tiles: the tokens that hold
// at least one pair, grouped by their rarest adapter (the last of their
// slots, adapters ascending), adapters ascending, in token order within an
// adapter.  Tokens that share their rarest adapter then share a tile, which
// shrinks the tiles' unions (the adapters whose B rows a tile reads): their
// other adapters are the more common ones, in many tiles whatever the order.
// In (adapter, token) order these tokens are the tuples of the sorted plan
// that are their token's last slot.  (Keeping the tokens whose rarest
// adapter is common in token order, as before, left the retained-rank
// batch's expand 20 us slower; the sparse prefill, whose requests already
// share adapters in token order, is 0.5-0.9 us slower grouped.)
// One launch over the tuples, one a thread: it flags each token's last slot
// and writes each workgroup's flagged tokens, in order, at the start of its
// kOrdThreads-entry slice of ord_item, and their count in ord_cnt.  Position
// i of the tile order is then entry i - (tokens of the earlier workgroups)
// of the workgroup whose tokens cover i: tile_prep finds the 64 entries of
// its tile from the counts.

// tuple i (in sorted order) when it is its token's last slot: the token
__device__ inline bool ord_flag(const PlanDev &d, int P, int *item) {
  const int i = blockIdx.x * kOrdThreads + threadIdx.x;
  if (i >= P) return false;
  const int t = d.tup_token[i], sl = d.tup_slot[i];
  *item = t;
  return sl >= 0 && sl < kSlotPad && sl == d.tok_n[t] - 1;
}

__global__ __launch_bounds__(kOrdThreads) void tile_order_count(PlanDev d) {
  __shared__ int tmp[kOrdThreads / 64];
  const bool ok = d.status[ST_CODE] == TCL_OK;
  const int P = ok ? d.status[ST_TUPLES] : 0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int item = 0;
  const bool f = ok && ord_flag(d, P, &item);
  const uint64_t m = __ballot(f);
  if (lane == 0) tmp[w] = __popcll(m);
  __syncthreads();
  int wb = 0, c = 0;
#pragma unroll
  for (int j = 0; j < kOrdThreads / 64; ++j) {
    wb += j < w ? tmp[j] : 0;
    c += tmp[j];
  }
  if (f) d.ord_item[blockIdx.x * kOrdThreads + wb + __popcll(m & ((uint64_t(1) << lane) - 1))] = item;
  if (threadIdx.x == 0) d.ord_cnt[blockIdx.x] = c;
}

// ---------------------------------------------------------------------------
// mapping of larger tables over many workgroups (PLAN_MULTI)
// ---------------------------------------------------------------------------
// Workgroup b owns the kMgGroups consecutive groups starting at b*kMgGroups,
// so earlier workgroups hold earlier tokens and the (adapter, token, slot)
// order of the result is that of the single-workgroup paths.
//   plan_m_local   checks its groups and pairs, computes slots, counts tuples
//                  per adapter, and ranks every pair among the earlier pairs
//                  of the same adapter in the workgroup (tickets into
//                  per-adapter buckets, as in the direct path);
//   plan_m_scan    (one workgroup) combines the workgroups' error bits and
//                  tuple totals, turns the per-(adapter, workgroup) counts
//                  into prefixes, and builds the segment table, the work
//                  items and the status words;
//   plan_m_scatter writes the tuples and the token index.  A pair's first
//                  tuple goes to (segment start of its adapter) + (tuples of
//                  that adapter in earlier workgroups) + (its rank).
struct MArgs {
  int32_t T, G, NP, N, cap, items_cap, NB;
  const int32_t *gtp, *gpp, *pa;
  const float *pw;
  PlanDev d;
};

// LDS of plan_m_local: six pair arrays of kMgPairs ints and two adapter arrays
static size_t m_local_lds_bytes(int N) {
  return (size_t(6) * kMgPairs + 2 * size_t(N) + 2 + 2 * (kMgGroups + 1) + 4 * kSlotInts) * 4;
}
static size_t lds_max_bytes() { return m_local_lds_bytes(kMultiMaxN); }

__global__ __launch_bounds__(kMgThreads) void plan_m_local(MArgs A) {
  extern __shared__ __align__(16) int m_lds[];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int T = A.T, G = A.G, NP = A.NP, N = A.N;
  int *l_pa = m_lds, *l_ptl = l_pa + kMgPairs, *l_grp = l_ptl + kMgPairs;
  int *l_tkt = l_grp + kMgPairs, *l_bkt = l_tkt + kMgPairs, *l_bkw = l_bkt + kMgPairs;
  int *l_cnt = l_bkw + kMgPairs;  // tuples per adapter
  int *l_pst = l_cnt + N;         // pairs per adapter, then bucket starts [N + 1]
  int *l_gtp = l_pst + N + 1, *l_gpp = l_gtp + kMgGroups + 1;
  int *tmp = l_gpp + kMgGroups + 1;

  const int g0 = min(G, b * kMgGroups), g1 = min(G, g0 + kMgGroups), ng = g1 - g0;
  if (tid <= ng) {
    l_gtp[tid] = A.gtp[g0 + tid];
    l_gpp[tid] = A.gpp[g0 + tid];
  }
  for (int a = tid; a < N; a += kMgThreads) {
    l_cnt[a] = 0;
    l_pst[a] = 0;
  }
  __syncthreads();

  // ---- groups
  int err = 0;
  if (b == 0 && tid == 0 &&
      (A.gtp[0] != 0 || A.gtp[G] != T || A.gpp[0] != 0 || A.gpp[G] > NP))
    err |= EB_INVAL;
  int gtup = 0;
  if (tid < ng) {
    const int t0 = l_gtp[tid], t1 = l_gtp[tid + 1], q0 = l_gpp[tid], q1 = l_gpp[tid + 1];
    if (!(0 <= t0 && t0 <= t1 && t1 <= T && 0 <= q0 && q0 <= q1 && q1 <= NP)) err |= EB_INVAL;
    else if (q1 - q0 > TCL_MAX_PAIRS_PER_GROUP) err |= EB_UNSUP;
    else gtup = (t1 - t0) * (q1 - q0);
  }
  int P_b;
  block_excl_scan<kMgThreads>(gtup, tmp + 0 * kSlotInts, &P_b);
  const int err_g = block_or<kMgThreads>(err, tmp + 1 * kSlotInts);
  const int qb0 = l_gpp[0];
  const int span = (err_g & EB_INVAL) ? 0 : l_gpp[ng] - qb0;
  if ((err_g & EB_INVAL) || span > kMgPairs || (err_g & EB_UNSUP)) {
    // the table is rejected: only look for invalid ids and weights (an
    // EINVAL outranks the other codes)
    err = err_g;
    if (!(err_g & EB_INVAL)) {
      for (int q = qb0 + tid; q < qb0 + span; q += kMgThreads) {
        const int aq = A.pa[q];
        if (aq < 0 || aq >= N) err |= EB_INVAL;
        if ((__float_as_uint(A.pw[q]) & 0x7f800000u) == 0x7f800000u) err |= EB_INVAL;
      }
      // duplicates in the groups within the pair limit
      if (tid < ng) {
        const int q0 = l_gpp[tid], q1 = l_gpp[tid + 1];
        if (q1 - q0 <= TCL_MAX_PAIRS_PER_GROUP)
          for (int q = q0; q < q1; ++q)
            for (int q2 = q + 1; q2 < q1; ++q2)
              if (A.pa[q] == A.pa[q2]) err |= EB_INVAL;
      }
    }
    err = block_or<kMgThreads>(err, tmp + 2 * kSlotInts);
    if (tid == 0) {
      A.d.m_blk[4 * b] = 0;
      A.d.m_blk[4 * b + 1] = err;
    }
    return;
  }

  // ---- pairs: stage, group index, checks, slots, counts and tickets
  for (int i = tid; i < span; i += kMgThreads) l_pa[i] = A.pa[qb0 + i];
  if (tid < ng) {
    const int q0 = l_gpp[tid] - qb0, q1 = l_gpp[tid + 1] - qb0;
    const int tl = l_gtp[tid + 1] - l_gtp[tid];
    for (int q = q0; q < q1; ++q) {
      l_grp[q] = tid;
      l_ptl[q] = tl;
    }
  }
  __syncthreads();
  err = 0;
  for (int i = tid; i < span; i += kMgThreads) {
    const int aq = l_pa[i];
    const bool a_ok = aq >= 0 && aq < N;
    if (!a_ok) err |= EB_INVAL;
    if ((__float_as_uint(A.pw[qb0 + i]) & 0x7f800000u) == 0x7f800000u) err |= EB_INVAL;
    const int g = l_grp[i];
    const int q0 = l_gpp[g] - qb0, q1 = l_gpp[g + 1] - qb0;
    int sl = 0, dup = 0;
    for (int q2 = q0; q2 < q1; q2 += 8) {
      int av[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) av[u] = q2 + u < q1 ? l_pa[q2 + u] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = q2 + u < q1;
        sl += (in && av[u] < aq) ? 1 : 0;
        dup |= (in && av[u] == aq && q2 + u != i) ? 1 : 0;
      }
    }
    if (dup) err |= EB_INVAL;
    A.d.s_slot[qb0 + i] = sl;
    if (a_ok) {
      atomicAdd(&l_cnt[aq], l_ptl[i]);
      l_tkt[i] = atomicAdd(&l_pst[aq], 1);
    }
  }
  err = block_or<kMgThreads>(err, tmp + 2 * kSlotInts);
  if (err) {
    if (tid == 0) {
      A.d.m_blk[4 * b] = 0;
      A.d.m_blk[4 * b + 1] = err;
    }
    return;
  }

  // ---- bucket starts (exclusive scan of the pair counts, in place)
  {
    const int per = (N + kMgThreads - 1) / kMgThreads;
    const int a0 = min(N, tid * per), a1 = min(N, a0 + per);
    int sum = 0;
    for (int a = a0; a < a1; ++a) sum += l_pst[a];
    int tot;
    int run = block_excl_scan<kMgThreads>(sum, tmp + 3 * kSlotInts, &tot);
    for (int a = a0; a < a1; ++a) {
      const int c = l_pst[a];
      l_pst[a] = run;
      run += c;
    }
    if (tid == 0) l_pst[N] = tot;
  }
  __syncthreads();
  for (int i = tid; i < span; i += kMgThreads) {
    const int e = l_pst[l_pa[i]] + l_tkt[i];
    l_bkt[e] = i;
    l_bkw[e] = l_ptl[i];
  }
  __syncthreads();
  // ---- rank: tuples of the same adapter's earlier pairs in this workgroup
  for (int i = tid; i < span; i += kMgThreads) {
    const int a = l_pa[i];
    const int b0 = l_pst[a], b1 = l_pst[a + 1];
    int r = 0;
    for (int e = b0; e < b1; e += 8) {
      int qq[8], ww[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        qq[u] = e + u < b1 ? l_bkt[e + u] : kMgPairs;
        ww[u] = e + u < b1 ? l_bkw[e + u] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) r += qq[u] < i ? ww[u] : 0;
    }
    A.d.s_pos[qb0 + i] = r;
  }
  for (int a = tid; a < N; a += kMgThreads) A.d.m_hist[int64_t(b) * N + a] = l_cnt[a];
  if (tid == 0) {
    A.d.m_blk[4 * b] = P_b;
    A.d.m_blk[4 * b + 1] = 0;
  }
}

// Orders the workgroup's LDS accesses around a barrier without waiting for
// its outstanding global stores (a plain __syncthreads() waits for those too).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__global__ __launch_bounds__(kPlanThreads) void plan_m_scan(MArgs A) {
  constexpr int NT = kPlanThreads;
  __shared__ int tmp[6 * kSlotInts];
  __shared__ int s_tot[kMultiMaxN];
  __shared__ int s_ib[kMultiMaxN], s_ec[kMultiMaxN], s_en[kMultiMaxN];  // per adapter
  const int tid = threadIdx.x, NB = A.NB, N = A.N;
  // ---- workgroup totals and error bits (NB <= kMultiMaxBlocks <= NT)
  int pb = 0, err = 0;
  if (tid < NB) {
    pb = A.d.m_blk[4 * tid];
    err = A.d.m_blk[4 * tid + 1];
  }
  int P;
  const int base = block_excl_scan<NT>(pb, tmp + 0 * kSlotInts, &P);
  if (tid < NB) A.d.m_blk[4 * tid + 2] = base;
  err = block_or<NT>(err, tmp + 1 * kSlotInts);
  const int code = (err & EB_INVAL) ? TCL_EINVAL
                 : (err & EB_UNSUP) ? TCL_EUNSUPPORTED
                 : (P > A.cap) ? TCL_ENOSPC : TCL_OK;
  if (code != TCL_OK) {
    if (tid == 0) {
      A.d.status[ST_CODE] = code;
      A.d.status[ST_TUPLES] = code == TCL_ENOSPC ? P : 0;
      A.d.status[ST_SEGMENTS] = 0;
      A.d.status[ST_ITEMS] = 0;
    }
    return;
  }
  // ---- per adapter: prefix over workgroups (in place) and total.  The
  //      counts are stored workgroup-major ([NB][N]), so for each workgroup
  //      the threads read consecutive adapters.  Pools of at most NT / 4
  //      adapters: G >= 4 consecutive lanes share an adapter, each loading
  //      its <= 32 workgroups' counts in one round, a scan across the group
  //      giving each lane its offset; larger pools: a lane per adapter, 32
  //      rows at a time (each batch of loads then waits for the stores
  //      before it).
  int G = 1;
  while (G < 64 && 2 * G * N <= NT) G *= 2;
  if (G >= 4) {
    const int a = tid / G, sub = tid & (G - 1);
    const int per = (NB + G - 1) / G;  // <= kMultiMaxBlocks / 4 = 32
    const int b0 = sub * per, b1 = min(NB, b0 + per);
    // rows b0 .. b1 - 1 of this adapter's column, through a pointer that
    // steps by N (offsets u * N kept as constants would each take scalar
    // registers)
    int32_t *const h0 = A.d.m_hist + (a < N ? a : 0) + int64_t(b0) * N;
    int v[32], sum = 0;
    {
      const int32_t *q = h0;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        v[u] = a < N && b0 + u < b1 ? *q : 0;
        sum += v[u];
        q += N;
      }
    }
    int inc = sum;
    for (int off = 1; off < G; off <<= 1) {
      const int t = __shfl_up(inc, off, 64);
      if (sub >= off) inc += t;
    }
    int run = inc - sum;
    if (a < N) {
      int32_t *q = h0;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        if (b0 + u < b1) *q = run;
        run += v[u];
        q += N;
      }
      if (sub == G - 1) s_tot[a] = run;
    }
  } else {
    for (int a = tid; a < N; a += NT) {
      int32_t *h = A.d.m_hist + a;
      int run = 0;
      for (int b0 = 0; b0 < NB; b0 += 32) {
        int v[32];
        const int32_t *q = h + int64_t(b0) * N;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          v[u] = b0 + u < NB ? *q : 0;
          q += N;
        }
        int32_t *o = h + int64_t(b0) * N;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          if (b0 + u < NB) *o = run;
          run += v[u];
          o += N;
        }
      }
      s_tot[a] = run;
    }
  }
  // s_tot complete; the prefixes stored to m_hist are the scatter kernel's
  // (no need to wait for them here)
  lds_barrier();
  // ---- segments and work items: one scan over adapters
  const int per = (N + NT - 1) / NT;
  const int a0 = min(N, tid * per), a1 = min(N, a0 + per);
  int sv[3] = {0, 0, 0}, st[3];
  for (int a = a0; a < a1; ++a) {
    const int c = s_tot[a];
    sv[0] += c;
    sv[1] += c > 0;
    sv[2] += (c + kTile - 1) / kTile;
  }
  block_excl_scan_n<NT, 3>(sv, tmp + 2 * kSlotInts, st);
  int ec = sv[0], en = sv[1], ei = sv[2];
  for (int a = a0; a < a1; ++a) {
    const int c = s_tot[a];
    A.d.m_sst[a] = ec;
    A.d.m_sib[a] = ei;
    A.d.s_seg[a] = en;
    s_ib[a] = ei;
    s_ec[a] = ec;
    s_en[a] = en;
    if (c > 0) {
      A.d.seg_adapter[en] = a;
      A.d.seg_begin[en] = ec;
      ++en;
      ei += (c + kTile - 1) / kTile;
    }
    ec += c;
  }
  lds_barrier();  // the per-adapter arrays in LDS (global stores may still be in flight)
  // work-item heads, one thread per item: the item's adapter is the last one
  // whose first item is at or before it (adapters without tuples own none)
  const int n_items = min(st[2], A.items_cap);
  for (int i = tid; i < n_items; i += NT) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_ib[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int a = lo, c = s_tot[a], j = i - s_ib[a];
    const int p0 = s_ec[a] + j * kTile;
    A.d.items[i].head = make_int4(a, p0, min(c - j * kTile, kTile), s_en[a]);
  }
  if (tid == 0) {
    A.d.seg_begin[st[1]] = P;
    A.d.status[ST_TUPLES] = P;
    A.d.status[ST_SEGMENTS] = st[1];
    A.d.status[ST_ITEMS] = st[2];
    A.d.status[ST_CODE] = TCL_OK;
  }
}

__global__ __launch_bounds__(kMgThreads) void plan_m_scatter(MArgs A) {
  __shared__ int l_gtp[kMgGroups + 1], l_gpp[kMgGroups + 1], l_gbase[kMgGroups];
  __shared__ int l_grp[kMgPairs];
  __shared__ int tmp[kSlotInts];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int T = A.T, G = A.G, NB = A.NB;
  if (A.d.status[ST_CODE] != TCL_OK) {
    // rejected: an empty token index, so that every later kernel is a no-op
    const int tper = (T + NB - 1) / NB;
    const int t0 = min(T, b * tper), t1 = min(T, t0 + tper);
    for (int t = t0 + tid; t < t1; t += kMgThreads) {
      A.d.tok_ptr[t] = 0;
      A.d.tok_n[t] = 0;
    }
    if (b == 0 && tid == 0) A.d.tok_ptr[T] = 0;
    return;
  }
  const int g0 = min(G, b * kMgGroups), g1 = min(G, g0 + kMgGroups), ng = g1 - g0;
  if (tid <= ng) {
    l_gtp[tid] = A.gtp[g0 + tid];
    l_gpp[tid] = A.gpp[g0 + tid];
  }
  __syncthreads();
  // group tuple bases and the token index
  const int gtup =
      tid < ng ? (l_gtp[tid + 1] - l_gtp[tid]) * (l_gpp[tid + 1] - l_gpp[tid]) : 0;
  int unused;
  const int gb = block_excl_scan<kMgThreads>(gtup, tmp, &unused) + A.d.m_blk[4 * b + 2];
  const int qb0 = l_gpp[0];
  if (tid < ng) {
    const int t0 = l_gtp[tid], t1 = l_gtp[tid + 1], q0 = l_gpp[tid], q1 = l_gpp[tid + 1];
    const int pl = q1 - q0;
    l_gbase[tid] = gb;
    for (int q = q0; q < q1; ++q) l_grp[q - qb0] = tid;
    for (int t = t0; t < t1; ++t) {
      A.d.tok_ptr[t] = gb + (t - t0) * pl;
      A.d.tok_n[t] = pl;
    }
  }
  if (b == NB - 1 && tid == 0) A.d.tok_ptr[T] = A.d.status[ST_TUPLES];
  __syncthreads();
  const int span = l_gpp[ng] - qb0;
  for (int i = tid; i < span; i += kMgThreads) {
    const int q = qb0 + i;
    const int g = l_grp[i];
    const int t0 = l_gtp[g], tl = l_gtp[g + 1] - t0, pl = l_gpp[g + 1] - l_gpp[g];
    const int a = A.pa[q], s = A.d.s_slot[q], gbase = l_gbase[g];
    const float w = A.pw[q];
    const int sst = A.d.m_sst[a];
    const int base = sst + A.d.m_hist[int64_t(b) * A.N + a] + A.d.s_pos[q];
    const int sg = A.d.s_seg[a], sib = A.d.m_sib[a];
    for (int k = 0; k < tl; ++k) {
      const int p = base + k;
      // positions are < P <= cap by construction; the guards keep a logic
      // error from writing outside the plan buffer
      if (p >= A.cap || gbase + k * pl + s >= A.cap || s >= kSlotPad) continue;
      A.d.tup_token[p] = t0 + k;
      A.d.tup_adapter[p] = a;
      A.d.tup_alpha[p] = w;
      A.d.tup_slot[p] = s;
      A.d.tok_tuple[gbase + k * pl + s] = p;
      A.d.tok_rec[int64_t(t0 + k) * kSlotPad + s] = make_int4(p, a, __float_as_int(w), sg);
      const int local = p - sst;
      const int it = sib + local / kTile;
      if (it < A.items_cap) A.d.items[it].tok[local % kTile] = t0 + k;
    }
  }
}

static int launch_plan_multi(tcl_plan *p, const tcl_composites *c, hipStream_t s) {
  MArgs A;
  A.T = p->L.T;
  A.G = p->L.G;
  A.NP = p->L.NP;
  A.N = p->L.N;
  A.cap = p->L.cap;
  A.items_cap = p->L.items_cap;
  A.NB = p->L.blocks;
  A.gtp = c->group_tok_ptr;
  A.gpp = c->group_pair_ptr;
  A.pa = c->pair_adapter;
  A.pw = c->pair_alpha;
  A.d = p->d;
  const size_t lds = m_local_lds_bytes(A.N);
  static bool attr_set = false;
  if (!attr_set) {
    TCL_HIP(hipFuncSetAttribute(reinterpret_cast<const void *>(plan_m_local),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_max_bytes())));
    attr_set = true;
  }
  logf("plan(multi): T=%d G=%d pairs=%d N=%d workgroups=%d lds=%zu", A.T, A.G, A.NP, A.N, A.NB,
       lds);
  hipLaunchKernelGGL(plan_m_local, dim3(A.NB), dim3(kMgThreads), lds, s, A);
  hipLaunchKernelGGL(plan_m_scan, dim3(1), dim3(kPlanThreads), 0, s, A);
  hipLaunchKernelGGL(plan_m_scatter, dim3(A.NB), dim3(kMgThreads), 0, s, A);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

static void bind(tcl_plan *p) {
  char *b = static_cast<char *>(p->buf);
  const PlanLayout &L = p->L;
  PlanDev &d = p->d;
  d.status = reinterpret_cast<int32_t *>(b + L.o_status);
  d.tup_token = reinterpret_cast<int32_t *>(b + L.o_tok);
  d.tup_adapter = reinterpret_cast<int32_t *>(b + L.o_ad);
  d.tup_slot = reinterpret_cast<int32_t *>(b + L.o_slot);
  d.tup_alpha = reinterpret_cast<float *>(b + L.o_alpha);
  d.tok_tuple = reinterpret_cast<int32_t *>(b + L.o_toktuple);
  d.tok_ptr = reinterpret_cast<int32_t *>(b + L.o_tokptr);
  d.tok_rec = reinterpret_cast<int4 *>(b + L.o_tokrec);
  d.tok_n = reinterpret_cast<int32_t *>(b + L.o_tokn);
  d.seg_adapter = reinterpret_cast<int32_t *>(b + L.o_segad);
  d.seg_begin = reinterpret_cast<int32_t *>(b + L.o_segbeg);
  d.items = reinterpret_cast<Item *>(b + L.o_items);
  d.s_slot = reinterpret_cast<int32_t *>(b + L.o_sslot);
  d.s_group = reinterpret_cast<int32_t *>(b + L.o_sgroup);
  d.s_pos = reinterpret_cast<int32_t *>(b + L.o_spos);
  d.s_gbase = reinterpret_cast<int32_t *>(b + L.o_sgbase);
  d.s_hist = reinterpret_cast<int32_t *>(b + L.o_shist);
  d.s_seg = reinterpret_cast<int32_t *>(b + L.o_sseg);
  d.m_hist = reinterpret_cast<int32_t *>(b + L.o_mhist);
  d.m_blk = reinterpret_cast<int32_t *>(b + L.o_mblk);
  d.m_sst = reinterpret_cast<int32_t *>(b + L.o_msst);
  d.m_sib = reinterpret_cast<int32_t *>(b + L.o_msib);
  d.ord_cnt = reinterpret_cast<int32_t *>(b + L.o_ocnt);
  d.ord_item = reinterpret_cast<int32_t *>(b + L.o_oitem);
}

void plan_fill_args(const tcl_plan *p, const tcl_composites *c, PlanArgs *out) {
  PlanArgs &A = *out;
  A.T = p->L.T;
  A.G = p->L.G;
  A.NP = p->L.NP;
  A.N = p->L.N;
  A.cap = p->L.cap;
  A.C = p->L.chunks;
  A.mode = p->L.mode;
  A.items_cap = p->L.items_cap;
  A.gtp = c->group_tok_ptr;
  A.gpp = c->group_pair_ptr;
  A.pa = c->pair_adapter;
  A.pw = c->pair_alpha;
  A.d = p->d;
}

int plan_direct_lds_ints(const tcl_plan *p) {
  return 8 * p->L.NP + 3 * p->L.G + 2 + 6 * p->L.N;
}

static int launch_plan(tcl_plan *p, const tcl_composites *c, hipStream_t s) {
  PlanArgs A;
  A.T = p->L.T;
  A.G = p->L.G;
  A.NP = p->L.NP;
  A.N = p->L.N;
  A.cap = p->L.cap;
  A.C = p->L.chunks;
  A.mode = p->L.mode;
  A.items_cap = p->L.items_cap;
  A.gtp = c->group_tok_ptr;
  A.gpp = c->group_pair_ptr;
  A.pa = c->pair_adapter;
  A.pw = c->pair_alpha;
  A.d = p->d;
  if (A.mode == PLAN_MULTI) {
    int rc = launch_plan_multi(p, c, s);
    if (rc) return rc;
    return plan_launch_tile_order(p, s);
  }
  logf("plan: T=%d G=%d pairs=%d N=%d cap=%d chunks=%d mode=%d threads=%d", A.T, A.G, A.NP, A.N,
       A.cap, A.C, A.mode, p->L.threads);
  if (A.mode == PLAN_DIRECT && p->L.threads == 64)
    hipLaunchKernelGGL((plan_kernel<64, PLAN_DIRECT>), dim3(1), dim3(64), 0, s, A);
  else if (A.mode == PLAN_DIRECT)
    hipLaunchKernelGGL((plan_kernel<256, PLAN_DIRECT>), dim3(1), dim3(256), 0, s, A);
  else if (A.mode == PLAN_COUNT_LDS)
    hipLaunchKernelGGL((plan_kernel<kPlanThreads, PLAN_COUNT_LDS>), dim3(1), dim3(kPlanThreads),
                       0, s, A);
  else
    hipLaunchKernelGGL((plan_kernel<kPlanThreads, PLAN_COUNT_GLOBAL>), dim3(1),
                       dim3(kPlanThreads), 0, s, A);
  TCL_HIP(hipGetLastError());
  return plan_launch_tile_order(p, s);
}

int plan_remap_prepare(const tcl_plan *p, const tcl_composites *c, tcl_plan *next) {
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  int rc = check_composites(c);
  if (rc) return rc;
  PlanLayout L;
  rc = plan_layout(c->n_tokens, c->n_groups, c->n_pairs, c->n_adapters, c->max_tuples, &L);
  if (rc) return rc;
  if (L.total > p->buf_bytes)
    return fail(TCL_ENOSPC, "plan buffer holds %zu bytes, needs %zu", p->buf_bytes, L.total);
  *next = *p;
  next->L = L;
  next->host_tuples = next->host_segments = -1;
  bind(next);
  return TCL_OK;
}

int plan_launch(tcl_plan *p, const tcl_composites *c, hipStream_t s) { return launch_plan(p, c, s); }

int plan_launch_tile_order(const tcl_plan *p, hipStream_t s) {
  if (p->L.tiles == 0) return TCL_OK;
  hipLaunchKernelGGL(tile_order_count, dim3(ord_blocks(p->L.cap)), dim3(kOrdThreads), 0, s, p->d);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

// The plan's status words {code, tuples, segments, work items} into a
// caller's device array, in stream order.
__global__ void status_copy_kernel(const int32_t *status, int32_t *out) {
  if (threadIdx.x < 4) out[threadIdx.x] = status[threadIdx.x];
}

// Copies the validated host table c into the plan buffer's table region
// through the plan's pinned staging buffer and points *dc at the device copy.
// The staging buffer is reused by the next host table once the previous copy
// has finished (its event).
static int stage_table(tcl_plan *p, const tcl_composites *c, hipStream_t s, tcl_composites *dc) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  TCL_HIP(hipStreamIsCapturing(s, &cs));
  if (cs != hipStreamCaptureStatusNone)
    return fail(TCL_EUNSUPPORTED, "host-resident tables are copied when called; they cannot "
                                  "be captured into a graph (use a device-resident table)");
  const size_t G = size_t(c->n_groups), NP = size_t(c->n_pairs);
  const size_t bytes = (2 * G + 2 + 2 * NP) * 4;
  if (p->stage_pending) {
    TCL_HIP(hipEventSynchronize(p->stage_ev));
    p->stage_pending = false;
  }
  if (!p->stage_ev) TCL_HIP(hipEventCreateWithFlags(&p->stage_ev, hipEventDisableTiming));
  if (p->stage_bytes < bytes) {
    if (p->stage) TCL_HIP(hipHostFree(p->stage));
    p->stage = nullptr;
    p->stage_bytes = 0;
    TCL_HIP(hipHostMalloc(&p->stage, bytes, hipHostMallocDefault));
    p->stage_bytes = bytes;
  }
  int32_t *h = static_cast<int32_t *>(p->stage);
  std::memcpy(h, c->group_tok_ptr, (G + 1) * 4);
  std::memcpy(h + G + 1, c->group_pair_ptr, (G + 1) * 4);
  if (NP) {
    std::memcpy(h + 2 * G + 2, c->pair_adapter, NP * 4);
    std::memcpy(h + 2 * G + 2 + NP, c->pair_alpha, NP * 4);
  }
  int32_t *d = reinterpret_cast<int32_t *>(static_cast<char *>(p->buf) + p->L.o_tab);
  TCL_HIP(hipMemcpyAsync(d, h, bytes, hipMemcpyHostToDevice, s));
  TCL_HIP(hipEventRecord(p->stage_ev, s));
  p->stage_pending = true;
  *dc = *c;
  dc->group_tok_ptr = d;
  dc->group_pair_ptr = d + G + 1;
  dc->pair_adapter = d + 2 * G + 2;
  dc->pair_alpha = reinterpret_cast<const float *>(d + 2 * G + 2 + NP);
  return TCL_OK;
}

}  // namespace tcl

using namespace tcl;

extern "C" {

int tcl_plan_map_host(const tcl_composites *c, void *dev_buf, size_t dev_bytes, void *stream,
                      tcl_plan **out) {
  if (!out) return fail(TCL_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_composites(c);
  if (rc) return rc;
  int64_t P = 0;
  int32_t U = 0;
  if ((rc = validate_host(c, &P, &U))) return rc;
  PlanLayout L;
  rc = plan_layout(c->n_tokens, c->n_groups, c->n_pairs, c->n_adapters, c->max_tuples, &L);
  if (rc) return rc;
  if (!dev_buf) return fail(TCL_EINVAL, "plan buffer is NULL");
  if (reinterpret_cast<uintptr_t>(dev_buf) & 255)
    return fail(TCL_EALIGN, "plan buffer must be 256-byte aligned");
  if (dev_bytes < L.total)
    return fail(TCL_ENOSPC, "plan buffer holds %zu bytes, needs %zu", dev_bytes, L.total);
  tcl_plan *p = new (std::nothrow) tcl_plan;
  if (!p) return fail(TCL_EINVAL, "out of host memory");
  p->L = L;
  p->buf = dev_buf;
  p->buf_bytes = dev_bytes;
  bind(p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  tcl_composites dc;
  rc = stage_table(p, c, s, &dc);
  if (!rc) rc = launch_plan(p, &dc, s);
  if (rc) {
    tcl_plan_free(p);
    return rc;
  }
  p->host_tuples = int32_t(P);
  p->host_segments = U;
  *out = p;
  return TCL_OK;
}

int tcl_plan_remap_host(tcl_plan *p, const tcl_composites *c, void *stream) {
  int rc = check_composites(c);
  if (rc) return rc;
  int64_t P = 0;
  int32_t U = 0;
  if ((rc = validate_host(c, &P, &U))) return rc;
  tcl_plan next;
  if ((rc = plan_remap_prepare(p, c, &next))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  *p = next;
  tcl_composites dc;
  p->host_tuples = p->host_segments = -1;
  if ((rc = stage_table(p, c, s, &dc))) return rc;
  if ((rc = launch_plan(p, &dc, s))) return rc;
  p->host_tuples = int32_t(P);
  p->host_segments = U;
  return TCL_OK;
}

int tcl_plan_info(const tcl_plan *p, int32_t *n_tuples, int32_t *n_segments) {
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  if (p->host_tuples < 0)
    return fail(TCL_EUNSUPPORTED, "the plan was mapped from a device-resident table: its "
                                  "counts are on the device (tcl_plan_status, "
                                  "tcl_plan_status_async)");
  if (n_tuples) *n_tuples = p->host_tuples;
  if (n_segments) *n_segments = p->host_segments;
  return TCL_OK;
}

int tcl_plan_status_async(const tcl_plan *p, int32_t *dev_status, void *stream) {
  if (!p || !dev_status) return fail(TCL_EINVAL, "plan and dev_status are required");
  if (reinterpret_cast<uintptr_t>(dev_status) & 3)
    return fail(TCL_EALIGN, "dev_status must be 4-byte aligned");
  hipLaunchKernelGGL(status_copy_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     p->d.status, dev_status);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

const char *tcl_version(void) { return "tclora 0.1 gfx950"; }

int tcl_plan_bytes(int32_t n_tokens, int32_t n_groups, int32_t n_pairs, int32_t n_adapters,
                   int32_t max_tuples, size_t *bytes) {
  if (!bytes) return fail(TCL_EINVAL, "bytes is NULL");
  PlanLayout L;
  int rc = plan_layout(n_tokens, n_groups, n_pairs, n_adapters, max_tuples, &L);
  if (rc) return rc;
  *bytes = L.total;
  return TCL_OK;
}

int tcl_plan_map(const tcl_composites *c, void *dev_buf, size_t dev_bytes, void *stream,
                 tcl_plan **out) {
  if (!out) return fail(TCL_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_composites(c);
  if (rc) return rc;
  PlanLayout L;
  rc = plan_layout(c->n_tokens, c->n_groups, c->n_pairs, c->n_adapters, c->max_tuples, &L);
  if (rc) return rc;
  if (!dev_buf) return fail(TCL_EINVAL, "plan buffer is NULL");
  if (reinterpret_cast<uintptr_t>(dev_buf) & 255)
    return fail(TCL_EALIGN, "plan buffer must be 256-byte aligned");
  if (dev_bytes < L.total)
    return fail(TCL_ENOSPC, "plan buffer holds %zu bytes, needs %zu", dev_bytes, L.total);
  tcl_plan *p = new (std::nothrow) tcl_plan;
  if (!p) return fail(TCL_EINVAL, "out of host memory");
  p->L = L;
  p->buf = dev_buf;
  p->buf_bytes = dev_bytes;
  bind(p);
  rc = launch_plan(p, c, static_cast<hipStream_t>(stream));
  if (rc) {
    delete p;
    return rc;
  }
  *out = p;
  return TCL_OK;
}

int tcl_plan_remap(tcl_plan *p, const tcl_composites *c, void *stream) {
  tcl_plan next;
  int rc = plan_remap_prepare(p, c, &next);
  if (rc) return rc;
  *p = next;
  return launch_plan(p, c, static_cast<hipStream_t>(stream));
}

int tcl_plan_status(const tcl_plan *p, void *stream, int32_t *n_tuples, int32_t *n_segments) {
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  int32_t st[4];
  hipStream_t s = static_cast<hipStream_t>(stream);
  TCL_HIP(hipMemcpyAsync(st, p->d.status, sizeof st, hipMemcpyDeviceToHost, s));
  TCL_HIP(hipStreamSynchronize(s));
  if (n_tuples) *n_tuples = st[ST_TUPLES];
  if (n_segments) *n_segments = st[ST_SEGMENTS];
  if (st[ST_CODE] != TCL_OK)
    return fail(st[ST_CODE], "mapping stage rejected the composite table (status %d)",
                st[ST_CODE]);
  return TCL_OK;
}

int tcl_plan_copy_out(const tcl_plan *p, int32_t *tup_token, int32_t *tup_adapter,
                      float *tup_alpha, int32_t *tup_slot, int32_t *seg_adapter,
                      int32_t *seg_begin, int32_t *tok_ptr, int32_t *tok_tuple, void *stream) {
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PlanLayout &L = p->L;
  auto cp = [&](void *dst, const void *src, size_t n) -> hipError_t {
    if (!dst || n == 0) return hipSuccess;
    return hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToHost, s);
  };
  TCL_HIP(cp(tup_token, p->d.tup_token, size_t(L.cap) * 4));
  TCL_HIP(cp(tup_adapter, p->d.tup_adapter, size_t(L.cap) * 4));
  TCL_HIP(cp(tup_alpha, p->d.tup_alpha, size_t(L.cap) * 4));
  TCL_HIP(cp(tup_slot, p->d.tup_slot, size_t(L.cap) * 4));
  TCL_HIP(cp(seg_adapter, p->d.seg_adapter, size_t(L.N) * 4));
  TCL_HIP(cp(seg_begin, p->d.seg_begin, size_t(L.N + 1) * 4));
  TCL_HIP(cp(tok_ptr, p->d.tok_ptr, size_t(L.T + 1) * 4));
  TCL_HIP(cp(tok_tuple, p->d.tok_tuple, size_t(L.cap) * 4));
  TCL_HIP(hipStreamSynchronize(s));
  return TCL_OK;
}

void tcl_plan_free(tcl_plan *p) {
  if (!p) return;
  if (p->stage_pending) (void)hipEventSynchronize(p->stage_ev);
  if (p->stage) (void)hipHostFree(p->stage);
  if (p->stage_ev) (void)hipEventDestroy(p->stage_ev);
  delete p;
}

}  // extern "C"
