// Device code of the mapping stage (the one-workgroup modes), shared by the
// mapping kernels and by the decode step that runs the mapping stage inside
// the shrink launch.  See plan.hip for the stage itself.
#pragma once

#include "tcl_internal.hpp"

namespace tcl {

// ---------------------------------------------------------------------------
// block-wide helpers (NT threads = NT/64 waves of 64)
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele steps of
// 1, 2, 4 and 8 lanes inside each row of 16 (DPP row shifts, lanes without a
// source add 0), then the last lane of row 0 is added to row 1 and 3 and the
// last lane of row 1 to rows 2 and 3 (DPP row broadcasts).  No LDS traffic.
__device__ inline int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Every block-wide operation below gets its own scratch slot of kSlotInts
// ints, so no trailing barrier is needed before the slot could be reused.
constexpr int kScanMax = 4;
constexpr int kSlotInts = kScanMax * (kPlanThreads / 64);

// OR of small bit sets (EB_* bits) over the block: one ballot per bit.
template <int NT>
__device__ inline int block_or(int v, int *slot) {
  constexpr int kWaves = NT / 64;
  int r = 0;
#pragma unroll
  for (int b = 0; b < 3; ++b)
    if (__ballot((v >> b) & 1)) r |= 1 << b;
  if (kWaves == 1) return r;
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = r;
  __syncthreads();
  r = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r |= slot[i];
  return r;
}

// Exclusive prefix of K values over thread order (one barrier): v[i] is
// replaced by its exclusive prefix and tot[i] receives the block total.
template <int NT, int K>
__device__ inline void block_excl_scan_n(int (&v)[K], int *slot, int (&tot)[K]) {
  static_assert(K <= kScanMax, "scan width");
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc[K];
#pragma unroll
  for (int i = 0; i < K; ++i) inc[i] = wave_incl_scan(v[i]);
  if (kWaves == 1) {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      tot[i] = __builtin_amdgcn_readlane(inc[i], 63);
      v[i] = inc[i] - v[i];
    }
    return;
  }
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < K; ++i) slot[i * kWaves + w] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < K; ++i) {
    int before = 0, t = 0;
#pragma unroll
    for (int j = 0; j < kWaves; ++j) {
      const int x = slot[i * kWaves + j];
      before += j < w ? x : 0;
      t += x;
    }
    tot[i] = t;
    v[i] = before + inc[i] - v[i];
  }
}

// Exclusive prefix of v over thread order; *total receives the block sum.
template <int NT>
__device__ inline int block_excl_scan(int v, int *slot, int *total) {
  int x[1] = {v}, t[1];
  block_excl_scan_n<NT, 1>(x, slot, t);
  *total = t[0];
  return x[0];
}

struct PlanArgs {
  int32_t T, G, NP, N, cap, C, mode, items_cap;
  const int32_t *gtp, *gpp, *pa;
  const float *pw;
  PlanDev d;
};

template <int NT>
__device__ inline void plan_fail(const PlanArgs &A, int code, int P) {
  for (int t = threadIdx.x; t <= A.T; t += NT) A.d.tok_ptr[t] = 0;
  for (int t = threadIdx.x; t < A.T; t += NT) A.d.tok_n[t] = 0;
  if (threadIdx.x == 0) {
    A.d.status[ST_CODE] = code;
    A.d.status[ST_TUPLES] = P;
    A.d.status[ST_SEGMENTS] = 0;
    A.d.status[ST_ITEMS] = 0;
  }
}

// Device arrays of the mapping stage: the staged composite table and the
// per-pair / per-group scratch.  In the LDS paths every pointer is derived
// from the kernel's __shared__ block only, so the compiler emits LDS (ds_*)
// instructions rather than flat ones.
struct PlanView {
  const int32_t *gtp, *gpp, *pa;
  const float *pw;
  int32_t *slot, *grp, *pos, *gbase, *hist, *ptl, *hcnt, *ssm, *sib;
  int32_t *cnt, *sst, *su;  // direct path: per-adapter count, segment start, segment index
  int32_t *pcnt, *sbk;      // direct path: per-adapter pair count and pair-bucket start
  int32_t *tkt, *bkt, *bkw; // direct path: pair ticket; bucket entries (pair, tokens)
};

template <int NT, int MODE>
__device__ inline PlanView plan_view(const PlanArgs &A, int *lds) {
  PlanView v;
  const int G = A.G, NP = A.NP;
  if constexpr (MODE == PLAN_COUNT_GLOBAL) {
    v.gtp = A.gtp;
    v.gpp = A.gpp;
    v.pa = A.pa;
    v.pw = A.pw;
    v.slot = A.d.s_slot;
    v.grp = A.d.s_group;
    v.pos = A.d.s_pos;
    v.gbase = A.d.s_gbase;
    v.hist = A.d.s_hist;
    v.ptl = nullptr;
    v.hcnt = nullptr;
    v.ssm = nullptr;
    v.sib = nullptr;
    v.cnt = v.sst = v.su = nullptr;
    v.pcnt = v.sbk = v.tkt = v.bkt = v.bkw = nullptr;
  } else if constexpr (MODE == PLAN_DIRECT) {
    const int N = A.N;
    int *p = lds;
    int *l_pa = p; p += NP;
    v.ptl = p; p += NP;
    v.pos = nullptr;
    float *l_pw = reinterpret_cast<float *>(p); p += NP;
    v.slot = p; p += NP;
    v.grp = p; p += NP;
    v.tkt = p; p += NP;
    v.bkt = p; p += NP;
    v.bkw = p; p += NP;
    int *l_gtp = p; p += G + 1;
    int *l_gpp = p; p += G + 1;
    v.gbase = p; p += G;
    v.cnt = p; p += N;
    v.pcnt = p; p += N;
    v.sst = p; p += N;
    v.sib = p; p += N;
    v.su = p; p += N;
    v.sbk = p; p += N;
    v.hist = nullptr;
    v.hcnt = nullptr;
    v.ssm = nullptr;
    for (int i = threadIdx.x; i <= G; i += NT) {
      l_gtp[i] = A.gtp[i];
      l_gpp[i] = A.gpp[i];
    }
    for (int i = threadIdx.x; i < NP; i += NT) {
      l_pa[i] = A.pa[i];
      l_pw[i] = A.pw[i];
    }
    for (int i = threadIdx.x; i < N; i += NT) {
      v.cnt[i] = 0;
      v.pcnt[i] = 0;
    }
    __syncthreads();
    v.gtp = l_gtp;
    v.gpp = l_gpp;
    v.pa = l_pa;
    v.pw = l_pw;
  } else {
    // stage the composite table in LDS with coalesced loads
    int *p = lds;
    int *l_gtp = p; p += G + 1;
    int *l_gpp = p; p += G + 1;
    int *l_pa = p; p += NP;
    float *l_pw = reinterpret_cast<float *>(p); p += NP;
    v.slot = p; p += NP;
    v.grp = p; p += NP;
    v.pos = p; p += NP;
    v.gbase = p; p += G;
    v.ptl = nullptr;
    v.hcnt = nullptr;
    v.ssm = nullptr;
    v.sib = nullptr;
    v.cnt = v.sst = v.su = nullptr;
    v.hist = p;
    v.pcnt = v.sbk = v.tkt = v.bkt = v.bkw = nullptr;
    for (int i = threadIdx.x; i <= G; i += NT) {
      l_gtp[i] = A.gtp[i];
      l_gpp[i] = A.gpp[i];
    }
    for (int i = threadIdx.x; i < NP; i += NT) {
      l_pa[i] = A.pa[i];
      l_pw[i] = A.pw[i];
    }
    __syncthreads();
    v.gtp = l_gtp;
    v.gpp = l_gpp;
    v.pa = l_pa;
    v.pw = l_pw;
  }
  return v;
}

// The direct mode for tables of at most NT groups and NT pairs (every
// decode-sized table): thread i owns group i and pair i.  Their table
// entries go from global memory straight into registers, and each phase
// below reads from LDS only what another thread produced, in one round trip
// where the general path below takes several.  The stage's time is the
// length of its dependent chain (LDS round trips, barriers and the
// instructions between them), not bandwidth.  The outputs, error codes and
// their precedence are those of the general path:
//   A  groups: bounds, tuple counts, pair -> group records; one scan gives
//      the group tuple bases and the structural verdict;
//   B  pairs: ids, weights, canonical slot (pairs of the group with a
//      smaller adapter id), duplicates, per-adapter tuple and pair counts;
//   C  adapters: one four-value scan gives segment starts, item bases,
//      segment indices and pair-bucket starts; segment table and work-item
//      heads are written here;
//   D  each pair enters its adapter's bucket at the ticket its count gave;
//   E  a pair's first tuple position is its segment start plus the tuples of
//      the bucket's pairs with a smaller pair index (earlier pairs hold
//      earlier tokens), which does not depend on the order inside a bucket;
//      tuples, token records and inlined work-item tokens are written.
// lds must hold 8 NP + G + 6 N ints (16-byte aligned); tmp 3 kSlotInts.
template <int NT>
__device__ inline int plan_run_small(const PlanArgs &A, int *lds, int *tmp, bool out, Item *li,
                                     int li_cap, int *n_items_out, bool heads_only = false) {
  const int tid = threadIdx.x;
  const int T = A.T, G = A.G, NP = A.NP, N = A.N;
  *n_items_out = 0;
  int4 *ainfo = reinterpret_cast<int4 *>(lds);   // [N] {seg start, item base, seg index, bucket}
  int4 *pinfo = ainfo + N;                       // [NP] {group's first pair, pairs, first token, tokens}
  int *l_pa = reinterpret_cast<int *>(pinfo + NP);  // [NP] adapter of every pair
  int *pg = l_pa + NP;                           // [NP] group of every pair
  int *bkt = pg + NP, *bkw = bkt + NP;           // [NP] bucket entries: pair, its tokens
  int *gbase = bkw + NP;                         // [G] first token-index entry of every group
  int *cnt = gbase + G, *pcnt = cnt + N;         // [N] tuples and pairs of every adapter

  // the table, straight into registers.  Every thread loads (indices
  // clamped into the arrays) so that the loads share one round trip: loads
  // under per-thread conditions made the compiler wait for each group of
  // them before issuing the next.  With no pairs, pa and pw may be empty;
  // then the group array stands in for them.
  const int gi = min(tid, G), gj = min(tid + 1, G);
  const int pj = NP > 0 ? min(tid, NP - 1) : 0;
  const int32_t *pap = NP > 0 ? A.pa : A.gtp;
  const float *pwp = NP > 0 ? A.pw : reinterpret_cast<const float *>(A.gtp);
  const int t0 = A.gtp[gi], t1 = A.gtp[gj], q0 = A.gpp[gi], q1 = A.gpp[gj];
  const int aq = pap[pj];
  const float w = pwp[pj];
  for (int i = tid; i < N; i += NT) {
    cnt[i] = 0;
    pcnt[i] = 0;
  }

  // ---- A: groups ----------------------------------------------------------
  int err = 0, local = 0;
  // table ends: gtp[0] and gpp[0] are thread 0's first entries, gtp[G] and
  // gpp[G] the second ones of thread max(G - 1, 0)
  if (tid == 0 && (t0 != 0 || q0 != 0)) err |= EB_INVAL;
  // (pairs at or beyond gpp[G] are unused capacity of the arrays)
  if (tid == max(G - 1, 0) && (t1 != T || q1 > NP)) err |= EB_INVAL;
  if (tid < G) {
    if (!(0 <= t0 && t0 <= t1 && t1 <= T && 0 <= q0 && q0 <= q1 && q1 <= NP)) {
      err |= EB_INVAL;
    } else {
      const int4 rec = make_int4(q0, q1 - q0, t0, t1 - t0);
      for (int q = q0; q < q1; ++q) {
        pinfo[q] = rec;
        pg[q] = tid;
      }
      if (q1 - q0 > TCL_MAX_PAIRS_PER_GROUP) err |= EB_UNSUP;
      else local = (t1 - t0) * (q1 - q0);
    }
  }
  int P = 0, err_groups = 0, gb = 0, NPe = 0;
  {
    // the table's pair count gpp[G] (the end of the last group's pairs)
    // travels with the scan
    const int end = tid == max(G - 1, 0) ? q1 : 0;
    int sv[4] = {local, err & EB_INVAL, (err & EB_UNSUP) >> 1, end}, st[4];
    block_excl_scan_n<NT, 4>(sv, tmp + 0 * kSlotInts, st);
    P = st[0];
    gb = sv[0];
    err_groups = (st[1] ? EB_INVAL : 0) | (st[2] ? EB_UNSUP : 0);
    NPe = st[3];
  }
  if (err_groups & EB_INVAL) {
    if (out) plan_fail<NT>(A, TCL_EINVAL, 0);
    return TCL_EINVAL;
  }
  // pairs of the table, and -1 for the unused capacity (never an adapter id)
  if (tid < NP) l_pa[tid] = tid < NPe ? aq : -1;
  if (tid < G) gbase[tid] = gb;

  // ---- B: pairs (the group table is sound from here on) -------------------
  err = 0;
  int s = 0, tkt = 0, g = 0;
  int4 pi = make_int4(0, 0, 0, 0);
  bool live = false;
  if (tid < NPe) {
    pi = pinfo[tid];
    g = pg[tid];
    const bool a_ok = aq >= 0 && aq < N;
    if (!a_ok) err |= EB_INVAL;
    if ((__float_as_uint(w) & 0x7f800000u) == 0x7f800000u) err |= EB_INVAL;
    if (pi.y <= TCL_MAX_PAIRS_PER_GROUP) {
      // counts first: the ticket's round trip then overlaps the slot search
      if (a_ok) {
        atomicAdd(&cnt[aq], pi.w);
        tkt = atomicAdd(&pcnt[aq], 1);
        live = true;
      }
      int dup = 0;
      // heads only: no slots, and the table's verdict is the plan writer's
      // (a table with duplicates or bad weights still yields in-range items)
      for (int q2 = pi.x; !heads_only && q2 < pi.x + pi.y; q2 += 8) {
        int av[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) av[u] = q2 + u < pi.x + pi.y ? l_pa[q2 + u] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool in = q2 + u < pi.x + pi.y;
          s += (in && av[u] < aq) ? 1 : 0;
          dup |= (in && av[u] == aq && q2 + u != tid) ? 1 : 0;
        }
      }
      if (dup) err |= EB_INVAL;
    }
  }
  if (heads_only) {
    __syncthreads();  // the counts are complete
    err = err_groups;
  } else {
    err = block_or<NT>(err, tmp + 1 * kSlotInts) | err_groups;
  }
  if (err) {
    const int code = (err & EB_INVAL) ? TCL_EINVAL : TCL_EUNSUPPORTED;
    if (out) plan_fail<NT>(A, code, 0);
    return code;
  }
  if (P > A.cap) {
    if (out) plan_fail<NT>(A, TCL_ENOSPC, P);
    return TCL_ENOSPC;
  }

  // ---- C: adapters ----------------------------------------------------------
  int n_items = 0, n_segs = 0;
  {
    const int per = (N + NT - 1) / NT;
    const int a0 = min(N, tid * per), a1 = min(N, a0 + per);
    int sv[4] = {0, 0, 0, 0}, st[4];
    int c1 = 0, pc1 = 0;  // the counts of adapter a0 (the only one when N <= NT)
    for (int a = a0; a < a1; ++a) {
      const int c = cnt[a], pc = pcnt[a];
      if (a == a0) {
        c1 = c;
        pc1 = pc;
      }
      sv[0] += c;
      sv[1] += c > 0;
      sv[2] += (c + kTile - 1) / kTile;
      sv[3] += pc;
    }
    block_excl_scan_n<NT, 4>(sv, tmp + 2 * kSlotInts, st);
    n_items = st[2];
    n_segs = st[1];
    int ec = sv[0], en = sv[1], ei = sv[2], eb = sv[3];
    for (int a = a0; a < a1; ++a) {
      const int c = a == a0 ? c1 : cnt[a], pc = a == a0 ? pc1 : pcnt[a];
      ainfo[a] = make_int4(ec, ei, en, (eb << 16) | pc);
      if (c > 0) {
        if (out) {
          A.d.seg_adapter[en] = a;
          A.d.seg_begin[en] = ec;
        }
        for (int p0 = ec, i = ei; p0 < ec + c; p0 += kTile, ++i) {
          const int4 h = make_int4(a, p0, min(ec + c, p0 + kTile) - p0, en);
          if (out && i < A.items_cap) A.d.items[i].head = h;
          if (li && i < li_cap) li[i].head = h;
        }
        en += 1;
      }
      ei += (c + kTile - 1) / kTile;
      eb += pc;
      ec += c;
    }
  }
  __syncthreads();
  if (heads_only) {
    // work-item heads only (no plan output): plan_small_item_tokens fills
    // the token lists of the items a caller needs
    *n_items_out = n_items;
    return TCL_OK;
  }

  // ---- D: buckets -----------------------------------------------------------
  int4 ai = make_int4(0, 0, 0, 0);
  if (live) {
    ai = ainfo[aq];
    const int e = (ai.w >> 16) + tkt;
    bkt[e] = tid;
    bkw[e] = pi.w;
  }
  __syncthreads();

  // ---- E: tuple positions and records ---------------------------------------
  if (live) {
    const int b0 = ai.w >> 16, b1 = b0 + (ai.w & 0xffff);
    int r = 0;
    for (int e = b0; e < b1; e += 8) {
      int qq[8], ww[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        qq[u] = e + u < b1 ? bkt[e + u] : NP;
        ww[u] = e + u < b1 ? bkw[e + u] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) r += qq[u] < tid ? ww[u] : 0;
    }
    const int base = ai.x + r, gbq = gbase[g], pl = pi.y, tq0 = pi.z;
    for (int i = 0; i < pi.w; ++i) {
      const int p = base + i;
      // positions are < P <= cap by construction; the guards keep a logic
      // error from writing outside the plan buffer
      if (p >= A.cap || gbq + i * pl + s >= A.cap || s >= kSlotPad) continue;
      if (out) {
        A.d.tup_token[p] = tq0 + i;
        A.d.tup_adapter[p] = aq;
        A.d.tup_alpha[p] = w;
        A.d.tup_slot[p] = s;
        A.d.tok_tuple[gbq + i * pl + s] = p;
        A.d.tok_rec[int64_t(tq0 + i) * kSlotPad + s] = make_int4(p, aq, __float_as_int(w), ai.z);
      }
      const int lp = p - ai.x;
      const int it = ai.y + lp / kTile;
      if (out && it < A.items_cap) A.d.items[it].tok[lp % kTile] = tq0 + i;
      if (li && it < li_cap) li[it].tok[lp % kTile] = tq0 + i;
    }
  }
  if (out) {
    if (tid < G) {
      for (int t = t0; t < t1; ++t) {
        A.d.tok_ptr[t] = gb + (t - t0) * (q1 - q0);
        A.d.tok_n[t] = q1 - q0;
      }
    }
    if (tid == 0) {
      A.d.tok_ptr[T] = P;
      A.d.seg_begin[n_segs] = P;
      A.d.status[ST_TUPLES] = P;
      A.d.status[ST_SEGMENTS] = n_segs;
      A.d.status[ST_ITEMS] = n_items;
      A.d.status[ST_CODE] = TCL_OK;
    }
  }
  *n_items_out = n_items;
  return TCL_OK;
}

// The token ids of work item `item` (its head in li), after plan_run_small
// ran with heads_only on the same lds: the pairs of the item's adapter, in
// pair order, each expanded to its group's tokens, are the adapter's tuples
// in (token, slot) order (a group holds an adapter at most once, and groups
// are in token order), so a pair's first tuple position is the segment
// start plus the token counts of the adapter's earlier pairs: one block
// scan.  Every thread of the workgroup calls it; calls in a row must
// alternate between two tmp slots (kSlotInts ints each).  The caller
// synchronises before the token lists are read.
template <int NT>
__device__ inline void plan_small_item_tokens(const PlanArgs &A, const int *lds, int *tmp,
                                              Item *li, int item) {
  const int tid = threadIdx.x, N = A.N, NP = A.NP;
  const int4 *ainfo = reinterpret_cast<const int4 *>(lds);
  const int4 *pinfo = ainfo + N;
  const int *l_pa = reinterpret_cast<const int *>(pinfo + NP);
  const int4 h = li[item].head;  // adapter, first tuple, tuples, segment
  int4 pi = make_int4(0, 0, 0, 0);
  if (tid < NP && l_pa[tid] == h.x) pi = pinfo[tid];
  int total;
  const int off = ainfo[h.x].x + block_excl_scan<NT>(pi.w, tmp, &total);
  for (int i = 0; i < pi.w; ++i) {
    const int pos = off + i;
    if (pos >= h.y && pos < h.y + h.z) li[item].tok[pos - h.y] = pi.z + i;
  }
}

// The mapping stage in the calling workgroup of NT threads.  lds: the LDS
// block of the mode (kPlanLdsInts ints, 4 for PLAN_COUNT_GLOBAL); tmp:
// 6 * kSlotInts ints of LDS.  out: write the plan (status words, tuples,
// token index, segment table, work items) to A.d.  li (LDS, direct mode
// only, may be null): also receive the work items there, at most li_cap of
// them, for a shrink in the same workgroup.  Returns TCL_OK or the error the
// table earned (uniform over the workgroup); *n_items receives the number
// of work items.  Without out the counting modes compute nothing usable.
template <int NT, int MODE>
__device__ inline int plan_run(const PlanArgs &A, int *lds, int *tmp, bool out, Item *li,
                               int li_cap, int *n_items_out, bool heads_only = false) {
  constexpr bool direct = MODE == PLAN_DIRECT;
  if constexpr (direct) {
    if (A.G <= NT && A.NP <= NT)
      return plan_run_small<NT>(A, lds, tmp, out, li, li_cap, n_items_out, heads_only);
  }
  const int tid = threadIdx.x;
  *n_items_out = 0;
  const int T = A.T, G = A.G, NP = A.NP, N = A.N, C = A.C;

  const PlanView V = plan_view<NT, MODE>(A, lds);
  const int32_t *gtp = V.gtp, *gpp = V.gpp, *pa = V.pa;
  const float *pw = V.pw;
  int32_t *slot = V.slot, *grp = V.grp, *pos = V.pos, *gbase = V.gbase, *hist = V.hist,
          *ptl = V.ptl, *cnt = V.cnt, *sst = V.sst, *sib = V.sib, *su = V.su, *pcnt = V.pcnt,
          *sbk = V.sbk, *tkt = V.tkt, *bkt = V.bkt, *bkw = V.bkw;

  // ---- groups: structure, tuples per group, group bases, token index -----
  // One thread per contiguous range of groups.  Structural errors stop the
  // mapping here; the per-pair checks below need a sound group table.
  int err = 0;
  // (pairs at or beyond gpp[G] are unused capacity of the arrays)
  if (tid == 0 && (gtp[0] != 0 || gtp[G] != T || gpp[0] != 0 || gpp[G] > NP)) err |= EB_INVAL;
  const int gper = (G + NT - 1) / NT;
  const int g0 = min(G, tid * gper), g1 = min(G, g0 + gper);
  int local = 0;
  for (int g = g0; g < g1; ++g) {
    const int t0 = gtp[g], t1 = gtp[g + 1], q0 = gpp[g], q1 = gpp[g + 1];
    if (!(0 <= t0 && t0 <= t1 && t1 <= T && 0 <= q0 && q0 <= q1 && q1 <= NP)) {
      err |= EB_INVAL;
      continue;
    }
    for (int q = q0; q < q1; ++q) {
      grp[q] = g;
      if constexpr (direct) ptl[q] = t1 - t0;
    }
    if (q1 - q0 > TCL_MAX_PAIRS_PER_GROUP) {
      err |= EB_UNSUP;
      continue;
    }
    local += (t1 - t0) * (q1 - q0);
  }
  int P = 0;
  {
    // group tuple bases; the token index itself is written at the very end,
    // so that no barrier below waits for those stores
    int run = block_excl_scan<NT>(local, tmp + 0 * kSlotInts, &P);
    if (!err) {
      for (int g = g0; g < g1; ++g) {
        gbase[g] = run;
        run += (gtp[g + 1] - gtp[g]) * (gpp[g + 1] - gpp[g]);
      }
    }
  }
  const int err_groups = block_or<NT>(err, tmp + 1 * kSlotInts);
  if (err_groups & EB_INVAL) {
    if (out) plan_fail<NT>(A, TCL_EINVAL, 0);
    return TCL_EINVAL;
  }
  const int NPe = gpp[G];  // the table's pairs; the rest of the arrays is unused

  // ---- pairs: ids, weights, canonical slots, duplicates --------------------
  // One thread per pair.  The slot is the number of the group's pairs with a
  // smaller adapter id.  Groups beyond the pair limit are already rejected
  // (EUNSUPPORTED) and are not searched for duplicates.  The direct path also
  // adds the pair's tuples to its adapter's count here.
  err = 0;
  for (int q = tid; q < NPe; q += NT) {
    const int aq = pa[q];
    const bool a_ok = aq >= 0 && aq < N;
    if (!a_ok) err |= EB_INVAL;
    const uint32_t bits = __float_as_uint(pw[q]);
    if ((bits & 0x7f800000u) == 0x7f800000u) err |= EB_INVAL;
    const int g = grp[q];
    const int q0 = gpp[g], q1 = gpp[g + 1];
    if (q1 - q0 > TCL_MAX_PAIRS_PER_GROUP) continue;
    int s = 0, dup = 0;
    for (int q2 = q0; q2 < q1; q2 += 8) {
      int av[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) av[u] = q2 + u < q1 ? pa[q2 + u] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = q2 + u < q1;
        s += (in && av[u] < aq) ? 1 : 0;
        dup |= (in && av[u] == aq && q2 + u != q) ? 1 : 0;
      }
    }
    if (dup) err |= EB_INVAL;
    slot[q] = s;
    if constexpr (direct) {
      if (a_ok) {
        atomicAdd(&cnt[aq], ptl[q]);
        tkt[q] = atomicAdd(&pcnt[aq], 1);  // the pair's place in its adapter's bucket
      }
    }
  }
  err = block_or<NT>(err, tmp + 2 * kSlotInts) | err_groups;
  if (err) {
    const int code = (err & EB_INVAL) ? TCL_EINVAL : TCL_EUNSUPPORTED;
    if (out) plan_fail<NT>(A, code, 0);
    return code;
  }
  if (P > A.cap) {
    if (out) plan_fail<NT>(A, TCL_ENOSPC, P);
    return TCL_ENOSPC;
  }

  int n_items = 0, n_segs = 0;
  if constexpr (direct) {
    // ---- direct: position = (tuples of smaller adapters) + (tokens of the
    //      same adapter's earlier pairs; earlier pairs hold earlier tokens).
    //      One four-value scan over per-adapter counts gives segment starts,
    //      segment indices, item bases and pair-bucket starts.  Every pair
    //      then enters its adapter's bucket at its ticket; the order inside a
    //      bucket is arbitrary, and the rank below sums over the bucket's
    //      pairs with a smaller index, which does not depend on that order.
    const int per = (N + NT - 1) / NT;
    const int a0 = min(N, tid * per), a1 = min(N, a0 + per);
    int sv[4] = {0, 0, 0, 0}, st[4];
    for (int a = a0; a < a1; ++a) {
      const int c = cnt[a];
      sv[0] += c;
      sv[1] += c > 0;
      sv[2] += (c + kTile - 1) / kTile;
      sv[3] += pcnt[a];
    }
    block_excl_scan_n<NT, 4>(sv, tmp + 3 * kSlotInts, st);
    {
      int ec = sv[0], en = sv[1], ei = sv[2], eb = sv[3];
      for (int a = a0; a < a1; ++a) {
        const int c = cnt[a];
        sst[a] = ec;
        sib[a] = ei;
        su[a] = en;
        sbk[a] = eb;
        en += c > 0;
        ei += (c + kTile - 1) / kTile;
        eb += pcnt[a];
        ec += c;
      }
    }
    n_items = st[2];
    n_segs = st[1];
    __syncthreads();
    for (int q = tid; q < NPe; q += NT) {
      const int e = sbk[pa[q]] + tkt[q];
      bkt[e] = q;
      bkw[e] = ptl[q];
    }
  } else {
    // ---- counting sort: per-chunk counts per adapter ----------------------
    const int M = N * C;
    for (int i = tid; i < M; i += NT) hist[i] = 0;
    __syncthreads();
    const int cg0 = int((int64_t(tid) * G) / C), cg1 = int((int64_t(tid + 1) * G) / C);
    if (tid < C) {
      for (int g = cg0; g < cg1; ++g) {
        const int tl = gtp[g + 1] - gtp[g];
        for (int q = gpp[g]; q < gpp[g + 1]; ++q) hist[pa[q] * C + tid] += tl;
      }
    }
    __syncthreads();
    // exclusive scan over (adapter, chunk), adapter-major
    {
      const int per = (M + NT - 1) / NT;
      const int i0 = min(M, tid * per), i1 = min(M, i0 + per);
      int local = 0;
      for (int i = i0; i < i1; ++i) local += hist[i];
      int tot;
      int run = block_excl_scan<NT>(local, tmp + 4 * kSlotInts, &tot);
      for (int i = i0; i < i1; ++i) {
        const int v = hist[i];
        hist[i] = run;
        run += v;
      }
    }
    __syncthreads();
    // segment table and shrink work items
    {
      const int per = (N + NT - 1) / NT;
      const int a0 = min(N, tid * per), a1 = min(N, a0 + per);
      int nseg = 0, nitem = 0;
      for (int a = a0; a < a1; ++a) {
        const int beg = hist[a * C], end = (a + 1 < N) ? hist[(a + 1) * C] : P;
        const int cnt = end - beg;
        nseg += cnt > 0;
        nitem += (cnt + kTile - 1) / kTile;
      }
      int sv[2] = {nseg, nitem}, st[2];
      block_excl_scan_n<NT, 2>(sv, tmp + 5 * kSlotInts, st);
      int u = sv[0], it = sv[1];
      const int U = st[0], NI = st[1];
      for (int a = a0; a < a1; ++a) {
        const int beg = hist[a * C], end = (a + 1 < N) ? hist[(a + 1) * C] : P;
        if (end > beg) {
          A.d.seg_adapter[u] = a;
          A.d.seg_begin[u] = beg;
          A.d.s_seg[a] = u;
          for (int p0 = beg; p0 < end; p0 += kTile, ++it)
            if (it < A.items_cap) A.d.items[it].head = make_int4(a, p0, min(end, p0 + kTile) - p0, u);
          ++u;
        }
      }
      n_items = NI;
      if (tid == 0) {
        A.d.seg_begin[U] = P;
        A.d.status[ST_TUPLES] = P;
        A.d.status[ST_SEGMENTS] = U;
        A.d.status[ST_ITEMS] = NI;
      }
    }
    __syncthreads();
    // each chunk hands out consecutive positions in pair order
    if (tid < C) {
      for (int g = cg0; g < cg1; ++g) {
        const int tl = gtp[g + 1] - gtp[g];
        for (int q = gpp[g]; q < gpp[g + 1]; ++q) {
          const int h = pa[q] * C + tid;
          pos[q] = hist[h];
          hist[h] += tl;
        }
      }
    }
  }
  __syncthreads();

  // ---- write the tuples and the per-token index ---------------------------
  for (int q = tid; q < NPe; q += NT) {
    const int g = grp[q];
    const int t0 = gtp[g], tl = gtp[g + 1] - t0, pl = gpp[g + 1] - gpp[g];
    const int a = pa[q], s = slot[q], gb = gbase[g];
    int base;
    if constexpr (direct) {
      const int b0 = sbk[a], b1 = b0 + pcnt[a];
      int r = 0;
      for (int e = b0; e < b1; e += 8) {
        int qq[8], ww[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          qq[u] = e + u < b1 ? bkt[e + u] : NP;
          ww[u] = e + u < b1 ? bkw[e + u] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) r += qq[u] < q ? ww[u] : 0;
      }
      base = sst[a] + r;
    } else {
      base = pos[q];
    }
    const float w = pw[q];
    int sg;  // segment of the adapter (its index in the segment table)
    if constexpr (direct) sg = su[a];
    else sg = A.d.s_seg[a];
    for (int i = 0; i < tl; ++i) {
      const int p = base + i;
      // positions are < P <= cap by construction; the guards keep a logic
      // error from writing outside the plan buffer
      if (p >= A.cap || gb + i * pl + s >= A.cap || s >= kSlotPad) continue;
      if (out) {
        A.d.tup_token[p] = t0 + i;
        A.d.tup_adapter[p] = a;
        A.d.tup_alpha[p] = w;
        A.d.tup_slot[p] = s;
        A.d.tok_tuple[gb + i * pl + s] = p;
        A.d.tok_rec[int64_t(t0 + i) * kSlotPad + s] = make_int4(p, a, __float_as_int(w), sg);
      }
      if constexpr (direct) {
        const int local = p - sst[a];
        const int it = sib[a] + local / kTile;
        if (out && it < A.items_cap) A.d.items[it].tok[local % kTile] = t0 + i;
        if (li && it < li_cap) li[it].tok[local % kTile] = t0 + i;
      }
    }
  }
  // ---- token index (deferred so that no barrier above waited for it) ------
  if (out) {
    for (int g = g0; g < g1; ++g) {
      const int t0 = gtp[g], t1 = gtp[g + 1], pl = gpp[g + 1] - gpp[g], run = gbase[g];
      for (int t = t0; t < t1; ++t) {
        A.d.tok_ptr[t] = run + (t - t0) * pl;
        A.d.tok_n[t] = pl;
      }
    }
    if (tid == 0) A.d.tok_ptr[T] = P;
  }
  if constexpr (direct) {
    // segment table, work-item heads and status words, also deferred
    const int per = (N + NT - 1) / NT;
    const int a0 = min(N, tid * per), a1 = min(N, a0 + per);
    for (int a = a0; a < a1; ++a) {
      const int c = cnt[a];
      if (c == 0) continue;
      const int ec = sst[a], en = su[a];
      if (out) {
        A.d.seg_adapter[en] = a;
        A.d.seg_begin[en] = ec;
      }
      for (int p0 = ec, i = sib[a]; p0 < ec + c; p0 += kTile, ++i) {
        const int4 h = make_int4(a, p0, min(ec + c, p0 + kTile) - p0, en);
        if (out && i < A.items_cap) A.d.items[i].head = h;
        if (li && i < li_cap) li[i].head = h;
      }
    }
    if (out && tid == 0) {
      A.d.seg_begin[n_segs] = P;
      A.d.status[ST_TUPLES] = P;
      A.d.status[ST_SEGMENTS] = n_segs;
      A.d.status[ST_ITEMS] = n_items;
      A.d.status[ST_CODE] = TCL_OK;
    }
    *n_items_out = n_items;
    return TCL_OK;
  }
  __syncthreads();

  // ---- inline the token ids of every work item -----------------------------
  for (int i = tid; i < n_items; i += NT) {
    const int4 h = A.d.items[i].head;
#pragma unroll
    for (int j = 0; j < kTile; ++j) A.d.items[i].tok[j] = A.d.tup_token[h.y + (j < h.z ? j : 0)];
  }
  if (tid == 0) A.d.status[ST_CODE] = TCL_OK;
  *n_items_out = n_items;
  return TCL_OK;
}

template <int NT, int MODE>
__global__ __launch_bounds__(NT) void plan_kernel(PlanArgs A) {
  __shared__ __align__(16) int lds[MODE == PLAN_COUNT_GLOBAL ? 4 : kPlanLdsInts];
  __shared__ int tmp[6 * kSlotInts];
  int n_items;
  plan_run<NT, MODE>(A, lds, tmp, true, nullptr, 0, &n_items);
}

// Host side of the shared mapping code (plan.hip).
// The kernel arguments of the mapping stage of plan p for table c.
void plan_fill_args(const tcl_plan *p, const tcl_composites *c, PlanArgs *out);
// LDS ints the direct mode's view of p's table takes (see plan_view).
int plan_direct_lds_ints(const tcl_plan *p);
// Host half of tcl_plan_remap: checks c and the buffer and describes in
// *next the plan that p becomes (nothing is launched, p is not changed).
int plan_remap_prepare(const tcl_plan *p, const tcl_composites *c, tcl_plan *next);
// Queue the mapping stage of p (already laid out for c) on stream s.
int plan_launch(tcl_plan *p, const tcl_composites *c, hipStream_t s);

}  // namespace tcl
