// Mapping stage of the composite multi-LoRA apply: composites -> tuples
// reordered by adapter id (DyMerge-LoRA summary page, section 4.3, the
// mapping step of the MAF-MVM kernel; the reorder by LoRA id is what lets one
// workgroup stream one adapter's factors over a contiguous token run).
//
// One workgroup of 1024 threads does the whole stage: validation, canonical
// slots, a stable counting sort keyed by adapter id, the segment table, the
// per-token tuple index and the shrink work list.  The sort is deterministic
// and uses no atomics: groups are split into C contiguous chunks, every chunk
// counts its tuples per adapter, one exclusive scan over the (adapter, chunk)
// matrix in adapter-major order gives every (adapter, chunk) its first output
// position, and each chunk then walks its pairs in order handing out
// consecutive positions.  Within an adapter, tuples therefore follow token
// order, which is the (adapter, token, slot) order because a token holds an
// adapter at most once.
//
// When the composite table is small (every decode batch) it is copied to LDS
// first with coalesced loads, so that the serial parts of the stage run on LDS
// latency instead of a chain of global-memory round trips.

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

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

int hip_fail(hipError_t e, const char *what) {
  return fail(TCL_EHIP, "%s failed: %s", what, hipGetErrorString(e));
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

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

  // LDS staging: gtp, gpp (G+1 each), adapter, alpha, slot, group, pos (NP
  // each), group tuple base (G), histogram (N * chunks).
  const int64_t fixed = 3 * int64_t(G) + 2 + 5 * int64_t(NP);
  int64_t c_small = (NP + 1) / 2;
  if (c_small < 1) c_small = 1;
  if (c_small > kPlanThreads) c_small = kPlanThreads;
  if (fixed + int64_t(N) * c_small > kPlanLdsInts) {
    int64_t room = kPlanLdsInts - fixed;
    c_small = room > 0 ? room / N : 0;
  }
  if (c_small >= 1) {
    l.small = 1;
    l.chunks = int32_t(c_small);
  } else {
    l.small = 0;
    int64_t c = (NP + 7) / 8;
    int64_t cmax = 65536 / N;
    if (c > cmax) c = cmax;
    if (c > kPlanThreads) c = kPlanThreads;
    if (c < 1) c = 1;
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
  l.o_tokptr = take(size_t(T + 1) * 4);
  l.o_segad = take(size_t(N) * 4);
  l.o_segbeg = take(size_t(N + 1) * 4);
  l.o_items = take(size_t(l.items_cap) * 16);
  l.o_sslot = take(size_t(NP) * 4);
  l.o_sgroup = take(size_t(NP) * 4);
  l.o_spos = take(size_t(NP) * 4);
  l.o_sgbase = take(size_t(G) * 4);
  l.o_shist = take(l.small ? 4 : size_t(N) * size_t(l.chunks) * 4);
  l.total = o;
  *L = l;
  return TCL_OK;
}

// ---------------------------------------------------------------------------
// block-wide helpers (1024 threads = 16 waves of 64)
// ---------------------------------------------------------------------------
constexpr int kWaves = kPlanThreads / 64;

__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

__device__ inline int block_or(int v, int *tmp) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v |= __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r |= tmp[i];
  __syncthreads();
  return r;
}

// Exclusive prefix of v over thread order; *total receives the block sum.
__device__ inline int block_excl_scan(int v, int *tmp, int *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int x = lane < kWaves ? tmp[lane] : 0;
    const int xi = wave_incl_scan(x);
    if (lane < kWaves) tmp[lane] = xi - x;
    if (lane == kWaves - 1) tmp[kWaves] = xi;
  }
  __syncthreads();
  const int r = tmp[w] + incl - v;
  *total = tmp[kWaves];
  __syncthreads();
  return r;
}

struct PlanArgs {
  int32_t T, G, NP, N, cap, C, small;
  const int32_t *gtp, *gpp, *pa;
  const float *pw;
  PlanDev d;
};

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs A) {
  __shared__ int lds[kPlanLdsInts];
  __shared__ int tmp[kWaves + 1];
  const int tid = threadIdx.x;
  const int T = A.T, G = A.G, NP = A.NP, N = A.N, C = A.C;

  const int32_t *gtp = A.gtp, *gpp = A.gpp, *pa = A.pa;
  const float *pw = A.pw;
  int32_t *slot = A.d.s_slot, *grp = A.d.s_group, *pos = A.d.s_pos, *gbase = A.d.s_gbase,
          *hist = A.d.s_hist;
  if (A.small) {
    int *p = lds;
    int *l_gtp = p; p += G + 1;
    int *l_gpp = p; p += G + 1;
    int *l_pa = p; p += NP;
    float *l_pw = reinterpret_cast<float *>(p); p += NP;
    slot = p; p += NP;
    grp = p; p += NP;
    pos = p; p += NP;
    gbase = p; p += G;
    hist = p;
    for (int i = tid; i <= G; i += kPlanThreads) {
      l_gtp[i] = A.gtp[i];
      l_gpp[i] = A.gpp[i];
    }
    for (int i = tid; i < NP; i += kPlanThreads) {
      l_pa[i] = A.pa[i];
      l_pw[i] = A.pw[i];
    }
    __syncthreads();
    gtp = l_gtp;
    gpp = l_gpp;
    pa = l_pa;
    pw = l_pw;
  }

  // ---- phase 0: validation, canonical slots ------------------------------
  int err = 0;
  if (tid == 0 && (gtp[0] != 0 || gtp[G] != T || gpp[0] != 0 || gpp[G] != NP)) err |= EB_INVAL;
  for (int g = tid; g < G; g += kPlanThreads) {
    const int t0 = gtp[g], t1 = gtp[g + 1], q0 = gpp[g], q1 = gpp[g + 1];
    if (!(0 <= t0 && t0 <= t1 && t1 <= T && 0 <= q0 && q0 <= q1 && q1 <= NP)) {
      err |= EB_INVAL;
      continue;
    }
    if (q1 - q0 > TCL_MAX_PAIRS_PER_GROUP) {
      err |= EB_UNSUP;
      continue;
    }
    for (int q = q0; q < q1; ++q) {
      const int aq = pa[q];
      int s = 0, dup = 0;
      for (int q2 = q0; q2 < q1; ++q2) {
        const int a2 = pa[q2];
        s += (a2 < aq);
        dup |= (a2 == aq) & (q2 != q);
      }
      if (dup) err |= EB_INVAL;
      slot[q] = s;
      grp[q] = g;
    }
  }
  for (int q = tid; q < NP; q += kPlanThreads) {
    const int aq = pa[q];
    if (aq < 0 || aq >= N) err |= EB_INVAL;
    const uint32_t bits = __float_as_uint(pw[q]);
    if ((bits & 0x7f800000u) == 0x7f800000u) err |= EB_INVAL;
  }
  err = block_or(err, tmp);
  if (err) {
    if (tid == 0) {
      A.d.status[ST_CODE] = (err & EB_INVAL) ? TCL_EINVAL : TCL_EUNSUPPORTED;
      A.d.status[ST_TUPLES] = 0;
      A.d.status[ST_SEGMENTS] = 0;
      A.d.status[ST_ITEMS] = 0;
    }
    return;
  }

  // ---- phase 1: tuples per group -> group base, token index --------------
  int P = 0;
  {
    const int per = (G + kPlanThreads - 1) / kPlanThreads;
    const int g0 = min(G, tid * per), g1 = min(G, g0 + per);
    int local = 0;
    for (int g = g0; g < g1; ++g) local += (gtp[g + 1] - gtp[g]) * (gpp[g + 1] - gpp[g]);
    int run = block_excl_scan(local, tmp, &P);
    for (int g = g0; g < g1; ++g) {
      const int t0 = gtp[g], t1 = gtp[g + 1], pl = gpp[g + 1] - gpp[g];
      gbase[g] = run;
      for (int t = t0; t < t1; ++t) A.d.tok_ptr[t] = run + (t - t0) * pl;
      run += (t1 - t0) * pl;
    }
    if (tid == 0) A.d.tok_ptr[T] = P;
  }
  if (P > A.cap) {
    if (tid == 0) {
      A.d.status[ST_CODE] = TCL_ENOSPC;
      A.d.status[ST_TUPLES] = P;
      A.d.status[ST_SEGMENTS] = 0;
      A.d.status[ST_ITEMS] = 0;
    }
    return;
  }

  // ---- phase 2: per-chunk tuple counts per adapter ------------------------
  const int M = N * C;
  for (int i = tid; i < M; i += kPlanThreads) hist[i] = 0;
  __syncthreads();
  const int cg0 = int((int64_t(tid) * G) / C), cg1 = int((int64_t(tid + 1) * G) / C);
  if (tid < C) {
    for (int g = cg0; g < cg1; ++g) {
      const int tl = gtp[g + 1] - gtp[g];
      for (int q = gpp[g]; q < gpp[g + 1]; ++q) hist[pa[q] * C + tid] += tl;
    }
  }
  __syncthreads();

  // ---- phase 3: exclusive scan over (adapter, chunk), adapter-major -------
  {
    const int per = (M + kPlanThreads - 1) / kPlanThreads;
    const int i0 = min(M, tid * per), i1 = min(M, i0 + per);
    int local = 0;
    for (int i = i0; i < i1; ++i) local += hist[i];
    int tot;
    int run = block_excl_scan(local, tmp, &tot);
    for (int i = i0; i < i1; ++i) {
      const int v = hist[i];
      hist[i] = run;
      run += v;
    }
  }
  __syncthreads();

  // ---- phase 4: segment table and shrink work items -----------------------
  {
    const int per = (N + kPlanThreads - 1) / kPlanThreads;
    const int a0 = min(N, tid * per), a1 = min(N, a0 + per);
    int nseg = 0, nitem = 0;
    for (int a = a0; a < a1; ++a) {
      const int beg = hist[a * C], end = (a + 1 < N) ? hist[(a + 1) * C] : P;
      const int cnt = end - beg;
      nseg += cnt > 0;
      nitem += (cnt + kTile - 1) / kTile;
    }
    int U, NI;
    int u = block_excl_scan(nseg, tmp, &U);
    int it = block_excl_scan(nitem, tmp, &NI);
    for (int a = a0; a < a1; ++a) {
      const int beg = hist[a * C], end = (a + 1 < N) ? hist[(a + 1) * C] : P;
      if (end > beg) {
        A.d.seg_adapter[u] = a;
        A.d.seg_begin[u] = beg;
        for (int p0 = beg; p0 < end; p0 += kTile)
          A.d.items[it++] = make_int4(a, p0, min(end, p0 + kTile), u);
        ++u;
      }
    }
    if (tid == 0) {
      A.d.seg_begin[U] = P;
      A.d.status[ST_TUPLES] = P;
      A.d.status[ST_SEGMENTS] = U;
      A.d.status[ST_ITEMS] = NI;
    }
  }
  __syncthreads();

  // ---- phase 5: each chunk hands out consecutive positions in pair order --
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
  __syncthreads();

  // ---- phase 6: write the tuples and the per-token index -----------------
  for (int q = tid; q < NP; q += kPlanThreads) {
    const int g = grp[q];
    const int t0 = gtp[g], tl = gtp[g + 1] - t0, pl = gpp[g + 1] - gpp[g];
    const int a = pa[q], s = slot[q], base = pos[q], gb = gbase[g];
    const float w = pw[q];
    for (int i = 0; i < tl; ++i) {
      const int p = base + i;
      A.d.tup_token[p] = t0 + i;
      A.d.tup_adapter[p] = a;
      A.d.tup_alpha[p] = w;
      A.d.tup_slot[p] = s;
      A.d.tok_tuple[gb + i * pl + s] = p;
    }
  }
  if (tid == 0) A.d.status[ST_CODE] = TCL_OK;
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
  d.seg_adapter = reinterpret_cast<int32_t *>(b + L.o_segad);
  d.seg_begin = reinterpret_cast<int32_t *>(b + L.o_segbeg);
  d.items = reinterpret_cast<int4 *>(b + L.o_items);
  d.s_slot = reinterpret_cast<int32_t *>(b + L.o_sslot);
  d.s_group = reinterpret_cast<int32_t *>(b + L.o_sgroup);
  d.s_pos = reinterpret_cast<int32_t *>(b + L.o_spos);
  d.s_gbase = reinterpret_cast<int32_t *>(b + L.o_sgbase);
  d.s_hist = reinterpret_cast<int32_t *>(b + L.o_shist);
}

static int check_composites(const tcl_composites *c) {
  if (!c) return fail(TCL_EINVAL, "composites is NULL");
  if (!c->group_tok_ptr || !c->group_pair_ptr)
    return fail(TCL_EINVAL, "group pointer arrays must not be NULL");
  if (c->n_pairs > 0 && (!c->pair_adapter || !c->pair_alpha))
    return fail(TCL_EINVAL, "pair arrays must not be NULL when n_pairs > 0");
  return TCL_OK;
}

static int launch_plan(tcl_plan *p, const tcl_composites *c, hipStream_t s) {
  PlanArgs A;
  A.T = p->L.T;
  A.G = p->L.G;
  A.NP = p->L.NP;
  A.N = p->L.N;
  A.cap = p->L.cap;
  A.C = p->L.chunks;
  A.small = p->L.small;
  A.gtp = c->group_tok_ptr;
  A.gpp = c->group_pair_ptr;
  A.pa = c->pair_adapter;
  A.pw = c->pair_alpha;
  A.d = p->d;
  logf("plan: T=%d G=%d pairs=%d N=%d cap=%d chunks=%d lds=%d", A.T, A.G, A.NP, A.N, A.cap, A.C,
       A.small);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, A);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

}  // namespace tcl

using namespace tcl;

extern "C" {

const char *tcl_last_error(void) { return g_err.c_str(); }

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
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  int rc = check_composites(c);
  if (rc) return rc;
  PlanLayout L;
  rc = plan_layout(c->n_tokens, c->n_groups, c->n_pairs, c->n_adapters, c->max_tuples, &L);
  if (rc) return rc;
  if (L.total > p->buf_bytes)
    return fail(TCL_ENOSPC, "plan buffer holds %zu bytes, needs %zu", p->buf_bytes, L.total);
  p->L = L;
  bind(p);
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

void tcl_plan_free(tcl_plan *p) { delete p; }

}  // extern "C"
