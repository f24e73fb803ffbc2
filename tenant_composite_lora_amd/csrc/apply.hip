// Shrink, expand and the fused apply of the composite multi-LoRA path.
//
//   shrink  (LoRAForge approach (4), segmented shrink): for one adapter's run
//           of tuples, z_p = A_a[:, :k]^T x_{t_p}.  One workgroup owns a work
//           item (an adapter, up to kTile consecutive tuples of its segment)
//           and a chunk of d_in; every wave owns a quarter of the rank rows,
//           every lane a 16-byte column granule, so A_a rows stream through
//           with coalesced 16-B loads and are reused across the item's
//           tokens.  Each lane keeps fp32 partial dot products that a
//           64-lane butterfly reduction folds in a fixed order.
//   expand  (LoRAForge approach (4), RowExpand; DyMerge-LoRA aggregation
//           stage): one wave owns 512 consecutive outputs of one token and
//           adds alpha_s * B_a[n, :k] z_s for the token's slots in order, in
//           fp32, then adds the total to y once.  Each output element has
//           exactly one owner; there are no atomics.
//
// All kernels first read the plan's device status and do nothing when the
// mapping stage rejected the composite table.

#include <cstdint>

#include "tcl_internal.hpp"

namespace tcl {

// ---------------------------------------------------------------------------
// element helpers
// ---------------------------------------------------------------------------
struct bf16_t {
  uint16_t bits;
};

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (finite inputs; NaN kept quiet).
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return uint16_t((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename TIN>
struct Gran;  // one 16-byte granule of inputs

template <>
struct Gran<bf16_t> {
  static constexpr int kElems = 8;
  uint4 v;
  __device__ inline void load(const void *p) { v = *reinterpret_cast<const uint4 *>(p); }
  __device__ inline float dot(const Gran &o, float acc) const {
    acc = fmaf(bf16_lo(v.x), bf16_lo(o.v.x), acc);
    acc = fmaf(bf16_hi(v.x), bf16_hi(o.v.x), acc);
    acc = fmaf(bf16_lo(v.y), bf16_lo(o.v.y), acc);
    acc = fmaf(bf16_hi(v.y), bf16_hi(o.v.y), acc);
    acc = fmaf(bf16_lo(v.z), bf16_lo(o.v.z), acc);
    acc = fmaf(bf16_hi(v.z), bf16_hi(o.v.z), acc);
    acc = fmaf(bf16_lo(v.w), bf16_lo(o.v.w), acc);
    acc = fmaf(bf16_hi(v.w), bf16_hi(o.v.w), acc);
    return acc;
  }
};

template <>
struct Gran<float> {
  static constexpr int kElems = 4;
  float4 v;
  __device__ inline void load(const void *p) { v = *reinterpret_cast<const float4 *>(p); }
  __device__ inline float dot(const Gran &o, float acc) const {
    acc = fmaf(v.x, o.v.x, acc);
    acc = fmaf(v.y, o.v.y, acc);
    acc = fmaf(v.z, o.v.z, acc);
    acc = fmaf(v.w, o.v.w, acc);
    return acc;
  }
};

// 8 consecutive weights of one B row, widened to fp32
template <typename TW>
__device__ inline void load8(const TW *p, float (&b)[8]);

template <>
__device__ inline void load8<bf16_t>(const bf16_t *p, float (&b)[8]) {
  const uint4 v = *reinterpret_cast<const uint4 *>(p);
  b[0] = bf16_lo(v.x); b[1] = bf16_hi(v.x);
  b[2] = bf16_lo(v.y); b[3] = bf16_hi(v.y);
  b[4] = bf16_lo(v.z); b[5] = bf16_hi(v.z);
  b[6] = bf16_lo(v.w); b[7] = bf16_hi(v.w);
}

template <>
__device__ inline void load8<float>(const float *p, float (&b)[8]) {
  const float4 u = reinterpret_cast<const float4 *>(p)[0];
  const float4 v = reinterpret_cast<const float4 *>(p)[1];
  b[0] = u.x; b[1] = u.y; b[2] = u.z; b[3] = u.w;
  b[4] = v.x; b[5] = v.y; b[6] = v.z; b[7] = v.w;
}

// y[0..8) += acc[0..8)
template <typename TY>
__device__ inline void add_store8(TY *p, const float (&acc)[8]);

template <>
__device__ inline void add_store8<float>(float *p, const float (&acc)[8]) {
  float4 *q = reinterpret_cast<float4 *>(p);
  float4 u = q[0], v = q[1];
  u.x += acc[0]; u.y += acc[1]; u.z += acc[2]; u.w += acc[3];
  v.x += acc[4]; v.y += acc[5]; v.z += acc[6]; v.w += acc[7];
  q[0] = u;
  q[1] = v;
}

template <>
__device__ inline void add_store8<bf16_t>(bf16_t *p, const float (&acc)[8]) {
  uint4 *q = reinterpret_cast<uint4 *>(p);
  uint4 v = *q;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t lo = f32_to_bf16(bf16_lo(w[i]) + acc[2 * i]);
    const uint16_t hi = f32_to_bf16(bf16_hi(w[i]) + acc[2 * i + 1]);
    w[i] = uint32_t(lo) | (uint32_t(hi) << 16);
  }
  *q = make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ inline int eff_rank(const int32_t *k_dev, int a, int r_max) {
  if (!k_dev) return r_max;
  const int k = k_dev[a];
  return k < 0 ? 0 : (k > r_max ? r_max : k);
}

// ---------------------------------------------------------------------------
// shrink
// ---------------------------------------------------------------------------
struct ShrinkArgs {
  const int32_t *status;
  const int4 *items;
  const int32_t *tup_token;
  const int32_t *k_dev;
  const void *A_t;
  const void *x;
  int64_t ldx;
  int32_t d_in, r_max, cap;
  int32_t n_chunks, chunk_gran;  // chunk width in 16-byte granules
  int32_t zero_tail;             // write zeros for k <= j < r_max
  float *z;                      // [n_chunks][cap][r_max]
};

template <int R, typename TIN>
__global__ __launch_bounds__(256) void shrink_valu(ShrinkArgs s) {
  if (s.status[ST_CODE] != TCL_OK) return;
  constexpr int VEC = Gran<TIN>::kElems;
  constexpr int RW = (R + 3) / 4;  // rank rows per wave
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n_items = s.status[ST_ITEMS];
  const int total = n_items * s.n_chunks;
  const int n_gran = s.d_in / VEC;
  const TIN *A = static_cast<const TIN *>(s.A_t);
  const TIN *X = static_cast<const TIN *>(s.x);

  for (int job = blockIdx.x; job < total; job += gridDim.x) {
    const int item = job / s.n_chunks, chunk = job - item * s.n_chunks;
    const int4 it = s.items[item];
    const int a = it.x, p0 = it.y, ntok = it.z - it.y;
    const int k = eff_rank(s.k_dev, a, s.r_max);
    int tok[kTile];
#pragma unroll
    for (int tt = 0; tt < kTile; ++tt) tok[tt] = tt < ntok ? s.tup_token[p0 + tt] : 0;

    float acc[RW][kTile];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int tt = 0; tt < kTile; ++tt) acc[i][tt] = 0.f;

    const int g0 = chunk * s.chunk_gran;
    const int g1 = min(n_gran, g0 + s.chunk_gran);
    for (int g = g0 + lane; g < g1; g += 64) {
      Gran<TIN> xv[kTile];
#pragma unroll
      for (int tt = 0; tt < kTile; ++tt)
        if (tt < ntok) xv[tt].load(X + int64_t(tok[tt]) * s.ldx + int64_t(g) * VEC);
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int j = w + 4 * i;
        if (j < k) {
          Gran<TIN> av;
          av.load(A + (int64_t(a) * s.r_max + j) * s.d_in + int64_t(g) * VEC);
#pragma unroll
          for (int tt = 0; tt < kTile; ++tt)
            if (tt < ntok) acc[i][tt] = av.dot(xv[tt], acc[i][tt]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int j = w + 4 * i;
      if (j >= s.r_max) continue;
      if (j < k) {
#pragma unroll
        for (int tt = 0; tt < kTile; ++tt) {
          if (tt < ntok) {
            const float v = wave_sum(acc[i][tt]);
            if (lane == 0) s.z[(int64_t(chunk) * s.cap + p0 + tt) * s.r_max + j] = v;
          }
        }
      } else if (s.zero_tail && lane == 0) {
        for (int tt = 0; tt < ntok; ++tt)
          s.z[(int64_t(chunk) * s.cap + p0 + tt) * s.r_max + j] = 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// expand
// ---------------------------------------------------------------------------
struct ExpandArgs {
  const int32_t *status;
  const int32_t *tok_ptr, *tok_tuple, *tup_adapter;
  const float *tup_alpha;
  const int32_t *k_dev;
  const void *B_t;
  const float *z;  // [n_chunks][cap][r_max]
  void *y;
  int64_t ldy;
  int32_t d_out, r_max, cap, n_chunks, n_coltiles;
};

template <int R, typename TW, typename TY>
__global__ __launch_bounds__(64) void expand_valu(ExpandArgs e) {
  if (e.status[ST_CODE] != TCL_OK) return;
  const int lane = threadIdx.x;
  const int t = blockIdx.x / e.n_coltiles, ct = blockIdx.x - t * e.n_coltiles;
  const int s0 = e.tok_ptr[t], s1 = e.tok_ptr[t + 1];
  if (s0 == s1) return;
  const int n0 = (ct * 64 + lane) * 8;
  if (n0 >= e.d_out) return;
  const TW *B = static_cast<const TW *>(e.B_t);

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int i = s0; i < s1; ++i) {
    const int p = e.tok_tuple[i];
    const int a = e.tup_adapter[p];
    const float al = e.tup_alpha[p];
    const int k = eff_rank(e.k_dev, a, e.r_max);
    for (int j = 0; j < k; ++j) {
      float zj = 0.f;
      for (int c = 0; c < e.n_chunks; ++c) zj += e.z[(int64_t(c) * e.cap + p) * e.r_max + j];
      const float wj = al * zj;
      float b[8];
      load8<TW>(B + (int64_t(a) * e.r_max + j) * e.d_out + n0, b);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj, b[q], acc[q]);
    }
  }
  TY *Y = static_cast<TY *>(e.y);
  add_store8<TY>(Y + int64_t(t) * e.ldy + n0, acc);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int rank_bucket(int r) { return r <= 8 ? 8 : r <= 16 ? 16 : r <= 32 ? 32 : 64; }

static int check_module(const tcl_module *m) {
  if (!m) return fail(TCL_EINVAL, "module is NULL");
  if (!m->A_t || !m->B_t) return fail(TCL_EINVAL, "module factors must not be NULL");
  if (m->n_adapters < 1 || m->d_in < 1 || m->d_out < 1)
    return fail(TCL_EINVAL, "module sizes must be positive (N %d, d_in %d, d_out %d)",
                m->n_adapters, m->d_in, m->d_out);
  if (m->r_max < 1 || m->r_max > TCL_MAX_RANK)
    return fail(TCL_EUNSUPPORTED, "r_max %d outside 1..%d", m->r_max, TCL_MAX_RANK);
  if (m->wdtype != TCL_BF16 && m->wdtype != TCL_F32)
    return fail(TCL_EINVAL, "unknown weight dtype %d", int(m->wdtype));
  if ((m->d_in % 8) || (m->d_out % 8))
    return fail(TCL_EALIGN, "d_in %d and d_out %d must be multiples of 8", m->d_in, m->d_out);
  if ((reinterpret_cast<uintptr_t>(m->A_t) | reinterpret_cast<uintptr_t>(m->B_t)) & 15)
    return fail(TCL_EALIGN, "A_t and B_t must be 16-byte aligned");
  return TCL_OK;
}

static int check_plan_module(const tcl_plan *p, const tcl_module *m) {
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  int rc = check_module(m);
  if (rc) return rc;
  if (m->n_adapters != p->L.N)
    return fail(TCL_EINVAL, "module has %d adapters, plan was built for %d", m->n_adapters,
                p->L.N);
  return TCL_OK;
}

static int check_io(const void *ptr, int64_t ld, int32_t d, const char *what) {
  if (!ptr) return fail(TCL_EINVAL, "%s is NULL", what);
  if (reinterpret_cast<uintptr_t>(ptr) & 15) return fail(TCL_EALIGN, "%s must be 16-byte aligned", what);
  if (ld < d) return fail(TCL_EINVAL, "leading dimension of %s (%lld) < %d", what, (long long)ld, d);
  if (ld % 8) return fail(TCL_EALIGN, "leading dimension of %s must be a multiple of 8", what);
  return TCL_OK;
}

static int check_dtypes(const tcl_module *m, tcl_dtype xd, tcl_dtype yd, bool need_y) {
  if (m->wdtype == TCL_BF16) {
    if (xd != TCL_BF16) return fail(TCL_EUNSUPPORTED, "bf16 weights need bf16 x");
    if (need_y && yd != TCL_F32 && yd != TCL_BF16)
      return fail(TCL_EUNSUPPORTED, "bf16 mode supports fp32 or bf16 y");
  } else {
    if (xd != TCL_F32) return fail(TCL_EUNSUPPORTED, "fp32 weights need fp32 x");
    if (need_y && yd != TCL_F32) return fail(TCL_EUNSUPPORTED, "fp32 mode needs fp32 y");
  }
  return TCL_OK;
}

// d_in chunks for the shrink: enough work items to fill the chip, chunks of
// at least one wave-step (64 granules).
static int shrink_chunks(const tcl_plan *p, const tcl_module *m, int allow_split) {
  if (!allow_split) return 1;
  const int vec = m->wdtype == TCL_BF16 ? 8 : 4;
  const int n_gran = m->d_in / vec;
  const int max_chunks = (n_gran + 63) / 64;
  int est_items = p->L.cap < p->L.N ? p->L.cap : p->L.N;
  est_items += p->L.cap / (4 * kTile);
  if (est_items < 1) est_items = 1;
  int c = (1024 + est_items - 1) / est_items;
  if (c > max_chunks) c = max_chunks;
  if (c < 1) c = 1;
  return c;
}

static int chunk_gran(const tcl_module *m, int n_chunks) {
  const int vec = m->wdtype == TCL_BF16 ? 8 : 4;
  const int n_gran = m->d_in / vec;
  int g = (n_gran + n_chunks - 1) / n_chunks;
  return (g + 63) / 64 * 64;
}

template <int R, typename TIN>
static void launch_shrink_t(const ShrinkArgs &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((shrink_valu<R, TIN>), dim3(grid), dim3(256), 0, s, a);
}

static int launch_shrink(const tcl_plan *p, const tcl_module *m, const void *x, int64_t ldx,
                         float *z, int n_chunks, int zero_tail, hipStream_t s) {
  ShrinkArgs a;
  a.status = p->d.status;
  a.items = p->d.items;
  a.tup_token = p->d.tup_token;
  a.k_dev = m->k_dev;
  a.A_t = m->A_t;
  a.x = x;
  a.ldx = ldx;
  a.d_in = m->d_in;
  a.r_max = m->r_max;
  a.cap = p->L.cap;
  a.n_chunks = n_chunks;
  a.chunk_gran = chunk_gran(m, n_chunks);
  a.zero_tail = zero_tail;
  a.z = z;
  int64_t grid = int64_t(p->L.items_cap) * n_chunks;
  if (grid > 16384) grid = 16384;
  if (grid < 1) grid = 1;
  const int R = rank_bucket(m->r_max);
  logf("shrink: d_in=%d r_max=%d R=%d chunks=%d gran=%d grid=%lld", m->d_in, m->r_max, R,
       n_chunks, a.chunk_gran, (long long)grid);
  const bool bf = m->wdtype == TCL_BF16;
#define TCL_SHRINK_CASE(RR)                                           \
  case RR:                                                            \
    if (bf) launch_shrink_t<RR, bf16_t>(a, int(grid), s);             \
    else launch_shrink_t<RR, float>(a, int(grid), s);                 \
    break;
  switch (R) {
    TCL_SHRINK_CASE(8)
    TCL_SHRINK_CASE(16)
    TCL_SHRINK_CASE(32)
    TCL_SHRINK_CASE(64)
  }
#undef TCL_SHRINK_CASE
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

template <int R, typename TW, typename TY>
static void launch_expand_t(const ExpandArgs &e, int grid, hipStream_t s) {
  hipLaunchKernelGGL((expand_valu<R, TW, TY>), dim3(grid), dim3(64), 0, s, e);
}

static int launch_expand(const tcl_plan *p, const tcl_module *m, const float *z, int n_chunks,
                         void *y, int64_t ldy, tcl_dtype yd, hipStream_t s) {
  if (p->L.T == 0) return TCL_OK;
  ExpandArgs e;
  e.status = p->d.status;
  e.tok_ptr = p->d.tok_ptr;
  e.tok_tuple = p->d.tok_tuple;
  e.tup_adapter = p->d.tup_adapter;
  e.tup_alpha = p->d.tup_alpha;
  e.k_dev = m->k_dev;
  e.B_t = m->B_t;
  e.z = z;
  e.y = y;
  e.ldy = ldy;
  e.d_out = m->d_out;
  e.r_max = m->r_max;
  e.cap = p->L.cap;
  e.n_chunks = n_chunks;
  e.n_coltiles = (m->d_out + 511) / 512;
  const int64_t grid = int64_t(p->L.T) * e.n_coltiles;
  if (grid > 0x7fffffff) return fail(TCL_EUNSUPPORTED, "expand grid too large");
  const int R = rank_bucket(m->r_max);
  logf("expand: d_out=%d R=%d coltiles=%d grid=%lld chunks=%d", m->d_out, R, e.n_coltiles,
       (long long)grid, n_chunks);
  const bool bf = m->wdtype == TCL_BF16;
  const bool ybf = yd == TCL_BF16;
#define TCL_EXPAND_CASE(RR)                                                   \
  case RR:                                                                    \
    if (bf && ybf) launch_expand_t<RR, bf16_t, bf16_t>(e, int(grid), s);      \
    else if (bf) launch_expand_t<RR, bf16_t, float>(e, int(grid), s);         \
    else launch_expand_t<RR, float, float>(e, int(grid), s);                  \
    break;
  switch (R) {
    TCL_EXPAND_CASE(8)
    TCL_EXPAND_CASE(16)
    TCL_EXPAND_CASE(32)
    TCL_EXPAND_CASE(64)
  }
#undef TCL_EXPAND_CASE
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

static size_t zpart_bytes(const tcl_plan *p, const tcl_module *m) {
  const int c = shrink_chunks(p, m, 1);
  return (size_t(c) * size_t(p->L.cap) * size_t(m->r_max) * 4 + 255) & ~size_t(255);
}

}  // namespace tcl

using namespace tcl;

extern "C" {

int tcl_module_load_ranks(tcl_module *m, const int32_t *k_host, int32_t *k_dev, void *stream) {
  if (!m || !k_host || !k_dev) return fail(TCL_EINVAL, "module, k_host and k_dev are required");
  if (m->n_adapters < 1) return fail(TCL_EINVAL, "module has no adapters");
  for (int a = 0; a < m->n_adapters; ++a)
    if (k_host[a] < 0 || k_host[a] > m->r_max)
      return fail(TCL_EINVAL, "effective rank k[%d] = %d outside [0, %d]", a, k_host[a], m->r_max);
  hipStream_t s = static_cast<hipStream_t>(stream);
  TCL_HIP(hipMemcpyAsync(k_dev, k_host, size_t(m->n_adapters) * 4, hipMemcpyHostToDevice, s));
  TCL_HIP(hipStreamSynchronize(s));
  m->k_dev = k_dev;
  return TCL_OK;
}

int tcl_workspace_bytes(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                        size_t *bytes) {
  if (!bytes) return fail(TCL_EINVAL, "bytes is NULL");
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  if (n_mods < 0 || (n_mods > 0 && !mods)) return fail(TCL_EINVAL, "bad module list");
  size_t need = 256;
  for (int i = 0; i < n_mods; ++i) {
    int rc = check_plan_module(p, &mods[i]);
    if (rc) return rc;
    const size_t b = zpart_bytes(p, &mods[i]);
    if (b > need) need = b;
  }
  *bytes = need;
  return TCL_OK;
}

int tcl_shrink(const tcl_plan *p, const tcl_module *m, const void *x, int64_t ldx, tcl_dtype xd,
               float *z, void *stream) {
  int rc = check_plan_module(p, m);
  if (rc) return rc;
  if ((rc = check_dtypes(m, xd, TCL_F32, false))) return rc;
  if ((rc = check_io(x, ldx, m->d_in, "x"))) return rc;
  if (!z) return fail(TCL_EINVAL, "z is NULL");
  if (reinterpret_cast<uintptr_t>(z) & 15) return fail(TCL_EALIGN, "z must be 16-byte aligned");
  return launch_shrink(p, m, x, ldx, z, 1, 1, static_cast<hipStream_t>(stream));
}

int tcl_expand(const tcl_plan *p, const tcl_module *m, const float *z, void *y, int64_t ldy,
               tcl_dtype yd, void *stream) {
  int rc = check_plan_module(p, m);
  if (rc) return rc;
  if ((rc = check_dtypes(m, m->wdtype, yd, true))) return rc;
  if ((rc = check_io(y, ldy, m->d_out, "y"))) return rc;
  if (!z) return fail(TCL_EINVAL, "z is NULL");
  return launch_expand(p, m, z, 1, y, ldy, yd, static_cast<hipStream_t>(stream));
}

int tcl_fused_apply(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                    const void *const *x, const int64_t *ldx, tcl_dtype xd, void *const *y,
                    const int64_t *ldy, tcl_dtype yd, void *ws, size_t ws_bytes,
                    void *stream) {
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  if (n_mods < 1 || !mods || !x || !ldx || !y || !ldy)
    return fail(TCL_EINVAL, "module, x and y lists are required");
  size_t need = 0;
  for (int i = 0; i < n_mods; ++i) {
    int rc = check_plan_module(p, &mods[i]);
    if (rc) return rc;
    if ((rc = check_dtypes(&mods[i], xd, yd, true))) return rc;
    if ((rc = check_io(x[i], ldx[i], mods[i].d_in, "x"))) return rc;
    if ((rc = check_io(y[i], ldy[i], mods[i].d_out, "y"))) return rc;
    const size_t b = zpart_bytes(p, &mods[i]);
    if (b > need) need = b;
  }
  if (!ws) return fail(TCL_EINVAL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(TCL_EALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(TCL_ENOSPC, "workspace holds %zu bytes, needs %zu", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *zp = static_cast<float *>(ws);
  for (int i = 0; i < n_mods; ++i) {
    const int c = shrink_chunks(p, &mods[i], 1);
    int rc = launch_shrink(p, &mods[i], x[i], ldx[i], zp, c, 0, s);
    if (rc) return rc;
    rc = launch_expand(p, &mods[i], zp, c, y[i], ldy[i], yd, s);
    if (rc) return rc;
  }
  return TCL_OK;
}

}  // extern "C"
