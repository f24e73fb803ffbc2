// Shrink, expand and the fused apply of the composite multi-LoRA path.
//
//   shrink  (LoRAForge approach (4), segmented shrink): z_p = A_a[:, :k]^T
//           x_{t_p} for one work item (an adapter and up to kTile consecutive
//           tuples of its segment) and one tile of 16 rank rows, on the
//           matrix cores in bf16 (shrink_mfma, shrink_mfma_pair, plan_shrink)
//           or with fp32 dot products and a wave butterfly (shrink_valu).
//           Decode batches split d_in into K chunks whose partial z rows the
//           expand adds in chunk order.
//   expand  (LoRAForge approach (4), RowExpand; DyMerge-LoRA aggregation
//           stage): one wave owns 64 * CPL consecutive outputs of one token
//           and adds alpha_s * B_a[n, :k] z_s for the token's slots in order,
//           in fp32, then adds the total to y once (expand_kernel).  Prefill
//           batches run over 64-token tiles on the matrix cores instead
//           (tile_prep + expand_tile).  Each output element has exactly one
//           owner; there are no atomics.
//
// A plan whose composite table was rejected has an empty token index and no
// work items, so every kernel below finds nothing to do.

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <type_traits>
#include <vector>

#include "plan_core.hpp"
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
// multi-module launch tables
// ---------------------------------------------------------------------------
// One launch covers up to kMaxMods modules (tcl_internal.hpp) that share the
// plan.

struct ModArgs {
  const void *W;          // shrink: A_t, expand: B_t
  void *io;               // shrink: x, expand: y
  const int32_t *k_dev;   // effective ranks or NULL
  float *z;               // [cap][zld]
  int64_t ld;             // leading dimension of io (elements)
  int32_t zld;            // row stride of z (r_max, or r_max rounded up to 4)
  int32_t d;              // shrink: d_in, expand: d_out
  int32_t r_max;
  int32_t first;          // shrink: first unit, expand: first job
  int32_t n_ct;           // expand: column tiles
  int32_t nkc;            // K chunks the shrink splits d_in into (z partial planes)
  int32_t kchunk;         // elements of d_in per K chunk (multiple of 32)
  int32_t zstride;        // floats per tuple row of z: nkc partial rows of zld
};

struct ShrinkArgs {
  const int32_t *status;
  const Item *items;
  int32_t n_mods, rg_total, items_cap;
  int32_t zero_tail;  // write zeros for k <= j < r_max
  ModArgs m[kMaxMods];
};

// Granules each lane has in flight per token pass.
constexpr int kShrinkUnroll = 8;

// fp32 path.  One workgroup = 4 waves = 4 consecutive rank rows j of one work
// item of one module.  A wave streams row j of A_a^T once per pair of tokens
// (the second pass over a row comes from L1/L2) together with the item's x
// rows, with kShrinkUnroll 16-byte granules per lane in flight, then folds
// each token's 64 lane partials with a butterfly in a fixed order and writes
// z final.
template <typename TIN>
__global__ __launch_bounds__(256) void shrink_valu(ShrinkArgs s) {
  constexpr int VEC = Gran<TIN>::kElems;
  constexpr int U = kShrinkUnroll;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n_items = s.status[ST_ITEMS];
  const int total = n_items * s.rg_total;

  for (int job = blockIdx.x; job < total; job += gridDim.x) {
    const int item = job / s.rg_total, rgg = job - item * s.rg_total;
    int mi = 0;
#pragma unroll
    for (int i = 1; i < kMaxMods; ++i)
      if (i < s.n_mods && rgg >= s.m[i].first) mi = i;
    const ModArgs M = s.m[mi];
    const int j = (rgg - M.first) * 4 + w;
    if (j >= M.r_max) continue;
    const Item it = s.items[item];
    const int a = it.head.x, p0 = it.head.y, ntok = it.head.z;
    const int k = eff_rank(M.k_dev, a, M.r_max);
    if (j >= k) {
      if (s.zero_tail && lane < ntok) M.z[int64_t(p0 + lane) * M.zld + j] = 0.f;
      continue;
    }
    const int n_gran = M.d / VEC;
    const int *tok = it.tok;
    const TIN *Arow = static_cast<const TIN *>(M.W) + (int64_t(a) * M.r_max + j) * M.d;
    const TIN *X = static_cast<const TIN *>(M.io);
#pragma unroll
    for (int tb = 0; tb < kTile; tb += 2) {
      if (tb >= ntok) break;
      const bool two = tb + 1 < ntok;
      const TIN *X0 = X + int64_t(tok[tb]) * M.ld;
      const TIN *X1 = X + int64_t(tok[two ? tb + 1 : tb]) * M.ld;
      float acc0 = 0.f, acc1 = 0.f;
      for (int g0 = lane; g0 < n_gran; g0 += 64 * U) {
        Gran<TIN> av[U], xa[U], xb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int g = g0 + 64 * u;
          if (g < n_gran) {
            av[u].load(Arow + int64_t(g) * VEC);
            xa[u].load(X0 + int64_t(g) * VEC);
            if (two) xb[u].load(X1 + int64_t(g) * VEC);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int g = g0 + 64 * u;
          if (g < n_gran) {
            acc0 = av[u].dot(xa[u], acc0);
            if (two) acc1 = av[u].dot(xb[u], acc1);
          }
        }
      }
      acc0 = wave_sum(acc0);
      if (lane == 0) M.z[int64_t(p0 + tb) * M.zld + j] = acc0;
      if (two) {
        acc1 = wave_sum(acc1);
        if (lane == 0) M.z[int64_t(p0 + tb + 1) * M.zld + j] = acc1;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// bf16 shrink on the matrix cores
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int kShrinkWaves = 8;   // waves per workgroup, splitting d_in
constexpr int kShrinkSteps = 8;   // 32-element K steps each lane has in flight

// z[tokens x ranks] = X[tokens x d_in] . A_a^T[d_in x ranks] for one work item
// (up to 16 tuples of one adapter) and one tile of 16 rank rows, with
// v_mfma_f32_16x16x32_bf16.  Both operands load straight from memory: lane l
// holds 8 consecutive d of token row (l % 16) for the first operand and of rank
// row (l % 16) of A_a^T (rank-major, so 16 contiguous bytes) for the second;
// rows past the item's tuple count or the adapter's effective rank are zero
// and never read.  The 8 waves split the K steps of d_in, each keeping
// kShrinkSteps steps of loads in flight, and their partial tiles are summed
// through LDS in wave order.  z is written final.
// Jobs job0, job0 + stride, ... of one workgroup (8 waves); each lane keeps
// STEPS K steps of loads in flight.
template <int STEPS>
__device__ inline void shrink_mfma_jobs(const ShrinkArgs &s, int job0, int stride,
                                        f32x4_t (*red)[64], const Item *litems = nullptr,
                                        int n_litems = 0) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  // The item record of the first job is fetched together with the item count
  // (clamped to the item table, which a padded grid may pass), which saves
  // one dependent memory round trip.
  // litems: the work items in LDS (a mapping stage run by this workgroup),
  // else the plan's item table
  const Item *items = litems ? litems : s.items;
  const int cap = litems ? max(n_litems, 1) : s.items_cap;
  int job = job0;
  const int item0 = min(job / s.rg_total, cap - 1);
  int4 head = items[item0].head;
  int tokl = items[item0].tok[row];
  const int n_items = litems ? n_litems : s.status[ST_ITEMS];
  const int total = n_items * s.rg_total;

  for (; job < total; job += stride) {
    const int item = job / s.rg_total, rgg = job - item * s.rg_total;
    if (job != job0 || item != item0) {
      head = items[item].head;
      tokl = items[item].tok[row];
    }
    int mi = 0;
#pragma unroll
    for (int i = 1; i < kMaxMods; ++i)
      if (i < s.n_mods && rgg >= s.m[i].first) mi = i;
    const int first = s.m[mi].first, dd = s.m[mi].d, r_max = s.m[mi].r_max, zld = s.m[mi].zld;
    const int nkc = s.m[mi].nkc, kchunk = s.m[mi].kchunk;
    const int64_t ld = s.m[mi].ld;
    const int32_t *k_dev = s.m[mi].k_dev;
    const bf16_t *Aw = static_cast<const bf16_t *>(s.m[mi].W);
    const bf16_t *Xw = static_cast<const bf16_t *>(s.m[mi].io);
    const int unit = rgg - first;
    const int rt = unit / nkc, kc = unit - rt * nkc;  // rank tile, K chunk
    const int zstride = s.m[mi].zstride;
    float *Z = s.m[mi].z + kc * zld;  // this chunk's partial row inside each tuple row
    const int j0 = rt * 16;
    const int a = head.x, p0 = head.y, ntok = head.z;
    const int k = eff_rank(k_dev, a, r_max);
    if (j0 >= k) {
      // whole rank tile beyond the effective rank
      if (s.zero_tail && w == 0) {
        const int j = j0 + row;
        for (int tt = kg; tt < ntok; tt += 4)
          if (j < r_max) Z[int64_t(p0 + tt) * zstride + j] = 0.f;
      }
      continue;
    }
    const int tok = row < ntok ? tokl : -1;
    const int jr = j0 + row;  // rank row this lane feeds
    const bf16_t *Xr = tok >= 0 ? Xw + int64_t(tok) * ld + kg * 8 : nullptr;
    const bf16_t *Ar = jr < k ? Aw + (int64_t(a) * r_max + jr) * dd + kg * 8 : nullptr;
    // K steps of this chunk, split over the waves
    const int c0 = kc * (kchunk / 32), c1 = min((dd + 31) / 32, c0 + kchunk / 32);
    const int per = (c1 - c0 + kShrinkWaves - 1) / kShrinkWaves;
    const int s0 = c0 + w * per, s1 = min(c1, s0 + per);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int st = s0; st < s1; st += STEPS) {
      bf16x8_t xv[STEPS], av[STEPS];
#pragma unroll
      for (int u = 0; u < STEPS; ++u) {
        const int e0 = (st + u) * 32 + kg * 8;  // first element of this lane's granule
        const bool in = st + u < s1 && e0 < dd;
        uint4 xb = make_uint4(0, 0, 0, 0), ab = make_uint4(0, 0, 0, 0);
        if (in && Xr) xb = *reinterpret_cast<const uint4 *>(Xr + (st + u) * 32);
        if (in && Ar) ab = *reinterpret_cast<const uint4 *>(Ar + (st + u) * 32);
        xv[u] = __builtin_bit_cast(bf16x8_t, xb);
        av[u] = __builtin_bit_cast(bf16x8_t, ab);
      }
#pragma unroll
      for (int u = 0; u < STEPS; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[u], av[u], acc, 0, 0, 0);
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
      f32x4_t sum = red[0][lane];
#pragma unroll
      for (int v = 1; v < kShrinkWaves; ++v) {
        const f32x4_t o = red[v][lane];
        sum[0] += o[0];
        sum[1] += o[1];
        sum[2] += o[2];
        sum[3] += o[3];
      }
      // lane holds tokens 4*kg .. 4*kg+3 of rank column j0 + row
      const int j = j0 + row;
      if (j < r_max) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = 4 * kg + i;
          if (tt < ntok) {
            if (j < k) Z[int64_t(p0 + tt) * zstride + j] = sum[i];
            else if (s.zero_tail) Z[int64_t(p0 + tt) * zstride + j] = 0.f;
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int STEPS>
__global__ __launch_bounds__(64 * kShrinkWaves) void shrink_mfma(ShrinkArgs s) {
  __shared__ f32x4_t red[kShrinkWaves][64];
  shrink_mfma_jobs<STEPS>(s, blockIdx.x, gridDim.x, red);
}

// Item pairs: one job takes work items 2q and 2q + 1 of one (rank tile, K
// chunk, module) unit.  When both belong to the same adapter (consecutive
// items of one segment) they share every A-row load and run two matrix-core
// accumulators, one per item; otherwise the items run one after the other.
// Each accumulator sees the same K steps in the same order as in
// shrink_mfma_jobs, and the wave partials are summed in the same wave order,
// so z is bit for bit that of shrink_mfma.  Half as many jobs, and half the A
// rows moved into the compute units, for prefill batches whose segments span
// several items.
template <int STEPS>
__device__ inline void shrink_pair_body(const ShrinkArgs &s, int rgg, int4 h0, int tok0,
                                        bool two, int4 h1, int tok1, f32x4_t (*red)[64]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  int mi = 0;
#pragma unroll
  for (int i = 1; i < kMaxMods; ++i)
    if (i < s.n_mods && rgg >= s.m[i].first) mi = i;
  const int first = s.m[mi].first, dd = s.m[mi].d, r_max = s.m[mi].r_max, zld = s.m[mi].zld;
  const int nkc = s.m[mi].nkc, kchunk = s.m[mi].kchunk;
  const int64_t ld = s.m[mi].ld;
  const bf16_t *Aw = static_cast<const bf16_t *>(s.m[mi].W);
  const bf16_t *Xw = static_cast<const bf16_t *>(s.m[mi].io);
  const int unit = rgg - first;
  const int rt = unit / nkc, kc = unit - rt * nkc;
  const int zstride = s.m[mi].zstride;
  float *Z = s.m[mi].z + kc * zld;
  const int j0 = rt * 16;
  const int a = h0.x;
  const int k = eff_rank(s.m[mi].k_dev, a, r_max);
  const int n0 = h0.z, n1 = two ? h1.z : 0;
  if (j0 >= k) {
    if (s.zero_tail && w == 0) {
      const int j = j0 + row;
      if (j < r_max) {
        for (int tt = kg; tt < n0; tt += 4) Z[int64_t(h0.y + tt) * zstride + j] = 0.f;
        for (int tt = kg; tt < n1; tt += 4) Z[int64_t(h1.y + tt) * zstride + j] = 0.f;
      }
    }
    return;
  }
  const int jr = j0 + row;
  const bf16_t *X0 = row < n0 ? Xw + int64_t(tok0) * ld + kg * 8 : nullptr;
  const bf16_t *X1 = row < n1 ? Xw + int64_t(tok1) * ld + kg * 8 : nullptr;
  const bf16_t *Ar = jr < k ? Aw + (int64_t(a) * r_max + jr) * dd + kg * 8 : nullptr;
  const int c0 = kc * (kchunk / 32), c1 = min((dd + 31) / 32, c0 + kchunk / 32);
  const int per = (c1 - c0 + kShrinkWaves - 1) / kShrinkWaves;
  const int s0 = c0 + w * per, s1 = min(c1, s0 + per);
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int st = s0; st < s1; st += STEPS) {
    bf16x8_t xv0[STEPS], xv1[STEPS], av[STEPS];
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const int e0 = (st + u) * 32 + kg * 8;
      const bool in = st + u < s1 && e0 < dd;
      uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0), ab = make_uint4(0, 0, 0, 0);
      if (in && Ar) ab = *reinterpret_cast<const uint4 *>(Ar + (st + u) * 32);
      if (in && X0) x0 = *reinterpret_cast<const uint4 *>(X0 + (st + u) * 32);
      if (in && X1) x1 = *reinterpret_cast<const uint4 *>(X1 + (st + u) * 32);
      xv0[u] = __builtin_bit_cast(bf16x8_t, x0);
      xv1[u] = __builtin_bit_cast(bf16x8_t, x1);
      av[u] = __builtin_bit_cast(bf16x8_t, ab);
    }
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv0[u], av[u], acc0, 0, 0, 0);
      if (two) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv1[u], av[u], acc1, 0, 0, 0);
    }
  }
  red[w][lane] = acc0;
  red[kShrinkWaves + w][lane] = acc1;
  __syncthreads();
  // wave 0 finishes the first item, wave 1 the second
  if (w < (two ? 2 : 1)) {
    const int base = w * kShrinkWaves, p0 = w ? h1.y : h0.y, nt = w ? n1 : n0;
    f32x4_t sum = red[base][lane];
#pragma unroll
    for (int v = 1; v < kShrinkWaves; ++v) {
      const f32x4_t o = red[base + v][lane];
      sum[0] += o[0];
      sum[1] += o[1];
      sum[2] += o[2];
      sum[3] += o[3];
    }
    const int j = j0 + row;
    if (j < r_max) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = 4 * kg + i;
        if (tt < nt) {
          if (j < k) Z[int64_t(p0 + tt) * zstride + j] = sum[i];
          else if (s.zero_tail) Z[int64_t(p0 + tt) * zstride + j] = 0.f;
        }
      }
    }
  }
  __syncthreads();
}

template <int STEPS>
__global__ __launch_bounds__(64 * kShrinkWaves) void shrink_mfma_pair(ShrinkArgs s) {
  __shared__ f32x4_t red[2 * kShrinkWaves][64];
  const int row = threadIdx.x & 15;
  const int n_items = min(s.status[ST_ITEMS], s.items_cap);
  const int total = (n_items + 1) / 2 * s.rg_total;
  for (int job = blockIdx.x; job < total; job += gridDim.x) {
    const int q = job / s.rg_total, rgg = job - q * s.rg_total;
    const int i0 = 2 * q, i1 = 2 * q + 1;
    const int4 h0 = s.items[i0].head;
    const int t0 = s.items[i0].tok[row];
    const bool has1 = i1 < n_items;
    int4 h1 = h0;
    int t1 = t0;
    if (has1) {
      h1 = s.items[i1].head;
      t1 = s.items[i1].tok[row];
    }
    if (has1 && h1.x == h0.x) {
      shrink_pair_body<STEPS>(s, rgg, h0, t0, true, h1, t1, red);
    } else {
      shrink_pair_body<STEPS>(s, rgg, h0, t0, false, h0, t0, red);
      if (has1) shrink_pair_body<STEPS>(s, rgg, h1, t1, false, h1, t1, red);
    }
  }
}

// ---------------------------------------------------------------------------
// decode step: the mapping stage inside the shrink launch
// ---------------------------------------------------------------------------
// For tables of the direct mapping mode (every decode batch) the mapping
// stage runs inside the shrink launch, on each workgroup's own LDS copy of
// the table (a few KiB: LDS work, no extra dependent memory round trip).
// Workgroup 0 runs all of it and writes the plan out for the expand and the
// host; it takes no shrink job.  Every other workgroup keeps the work items
// in LDS and runs its shrink jobs on them: on small tables it stops the
// mapping stage at the item heads and fills the token lists of its own items
// only.  The mapping stage is deterministic, so every workgroup derives the
// same items and the jobs split exactly as in shrink_mfma.  The verdict on
// the table is workgroup 0's: a rejected table leaves an empty token index,
// so the expand does nothing.  This takes one launch and the plan's
// write-then-read round trip off a decode step.
constexpr int kFusedLdsInts = 12288;  // direct-mode mapping scratch (48 KiB)
constexpr int kFusedItems = 192;      // work items held in LDS (15 KiB)

template <int STEPS>
__global__ __launch_bounds__(64 * kShrinkWaves) void plan_shrink(PlanArgs A, ShrinkArgs s) {
  __shared__ __align__(16) int lds[kFusedLdsInts];
  __shared__ int tmp[6 * kSlotInts];
  __shared__ Item li[kFusedItems];
  __shared__ f32x4_t red[kShrinkWaves][64];
  constexpr int NT = 64 * kShrinkWaves;
  // Workgroup 0 runs the whole mapping stage and writes the plan; it has no
  // shrink job.  The others need only the work items of their own jobs: on
  // small tables they stop the mapping stage at the item heads and fill the
  // token lists of just those items.
  const bool lead = blockIdx.x == 0, small = A.G <= NT && A.NP <= NT;
  int n_items;
  const int rc = plan_run<NT, PLAN_DIRECT>(A, lds, tmp, lead, li, kFusedItems, &n_items,
                                           small && !lead);
  if (rc != TCL_OK || lead) return;
  const int job0 = blockIdx.x - 1, stride = gridDim.x - 1;
  if (small) {
    const int total = n_items * s.rg_total;
    int last = -1, calls = 0;
    for (int job = job0; job < total; job += stride) {
      const int item = job / s.rg_total;
      if (item == last) continue;
      plan_small_item_tokens<NT>(A, lds, tmp + (3 + (calls & 1)) * kSlotInts, li, item);
      last = item;
      ++calls;
    }
  }
  __syncthreads();  // the items in LDS are complete
  shrink_mfma_jobs<STEPS>(s, job0, stride, red, li, n_items);
}

// ---------------------------------------------------------------------------
// expand
// ---------------------------------------------------------------------------
struct ExpandArgs {
  const int32_t *tok_n;
  const int4 *tok_rec;  // [T][kSlotPad]
  int32_t T, n_mods, jobs, jobs_per_xcd;
  ModArgs m[kMaxMods];
};


// C consecutive weights of one B row (C = 2, 4 or 8)
template <typename TW, int C>
struct RowN;

template <int C>
struct RowN<bf16_t, C> {
  uint32_t w[C / 2];
  __device__ inline void load(const bf16_t *p) {
    if constexpr (C == 8) {
      const uint4 v = *reinterpret_cast<const uint4 *>(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (C == 4) {
      const uint2 v = *reinterpret_cast<const uint2 *>(p);
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t *>(p);
    }
  }
  __device__ inline void zero() {
#pragma unroll
    for (int i = 0; i < C / 2; ++i) w[i] = 0;
  }
  __device__ inline void fma_into(float x, float (&acc)[C]) const {
#pragma unroll
    for (int i = 0; i < C / 2; ++i) {
      acc[2 * i] = fmaf(x, bf16_lo(w[i]), acc[2 * i]);
      acc[2 * i + 1] = fmaf(x, bf16_hi(w[i]), acc[2 * i + 1]);
    }
  }
};

template <int C>
struct RowN<float, C> {
  float f[C];
  __device__ inline void load(const float *p) {
#pragma unroll
    for (int i = 0; i < C; i += 2) {
      const float2 v = reinterpret_cast<const float2 *>(p)[i / 2];
      f[i] = v.x;
      f[i + 1] = v.y;
    }
  }
  __device__ inline void zero() {
#pragma unroll
    for (int i = 0; i < C; ++i) f[i] = 0.f;
  }
  __device__ inline void fma_into(float x, float (&acc)[C]) const {
#pragma unroll
    for (int i = 0; i < C; ++i) acc[i] = fmaf(x, f[i], acc[i]);
  }
};

// C consecutive outputs
template <typename TY, int C>
struct OutN;

// y is touched once per launch: its loads and stores carry the non-temporal
// hint so that the streamed rows do not evict the B rows held in L2.
typedef float nt_f2 __attribute__((ext_vector_type(2)));
typedef float nt_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u2 __attribute__((ext_vector_type(2)));
typedef uint32_t nt_u4 __attribute__((ext_vector_type(4)));

template <>
struct OutN<float, 1> {
  float f;
  __device__ inline void load(const float *p) { f = __builtin_nontemporal_load(p); }
  __device__ inline void add_store(float *p, const float (&acc)[1]) {
    __builtin_nontemporal_store(f + acc[0], p);
  }
};

template <>
struct OutN<bf16_t, 1> {
  uint16_t h;
  __device__ inline void load(const bf16_t *p) {
    h = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
  }
  __device__ inline void add_store(bf16_t *p, const float (&acc)[1]) {
    const uint16_t o = f32_to_bf16(__uint_as_float(uint32_t(h) << 16) + acc[0]);
    __builtin_nontemporal_store(o, reinterpret_cast<uint16_t *>(p));
  }
};

template <int C>
struct OutN<float, C> {
  float f[C];
  __device__ inline void load(const float *p) {
    if constexpr (C % 4 == 0) {
#pragma unroll
      for (int i = 0; i < C; i += 4) {
        const nt_f4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f4 *>(p) + i / 4);
        f[i] = v.x; f[i + 1] = v.y; f[i + 2] = v.z; f[i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < C; i += 2) {
        const nt_f2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f2 *>(p) + i / 2);
        f[i] = v.x; f[i + 1] = v.y;
      }
    }
  }
  __device__ inline void add_store(float *p, const float (&acc)[C]) {
    if constexpr (C % 4 == 0) {
#pragma unroll
      for (int i = 0; i < C; i += 4) {
        nt_f4 v;
        v.x = f[i] + acc[i]; v.y = f[i + 1] + acc[i + 1];
        v.z = f[i + 2] + acc[i + 2]; v.w = f[i + 3] + acc[i + 3];
        __builtin_nontemporal_store(v, reinterpret_cast<nt_f4 *>(p) + i / 4);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C; i += 2) {
        nt_f2 v;
        v.x = f[i] + acc[i]; v.y = f[i + 1] + acc[i + 1];
        __builtin_nontemporal_store(v, reinterpret_cast<nt_f2 *>(p) + i / 2);
      }
    }
  }
};

template <int C>
struct OutN<bf16_t, C> {
  uint32_t w[C / 2];
  __device__ inline void load(const bf16_t *p) {
    if constexpr (C == 8) {
      const nt_u4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u4 *>(p));
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (C == 4) {
      const nt_u2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u2 *>(p));
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
    }
  }
  __device__ inline void add_store(bf16_t *p, const float (&acc)[C]) {
    uint32_t o[C / 2];
#pragma unroll
    for (int i = 0; i < C / 2; ++i) {
      const uint16_t lo = f32_to_bf16(bf16_lo(w[i]) + acc[2 * i]);
      const uint16_t hi = f32_to_bf16(bf16_hi(w[i]) + acc[2 * i + 1]);
      o[i] = uint32_t(lo) | (uint32_t(hi) << 16);
    }
    if constexpr (C == 8) {
      nt_u4 v;
      v.x = o[0]; v.y = o[1]; v.z = o[2]; v.w = o[3];
      __builtin_nontemporal_store(v, reinterpret_cast<nt_u4 *>(p));
    } else if constexpr (C == 4) {
      nt_u2 v;
      v.x = o[0]; v.y = o[1];
      __builtin_nontemporal_store(v, reinterpret_cast<nt_u2 *>(p));
    } else {
      __builtin_nontemporal_store(o[0], reinterpret_cast<uint32_t *>(p));
    }
  }
};

// One wave = 64 * CPL consecutive outputs (CPL per lane) of one token of one
// module.  Block ids are spread so that every XCD owns a contiguous range of
// (module, column tile) and all tokens of it: the B rows of a column tile are
// fetched into one XCD's L2 once and reused by every token that needs them.
// The token's slot records (padded table, one per lane), its slot count and
// its y values are loaded together at the start; then the B rows of up to 32
// (slot, rank) pairs are loaded before any of them is used.  z is the sum of
// the shrink's K-chunk partials, added in chunk order.  Accumulation is fp32
// in slot order, rank order within a slot; y is added once at the end.
// One expand job (token, 64 * CPL outputs of one module) for the calling wave;
// BR (slot, rank) rows of B are loaded per batch.
template <int R, int CPL, bool SPLIT, typename TW, typename TY, int BR>
__device__ inline void expand_job(const ExpandArgs &e, int job) {
  constexpr int RB = R < BR ? R : BR;  // ranks per batch
  constexpr int SB = BR / RB;          // slots per batch
  const int lane = threadIdx.x & 63;
  if (job >= e.jobs) return;
  int mi = 0;
#pragma unroll
  for (int i = 1; i < kMaxMods; ++i)
    if (i < e.n_mods && job >= e.m[i].first) mi = i;
  // uniform copies of the selected module's fields (kept in SGPRs, loaded once)
  const int first = e.m[mi].first, d = e.m[mi].d, r_max = e.m[mi].r_max, zld = e.m[mi].zld;
  const int nkc = e.m[mi].nkc, zstride = e.m[mi].zstride;
  const int64_t ld = e.m[mi].ld;
  const int32_t *k_dev = e.m[mi].k_dev;
  const float *Z = e.m[mi].z;
  const TW *B = static_cast<const TW *>(e.m[mi].W);
  TY *Y = static_cast<TY *>(e.m[mi].io);
  const int local = job - first;
  const int ct = local / e.T, t = local - ct * e.T;
  const int n0 = (ct * 64 + lane) * CPL;
  const bool active = n0 < d;
  TY *Yp = Y + int64_t(t) * ld + n0;
  OutN<TY, CPL> yv;
  const int ns = e.tok_n[t];
  const int4 rec = e.tok_rec[int64_t(t) * kSlotPad + lane];
  if (ns <= 0) return;

  float acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
  for (int sb = 0; sb < ns; sb += SB) {
    int pp[SB], aa[SB], kk[SB];
    float al[SB];
#pragma unroll
    for (int b = 0; b < SB; ++b) {
      const int sl = sb + b;
      if (sl < ns) {
        pp[b] = __builtin_amdgcn_readlane(rec.x, sl);
        aa[b] = __builtin_amdgcn_readlane(rec.y, sl);
        al[b] = __int_as_float(__builtin_amdgcn_readlane(rec.z, sl));
        kk[b] = eff_rank(k_dev, aa[b], r_max);
      } else {
        pp[b] = 0;
        aa[b] = 0;
        al[b] = 0.f;
        kk[b] = 0;
      }
    }
#pragma unroll
    for (int jb = 0; jb < R; jb += RB) {
      RowN<TW, CPL> bv[SB][RB];
      float zv[SB][RB];
      // all loads of the batch first: B rows of the retained ranks and z
      // (entries at or beyond the effective rank are never used).  A split
      // shrink leaves nkc partial rows per tuple, added here in chunk order.
#pragma unroll
      for (int b = 0; b < SB; ++b) {
#pragma unroll
        for (int jj = 0; jj < RB; ++jj) {
          const int j = jb + jj;
          if (j < kk[b] && active) bv[b][jj].load(B + (int64_t(aa[b]) * r_max + j) * d + n0);
          else bv[b][jj].zero();
        }
        // y right after the first batch's B rows: its latency then overlaps
        // theirs instead of the slot records' (the memory counter is in
        // order, so a load issued before the slot records would be waited
        // for together with them)
        if (sb == 0 && jb == 0 && b == 0 && active) yv.load(Yp);
        if constexpr (!SPLIT) {
          // one z row per tuple, read as whole vectors
          const float *zrow = Z + int64_t(pp[b]) * zld + jb;
          if ((zld & 3) == 0) {
            const float4 *zr = reinterpret_cast<const float4 *>(zrow);
#pragma unroll
            for (int jj = 0; jj < RB; jj += 4) {
              float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
              if (jb + jj < kk[b]) v = zr[jj / 4];
              zv[b][jj] = v.x;
              zv[b][jj + 1] = v.y;
              zv[b][jj + 2] = v.z;
              zv[b][jj + 3] = v.w;
            }
          } else {
#pragma unroll
            for (int jj = 0; jj < RB; ++jj) zv[b][jj] = jb + jj < kk[b] ? zrow[jj] : 0.f;
          }
        } else {
          // nkc partial rows per tuple (zld is a multiple of 4 here)
#pragma unroll
          for (int jj = 0; jj < RB; ++jj) zv[b][jj] = 0.f;
          for (int c = 0; c < nkc; ++c) {
            const float4 *zr = reinterpret_cast<const float4 *>(Z + int64_t(pp[b]) * zstride + c * zld + jb);
#pragma unroll
            for (int jj = 0; jj < RB; jj += 4) {
              if (jb + jj < kk[b]) {
                const float4 v = zr[jj / 4];
                zv[b][jj] += v.x;
                zv[b][jj + 1] += v.y;
                zv[b][jj + 2] += v.z;
                zv[b][jj + 3] += v.w;
              }
            }
          }
        }
      }
#pragma unroll
      for (int b = 0; b < SB; ++b)
#pragma unroll
        for (int jj = 0; jj < RB; ++jj)
          if (jb + jj < kk[b]) bv[b][jj].fma_into(al[b] * zv[b][jj], acc);
    }
  }
  if (active) yv.add_store(Yp, acc);
}

// W waves (jobs) per workgroup.  XCD-aware job index: workgroups are dealt
// to the 8 XCDs round-robin, and each XCD owns a contiguous range of
// jobs_per_xcd workgroups' jobs.
template <int R, int CPL, bool SPLIT, typename TW, typename TY, int W, int BR>
__global__ __launch_bounds__(64 * W) void expand_kernel(ExpandArgs e) {
  const int blk = (blockIdx.x & 7) * e.jobs_per_xcd + (blockIdx.x >> 3);
  // the job is uniform across the wave: say so, so that everything derived
  // from it stays in scalar registers
  const int job = __builtin_amdgcn_readfirstlane(blk * W + int(threadIdx.x >> 6));
  expand_job<R, CPL, SPLIT, TW, TY, BR>(e, job);
}

// ---------------------------------------------------------------------------
// helpers of the prefill expand
// ---------------------------------------------------------------------------
constexpr int kXCols = 256;  // output columns per tile job (4 waves x 64)

// Exclusive prefix sums of two values over the 256 threads, and their totals.
__device__ inline void block_scan2(int v0, int v1, int *tmp, int &x0, int &x1, int &s0,
                                   int &s1) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int i0 = v0, i1 = v1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a0 = __shfl_up(i0, off, 64), a1 = __shfl_up(i1, off, 64);
    if (lane >= off) {
      i0 += a0;
      i1 += a1;
    }
  }
  if (lane == 63) {
    tmp[w] = i0;
    tmp[4 + w] = i1;
  }
  __syncthreads();
  int b0 = 0, b1 = 0;
  s0 = 0;
  s1 = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c0 = tmp[j], c1 = tmp[4 + j];
    if (j < w) {
      b0 += c0;
      b1 += c1;
    }
    s0 += c0;
    s1 += c1;
  }
  __syncthreads();
  x0 = b0 + i0 - v0;
  x1 = b1 + i1 - v1;
}

// The last i in [lo, hi) with a[i] <= v (a ascending, a[lo] <= v).
__device__ inline int last_le(const int *a, int lo, int hi, int v) {
  --hi;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Four consecutive y values.  Plain (not non-temporal) accesses: measured
// faster here than the streaming hint.
template <typename TY>
__device__ inline f32x4_t load_y4(const TY *p) {
  if constexpr (sizeof(TY) == 4) {
    const nt_f4 v = *reinterpret_cast<const nt_f4 *>(p);
    return f32x4_t{v.x, v.y, v.z, v.w};
  } else {
    const nt_u2 v = *reinterpret_cast<const nt_u2 *>(p);
    return f32x4_t{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
  }
}

template <typename TY>
__device__ inline void store_y4(TY *p, f32x4_t v) {
  if constexpr (sizeof(TY) == 4) {
    *reinterpret_cast<nt_f4 *>(p) = nt_f4{v[0], v[1], v[2], v[3]};
  } else {
    *reinterpret_cast<nt_u2 *>(p) =
        nt_u2{uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16),
              uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16)};
  }
}

// ---------------------------------------------------------------------------
// prefill expand over token tiles on the matrix cores
// ---------------------------------------------------------------------------
// The expand of a prefill-sized batch is, per 64-token tile and block of 256
// output columns, a product Y[tokens x cols] += W[tokens x K] . Bcat[K x cols]
// over the tile's union: the adapters its tokens hold, in the plan's segment
// order (ascending id), each contributing its retained ranks in octets of 8
// (ceil(k / 8) octets).  W[t][(a, j)] = bf16(alpha_{t,a} z_{t,a}[j]) when
// token t holds adapter a, else 0 (LoRAForge approach (4), RowExpand: an
// adapter's B rows serve every token of the tile that holds it; DyMerge-LoRA
// section 4.3: one kernel aggregates every (token, adapter) pair).
//
// The matrix cores want both operands with 8 consecutive K values per lane.
// K is the rank here, so the expand reads a packed, rank-contiguous copy of
// the pool (tcl_module_pack, made once when the adapters are loaded: per
// adapter and column its ceil(k / 8) rank octets); its octets load straight
// from memory into the operand registers, with no LDS staging and no
// transposes.  The tiles follow the plan's tile order, which groups tokens
// that share a rare adapter.
//
// tile_prep (one workgroup per (module, tile)) writes the tile's record: its
// tokens (the plan's tile order) and their slot counts; the octet table (for
// octet h of the concatenated K: the octet's first 16-byte unit in the
// packed pool, the union entry, the octet's index inside the adapter and the
// adapter's octet count); the coefficient octets bf16(alpha * z[j]) of every
// tuple of the tile (z summed over the shrink's K-chunk partials in chunk
// order; ranks at or beyond k zero); and, per (token, union entry), the first
// coefficient octet of that pair or -1.  Tiles beyond the record's limits
// (kRMaxQ tuples, kRMaxU union entries, kRHcap octets, kRMaxCoef coefficient
// octets) are marked instead; their jobs run a per-token fp32 loop with the
// arithmetic of expand_kernel.
//
// expand_tile (one workgroup of 4 waves per (module, tile, 256 columns); wave
// w owns 64 columns of all 64 tokens) copies the record into LDS and loads
// its y rows into the accumulators, then walks K four octets (32 ranks) per
// step: each lane loads, three steps ahead, the packed-pool octet of its
// column for each of the four 16-column blocks, and reads from LDS the
// coefficient octet of its token for each of the four 16-token blocks (zero
// where the token does not hold the octet's adapter).
constexpr int kRMaxQ = 1024;     // tuples per tile
constexpr int kRMaxU = 128;      // union entries
constexpr int kRHcap = 256;      // K octets (2048 ranks) per tile
constexpr int kRMaxCoef = 1024;  // coefficient octets per tile
constexpr int kRMaxWords = 128;  // adapter bitmap words: pools of at most 4096 adapters
// record layout (int32 words): header {Q, H, fast, C, U, idx offset, coef
// offset, -}, the tile's tokens, their slot counts, octet table A (first
// 16-byte unit of the octet in the packed pool), octet table B (union entry |
// octet in adapter << 9 | adapter's octets << 12), then at the offsets the
// header gives: idx [64][U] int16 and the coefficient octets [C + 8] (the
// last eight zero).
constexpr int kRTok = 8;
constexpr int kRTokN = kRTok + kXTok;
constexpr int kROctA = kRTokN + kXTok;
constexpr int kRWords = kROctA + 2 * kRHcap + kXTok * kRMaxU / 2 + 4 + 4 * (kRMaxCoef + 8);
static_assert(kROctA % 4 == 0 && kRWords % 4 == 0, "record regions of whole 16-byte units");
static_assert(kXTok * 4 == 256, "four threads per token of a tile");

struct TileArgs {
  const int32_t *status;
  const int32_t *tok_n;
  const int4 *tok_rec;     // [T][kSlotPad]
  const int32_t *tile_tok;  // token order of the tiles (status[ST_BUSY] entries)
  int32_t *rec;            // [n_mods][tiles][kRWords]
  int32_t T, N, tiles, n_mods, jobs, jobs_per_xcd;
  // packed pools (tcl_module_pack): per adapter its first 16-byte unit, and
  // the data, [d_out][ceil(k / 8)] octets per adapter
  const int32_t *bk_off[kMaxMods];
  const uint4 *bk_data[kMaxMods];
  const uint4 *bk_zero[kMaxMods];  // a zero 16-byte unit of each packed pool
  ModArgs m[kMaxMods];  // first = first job; n_ct = column tiles of kXCols
};

// In-place exclusive prefix sum of a[0..n), n <= 1024, over the 256 threads
// (a complete before the call); returns the total.
__device__ inline int lds_scan(int *a, int n, int *tmp) {
  const int tid = threadIdx.x;
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = 4 * tid + i;
    v[i] = idx < n ? a[idx] : 0;
    s += v[i];
  }
  int x0, x1, s0, s1;
  block_scan2(s, 0, tmp, x0, x1, s0, s1);
  int run = x0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = 4 * tid + i;
    if (idx < n) a[idx] = run;
    run += v[i];
  }
  __syncthreads();
  return s0;
}

__global__ __launch_bounds__(256) void tile_prep(TileArgs e) {
  __shared__ int s_n[kXTok], s_t[kXTok], s_off[kXTok + 1];
  __shared__ unsigned s_bm[kRMaxWords];
  __shared__ int s_wp[kRMaxWords];
  __shared__ int s_p[kRMaxQ], s_a[kRMaxQ], s_u[kRMaxQ], s_k[kRMaxQ], s_c[kRMaxQ];
  __shared__ float s_al[kRMaxQ];
  __shared__ int u_h0[kRMaxU + 1], u_a[kRMaxU], u_k[kRMaxU];
  __shared__ int tmp[8];
  __shared__ int s_info[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int mi = blockIdx.x / e.tiles, tile = blockIdx.x - mi * e.tiles;
  int sel = 0;
#pragma unroll
  for (int i = 1; i < kMaxMods; ++i)
    if (i < e.n_mods && mi >= i) sel = i;
  const int r_max = e.m[sel].r_max, zld = e.m[sel].zld, nkc = e.m[sel].nkc;
  const int zstride = e.m[sel].zstride;
  const int32_t *k_dev = e.m[sel].k_dev;
  const float *Z = e.m[sel].z;
  const int32_t *bk_off = e.bk_off[sel];
  int32_t *rec = e.rec + int64_t(blockIdx.x) * kRWords;
  const bool ok = e.status[ST_CODE] == TCL_OK;
  const int busy = ok ? e.status[ST_BUSY] : 0;
  if (tid < kXTok) {
    // row tid of the tile: the plan's tile order
    const int i = tile * kXTok + tid;
    const int t = i < busy ? e.tile_tok[i] : -1;
    int n = t >= 0 ? e.tok_n[t] : 0;
    n = n < 0 ? 0 : (n > kSlotPad ? kSlotPad : n);
    s_n[tid] = n;
    s_t[tid] = t;
    rec[kRTok + tid] = t;
    rec[kRTokN + tid] = n;
  }
  if (tid < kRMaxWords) s_bm[tid] = 0u;
  __syncthreads();
  if (tid < 64) {  // prefix of the slot counts
    const int n = s_n[lane];
    int inc = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(inc, off, 64);
      if (lane >= off) inc += v;
    }
    s_off[lane] = inc - n;
    if (lane == 63) {
      s_off[kXTok] = inc;
      s_info[0] = inc;
    }
  }
  __syncthreads();
  const int Q = s_info[0];
  auto header = [&](int q, int h, int fast, int c, int u, int oidx, int ocoef) {
    if (tid == 0) {
      rec[0] = q;
      rec[1] = h;
      rec[2] = fast;
      rec[3] = c;
      rec[4] = u;
      rec[5] = oidx;
      rec[6] = ocoef;
      rec[7] = 0;
    }
  };
  if (Q == 0) return header(0, 0, 1, 0, 0, 0, 0);
  if (Q > kRMaxQ || e.N > 32 * kRMaxWords) return header(Q, 0, 0, 0, 0, 0, 0);
  // the tile's tuples: thread (token r, sub) takes slots sub, sub + 4, ...
  const int r = tid >> 2, sub = tid & 3;
  const int nr = s_n[r], offr = s_off[r];
  const int tr = s_t[r];
  for (int s = sub; s < nr; s += 4) {
    const int4 rc = e.tok_rec[int64_t(tr) * kSlotPad + s];
    const int q = offr + s;
    const int u = min(max(rc.w, 0), 32 * kRMaxWords - 1);
    s_p[q] = rc.x;
    s_a[q] = rc.y;
    s_al[q] = __int_as_float(rc.z);
    s_u[q] = u;
    atomicOr(&s_bm[u >> 5], 1u << (u & 31));
    s_k[q] = eff_rank(k_dev, rc.y, r_max);
  }
  __syncthreads();
  if (tid < 64) {  // prefix of the bitmap words' bit counts, two words per lane
    const int c0 = __popc(s_bm[2 * lane]), c1 = __popc(s_bm[2 * lane + 1]);
    int inc = c0 + c1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(inc, off, 64);
      if (lane >= off) inc += v;
    }
    s_wp[2 * lane] = inc - c0 - c1;
    s_wp[2 * lane + 1] = inc - c1;
    if (lane == 63) s_info[2] = inc;
  }
  __syncthreads();
  const int nU = s_info[2];
  if (nU > kRMaxU) return header(Q, 0, 0, 0, nU, 0, 0);
  // union entry of each tuple (segments ascending = adapters ascending); per
  // entry its adapter, rank and octet count (every tuple of an entry writes
  // the same values)
  for (int s = sub; s < nr; s += 4) {
    const int q = offr + s, u = s_u[q];
    const int ui = s_wp[u >> 5] + __popc(s_bm[u >> 5] & ((1u << (u & 31)) - 1u));
    const int oc = (s_k[q] + 7) >> 3;
    s_u[q] = ui;
    u_a[ui] = s_a[q];
    u_k[ui] = s_k[q];
    u_h0[ui] = oc;
    s_c[q] = oc;
  }
  __syncthreads();
  const int H = lds_scan(u_h0, nU, tmp);  // first octet of each entry
  const int C = lds_scan(s_c, Q, tmp);    // first coefficient octet of each tuple
  if (H > kRHcap || C > kRMaxCoef) return header(Q, H, 0, C, nU, 0, 0);
  const int oidx = kROctA + 2 * H;                   // int16 [64][nU]
  const int ocoef = (oidx + (kXTok * nU + 1) / 2 + 3) & ~3;  // 16-byte aligned
  // the coefficient octets are followed by eight zero octets, the entry of
  // every (token, union entry) pair the tile does not hold
  if (tid == 0) u_h0[nU] = H;
  __syncthreads();
  for (int h = tid; h < H; h += 256) {
    const int i = last_le(u_h0, 0, nU, h);  // entries without octets (k = 0) are passed over
    const int oi = h - u_h0[i], octs = (u_k[i] + 7) >> 3;
    rec[kROctA + h] = bk_off[u_a[i]] + oi;
    rec[kROctA + H + h] = i | (oi << 9) | (octs << 12);
  }
  // per (token, union entry): first coefficient octet, or the zero octets
  int16_t *idx = reinterpret_cast<int16_t *>(rec + oidx);
  for (int i = tid; i < kXTok * nU; i += 256) idx[i] = int16_t(C);
  __syncthreads();
  for (int s = sub; s < nr; s += 4) {
    const int q = offr + s;
    idx[r * nU + s_u[q]] = int16_t(s_c[q]);
  }
  // coefficient octets bf16(alpha * z) of every tuple
  uint4 *coef = reinterpret_cast<uint4 *>(rec + ocoef);
  for (int f = tid; f < C; f += 256) {
    const int q = last_le(s_c, 0, Q, f);
    const int o = f - s_c[q], j0 = 8 * o, k = s_k[q];
    const float al = s_al[q];
    float zv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) zv[i] = 0.f;
    for (int c = 0; c < nkc; ++c) {
      const float *zr = Z + int64_t(s_p[q]) * zstride + c * zld + j0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i < k) zv[i] += zr[i];
    }
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v0 = j0 + 2 * i < k ? al * zv[2 * i] : 0.f;
      const float v1 = j0 + 2 * i + 1 < k ? al * zv[2 * i + 1] : 0.f;
      pk[i] = uint32_t(f32_to_bf16(v0)) | (uint32_t(f32_to_bf16(v1)) << 16);
    }
    coef[f] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
  if (tid < 8) coef[C + tid] = make_uint4(0, 0, 0, 0);
  header(Q, H, 1, C, nU, oidx, ocoef);
}

// Orders LDS accesses of the workgroup around a barrier without waiting for
// outstanding global loads (a plain __syncthreads() waits for those too).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A tile beyond the record's limits: per token, per slot in order, per rank in
// order, acc = fma(alpha * z_j, B[j][n], acc), then y += acc, as in
// expand_kernel; lane = one column of the wave's 64.
template <typename TY>
__device__ void tile_fallback(const TileArgs &e, int sel, const int *tok, int cw) {
  const int lane = threadIdx.x & 63;
  const int d = e.m[sel].d, r_max = e.m[sel].r_max, zld = e.m[sel].zld;
  const int nkc = e.m[sel].nkc, zstride = e.m[sel].zstride;
  const int64_t ld = e.m[sel].ld;
  const int32_t *k_dev = e.m[sel].k_dev;
  const float *Z = e.m[sel].z;
  const bf16_t *B = static_cast<const bf16_t *>(e.m[sel].W);
  TY *Y = static_cast<TY *>(e.m[sel].io);
  const int col = cw + lane;
  for (int rr = 0; rr < kXTok; ++rr) {
    const int t = tok[rr];
    if (t < 0) break;
    const int n = min(e.tok_n[t], kSlotPad);
    if (n <= 0) continue;
    float acc = 0.f;
    for (int s = 0; s < n; ++s) {
      const int4 rc = e.tok_rec[int64_t(t) * kSlotPad + s];
      const int k = eff_rank(k_dev, rc.y, r_max);
      const float al = __int_as_float(rc.z);
      for (int j = 0; j < k; ++j) {
        float zj = 0.f;
        if (nkc == 1) {
          zj = Z[int64_t(rc.x) * zstride + j];
        } else {
          for (int c = 0; c < nkc; ++c) zj += Z[int64_t(rc.x) * zstride + c * zld + j];
        }
        if (col < d) {
          const float b = __uint_as_float(uint32_t(B[(int64_t(rc.y) * r_max + j) * d + col].bits) << 16);
          acc = fmaf(al * zj, b, acc);
        }
      }
    }
    if (col < d) {
      TY *yp = Y + int64_t(t) * ld + col;
      if constexpr (sizeof(TY) == 4) {
        *reinterpret_cast<float *>(yp) = *reinterpret_cast<const float *>(yp) + acc;
      } else {
        const float yv = __uint_as_float(uint32_t(reinterpret_cast<const bf16_t *>(yp)->bits) << 16);
        reinterpret_cast<bf16_t *>(yp)->bits = f32_to_bf16(yv + acc);
      }
    }
  }
}

template <typename TY>
__global__ __launch_bounds__(256) void expand_tile(TileArgs e) {
  __shared__ __align__(16) int rl[kRWords + 256];  // the tile's record (+ a chunk)
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, kg = lane >> 4;
  // XCD-aware job index: each XCD takes a contiguous range of jobs, which
  // run the tiles of one column block in turn (its packed B columns stay in
  // that XCD's L2)
  const int job = (blockIdx.x & 7) * e.jobs_per_xcd + (blockIdx.x >> 3);
  if (job >= e.jobs) return;
  int sel = 0;
#pragma unroll
  for (int i = 1; i < kMaxMods; ++i)
    if (i < e.n_mods && job >= e.m[i].first) sel = i;
  const int first = e.m[sel].first, d = e.m[sel].d;
  const int64_t ld = e.m[sel].ld;
  const uint4 *Bk = e.bk_data[sel];
  TY *Y = static_cast<TY *>(e.m[sel].io);
  const int local = job - first;
  const int ct = local / e.tiles, tile = local - ct * e.tiles;
  const int cw = ct * kXCols + 64 * w;
  const int32_t *rg = e.rec + (int64_t(sel) * e.tiles + tile) * kRWords;
  // header, tokens and slot counts, then the rest of the record that is in use
  if (tid < kROctA / 4)
    reinterpret_cast<uint4 *>(rl)[tid] = reinterpret_cast<const uint4 *>(rg)[tid];
  __syncthreads();
  const int Q = rl[0], H = rl[1], fast = rl[2], C = rl[3], U = rl[4];
  const int oidx = rl[5], ocoef = rl[6];
  if (Q == 0) return;
  if (!fast) {
    tile_fallback<TY>(e, sel, rl + kRTok, cw);
    return;
  }
  // the rest of the record in use, copied straight into LDS (no registers):
  // wave w takes 1 KiB chunks w, w + 4, ... (past the used part the lanes
  // repeat its last 16 bytes; rl has room for a whole last chunk)
  const int used4 = (ocoef + 4 * (C + 8)) / 4;
  {
    const int nchunk = (used4 - kROctA / 4 + 63) / 64;
    const uint4 *src = reinterpret_cast<const uint4 *>(rg);
    uint4 *dst = reinterpret_cast<uint4 *>(rl);
    for (int c = w; c < nchunk; c += 4) {
      const int j = kROctA / 4 + c * 64;
      __builtin_amdgcn_global_load_lds(src + min(j + lane, used4 - 1), dst + j, 16, 0, 0);
    }
  }
  lds_barrier();  // (the compiler waits for the copies before it)
  // y of the tile's tokens into the accumulators.  Every load of this
  // kernel is issued whatever its lane's condition (at a clamped address,
  // masked afterwards where it matters): loads under per-lane branches keep
  // the compiler from counting them, and it then waits for all of them at
  // once.
  f32x4_t acc[4][4];  // [column block][token block]
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = rl[kRTok + 16 * tb + r16];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int col = cw + 16 * nb + 4 * kg;
      acc[nb][tb] = load_y4(Y + int64_t(max(t, 0)) * ld + min(col, d - 4));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int *octA = rl + kROctA, *octB = rl + kROctA + H;
  const int16_t *idx = reinterpret_cast<const int16_t *>(rl + oidx);
  const uint4 *coef = reinterpret_cast<const uint4 *>(rl + ocoef);
  const int nsteps = (H + 3) >> 2;
  // packed-pool octets of this lane's column in the four 16-column blocks
  // (lanes past the union or past d_out read the pool's zero unit, so no
  // loaded value needs masking: a mask would wait for the load at once)
  const uint4 *Bz = e.bk_zero[sel];
  auto load = [&](uint4 (&a)[4], int st) {
    const int h = 4 * st + kg;
    const bool in = h < H;
    const int hc = in ? h : 0;
    const int base = octA[hc], stride = (octB[hc] >> 12) & 0xf;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = cw + 16 * nb + r16;
      const uint4 *src = in && n < d ? Bk + (int64_t(base) + int64_t(n) * stride) : Bz;
      a[nb] = *src;
    }
  };
  // coefficient octets of this lane's token in the four 16-token blocks
  // (zero where the token does not hold the octet's adapter)
  // (a token without the octet's adapter reads the record's zero octets;
  // past the union the pool octets are zero, so any finite value serves)
  auto coefs = [&](uint4 (&b)[4], int st) {
    const int h = 4 * st + kg;
    const int pk = octB[h < H ? h : 0];
    const int ui = pk & 0x1ff, oi = (pk >> 9) & 7;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) b[tb] = coef[idx[(16 * tb + r16) * U + ui] + oi];
  };
  auto mult = [&](const uint4 (&a)[4], const uint4 (&b)[4]) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        acc[nb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, a[nb]), __builtin_bit_cast(bf16x8_t, b[tb]),
            acc[nb][tb], 0, 0, 0);
  };
  // B three steps ahead of the matrix cores, the coefficients one step
  // ahead.  Scheduling barriers keep the loads in program order, so that
  // each step waits only for its own operands (the memory counter is in
  // order) and the later steps' loads stay in flight.
  uint4 a0[4], a1[4], a2[4], b0[4], b1[4];
  load(a0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(a1, 1);
  __builtin_amdgcn_sched_barrier(0);
  load(a2, 2);
  __builtin_amdgcn_sched_barrier(0);
  coefs(b0, 0);
  auto step = [&](uint4 (&a)[4], const uint4 (&b)[4], uint4 (&bn)[4], int st) {
    coefs(bn, st + 1);
    mult(a, b);
    __builtin_amdgcn_sched_barrier(0);
    load(a, st + 3);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int st = 0; st < nsteps; st += 6) {
    step(a0, b0, b1, st);
    if (st + 1 >= nsteps) break;
    step(a1, b1, b0, st + 1);
    if (st + 2 >= nsteps) break;
    step(a2, b0, b1, st + 2);
    if (st + 3 >= nsteps) break;
    step(a0, b1, b0, st + 3);
    if (st + 4 >= nsteps) break;
    step(a1, b0, b1, st + 4);
    if (st + 5 >= nsteps) break;
    step(a2, b1, b0, st + 5);
  }
  // y = accumulators, for tokens that hold at least one pair
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int rrow = 16 * tb + r16, t = rl[kRTok + rrow];
    if (t < 0 || rl[kRTokN + rrow] <= 0) continue;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int col = cw + 16 * nb + 4 * kg;
      if (col < d) store_y4(Y + int64_t(t) * ld + col, acc[nb][tb]);
    }
  }
}

// Packed, rank-contiguous copy of a pool's B for the prefill expand: adapter
// a keeps ceil(k_a / 8) octets per output column, B_k[n][o] = ranks 8o ..
// 8o + 7 of column n (zero at and beyond k_a), starting at its first 16-byte
// unit off[a] (a prefix over the adapters of d_out * ceil(k / 8)).  A column's
// retained ranks are then 16-byte loads in the matrix cores' operand order,
// and an adapter takes only the room its rank needs (the tiles' working set
// in L2 scales with the retained ranks, not with r_max).
constexpr int kPackThreads = 1024;

__global__ __launch_bounds__(kPackThreads) void pack_offsets_kernel(const int32_t *k_dev,
                                                                    int32_t N, int32_t r_max,
                                                                    int32_t d, int32_t *off,
                                                                    uint4 *zero) {
  __shared__ int tmp[kPackThreads / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) *zero = make_uint4(0, 0, 0, 0);
  int base = 0;
  for (int a0 = 0; a0 < N; a0 += kPackThreads) {
    const int a = a0 + threadIdx.x;
    const int v = a < N ? ((eff_rank(k_dev, a, r_max) + 7) >> 3) * d : 0;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    if (lane == 63) tmp[w] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int j = 0; j < kPackThreads / 64; ++j) {
      if (j < w) before += tmp[j];
      total += tmp[j];
    }
    __syncthreads();
    if (a < N) off[a] = base + before + inc - v;
    base += total;
  }
}

// One thread per (adapter, column): k loads along the rank (each coalesced
// across the threads of a workgroup), ceil(k / 8) 16-byte stores.
__global__ __launch_bounds__(256) void pack_b_kernel(const uint16_t *Bt, const int32_t *k_dev,
                                                     int32_t N, int32_t r_max, int32_t d,
                                                     const int32_t *off, uint4 *Bk) {
  const int blocks = (d + 255) / 256;
  const int a = blockIdx.x / blocks, n = (blockIdx.x - a * blocks) * 256 + threadIdx.x;
  if (a >= N || n >= d) return;
  const int k = eff_rank(k_dev, a, r_max), octs = (k + 7) >> 3;
  const uint16_t *src = Bt + int64_t(a) * r_max * d + n;
  uint4 *dst = Bk + int64_t(off[a]) + int64_t(n) * octs;
  for (int o = 0; o < octs; ++o) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j0 = 8 * o + 2 * i;
      const uint32_t lo = j0 < k ? src[int64_t(j0) * d] : 0u;
      const uint32_t hi = j0 + 1 < k ? src[int64_t(j0 + 1) * d] : 0u;
      w[i] = lo | (hi << 16);
    }
    dst[o] = make_uint4(w[0], w[1], w[2], w[3]);
  }
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

// K-chunk width of the fused shrink: d_in is cut into chunks so that the
// batch yields enough (item, rank tile, chunk) workgroups to keep every CU
// issuing loads (a decode batch has only as many items as touched adapters).
// Partial z planes are added by the expand in chunk order.  The public
// single-module shrink writes final z (one chunk).
static int env_int(const char *name, int dflt) {
  const char *s = std::getenv(name);
  return (s && *s) ? std::atoi(s) : dflt;
}

// Compute units of the current device (256 when the query fails).
static int cus() {
  static const int n = [] {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
      c = 256;
    return c;
  }();
  return n;
}

static int shrink_kchunk(const tcl_plan *p, const tcl_module *mods, int n) {
  if (mods[0].wdtype != TCL_BF16) return 1 << 30;
  int kchunk;
  // TCL_KCHUNK=<elements> fixes the chunk width (tuning knob; 0 = policy)
  const int forced = env_int("TCL_KCHUNK", 0);
  if (forced > 0) {
    kchunk = (forced + 31) / 32 * 32;
  } else {
    // measured on decode batches: tiny batches (fewer workgroups than CUs)
    // gain most from 2048-element chunks, larger decode batches from
    // 4096-element chunks, prefill-sized batches lose from any split
    int64_t est_items = (p->L.cap < p->L.N ? p->L.cap : p->L.N) + p->L.cap / kTile;
    int64_t units = 0;
    for (int i = 0; i < n; ++i) units += (mods[i].r_max + 15) / 16;
    const int64_t wgs = est_items * units;
    kchunk = wgs < 256 ? 2048 : (wgs < 4096 ? 4096 : (1 << 30));
  }
  // keep a tuple's z row (all partial rows) within 128 floats
  for (int i = 0; i < n; ++i) {
    const int zl = (mods[i].r_max + 3) / 4 * 4;
    const int max_chunks = 128 / zl;
    if (max_chunks < 1) return 1 << 30;
    const int min_kchunk = (mods[i].d_in + max_chunks - 1) / max_chunks;
    if (kchunk < min_kchunk) kchunk = (min_kchunk + 31) / 32 * 32;
  }
  return kchunk;
}

static int n_kchunks(const tcl_module *m, int kchunk) {
  return (m->d_in + kchunk - 1) / kchunk;
}

// Shrink of n (<= kMaxMods) modules in one launch; z[i] is module i's output
// ([nkc][cap][zld] partial planes when kchunk < d_in).
// Launch table and grid of the shrink of n (<= kMaxMods) modules.
static int64_t shrink_args(const tcl_plan *p, const tcl_module *mods, int n,
                           const void *const *x, const int64_t *ldx, float *const *z,
                           const int *zld, int kchunk, int zero_tail, ShrinkArgs &a) {
  const bool bf = mods[0].wdtype == TCL_BF16;
  const int rows = bf ? 16 : 4;  // rank rows per workgroup job
  a = ShrinkArgs{};
  a.status = p->d.status;
  a.items = p->d.items;
  a.n_mods = n;
  a.items_cap = p->L.items_cap;
  a.zero_tail = zero_tail;
  int units = 0;
  for (int i = 0; i < n; ++i) {
    ModArgs &M = a.m[i];
    M.W = mods[i].A_t;
    M.io = const_cast<void *>(x[i]);
    M.k_dev = mods[i].k_dev;
    M.z = z[i];
    M.zld = zld[i];
    M.ld = ldx[i];
    M.d = mods[i].d_in;
    M.r_max = mods[i].r_max;
    M.first = units;
    M.n_ct = 0;
    M.nkc = bf ? n_kchunks(&mods[i], kchunk) : 1;
    M.kchunk = bf ? kchunk : (mods[i].d_in + 31) / 32 * 32;
    M.zstride = M.nkc * zld[i];
    units += (mods[i].r_max + rows - 1) / rows * M.nkc;
  }
  a.rg_total = units;
  int64_t grid = int64_t(p->L.items_cap) * units;
  if (grid > 32768) grid = 32768;
  if (grid < 1) grid = 1;
  return grid;
}

// Shrink of n (<= kMaxMods) modules in one launch; z[i] is module i's output.
static int launch_shrink(const tcl_plan *p, const tcl_module *mods, int n,
                         const void *const *x, const int64_t *ldx, float *const *z,
                         const int *zld, int kchunk, int zero_tail, hipStream_t s) {
  const bool bf = mods[0].wdtype == TCL_BF16;
  ShrinkArgs a;
  const int64_t grid = shrink_args(p, mods, n, x, ldx, z, zld, kchunk, zero_tail, a);
  logf("shrink(%s): modules=%d units/item=%d kchunk=%d grid=%lld", bf ? "mfma" : "valu", n,
       a.rg_total, kchunk, (long long)grid);
  // K steps in flight per lane: 8 (95 VGPRs, two workgroups per CU) measured
  // faster than 16 (161 VGPRs, one per CU); TCL_SSTEPS=16 forces the deeper one
  const int steps = env_int("TCL_SSTEPS", kShrinkSteps) == 16 ? 16 : 8;
  // Item pairs when the paired launch still has at least two rounds of
  // resident workgroups (1024 jobs: 2 per CU, twice over): measured on the
  // retained-rank batch 156.9 -> 142.6 us; with fewer jobs the CUs run short
  // of work (sparse prefill, 386 pair jobs: 26.2 -> 29.3 us).
  // TCL_SHRINK_PAIR=0/1 forces; TCL_PSTEPS=8 puts 8 K steps in flight, not 4
  // (slower on both).
  int64_t pg = (int64_t(p->L.items_cap) + 1) / 2 * a.rg_total;
  const int pair_env = env_int("TCL_SHRINK_PAIR", -1);
  const bool pair = pair_env == 1 || (pair_env != 0 && pg >= 4 * int64_t(cus()));
  if (bf && pair) {
    if (pg > 32768) pg = 32768;
    if (pg < 1) pg = 1;
    if (env_int("TCL_PSTEPS", 4) == 8)
      hipLaunchKernelGGL(shrink_mfma_pair<8>, dim3(int(pg)), dim3(64 * kShrinkWaves), 0, s, a);
    else
      hipLaunchKernelGGL(shrink_mfma_pair<4>, dim3(int(pg)), dim3(64 * kShrinkWaves), 0, s, a);
  } else if (bf && steps == 8)
    hipLaunchKernelGGL(shrink_mfma<8>, dim3(int(grid)), dim3(64 * kShrinkWaves), 0, s, a);
  else if (bf)
    hipLaunchKernelGGL(shrink_mfma<16>, dim3(int(grid)), dim3(64 * kShrinkWaves), 0, s, a);
  else
    hipLaunchKernelGGL((shrink_valu<float>), dim3(int(grid)), dim3(256), 0, s, a);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

// Launch of kernel k with W waves per workgroup; e.jobs_per_xcd becomes the
// number of workgroups per XCD.
template <int W, typename K>
static void launch_expand_k(K k, ExpandArgs e, hipStream_t s) {
  const int64_t blocks = (int64_t(e.jobs) + W - 1) / W;
  e.jobs_per_xcd = int32_t((blocks + 7) / 8);
  hipLaunchKernelGGL(k, dim3(8 * e.jobs_per_xcd), dim3(64 * W), 0, s, e);
}

template <int R, int CPL, bool SPLIT, typename TW, typename TY>
static void launch_expand_w(const ExpandArgs &e, int waves, hipStream_t s) {
  // rows of B per load batch: 16 when a lane holds 8 outputs (fewer VGPRs,
  // more waves per SIMD), else 32; TCL_EBATCH=16/32 forces
  const int ebf = env_int("TCL_EBATCH", 0);
  const int br = ebf == 16 || ebf == 32 ? ebf : (CPL == 8 ? 16 : 32);
  if (waves == 4 && br == 16) launch_expand_k<4>(expand_kernel<R, CPL, SPLIT, TW, TY, 4, 16>, e, s);
  else if (waves == 4) launch_expand_k<4>(expand_kernel<R, CPL, SPLIT, TW, TY, 4, 32>, e, s);
  else if (br == 16) launch_expand_k<1>(expand_kernel<R, CPL, SPLIT, TW, TY, 1, 16>, e, s);
  else launch_expand_k<1>(expand_kernel<R, CPL, SPLIT, TW, TY, 1, 32>, e, s);
}

template <int R, bool SPLIT, typename TW, typename TY>
static void launch_expand_t(const ExpandArgs &e, int cpl, int waves, hipStream_t s) {
  if (cpl == 8) launch_expand_w<R, 8, SPLIT, TW, TY>(e, waves, s);
  else if (cpl == 4) launch_expand_w<R, 4, SPLIT, TW, TY>(e, waves, s);
  else launch_expand_w<R, 2, SPLIT, TW, TY>(e, waves, s);
}

// Which expand runs.  Batches with token tiles (prefill-sized: at least
// kMfmaMinTokens tokens) of bf16 pools whose modules carry the packed copy of
// B run the token-tile expand on the matrix cores (tile_prep + expand_tile);
// every other batch runs the per-token kernel.  TCL_DISPATCH=valu forces the
// per-token kernel.
static int dispatch_override() {
  const char *s = std::getenv("TCL_DISPATCH");
  if (!s) return 0;
  if (!std::strcmp(s, "valu")) return 1;
  return 0;
}

// The prefill expand over token tiles (tile_prep + expand_tile): bf16 pools,
// batches with token tiles, pools within the record's adapter bitmap.
// TCL_DISPATCH=valu forces the per-token kernel.
static bool use_tile_expand(const tcl_plan *p, const tcl_module *mods, int n) {
  if (mods[0].wdtype != TCL_BF16 || p->L.T < kMfmaMinTokens || p->L.N > 32 * kRMaxWords)
    return false;
  for (int i = 0; i < n; ++i)
    if (!mods[i].B_k) return false;
  return dispatch_override() == 0;
}

static int r_pad(const tcl_module *m) { return (m->r_max + 7) / 8 * 8; }

// bytes before the packed data: the adapters' first 16-byte units, then a
// zero 16-byte unit right before the data
static size_t pack_head_bytes(const tcl_module *m) {
  return (size_t(m->n_adapters) * 4 + 16 + 255) & ~size_t(255);
}

static int n_tiles(const tcl_plan *p) { return (p->L.T + kXTok - 1) / kXTok; }

// workspace bytes of the per-tile records of one launch of n modules
static size_t tile_rec_bytes(const tcl_plan *p, const tcl_module *mods, int n) {
  if (!use_tile_expand(p, mods, n)) return 0;
  return size_t(n) * size_t(n_tiles(p)) * kRWords * 4;
}

// tile_prep then expand_tile for n (<= kMaxMods) modules; rec: the records'
// workspace (tile_rec_bytes)
static int launch_expand_tile(const tcl_plan *p, const tcl_module *mods, int n,
                              float *const *z, const int *zld, int kchunk, void *const *y,
                              const int64_t *ldy, tcl_dtype yd, int32_t *rec, hipStream_t s) {
  TileArgs e{};
  e.status = p->d.status;
  e.tok_n = p->d.tok_n;
  e.tok_rec = p->d.tok_rec;
  e.rec = rec;
  e.T = p->L.T;
  e.N = p->L.N;
  e.tiles = n_tiles(p);
  e.n_mods = n;
  int64_t jobs = 0;
  for (int i = 0; i < n; ++i) {
    ModArgs &M = e.m[i];
    M.W = mods[i].B_t;
    M.io = y[i];
    M.k_dev = mods[i].k_dev;
    M.z = z[i];
    M.zld = zld[i];
    M.ld = ldy[i];
    M.d = mods[i].d_out;
    M.r_max = mods[i].r_max;
    M.n_ct = (mods[i].d_out + kXCols - 1) / kXCols;
    M.nkc = n_kchunks(&mods[i], kchunk);
    M.zstride = M.nkc * zld[i];
    M.first = int32_t(jobs);
    jobs += int64_t(M.n_ct) * e.tiles;
    e.bk_off[i] = static_cast<const int32_t *>(mods[i].B_k);
    e.bk_data[i] = reinterpret_cast<const uint4 *>(static_cast<const char *>(mods[i].B_k) +
                                                   pack_head_bytes(&mods[i]));
    e.bk_zero[i] = e.bk_data[i] - 1;
  }
  if (jobs > (int64_t(1) << 30)) return fail(TCL_EUNSUPPORTED, "expand grid too large");
  e.jobs = int32_t(jobs);
  e.jobs_per_xcd = int32_t((jobs + 7) / 8);
  e.tile_tok = p->d.tile_tok;
  logf("expand(tile): modules=%d tiles=%d jobs=%lld", n, e.tiles, (long long)jobs);
  hipLaunchKernelGGL(tile_prep, dim3(n * e.tiles), dim3(256), 0, s, e);
  if (yd == TCL_BF16)
    hipLaunchKernelGGL((expand_tile<bf16_t>), dim3(8 * e.jobs_per_xcd), dim3(256), 0, s, e);
  else
    hipLaunchKernelGGL((expand_tile<float>), dim3(8 * e.jobs_per_xcd), dim3(256), 0, s, e);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

// Expand of n (<= kMaxMods) modules in one launch.
static int expand_args(const tcl_plan *p, const tcl_module *mods, int n, float *const *z,
                       const int *zld, int kchunk, void *const *y, const int64_t *ldy,
                       ExpandArgs &e, int &cpl, int &R, bool &split, int cpl_min = 2);

// The per-token expand of every token.
static int launch_expand_valu(const tcl_plan *p, const tcl_module *mods, int n,
                              float *const *z, const int *zld, int kchunk, void *const *y,
                              const int64_t *ldy, tcl_dtype yd, hipStream_t s) {
  ExpandArgs e;
  int cpl, R;
  bool split;
  int rc = expand_args(p, mods, n, z, zld, kchunk, y, ldy, e, cpl, R, split);
  if (rc) return rc;
  // jobs per workgroup: four for launches of at least 4096 jobs of ranks up
  // to 16 (measured faster: sparse prefill 148 -> 141 us, 7-projection decode
  // step 38.6 -> 37.5 us), one otherwise (four measured slower for rank 32:
  // retained-rank batch 1037 -> 1206 us; and on the 1024-job decode batch,
  // 14.99 -> 15.05 us); TCL_EWAVES=1/4 forces
  const int ew = env_int("TCL_EWAVES", 0);
  const int waves = ew == 1 || ew == 4 ? ew : (e.jobs >= 4096 && R <= 16 ? 4 : 1);
  logf("expand(valu): modules=%d R=%d cpl=%d jobs=%d waves/workgroup=%d", n, R, cpl, e.jobs,
       waves);
  const bool bf = mods[0].wdtype == TCL_BF16;
  const bool ybf = yd == TCL_BF16;
#define TCL_EXPAND_CASE(RR)                                                                    \
  case RR:                                                                                     \
    if (bf && ybf && split) launch_expand_t<RR, true, bf16_t, bf16_t>(e, cpl, waves, s);       \
    else if (bf && ybf) launch_expand_t<RR, false, bf16_t, bf16_t>(e, cpl, waves, s);          \
    else if (bf && split) launch_expand_t<RR, true, bf16_t, float>(e, cpl, waves, s);          \
    else if (bf) launch_expand_t<RR, false, bf16_t, float>(e, cpl, waves, s);                  \
    else launch_expand_t<RR, false, float, float>(e, cpl, waves, s);                           \
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

static int launch_expand(const tcl_plan *p, const tcl_module *mods, int n,
                         float *const *z, const int *zld, int kchunk, void *const *y,
                         const int64_t *ldy, tcl_dtype yd, int32_t *rec, hipStream_t s) {
  if (p->L.T == 0) return TCL_OK;
  if (rec && use_tile_expand(p, mods, n))
    return launch_expand_tile(p, mods, n, z, zld, kchunk, y, ldy, yd, rec, s);
  return launch_expand_valu(p, mods, n, z, zld, kchunk, y, ldy, yd, s);
}

// Launch table of the per-token expand of n (<= kMaxMods) modules: outputs
// per lane, rank bucket and whether z holds split-K partial rows.
static int expand_args(const tcl_plan *p, const tcl_module *mods, int n, float *const *z,
                       const int *zld, int kchunk, void *const *y, const int64_t *ldy,
                       ExpandArgs &e, int &cpl, int &R, bool &split, int cpl_min) {
  const bool bfw = mods[0].wdtype == TCL_BF16;
  e = ExpandArgs{};
  e.tok_n = p->d.tok_n;
  e.tok_rec = p->d.tok_rec;
  e.T = p->L.T;
  e.n_mods = n;
  // outputs per lane: 8 unless the batch would then give too few waves
  int64_t jobs8 = 0;
  for (int i = 0; i < n; ++i) jobs8 += int64_t((mods[i].d_out + 511) / 512) * p->L.T;
  cpl = jobs8 >= 1024 ? 8 : (jobs8 >= 512 ? 4 : 2);
  if (cpl < cpl_min) cpl = cpl_min;
  const int forced_cpl = env_int("TCL_CPL", 0);  // tuning knob: 2, 4 or 8
  if (forced_cpl == 2 || forced_cpl == 4 || forced_cpl == 8) cpl = forced_cpl;
  int64_t jobs = 0;
  int rmax = 1;
  split = false;
  for (int i = 0; i < n; ++i) {
    ModArgs &M = e.m[i];
    M.W = mods[i].B_t;
    M.io = y[i];
    M.k_dev = mods[i].k_dev;
    M.z = z[i];
    M.zld = zld[i];
    M.ld = ldy[i];
    M.d = mods[i].d_out;
    M.r_max = mods[i].r_max;
    M.n_ct = (mods[i].d_out + 64 * cpl - 1) / (64 * cpl);
    M.nkc = bfw ? n_kchunks(&mods[i], kchunk) : 1;
    M.zstride = M.nkc * zld[i];
    if (M.nkc > 1) split = true;
    M.first = int32_t(jobs);
    jobs += int64_t(M.n_ct) * p->L.T;
    if (mods[i].r_max > rmax) rmax = mods[i].r_max;
  }
  if (jobs > (int64_t(1) << 30)) return fail(TCL_EUNSUPPORTED, "expand grid too large");
  e.jobs = int32_t(jobs);
  e.jobs_per_xcd = int32_t((jobs + 7) / 8);
  R = rank_bucket(rmax);
  return TCL_OK;
}

static int z_ld(const tcl_module *m) { return (m->r_max + 3) / 4 * 4; }

static size_t z_bytes(const tcl_plan *p, const tcl_module *m, int kchunk) {
  const size_t planes = m->wdtype == TCL_BF16 ? size_t(n_kchunks(m, kchunk)) : 1;
  return (planes * size_t(p->L.cap) * size_t(z_ld(m)) * 4 + 255) & ~size_t(255);
}

// Workspace layout: z of every module (batches of up to kMaxMods modules in
// order), then the per-tile records of the prefill expand, one region shared
// by the batches (they run in stream order).
static size_t ws_z_bytes(const tcl_plan *p, const tcl_module *mods, int n_mods) {
  size_t z = 0;
  for (int i0 = 0; i0 < n_mods; i0 += kMaxMods) {
    const int n = n_mods - i0 < kMaxMods ? n_mods - i0 : kMaxMods;
    const int kchunk = shrink_kchunk(p, mods + i0, n);
    for (int i = 0; i < n; ++i) z += z_bytes(p, &mods[i0 + i], kchunk);
  }
  return z;
}

static size_t ws_need(const tcl_plan *p, const tcl_module *mods, int n_mods) {
  size_t rec = 0;
  for (int i0 = 0; i0 < n_mods; i0 += kMaxMods) {
    const int n = n_mods - i0 < kMaxMods ? n_mods - i0 : kMaxMods;
    const size_t b = tile_rec_bytes(p, mods + i0, n);
    if (b > rec) rec = b;
  }
  return 256 + ws_z_bytes(p, mods, n_mods) + ((rec + 255) & ~size_t(255));
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

int tcl_module_init(tcl_module *m, const int32_t *k_host, int32_t *k_dev, void *stream) {
  int rc = check_module(m);
  if (rc) return rc;
  if (!k_host) {
    m->k_dev = nullptr;
    return TCL_OK;
  }
  return tcl_module_load_ranks(m, k_host, k_dev, stream);
}

int tcl_module_pack_bytes(const tcl_module *m, size_t *bytes) {
  if (!bytes) return fail(TCL_EINVAL, "bytes is NULL");
  int rc = check_module(m);
  if (rc) return rc;
  *bytes = pack_head_bytes(m) + size_t(m->n_adapters) * size_t(m->d_out) * size_t(r_pad(m)) * 2;
  return TCL_OK;
}

int tcl_module_pack(tcl_module *m, void *B_k, size_t bytes, void *stream) {
  size_t need = 0;
  int rc = tcl_module_pack_bytes(m, &need);
  if (rc) return rc;
  if (m->wdtype != TCL_BF16) return fail(TCL_EUNSUPPORTED, "the packed copy is for bf16 pools");
  if (!B_k) return fail(TCL_EINVAL, "B_k is NULL");
  if (reinterpret_cast<uintptr_t>(B_k) & 255)
    return fail(TCL_EALIGN, "B_k must be 256-byte aligned");
  if (bytes < need) return fail(TCL_ENOSPC, "B_k holds %zu bytes, needs %zu", bytes, need);
  const int blocks = (m->d_out + 255) / 256;
  const int64_t grid = int64_t(m->n_adapters) * blocks;
  const int64_t units = int64_t(m->n_adapters) * m->d_out * (r_pad(m) / 8);
  if (grid > (int64_t(1) << 31) - 1 || units > (int64_t(1) << 31) - 1)
    return fail(TCL_EUNSUPPORTED, "pool too large to pack");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t *off = static_cast<int32_t *>(B_k);
  hipLaunchKernelGGL(pack_offsets_kernel, dim3(1), dim3(kPackThreads), 0, s, m->k_dev,
                     m->n_adapters, m->r_max, m->d_out, off,
                     reinterpret_cast<uint4 *>(static_cast<char *>(B_k) + pack_head_bytes(m)) - 1);
  hipLaunchKernelGGL(pack_b_kernel, dim3(unsigned(grid)), dim3(256), 0, s,
                     static_cast<const uint16_t *>(m->B_t), m->k_dev, m->n_adapters, m->r_max,
                     m->d_out, off,
                     reinterpret_cast<uint4 *>(static_cast<char *>(B_k) + pack_head_bytes(m)));
  TCL_HIP(hipGetLastError());
  m->B_k = B_k;
  return TCL_OK;
}

int tcl_workspace_bytes(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                        size_t *bytes) {
  if (!bytes) return fail(TCL_EINVAL, "bytes is NULL");
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  if (n_mods < 0 || (n_mods > 0 && !mods)) return fail(TCL_EINVAL, "bad module list");
  for (int i = 0; i < n_mods; ++i) {
    int rc = check_plan_module(p, &mods[i]);
    if (rc) return rc;
  }
  *bytes = ws_need(p, mods, n_mods);
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
  const int zld = m->r_max;
  return launch_shrink(p, m, 1, &x, &ldx, &z, &zld, 1 << 30, 1, static_cast<hipStream_t>(stream));
}

int tcl_expand(const tcl_plan *p, const tcl_module *m, const float *z, void *y, int64_t ldy,
               tcl_dtype yd, void *stream) {
  int rc = check_plan_module(p, m);
  if (rc) return rc;
  if ((rc = check_dtypes(m, m->wdtype, yd, true))) return rc;
  if ((rc = check_io(y, ldy, m->d_out, "y"))) return rc;
  if (!z) return fail(TCL_EINVAL, "z is NULL");
  float *zz = const_cast<float *>(z);
  const int zld = m->r_max;
  return launch_expand(p, m, 1, &zz, &zld, 1 << 30, &y, &ldy, yd, nullptr,
                       static_cast<hipStream_t>(stream));
}

// Checks shared by the fused entry points; returns the workspace bytes needed.
static int check_fused(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                       const void *const *x, const int64_t *ldx, tcl_dtype xd, void *const *y,
                       const int64_t *ldy, tcl_dtype yd, void *ws, size_t ws_bytes) {
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  if (n_mods < 1 || !mods) return fail(TCL_EINVAL, "module list is required");
  if ((x && !ldx) || (y && !ldy)) return fail(TCL_EINVAL, "leading dimensions are required");
  for (int i = 0; i < n_mods; ++i) {
    int rc = check_plan_module(p, &mods[i]);
    if (rc) return rc;
    if ((rc = check_dtypes(&mods[i], x ? xd : mods[i].wdtype, yd, y != nullptr))) return rc;
    if (x && (rc = check_io(x[i], ldx[i], mods[i].d_in, "x"))) return rc;
    if (y && (rc = check_io(y[i], ldy[i], mods[i].d_out, "y"))) return rc;
    if (mods[i].wdtype != mods[0].wdtype)
      return fail(TCL_EUNSUPPORTED, "modules of one call must share a weight dtype");
  }
  const size_t need = ws_need(p, mods, n_mods);
  if (!ws) return fail(TCL_EINVAL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(TCL_EALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(TCL_ENOSPC, "workspace holds %zu bytes, needs %zu", ws_bytes, need);
  return TCL_OK;
}

// z of module i lives in the workspace after the z of modules 0..i-1
static void z_slices(const tcl_plan *p, const tcl_module *mods, int i0, int n, void *ws,
                     float **z, int *zld, int *kchunk_out) {
  char *wp = static_cast<char *>(ws);
  for (int b = 0; b < i0; b += kMaxMods) {
    const int nb = i0 - b < kMaxMods ? i0 - b : kMaxMods;
    const int kc = shrink_kchunk(p, mods + b, nb);
    for (int i = 0; i < nb; ++i) wp += z_bytes(p, &mods[b + i], kc);
  }
  const int kchunk = shrink_kchunk(p, mods + i0, n);
  for (int i = 0; i < n; ++i) {
    z[i] = reinterpret_cast<float *>(wp);
    zld[i] = z_ld(&mods[i0 + i]);
    wp += z_bytes(p, &mods[i0 + i], kchunk);
  }
  *kchunk_out = kchunk;
}

static int run_fused(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                     const void *const *x, const int64_t *ldx, void *const *y,
                     const int64_t *ldy, tcl_dtype yd, void *ws, hipStream_t s) {
  int32_t *rec = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + ws_z_bytes(p, mods, n_mods));
  for (int i0 = 0; i0 < n_mods; i0 += kMaxMods) {
    const int n = n_mods - i0 < kMaxMods ? n_mods - i0 : kMaxMods;
    float *z[kMaxMods];
    int zld[kMaxMods], kchunk;
    z_slices(p, mods, i0, n, ws, z, zld, &kchunk);
    if (x) {
      int rc = launch_shrink(p, mods + i0, n, x + i0, ldx + i0, z, zld, kchunk, 0, s);
      if (rc) return rc;
    }
    if (y) {
      int rc = launch_expand(p, mods + i0, n, z, zld, kchunk, y + i0, ldy + i0, yd, rec, s);
      if (rc) return rc;
    }
  }
  return TCL_OK;
}

int tcl_fused_apply(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                    const void *const *x, const int64_t *ldx, tcl_dtype xd, void *const *y,
                    const int64_t *ldy, tcl_dtype yd, void *ws, size_t ws_bytes,
                    void *stream) {
  if (!x || !y) return fail(TCL_EINVAL, "x and y lists are required");
  int rc = check_fused(p, mods, n_mods, x, ldx, xd, y, ldy, yd, ws, ws_bytes);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // shrink and expand alternate per batch of up to kMaxMods modules
  return run_fused(p, mods, n_mods, x, ldx, y, ldy, yd, ws, s);
}


// The decode step's shrink with the mapping stage inside (plan_shrink):
// direct-mode tables whose LDS view and work items fit the kernel's budget,
// bf16 pools, one launch's worth of modules.  TCL_FUSED_MAPPING=0 turns it
// off (the mapping kernel then runs on its own before the shrink).
static bool fused_mapping(const tcl_plan *p, const tcl_module *mods, int n_mods) {
  if (p->L.mode != PLAN_DIRECT || mods[0].wdtype != TCL_BF16 || n_mods > kMaxMods) return false;
  if (plan_direct_lds_ints(p) > kFusedLdsInts || p->L.items_cap > kFusedItems) return false;
  const char *e = std::getenv("TCL_FUSED_MAPPING");
  return !(e && !std::strcmp(e, "0"));
}

// Mapping stage of p (just laid out for c) and the shrink of every module.
static int remap_shrink(tcl_plan *p, const tcl_composites *c, const tcl_module *mods,
                        int32_t n_mods, const void *const *x, const int64_t *ldx, void *ws,
                        hipStream_t s) {
  if (!fused_mapping(p, mods, n_mods)) {
    int rc = plan_launch(p, c, s);
    if (rc) return rc;
    return run_fused(p, mods, n_mods, x, ldx, nullptr, nullptr, TCL_F32, ws, s);
  }
  float *z[kMaxMods];
  int zld[kMaxMods], kchunk;
  z_slices(p, mods, 0, n_mods, ws, z, zld, &kchunk);
  PlanArgs A;
  plan_fill_args(p, c, &A);
  ShrinkArgs a;
  int64_t grid = shrink_args(p, mods, n_mods, x, ldx, z, zld, kchunk, 0, a);
  // every workgroup maps the table once: at most two per CU (what the LDS
  // allows at once), each looping over its share of the shrink jobs, plus
  // workgroup 0, which writes the plan and has no shrink job
  const int cap = env_int("TCL_FUSED_GRID", 2 * cus() - 1);
  if (grid > cap) grid = cap;
  grid += 1;
  logf("plan+shrink: T=%d pairs=%d N=%d modules=%d units/item=%d kchunk=%d grid=%lld", p->L.T,
       p->L.NP, p->L.N, n_mods, a.rg_total, kchunk, (long long)grid);
  if (env_int("TCL_SSTEPS", kShrinkSteps) == 16)
    hipLaunchKernelGGL(plan_shrink<16>, dim3(int(grid)), dim3(64 * kShrinkWaves), 0, s, A, a);
  else
    hipLaunchKernelGGL(plan_shrink<8>, dim3(int(grid)), dim3(64 * kShrinkWaves), 0, s, A, a);
  TCL_HIP(hipGetLastError());
  return plan_launch_tile_order(p, s);
}

int tcl_remap_shrink(tcl_plan *p, const tcl_composites *c, const tcl_module *mods,
                     int32_t n_mods, const void *const *x, const int64_t *ldx, tcl_dtype xd,
                     void *ws, size_t ws_bytes, void *stream) {
  if (!x) return fail(TCL_EINVAL, "x list is required");
  tcl_plan next;
  int rc = plan_remap_prepare(p, c, &next);
  if (rc) return rc;
  rc = check_fused(&next, mods, n_mods, x, ldx, xd, nullptr, nullptr, TCL_F32, ws, ws_bytes);
  if (rc) return rc;
  *p = next;
  return remap_shrink(p, c, mods, n_mods, x, ldx, ws, static_cast<hipStream_t>(stream));
}

int tcl_remap_apply(tcl_plan *p, const tcl_composites *c, const tcl_module *mods,
                    int32_t n_mods, const void *const *x, const int64_t *ldx, tcl_dtype xd,
                    void *const *y, const int64_t *ldy, tcl_dtype yd, void *ws,
                    size_t ws_bytes, void *stream) {
  if (!x || !y) return fail(TCL_EINVAL, "x and y lists are required");
  tcl_plan next;
  int rc = plan_remap_prepare(p, c, &next);
  if (rc) return rc;
  rc = check_fused(&next, mods, n_mods, x, ldx, xd, y, ldy, yd, ws, ws_bytes);
  if (rc) return rc;
  *p = next;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!fused_mapping(p, mods, n_mods)) {
    // mapping kernel(s), then shrink and expand alternating per module batch
    rc = plan_launch(p, c, s);
    if (rc) return rc;
    return run_fused(p, mods, n_mods, x, ldx, y, ldy, yd, ws, s);
  }
  rc = remap_shrink(p, c, mods, n_mods, x, ldx, ws, s);
  if (rc) return rc;
  return run_fused(p, mods, n_mods, nullptr, nullptr, y, ldy, yd, ws, s);
}

int tcl_fused_shrink(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                     const void *const *x, const int64_t *ldx, tcl_dtype xd, void *ws,
                     size_t ws_bytes, void *stream) {
  if (!x) return fail(TCL_EINVAL, "x list is required");
  int rc = check_fused(p, mods, n_mods, x, ldx, xd, nullptr, nullptr, TCL_F32, ws, ws_bytes);
  if (rc) return rc;
  return run_fused(p, mods, n_mods, x, ldx, nullptr, nullptr, TCL_F32, ws,
                   static_cast<hipStream_t>(stream));
}

int tcl_fused_expand(const tcl_plan *p, const tcl_module *mods, int32_t n_mods, void *ws,
                     size_t ws_bytes, void *const *y, const int64_t *ldy, tcl_dtype yd,
                     void *stream) {
  if (!y) return fail(TCL_EINVAL, "y list is required");
  int rc = check_fused(p, mods, n_mods, nullptr, nullptr, TCL_BF16, y, ldy, yd, ws, ws_bytes);
  if (rc) return rc;
  return run_fused(p, mods, n_mods, nullptr, nullptr, y, ldy, yd, ws,
                   static_cast<hipStream_t>(stream));
}

}  // extern "C"
