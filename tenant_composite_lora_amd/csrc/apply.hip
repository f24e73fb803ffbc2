// Shrink, expand and the fused apply of the composite multi-LoRA path.
//
//   shrink  (LoRAForge approach (4), segmented shrink): z_p = A_a[:, :k]^T
//           x_{t_p} for one work item (an adapter and up to kTile consecutive
//           tuples of its segment) and one or two tiles of 16 rank rows, on
//           the matrix cores in bf16 (shrink_mfma, shrink_mfma_pair, plan_shrink)
//           or with fp32 dot products and a wave butterfly (shrink_valu).
//           Decode batches split d_in into K chunks whose partial z rows the
//           expand adds in chunk order.
//   expand  (LoRAForge approach (4), RowExpand; DyMerge-LoRA aggregation
//           stage): one wave owns 64 * CPL consecutive outputs of one token
//           and adds alpha_s * B_a[n, :k] z_s for the token's slots in order,
//           in fp32, then adds the total to y once (expand_kernel).  Prefill
//           batches run over 64-token tiles on the matrix cores instead
//           (tile_prep + expand_tile, in tile.hip).  Each output element has
//           exactly one owner; there are no atomics.
//
// Also here: the host side of every apply entry point (checks, workspace
// layout, dispatch), the allocation-free apply over a static device
// workspace, and the loads of an adapter slot pool (DyMerge-LoRA section 4,
// BAM).  A plan whose composite table was rejected has an empty token index
// and no work items, so every kernel below finds nothing to do.

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "kern_common.hpp"
#include "plan_core.hpp"
#include "tcl_internal.hpp"
#include "tile.hpp"

namespace tcl {

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

constexpr int kShrinkWaves = 8;   // waves per workgroup, splitting d_in
constexpr int kShrinkSteps = 8;   // 32-element K steps each lane has in flight

// z[tokens x ranks] = X[tokens x d_in] . A_a^T[d_in x ranks] for one work item
// (up to 16 tuples of one adapter) and RT tiles of 16 rank rows (RT = 2: two
// accumulators on the same x fragments, so x is loaded once for 32 ranks),
// with v_mfma_f32_16x16x32_bf16.  Both operands load straight from memory: lane l
// holds 8 consecutive d of token row (l % 16) for the first operand and of rank
// row (l % 16) of A_a^T (rank-major, so 16 contiguous bytes) for the second;
// rows past the item's tuple count or the adapter's effective rank are zero
// and never read.  The 8 waves split the K steps of d_in, each keeping
// kShrinkSteps steps of loads in flight, and their partial tiles are summed
// through LDS in wave order.  z is written final.
// The A fragments of the first STEPS K steps of job `job` (rank tile of one
// 16-row tile, the calling lane's rank row and granule), as the job loop
// below loads them: zero where the row is at or beyond the adapter's
// effective rank or the step is past the wave's share or d_in.  A caller
// that knows the job's item before its token lists (the decode step's
// mapping stage) issues these loads early and hands them to the loop.
template <int STEPS>
__device__ inline void shrink_first_a(const ShrinkArgs &s, int job, int4 head,
                                      uint4 (&pa)[STEPS]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int item = job / s.rg_total, rgg = job - item * s.rg_total;
  (void)item;
  int mi = 0;
#pragma unroll
  for (int i = 1; i < kMaxMods; ++i)
    if (i < s.n_mods && rgg >= s.m[i].first) mi = i;
  const int dd = s.m[mi].d, r_max = s.m[mi].r_max;
  const int nkc = s.m[mi].nkc, kchunk = s.m[mi].kchunk;
  const int unit = rgg - s.m[mi].first;
  const int rt = unit / nkc, kc = unit - rt * nkc;
  const int j0 = rt * 16;
  const int k = eff_rank(s.m[mi].k_dev, head.x, r_max);
  const int jr = j0 + row;
  const bf16_t *Aw = static_cast<const bf16_t *>(s.m[mi].W);
  const bf16_t *Ar = j0 < k && jr < k ? Aw + (int64_t(head.x) * r_max + jr) * dd + kg * 8 : nullptr;
  const int c0 = kc * (kchunk / 32), c1 = min((dd + 31) / 32, c0 + kchunk / 32);
  const int per = (c1 - c0 + kShrinkWaves - 1) / kShrinkWaves;
  const int s0 = c0 + w * per, s1 = min(c1, s0 + per);
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const int e0 = (s0 + u) * 32 + kg * 8;
    uint4 ab = make_uint4(0, 0, 0, 0);
    if (s0 + u < s1 && e0 < dd && Ar) ab = *reinterpret_cast<const uint4 *>(Ar + (s0 + u) * 32);
    pa[u] = ab;
  }
}

// Jobs job0, job0 + stride, ... of one workgroup (8 waves); each lane keeps
// STEPS K steps of loads in flight.  With has_pre, pre holds the A fragments
// of job0's first STEPS K steps, loaded by shrink_first_a (one rank tile a
// job only).  LOCAL: the work items are litems, in this workgroup's LDS
// (its own mapping stage), read with LDS loads; else the plan's item table.
template <int STEPS, int RT = 1, bool LOCAL = false>
__device__ inline void shrink_mfma_jobs_pre(const ShrinkArgs &s, int job0, int stride,
                                            f32x4_t (*red)[64], const Item *litems,
                                            int n_litems, const uint4 (&pre)[STEPS],
                                            bool has_pre) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  // The item record of the first job is fetched together with the item count
  // (clamped to the item table, which a padded grid may pass), which saves
  // one dependent memory round trip.
  // litems: the work items in LDS (a mapping stage run by this workgroup),
  // else the plan's item table
  const Item *items = LOCAL ? litems : s.items;
  const int cap = LOCAL ? max(n_litems, 1) : s.items_cap;
  int job = job0;
  const int item0 = min(job / s.rg_total, cap - 1);
  int4 head = items[item0].head;
  int tokl = items[item0].tok[row];
  const int n_items = LOCAL ? n_litems : s.status[ST_ITEMS];
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
    const int rt = unit / nkc, kc = unit - rt * nkc;  // rank tile group, K chunk
    const int zstride = s.m[mi].zstride;
    float *Z = s.m[mi].z + kc * zld;  // this chunk's partial row inside each tuple row
    const int j0 = rt * 16 * RT;
    const int a = head.x, p0 = head.y, ntok = head.z;
    const int k = eff_rank(k_dev, a, r_max);
    if (j0 >= k) {
      // every rank tile of the job beyond the effective rank
      if (s.zero_tail && w < RT) {
        const int j = j0 + 16 * w + row;
        for (int tt = kg; tt < ntok; tt += 4)
          if (j < r_max) Z[int64_t(p0 + tt) * zstride + j] = 0.f;
      }
      continue;
    }
    const bool hi = RT == 2 && j0 + 16 < k;  // the second rank tile holds ranks
    const int tok = row < ntok ? tokl : -1;
    const int jr = j0 + row;  // rank row this lane feeds (and jr + 16)
    const bf16_t *Xr = tok >= 0 ? Xw + int64_t(tok) * ld + kg * 8 : nullptr;
    const bf16_t *Ar = jr < k ? Aw + (int64_t(a) * r_max + jr) * dd + kg * 8 : nullptr;
    const bf16_t *Ar1 =
        RT == 2 && jr + 16 < k ? Aw + (int64_t(a) * r_max + jr + 16) * dd + kg * 8 : nullptr;
    // K steps of this chunk, split over the waves
    const int c0 = kc * (kchunk / 32), c1 = min((dd + 31) / 32, c0 + kchunk / 32);
    const int per = (c1 - c0 + kShrinkWaves - 1) / kShrinkWaves;
    const int s0 = c0 + w * per, s1 = min(c1, s0 + per);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int st = s0; st < s1; st += STEPS) {
      bf16x8_t xv[STEPS], av[STEPS], av1[RT == 2 ? STEPS : 1];
      auto mult = [&]() {
#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[u], av[u], acc, 0, 0, 0);
          if constexpr (RT == 2)
            if (hi) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[u], av1[u], acc1, 0, 0, 0);
        }
      };
      if (RT == 1 && has_pre && job == job0 && st == s0) {
        // the A fragments are in flight already: issue the x loads, then
        // multiply.  This path has its own multiply, so that the compiler's
        // wait analysis does not merge it with the other path's loads (it
        // would then wait for every load in flight before the first x load).
#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
          const int e0 = (st + u) * 32 + kg * 8;
          uint4 xb = make_uint4(0, 0, 0, 0);
          if (st + u < s1 && e0 < dd && Xr) xb = *reinterpret_cast<const uint4 *>(Xr + (st + u) * 32);
          xv[u] = __builtin_bit_cast(bf16x8_t, xb);
        }
#pragma unroll
        for (int u = 0; u < STEPS; ++u) av[u] = __builtin_bit_cast(bf16x8_t, pre[u]);
        mult();
      } else {
#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
          const int e0 = (st + u) * 32 + kg * 8;  // first element of this lane's granule
          const bool in = st + u < s1 && e0 < dd;
          uint4 xb = make_uint4(0, 0, 0, 0), ab = make_uint4(0, 0, 0, 0);
          if (in && Xr) xb = *reinterpret_cast<const uint4 *>(Xr + (st + u) * 32);
          if (in && Ar) ab = *reinterpret_cast<const uint4 *>(Ar + (st + u) * 32);
          xv[u] = __builtin_bit_cast(bf16x8_t, xb);
          av[u] = __builtin_bit_cast(bf16x8_t, ab);
          if constexpr (RT == 2) {
            uint4 ab1 = make_uint4(0, 0, 0, 0);
            if (in && Ar1) ab1 = *reinterpret_cast<const uint4 *>(Ar1 + (st + u) * 32);
            av1[u] = __builtin_bit_cast(bf16x8_t, ab1);
          }
        }
        mult();
      }
    }
    red[w][lane] = acc;
    if constexpr (RT == 2) red[kShrinkWaves + w][lane] = acc1;
    __syncthreads();
    if (w < RT) {  // wave t finishes rank tile t of the job
      const int base = w * kShrinkWaves;
      f32x4_t sum = red[base][lane];
#pragma unroll
      for (int v = 1; v < kShrinkWaves; ++v) {
        const f32x4_t o = red[base + v][lane];
        sum[0] += o[0];
        sum[1] += o[1];
        sum[2] += o[2];
        sum[3] += o[3];
      }
      // lane holds tokens 4*kg .. 4*kg+3 of rank column j0 + 16 w + row
      const int j = j0 + 16 * w + row;
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

template <int STEPS, int RT = 1>
__device__ inline void shrink_mfma_jobs(const ShrinkArgs &s, int job0, int stride,
                                        f32x4_t (*red)[64]) {
  const uint4 none[STEPS] = {};
  shrink_mfma_jobs_pre<STEPS, RT, false>(s, job0, stride, red, nullptr, 0, none, false);
}

template <int STEPS, int RT>
__global__ __launch_bounds__(64 * kShrinkWaves) void shrink_mfma(ShrinkArgs s) {
  __shared__ f32x4_t red[RT * kShrinkWaves][64];
  shrink_mfma_jobs<STEPS, RT>(s, blockIdx.x, gridDim.x, red);
}

// Item pairs: one job takes work items 2q and 2q + 1 of one (RT rank tiles,
// K chunk, module) unit.  When both belong to the same adapter (consecutive
// items of one segment) they share every A-row load and run two matrix-core
// accumulators, one per item; otherwise the items run one after the other.
// Each accumulator sees the same K steps in the same order as in
// shrink_mfma_jobs, and the wave partials are summed in the same wave order,
// so z is bit for bit that of shrink_mfma.  Half as many jobs, and half the A
// rows moved into the compute units, for prefill batches whose segments span
// several items.
template <int STEPS, int RT>
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
  const int j0 = rt * 16 * RT;
  const int a = h0.x;
  const int k = eff_rank(s.m[mi].k_dev, a, r_max);
  const int n0 = h0.z, n1 = two ? h1.z : 0;
  if (j0 >= k) {
    if (s.zero_tail && w < RT) {
      const int j = j0 + 16 * w + row;
      if (j < r_max) {
        for (int tt = kg; tt < n0; tt += 4) Z[int64_t(h0.y + tt) * zstride + j] = 0.f;
        for (int tt = kg; tt < n1; tt += 4) Z[int64_t(h1.y + tt) * zstride + j] = 0.f;
      }
    }
    return;
  }
  const bool hi = RT == 2 && j0 + 16 < k;  // the second rank tile holds ranks
  const int jr = j0 + row;
  const bf16_t *X0 = row < n0 ? Xw + int64_t(tok0) * ld + kg * 8 : nullptr;
  const bf16_t *X1 = row < n1 ? Xw + int64_t(tok1) * ld + kg * 8 : nullptr;
  const bf16_t *Ar = jr < k ? Aw + (int64_t(a) * r_max + jr) * dd + kg * 8 : nullptr;
  const bf16_t *Ar1 =
      RT == 2 && jr + 16 < k ? Aw + (int64_t(a) * r_max + jr + 16) * dd + kg * 8 : nullptr;
  const int c0 = kc * (kchunk / 32), c1 = min((dd + 31) / 32, c0 + kchunk / 32);
  const int per = (c1 - c0 + kShrinkWaves - 1) / kShrinkWaves;
  const int s0 = c0 + w * per, s1 = min(c1, s0 + per);
  // [item][rank tile]
  f32x4_t acc00 = {0.f, 0.f, 0.f, 0.f}, acc10 = acc00, acc01 = acc00, acc11 = acc00;
  for (int st = s0; st < s1; st += STEPS) {
    bf16x8_t xv0[STEPS], xv1[STEPS], av[STEPS], av1[RT == 2 ? STEPS : 1];
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
      if constexpr (RT == 2) {
        uint4 ab1 = make_uint4(0, 0, 0, 0);
        if (in && Ar1) ab1 = *reinterpret_cast<const uint4 *>(Ar1 + (st + u) * 32);
        av1[u] = __builtin_bit_cast(bf16x8_t, ab1);
      }
    }
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      acc00 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv0[u], av[u], acc00, 0, 0, 0);
      if (two) acc10 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv1[u], av[u], acc10, 0, 0, 0);
      if constexpr (RT == 2) {
        if (hi) {
          acc01 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv0[u], av1[u], acc01, 0, 0, 0);
          if (two) acc11 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv1[u], av1[u], acc11, 0, 0, 0);
        }
      }
    }
  }
  // partial tiles: slot (item, rank tile) = item * RT + tile, kShrinkWaves rows each
  red[w][lane] = acc00;
  red[RT * kShrinkWaves + w][lane] = acc10;
  if constexpr (RT == 2) {
    red[kShrinkWaves + w][lane] = acc01;
    red[3 * kShrinkWaves + w][lane] = acc11;
  }
  __syncthreads();
  // wave it * RT + t finishes rank tile t of item it
  const int it = w / RT, t = w - it * RT;
  if (w < (two ? 2 : 1) * RT) {
    const int base = w * kShrinkWaves, p0 = it ? h1.y : h0.y, nt = it ? n1 : n0;
    f32x4_t sum = red[base][lane];
#pragma unroll
    for (int v = 1; v < kShrinkWaves; ++v) {
      const f32x4_t o = red[base + v][lane];
      sum[0] += o[0];
      sum[1] += o[1];
      sum[2] += o[2];
      sum[3] += o[3];
    }
    const int j = j0 + 16 * t + row;
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

template <int STEPS, int RT>
__global__ __launch_bounds__(64 * kShrinkWaves) void shrink_mfma_pair(ShrinkArgs s) {
  __shared__ f32x4_t red[2 * RT * kShrinkWaves][64];
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
      shrink_pair_body<STEPS, RT>(s, rgg, h0, t0, true, h1, t1, red);
    } else {
      shrink_pair_body<STEPS, RT>(s, rgg, h0, t0, false, h0, t0, red);
      if (has1) shrink_pair_body<STEPS, RT>(s, rgg, h1, t1, false, h1, t1, red);
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
__global__ __launch_bounds__(64 * kShrinkWaves)
__attribute__((amdgpu_waves_per_eu(STEPS <= 8 ? 4 : 1))) void plan_shrink(PlanArgs A,
                                                                          ShrinkArgs s) {
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
  // the first job's A fragments depend only on its item's head: issue them
  // now, so that their latency overlaps the token lists below
  // (8 K steps: 32 more registers, within four waves a SIMD)
  const bool pre = STEPS <= 8 && job0 < n_items * s.rg_total;
  uint4 pa[STEPS] = {};
  if (pre) shrink_first_a<STEPS>(s, job0, li[job0 / s.rg_total].head, pa);
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
  shrink_mfma_jobs_pre<STEPS, 1, true>(s, job0, stride, red, li, n_items, pa, pre);
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

// C consecutive outputs.  y is touched once per launch: its loads and stores
// carry the non-temporal hint so that the streamed rows do not evict the B
// rows held in L2.
template <typename TY, int C>
struct OutN;


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
      // z of the batch (entries at or beyond the effective rank are never
      // used; a split shrink leaves nkc partial rows per tuple, added in
      // chunk order).  Batches of four or more slots take it through vector
      // loads issued before the B rows: lane l holds rank jb + l % RB of slot
      // l / RB (SB * RB = BR <= 32 lanes), so the batch waits for one memory
      // round trip.  Through the scalar loads below, each slot's z rows were
      // waited for before the next slot's B rows were issued: distinct
      // decode, four slots a batch, 15.0 -> 14.3 us a step.  Batches of two
      // slots measured faster with the scalar loads (skewed decode, 38.3 vs
      // 38.5-38.9 us), and keep them.
      constexpr bool kVecZ = SB >= 4;
      float zv[SB][RB];
      float zc[kVecZ ? (SPLIT ? 4 : 1) : 1];
      bool zin = false;
      const float *zrow = Z;
      if constexpr (kVecZ) {
        const int zb = lane / RB, zj = lane % RB;
        int zp = 0, zk = 0;
#pragma unroll
        for (int b = 0; b < SB; ++b)
          if (zb == b) {
            zp = pp[b];
            zk = kk[b];
          }
        zin = zb < SB && jb + zj < zk;
        zrow = Z + int64_t(zp) * (SPLIT ? zstride : zld) + jb + zj;
#pragma unroll
        for (int i = 0; i < (SPLIT ? 4 : 1); ++i) {
          zc[i] = 0.f;
          if (zin && i < nkc) zc[i] = zrow[i * zld];
        }
      }
#pragma unroll
      for (int b = 0; b < SB; ++b) {
#pragma unroll
        for (int jj = 0; jj < RB; ++jj) {
          const int j = jb + jj;
          if (j < kk[b] && active) bv[b][jj].load(B + (int64_t(aa[b]) * r_max + j) * d + n0);
          else bv[b][jj].zero();
        }
        // y right after the first batch's first B rows: its latency then
        // overlaps theirs instead of the slot records' (the memory counter
        // is in order, so a load issued before the slot records would be
        // waited for together with them)
        if (sb == 0 && jb == 0 && b == 0 && active) yv.load(Yp);
        if constexpr (kVecZ) {
          // z came in above
        } else if constexpr (!SPLIT) {
          // one z row per tuple, read as whole vectors
          const float *zr1 = Z + int64_t(pp[b]) * zld + jb;
          if ((zld & 3) == 0) {
            const float4 *zr = reinterpret_cast<const float4 *>(zr1);
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
            for (int jj = 0; jj < RB; ++jj) zv[b][jj] = jb + jj < kk[b] ? zr1[jj] : 0.f;
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
      float zl = 0.f;
      if constexpr (kVecZ) {
        if constexpr (SPLIT) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < nkc) zl += zc[i];
          for (int c = 4; c < nkc; ++c)  // beyond four chunks, one at a time
            if (zin) zl += zrow[c * zld];
        } else {
          zl = zc[0];
        }
      }
#pragma unroll
      for (int b = 0; b < SB; ++b)
#pragma unroll
        for (int jj = 0; jj < RB; ++jj)
          if (jb + jj < kk[b]) {
            const float z =
                kVecZ ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zl), b * RB + jj))
                      : zv[b][jj];
            bv[b][jj].fma_into(al[b] * z, acc);
          }
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
// Matrix-core shrink for bf16 pools.  TCL_SHRINK=valu runs the fp32 VALU
// kernel on them instead (whole-d_in z rows, no fused mapping): the
// measurement of the two decode shrinks against each other.
static bool mfma_shrink(const tcl_module *mods) {
  if (mods[0].wdtype != TCL_BF16) return false;
  const char *e = std::getenv("TCL_SHRINK");
  return !(e && !std::strcmp(e, "valu"));
}

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
  if (!mfma_shrink(mods)) return 1 << 30;
  int kchunk;
  // TCL_KCHUNK=<elements> fixes the chunk width (tuning knob; 0 = policy)
  const int forced = env_int("TCL_KCHUNK", 0);
  if (forced > 0) {
    kchunk = (forced + 31) / 32 * 32;
  } else {
    // measured on decode batches: tiny batches (fewer workgroups than CUs)
    // gain most from 2048-element chunks, larger decode batches from
    // 4096-element chunks, prefill-sized batches lose from any split.
    // Prefill batches (with token tiles, whose expand sums the partial
    // planes eight at a time) of fewer than 1024 workgroups take
    // 2048-element chunks: sparse gated prefill (768 -> 1536 workgroups)
    // shrink 26.9 -> 23.6 us, step 138.9 -> 136.3 us.
    int64_t est_items = (p->L.cap < p->L.N ? p->L.cap : p->L.N) + p->L.cap / kTile;
    int64_t units = 0;
    for (int i = 0; i < n; ++i) units += (mods[i].r_max + 15) / 16;
    const int64_t wgs = est_items * units;
    if (p->L.tiles > 0 && wgs < 1024) kchunk = 2048;
    else kchunk = wgs < 256 ? 2048 : (wgs < 4096 ? 4096 : (1 << 30));
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

// Launch table and grid of the shrink of n (<= kMaxMods) modules; z[i] is
// module i's output, a row of nkc partial planes of zld[i] floats per tuple
// when kchunk < d_in.  rt: 16-rank tiles per matrix-core job.
static int64_t shrink_args(const tcl_plan *p, const tcl_module *mods, int n,
                           const void *const *x, const int64_t *ldx, float *const *z,
                           const int *zld, int kchunk, int zero_tail, ShrinkArgs &a,
                           int rt = 1) {
  const bool bf = mfma_shrink(mods);
  const int rows = bf ? 16 * rt : 4;  // rank rows per workgroup job
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
  const bool bf = mfma_shrink(mods);
  // Both 16-rank tiles of an item in one job (two accumulators on the same x
  // fragments, so x is loaded once for 32 ranks) when a module keeps more
  // than 16 ranks.  Retained-rank batch (r_max 32, item pairs): 141.7 ->
  // 97.7 us (without item pairs 156.9 -> 131.0 us).  TCL_SHRINK_RT=1 keeps
  // one tile a job.
  int r_top = 0;
  for (int i = 0; i < n; ++i) r_top = mods[i].r_max > r_top ? mods[i].r_max : r_top;
  const int rt = bf && r_top > 16 && env_int("TCL_SHRINK_RT", 2) == 2 ? 2 : 1;
  ShrinkArgs a;
  const int64_t grid = shrink_args(p, mods, n, x, ldx, z, zld, kchunk, zero_tail, a, rt);
  logf("shrink(%s): modules=%d units/item=%d kchunk=%d rank tiles/job=%d grid=%lld",
       bf ? "mfma" : "valu", n, a.rg_total, kchunk, rt, (long long)grid);
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
    if (rt == 2)
      hipLaunchKernelGGL((shrink_mfma_pair<4, 2>), dim3(int(pg)), dim3(64 * kShrinkWaves), 0, s,
                         a);
    else if (env_int("TCL_PSTEPS", 4) == 8)
      hipLaunchKernelGGL((shrink_mfma_pair<8, 1>), dim3(int(pg)), dim3(64 * kShrinkWaves), 0, s,
                         a);
    else
      hipLaunchKernelGGL((shrink_mfma_pair<4, 1>), dim3(int(pg)), dim3(64 * kShrinkWaves), 0, s,
                         a);
  } else if (bf && rt == 2)
    hipLaunchKernelGGL((shrink_mfma<8, 2>), dim3(int(grid)), dim3(64 * kShrinkWaves), 0, s, a);
  else if (bf && steps == 8)
    hipLaunchKernelGGL((shrink_mfma<8, 1>), dim3(int(grid)), dim3(64 * kShrinkWaves), 0, s, a);
  else if (bf)
    hipLaunchKernelGGL((shrink_mfma<16, 1>), dim3(int(grid)), dim3(64 * kShrinkWaves), 0, s, a);
  else if (mods[0].wdtype == TCL_BF16)
    hipLaunchKernelGGL((shrink_valu<bf16_t>), dim3(int(grid)), dim3(256), 0, s, a);
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
  if (mods[0].wdtype != TCL_BF16 || p->L.T < kMfmaMinTokens || p->L.N > kTileMaxAdapters)
    return false;
  for (int i = 0; i < n; ++i)
    if (!mods[i].B_k) return false;
  return dispatch_override() == 0;
}

// workspace bytes of the per-tile records of one launch of n modules
static size_t tile_rec_bytes(const tcl_plan *p, const tcl_module *mods, int n) {
  return use_tile_expand(p, mods, n) ? tile_records_bytes(p, n) : 0;
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
  if (rec && use_tile_expand(p, mods, n)) {
    int nkc[kMaxMods];
    for (int i = 0; i < n; ++i) nkc[i] = n_kchunks(&mods[i], kchunk);
    return launch_expand_tile(p, mods, n, z, zld, nkc, y, ldy, yd, rec, s);
  }
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
  *bytes = tile_pack_bytes(m);
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
  rc = launch_module_pack(m, B_k, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  m->B_k = B_k;
  return TCL_OK;
}

int tcl_bam_pool_init(tcl_module *m, int32_t *k_dev, void *B_k, size_t bytes, void *stream) {
  int rc = check_module(m);
  if (rc) return rc;
  if (!k_dev) return fail(TCL_EINVAL, "k_dev is NULL");
  if (reinterpret_cast<uintptr_t>(k_dev) & 3) return fail(TCL_EALIGN, "k_dev must be 4-byte aligned");
  if (B_k) {
    if (m->wdtype != TCL_BF16) return fail(TCL_EUNSUPPORTED, "the packed copy is for bf16 pools");
    if (reinterpret_cast<uintptr_t>(B_k) & 255)
      return fail(TCL_EALIGN, "B_k must be 256-byte aligned");
    if (bytes < tile_pack_bytes(m))
      return fail(TCL_ENOSPC, "B_k holds %zu bytes, needs %zu", bytes, tile_pack_bytes(m));
  }
  rc = launch_slot_pool_init(m, k_dev, B_k, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  m->k_dev = k_dev;
  m->B_k = B_k;
  return TCL_OK;
}

int tcl_bam_load(const tcl_module *m, const void *A_host, const void *B_host,
                 const int32_t *k_host, int32_t n_logical, int32_t n_loads,
                 const int32_t *load_slot, const int32_t *load_adapter, void *stream) {
  int rc = check_module(m);
  if (rc) return rc;
  if (!m->k_dev) return fail(TCL_EINVAL, "module is not a slot pool (k_dev NULL): tcl_bam_pool_init");
  if (n_loads < 0 || n_logical < 1) return fail(TCL_EINVAL, "n_loads < 0 or n_logical < 1");
  if (n_loads == 0) return TCL_OK;
  if (!A_host || !B_host || !load_slot || !load_adapter)
    return fail(TCL_EINVAL, "host pools and load lists are required");
  std::vector<int32_t> ranks(n_loads);
  for (int i = 0; i < n_loads; ++i) {
    const int sl = load_slot[i], a = load_adapter[i];
    if (sl < 0 || sl >= m->n_adapters)
      return fail(TCL_EINVAL, "load %d: slot %d outside [0, %d)", i, sl, m->n_adapters);
    if (a < 0 || a >= n_logical)
      return fail(TCL_EINVAL, "load %d: adapter %d outside [0, %d)", i, a, n_logical);
    for (int j = 0; j < i; ++j)
      if (load_slot[j] == sl) return fail(TCL_EINVAL, "slot %d loaded twice in one call", sl);
    const int k = k_host ? k_host[a] : m->r_max;
    if (k < 0 || k > m->r_max)
      return fail(TCL_EINVAL, "adapter %d: rank %d outside [0, %d]", a, k, m->r_max);
    ranks[i] = k;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t es = m->wdtype == TCL_BF16 ? 2 : 4;
  const size_t rowA = size_t(m->d_in) * es, rowB = size_t(m->d_out) * es;
  const size_t slotA = size_t(m->r_max) * rowA, slotB = size_t(m->r_max) * rowB;
  for (int i = 0; i < n_loads; ++i) {
    // rows at or beyond the retained rank are never read: copy rows < k only
    const size_t sl = size_t(load_slot[i]), a = size_t(load_adapter[i]), k = size_t(ranks[i]);
    if (k == 0) continue;
    TCL_HIP(hipMemcpyAsync(static_cast<char *>(const_cast<void *>(m->A_t)) + sl * slotA,
                           static_cast<const char *>(A_host) + a * slotA, k * rowA,
                           hipMemcpyHostToDevice, s));
    TCL_HIP(hipMemcpyAsync(static_cast<char *>(const_cast<void *>(m->B_t)) + sl * slotB,
                           static_cast<const char *>(B_host) + a * slotB, k * rowB,
                           hipMemcpyHostToDevice, s));
  }
  return launch_slot_update(m, load_slot, ranks.data(), n_loads, s);
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


}  // extern "C"

namespace tcl {

// Workspace of tcl_fused_apply_noalloc: a file-scope device array (each GPU
// holds its own copy at its own address from module load to process end).
// Host code never passes the array's name to a kernel or a copy (on the host
// it is a stand-in, not a device address): it looks the device address up
// once per device and uses that.
static __device__ __align__(256) unsigned char scratch[TCL_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
static void *g_scratch_dev[kScratchDevices];
static std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on the first call on
// that device with the device current.
static int scratch_address(void **out) {
  int dev = 0;
  TCL_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kScratchDevices)
    return fail(TCL_EUNSUPPORTED, "device %d beyond the %d the scratch table covers", dev,
                kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *ptr = nullptr;
    TCL_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(TCL_EHIP, "no device address for the scratch array");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return TCL_OK;
}

}  // namespace tcl

extern "C" {

int tcl_fused_apply_noalloc(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                            const void *const *x, const int64_t *ldx, tcl_dtype xd,
                            void *const *y, const int64_t *ldy, tcl_dtype yd, void *stream) {
  if (!x || !y) return fail(TCL_EINVAL, "x and y lists are required");
  if (!p) return fail(TCL_EINVAL, "plan is NULL");
  if (n_mods < 1 || !mods) return fail(TCL_EINVAL, "module list is required");
  for (int i = 0; i < n_mods; ++i) {
    int rc = check_plan_module(p, &mods[i]);
    if (rc) return rc;
  }
  const size_t need = ws_need(p, mods, n_mods);
  if (need > TCL_SCRATCH_BYTES)
    return fail(TCL_ENOSPC,
                "batch needs %zu bytes of workspace, the allocation-free apply holds %zu; "
                "use tcl_fused_apply with a caller workspace",
                need, size_t(TCL_SCRATCH_BYTES));
  void *ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc) return rc;
  rc = check_fused(p, mods, n_mods, x, ldx, xd, y, ldy, yd, ws, TCL_SCRATCH_BYTES);
  if (rc) return rc;
  // every workspace byte the kernels read was written earlier in the same
  // call (z by the shrink, the tile records by tile_prep): nothing to clear
  return run_fused(p, mods, n_mods, x, ldx, y, ldy, yd, ws, static_cast<hipStream_t>(stream));
}

// The decode step's shrink with the mapping stage inside (plan_shrink):
// direct-mode tables whose LDS view and work items fit the kernel's budget,
// bf16 pools, one launch's worth of modules.  TCL_FUSED_MAPPING=0 turns it
// off (the mapping kernel then runs on its own before the shrink).
static bool fused_mapping(const tcl_plan *p, const tcl_module *mods, int n_mods) {
  if (p->L.mode != PLAN_DIRECT || !mfma_shrink(mods) || n_mods > kMaxMods) return false;
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
