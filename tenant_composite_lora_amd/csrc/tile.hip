// Prefill expand over 64-token tiles on the matrix cores (it reads the packed
// rank-contiguous copy of B that pack.hip writes).
//
// LoRAForge approach (4), RowExpand: an adapter's B rows serve every token of
// a tile that holds the adapter.  DyMerge-LoRA section 4.3: one kernel
// aggregates every (token, adapter) pair of the batch.

#include <cstdint>

#include "kern_common.hpp"
#include "tcl_internal.hpp"
#include "tile.hpp"

namespace tcl {

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
constexpr int kRHcap = 512;      // K octets (4096 ranks) per tile
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
  // the tile order: per workgroup of the plan's flagging launch the count
  // of its flagged items, listed at the start of its kOrdThreads-entry slice
  const int32_t *ord_cnt, *ord_item;
  int32_t ord_blocks;
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
  // row tid of the tile: position tile * kXTok + tid of the plan's tile
  // order.  The flagging launch's counts are scanned kOrdThreads at a time
  // until they pass the tile's last position; each row finds the workgroup
  // that lists its position with a binary search over the scanned counts
  // (s_p is free until the tuples are gathered below).
  int t = -1;
  {
    const int want0 = tile * kXTok, want = want0 + tid;
    int base = 0;
    for (int c0 = 0; ok && c0 < e.ord_blocks; c0 += kOrdThreads) {
      const int j = c0 + tid;
      s_p[tid] = j < e.ord_blocks ? e.ord_cnt[j] : 0;
      __syncthreads();
      const int total = lds_scan(s_p, kOrdThreads, tmp);  // exclusive, in place
      if (tid < kXTok && want >= base && want < base + total) {
        const int r = want - base;
        int lo = 0, hi = kOrdThreads - 1;  // the last workgroup listed at or before r
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_p[mid] <= r) lo = mid;
          else hi = mid - 1;
        }
        t = e.ord_item[int64_t(c0 + lo) * kOrdThreads + (r - s_p[lo])];
      }
      base += total;
      __syncthreads();  // s_p is rewritten by the next pass
      if (base >= want0 + kXTok) break;
    }
  }
  if (tid < kXTok) {
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
    // the partial planes in order, eight at a time with every load issued
    // before the sums (a plane row holds the octet's first four floats, and
    // the next four when the octet reaches past rank j0 + 4); floats at or
    // beyond k are dropped below
    float zv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) zv[i] = 0.f;
    const float *zr = Z + int64_t(s_p[q]) * zstride + j0;
    const bool hi = j0 + 4 < k;
    for (int c0 = 0; c0 < nkc; c0 += 8) {
      float4 v[8][2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float4 *src = reinterpret_cast<const float4 *>(zr + (c0 + u) * zld);
        const bool in = c0 + u < nkc;
        v[u][0] = in ? src[0] : make_float4(0.f, 0.f, 0.f, 0.f);
        v[u][1] = in && hi ? src[1] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u >= nkc) break;
        zv[0] += v[u][0].x;
        zv[1] += v[u][0].y;
        zv[2] += v[u][0].z;
        zv[3] += v[u][0].w;
        zv[4] += v[u][1].x;
        zv[5] += v[u][1].y;
        zv[6] += v[u][1].z;
        zv[7] += v[u][1].w;
      }
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
  // that XCD's L2).  A column block's tiles run in the plan's tile order:
  // tokens grouped by their rarest adapter, so neighbouring tiles, running
  // together, share most of their unions' B octets in L2.
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
  // (the header is the same for every lane: scalar registers make the
  // step loop's trip count uniform and its branches scalar)
  const int Q = __builtin_amdgcn_readfirstlane(rl[0]), H = __builtin_amdgcn_readfirstlane(rl[1]);
  const int fast = __builtin_amdgcn_readfirstlane(rl[2]), C = __builtin_amdgcn_readfirstlane(rl[3]);
  const int U = __builtin_amdgcn_readfirstlane(rl[4]);
  const int oidx = __builtin_amdgcn_readfirstlane(rl[5]), ocoef = __builtin_amdgcn_readfirstlane(rl[6]);
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
  // order) and the later steps' loads stay in flight.  The loop runs whole
  // groups of six steps (the register rotation's period) and leaves by its
  // latch alone, the last steps following it: an exit from inside the body
  // makes the compiler merge that exit's counter state into the top of the
  // loop, which then waits for every load in flight once a pass.
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
  int st = 0;
  for (; st + 6 <= nsteps; st += 6) {
    step(a0, b0, b1, st);
    step(a1, b1, b0, st + 1);
    step(a2, b0, b1, st + 2);
    step(a0, b1, b0, st + 3);
    step(a1, b0, b1, st + 4);
    step(a2, b1, b0, st + 5);
  }
  if (st < nsteps) {
    step(a0, b0, b1, st);
    if (st + 1 < nsteps) {
      step(a1, b1, b0, st + 1);
      if (st + 2 < nsteps) {
        step(a2, b0, b1, st + 2);
        if (st + 3 < nsteps) {
          step(a0, b1, b0, st + 3);
          if (st + 4 < nsteps) step(a1, b0, b1, st + 4);
        }
      }
    }
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

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static_assert(kRMaxQ >= kOrdThreads, "tile_prep scans the tile order's counts in s_p");
static_assert(32 * kRMaxWords == kTileMaxAdapters, "record bitmap covers the adapter limit");

static int n_tiles(const tcl_plan *p) { return (p->L.T + kXTok - 1) / kXTok; }

size_t tile_records_bytes(const tcl_plan *p, int n_mods) {
  return size_t(n_mods) * size_t(n_tiles(p)) * kRWords * 4;
}

int launch_expand_tile(const tcl_plan *p, const tcl_module *mods, int n, float *const *z,
                       const int *zld, const int *nkc, void *const *y, const int64_t *ldy,
                       tcl_dtype yd, int32_t *rec, hipStream_t s) {
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
    M.nkc = nkc[i];
    M.zstride = M.nkc * zld[i];
    M.first = int32_t(jobs);
    jobs += int64_t(M.n_ct) * e.tiles;
    e.bk_off[i] = static_cast<const int32_t *>(mods[i].B_k);
    e.bk_data[i] = reinterpret_cast<const uint4 *>(static_cast<const char *>(mods[i].B_k) +
                                                   tile_pack_head_bytes(&mods[i]));
    e.bk_zero[i] = e.bk_data[i] - 1;
  }
  if (jobs > (int64_t(1) << 30)) return fail(TCL_EUNSUPPORTED, "expand grid too large");
  e.jobs = int32_t(jobs);
  e.jobs_per_xcd = int32_t((jobs + 7) / 8);
  e.ord_cnt = p->d.ord_cnt;
  e.ord_item = p->d.ord_item;
  e.ord_blocks = ord_blocks(p->L.cap);
  logf("expand(tile): modules=%d tiles=%d jobs=%lld", n, e.tiles, (long long)jobs);
  hipLaunchKernelGGL(tile_prep, dim3(n * e.tiles), dim3(256), 0, s, e);
  if (yd == TCL_BF16)
    hipLaunchKernelGGL((expand_tile<bf16_t>), dim3(8 * e.jobs_per_xcd), dim3(256), 0, s, e);
  else
    hipLaunchKernelGGL((expand_tile<float>), dim3(8 * e.jobs_per_xcd), dim3(256), 0, s, e);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

}  // namespace tcl
