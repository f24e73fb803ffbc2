// The packed, rank-contiguous copy of a bf16 pool's B that the prefill expand
// over token tiles reads (tcl_module_pack), and the slot updates of an
// adapter slot pool that keep it current (tcl_bam_pool_init, tcl_bam_load;
// DyMerge-LoRA section 4, BAM).

#include <cstdint>

#include "kern_common.hpp"
#include "tcl_internal.hpp"
#include "tile.hpp"

namespace tcl {

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

// Column n of one adapter's packed copy: its k retained B rows (src points at
// row 0, column n; rows d apart) as ceil(k / 8) 16-byte octets.
__device__ inline void pack_column(const uint16_t *src, int d, int k, uint4 *dst) {
  const int octs = (k + 7) >> 3;
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

// One thread per (adapter, column): k loads along the rank (each coalesced
// across the threads of a workgroup), ceil(k / 8) 16-byte stores.
__global__ __launch_bounds__(256) void pack_b_kernel(const uint16_t *Bt, const int32_t *k_dev,
                                                     int32_t N, int32_t r_max, int32_t d,
                                                     const int32_t *off, uint4 *Bk) {
  const int blocks = (d + 255) / 256;
  const int a = blockIdx.x / blocks, n = (blockIdx.x - a * blocks) * 256 + threadIdx.x;
  if (a >= N || n >= d) return;
  const int k = eff_rank(k_dev, a, r_max);
  pack_column(Bt + int64_t(a) * r_max * d + n, d, k, Bk + int64_t(off[a]) + int64_t(n) * ((k + 7) >> 3));
}

// Slot updates of an adapter slot pool (DyMerge-LoRA section 4, BAM: the
// slots hold raw adapter factors; a load replaces a slot's adapter).  The
// pool's packed copy has a fixed region per slot (offsets of a pack with
// every slot at r_max), so a load re-packs only its own slot.  One thread
// per (load, column); the thread of column 0 also writes the slot's rank.
constexpr int kSlotBatch = 64;
struct SlotArgs {
  int32_t n;
  int32_t slot[kSlotBatch];
  int32_t k[kSlotBatch];
};

__global__ __launch_bounds__(256) void slot_update_kernel(const uint16_t *Bt, int32_t *k_dev,
                                                          int32_t r_max, int32_t d,
                                                          const int32_t *off, uint4 *Bk,
                                                          SlotArgs a) {
  const int blocks = (d + 255) / 256;
  const int i = blockIdx.x / blocks, n = (blockIdx.x - i * blocks) * 256 + threadIdx.x;
  if (i >= a.n || n >= d) return;
  const int sl = a.slot[i], k = a.k[i];
  if (n == 0) k_dev[sl] = k;
  if (Bk) pack_column(Bt + int64_t(sl) * r_max * d + n, d, k, Bk + int64_t(off[sl]) + int64_t(n) * ((k + 7) >> 3));
}

// Every slot of a new pool empty: rank 0.
__global__ __launch_bounds__(256) void slot_clear_kernel(int32_t *k_dev, int32_t n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) k_dev[i] = 0;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int r_pad(const tcl_module *m) { return (m->r_max + 7) / 8 * 8; }

// bytes before the packed data: the adapters' first 16-byte units, then a
// zero 16-byte unit right before the data
size_t tile_pack_head_bytes(const tcl_module *m) {
  return (size_t(m->n_adapters) * 4 + 16 + 255) & ~size_t(255);
}

size_t tile_pack_bytes(const tcl_module *m) {
  return tile_pack_head_bytes(m) + size_t(m->n_adapters) * size_t(m->d_out) * size_t(r_pad(m)) * 2;
}

int launch_module_pack(const tcl_module *m, void *B_k, hipStream_t s) {
  const int blocks = (m->d_out + 255) / 256;
  const int64_t grid = int64_t(m->n_adapters) * blocks;
  const int64_t units = int64_t(m->n_adapters) * m->d_out * (r_pad(m) / 8);
  if (grid > (int64_t(1) << 31) - 1 || units > (int64_t(1) << 31) - 1)
    return fail(TCL_EUNSUPPORTED, "pool too large to pack");
  int32_t *off = static_cast<int32_t *>(B_k);
  uint4 *data = reinterpret_cast<uint4 *>(static_cast<char *>(B_k) + tile_pack_head_bytes(m));
  hipLaunchKernelGGL(pack_offsets_kernel, dim3(1), dim3(kPackThreads), 0, s, m->k_dev,
                     m->n_adapters, m->r_max, m->d_out, off, data - 1);
  hipLaunchKernelGGL(pack_b_kernel, dim3(unsigned(grid)), dim3(256), 0, s,
                     static_cast<const uint16_t *>(m->B_t), m->k_dev, m->n_adapters, m->r_max,
                     m->d_out, off, data);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

int launch_slot_pool_init(const tcl_module *m, int32_t *k_dev, void *B_k, hipStream_t s) {
  const int64_t units = int64_t(m->n_adapters) * m->d_out * (r_pad(m) / 8);
  if (units > (int64_t(1) << 31) - 1) return fail(TCL_EUNSUPPORTED, "pool too large to pack");
  if (B_k) {
    // offsets of a pack with every slot at r_max: slot s starts at s * d * ceil(r_max / 8)
    uint4 *data = reinterpret_cast<uint4 *>(static_cast<char *>(B_k) + tile_pack_head_bytes(m));
    hipLaunchKernelGGL(pack_offsets_kernel, dim3(1), dim3(kPackThreads), 0, s, nullptr,
                       m->n_adapters, m->r_max, m->d_out, static_cast<int32_t *>(B_k), data - 1);
  }
  hipLaunchKernelGGL(slot_clear_kernel, dim3((m->n_adapters + 255) / 256), dim3(256), 0, s, k_dev,
                     m->n_adapters);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

int launch_slot_update(const tcl_module *m, const int32_t *slots, const int32_t *ranks, int n,
                       hipStream_t s) {
  const int blocks = (m->d_out + 255) / 256;
  const int32_t *off = static_cast<const int32_t *>(m->B_k);
  uint4 *data = m->B_k ? reinterpret_cast<uint4 *>(static_cast<char *>(const_cast<void *>(m->B_k)) +
                                                   tile_pack_head_bytes(m))
                       : nullptr;
  for (int i0 = 0; i0 < n; i0 += kSlotBatch) {
    SlotArgs a{};
    a.n = n - i0 < kSlotBatch ? n - i0 : kSlotBatch;
    for (int i = 0; i < a.n; ++i) {
      a.slot[i] = slots[i0 + i];
      a.k[i] = ranks[i0 + i];
    }
    hipLaunchKernelGGL(slot_update_kernel, dim3(unsigned(int64_t(a.n) * blocks)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(m->B_t), const_cast<int32_t *>(m->k_dev), m->r_max, m->d_out, off,
                       data, a);
  }
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

}  // namespace tcl
