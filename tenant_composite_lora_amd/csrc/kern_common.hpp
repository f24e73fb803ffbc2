// Device helpers and launch-table types shared by the apply kernels.
#pragma once

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

// matrix-core operand types
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// 2- and 4-element vectors of the plain and non-temporal y accesses
typedef float nt_f2 __attribute__((ext_vector_type(2)));
typedef float nt_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u2 __attribute__((ext_vector_type(2)));
typedef uint32_t nt_u4 __attribute__((ext_vector_type(4)));

}  // namespace tcl
