// Token-level gate: the composite table of dynamic composition from gate
// logits (DyMerge-LoRA, section 3.1 dynamic composition; section 5.1 Sparse
// workload).  One wave per token, one lane per candidate: the softmax over
// the valid candidates, then k rounds of a wave-wide maximum pick the kept
// pairs.  The table goes straight to the mapping stage in device memory.
#include <cmath>

#include "tcl_internal.hpp"

namespace tcl {
namespace {

constexpr int kGateWaves = 4;  // tokens per workgroup

struct GateArgs {
  const float *logits;
  const int32_t *cand;
  int64_t ldl, ldc;
  int32_t T, C, k;
  int32_t *gtp, *gpp, *pa;
  float *pw;
};

// Butterfly reductions over the 64 lanes.  Every lane ends with the same
// value: each step adds (or compares) two partial results that two lanes
// hold in swapped order, and both operations are commutative.
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__global__ __launch_bounds__(64 * kGateWaves) void gate_topk_kernel(GateArgs g) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kGateWaves + (threadIdx.x >> 6);
  if (t > g.T) return;
  if (t == g.T) {
    // the end entries of the two pointer arrays
    if (lane == 0) {
      g.gtp[t] = t;
      g.gpp[t] = t * g.k;
    }
    return;
  }
  const bool in = lane < g.C;
  const int id = in ? g.cand[int64_t(t) * g.ldc + lane] : -1;
  const bool valid = id >= 0;
  const float l = valid ? g.logits[int64_t(t) * g.ldl + lane] : 0.f;
  const bool bad = __ballot(valid && !isfinite(l)) != 0;
  const float m = wave_max(valid ? l : -INFINITY);
  const float e = valid ? expf(l - m) : 0.f;
  const float p = e / wave_sum(e);

  // k rounds: the remaining valid lane with the largest logit, the lowest
  // such lane on ties; lane i keeps round i's pick
  uint64_t left = __ballot(valid);
  int my_a = -1;
  float my_p = 0.f;
  for (int i = 0; i < g.k; ++i) {
    const bool cand_here = (left >> lane) & 1;
    const float mx = wave_max(cand_here ? l : -INFINITY);
    const uint64_t win = __ballot(cand_here && l == mx);
    if (win == 0) break;  // fewer valid candidates than k
    const int wl = __builtin_ctzll(win);
    const int a = __shfl(id, wl, 64);
    const float pv = __shfl(p, wl, 64);
    if (lane == i) {
      my_a = a;
      my_p = pv;
    }
    left &= ~(uint64_t(1) << wl);
  }
  if (bad) {
    my_a = -1;
    my_p = 0.f;
  }
  if (lane < g.k) {
    g.pa[int64_t(t) * g.k + lane] = my_a;
    g.pw[int64_t(t) * g.k + lane] = my_p;
  }
  if (lane == 0) {
    g.gtp[t] = t;
    g.gpp[t] = t * g.k;
  }
}

}  // namespace
}  // namespace tcl

using namespace tcl;

extern "C" int tcl_gate_topk(const float *logits, int64_t ld_logits, const int32_t *candidates,
                             int64_t ld_candidates, int32_t n_tokens, int32_t n_candidates,
                             int32_t k, int32_t *group_tok_ptr, int32_t *group_pair_ptr,
                             int32_t *pair_adapter, float *pair_alpha, void *stream) {
  if (!group_tok_ptr || !group_pair_ptr || !pair_adapter || !pair_alpha)
    return fail(TCL_EINVAL, "gate: the output pointers are required");
  if ((!logits || !candidates) && n_tokens > 0)
    return fail(TCL_EINVAL, "gate: logits and candidates are required");
  if (n_tokens < 0) return fail(TCL_EINVAL, "gate: n_tokens %d < 0", n_tokens);
  if (n_candidates < 1 || n_candidates > 64)
    return fail(TCL_EINVAL, "gate: n_candidates %d outside 1..64", n_candidates);
  if (k < 1 || k > n_candidates || k > TCL_MAX_PAIRS_PER_GROUP)
    return fail(TCL_EINVAL, "gate: k %d outside 1..min(n_candidates, %d)", k,
                TCL_MAX_PAIRS_PER_GROUP);
  if (ld_logits < n_candidates || ld_candidates < n_candidates)
    return fail(TCL_EINVAL, "gate: leading dimensions must be >= n_candidates");
  if (int64_t(n_tokens) * k >= (int64_t(1) << 31))
    return fail(TCL_EINVAL, "gate: n_tokens * k beyond 32-bit indexing");
  const uintptr_t al = reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(candidates) |
                       reinterpret_cast<uintptr_t>(group_tok_ptr) |
                       reinterpret_cast<uintptr_t>(group_pair_ptr) |
                       reinterpret_cast<uintptr_t>(pair_adapter) |
                       reinterpret_cast<uintptr_t>(pair_alpha);
  if (al & 3) return fail(TCL_EALIGN, "gate: pointers must be 4-byte aligned");
  GateArgs g{logits, candidates, ld_logits, ld_candidates, n_tokens, n_candidates, k,
             group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha};
  // one wave per token plus one for the end entries of the pointer arrays
  const int64_t waves = int64_t(n_tokens) + 1;
  const int blocks = int((waves + kGateWaves - 1) / kGateWaves);
  hipLaunchKernelGGL(gate_topk_kernel, dim3(blocks), dim3(64 * kGateWaves), 0,
                     static_cast<hipStream_t>(stream), g);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}
