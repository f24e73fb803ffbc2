// Token-level gate: the composite table of dynamic composition from gate
// logits (DyMerge-LoRA, section 3.1 dynamic composition; section 5.1 Sparse
// workload).  One wave per token, one lane per candidate: the softmax over
// the valid candidates, then k rounds of a wave-wide maximum pick the kept
// pairs.  The table goes straight to the mapping stage in device memory.
// The work per token is a few dozen instructions; the time is the launch
// and one load round trip.
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

// Reductions over the 64 lanes with DPP moves (no LDS traffic): steps of
// 1, 2, 4 and 8 lanes inside each row of 16, then the row broadcasts carry
// rows 0 and 1 into rows 1 and 3 and rows 2 and 3, so lane 63 ends with the
// whole wave's result, which is then read as a uniform value.  Lanes without
// a source take the operation's identity.  The order of the operations is
// fixed, so the result is the same on every run.
template <int CTRL, int ROW_MASK, typename Op>
__device__ inline float dpp_step(float v, int identity, Op op) {
  const float o = __int_as_float(
      __builtin_amdgcn_update_dpp(identity, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
  return op(v, o);
}

template <typename Op>
__device__ inline float wave_reduce(float v, float identity, Op op) {
  const int id = __float_as_int(identity);
  v = dpp_step<0x111, 0xf>(v, id, op);  // row_shr:1
  v = dpp_step<0x112, 0xf>(v, id, op);  // row_shr:2
  v = dpp_step<0x114, 0xf>(v, id, op);  // row_shr:4
  v = dpp_step<0x118, 0xf>(v, id, op);  // row_shr:8
  v = dpp_step<0x142, 0xa>(v, id, op);  // row_bcast:15
  v = dpp_step<0x143, 0xc>(v, id, op);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ inline float wave_max(float v) {
  return wave_reduce(v, -INFINITY, [](float a, float b) { return fmaxf(a, b); });
}

__device__ inline float wave_sum(float v) {
  return wave_reduce(v, 0.f, [](float a, float b) { return a + b; });
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
  // both loads at once (the logit does not wait for the id)
  const bool in = lane < g.C;
  const int id = in ? g.cand[int64_t(t) * g.ldc + lane] : -1;
  const float lin = in ? g.logits[int64_t(t) * g.ldl + lane] : 0.f;
  const bool valid = id >= 0;
  const float l = valid ? lin : 0.f;
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
    const int a = __builtin_amdgcn_readlane(id, wl);
    const float pv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), wl));
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
