// Token-level gate: the composite table of dynamic composition from gate
// logits (DyMerge-LoRA, section 3.1 dynamic composition; section 5.1 Sparse
// workload; the one-minute summary's padding and masking of the gate's
// vectorised form).  Three launches:
//   gate_count_kernel  one wave per token: how many pairs the token keeps
//                      (k, fewer when it has fewer valid candidates, k again
//                      for a token with a non-finite logit, whose pairs name
//                      adapter -1 so that the mapping stage rejects the
//                      table), into group_pair_ptr[t + 1];
//   gate_scan_kernel   one workgroup: those counts into the pair offsets;
//   gate_topk_kernel   one wave per token, one lane per candidate: the
//                      softmax over the valid candidates, then rounds of a
//                      wave-wide maximum pick the kept pairs, written at the
//                      token's offset; each token also writes its share of
//                      the unused tail of the pair arrays (adapter -1,
//                      weight 0), so every entry is defined.
// The table goes straight to the mapping stage in device memory.  The work
// per token is a few dozen instructions; the time is the launches and a load
// round trip each.
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

// The candidate row of token t: one lane per candidate.
struct GateRow {
  int id;
  float l;
  bool valid;
};

__device__ inline GateRow gate_row(const GateArgs &g, int t, int lane) {
  // both loads at once (the logit does not wait for the id)
  const bool in = lane < g.C;
  const int id = in ? g.cand[int64_t(t) * g.ldc + lane] : -1;
  const float lin = in ? g.logits[int64_t(t) * g.ldl + lane] : 0.f;
  const bool valid = id >= 0;
  return {id, valid ? lin : 0.f, valid};
}

// pairs token t keeps: min(k, valid candidates), or k when a valid logit is
// not finite (those pairs name adapter -1)
__device__ inline int gate_kept(const GateArgs &g, const GateRow &r) {
  const bool bad = __ballot(r.valid && !isfinite(r.l)) != 0;
  const int nv = __popcll(__ballot(r.valid));
  return bad ? g.k : min(g.k, nv);
}

__global__ __launch_bounds__(64 * kGateWaves) void gate_count_kernel(GateArgs g) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kGateWaves + (threadIdx.x >> 6);
  if (t >= g.T) return;
  const GateRow r = gate_row(g, t, lane);
  const int n = gate_kept(g, r);
  if (lane == 0) g.gpp[t + 1] = n;
}

// In place: group_pair_ptr[t + 1] from the count of token t to the end of its
// pairs.  Thread i owns a contiguous run of tokens.  (Counting inside this
// one workgroup instead of in gate_count_kernel serialises a load round trip
// per token a wave: 46 us for 2048 tokens against 7 us for the three
// launches.)
constexpr int kGateScanThreads = 1024;

__global__ __launch_bounds__(kGateScanThreads) void gate_scan_kernel(int32_t *gpp, int32_t T) {
  __shared__ int wsum[kGateScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (T + kGateScanThreads - 1) / kGateScanThreads;
  const int t0 = min(T, tid * per), t1 = min(T, t0 + per);
  int own = 0;
  for (int t = t0; t < t1; ++t) own += gpp[t + 1];
  int inc = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o, 64);
    if (lane >= o) inc += u;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int run = inc - own;
  for (int j = 0; j < w; ++j) run += wsum[j];
  for (int t = t0; t < t1; ++t) {
    const int c = gpp[t + 1];
    run += c;
    gpp[t + 1] = run;
  }
  if (tid == 0) gpp[0] = 0;
}

__global__ __launch_bounds__(64 * kGateWaves) void gate_topk_kernel(GateArgs g) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kGateWaves + (threadIdx.x >> 6);
  if (t > g.T) return;
  if (t == g.T) {
    if (lane == 0) g.gtp[t] = t;  // the end entry (group_pair_ptr's is the scan's)
    return;
  }
  const GateRow r = gate_row(g, t, lane);
  const int base = g.gpp[t], n = g.gpp[t + 1] - base, total = g.gpp[g.T];
  const bool bad = __ballot(r.valid && !isfinite(r.l)) != 0;
  const float m = wave_max(r.valid ? r.l : -INFINITY);
  const float e = r.valid ? expf(r.l - m) : 0.f;
  const float p = e / wave_sum(e);

  // n rounds: the remaining valid lane with the largest logit, the lowest
  // such lane on ties; lane i keeps round i's pick
  uint64_t left = __ballot(r.valid);
  int my_a = -1;
  float my_p = 0.f;
  for (int i = 0; i < n && !bad; ++i) {
    const bool cand_here = (left >> lane) & 1;
    const float mx = wave_max(cand_here ? r.l : -INFINITY);
    const uint64_t win = __ballot(cand_here && r.l == mx);
    if (win == 0) break;
    const int wl = __builtin_ctzll(win);
    const int a = __builtin_amdgcn_readlane(r.id, wl);
    const float pv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), wl));
    if (lane == i) {
      my_a = a;
      my_p = pv;
    }
    left &= ~(uint64_t(1) << wl);
  }
  // lanes [0, n): the kept pairs at the token's offset; lanes [n, k): the
  // token's share of the unused tail, after the total (the tokens before it
  // left t * k - base entries of the tail)
  if (lane < g.k) {
    const int64_t at = lane < n ? int64_t(base) + lane
                                : int64_t(total) + int64_t(t) * g.k - base + (lane - n);
    g.pa[at] = lane < n ? my_a : -1;
    g.pw[at] = lane < n ? my_p : 0.f;
  }
  if (lane == 0) g.gtp[t] = t;
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int count_blocks = int((int64_t(n_tokens) + kGateWaves - 1) / kGateWaves);
  if (count_blocks > 0)
    hipLaunchKernelGGL(gate_count_kernel, dim3(count_blocks), dim3(64 * kGateWaves), 0, s, g);
  hipLaunchKernelGGL(gate_scan_kernel, dim3(1), dim3(kGateScanThreads), 0, s, group_pair_ptr,
                     n_tokens);
  // one wave per token plus one for the end entry of group_tok_ptr
  const int64_t waves = int64_t(n_tokens) + 1;
  const int blocks = int((waves + kGateWaves - 1) / kGateWaves);
  hipLaunchKernelGGL(gate_topk_kernel, dim3(blocks), dim3(64 * kGateWaves), 0, s, g);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}
