// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "tcl.h"

namespace tcl {

// ---------------------------------------------------------------------------
// error reporting
// ---------------------------------------------------------------------------
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_fail(hipError_t e, const char *what);
bool log_enabled();
void logf(const char *fmt, ...) __attribute__((format(printf, 1, 2)));

#define TCL_HIP(call)                                 \
  do {                                                \
    hipError_t e_ = (call);                           \
    if (e_ != hipSuccess) return ::tcl::hip_fail(e_, #call); \
  } while (0)

// ---------------------------------------------------------------------------
// plan layout
// ---------------------------------------------------------------------------

// Tokens per shrink work item: a segment of L tuples is cut into ceil(L/kTile)
// items of at most kTile consecutive tuples.
constexpr int kTile = 8;
// Threads of the single-workgroup mapping kernel.
constexpr int kPlanThreads = 1024;
// int32 words of LDS the mapping kernel may use to stage the composite table.
constexpr int kPlanLdsInts = 14336;

// device status words
enum { ST_CODE = 0, ST_TUPLES = 1, ST_SEGMENTS = 2, ST_ITEMS = 3, ST_WORDS = 64 };

// error bits raised by the mapping kernel
enum { EB_INVAL = 1, EB_UNSUP = 2, EB_NOSPC = 4 };

struct PlanLayout {
  // sizes
  int32_t T, G, NP, N, cap, items_cap;
  int32_t chunks;   // groups are split into this many contiguous chunks
  int32_t small;    // 1: stage the table and scratch in LDS
  // byte offsets inside the device buffer
  size_t o_status, o_tok, o_ad, o_slot, o_alpha, o_toktuple, o_tokptr, o_segad, o_segbeg,
      o_items, o_sslot, o_sgroup, o_spos, o_sgbase, o_shist, total;
};

int plan_layout(int32_t T, int32_t G, int32_t NP, int32_t N, int32_t cap, PlanLayout *L);

struct PlanDev {
  int32_t *status;
  int32_t *tup_token, *tup_adapter, *tup_slot;
  float *tup_alpha;
  int32_t *tok_tuple, *tok_ptr;
  int32_t *seg_adapter, *seg_begin;
  int4 *items;
  int32_t *s_slot, *s_group, *s_pos, *s_gbase, *s_hist;
};

}  // namespace tcl

struct tcl_plan {
  tcl::PlanLayout L;
  tcl::PlanDev d;
  void *buf;
  size_t buf_bytes;
};
