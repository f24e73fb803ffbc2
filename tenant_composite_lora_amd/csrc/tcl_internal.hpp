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

// Tuples per shrink work item: a segment of L tuples is cut into
// ceil(L/kTile) items of at most kTile consecutive tuples (the M dimension of
// a 16x16 MFMA tile).
constexpr int kTile = 16;
// Largest workgroup of the single-workgroup mapping kernel.
constexpr int kPlanThreads = 1024;
// Largest pair count handled by the direct-count mapping path.
constexpr int kDirectMaxPairs = 512;
// Slot records per token in the padded token table (= the most pairs a
// composite may hold).
constexpr int kSlotPad = TCL_MAX_PAIRS_PER_GROUP;
// int32 words of LDS the mapping kernel may use to stage the composite table.
// gfx950 gives a workgroup up to 160 KiB of LDS; the mapping stage uses 128.
constexpr int kPlanLdsInts = 32768;

// Prefill expand on the matrix cores: tokens per tile, and the smallest token
// count for which a plan orders its tokens into such tiles.
constexpr int kXTok = 64;
constexpr int kMfmaMinTokens = 256;
// Tuples per workgroup of the launch that flags the tile order; each
// workgroup lists its flagged tokens in a slice this long.
constexpr int kOrdThreads = 256;
inline int ord_blocks(int cap) { return (cap + kOrdThreads - 1) / kOrdThreads; }

// One apply launch covers up to kMaxMods modules that share the plan (e.g.
// the seven projections of a transformer layer).
constexpr int kMaxMods = 8;

// device status words
enum { ST_CODE = 0, ST_TUPLES = 1, ST_SEGMENTS = 2, ST_ITEMS = 3, ST_WORDS = 64 };

// error bits raised by the mapping kernel
enum { EB_INVAL = 1, EB_UNSUP = 2, EB_NOSPC = 4 };

struct PlanLayout {
  // sizes
  int32_t T, G, NP, N, cap, items_cap;
  int32_t chunks;   // counting path: groups are split into this many chunks
  int32_t mode;     // PLAN_DIRECT, PLAN_MULTI, PLAN_COUNT_LDS or PLAN_COUNT_GLOBAL
  int32_t blocks;   // PLAN_MULTI: workgroups of the local and scatter kernels
  int32_t threads;  // workgroup size of the mapping kernel (64, 256 or 1024)
  int32_t tiles;    // token tiles of kXTok of the prefill expand (0: none)
  // byte offsets inside the device buffer
  size_t o_status, o_tok, o_ad, o_slot, o_alpha, o_toktuple, o_tokrec, o_tokn, o_tokptr,
      o_segad, o_segbeg, o_items, o_sslot, o_sgroup, o_spos, o_sgbase, o_shist, o_sseg, o_ocnt,
      o_oitem, o_mhist, o_mblk, o_msst, o_msib, o_tab, total;
};

// Mapping-stage algorithms: small tables run in one workgroup with the table
// in LDS (direct); larger ones over many workgroups of consecutive groups
// (multi: local counts and ranks, one scan, scatter); tables beyond the
// multi path's limits run the chunked counting sort in one workgroup, with
// its scratch in LDS or, beyond LDS, in the plan buffer.
enum { PLAN_DIRECT = 0, PLAN_COUNT_LDS = 1, PLAN_COUNT_GLOBAL = 2, PLAN_MULTI = 3 };

int plan_layout(int32_t T, int32_t G, int32_t NP, int32_t N, int32_t cap, PlanLayout *L);

// host.cpp: NULL checks of a composite table's pointers, and the whole check
// of a host-resident table (codes and their precedence those of the mapping
// stage) with its tuple and touched-adapter counts
int check_composites(const tcl_composites *c);
int validate_host(const tcl_composites *c, int64_t *P_out, int32_t *U_out);

// A shrink work item: up to kTile consecutive tuples of one adapter's
// segment, with their token ids inlined so a wave needs one load to start.
struct Item {
  int4 head;    // adapter, first tuple, tuple count, segment index
  int tok[kTile];  // token ids of the tuples (unused entries repeat the first)
};

struct PlanDev {
  int32_t *status;
  int32_t *tup_token, *tup_adapter, *tup_slot;
  float *tup_alpha;
  int32_t *tok_tuple, *tok_ptr;
  int4 *tok_rec;   // [T][kSlotPad]: {tuple index, adapter, alpha bits, segment index}
  int32_t *tok_n;  // [T] slots per token
  int32_t *seg_adapter, *seg_begin;
  Item *items;
  int32_t *s_slot, *s_group, *s_pos, *s_gbase, *s_hist;
  int32_t *s_seg;  // counting / multi path: segment index of every touched adapter [N]
  // multi-workgroup path: per-(adapter, workgroup) tuple counts then bases
  // [blocks][N] (workgroup-major), per-workgroup {tuples, error bits, tuple
  // base, -} [blocks][4],
  // per-adapter segment start and first work item [N]
  int32_t *m_hist, *m_blk, *m_sst, *m_sib;
  // tile order: per workgroup of the flagging launch, its flagged items
  // (first ord_cnt[w] entries of slice w of ord_item, kOrdThreads each)
  int32_t *ord_cnt;
  int32_t *ord_item;
};

}  // namespace tcl

struct tcl_plan {
  tcl::PlanLayout L;
  tcl::PlanDev d;
  void *buf;
  size_t buf_bytes;
  // host-resident tables (tcl_plan_map_host, tcl_plan_remap_host): a pinned
  // staging copy the H2D copy reads from, and the event after that copy
  void *stage = nullptr;
  size_t stage_bytes = 0;
  hipEvent_t stage_ev = nullptr;
  bool stage_pending = false;
  // tuple and segment counts known on the host (the last table was a host
  // table, validated and counted there); -1 otherwise
  int32_t host_tuples = -1, host_segments = -1;
};

namespace tcl {
// Queue the token order of the prefill expand's tiles of p on stream s,
// behind the mapping kernel(s) that wrote the plan (no-op for batches without
// token tiles).  Every mapping launch ends with it, so the order always
// belongs to the plan the stream last wrote.
int plan_launch_tile_order(const tcl_plan *p, hipStream_t s);
}
