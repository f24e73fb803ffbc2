// Host side of the prefill expand over token tiles (tile.hip) and of the
// packed copy of B it reads (pack.hip), as the apply entry points call them.
#pragma once

#include <cstddef>
#include <cstdint>

#include "tcl_internal.hpp"

namespace tcl {

// Adapters a tile record's adapter bitmap covers: larger pools run the
// per-token expand.
constexpr int kTileMaxAdapters = 4096;

// Workspace bytes of the per-tile records of one launch over n_mods modules.
size_t tile_records_bytes(const tcl_plan *p, int n_mods);

// Bytes before the packed data of a module's packed copy of B: the adapters'
// first 16-byte units, then a zero 16-byte unit right before the data.
size_t tile_pack_head_bytes(const tcl_module *m);

// Bytes of a module's packed rank-contiguous copy of B (tcl_module_pack).
size_t tile_pack_bytes(const tcl_module *m);

// Enqueue the two kernels that write the packed copy of m->B_t into B_k
// (tile_pack_bytes(m) bytes, 256-byte aligned; checked by the caller).
int launch_module_pack(const tcl_module *m, void *B_k, hipStream_t s);

// A new adapter slot pool: every slot's rank 0 in k_dev, and (B_k non-NULL)
// the offsets of the packed copy fixed at s * d_out * ceil(r_max / 8) units
// (tile_pack_bytes(m) bytes, 256-byte aligned; checked by the caller).
int launch_slot_pool_init(const tcl_module *m, int32_t *k_dev, void *B_k, hipStream_t s);

// n loads into a slot pool whose factors are already in place: slot
// slots[i] gets rank ranks[i] in m->k_dev and, when m->B_k is set, its packed
// columns re-written.  Kernel arguments carry the lists (no device copies).
int launch_slot_update(const tcl_module *m, const int32_t *slots, const int32_t *ranks, int n,
                       hipStream_t s);

// tile_prep then expand_tile for n (<= kMaxMods) modules.  z[i]: module i's
// shrink output with zld[i] floats a row and nkc[i] K-chunk partial planes;
// rec: tile_records_bytes(p, n) bytes of workspace.
int launch_expand_tile(const tcl_plan *p, const tcl_module *mods, int n, float *const *z,
                       const int *zld, const int *nkc, void *const *y, const int64_t *ldy,
                       tcl_dtype yd, int32_t *rec, hipStream_t s);

}  // namespace tcl
