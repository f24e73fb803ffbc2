/*
 * tcl.h -- C ABI of the batched composite multi-LoRA apply for MI355X (gfx950).
 *
 * What the library computes (pages cited by title and section):
 *
 *   DyMerge-LoRA, section 3.1 (M1): a composite update is the weighted sum of
 *   low-rank adapter updates, Delta W = sum_i alpha_i B_i A_i^T.  Evaluating it
 *   after the merge point (DyMerge-LoRA, one-minute summary: on-GPU post-merge
 *   fusion) gives, for every token t with composite C_t = {(i, alpha)},
 *
 *       y_t = y_t + sum_{(i, alpha) in C_t} alpha * B_i (A_i^T x_t)
 *
 *   with A_i of size d_in x r and B_i of size d_out x r.  ELORA (section III-A,
 *   Eq. 1) is the one-adapter case with alpha = 1.
 *
 *   LoRAForge, approach (1): retained-rank contract.  Each adapter of a module
 *   keeps an ordered factor prefix and an effective rank k (0 <= k <= r_max);
 *   only the first k rank directions are read and used.  Stores padded to
 *   r_max are accepted; rows at and beyond k are never read.
 *
 *   DyMerge-LoRA, section 4.3: the mapping stage turns token-adapter pairs
 *   into tuples and reorders them by adapter (LoRA) id so that one adapter's
 *   tokens are contiguous; aggregation then sums each token's pairs.
 *   LoRAForge, approach (4)/(5): shrink (A_i^T x) and expand (B_i z) kernels,
 *   chosen by phase, rank and shape.
 *
 * Conventions
 *   - Adapter pools are rank-major: A_t[a][j][0..d_in) is row j of A_a^T and
 *     B_t[a][j][0..d_out) is row j of B_a^T, a in [0, n_adapters),
 *     j in [0, r_max).  The retained prefix of adapter a is rows 0..k_a-1.
 *   - Tuples are (token, adapter, alpha, slot).  The slot of a pair is its
 *     position in its composite after the composite is ordered by adapter id.
 *     The plan lists tuples in ascending (adapter, token, slot) order.
 *   - Each output element y[t][n] is produced by one thread which sums its
 *     token's pairs in slot order in fp32 (alpha * z_j * B[j][n], j ascending)
 *     and adds the result to y once.  No atomics; results are bitwise
 *     reproducible run to run.
 *   - dtypes: TCL_BF16 mode = bf16 x / A_t / B_t with fp32 or bf16 y;
 *     TCL_F32 mode = fp32 everywhere.  z and accumulation are fp32.
 *   - Device pointers are caller-owned (e.g. allocated by PyTorch) and must be
 *     16-byte aligned; d_in, d_out and leading dimensions must be multiples of
 *     8 elements.  Host pointers are only read during the call.
 *   - Every GPU call is asynchronous on the caller's stream (a hipStream_t
 *     passed as void*, NULL = the default stream).  Only tcl_plan_copy_out and
 *     tcl_plan_status (they read plan data back to the host) and
 *     tcl_module_init / tcl_module_load_ranks (their host ranks may be freed
 *     on return) synchronise.
 *   - Every function returns a status code (TCL_OK = 0 or a negative TCL_E*).
 *     Host-side checks run before any HIP call, so they need no GPU.  The
 *     message of the last failure on the calling thread is tcl_last_error().
 *     The library never aborts and prints only when TCL_LOG is set.
 */
#ifndef TCL_H
#define TCL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TCL_OK = 0,
  TCL_EINVAL = -1,       /* bad argument or malformed composite table        */
  TCL_EALIGN = -2,       /* pointer not 16-B aligned, size not multiple of 8 */
  TCL_ENOSPC = -3,       /* buffer or capacity too small                     */
  TCL_EUNSUPPORTED = -4, /* dtype combination, rank or group size not built  */
  TCL_EHIP = -5          /* a HIP runtime call failed                        */
};

typedef enum { TCL_BF16 = 0, TCL_F32 = 1 } tcl_dtype;

/* Largest r_max the kernels are built for, and the most pairs one
 * composite (group) may hold. */
#define TCL_MAX_RANK 64
#define TCL_MAX_PAIRS_PER_GROUP 64

/*
 * Composite table (DyMerge-LoRA section 3.1: static composition fixes alpha per
 * request, dynamic composition per token).  A group is a run of consecutive
 * tokens sharing one list of (adapter, alpha) pairs; one group per token is
 * token-level (dynamic) composition.  For tcl_plan_map, tcl_plan_remap and
 * the step calls every array is DEVICE memory, so that a gate running on the
 * GPU can feed the plan directly; tcl_plan_map_host and tcl_plan_remap_host
 * take the same struct with HOST arrays.
 *
 *   group_tok_ptr [n_groups+1]: group g covers tokens [ptr[g], ptr[g+1]);
 *                               ptr[0] = 0, non-decreasing, ptr[G] = n_tokens.
 *   group_pair_ptr[n_groups+1]: group g owns pairs [ptr[g], ptr[g+1]);
 *                               ptr[0] = 0, non-decreasing, ptr[G] <= n_pairs.
 *   pair_adapter [n_pairs]    : adapter id in [0, n_adapters), no id twice in
 *                               one group.
 *   pair_alpha   [n_pairs]    : finite fp32 weight (copied bit for bit).
 *   n_pairs is the length of the two pair arrays.  The table's pairs are
 *   those below group_pair_ptr[G]; entries at or beyond it are unused
 *   capacity and are never read (a gate on the GPU writes variable-length
 *   pair lists into arrays sized for the largest; DyMerge-LoRA one-minute
 *   summary, padding and masking).
 *   max_tuples                : capacity for P = sum_g tokens_g * pairs_g.
 *
 * A device-resident table is validated on the device by the mapping stage;
 * a bad table leaves an error in the plan's device status (read it with
 * tcl_plan_status, which synchronises, or tcl_plan_status_async, which does
 * not) and every later apply call on that plan changes nothing.  A
 * host-resident table is validated on the host, before any HIP call, and a
 * bad one is refused with its code.
 */
typedef struct {
  int32_t n_tokens;
  int32_t n_groups;
  int32_t n_pairs;
  int32_t n_adapters;
  int32_t max_tuples;
  const int32_t *group_tok_ptr;
  const int32_t *group_pair_ptr;
  const int32_t *pair_adapter;
  const float *pair_alpha;
} tcl_composites;

/*
 * One projection's adapter pool (the loader output of the LoRAForge
 * retained-rank contract).  k_dev is DEVICE int32 [n_adapters] of effective
 * ranks in [0, r_max], or NULL for "every adapter uses r_max"; fill it with
 * tcl_module_init (or tcl_module_load_ranks).
 *
 * B_k is an optional DEVICE rank-contiguous copy of B for the prefill expand
 * on the matrix cores (tcl_module_pack_bytes bytes): a header of int32
 * first-unit offsets per adapter and one zero 16-byte unit, padded to 256
 * bytes, then per adapter a [d_out][ceil(k_a / 8)] array of 16-byte units,
 * unit (n, o) holding ranks 8o .. 8o + 7 of column n of B_a^T as bf16 (zero
 * at and beyond k_a).  Fill it with tcl_module_pack after the ranks are
 * loaded (and again whenever B_t or the ranks change), or with
 * tcl_bam_pool_init / tcl_bam_load for a slot pool.  NULL: the prefill
 * expand runs on the per-token kernel over B_t.
 */
typedef struct {
  int32_t n_adapters;
  int32_t d_in;
  int32_t d_out;
  int32_t r_max;       /* 1..TCL_MAX_RANK */
  tcl_dtype wdtype;    /* dtype of A_t and B_t */
  const void *A_t;     /* device [n_adapters][r_max][d_in]  */
  const void *B_t;     /* device [n_adapters][r_max][d_out] */
  const int32_t *k_dev;
  const void *B_k;     /* device [n_adapters][d_out][r_pad] or NULL */
} tcl_module;

typedef struct tcl_plan tcl_plan; /* opaque host handle; device arrays live in
                                     the caller's plan buffer */

/* Message of the last non-OK return on the calling thread ("" if none). */
const char *tcl_last_error(void);

/* Library version string. */
const char *tcl_version(void);

/*
 * Device bytes a plan buffer needs for these sizes (host only, no GPU).
 * Errors: TCL_EINVAL for negative sizes, n_adapters < 1, or a count that
 * overflows 32-bit indexing.
 */
int tcl_plan_bytes(int32_t n_tokens, int32_t n_groups, int32_t n_pairs,
                   int32_t n_adapters, int32_t max_tuples, size_t *bytes);

/*
 * Mapping stage (DyMerge-LoRA section 4.3).  Validates the composite table,
 * orders each composite by adapter id (which fixes the slots), expands the
 * groups into tuples and stably counting-sorts them by adapter id, then
 * builds the segment table (one run per adapter that has tuples, ascending),
 * the per-token tuple index and the work lists of the apply kernels.
 *
 * dev_buf: caller-owned device buffer of at least tcl_plan_bytes() bytes,
 * 256-B aligned; it holds every device array of the plan and must outlive it.
 * *out receives a new host handle (free with tcl_plan_free).  One plan serves
 * every module and layer of the batch.  Asynchronous on `stream`.
 * Host errors: TCL_EINVAL (null pointer, sizes), TCL_EALIGN (dev_buf),
 * TCL_ENOSPC (dev_bytes too small), TCL_EHIP.
 * Device-detected errors (reported by tcl_plan_status): TCL_EINVAL (malformed
 * CSR, adapter id out of range, non-finite alpha, duplicate adapter in a
 * group), TCL_EUNSUPPORTED (a group with more than TCL_MAX_PAIRS_PER_GROUP
 * pairs), TCL_ENOSPC (more tuples than max_tuples), in that precedence.
 */
int tcl_plan_map(const tcl_composites *c, void *dev_buf, size_t dev_bytes,
                 void *stream, tcl_plan **out);

/* Re-run the mapping stage of an existing plan with a new table of the same
 * or smaller sizes (no host allocation).  Same errors as tcl_plan_map. */
int tcl_plan_remap(tcl_plan *p, const tcl_composites *c, void *stream);

/* Synchronises `stream` and returns the device-detected status of the plan
 * (TCL_OK or a code listed under tcl_plan_map), with its tuple and segment
 * counts (either pointer may be NULL). */
int tcl_plan_status(const tcl_plan *p, void *stream, int32_t *n_tuples,
                    int32_t *n_segments);

/*
 * Copies the plan to host arrays (synchronises `stream`).  Capacities: the
 * tuple arrays and tok_tuple hold max_tuples entries, seg_adapter n_adapters,
 * seg_begin n_adapters+1, tok_ptr n_tokens+1; only the first P (tuples), U
 * (segments) entries are meaningful.  Any pointer may be NULL to skip it.
 */
int tcl_plan_copy_out(const tcl_plan *p, int32_t *tup_token, int32_t *tup_adapter,
                      float *tup_alpha, int32_t *tup_slot, int32_t *seg_adapter,
                      int32_t *seg_begin, int32_t *tok_ptr, int32_t *tok_tuple,
                      void *stream);

void tcl_plan_free(tcl_plan *p);

/*
 * Host-resident composite tables.  The same tcl_composites, with every
 * array in HOST memory.  The table is validated on the host before any HIP
 * call, by the rules the mapping stage applies on the device and with the
 * same codes and precedence: TCL_EINVAL (CSR pointers that do not start at
 * 0, do not end at n_tokens, end beyond n_pairs or decrease; among the
 * table's pairs, an adapter id outside [0, n_adapters) or a non-finite
 * alpha; an adapter twice in one composite of
 * at most TCL_MAX_PAIRS_PER_GROUP pairs) before TCL_EUNSUPPORTED (a larger
 * composite) before TCL_ENOSPC (more tuples than max_tuples).
 *
 * tcl_composites_validate: that check alone (host only, no GPU); on success
 * *n_tuples = the tuple count P and *n_segments = the adapters that own at
 * least one tuple (either pointer may be NULL).
 *
 * tcl_plan_map_host / tcl_plan_remap_host: the check, then the table is
 * copied into the plan buffer (tcl_plan_bytes includes room for it) through
 * a pinned staging buffer the plan owns, and the mapping stage runs on the
 * device copy exactly as tcl_plan_map / tcl_plan_remap do.  The caller's
 * arrays may be freed or reused as soon as the call returns.  A rejected
 * table returns its code and queues nothing (the plan of a failed remap is
 * unchanged).  The copy reads the table when called, so these calls must not
 * be captured into a graph (TCL_EUNSUPPORTED on a capturing stream); a later
 * host remap waits for the previous one's copy to finish before reusing the
 * staging buffer.
 */
int tcl_composites_validate(const tcl_composites *c, int32_t *n_tuples, int32_t *n_segments);
int tcl_plan_map_host(const tcl_composites *c, void *dev_buf, size_t dev_bytes, void *stream,
                      tcl_plan **out);
int tcl_plan_remap_host(tcl_plan *p, const tcl_composites *c, void *stream);

/*
 * Tuple and segment counts of a plan whose last table was host-resident
 * (known on the host from the validation; no GPU call).  TCL_EUNSUPPORTED
 * for a plan mapped from a device-resident table: its counts live on the
 * device (tcl_plan_status, tcl_plan_status_async).
 */
int tcl_plan_info(const tcl_plan *p, int32_t *n_tuples, int32_t *n_segments);

/*
 * The plan's device verdict without a host synchronisation: queues on
 * `stream` a copy of {status code, tuples, segments, work items} into the
 * caller's device array dev_status[4] (int32, 4-byte aligned).  Queued after
 * a mapping call (or a step, which maps first) on the same stream it reads
 * that mapping's verdict: TCL_OK, or the code listed under tcl_plan_map for a
 * rejected table, whose apply calls change nothing.  Graph-capturable.
 */
int tcl_plan_status_async(const tcl_plan *p, int32_t *dev_status, void *stream);

/*
 * Loader step of the retained-rank contract (LoRAForge approach (1)): checks
 * host ranks k_host[n_adapters] in [0, r_max] and copies them to the device
 * array k_dev (caller-owned, n_adapters int32), then sets m->k_dev = k_dev.
 * Errors: TCL_EINVAL (null, rank out of range), TCL_EHIP.
 */
int tcl_module_load_ranks(tcl_module *m, const int32_t *k_host, int32_t *k_dev,
                          void *stream);

/*
 * Module set-up: validates the whole module (sizes, r_max in
 * 1..TCL_MAX_RANK, weight dtype, d_in and d_out multiples of 8, 16-byte
 * aligned A_t and B_t) and, when k_host is given, its ranks as
 * tcl_module_load_ranks does (k_host[n_adapters] in [0, r_max], copied to
 * the caller's device array k_dev, then m->k_dev = k_dev; synchronises the
 * stream so that k_host may be freed on return).  k_host NULL sets
 * m->k_dev = NULL (every adapter at r_max).  All checks run before any HIP
 * call.  Errors: TCL_EINVAL, TCL_EALIGN, TCL_EUNSUPPORTED, TCL_EHIP.
 */
int tcl_module_init(tcl_module *m, const int32_t *k_host, int32_t *k_dev, void *stream);

/*
 * The rank-contiguous copy B_k of a bf16 module's B_t (see tcl_module),
 * written on `stream` from B_t and the module's ranks (m->k_dev, or r_max for
 * every adapter when NULL); then m->B_k = B_k.  Rows of B_t at or beyond an
 * adapter's rank are not read.  B_k: caller-owned device memory of at least
 * tcl_module_pack_bytes bytes, 256-byte aligned.  The pack reads the ranks
 * queued before it on the stream; re-pack after new ranks or new factors.
 * Errors: those of tcl_module_init's module checks; TCL_EUNSUPPORTED (fp32
 * pool), TCL_EINVAL (B_k NULL), TCL_EALIGN, TCL_ENOSPC (bytes too small),
 * TCL_EHIP.
 */
int tcl_module_pack_bytes(const tcl_module *m, size_t *bytes);
int tcl_module_pack(tcl_module *m, void *B_k, size_t bytes, void *stream);

/* Device workspace tcl_fused_apply needs for these modules (host only). */
int tcl_workspace_bytes(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                        size_t *bytes);

/*
 * Shrink (LoRAForge approach (4)): z[p][j] = sum_d A_t[a_p][j][d] * x[t_p][d]
 * for j < k_{a_p}, zero for k_{a_p} <= j < r_max, for every tuple p in the
 * plan's sorted order.  alpha is not applied.  x: device [n_tokens][ldx] of
 * dtype xd (= module dtype).  z: device fp32 [max_tuples][r_max].
 * Errors: TCL_EINVAL, TCL_EALIGN, TCL_EUNSUPPORTED, TCL_EHIP.
 */
int tcl_shrink(const tcl_plan *p, const tcl_module *m, const void *x, int64_t ldx,
               tcl_dtype xd, float *z, void *stream);

/*
 * Expand and aggregate (LoRAForge approach (4), RowExpand; DyMerge-LoRA
 * aggregation stage): y[t][n] += sum over token t's slots s, in order, of
 * alpha_s * sum_{j < k} B_t[a_s][j][n] * z[p_s][j].  z is the tcl_shrink
 * layout.  y: device [n_tokens][ldy] of dtype yd, updated in place; tokens
 * with an empty composite are not written.
 */
int tcl_expand(const tcl_plan *p, const tcl_module *m, const float *z, void *y,
               int64_t ldy, tcl_dtype yd, void *stream);

/*
 * Shrink + expand for n_mods modules that share the plan (e.g. the seven
 * projections of a transformer layer), each with its own x[i] (leading
 * dimension ldx[i]) and y[i] (ldy[i]).  ws: device workspace of at least
 * tcl_workspace_bytes() bytes, 256-B aligned.  Same arithmetic as tcl_shrink
 * followed by tcl_expand, except that the shrink may split d_in into chunks
 * whose partial sums the expand adds in a fixed order.
 */
int tcl_fused_apply(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                    const void *const *x, const int64_t *ldx, tcl_dtype xd,
                    void *const *y, const int64_t *ldy, tcl_dtype yd, void *ws,
                    size_t ws_bytes, void *stream);

/*
 * Allocation-free tcl_fused_apply, for callers that cannot allocate device
 * memory (code under stream or graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, arithmetic and errors as
 * tcl_fused_apply, without ws / ws_bytes: the workspace is a static device
 * array of TCL_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; its device address is looked up on the first call
 * on a device, with that device current.  No call allocates or frees.
 * Batches whose workspace (tcl_workspace_bytes) exceeds TCL_SCRATCH_BYTES
 * return TCL_ENOSPC before any launch.  Every call on one GPU shares that
 * GPU's array: calls that may overlap on one GPU (different streams, or
 * graphs replayed concurrently) race and must be ordered by the caller.
 */
#define TCL_SCRATCH_BYTES (32u << 20)
int tcl_fused_apply_noalloc(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                            const void *const *x, const int64_t *ldx, tcl_dtype xd,
                            void *const *y, const int64_t *ldy, tcl_dtype yd, void *stream);

/*
 * The two halves of tcl_fused_apply, for callers that schedule them apart
 * (e.g. to overlap the expand with other work) and for per-kernel timing:
 * tcl_fused_shrink launches the multi-module shrink and leaves z in `ws`
 * (tcl_workspace_bytes); tcl_fused_expand reads z from `ws` and updates y.
 * Called back to back on one stream with the same plan, modules and
 * workspace they compute exactly what tcl_fused_apply computes.  Each is one
 * kernel launch for up to 8 modules.  Same arguments and errors as
 * tcl_fused_apply.
 */
int tcl_fused_shrink(const tcl_plan *p, const tcl_module *mods, int32_t n_mods,
                     const void *const *x, const int64_t *ldx, tcl_dtype xd, void *ws,
                     size_t ws_bytes, void *stream);
int tcl_fused_expand(const tcl_plan *p, const tcl_module *mods, int32_t n_mods, void *ws,
                     size_t ws_bytes, void *const *y, const int64_t *ldy, tcl_dtype yd,
                     void *stream);

/*
 * One step: tcl_plan_remap(p, c) followed by tcl_fused_apply on the new plan,
 * with the same arguments, results and errors as those two calls (the
 * DyMerge-LoRA pipeline: the mapping stage, then the fused shrink and the
 * aggregation).  Every host check of both runs before anything is queued.
 * For tables of the one-workgroup mapping mode (every decode batch) and bf16
 * pools, the mapping stage runs inside the shrink launch: each shrink
 * workgroup maps the table in its own LDS and keeps its work items there,
 * the first one also writes the plan out, so the step is two launches
 * (TCL_FUSED_MAPPING=0 in the environment turns that off).  Results are bit
 * for bit those of the separate calls.
 */
int tcl_remap_apply(tcl_plan *p, const tcl_composites *c, const tcl_module *mods,
                    int32_t n_mods, const void *const *x, const int64_t *ldx, tcl_dtype xd,
                    void *const *y, const int64_t *ldy, tcl_dtype yd, void *ws,
                    size_t ws_bytes, void *stream);

/*
 * The first half of tcl_remap_apply: tcl_plan_remap(p, c) and
 * tcl_fused_shrink, in one launch where tcl_remap_apply would use one.
 * tcl_fused_expand with the same plan, modules and workspace completes the
 * step.  Same arguments and errors as those calls.
 */
int tcl_remap_shrink(tcl_plan *p, const tcl_composites *c, const tcl_module *mods,
                     int32_t n_mods, const void *const *x, const int64_t *ldx, tcl_dtype xd,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Token-level gate: the composite table of dynamic composition from gate
 * logits, on the GPU (DyMerge-LoRA, section 3.1: under dynamic composition
 * alpha is computed per token; section 5.1, Sparse workload: a request
 * references 5-8 adapters and two are active per token; the one-minute
 * summary names padding and masking for the gate's vectorised form).
 *
 * Token t has n_candidates candidate adapters candidates[t * ld_candidates
 * + c] (an id < 0 is padding, not a candidate) with gate logits
 * logits[t * ld_logits + c], fp32, c in [0, n_candidates).  Its weights are
 * the softmax of the logits over the valid candidates, computed in fp32; the
 * k largest are kept, not renormalised, ties going to the smaller c (the
 * order of the logits, since the softmax is increasing).  A token keeps
 * k pairs, or all its valid candidates when it has fewer than k (none: an
 * empty composite, the token is left unchanged).  A token with a non-finite
 * valid logit gets k pairs of adapter -1 (weight 0): the mapping stage
 * rejects such a table with TCL_EINVAL.  Output, one group per token, device
 * arrays of the caller:
 *   group_tok_ptr[t] = t                       (n_tokens + 1 entries)
 *   group_pair_ptr[t] = pairs of tokens < t    (n_tokens + 1 entries)
 *   pair_adapter[group_pair_ptr[t] + i], pair_alpha[...], i below token t's
 *     count: its pairs, largest weight first   (n_tokens * k entries each;
 *     the entries at or beyond group_pair_ptr[n_tokens] are unused capacity,
 *     written as adapter -1 and weight 0)
 * Pass n_pairs = n_tokens * k to the mapping calls.  Three launches (counts,
 * their scan in one workgroup, the pairs).  Candidate ids are not range-checked here; the
 * mapping stage does that.  The table is ready for tcl_plan_map, tcl_plan_remap or
 * tcl_remap_apply without a trip through host memory.
 * Host checks: 1 <= n_candidates <= 64, 1 <= k <= n_candidates, k <=
 * TCL_MAX_PAIRS_PER_GROUP, leading dimensions >= n_candidates, n_tokens >= 0,
 * n_tokens * k < 2^31, every pointer 4-byte aligned and non-NULL (logits
 * and candidates may be NULL when n_tokens is 0).
 */
int tcl_gate_topk(const float *logits, int64_t ld_logits, const int32_t *candidates,
                  int64_t ld_candidates, int32_t n_tokens, int32_t n_candidates, int32_t k,
                  int32_t *group_tok_ptr, int32_t *group_pair_ptr, int32_t *pair_adapter,
                  float *pair_alpha, void *stream);

/* ------------------------------------------------------------------------
 * Retained-rank producer (LoRAForge, approach (2) rank allocation and
 * approach (3) factor construction; Figure 3 for the batched QR schedule).
 * ------------------------------------------------------------------------ */

/* Workspace (device bytes) that tcl_factor_balanced needs for a batch of
 * n_modules modules of shape (d_out, d_in) and rank `rank`.
 * Errors: TCL_EINVAL (NULL bytes, n_modules outside 0..65535, d_out < 2,
 * d_in < 8), TCL_EALIGN (d_out odd or d_in not a multiple of 8),
 * TCL_EUNSUPPORTED (rank outside 1..32). */
int tcl_factor_workspace_bytes(int32_t n_modules, int32_t d_out, int32_t d_in, int32_t rank,
                               size_t *bytes);

/* Balanced factors of a batch of LoRA modules, on the GPU.  Module m's
 * update is Delta W_m = B_m A_m^T with B_t[m] (rank x d_out, row j = column j
 * of B_m) and A_t[m] (rank x d_in, row j = column j of A_m), bf16, row-major
 * and contiguous: B_t[(m * rank + j) * d_out + i], A_t[(m * rank + j) * d_in
 * + i].  Following LoRAForge approach (3): a thin QR of B_m gives R, H = R
 * A_m^T, the eigendecomposition of H H^T gives the spectrum, and the
 * balanced factors F = Q U S^(1/2), T = S^(-1/2) U^T H are written in the
 * same layout as the inputs (device arrays of the caller, bf16):
 *   F_t[m] (rank x d_out): row j = column j of F, the new B_t rows;
 *   T[m]   (rank x d_in):  row j of T, the new A_t rows;
 *   sigma[m * rank + j] (fp32): singular values, largest first.
 * F T = Delta W, and the first k rows of F_t and T are the rank-k truncated
 * SVD of Delta W: the ordered prefix that the retained-rank contract of
 * approach (1) consumes.  Directions whose eigenvalue is at most 2^-23 of
 * the largest are returned as zero (sigma 0, zero rows).  The QR and the
 * Gram Y Y^T run in fp32 (bf16 products), the r x r eigenproblem in fp64.
 * ws: device workspace of at least tcl_factor_workspace_bytes bytes,
 * 16-byte aligned; its contents need no initialisation.  Asynchronous on
 * `stream`; n_modules == 0 is a no-op.
 * Errors: those of tcl_factor_workspace_bytes; TCL_EINVAL (a NULL pointer),
 * TCL_EALIGN (A_t or ws not 16-byte aligned, B_t, F_t, T or sigma not 4-byte
 * aligned), TCL_ENOSPC (ws_bytes too small), TCL_EHIP. */
int tcl_factor_balanced(const void *B_t, const void *A_t, int32_t n_modules, int32_t d_out,
                        int32_t d_in, int32_t rank, void *F_t, void *T, float *sigma, void *ws,
                        size_t ws_bytes, void *stream);

/* LoRAForge-U (LoRAForge, approach (2)), on the host: module m keeps
 * u_out[m] = max(1, floor(ranks[m] / denominator)) directions, and the
 * parameter budget is *budget_out = sum_m u_out[m] * costs[m], costs[m] =
 * d_in + d_out of the module.  Host arrays of n_modules entries.
 * Errors: TCL_EINVAL (NULL pointer, n_modules < 0, denominator < 1, a rank
 * < 0 or a cost < 1). */
int tcl_rank_uniform(const int32_t *ranks, const int64_t *costs, int32_t n_modules,
                     int32_t denominator, int32_t *u_out, int64_t *budget_out);

/* LoRAForge-S (LoRAForge, approach (2)), on the host: spend `budget`
 * parameters on the directions with the most spectral energy per parameter.
 * Module m has ranks[m] singular values sigma[m * ld_sigma + j], largest
 * first, and each kept direction costs costs[m] (= d_in + d_out).  Every
 * module first keeps min(floors[m], ranks[m]) directions; the remaining ones
 * are visited by decreasing eta = sigma^2 / cost (computed in fp64; equal
 * values in the order of module, then direction) and kept when the module's
 * previous direction is kept and the cost fits in what is left of the
 * budget.  k_out[m] receives the kept count (a prefix).  Host arrays.
 * Errors: TCL_EINVAL (NULL pointer, n_modules < 0, a rank < 0 or > ld_sigma,
 * a cost < 1, a floor < 0, a sigma that is negative or not finite). */
int tcl_rank_spectral(const double *sigma, int64_t ld_sigma, const int32_t *ranks,
                      const int64_t *costs, const int32_t *floors, int32_t n_modules,
                      int64_t budget, int32_t *k_out);

/* ------------------------------------------------------------------------
 * Adapter residency and batch choice, on the host (DyMerge-LoRA, section 4:
 * BAM and the LAG scheduler).
 * ------------------------------------------------------------------------ */

typedef struct tcl_bam tcl_bam;

/* A pool of n_slots adapter slots (BAM), all empty.  The caller owns the
 * GPU memory of the slots (for instance a [n_slots][r][d] pool per module)
 * and copies an adapter's factors into its slot when told to load it.
 * Errors: TCL_EINVAL (out NULL, n_slots < 1). */
int tcl_bam_create(int32_t n_slots, tcl_bam **out);
void tcl_bam_free(tcl_bam *bam);

/* Makes the adapters of one batch resident.  adapters[0..n) (ids >= 0,
 * repeats allowed) are the batch's adapters.  Its adapters already in a slot
 * are pinned for this call and their last use becomes now (one tick per
 * call); each missing adapter, in order of first appearance, takes the
 * lowest-numbered empty slot, else the slot used longest ago among those
 * not pinned by this batch (equal: the lower slot), and is pinned there.
 * Output: slot_of[i] = the slot of adapters[i]; load_slot / load_adapter /
 * load_evicted[0..*n_loads) = the loads the caller must perform, in order
 * (load_evicted -1 for an empty slot).  Host arrays of n entries each.
 * Errors: TCL_EINVAL (NULL pointer, n < 0, an id < 0), TCL_ENOSPC (more
 * distinct adapters than slots: nothing changes, *n_loads = 0; the tick
 * still advances). */
int tcl_bam_acquire(tcl_bam *bam, const int32_t *adapters, int32_t n, int32_t *slot_of,
                    int32_t *load_slot, int32_t *load_adapter, int32_t *load_evicted,
                    int32_t *n_loads);

/* The adapter in every slot (-1 when empty): n_slots entries. */
int tcl_bam_slots(const tcl_bam *bam, int32_t *slot_adapter);

/* The GPU half of the slot pool.  A slot pool is a tcl_module whose
 * n_adapters entries are slots: A_t [n_slots][r_max][d_in] and B_t
 * [n_slots][r_max][d_out] on the device, owned by the caller.
 *
 * tcl_bam_pool_init sets every slot empty (rank 0 in k_dev, caller-owned
 * device int[n_slots]) and, with B_k (bf16 pools; tcl_module_pack_bytes
 * bytes, 256-byte aligned), lays out the packed copy of B with a fixed
 * region per slot, so that a load re-packs only its slot; then m->k_dev =
 * k_dev and m->B_k = B_k.  Enqueued on `stream`.  Errors: those of
 * tcl_module_init's module checks; TCL_EINVAL (k_dev NULL), TCL_EALIGN,
 * TCL_EUNSUPPORTED (B_k with an fp32 pool), TCL_ENOSPC, TCL_EHIP.
 *
 * tcl_bam_load performs the loads tcl_bam_acquire returned (DyMerge-LoRA
 * section 4: BAM keeps the raw factors of resident adapters on the GPU):
 * for load i, rows j < k of adapter load_adapter[i] of the caller's host
 * pools A_host [n_logical][r_max][d_in] and B_host [n_logical][r_max][d_out]
 * (the module's dtype; pinned memory, e.g. hipHostMalloc, for the copies to
 * be asynchronous) go to slot load_slot[i], whose rank becomes k =
 * k_host[load_adapter[i]] (k_host NULL: r_max), and its packed columns are
 * re-written.  Rows at or beyond k are neither copied nor read later.  All
 * on `stream`: host-to-device copies, then one kernel per 64 loads.  The
 * host pools must stay unchanged until the copies have run.  Apply over the
 * pool with slot ids as adapter ids (tcl_bam_acquire's slot_of).  Checks,
 * all before any HIP call: the module is a slot pool (k_dev set), slots in
 * [0, n_slots) and distinct within the call, adapters in [0, n_logical),
 * ranks in [0, r_max].  Errors: TCL_EINVAL, TCL_EALIGN, TCL_EUNSUPPORTED,
 * TCL_EHIP. */
int tcl_bam_pool_init(tcl_module *m, int32_t *k_dev, void *B_k, size_t bytes, void *stream);
int tcl_bam_load(const tcl_module *m, const void *A_host, const void *B_host,
                 const int32_t *k_host, int32_t n_logical, int32_t n_loads,
                 const int32_t *load_slot, const int32_t *load_adapter, void *stream);

/* The next batch, chosen the LAG way.  Request i (of n_requests) arrived at
 * arrival[i] and uses the adapters req_adapters[req_ptr[i] .. req_ptr[i +
 * 1]) (ids >= 0, repeats count once).  resident[0..n_resident) are the
 * adapters now in slots.  A batch holds at most max_batch requests, and the
 * distinct adapters of its requests must fit in n_slots.  First the requests
 * with now - arrival > theta, by arrival (equal: lower index), each taken if
 * it still fits; then, while there is room, the request with the fewest
 * adapters neither resident nor already in the batch, among those that fit,
 * ties by arrival then index.  chosen[0..*n_chosen) receives the request
 * indices in the order taken (room for min(max_batch, n_requests)).
 * Errors: TCL_EINVAL (NULL pointer, negative sizes, req_ptr not starting at
 * 0 or decreasing, an id < 0, a NaN time). */
int tcl_lag_select(const double *arrival, const int32_t *req_ptr, const int32_t *req_adapters,
                   int32_t n_requests, const int32_t *resident, int32_t n_resident, double now,
                   double theta, int32_t max_batch, int32_t n_slots, int32_t *chosen,
                   int32_t *n_chosen);

#ifdef __cplusplus
}
#endif

#endif /* TCL_H */
