/*
 * lora.h -- C ABI of the MI355X (gfx950) unmerged multi-LoRA library.
 *
 * What the library computes.  "Serving several LoRAs, ControlNet and
 * IP-Adapter", section "LoRA: merged or alongside": a LoRA adds the low-rank
 * increment W' = W + BA with A of shape r x d and B of shape d x r, and the
 * unmerged form adds x A^T B^T to the base output x W^T in every adapted
 * layer.  Here A is r x d_in and B is d_out x r.  The same page, self-test
 * answer on mixing LoRAs and the "Exercises" answer on four requests: each
 * request names its own adapter; rows are partitioned by adapter, a single
 * kernel covers all partitions, and each result goes back to the row it came
 * from.  "Punica: Multi-Tenant LoRA Serving" (contribution 1) describes the
 * same scheme as segmented gather matrix-vector (SGMV) kernels for batches
 * that mix adapters.  With several LoRAs stacked, each one contributes its
 * own alongside product and the products add up (comparison table, stacking
 * row); a per-slot scale plays the part of the LoRA weight that diffusion
 * schedules vary over timesteps (same section, the paragraph on diffusion).
 *
 * For each request s, each row t of that request, and each slot k whose index
 * i = idx[s][k] is valid:
 *
 *     y[t][:] += scale[s][k] * (x[t][:] . A_i^T) . B_i^T
 *
 * accumulated in fp32 and rounded once (round-to-nearest-even) to y's type.
 * Rows whose request has no valid slot, and rows covered by no request, are
 * never written (their bits are left exactly as they were).
 *
 * Memory and ownership.  Every pointer in a struct or argument below is a
 * DEVICE pointer unless its comment says "host".  All buffers are allocated
 * and owned by the caller; the library allocates and frees nothing and is
 * re-entrant.  The only state it keeps between calls is looked up or created
 * once and never changes: each device's compute-unit count, the kernels' LDS
 * limit, the tuning values read from the environment at the first call, each
 * device's address of the fixed plan array that lora_apply_noalloc uses (a
 * static device array of the library, not an allocation), and, created at the
 * first multi-problem launch with prefill tiles on a device, one extra stream
 * and two events of that device (such launches run their decode tiles on it,
 * beside the prefill tiles, and the caller's stream waits for both; the
 * launch stays asynchronous and can be captured in a graph).  Every
 * compute call is asynchronous on the given stream and never synchronizes,
 * except lora_read_device_errors.
 * x and y must not overlap; v must overlap neither x nor y.
 *
 * Errors.  Problems visible on the host (NULL pointers, non-positive sizes,
 * unsupported rank or slot count, ld < d, a workspace that is too small,
 * overlapping x/y) return a status and launch nothing.  Adapter indices and
 * segment offsets live on the device and cannot be checked there: an index
 * below -1 or >= n_adapters is skipped as if it were -1, and decreasing or
 * out-of-range offsets are clamped into non-overlapping segments (segment s
 * becomes [max(seg_off[0..s]), max(seg_off[0..s+1])) clipped to [0, T]); both
 * are counted in a device error word read by lora_read_device_errors.
 */
#ifndef RANK_SGMV_BGMV_LORA_H
#define RANK_SGMV_BGMV_LORA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LORA_OK = 0,
  LORA_EINVAL = -1,       /* NULL pointer, overlapping buffers, bad enum */
  LORA_ESHAPE = -2,       /* non-positive size, ld < d, bad counts */
  LORA_EWORKSPACE = -3,   /* workspace missing or smaller than lora_workspace_size */
  LORA_EUNSUPPORTED = -4, /* rank, slot count or size beyond the limits below */
  LORA_EHIP = -5          /* a HIP runtime call (launch) failed */
} lora_status;

/* x, y, A and B share one element type.  The intermediate of lora_shrink /
 * lora_expand is always float32. */
typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

#define LORA_MAX_RANK 256        /* 1 <= rank <= 256 */
#define LORA_MAX_SLOTS 8         /* 1 <= max_slots <= 8 */
#define LORA_MAX_SLOT_RANK 1024  /* max_slots * rank <= 1024 */
#define LORA_MAX_SLICES 8        /* projections per group of lora_apply_sliced */

/* One adapted linear layer's resident, stacked adapter pool ("Serving several
 * LoRAs ...", section "Placement": every LoRA stays resident).
 *   A: [n_adapters][rank][d_in]   row-major, dtype
 *   B: [n_adapters][d_out][rank]  row-major, dtype
 *   ranks: DEVICE [n_adapters] int32, or NULL.  Adapters of different ranks
 *          in one pool ("LoRA: merged or alongside": r is usually 8 to 128)
 *          are stored at `rank`; adapter i uses rows j < ranks[i] of A_i and
 *          columns j < ranks[i] of B_i only (values are clamped to [1, rank]).
 *          What lies past an adapter's rank is not read when its rank is a
 *          multiple of 8 (bf16) or 4 (fp32); otherwise the rest of the last
 *          16-byte piece is read and multiplied by zero, so it must hold finite
 *          values.  NULL: every adapter has rank `rank`.                  */
typedef struct {
  const void *A;
  const void *B;
  int32_t n_adapters;
  int32_t rank;
  int32_t d_in;
  int32_t d_out;
  lora_dtype dtype;
  const int32_t *ranks;
} lora_pool;

/* The batch: which adapters apply to which rows.
 *   n_tokens   T, rows of x and y.
 *   n_segments S, number of requests; ignored when seg_off is NULL.
 *   seg_off    [S+1] int32, request s owns rows [seg_off[s], seg_off[s+1]);
 *              non-decreasing, 0 <= seg_off[0], seg_off[S] <= T.  Rows outside
 *              [seg_off[0], seg_off[S]) belong to no request.  NULL selects
 *              per-token mode: S = T and request s is row s (decode / BGMV).
 *   idx        [S][max_slots] int32 adapter indices; -1 = empty slot.
 *   max_slots  K, slots per request (stacked adapters are summed).
 *   scale      [S][max_slots] float32 per-slot scale, or NULL for 1.0.     */
typedef struct {
  int32_t n_tokens;
  int32_t n_segments;
  const int32_t *seg_off;
  const int32_t *idx;
  int32_t max_slots;
  const float *scale;
} lora_batch;

/* One problem of a lora_apply_multi launch: a pool and its activations.  The
 * array of these lives in DEVICE memory; all problems share the shape given
 * by the `shape` argument of lora_apply_multi.                           */
typedef struct {
  const void *A;   /* [n][rank][d_in]  */
  const void *B;   /* [n][d_out][rank] */
  const void *x;   /* [T][ldx] */
  void *y;         /* [T][ldy], updated in place */
  int64_t ldx;
  int64_t ldy;
} lora_problem;

/* Bytes of device workspace (the plan) for a batch and pool size.  The plan
 * holds the grouping of requests by adapter -- the partition of the batch by
 * LoRA index that "Serving several LoRAs, ControlNet and IP-Adapter",
 * "Exercises" (the four-request answer), computes before one kernel covers
 * every partition -- and it is stable across layers: build it once per batch
 * and reuse it for every adapted layer.  Host only (nothing is launched);
 * returns 0 when the batch description itself is invalid. */
size_t lora_workspace_size(const lora_batch *batch, int32_t n_adapters);

/* Build the plan for `batch` into `ws` on `stream`: sort requests by adapter
 * (the grouping of the "Exercises" answer), split groups into row tiles, and
 * record the device error word.  seg_off and idx must stay unchanged until
 * every call that uses the plan has run.  The plan depends on them (and on T,
 * S, K) only: scale is read by every call that uses the plan, so a per-step
 * scale schedule ("LoRA: merged or alongside", the paragraph on diffusion:
 * the LoRA's weight may change with the timestep) passes each step's scale
 * array with the same plan. */
lora_status lora_plan_build(const lora_batch *batch, int32_t n_adapters, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* Fused apply ("Serving several LoRAs, ControlNet and IP-Adapter", section
 * "LoRA: merged or alongside": the unmerged form adds x A^T B^T to the base
 * output; "Exercises": rows grouped by adapter, one kernel for every group,
 * results back in their rows; comparison table, stacking row: stacked LoRAs
 * each add their own product): y += sum_k scale * (x A_i^T) B_i^T for every
 * touched row.  Builds the plan into ws, then runs the fused kernels.
 *   x: [T][ldx] dtype, ldx >= d_in;  y: [T][ldy] dtype, ldy >= d_out.    */
lora_status lora_apply(const lora_pool *pool, const lora_batch *batch, const void *x, int64_t ldx, void *y,
                       int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream);

/* lora_apply for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels, with the plan built into a device array the
 * library holds for the life of the process instead of a caller workspace.
 * That array is LORA_NOALLOC_PLAN_BYTES (8 MiB) on every GPU the library runs
 * on; a batch whose plan needs more (lora_workspace_size) is refused with
 * LORA_EUNSUPPORTED before anything is launched (about 40 000 one-token
 * requests, or segmented batches of up to about 60 000 rows and a few
 * thousand requests, fit).  Nothing is allocated or freed, by the library or
 * any routine it calls.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's plan: calls that may overlap on one GPU (two streams,
 * or two host threads) race and must be ordered by the caller.  The stream
 * must belong to the current device.  Errors as for lora_apply; the device
 * error word is not readable for these calls. */
#define LORA_NOALLOC_PLAN_BYTES (8u << 20)
lora_status lora_apply_noalloc(const lora_pool *pool, const lora_batch *batch, const void *x, int64_t ldx, void *y,
                               int64_t ldy, hipStream_t stream);

/* Shrink half ("Serving several LoRAs, ControlNet and IP-Adapter", section
 * "LoRA: merged or alongside": the alongside form is two thin products, x A^T
 * from d_in down to rank r, then that times B^T back up to d_out -- this is
 * the first): v[t][k*rank + j] = scale[s][k] * sum_c x[t][c] A_i[j][c] for
 * every touched row t and slot k (zeros for a -1 slot of a touched row).
 * v: [T][ldv] float32, ldv >= max_slots*rank.  Rows that are not touched are
 * not written. */
lora_status lora_shrink(const lora_pool *pool, const lora_batch *batch, const void *x, int64_t ldx, float *v,
                        int64_t ldv, void *ws, size_t ws_bytes, hipStream_t stream);

/* Expand half (same section: the second thin product, rank r up to d_out,
 * added to the base output): y[t][o] += sum_{k valid} sum_j v[t][k*rank + j]
 * B_i[o][j] for every touched row (the scale is not applied again:
 * lora_shrink folded it in, so lora_expand(lora_shrink(x)) computes what
 * lora_apply does).  v is float32 [T][ldv], rows of untouched requests are
 * not read. */
lora_status lora_expand(const lora_pool *pool, const lora_batch *batch, const float *v, int64_t ldv, void *y,
                        int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream);

/* The same three operations on a plan built earlier by lora_plan_build for
 * this batch (plan_bytes as returned by lora_workspace_size): the grouping of
 * the "Exercises" answer done once per batch and reused by every adapted
 * layer.  A plan built for another batch shape or pool size is detected on
 * the device: the kernels then write nothing and count the call in the
 * plan's error word (lora_read_device_errors). */
lora_status lora_apply_planned(const lora_pool *pool, const lora_batch *batch, const void *plan, size_t plan_bytes,
                               const void *x, int64_t ldx, void *y, int64_t ldy, hipStream_t stream);
lora_status lora_shrink_planned(const lora_pool *pool, const lora_batch *batch, const void *plan, size_t plan_bytes,
                                const void *x, int64_t ldx, float *v, int64_t ldv, hipStream_t stream);
lora_status lora_expand_planned(const lora_pool *pool, const lora_batch *batch, const void *plan, size_t plan_bytes,
                                const float *v, int64_t ldv, void *y, int64_t ldy, hipStream_t stream);

/* Many adapted layers of one shape in ONE launch, sharing one plan ("Serving
 * several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
 * alongside": every adapted linear layer of the model -- its cost table
 * counts the attention projections of all 57 layers -- gets its own
 * alongside product for the same requests; "Exercises": one kernel for every
 * group).  For each of the n_problems entries of `problems` (a DEVICE array,
 * read by the kernels, so that a launch needs no host copy of it), the fused
 * apply with that problem's pool, x and y.  `shape` gives rank, d_in, d_out,
 * n_adapters, dtype and ranks (its A and B are ignored; its rank array, if
 * any, applies to every problem).  The library cannot check
 * the pointers inside the device array; they must satisfy the alignment and
 * ld rules of lora_apply for this shape (16-byte aligned, ld a multiple of 8
 * elements for bf16 or 4 for fp32, for the vectorised path) or the launch
 * uses the scalar path only when `problems_aligned` is 0. */
lora_status lora_apply_multi(const lora_pool *shape, const lora_batch *batch, const void *plan, size_t plan_bytes,
                             int32_t n_problems, const lora_problem *problems, int32_t problems_aligned,
                             hipStream_t stream);

/* Several projections that read the same input, in ONE launch ("Serving
 * several LoRAs, ControlNet and IP-Adapter", answers to the self-test, the
 * first: a LoRA attaches to attention's query, key, value and output
 * projections, sometimes to the MLP too -- query, key and value read one
 * input, as do an MLP's gate and up projections).
 *
 * `problems` (a DEVICE array of n_groups * n_slices entries) holds n_groups
 * groups of n_slices projections each: entry g * n_slices + p is projection
 * ("slice") p of group g, with its own pool, x and y.  Slice p's output width
 * is d_outs[p] (a HOST array of n_slices values, the same for every group);
 * every other size -- n_adapters, rank, d_in, dtype, ranks -- is the
 * `shape`'s (its A, B and d_out are ignored).  1 <= n_slices <= 8.
 *
 * Result: for every entry, exactly what lora_apply_multi would compute for it
 * (y += sum_k scale * (x A_i^T) B_i^T on that entry's x, pool and y).  Work is
 * ordered tile by tile across the slices of a group, so when the slices of a
 * group name the same x (the intended use) each row tile of x is read from
 * HBM once for all of them and reused from cache by the others.  The y arrays
 * of one group must not overlap each other (distinct outputs, or disjoint
 * column ranges of one fused output with a shared ldy).  Alignment, ld rules
 * and `problems_aligned` as for lora_apply_multi, with d_outs[p] in place of
 * d_out; errors: LORA_ESHAPE for n_groups < 0, n_slices outside 1..8 or a
 * d_outs value below 1, LORA_EINVAL for NULL arrays. */
lora_status lora_apply_sliced(const lora_pool *shape, const lora_batch *batch, const void *plan, size_t plan_bytes,
                              int32_t n_groups, int32_t n_slices, const int32_t *d_outs,
                              const lora_problem *problems, int32_t problems_aligned, hipStream_t stream);

/* Merge stacked adapters into a weight, or unmerge them, in place ("Serving
 * several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
 * alongside": the merged form adds BA into W ahead of time; stacked LoRAs
 * merge as a weighted sum, comparison table, stacking row; switching
 * unmerges the old adapter and merges the new one):
 *
 *     W[o][c] += alpha * sum_k scale[k] * sum_j B_{idx[k]}[o][j] * A_{idx[k]}[j][c]
 *
 * for every o < d_out and c < d_in, accumulated in fp32 and rounded once
 * (round-to-nearest-even) to W's type.  alpha = 1 merges, alpha = -1
 * unmerges; in bf16 a merge followed by an unmerge returns W up to one
 * rounding of each step.
 *   idx    HOST [n_slots] adapter indices, 1 <= n_slots <= LORA_MAX_SLOTS;
 *          -1 skips the slot, any other value outside [0, n_adapters) is
 *          rejected (LORA_EINVAL) and nothing is launched.
 *   scale  HOST [n_slots] per-slot weights, or NULL for 1.0.
 *   W      DEVICE [d_out][ldw], the pool's dtype, ldw >= d_in; must not
 *          overlap the pool.
 * Asynchronous on `stream`; allocates nothing.  Every element of W is read
 * and written once: the bound is 2 * d_out * d_in * sizeof(element) bytes of
 * HBM traffic. */
lora_status lora_merge(const lora_pool *pool, const int32_t *idx, const float *scale, int32_t n_slots, float alpha,
                       void *W, int64_t ldw, hipStream_t stream);

/* One weight of a lora_merge_multi launch: its adapter pool (same shape for
 * every problem) and the weight.  The array of these lives in DEVICE memory. */
typedef struct {
  const void *A;  /* [n][rank][d_in]  */
  const void *B;  /* [n][d_out][rank] */
  void *W;        /* [d_out][ldw], updated in place */
  int64_t ldw;
} lora_merge_problem;

/* lora_merge for n_problems weights of one shape in ONE launch (same section:
 * merging touches every affected weight of the model, the page's cost model
 * counts all of them): for each entry of `problems` (a DEVICE array),
 * W += alpha * sum_k scale[k] B_i A_i
 * with i = idx[k] taken from that entry's pool.  `shape` gives rank, d_in,
 * d_out, n_adapters, dtype and ranks (its A and B are ignored; its rank
 * array, if any, applies to every problem); idx and scale are
 * HOST arrays as for lora_merge and apply to every problem.  The library
 * cannot check the pointers inside the device array: the weights must not
 * overlap one another or any pool, ldw >= d_in, and the matrix-core path
 * (bf16) is taken only when `problems_aligned` is 1, which promises 16-byte
 * aligned A, B and W and ldw a multiple of 8. */
lora_status lora_merge_multi(const lora_pool *shape, const int32_t *idx, const float *scale, int32_t n_slots,
                             float alpha, int32_t n_problems, const lora_merge_problem *problems,
                             int32_t problems_aligned, hipStream_t stream);

/* Copy one adapter from host memory into slot `slot` of a resident pool
 * ("Serving several LoRAs, ControlNet and IP-Adapter", section "Placement":
 * LoRAs stay resident; what does not stay resident is moved from page-locked
 * host memory on demand, at PCIe speed).
 *   A_host  HOST [rank][d_in], B_host HOST [d_out][rank], the pool's dtype,
 *           contiguous.  Page-locked memory (hipHostMalloc, or a torch tensor
 *           with pin_memory) makes the copy asynchronous on `stream`;
 *           pageable memory is copied too, but the call may return only after
 *           the host side has been read.
 *   slot    0 <= slot < n_adapters.  The pool's A and B name device memory the
 *           caller owns and allows to be written.
 * Calls that read the slot must be ordered after the copy (the same stream,
 * or an event recorded after it): a copy on a second stream then overlaps
 * with applies that use other slots.  Allocates nothing. */
lora_status lora_pool_load(const lora_pool *pool, int32_t slot, const void *A_host, const void *B_host,
                           hipStream_t stream);

/* Not an operation of the method: the pages define no error reporting.  It
 * reads what the device could not check on the host -- the adapter indices
 * below -1 or >= n_adapters that the last plan build skipped, the segment
 * offsets it clamped, and one for every apply launch that found the plan not
 * matching its call (another batch shape or pool size, or no plan at all) and
 * did nothing.  Synchronizes `stream` (the only call that does) and stores the
 * count in *count (a HOST pointer); the return value is the call's own status
 * (LORA_EINVAL for NULL arguments, LORA_EWORKSPACE for a plan_bytes too small
 * to hold the header, LORA_EHIP if the copy or the synchronization fails). */
lora_status lora_read_device_errors(const void *plan, size_t plan_bytes, int32_t *count, hipStream_t stream);

/* Static, human-readable text for a status (not an operation of the method). */
const char *lora_status_string(lora_status status);

/* ABI version of this header (major * 100 + minor; not an operation of the method). */
int32_t lora_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RANK_SGMV_BGMV_LORA_H */
