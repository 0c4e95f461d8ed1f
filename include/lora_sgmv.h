/*
 * lora_sgmv.h -- C ABI of the MI355X (gfx950) multi-adapter LoRA delta library.
 *
 * The library computes, for a heterogeneous batch of token rows in which each
 * contiguous segment of tokens names one adapter of an HBM-resident pool,
 *
 *     y[t, off_p : off_p + h_out_p] (+)= s_i * B_i,p (A_i,p x[t])       (*)
 *
 * where i is the adapter of the segment holding token t and p the adapted
 * projection.  Sources for the operation:
 *   - LoRA: the base weight stays frozen and two small trained matrices A and
 *     B carry the update ("TGI Multi-LoRA: Deploy Once, Serve 30 Models",
 *     section "Technical Foundation: Low-Rank Adaptation (LoRA)").
 *   - One request names one adapter, so one batch mixes adapters (same page,
 *     "How Multi-LoRA Serving Works"); grouping the requests that share an
 *     adapter is the segmented gather of SGMV ("Compress then Serve", the
 *     rebuttal paragraph on Punica).
 *   - The A step runs with scale 1.0 into a float32 buffer of shape
 *     (tokens, R); the B step applies the scale and updates a slice of y
 *     given by y_offset and y_slice_size ("Compress then Serve", rebuttal
 *     pseudocode of add_lora_slice_with_sigma, buffer creation and steps 1
 *     and 3).
 *   - Adapters of different ranks in one batch ("how does this differ from
 *     s-Lora?" issue thread: the multi-rank kernel and the rank caveats).
 *
 * Conventions shared by every entry point:
 *   - Matrices are row-major.  A_i,p is r_i x h_in_p and B_i,p is h_out_p x r_i.
 *   - The caller owns ALL device memory (the pool slab, activations, outputs,
 *     the intermediate v and the plan workspace).  The library never calls
 *     hipMalloc or hipFree.  It owns host metadata only, plus one pinned
 *     host staging buffer per plan.
 *   - Calls that take `stream` (a hipStream_t, passed as void*) only enqueue
 *     work on it and do not synchronise; results are valid in stream order.
 *   - Every argument is validated on the host before anything is enqueued.
 *     A status other than LORA_OK means nothing was enqueued and no library
 *     state changed; lora_last_error() then holds a message (thread-local).
 *   - Element type of x, y, base_out and pool weights is the pool's dtype
 *     (bf16 or f32).  v is always float32.  Device pointers must be 16-byte
 *     aligned and leading dimensions multiples of 16 bytes' worth of elements
 *     (8 for bf16, 4 for f32); h_in_p and h_out_p must be multiples of 8.
 *   - Arithmetic: products of inputs are formed exactly and summed in float32
 *     (the float32 intermediate of the pseudocode); y is rounded once, to
 *     nearest-even, to the output type.  Results are deterministic: the same
 *     call on the same inputs gives the same bits.
 *   - Thread safety: calls on different pools/plans are independent.  Pool
 *     mutation must not overlap launches that read the same slots, and one
 *     plan workspace must not be used by two streams at once.
 *   - Names follow the problem statement of the pages: a pool of adapters
 *     resident in HBM, per-segment adapter ids and offsets into the token
 *     rows, per-adapter rank and scale; the A step (shrink, input width to
 *     rank) and the B step (expand, rank to output width) of the pseudocode
 *     cited above.
 */
#ifndef LORA_SGMV_H
#define LORA_SGMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LORA_OK = 0,
    LORA_EINVAL = -1,  /* bad argument: null pointer, size, stride, alignment */
    LORA_ENOSPC = -2,  /* pool slab or slot table full */
    LORA_ENOENT = -3,  /* adapter id not registered */
    LORA_ERANK = -4,   /* rank < 1 or rank > r_max */
    LORA_EDTYPE = -5,  /* unsupported element type */
    LORA_ESEG = -6,    /* malformed segment table */
    LORA_EHIP = -7,    /* a HIP runtime call failed */
    LORA_EEXIST = -8,  /* adapter id already registered */
    LORA_ESTATE = -9   /* plan not uploaded, or its workspace is too small */
} lora_status;

typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

/* Core kinds of jointly compressed adapters ("Compress then Serve": JD-Diag
 * keeps a diagonal core per adapter, JD-Full a full one). */
typedef enum { LORA_SIGMA_DIAG = 1, LORA_SIGMA_FULL = 2 } lora_sigma_kind;

#define LORA_MAX_PROJ 8   /* adapted projections per pool (q, k, v, o, gate, up, down, ...) */
#define LORA_MAX_RANK 64  /* largest supported r_max */
#define LORA_MAX_MERGE 4  /* adapters merged per request (lora_plan_create_merge) */

/* Shape of a pool: every adapter carries A and B for each (layer, projection). */
typedef struct {
    int32_t num_layers;             /* L >= 1 */
    int32_t num_proj;               /* 1 .. LORA_MAX_PROJ */
    int32_t h_in[LORA_MAX_PROJ];    /* input width of projection p (multiple of 8) */
    int32_t h_out[LORA_MAX_PROJ];   /* output width of projection p (multiple of 8) */
    int32_t r_max;                  /* largest rank accepted; multiple of rank_granule, <= 64 */
    int32_t rank_granule;           /* ranks are zero-padded to a multiple of this (8 or 16) */
    int32_t max_slots;              /* most adapters resident at once */
    int32_t dtype;                  /* lora_dtype of weights, activations and outputs */
} lora_pool_desc;

typedef struct lora_pool lora_pool;
typedef struct lora_plan lora_plan;

/* Message for the last non-OK status returned on this thread. */
const char *lora_last_error(void);

/* ---------------------------------------------------------------- pool ---- */

/* Bytes of one adapter at its true rank: sum over layers and projections of
 * rank * (h_in + h_out) * element size -- the storage accounting behind the
 * adapter size the pages quote ("TGI Multi-LoRA: Deploy Once, Serve 30
 * Models", section "Technical Foundation": a 13.6 MB adapter beside a
 * 14.48 GB Mistral-7B base).  Which projections, rank and element size that
 * adapter has is not stated; 13,631,488 bytes is, for example, q and v at
 * rank 16 in 16-bit.  0 on a bad descriptor or rank < 1.  (The bytes an
 * adapter takes in the slab, with padding, are lora_pool_extent_bytes.) */
uint64_t lora_pool_bytes_for(const lora_pool_desc *d, int32_t rank);

/* Bytes one adapter occupies in the slab: the same sum at the padded rank
 * with h_in rounded up to whole K-blocks (32 bf16 / 16 f32 elements),
 * rounded up to 256 bytes.  0 on a bad descriptor or rank. */
uint64_t lora_pool_extent_bytes(const lora_pool_desc *d, int32_t rank);

/* Create a pool of HBM-resident adapters ("Compress then Serve", rebuttal
 * pseudocode: the stacked adapter weights every call indexes by adapter and
 * layer; "TGI Multi-LoRA", "How Multi-LoRA Serving Works": the adapters stay
 * loaded beside one base model) over a caller-owned device buffer `slab` of
 * `slab_bytes` (256-byte aligned).  Each adapter occupies one contiguous extent of the
 * slab; inside it, for layer l and projection p, the A block is followed by
 * the B block, layers outermost.  A is stored K-blocked,
 * [h_in_pad_p / S][r_pad][S] with S = 32 (bf16) or 16 (f32) and h_in_pad_p =
 * h_in_p rounded up to S, so that 16 rank rows x S columns are one
 * contiguous run.  B holds h_out_p rows of r_pad elements (nv = r_pad * e / 16
 * vectors of 16 bytes a row, e the element size) in row slices of 64 * rpl
 * rows, rpl = 1 when nv rounded up to a power of two is 8 or more, else 2
 * (the last slice shorter): in a slice of n rows from row `base`, vector v of
 * row base + rpl * l + i (i < rpl, l < n / rpl) is the slice's 16-byte vector
 * number (i * nv + v) * (n / rpl) + l, so that the rows a 64-lane wave
 * streams arrive as whole contiguous runs; the block is h_out_p * r_pad
 * elements, as row-major would be.  Pad rows and columns are zero.  The slab is not touched here and is not freed by lora_pool_destroy.
 * Errors: LORA_EINVAL (null pointer, bad descriptor or slab alignment),
 * LORA_EDTYPE. */
lora_status lora_pool_create(lora_pool **out, const lora_pool_desc *d,
                             void *slab, uint64_t slab_bytes);
lora_status lora_pool_destroy(lora_pool *p);

/* Reserve an extent and a slot for `adapter_id` (>= 0) at `rank` with scale
 * `scale` (the adapter's alpha / r).  The extent's contents are undefined
 * until uploaded.  Errors: LORA_EEXIST, LORA_ERANK, LORA_ENOSPC, LORA_EINVAL. */
lora_status lora_pool_reserve(lora_pool *p, int32_t adapter_id, int32_t rank, float scale);

/* Copy the weights of one (layer, proj) of a reserved adapter into its
 * extent, zero-filling the rank padding.  A: [rank][h_in_p], B: [h_out_p][rank],
 * both dense row-major in the pool dtype, in host memory (src_on_host = 1) or
 * device memory (0).  Enqueued on `stream`; host sources are copied before
 * the call returns. */
lora_status lora_pool_upload(lora_pool *p, int32_t adapter_id, int32_t layer, int32_t proj,
                             const void *A, const void *B, int32_t src_on_host, void *stream);

/* Register an adapter: reserve its slot and extent, then upload every
 * (layer, proj): A[p] -> [L][rank][h_in_p] and B[p] -> [L][h_out_p][rank]
 * (arrays of num_proj pointers), the two small matrices of a LoRA adapter
 * ("TGI Multi-LoRA", "Technical Foundation") under its id, the id a request
 * names ("How Multi-LoRA Serving Works").  On an upload error the
 * reservation is released again.  Errors as lora_pool_reserve and
 * lora_pool_upload. */
lora_status lora_pool_register(lora_pool *p, int32_t adapter_id, int32_t rank, float scale,
                               const void *const *A, const void *const *B,
                               int32_t src_on_host, void *stream);

/* Release an adapter's slot and extent (the offload of an adapter from GPU
 * memory, "Lorax" tool listing, "What is Lorax?").  Plans built before are
 * refused from then on (LORA_ESTATE).  The extent is free at once: the caller
 * must order this call, and any reuse of the extent (a later register or
 * image upload on any stream), after the last launch that reads the adapter,
 * e.g. by waiting for an event recorded after those launches.  (The exchange
 * cache below does this ordering itself.)  Errors: LORA_EINVAL, LORA_ENOENT. */
lora_status lora_pool_unregister(lora_pool *p, int32_t adapter_id);

/* Pack one adapter, on the host, into the byte image of its slab extent: the
 * layout described at lora_pool_create, pad rows, pad columns and the
 * 256-byte tail zero.  A[p] -> [L][rank][h_in_p] and B[p] -> [L][h_out_p][rank]
 * (arrays of num_proj host pointers, pool dtype); `image` (host, caller-owned)
 * holds at least lora_pool_extent_bytes(d, rank) bytes.  A packed image
 * reaches the device as one contiguous copy (lora_pool_upload_image), the
 * unit an adapter exchange moves.  No device call is made.
 * Errors: LORA_EINVAL (null pointers, image too small), LORA_ERANK. */
lora_status lora_pack_adapter(const lora_pool_desc *d, int32_t rank, const void *const *A,
                              const void *const *B, void *image, uint64_t image_bytes);

/* Copy a packed image into the extent of a reserved adapter: one copy of
 * lora_pool_extent_bytes(rank) bytes enqueued on `stream`, from host memory
 * (src_on_host = 1; pinned memory makes it asynchronous) or device memory
 * (0, 16-byte aligned).  The image must stay valid until the stream has
 * passed the copy.  Errors: LORA_EINVAL, LORA_ENOENT, LORA_EHIP. */
lora_status lora_pool_upload_image(lora_pool *p, int32_t adapter_id, const void *image,
                                   int32_t src_on_host, void *stream);

/* lora_pool_reserve, then lora_pool_upload_image; on an upload error the
 * reservation is released again. */
lora_status lora_pool_register_image(lora_pool *p, int32_t adapter_id, int32_t rank, float scale,
                                     const void *image, int32_t src_on_host, void *stream);

/* The descriptor the pool was created with. */
lora_status lora_pool_get_desc(const lora_pool *p, lora_pool_desc *d);

/* Where an adapter lives: rank, padded rank, scale and extent byte offset in
 * the slab (any output pointer may be NULL).  LORA_ENOENT if absent. */
lora_status lora_pool_query(const lora_pool *p, int32_t adapter_id, int32_t *rank,
                            int32_t *r_pad, float *scale, uint64_t *extent_offset);

/* Number of resident adapters and free slab bytes. */
lora_status lora_pool_stats(const lora_pool *p, int32_t *num_adapters, uint64_t *free_bytes);

/* ------------------------------------------------------------ exchange ---- */
/* Adapter exchange: a residency cache over a pool.  Adapters stay packed in
 * host memory (lora_pack_adapter images, caller-owned, pinned for overlap)
 * and are made resident on demand by one image copy each on a copy stream,
 * while earlier batches run on the compute stream; when the slab or the slot
 * table is full, the least recently used adapter that the outstanding batch
 * does not hold is evicted (its device copy dropped: adapters are read-only,
 * nothing moves back).  This is the asynchronous prefetch and offload of
 * adapters between CPU and GPU memory of the LoRAX pages ("Lorax" tool
 * listing, "What is Lorax?": adapter exchange scheduling; "predibase/lorax"
 * listing: adapter offloading, just-in-time weight loading; "how does this
 * differ from s-Lora?": adapters loaded asynchronously during inference).
 *
 * Use per batch: lora_cache_acquire(ids) -> lora_cache_prefetch(the next
 * batch's ids, when known) -> build the plan -> launch the batch's sgmv calls
 * on the compute stream -> lora_cache_release(compute stream).  Prefetching
 * before the launches lets the copies run under this batch's kernels; the
 * batch's own adapters are held and cannot be evicted by it.  Ordering is by
 * events, the host never waits:
 *   - acquire makes the compute stream wait for every copy enqueued so far;
 *   - a copy into an extent freed by an eviction waits for the release fence
 *     of the last batch that read the evicted adapter.
 * Evictions unregister adapters, so plans built before an acquire or a
 * prefetch that evicted must not be launched afterwards (the launch reports
 * LORA_ESTATE).  The cache manages only the adapters added to it; it is not
 * thread-safe and is not for use under graph capture.  An error from acquire
 * or prefetch may leave adapters it brought in resident (and not held); no
 * other state changes. */
typedef struct lora_cache lora_cache;

/* A cache over pool `p`, copying on `copy_stream` (a hipStream_t). */
lora_status lora_cache_create(lora_cache **out, lora_pool *p, void *copy_stream);

/* Frees the cache's host state and events; resident adapters stay in the
 * pool.  Call after the streams have passed the cache's work. */
lora_status lora_cache_destroy(lora_cache *c);

/* Adds a host-resident adapter: `image` is its packed extent image
 * (lora_pack_adapter at `rank`), kept valid by the caller while the cache
 * lives.  Errors: LORA_EINVAL, LORA_ERANK, LORA_EEXIST (added already, or
 * registered in the pool by other means). */
lora_status lora_cache_add(lora_cache *c, int32_t adapter_id, int32_t rank, float scale,
                           const void *image);

/* Makes the adapters `ids[0..n)` (-1 entries ignored, repeats allowed)
 * resident and holds them until lora_cache_release: misses are copied on the
 * copy stream in first-appearance order, evicting unheld adapters by least
 * recent use; `compute_stream` is made to wait for the copies.
 * *num_uploaded (may be NULL) = misses copied by this call.
 * Errors: LORA_ESTATE (a batch is outstanding), LORA_ENOENT (id not added),
 * LORA_ENOSPC (the batch's adapters do not fit the pool together, or the free
 * space around those already brought in is too fragmented), LORA_EHIP. */
lora_status lora_cache_acquire(lora_cache *c, int32_t n, const int32_t *ids, void *compute_stream,
                               int32_t *num_uploaded);

/* Ends the outstanding batch: records its fence on `compute_stream` (after
 * the batch's launches) and lets its adapters be evicted again.
 * Errors: LORA_ESTATE (no batch outstanding), LORA_EHIP. */
lora_status lora_cache_release(lora_cache *c, void *compute_stream);

/* Starts copies of the adapters of a coming batch (-1 ignored): each one not
 * resident is copied on the copy stream, evicting unheld adapters by least
 * recent use, until one does not fit (not an error).  Prefetched adapters
 * count as just used.  *num_uploaded (may be NULL) = copies started. */
lora_status lora_cache_prefetch(lora_cache *c, int32_t n, const int32_t *ids,
                                int32_t *num_uploaded);

/* Whether an added adapter is resident and whether the outstanding batch
 * holds it.  LORA_ENOENT if it was not added. */
lora_status lora_cache_query(const lora_cache *c, int32_t adapter_id, int32_t *resident,
                             int32_t *held);

/* Counters: resident adapters; ids found resident by acquire (hits) and
 * copied by it (misses); copies started by prefetch; evictions; bytes
 * copied in all.  Any output pointer may be NULL. */
lora_status lora_cache_stats(const lora_cache *c, int32_t *resident, uint64_t *hits,
                             uint64_t *misses, uint64_t *prefetched, uint64_t *evictions,
                             uint64_t *bytes_uploaded);

/* ---------------------------------------------------------------- plan ---- */

/* Build the gather plan of one heterogeneous batch (host memory inputs):
 * the tokens of a continuous batch, each request naming its adapter ("Lorax"
 * tool listing, "What is Lorax?": heterogeneous continuous batching; "TGI
 * Multi-LoRA", "How Multi-LoRA Serving Works"), grouped by adapter as SGMV
 * does ("Compress then Serve", rebuttal paragraph on Punica; the
 * pseudocode's `indices` name each token's adapter).
 *   num_tokens T >= 0; seg_starts[S+1] with seg_starts[0] = 0, non-decreasing,
 *   seg_starts[S] = T; seg_adapter[S] holds adapter ids, -1 = no adapter.
 *   Empty segments are allowed and ids may repeat.
 * Segments are grouped by adapter in first-appearance order (the segmented
 * gather), each group is cut into blocks (at most 16 tokens, or 64 for a
 * long group: see lora_plan_opts; a decode batch's blocks are cut again into
 * blocks of at most 4 tokens for the expand), and every id is resolved to
 * its slot, rank and scale.  The plan takes the pool's plan options.
 * Errors: LORA_ESEG, LORA_ENOENT.
 * The plan stays valid while its adapters stay registered. */
lora_status lora_plan_create(lora_plan **out, const lora_pool *p, int32_t num_tokens,
                             const int32_t *seg_starts, const int32_t *seg_adapter,
                             int32_t num_segs);

/* The same with a weight per segment: every call with this plan scales a
 * token's delta by its segment's weight (with the adapter's scale s: y = y_in
 * + (w * s) * B (A x), the product w * s rounded to float32 once): one
 * weighted adapter per request.  Errors as lora_plan_create, and LORA_EINVAL
 * for a weight that is not finite. */
lora_status lora_plan_create_weighted(lora_plan **out, const lora_pool *p, int32_t num_tokens,
                                      const int32_t *seg_starts, const int32_t *seg_adapter,
                                      const float *seg_weight, int32_t num_segs);

/* A weighted merge of several adapters per request ("predibase/lorax"
 * repository listing, feature list: adapters merged per request with
 * weighted merge strategies; "Lorax" tool listing, pros: per-request merges
 * into ensembles), read as the linear merge
 *     y = y_in + sum_k (w_k s_k) B_k (A_k x)
 * (the pages name no other strategy).  Segment s carries num_slots (K <=
 * LORA_MAX_MERGE) slots: adapter seg_adapters[s * K + k] (-1: an empty slot)
 * with weight seg_weights[s * K + k]; w_k s_k is rounded to float32 once.
 * sgmv_fused, sgmv_fused_static and the partials calls run it in one pass:
 * one shrink over every (token, slot) row, grouped by adapter, then one
 * expand that sums the K weighted deltas of each token in float32, slot by
 * slot in order, onto y_in, and rounds y once (y is read and written once).
 * A token whose slots are all empty keeps y_in.  The calls through a
 * caller's v (sgmv_shrink, sgmv_expand) and the core calls refuse a merge
 * plan (LORA_EINVAL), and so does lora_plan_export.  Errors as
 * lora_plan_create, and LORA_EINVAL for K out of range or a weight that is
 * not finite. */
lora_status lora_plan_create_merge(lora_plan **out, const lora_pool *p, int32_t num_tokens,
                                   const int32_t *seg_starts, int32_t num_segs, int32_t num_slots,
                                   const int32_t *seg_adapters, const float *seg_weights);

/* The same for jointly compressed adapters ("Compress then Serve", rebuttal
 * pseudocode of add_lora_slice_with_sigma): seg_adapter names the pool entry
 * that holds the segment's shared basis A, B (a cluster's), and
 * seg_sigma[S] its core: an index into the core table passed to the
 * *_sigma calls, or -1 for none (the identity: plain LoRA).  Segments of
 * different cores share one group when they share a basis.
 * Errors as lora_plan_create, and LORA_EINVAL for a core index < -1 (the
 * upper bound is checked by each call against its table). */
lora_status lora_plan_create_sigma(lora_plan **out, const lora_pool *p, int32_t num_tokens,
                                   const int32_t *seg_starts, const int32_t *seg_adapter,
                                   const int32_t *seg_sigma, int32_t num_segs);
/* Re-plan an existing plan for the next batch over the same pool: the
 * segment table as for the create calls, with optional per-segment cores
 * (seg_sigma, as lora_plan_create_sigma) or weights (seg_weight, as
 * lora_plan_create_weighted), NULL for none.  A serving loop plans every
 * step (the batch changes as requests come and go), so this reuses the
 * plan's host tables and pinned staging and allocates nothing on the device
 * or in pinned memory unless the batch is larger than any before.  The plan
 * must be uploaded again before its next call; an error leaves the plan as it
 * was.  The plan is made against the pool as it is at the rebuild, so a plan
 * that an unregister (or an exchange eviction) left stale is current again.
 * Each call fixes its launches from the plan as it then is (grids, unit
 * counts, and the kernel build chosen for the batch's blocks), so a HIP
 * graph captured from calls on the plan before a rebuild must not be
 * replayed after it: capture again, or call eagerly.
 * Errors as the create calls. */
lora_status lora_plan_rebuild(lora_plan *pl, int32_t num_tokens, const int32_t *seg_starts,
                              const int32_t *seg_adapter, const int32_t *seg_sigma,
                              const float *seg_weight, int32_t num_segs);

/* Frees the plan; waits for its last uploads to leave its staging buffers. */
lora_status lora_plan_destroy(lora_plan *pl);

/* Device bytes the plan needs: its tables and the per-call partial sums of
 * the shrink, sized for calls of up to `max_proj` projections at once.
 * 0 on error. */
uint64_t lora_plan_workspace_bytes(const lora_plan *pl, int32_t max_proj);

/* An upper bound of lora_plan_workspace_bytes for every plan over pool `p`
 * of at most num_tokens tokens and num_segs segments, built with the pool's
 * current plan options, for calls of up to `max_proj` projections: one
 * workspace of this size serves every batch of a serving loop, allocated
 * once.  (For a merge plan count a token per
 * (token, non-empty slot) and a segment per (segment, slot).)  0 on a bad
 * argument. */
uint64_t lora_workspace_bytes(const lora_pool *p, int32_t num_tokens, int32_t num_segs,
                              int32_t max_proj);

/* Copy the plan's tables into the caller-owned device workspace `ws`
 * (256-byte aligned, at least lora_plan_workspace_bytes(pl, max_proj)), on
 * `stream`, through pinned staging (two buffers used in turn: the host waits
 * only for the copy out of the buffer it reuses, that of the upload before
 * last).  Every sgmv call with this plan then uses `ws` (its tables, and
 * scratch for the shrink's partial sums); calls must be ordered after this
 * upload, and calls that share `ws` must not run concurrently.  A workspace
 * holds the tables of the plan uploaded into it last: a call with another
 * plan that was uploaded into it before is refused with LORA_ESTATE (upload
 * that plan again).  Errors: LORA_EINVAL (bad max_proj, null or misaligned
 * ws), LORA_ESTATE (ws_bytes too small), LORA_EHIP. */
lora_status lora_plan_upload(lora_plan *pl, void *ws, uint64_t ws_bytes, int32_t max_proj,
                             void *stream);

/* Tunables of the grouping and of the launch geometry, held by a pool.
 * SGMV groups a batch's requests by adapter ("Compress then Serve",
 * rebuttal paragraph on Punica); how a group is then cut and launched is a
 * GPU choice that these set.  A plan copies its pool's options when it is
 * built (created or rebuilt), so its tables, workspace size and launches
 * follow the options it was built with, whatever the pool holds later.
 *   long_group      a group of at least this many tokens is long: 64-token
 *                   blocks run by the one-launch prompt kernel ...
 *   long_batch      ... once the batch's long groups hold at least this many
 *                   tokens between them (otherwise every group takes the
 *                   decode cut: shrink blocks of 16 tokens, expand blocks of 4)
 *   shrink_groups   workgroups a decode shrink launch aims for: it sets the
 *                   launch's k-chunks (more chunks: more workgroups, more
 *                   partial sums for the expand to add)
 *   prefill_groups  workgroups a prompt launch aims for: a launch of fewer
 *                   16-token tiles splits each tile's output rows over up to
 *                   4 workgroups
 * Defaults (lora_plan_opts_default): 48, 1024, 128, 256, the values measured
 * best on MI355X for decode batches of 64-256 tokens and a 4096-token prompt
 * batch of Mistral-7B shapes. */
typedef struct lora_plan_opts {
    int32_t long_group;
    int32_t long_batch;
    int32_t shrink_groups;
    int32_t prefill_groups;
} lora_plan_opts;

/* Fills `o` with the defaults. */
void lora_plan_opts_default(lora_plan_opts *o);

/* Sets the options plans built from `p` afterwards take; lora_workspace_bytes
 * bounds workspaces for them.  Errors: LORA_EINVAL (null pointer, long_group
 * or long_batch < 1, shrink_groups or prefill_groups not in 1..65536); the
 * pool's options are then unchanged. */
lora_status lora_pool_set_plan_opts(lora_pool *p, const lora_plan_opts *o);

/* The pool's current options, and the options a plan was built with.
 * Errors: LORA_EINVAL (null pointer). */
lora_status lora_pool_get_plan_opts(const lora_pool *p, lora_plan_opts *o);
lora_status lora_plan_get_opts(const lora_plan *pl, lora_plan_opts *o);

/* Plan summary: groups, blocks, tokens with an adapter, largest block. */
lora_status lora_plan_stats(const lora_plan *pl, int32_t *num_groups, int32_t *num_blocks,
                            int32_t *num_active_tokens, int32_t *max_block_tokens);

/* Export the plan's gather tables (host arrays, any may be NULL):
 *   token_order[T]     token rows in plan order (grouped; no-adapter tokens last)
 *   token_group[T]     group index of each token row (-1 = no adapter)
 *   group_adapter[G]   adapter id of each group, first-appearance order
 *   group_rank[G]      its rank */
lora_status lora_plan_export(const lora_plan *pl, int32_t *token_order, int32_t *token_group,
                             int32_t *group_adapter, int32_t *group_rank);

/* ---------------------------------------------------------------- sgmv ---- */
/* The delta itself.  "Compress then Serve" (rebuttal pseudocode of
 * add_lora_slice_with_sigma, and of the BGMV dispatch it stands for) gives
 * the two steps these calls take: the A step at scale 1.0 into a float32
 * buffer of shape (tokens, R), then the B step with `scale` into the slice of
 * y at y_offset of width y_slice_size; here the tokens' adapters come from
 * the plan (the pseudocode's `indices`), the layer from `layer`, the scale
 * from each adapter's registration, and y_offset / y_slice_size from
 * y_offsets and each projection's h_out.  For all of them: `projs` lists `nproj` projection indices of the pool that
 * read the same input x (e.g. q, k, v), so x has width h_in of all of them
 * (they must agree).  For projection i of the list, its output is the
 * column slice y[:, y_offsets[i] : y_offsets[i] + h_out] (the pseudocode's
 * y_offset and y_slice_size), and its v columns are
 * v[:, i * r_max : i * r_max + r_max].  With num_tokens = 0 the calls
 * validate the pool, plan and projection list and do nothing else.
 * Every device tensor a call addresses (x, y, base, v) spans at most 2 GiB,
 * and so do the shrink's partial sums of one call (rank tiles x k-chunks x
 * projections x 1 KiB per 16-token tile): a larger call is refused with
 * LORA_EINVAL before anything is enqueued (split the batch).
 * Errors of every call: LORA_EINVAL (null or misaligned pointers, bad
 * layer, projections, strides or sizes), LORA_ESTATE (plan not uploaded,
 * built before an adapter was unregistered, or its workspace since given to
 * another plan), LORA_EHIP (a launch failed). */

/* Shrink (the A step, scale 1.0, "Compress then Serve", rebuttal pseudocode,
 * step 1): v[t][i*r_max + j] = sum_k A_i,p[j][k] x[t][k]
 * for every token with an adapter, j < r_max (columns j >= rank are zero).
 * Rows of tokens without an adapter are not written.
 * x: [T][ldx] device; v: [T][ldv] float32 device, ldv >= nproj * r_max. */
lora_status sgmv_shrink(const lora_pool *p, const lora_plan *pl, int32_t layer,
                        int32_t nproj, const int32_t *projs,
                        const void *x, int64_t ldx, float *v, int64_t ldv, void *stream);

/* Expand (the B step, "Compress then Serve", rebuttal pseudocode, step 3):
 * y[t][y_offsets[i] + o] += s_i * sum_j B_i,p[o][j] v[t][i*r_max + j]
 * for every token with an adapter, computed in float32 from the current y
 * and rounded once.  Rows of tokens without an adapter are not written.
 * v: [T][ldv] float32 device; y: [T][ldy] device. */
lora_status sgmv_expand(const lora_pool *p, const lora_plan *pl, int32_t layer,
                        int32_t nproj, const int32_t *projs, const int32_t *y_offsets,
                        const float *v, int64_t ldv, void *y, int64_t ldy, void *stream);

/* Fused shrink then expand (steps 1 and 3 of the same pseudocode in one call;
 * "TGI Multi-LoRA", "Technical Foundation": the frozen layer's output plus the
 * adapter's B A x): y = y_in + s_i * B_i,p (A_i,p x), with y_in = base
 * (base_out of the frozen layer, same column layout as y, [T][ldb]) when base
 * is non-NULL, else the current y.  Tokens without an adapter get y = base
 * (or are left untouched when base is NULL).  v is never written to memory:
 * for short groups (decode steps) the expand sums the shrink's partials
 * itself; a long group's (a prompt's, once the batch's long groups hold 1024
 * tokens) whole delta runs in one kernel whose workgroups keep v in LDS. */
lora_status sgmv_fused(const lora_pool *p, const lora_plan *pl, int32_t layer,
                       int32_t nproj, const int32_t *projs, const int32_t *y_offsets,
                       const void *x, int64_t ldx, const void *base, int64_t ldb,
                       void *y, int64_t ldy, void *stream);

/* sgmv_fused in two calls (the A step, scale 1.0, "Compress then Serve"
 * rebuttal pseudocode, step 1; then step 3): the shrink leaves float32
 * partial sums of v for the plan's short groups and the v rows of its long
 * groups (prompts) in the plan's workspace; the expand reads them and
 * writes y exactly as sgmv_fused does (the same bits).  The shrink needs
 * only x, so a caller can run it beside the frozen layer's own product and
 * the expand after it.  The workspace holds the partials of the last shrink
 * run with the plan (this one, sgmv_fused's or sgmv_shrink's; the long
 * groups' v rows only this one's: sgmv_fused keeps them inside its kernel);
 * the expand must name that call's layer and projections and, for a plan
 * with long groups, follow sgmv_shrink_partials (LORA_ESTATE otherwise), and
 * runs on a stream ordered after that shrink.  Arguments and errors as
 * sgmv_fused. */
lora_status sgmv_shrink_partials(const lora_pool *p, const lora_plan *pl, int32_t layer,
                                 int32_t nproj, const int32_t *projs, const void *x, int64_t ldx,
                                 void *stream);
lora_status sgmv_expand_partials(const lora_pool *p, const lora_plan *pl, int32_t layer,
                                 int32_t nproj, const int32_t *projs, const int32_t *y_offsets,
                                 const void *base, int64_t ldb, void *y, int64_t ldy,
                                 void *stream);
/* The same expand with the core step of jointly compressed adapters (the
 * core table as for sgmv_fused_sigma). */
lora_status sgmv_expand_partials_sigma(const lora_pool *p, const lora_plan *pl, int32_t layer,
                                       int32_t nproj, const int32_t *projs,
                                       const int32_t *y_offsets, const float *sigma,
                                       int32_t sigma_kind, int32_t num_sigma, const void *base,
                                       int64_t ldb, void *y, int64_t ldy, void *stream);

/* The three-step delta of jointly compressed adapters ("Compress then
 * Serve", rebuttal pseudocode of add_lora_slice_with_sigma: step 1 A into a
 * float32 buffer, step 2 the core Sigma into a second float32 buffer, step 3
 * B with the scale into the y slice):
 *   y[t][y_offsets[i] + o] = y_in + s_c * sum_j B_c,p[o][j] (Sigma_k v)[j],
 *   (Sigma_k v)[j] = sum_l Sigma_k,l,p[j][l] v[l]   (full, l ascending), or
 *                  = Sigma_k,l,p[j] v[j]             (diagonal),
 * with c the token's pool entry, k its core (plan_create_sigma), v = A_c,p x
 * (fused) or the caller's v (expand), all in float32; a token without a
 * core uses v itself.  sigma: device float32 table, 16-byte aligned,
 * [num_sigma][num_layers][num_proj][r_max][r_max] (LORA_SIGMA_FULL) or
 * [num_sigma][num_layers][num_proj][r_max] (LORA_SIGMA_DIAG); entries at or
 * beyond an entry's padded rank are not read, entries between its rank and
 * padded rank multiply zeros and must be finite.  Errors as the plain calls,
 * and LORA_EINVAL for a bad kind, table pointer, or a plan naming a core
 * >= num_sigma.  With a plan from lora_plan_create (no cores) these equal
 * the plain calls bit for bit. */
lora_status sgmv_expand_sigma(const lora_pool *p, const lora_plan *pl, int32_t layer,
                              int32_t nproj, const int32_t *projs, const int32_t *y_offsets,
                              const float *v, int64_t ldv, const float *sigma,
                              int32_t sigma_kind, int32_t num_sigma, void *y, int64_t ldy,
                              void *stream);
lora_status sgmv_fused_sigma(const lora_pool *p, const lora_plan *pl, int32_t layer,
                             int32_t nproj, const int32_t *projs, const int32_t *y_offsets,
                             const void *x, int64_t ldx, const float *sigma, int32_t sigma_kind,
                             int32_t num_sigma, const void *base, int64_t ldb, void *y,
                             int64_t ldy, void *stream);

/* --------------------------------------------------------------- debug ---- */
/* The library built with LORA_SGMV_DEBUG (libhab_lora_debug.so, for
 * debugging the kernels or a caller's plan memory) checks in every work unit
 * that each adapter block it addresses lies inside the pool's slab
 * (LORA_DEBUG_SLAB), that each token row it reads from the plan lies in
 * [0, num_tokens) or is the -1 of an absent row (LORA_DEBUG_TOKEN), and that
 * each plan position it indexes a per-row table with lies inside the plan
 * (LORA_DEBUG_ROW).  A failed check sets its bit in a device-wide error word
 * and switches that access off (the block reads as zeros, the row is taken
 * as absent), so the launch ends normally with a wrong result instead of
 * reading outside the slab or the caller's tensors.  The release build
 * compiles the checks out.
 * lora_debug_checks reports whether the loaded build checks (*enabled, 1 or
 * 0) and the error bits set on the current device since the last clear
 * (*errors; always 0 in the release build), and with `clear` resets them.
 * It waits for the current device to finish its work.  Either pointer may be
 * NULL.  Errors: LORA_EHIP. */
#define LORA_DEBUG_SLAB 1u
#define LORA_DEBUG_TOKEN 2u
#define LORA_DEBUG_ROW 4u
lora_status lora_debug_checks(int32_t *enabled, uint32_t *errors, int32_t clear);

/* ------------------------------------------------------- no allocation ---- */
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): sgmv_fused
 * with the shrink's partial sums in the library's static device scratch of
 * LORA_STATIC_SCRATCH_MIB MiB instead of the plan workspace's partial region.
 * The call makes no hipMalloc, hipFree or other allocating call; the caller
 * still passes x, base and y and a plan uploaded before, whose tables the
 * kernels read.  Each GPU has its own scratch, held from the first call on
 * that GPU until the process ends, and every call on one GPU shares it:
 * calls that overlap on one GPU (on different streams) race and give wrong
 * results, so order them.  Nothing in the scratch needs clearing (every
 * partial a call reads, the same call wrote before), and it keeps the last
 * call's partials.  A call whose partials exceed the scratch is refused with
 * LORA_EINVAL (split the batch).  Afterwards the plan's workspace holds no
 * partials for sgmv_expand_partials.  Arguments, results (bit for bit) and
 * other errors as sgmv_fused. */
#define LORA_STATIC_SCRATCH_MIB 64
lora_status sgmv_fused_static(const lora_pool *p, const lora_plan *pl, int32_t layer,
                              int32_t nproj, const int32_t *projs, const int32_t *y_offsets,
                              const void *x, int64_t ldx, const void *base, int64_t ldb,
                              void *y, int64_t ldy, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_SGMV_H */
