/*
 * agmm — all-gather fused matmul for AMD Instinct MI355X (gfx950).
 *
 * One GPU's share of the all-gather matmul
 *
 *     C[m, n_local] = concat_r(A_r[m_per_shard, k]) @ B[k, n_local]
 *     m = num_shards * m_per_shard
 *
 * as the tpu-inference page defines it ("all_gather_matmul.py",
 * `all_gather_matmul`: the result is all-gather(x, axis=0) @ y, x sharded by
 * rows over the ring, y sharded by columns so each device owns n_local of
 * them and produces C[:, n_local]) and as the Triton-distributed-Ascend
 * tutorial "AllGather-GEMM" checks it (golden `torch_allgather_gemm`:
 * all-gather, concatenate along dim 0, matmul).  With rhs_transpose, B is
 * stored [n_local, k] and contracted on its second dimension (tpu-inference
 * `_do_mxu`, dot_general over dims ((1,),(1,))).
 *
 * On one GPU the peers' shards are separate device buffers; the caller
 * passes their addresses as a table (the role the per-peer pointer table
 * plays in the Mosaic-GPU launch_context page).
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device addresses (hipMalloc / torch CUDA
 *     tensors).  Host pointers are marked "host".
 *   - Layouts are dense row-major: shard r is [m_per_shard, k] (leading
 *     dimension k); B is [k, n_local] (ld n_local) or, with rhs_transpose,
 *     [n_local, k] (ld k); C is [m, n_local] (ld n_local), and row
 *     r*m_per_shard + i of C is row i of shard r.
 *   - Element type: every operand has the plan's dtype; C too (the cast
 *     rounds to nearest even).  bf16/fp16 accumulate in fp32; fp32 inputs
 *     accumulate in fp64 and round once to fp32.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream).  Work is enqueued asynchronously: it starts after everything
 *     earlier on `stream`, and later work on `stream` sees its results.
 *   - Errors: functions return an agmm_status (or NULL for plan creation)
 *     and record a thread-local status and message readable with
 *     agmm_last_status() / agmm_last_error().  No entry point aborts the
 *     process.  Invalid input is reported, never silently computed.
 *   - Ownership: the caller owns every buffer it passes and the stream; it
 *     must keep buffers alive until the enqueued work has finished.  The plan
 *     owns its workspace, its internal streams and events.
 */
#ifndef AGMM_H
#define AGMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct agmm_plan agmm_plan;
typedef agmm_plan *agmm_plan_t;

typedef enum {
  AGMM_BF16 = 0,
  AGMM_FP16 = 1,
  AGMM_FP32 = 2
} agmm_dtype;

typedef enum {
  AGMM_OK = 0,
  AGMM_ERR_INVALID_ARG = 1, /* NULL pointer, size < 1, unknown key or dtype */
  AGMM_ERR_UNSUPPORTED = 2, /* valid request this build does not implement
                               (alignment, shape rule, too many shards) */
  AGMM_ERR_OOM = 3,         /* device allocation failed */
  AGMM_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} agmm_status;

/* Paths an agmm_run can take (key "variant" of agmm_plan_set_int). */
typedef enum {
  AGMM_VARIANT_AUTO = 0,    /* plan picks: fused, or skinny for m <= 256 */
  AGMM_VARIANT_FUSED = 1,   /* GEMM reads A rows straight from the shard
                               buffers; no gathered copy (Ascend tutorial,
                               "AllGather + GEMM (Fused Distributed Kernel)":
                               no intermediate write between the phases) */
  AGMM_VARIANT_STAGED = 2,  /* chunked gather into a ring of nbuf slots on a
                               second stream, overlapped with the GEMM of the
                               previous chunk (Ascend tutorial, "Double
                               Buffering" and "pvalue Parameter") */
  AGMM_VARIANT_UNFUSED = 3, /* gather all of A, then one GEMM, one stream (the
                               decomposed approach the tutorial compares to) */
  AGMM_VARIANT_SKINNY = 4   /* small m, from the shard buffers: with B
                               stored n x k and m <= 128 a kernel of narrow
                               tiles over all of k (one launch) where those
                               tiles give every CU a workgroup, over k ranges
                               otherwise; other shapes split-K GEMM tiles;
                               k ranges are added by a fixed-order reduction
                               launch (tpu-inference `grid_k`) */
} agmm_variant;

/*
 * Check a problem description without touching the GPU.
 * Returns AGMM_OK if agmm_plan_create would accept it, otherwise the status
 * it would fail with (and sets agmm_last_error()).
 *   num_shards    1 .. 64
 *   m_per_shard, k, n_local >= 1, with m = num_shards * m_per_shard, k and
 *                 n_local < 2^30 and m*k, k*n_local, m*n_local < 2^40
 *                 (else AGMM_ERR_UNSUPPORTED)
 *   dtype         agmm_dtype
 *   rhs_transpose 0: B is [k, n_local]; 1: B is [n_local, k]
 * Any k and n_local are accepted.  bf16/fp16 rows that are not whole
 * 16-byte vectors (k % 8 != 0, or n_local % 8 != 0 with B stored k x n) are
 * computed on zero-padded copies of A ([m][k rounded up to 8]) and B that the
 * plan keeps in its workspace, the way the Ascend tutorial's kernel masks its
 * K and N tails: every requested variant then runs as gather-then-GEMM.  The
 * staged and unfused variants of fp32 plans with k % 4 != 0 run the same way
 * (on rows zero-padded to a multiple of 4; the fused fp32 path reads any
 * row length).  (The tpu-inference page's own `validate_inputs`
 * rules - 2-D inputs, equal dtypes, matching k - are implied by this
 * signature; its TPU tiling rules are not imposed.)
 */
int agmm_plan_validate(int num_shards, int64_t m_per_shard, int64_t k, int64_t n_local,
                       int dtype, int rhs_transpose);

/*
 * Create a plan on the current HIP device.  Validates as above, picks tiles
 * and the default variant, and allocates everything a run needs (ring
 * workspace, split-K partials, tile-order tables, internal stream and
 * events), so agmm_run itself never allocates.
 * Returns NULL on failure (see agmm_last_status / agmm_last_error).
 */
agmm_plan_t agmm_plan_create(int num_shards, int64_t m_per_shard, int64_t k, int64_t n_local,
                             int dtype, int rhs_transpose);

/*
 * Enqueue C = concat(A_r) @ B (or @ B^T) on `stream`.
 *   shard_ptrs  host array of num_shards device pointers, shard r = [m_per_shard, k]
 *               with rows "lda" elements apart; read during the call only (may be
 *               freed on return)
 *   B           device, [k, n_local] or [n_local, k] (rhs_transpose), rows "ldb"
 *               elements apart
 *   C           device, [m, n_local], rows "ldc" elements apart; must not overlap
 *               any input
 *   stream      hipStream_t as void*
 * Row strides are the plan's "lda", "ldb", "ldc" settings (default: dense,
 * i.e. k, n_local or k, n_local); every buffer must hold its last row in full.
 * All device pointers must be 16-byte aligned.
 * Ordering between calls on one plan: every call that enqueues work on the
 * plan (agmm_run, agmm_run_gathered, agmm_run_gather_out, agmm_plan_autotune)
 * records the plan's completion event on its stream after the plan's internal
 * streams have joined that stream, and the next such call's stream waits on
 * it before any of its own work.  So calls on different streams, or from
 * different host threads (a mutex serialises the host side), run one after
 * the other on the GPU and never overwrite ring slots or split-K partial sums
 * a previous call still reads (the Ascend tutorial's "Double Buffering": a
 * slot is not refilled before the chunk reading it has been consumed).
 * Within one graph capture calls are ordered the same way.  Across a capture
 * boundary (a graph replay against eager calls) no event links them: the
 * caller orders replays with its streams, as for any graph.
 * Graph capture of the staged variant is limited to the replayed and tested
 * form: one staged call of a plan per captured graph, and at most as many
 * chunks as ring slots (ceil(m_per_shard / (pvalue * tile rows)) <= nbuf);
 * other staged calls under capture return AGMM_ERR_UNSUPPORTED before
 * enqueuing anything (the capture stays valid).
 * Returns AGMM_OK, AGMM_ERR_INVALID_ARG (NULL plan/pointer),
 * AGMM_ERR_UNSUPPORTED (misaligned pointer, staged form not capturable),
 * AGMM_ERR_HIP (launch failed), or the status that left the plan unusable
 * (see agmm_plan_set_int).
 */
int agmm_run(agmm_plan_t plan, const void *const *shard_ptrs, const void *B, void *C,
             void *stream);

/*
 * Enqueue only the all-gather: gathered[r*m_per_shard + i, :] = shard r row i,
 * a bit-exact copy.  gathered is a device buffer [m, k] of the plan's dtype,
 * 16-byte aligned (rows of any length: a vector copy for whole 16-byte rows,
 * an element copy otherwise).  (The gathered operand the tpu-inference kernel returns as
 * its second output, `x_hbm_scratch`.)  Same pointer and stream rules as
 * agmm_run.  It uses none of the plan's workspace and so takes no part in
 * the ordering between the plan's calls: order it against other work that
 * reads or writes `gathered` with the caller's streams.
 */
int agmm_gather(agmm_plan_t plan, const void *const *shard_ptrs, void *gathered, void *stream);

/*
 * Enqueue C = G @ B for an already gathered operand G [m, k] (device), e.g.
 * the output of agmm_gather or a staged run — the second half of the
 * tpu-inference page's "split n" idea (matmul the gathered x against another
 * column block of y without gathering again).  Shapes and dtype are the
 * plan's.  Same rules as agmm_run.
 */
int agmm_run_gathered(agmm_plan_t plan, const void *gathered, const void *B, void *C,
                      void *stream);

/*
 * Enqueue C = concat_r(A_r) @ B exactly as agmm_run, and also write the
 * gathered operand G[r*m_per_shard + i, :] = shard r row i (a bit-exact copy)
 * to `gathered` [m, k]: the gathered input handed back as a second output,
 * as the tpu-inference kernel does with its HBM scratch, so that a later
 * agmm_run_gathered can multiply it against another column block of B
 * without gathering again (that page's "split n" note).
 *   staged plans:  each chunk is copied straight to its place in `gathered`
 *                  and that chunk's GEMM reads it from there (no ring slot);
 *   unfused plans: gather into `gathered`, then the GEMM reads it;
 *   fused, skinny and fp32 plans: key "gather_out" 1: the GEMM reads the
 *                  shards on `stream` while the plan's second stream writes
 *                  `gathered`; 2: `gathered` is written first and the GEMM
 *                  reads it (same tile and k order, so the same C);
 *                  0 (default): 2, measured faster (the chip is power-limited
 *                  under MFMA load, so a copy beside the GEMM slows it by more
 *                  than the copy costs).
 * `gathered` is a caller-owned device buffer of the plan's dtype, 16-byte
 * aligned, not aliasing the shards, B or C.  Same stream rules and return
 * codes as agmm_run; work enqueued later on `stream` sees both outputs
 * complete.
 */
int agmm_run_gather_out(agmm_plan_t plan, const void *const *shard_ptrs, const void *B, void *C,
                        void *gathered, void *stream);

/*
 * Measure and keep the fastest settings for this plan's problem.  The
 * tpu-inference kernel picks its block sizes from a tuned table that the page
 * refers to but does not give; here the plan times its own candidates on the
 * caller's buffers instead: the compiled bf16/fp16 tile shapes that fit the B
 * layout, automatic / 1 / 2 / 4 / 8 k-splits and 4 / 8 row blocks walked
 * together, each configuration that resolves differently timed once (one
 * warm-up run, then `iters` runs, 1 <= iters <= 1000, with HIP events on
 * `stream`).  The plan keeps the fastest ("tile", "splits", "group_m" then read
 * back the choice) and *best_ms (may be NULL) receives its mean time per run.
 * fp32 plans are only timed.  Same buffers and rules as agmm_run; C is
 * overwritten with the product; synchronous (returns after the last run);
 * may reallocate the plan's workspace.  Returns AGMM_OK or the first error of
 * agmm_run's kinds (AGMM_ERR_HIP when no candidate ran).
 */
int agmm_plan_autotune(agmm_plan_t plan, const void *const *shard_ptrs, const void *B, void *C,
                       void *stream, int iters, double *best_ms);

/*
 * Tune a plan.  Keys (value ranges):
 *   "variant"       agmm_variant
 *   "pvalue"        >= 1: tile-rows of each shard per staged chunk
 *   "nbuf"          >= 1: ring slots for the staged variant
 *   "tile"          -1: automatic, else a compiled bf16/fp16 tile shape:
 *                   0 256x256 (32-deep k-tiles, 4 LDS stages; automatic for
 *                   k < 256), 1 128x128 and 2 256x128 (same loop, two
 *                   workgroups per CU), 3 128x64 and 4 128x64 with 8 stages
 *                   (rhs_transpose only), 5 256x256, 6 128x128 and 7 128x64
 *                   (rhs_transpose only) with 64-deep k-tiles in a 5-slot
 *                   operand ring, 8 256x256 and 9 128x128 in the same ring on
 *                   16x16x32 MFMAs (the automatic choices for k >= 256),
 *                   10 the skinny kernel (rhs_transpose only; tile from
 *                   "skinny_shape"; whole k per workgroup, or k ranges as
 *                   "splits" says; the automatic skinny choice for
 *                   m <= 128; 7 for 128 < m <= 256), 11 256x224
 *                   in the 16x16x32 ring (rhs_transpose only; automatic where
 *                   its 224-column tiles fill whole rounds of workgroups that
 *                   256x256 tiles would leave partly idle).  A tile that
 *                   needs rhs_transpose on a plan without it (and without
 *                   the transposed copy of B, "b_transpose") is rejected
 *                   with AGMM_ERR_UNSUPPORTED.
 *   "splits"        0: automatic, else k-splits (fp32 partial sums, then a
 *                   fixed-order reduction) of every bf16/fp16 launch (for the
 *                   staged variant: of each chunk's launch); automatic splits
 *                   are used by the skinny tiles (as many k ranges as
 *                   fill the CUs, each at least 64 elements per wave of
 *                   tile 10) and by launches whose output tiles fill at
 *                   most half of the workgroup slots
 *   "local_shard"   0 .. num_shards-1: where the ring order starts
 *   "order"         0: ring order from local_shard, 1: natural order
 *   "group_m"       row blocks walked together (L2 reuse); 0 (default):
 *                   chosen per launch shape, the count whose tiles on one XCD
 *                   touch the fewest A row blocks plus B column blocks
 *   "xcd_remap"     0/1: keep consecutive tiles on one XCD
 *   "copy_wgs"      >= 0: workgroups of each staged chunk copy (0 = auto:
 *                   sized to the whole GPU) and of the side gather of
 *                   agmm_run_gather_out (0 = one per CU)
 *   "skinny_shape"  -1 (automatic: 5, or 7 where 32 x 32 tiles would
 *                   need more than one workgroup per CU and 64 x 64 tiles
 *                   would not) or 0..7: output tile of the skinny kernel
 *                   (tile 10), rows x columns: 0 64 x 16, 1 32 x 32,
 *                   2 32 x 16, 3 16 x 32, 4 64 x 32, 7 64 x 64 (4 waves);
 *                   5 32 x 32, 6 64 x 16 (8 waves).  Reads back the shape in
 *                   use.
 *   "copy_engine"   0 (default) or 1: what performs the copies that run
 *                   beside a GEMM (staged chunks after the first, the side
 *                   gather of agmm_run_gather_out).  0: the gather kernel on
 *                   the CUs.  1: the SDMA engines (hipMemcpyDeviceToDeviceNoCU),
 *                   used only for dense shard rows (lda == k) and never while
 *                   the caller's stream is being captured into a graph (the
 *                   kernel copies then).  Both are bit copies.
 *   "lda", "ldb", "ldc"  0 (dense, the default) or the element stride between
 *                   rows of the shards, of B as stored and of C: at least the
 *                   row length; lda and ldb also a multiple of 16 bytes
 *                   (any value for plans on padded copies, see
 *                   agmm_plan_validate).  The
 *                   gathered buffers of agmm_gather / agmm_run_gathered /
 *                   agmm_run_gather_out stay dense [m, k].  get returns the
 *                   stride in use.
 *   "gemm_streams"  1 or 2 (default 2): staged chunk GEMMs alternate over
 *                   this many streams, so one chunk's workgroups fill the
 *                   CUs the previous chunk's leave (1 with split-K)
 *   "local_first"   0 (default) or 1: with two or more chunks, the staged
 *                   variant computes the local
 *                   shard's rows (shard "local_shard") first, straight from
 *                   its buffer and beside the first chunk's copy (it needs no
 *                   copy: tpu-inference `all_gather_matmul`, a device's own
 *                   x block); the chunk GEMMs then cover the other shards'
 *                   rows.  The ring slots still hold every shard's rows.
 *   "gather_out"    0, 1 or 2: how agmm_run_gather_out produces the gathered
 *                   operand on fused, skinny and fp32 plans (see there)
 *   "debug_keep_slots" 0/1: staged variant uses one slot per chunk (nothing
 *                   is overwritten; for inspection by agmm_plan_slot_ptr)
 *   "b_transpose"   -1 (automatic, the default), 0 or 1: for bf16/fp16 B
 *                   stored k x n (no rhs_transpose; rows of whole 16-byte
 *                   vectors) on the fused, unfused and staged variants, each
 *                   call first writes B^T [n_local][k] into the workspace
 *                   (a bit copy) and the GEMM then reads B as n x k: a
 *                   plain 16-byte LDS read per B fragment instead of two
 *                   transposing reads.  Automatic: on for k >= 256 and
 *                   m >= 24576 (measured on 8x4096x8192 -> 7168 bf16: GEMM
 *                   2700 -> 2619 us for a 44 us transpose; break-even near
 *                   m = 18K).  The tile, k order and so the result are those
 *                   of reading B directly.  get "b_transposed" reads 1 when
 *                   the copy is in use.
 * A change waits for the plan's previous call to finish, then keeps the
 * workspace allocation if the new layout fits in it and reallocates it
 * otherwise.  It is all or nothing: when the new value is rejected (range,
 * a tile the layout cannot use, AGMM_ERR_OOM) the plan keeps its previous
 * settings and a workspace for them.  Only if even that workspace cannot be
 * allocated again is the plan left unusable: every later call on it then
 * fails with the status of that failure (get "usable" reads 0).  A plan that
 * a graph has captured keeps its settings for good (the graph holds its
 * workspace addresses and tile tables): set_int then returns
 * AGMM_ERR_UNSUPPORTED (get "captured" reads 1).
 * Returns AGMM_OK, AGMM_ERR_INVALID_ARG (unknown key / out of range),
 * AGMM_ERR_UNSUPPORTED (captured plan, tile not usable) or AGMM_ERR_OOM.
 */
int agmm_plan_set_int(agmm_plan_t plan, const char *key, int64_t value);

/* Read a plan setting (keys above, plus "num_chunks", "rows_per_chunk",
 * "num_slots", "tile_bm", "tile_bn", "k_per_split", "num_row_blocks",
 * "cu_count", the resolved "variant_used", "group_m_used": the row-block
 * group a launch over the whole problem uses, "b_transposed": 1 when calls
 * copy B transposed first, "captured": 1 once a call was captured into a
 * graph, and "usable": 0 after a failed reconfiguration left the plan
 * without a workspace).  value: host pointer.  Returns AGMM_OK or
 * AGMM_ERR_INVALID_ARG. */
int agmm_plan_get_int(agmm_plan_t plan, const char *key, int64_t *value);

/* Bytes of device workspace the plan holds (ring, partials, B copy, tables; the
 * allocation is kept when a new layout needs less). */
size_t agmm_plan_workspace_bytes(agmm_plan_t plan);

/* Device address of ring slot `slot` ([num_shards][rows_per_chunk][k]) or
 * NULL; for tests of the staged gather. */
const void *agmm_plan_slot_ptr(agmm_plan_t plan, int slot);

/*
 * Row-block visit order the plan's GEMM uses (host array `out` of at least
 * "num_row_blocks" entries for chunk `chunk`; chunk 0 for non-staged).
 * Ring order from local shard r0: step s takes the first half of shard
 * (r0+s) mod N and then the second half of shard (r0-s) mod N (tpu-inference
 * `_all_gather_kernel`: the bidirectional ring sends the top half of a shard
 * left and the bottom half right, so at step s a device holds the top half of
 * shard d+s and the bottom half of shard d-s; `_do_o_local_copy` writes them
 * to those rows).  A row block waits for the latest of its rows.
 * Returns the number of entries written, or -1 on error.
 */
int agmm_plan_tile_order(agmm_plan_t plan, int chunk, int32_t *out, int capacity);

/*
 * Per-launch timing of the plan's main GEMM kernel with HIP events recorded
 * on the stream that kernel is launched on.  begin: clear and enable;
 * read: wait for the recorded events and return the summed kernel time (ms)
 * and the number of launches timed; end: disable.
 */
int agmm_plan_timing_begin(agmm_plan_t plan);
int agmm_plan_timing_read(agmm_plan_t plan, double *total_ms, int64_t *launches);
int agmm_plan_timing_end(agmm_plan_t plan);

/* Wait for the plan's last call and its internal streams (nothing else on
 * the device), then free its workspace, streams and events.  NULL is a
 * no-op.  Destroy a plan only after every graph that captured it has been
 * destroyed or has finished its last replay: the graph uses its workspace. */
void agmm_plan_destroy(agmm_plan_t plan);

/*
 * For callers that cannot allocate device memory (code being captured into a
 * graph, tight serving loops, harnesses that forbid hipMalloc): the work of
 * agmm_run on a newly created plan for this problem (automatic variant, tile
 * and k split; the fused and skinny paths only), with no plan and nothing
 * allocated.  The split-K partial sums go into a scratch array of
 * AGMM_NOALLOC_SCRATCH_BYTES that the library keeps in the memory of every
 * GPU it runs on until the process ends; its device address is looked up on
 * the first call on each device (make that first call outside graph
 * capture).  Arguments, layouts (dense rows), alignment and stream rules are
 * agmm_run's.  Tile visit order is the natural one (the values do not depend
 * on it), and B stored k x n is read directly (the transposed copy of B,
 * "b_transpose", needs a plan's workspace; it does not change the bits), so
 * C is bit-identical to agmm_run's on a default plan.
 * Every call on one GPU shares that GPU's scratch and leaves its partial sums
 * there: calls whose work overlaps on one GPU (different streams without an
 * ordering between them, or host threads) race and may return wrong values;
 * order them on one stream.  Nothing needs clearing between calls: every
 * partial sum a call reads was written by that call.
 * Returns AGMM_OK, agmm_plan_validate's statuses, agmm_run's pointer
 * statuses, AGMM_ERR_UNSUPPORTED when the problem resolves to the staged or
 * unfused path or its partial sums need more than
 * AGMM_NOALLOC_SCRATCH_BYTES (nothing is launched then), or AGMM_ERR_HIP.
 */
#define AGMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int agmm_run_noalloc(int num_shards, int64_t m_per_shard, int64_t k, int64_t n_local, int dtype,
                     int rhs_transpose, const void *const *shard_ptrs, const void *B, void *C,
                     void *stream);

/* Thread-local status / message of this thread's most recent call into the
 * library (AGMM_OK and "" after a call that succeeded; calls on other threads
 * never change them). */
int agmm_last_status(void);
const char *agmm_last_error(void);

/* Library version string. */
const char *agmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AGMM_H */
