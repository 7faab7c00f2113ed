/*
 * tide.h -- C ABI of the layout-aware FSDP2 collective local stages on one
 * MI355X (gfx950) GPU.
 *
 * Operations, after "The Endgame of FSDP Communication: Layout-Aware
 * Collectives on Copy Engines, RDMA, and NVSwitch" (Wang et al.):
 *
 *   reduce-scatter local stage (Section 4, Equation 5; Section 4.1): W ranks'
 *     per-parameter bf16 (or fp32) gradients, all resident in this GPU's
 *     memory, are summed into W packed per-rank fp32 shards, then scaled and
 *     optionally accumulated (Equation 5).  The dimension-0 shard placement
 *     of Section 2.1 is folded into the addressing: no packed intermediate
 *     buffer (Equation 3) is formed.
 *
 *   all-gather copy-out (Section 2.1): a flat rank-major bf16 buffer is
 *     scattered into per-parameter tensors.
 *
 *   all-gather copy-in (Section 2.1, with the cast of Section 3.1): every
 *     rank's local fp32 (or bf16) shards are packed into the rank-major bf16
 *     buffer the all-gather would produce; the inverse of the copy-out.
 *
 *   stock gradient pack (Section 2.1, Equation 3): the step that the layout-
 *     aware reduce-scatter removes, provided as the baseline: one rank's bf16
 *     gradients are sliced, zero-padded, widened and packed rank-major into
 *     the fp32 buffer a stock reduce-scatter reads.
 *
 * Shard geometry (Section 2.1), in ELEMENTS.  Parameter p has shape
 * (d_0, ..., d_{m-1}), m >= 1, viewed as D_p = d_0 rows of K_p = d_1*...*d_{m-1}
 * elements (K_p = 1 for m = 1).  Each of the W ranks owns R_p = ceil(D_p / W)
 * rows: rank r owns rows [r R_p, (r+1) R_p), rows at or past D_p are padding.
 * Shard size n_p = R_p K_p, prefix offset o_p = sum_{i<p} n_i (no alignment
 * padding between parameters), per-rank shard size S = sum_p n_p.  The real
 * element count of rank r's shard of p is
 *   n_real(p, r) = clamp(D_p - r R_p, 0, R_p) * K_p.
 *
 * Conventions for every call:
 *   - Every call returns a tide_status; TIDE_OK is 0.  On failure,
 *     tide_last_error() holds a message (thread-local, valid until the
 *     calling thread's next tide_* call).
 *   - Argument checks happen before any device work: a call that fails them
 *     enqueues nothing and leaves every output untouched.
 *   - Device buffers are owned by the caller and must stay alive until the
 *     work enqueued on `stream` has finished.  Host arrays passed in are read
 *     during the call only.
 *   - `stream` is a hipStream_t (NULL means the null stream).  Calls are
 *     asynchronous on it; nothing blocks the host except the one-time
 *     device set-up of a plan (see below).
 *   - Outputs must not overlap inputs or each other.
 *   - A plan may be used by one host thread and one stream at a time: its
 *     device pointer tables are rewritten (stream-ordered) when a call passes
 *     different pointers from the previous call.
 *   - Results never depend on tide_options: every option only changes how the
 *     work is split, never which additions happen or in what order.
 *   - Graph capture: once a plan has run an operation with the same pointers
 *     (and options) on the current device, a call of that operation enqueues
 *     kernel launches only (no allocation, copy or synchronization), so it may
 *     be recorded into a HIP graph and replayed.  The recorded launches read
 *     the plan's device tables each time they run: the plan must outlive the
 *     graph, and a later call of that operation with other pointers, or
 *     tide_plan_set_options, rewrites those tables and so changes what a
 *     replay does (use one plan per set of buffers that a graph records).
 *     A call on a stream that is capturing, which would set up or upload
 *     those tables (the plan's first call of that operation, other pointers
 *     or other options than the previous call's), returns TIDE_ERR_INVALID
 *     and enqueues nothing.
 */
#ifndef TIDE_H
#define TIDE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TIDE_OK = 0,
    TIDE_ERR_INVALID = -1,     /* null or out-of-range argument, bad shape, unknown/destroyed plan */
    TIDE_ERR_RANGE = -2,       /* a size overflows int64 or exceeds a documented limit */
    TIDE_ERR_ALIGN = -3,       /* a pointer is not aligned to its element size */
    TIDE_ERR_NOMEM = -4,       /* host, pinned or device allocation failed */
    TIDE_ERR_HIP = -5,         /* a HIP runtime call failed (its text is in tide_last_error) */
    TIDE_ERR_UNSUPPORTED = -6  /* reserved: no current call returns it */
} tide_status;

/* Element types (the copy-in's shard_dtype). */
#define TIDE_DTYPE_BF16 0
#define TIDE_DTYPE_F32 1

/* Largest number of simulated ranks a plan may have. */
#define TIDE_MAX_WORLD 256

/* tide_options.flags.  By default every kernel streams: loads and stores
 * carry the non-temporal hint (the data is touched once). */
#define TIDE_FLAG_CACHED_LOADS 0x1u  /* plain (temporal) loads instead */
#define TIDE_FLAG_CACHED_STORES 0x2u /* plain (temporal) stores instead */
/* Keep the chunk -> segment table in global memory instead of staging it in
 * LDS: the kernels then allocate no LDS, so a co-running kernel that claims a
 * whole CU's LDS (a large GEMM tile, the probe below) is never kept off a CU
 * by them (Section 2.2: placement decides which kernels are displaced). */
#define TIDE_FLAG_NO_LDS 0x4u

/*
 * Launch knobs.  A numeric field of 0 selects the default of the operation
 * being launched.  None of them changes any result bit (Section 4.3: tuning
 * knobs preserve operand grouping).
 *   cu_budget   the persistent grid has cu_budget * wg_per_cu workgroups
 *               (fewer if there are fewer chunks than waves, and at most
 *               2^27); default: the
 *               device's CU count.  Workgroups are dispatched round-robin over
 *               the 8 XCDs, so a budget is a grid size, not a CU mask.
 *   wg_per_cu   workgroups (256 threads, four waves) per budgeted CU;
 *               default 1.
 *   chunk_elems elements per chunk (the unit a wave takes), a multiple of 8,
 *               at most 2^28; default 1024 (reduce-scatter; 2048 when W <= 3), 256
 *               (reduce-scatter of fp32 gradients), 4096 (copy-out, copy-in),
 *               2048 (stock pack).
 *               A plan may have at most 2^30 chunks per operation.
 *   flags       TIDE_FLAG_* bits.
 *   wave_chunks at most this many chunks per wave in one kernel launch; an
 *               operation with more chunks than waves * wave_chunks is run as
 *               several launches of about equal length, back to back on the
 *               stream (waves of one long launch drift apart and spread their
 *               memory traffic).  In a reduce-scatter, a rank's shard of
 *               at least one round that would start mid-round opens a launch
 *               of its own once the previous group holds wave_chunks/2
 *               rounds (tide_plan_launches lists the result).
 *               At most 2^30 (one launch for any plan); default 64.
 */
typedef struct {
    int32_t cu_budget;
    int32_t wg_per_cu;
    int64_t chunk_elems;
    uint32_t flags;
    int32_t wave_chunks;
} tide_options;

typedef struct tide_plan tide_plan; /* opaque, owned by the library */

/*
 * Create a plan for W = `world` simulated ranks and P = `nparams` parameters.
 *   world      1 <= W <= TIDE_MAX_WORLD
 *   nparams    P >= 1
 *   ndims      [P] number of dimensions of each parameter, each >= 1
 *   dims       all dimensions, concatenated in parameter order
 *              (sum_p ndims[p] entries), each >= 0
 *   opt        launch knobs, or NULL for defaults
 *   out_plan   receives the plan
 * Host only: no device call is made.  The plan's device tables are allocated
 * and uploaded by the first data-moving call that uses it, on
 * the device current at that time (that first call blocks the host for the
 * allocation); the plan is bound to that device afterwards.
 * Errors: TIDE_ERR_INVALID (bad counts, shapes, options, null pointers),
 * TIDE_ERR_RANGE (W * S above 2^61 elements, so that byte offsets fit
 * int64; too many chunks), TIDE_ERR_NOMEM.
 */
tide_status tide_plan_create(int32_t world, int32_t nparams, const int32_t* ndims, const int64_t* dims,
                             const tide_options* opt, tide_plan** out_plan);

/*
 * Shard geometry of a plan, in elements (Section 2.1).  Any output pointer
 * may be NULL.
 *   rows_per_rank  [P] R_p
 *   shard_offset   [P] o_p
 *   shard_elems    [1] S
 */
tide_status tide_plan_layout(const tide_plan* plan, int64_t* rows_per_rank, int64_t* shard_offset,
                             int64_t* shard_elems);

/*
 * Element counts of a plan's tensors (Section 2.1), for sizing the buffers a
 * call takes.  Any output pointer may be NULL.
 *   param_elems  [P] D_p * K_p: the elements of parameter p (of each rank's
 *                gradient of p, and of the copy-out's destination params[p])
 *   real_elems   [W*P] at index r*P + p, n_real(p, r): the real (non-padding)
 *                elements of rank r's shard of p, i.e. of the local shard
 *                that tide_allgather_copyin reads as shards[r*P + p]
 */
tide_status tide_plan_sizes(const tide_plan* plan, int64_t* param_elems, int64_t* real_elems);

/*
 * The plan's work segments, for inspection and tests.  op 0 = reduce-scatter,
 * 1 = copy-out, 2 = copy-in, 3 = stock pack, 4 = reduce-scatter of fp32
 * gradients (the same segments as op 0; it has its own chunk table and
 * launch knobs).  Each segment is 6 int64 values:
 *   kind     0 = sum of the W ranks' sources, 1 = zero fill (padding),
 *            2 = copy (the copy-in casts instead when its shards are fp32;
 *            the stock pack widens bf16 to fp32)
 *   src_idx  reduce-scatter, stock pack: parameter p; copy-out: 0 (the
 *            rank-major buffer); copy-in: shard index r*P + p
 *   dst_idx  reduce-scatter: destination rank r; copy-out: parameter p;
 *            copy-in, stock pack: 0 (the rank-major buffer)
 *   src_off  element offset in each source tensor (in the rank-major buffer
 *            for the copy-out)
 *   dst_off  element offset in the destination tensor (in the rank-major
 *            buffer for the copy-in and the stock pack)
 *   len      elements (> 0)
 * Writes min(capacity, count) segments to `table` (may be NULL when
 * capacity is 0) and the total count to *count.
 */
tide_status tide_plan_segments(const tide_plan* plan, int32_t op, int64_t* table, int64_t capacity,
                               int64_t* count);

/*
 * How one call of `op` is split into kernel launches under the plan's current
 * options, for inspection and tests (host only).  A launch covers chunks
 * [first, end) of the operation, which fall in its segments [seg, seg_end)
 * (indices into tide_plan_segments' table), with `workgroups` workgroups.
 * Each launch is 5 int64 values: first, end, seg, seg_end, workgroups.
 *   cu_count  the CU count that a cu_budget of 0 stands for; 0 = that of the
 *             device the plan is bound to (TIDE_ERR_INVALID if it is not
 *             bound and the options set no cu_budget).
 * Writes min(capacity, count) launches to `table` (may be NULL when capacity
 * is 0) and the total count to *count (0 when the operation has no work).
 */
tide_status tide_plan_launches(const tide_plan* plan, int32_t op, int32_t cu_count, int64_t* table,
                               int64_t capacity, int64_t* count);

/*
 * Which code path the elements of the latest call of `op` take, for spotting a
 * slow layout at run time (host only).  The latest call's pointers decide it:
 * a segment's vector body starts where its destination is aligned to the
 * vector group; the source may sit at another phase there.
 *   out[0]  elements moved by aligned vector bodies
 *   out[1]  elements moved by realigned vector bodies (the source at another
 *           phase than the destination; every operation but the stock pack
 *           realigns in registers, the reduce-scatter only when out[3] is 1)
 *   out[2]  elements moved one by one: heads and tails of segments, segments
 *           whose W sources sit at different phases, and the reduce-scatter's
 *           off-phase bodies when out[3] is 0
 *   out[3]  reduce-scatter only: 1 when the call runs the realigning instance
 *           (off-phase sum segments hold more than 1/50 of its elements)
 * out[0] + out[1] + out[2] is the elements the operation writes.
 * Errors: TIDE_ERR_INVALID (bad plan, op or out; no call of `op` made yet).
 */
tide_status tide_plan_paths(const tide_plan* plan, int32_t op, int64_t* out);

/* Replace the launch knobs (NULL = defaults).  Results are unaffected.
 * Errors: TIDE_ERR_INVALID, TIDE_ERR_RANGE (too many chunks). */
tide_status tide_plan_set_options(tide_plan* plan, const tide_options* opt);

/* The launch knobs in effect for op 0 (reduce-scatter), 1 (copy-out),
 * 2 (copy-in), 3 (stock pack) or 4 (reduce-scatter of fp32 gradients), with
 * defaults resolved (cu_budget is resolved once the plan is bound to a
 * device, 0 before). */
tide_status tide_plan_get_options(const tide_plan* plan, int32_t op, tide_options* out);

/*
 * Reduce-scatter local stage (Section 4, Equation 5; Section 4.3).
 *   grads   [W*P] host array of device pointers; grads[u*P + p] is rank u's
 *           bf16 gradient of parameter p: D_p*K_p elements, row-major, 2-byte
 *           aligned.  May be NULL only where D_p*K_p = 0.
 *   out     [W] host array of device pointers; out[r] receives rank r's
 *           packed fp32 shard: S elements, 4-byte aligned, written in full.
 *   alpha   Equation 5's scale (any value; 1.0f leaves the sum unchanged).
 *   accumulate
 *           0: the shards are overwritten; 1: the result is added to the
 *           values already in out[r] (which are then read), Equation 5's
 *           accumulate.  Other values: TIDE_ERR_INVALID.
 * For r in [0, W), p in [0, P), e in [0, n_p), with
 *   s = g_0 + g_1 + ... + g_{W-1}   for e < n_real(p, r),
 *       g_u = grads[u*P+p][r R_p K_p + e] widened exactly to fp32, added left
 *       to right (rank order 0..W-1) in IEEE binary32, round to nearest even,
 *       subnormals kept, no fused operations;
 *   s = +0.0f                       for padding (e >= n_real: every rank's
 *       padding rows are zeros);
 *   out[r][o_p + e] = s                       (alpha = 1, accumulate = 0)
 *   out[r][o_p + e] = alpha * s               (accumulate = 0)
 *   out[r][o_p + e] = old + alpha * s         (accumulate = 1)
 * each operation one binary32 rounding.  With alpha = 1 and accumulate = 0
 * the product is skipped (it is exact anyway).
 * The result is bit-identical for every tide_options setting.
 * Errors: TIDE_ERR_INVALID (null plan/arrays/pointers, accumulate not 0/1),
 * TIDE_ERR_ALIGN, TIDE_ERR_NOMEM, TIDE_ERR_HIP.
 */
tide_status tide_reduce_scatter_local(tide_plan* plan, const uint16_t* const* grads, float* const* out,
                                      float alpha, int32_t accumulate, void* stream);

/*
 * Allocation-free reduce-scatter, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and errors as
 * tide_reduce_scatter_local, bit for bit, with these differences:
 *   - No call allocates anything (no hipMalloc, hipFree, pinned or other
 *     allocation) and none uses the plan's device tables or binds the plan
 *     to a device: every call rebuilds its tables in host buffers the plan
 *     made when it was created, and writes them into a fixed scratch array
 *     of TIDE_NOALLOC_SCRATCH_BYTES in device memory, which the library holds
 *     on each device it runs on until the process ends.  The writes are
 *     kernel launches on `stream` carrying the table words as arguments, so
 *     the call is asynchronous and may be captured into a graph (a replay
 *     rewrites the recorded tables before the recorded reduce-scatter).  The
 *     first call on a device also looks up the array's device address; make
 *     one call on the device before capturing.
 *   - The tables of a plan of P parameters and W ranks, with N reduce-
 *     scatter segments (at most 2*W*P: a sum and a padding segment per rank
 *     and parameter), take 4*(N+1) bytes rounded up to 16, plus
 *     16*N + 8*(W+1)*N bytes (at W = 8 without padding, N = W*P segments of
 *     92 bytes: up to about 1,400 parameters); above
 *     TIDE_NOALLOC_SCRATCH_BYTES the call returns TIDE_ERR_RANGE and
 *     enqueues nothing.
 *   - All calls on one device share its scratch array, which keeps the
 *     tables of the last call: calls on one stream (or otherwise ordered)
 *     are safe, while calls that may overlap on the device (other streams,
 *     other host threads) race for it and give undefined results.
 */
#define TIDE_NOALLOC_SCRATCH_BYTES (1u << 20)
tide_status tide_reduce_scatter_local_noalloc(tide_plan* plan, const uint16_t* const* grads, float* const* out,
                                              float alpha, int32_t accumulate, void* stream);

/*
 * Reduce-scatter local stage from fp32 gradients (Section 4; the fp32
 * reduce-scatter of Section 4.3): as tide_reduce_scatter_local with
 * grads[u*P + p] fp32 (4-byte aligned) and g_u its value as it is.  With a
 * plan of one parameter of shape (W, S) this is also the reduce-scatter of
 * W ranks' pre-packed fp32 buffers (the stock path after its pack).  Its
 * launch knobs are those of op 4.
 */
tide_status tide_reduce_scatter_local_f32(tide_plan* plan, const float* const* grads, float* const* out,
                                          float alpha, int32_t accumulate, void* stream);

/*
 * All-gather copy-out (Section 2.1).
 *   rank_major  device pointer to W*S bf16 elements, 2-byte aligned: rank
 *               r's shard of parameter p starts at element r*S + o_p.
 *   params      [P] host array of device pointers; params[p] receives the
 *               D_p*K_p elements of parameter p (row-major, 2-byte aligned).
 *               May be NULL only where D_p*K_p = 0.
 * For every p, r and e < n_real(p, r):
 *   params[p][r R_p K_p + e] = rank_major[r S + o_p + e]   (16-bit moves)
 * Padding elements of the rank-major buffer are never read; every element
 * of every params[p] is written exactly once.
 * Errors: TIDE_ERR_INVALID, TIDE_ERR_ALIGN, TIDE_ERR_NOMEM, TIDE_ERR_HIP.
 */
tide_status tide_allgather_copyout(tide_plan* plan, const uint16_t* rank_major, uint16_t* const* params,
                                   void* stream);

/*
 * All-gather copy-in (Section 2.1; the mixed-precision cast of Section 3.1):
 * every rank's local shards are packed into the rank-major buffer the
 * all-gather produces.
 *   shards       [W*P] host array of device pointers; shards[r*P + p] is rank
 *                r's local shard of parameter p: its n_real(p, r) elements
 *                (rows [r R_p, r R_p + n_real/K_p) of the parameter, row-major),
 *                aligned to the element size.  May be NULL where n_real = 0.
 *   shard_dtype  TIDE_DTYPE_F32: fp32 shards, cast to bf16 by round to
 *                nearest even (a NaN stays a quiet NaN of the same sign with
 *                its top payload bits); TIDE_DTYPE_BF16: bf16 shards, copied.
 *   rank_major   device pointer to W*S bf16 elements, 2-byte aligned, written
 *                in full: rank r's shard of p at r*S + o_p, bf16 +0 (0x0000)
 *                in the padding of each slot.
 * Errors: TIDE_ERR_INVALID, TIDE_ERR_ALIGN, TIDE_ERR_NOMEM, TIDE_ERR_HIP.
 */
tide_status tide_allgather_copyin(tide_plan* plan, const void* const* shards, int32_t shard_dtype,
                                  uint16_t* rank_major, void* stream);

/*
 * Stock gradient pack of one rank (Section 2.1, Equation 3): what stock FSDP2
 * does before its reduce-scatter, kept as the baseline of the layout-aware
 * reduce-scatter above.
 *   grads   [P] host array of device pointers: this rank's bf16 gradients,
 *           grads[p] holding D_p*K_p elements, 2-byte aligned.  May be NULL
 *           only where D_p*K_p = 0.
 *   packed  device pointer to W*S fp32 elements, 4-byte aligned, written in
 *           full: for every p, r and e < n_p,
 *             packed[r S + o_p + e] = grads[p][r R_p K_p + e] widened exactly
 *                                     (e < n_real(p, r)),  +0.0f otherwise.
 * The W ranks' packed buffers, reduce-scattered with
 * tide_reduce_scatter_local_f32 on a (W, S) plan, give exactly the shards
 * tide_reduce_scatter_local gives (same additions in the same order).
 * Errors: TIDE_ERR_INVALID, TIDE_ERR_ALIGN, TIDE_ERR_NOMEM, TIDE_ERR_HIP.
 */
tide_status tide_stock_chunk_cat(tide_plan* plan, const uint16_t* const* grads, float* packed, void* stream);

/* ------------------------------------------------------------------------
 * Interference instruments (Section 2.2 "SM Wave Quantization", Equation 4,
 * Figure 3, Table 4 and Table 5): what one GPU can show of the cost a
 * collective's kernels impose on the compute they overlap.  None of these
 * touches a plan.
 * ------------------------------------------------------------------------ */

/*
 * Properties of the current device: its CU count, the largest LDS allocation
 * one workgroup may make and the LDS of one CU (bytes), and the rate of the
 * constant wall clock the probe records (kHz).  Any output pointer may be
 * NULL.
 * Errors: TIDE_ERR_HIP.
 */
tide_status tide_device_info(int32_t* cu_count, int32_t* max_lds_per_workgroup, int32_t* lds_per_cu,
                             int32_t* wall_clock_khz);

/*
 * Hardware-ID probe, the analog of the pages' SM-id probe (Table 5, Figure 3):
 * `grid` workgroups of 256 threads, each allocating `lds_bytes` of LDS (so
 * that at most floor(LDS per CU / lds_bytes) probe workgroups, and nothing
 * else that needs the rest, share a CU), each holding its CU for `hold_ns`
 * nanoseconds of wall-clock time and then writing one record of 8 uint32
 * words to records[8*b .. 8*b+7]:
 *   [0] b (the workgroup index)
 *   [1] the wave's HW_ID hardware register (CDNA ISA: wave id bits 3:0, SIMD
 *       id 5:4, pipe id 7:6, CU id 11:8, shader-array id 12, shader-engine
 *       id 15:13, ...)
 *   [2] the XCC_ID hardware register (accelerator-complex die id in bits 3:0)
 *   [3] 0 when the workgroup's LDS read back what it wrote (or lds_bytes < 4)
 *   [4],[5] entry time, [6],[7] exit time: wall-clock ticks (low, high word)
 *   records    device pointer to grid*8 uint32, 4-byte aligned
 *   grid       1 <= grid <= 65536
 *   lds_bytes  0 <= lds_bytes <= max_lds_per_workgroup
 *   hold_ns    0 <= hold_ns <= 1e9
 * Errors: TIDE_ERR_INVALID, TIDE_ERR_ALIGN, TIDE_ERR_HIP.
 */
tide_status tide_probe_launch(uint32_t* records, int32_t grid, int32_t lds_bytes, int64_t hold_ns, void* stream);

/*
 * The memory-bound elementwise victim (Table 4's 256 MiB elementwise
 * kernel; the pages do not give its operation): y[i] = a * x[i] + b for i in
 * [0, n), the product rounded to binary32 and then the sum (no fused
 * multiply-add), one thread per element or per group of four (16-byte
 * accesses when x and y are 16-byte aligned and n is a multiple of 4).
 *   x, y  device pointers to n fp32 elements, 4-byte aligned (may be NULL
 *         when n = 0); y may equal x, other overlaps are not allowed.
 * Errors: TIDE_ERR_INVALID, TIDE_ERR_ALIGN, TIDE_ERR_RANGE, TIDE_ERR_HIP.
 */
tide_status tide_victim_axpb(const float* x, float* y, int64_t n, float a, float b, void* stream);

/*
 * A stream of default priority for the current device.  cu_mask NULL: an
 * ordinary non-blocking stream.  Otherwise the stream's kernels may only use
 * the CUs whose bits are set (bit i of cu_mask[i / 32] is the runtime's CU i;
 * mask_words >= ceil(cu_count / 32), at least one bit set): a hard CU budget,
 * where tide_options.cu_budget only limits the grid.  *out_stream receives a
 * hipStream_t, to be freed with tide_stream_destroy.
 * Errors: TIDE_ERR_INVALID, TIDE_ERR_HIP.
 */
tide_status tide_stream_create(const uint32_t* cu_mask, int32_t mask_words, void** out_stream);
tide_status tide_stream_destroy(void* stream); /* NULL is accepted */

/* Free a plan and its device tables (waits for the device to finish using
 * them).  NULL is accepted. */
void tide_plan_destroy(tide_plan* plan);

/* Message describing the calling thread's last failure ("" if none). */
const char* tide_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TIDE_H */
