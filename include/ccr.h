/*
 * ccr.h -- C ABI of the MI355X ring all-reduce hot path.
 *
 * R "virtual ranks" live as R separate device buffers in one GPU's HBM.  A
 * collective over them is executed the way a ring collective runs across R
 * GPUs: as a sequence of point-to-point hops, each hop a separate pass over
 * memory.  The reduce runs on compute units; copies run either as a
 * compute-unit kernel or on the SDMA engines (no compute units).
 *
 * Source of the method: "HOCCL: Offloading Collective Communication from GPU
 * Cores to Accelerate Distributed Training" (Fei et al.).  HOCCL moves copies
 * off the GPU cores onto DMA engines (Abstract; §2.3 DMA Engines; Fig. 1c),
 * keeps reductions on the cores (§5 Limitations), orders communication
 * against surrounding kernels on the caller's stream (§3.2 Stream Manager),
 * stages P2P transfers through a pool of chunk slots (§3.3.1, Fig. 4/5a) and
 * expresses collectives as P2P flows (§3.4, Fig. 6).  The ring itself is the
 * textbook ring: rank q sends to rank q+1 (mod R); reduce-scatter hop k makes
 * every rank q add chunk (q-k-2) mod R of rank q-1 into its own copy;
 * all-gather hop k copies chunk (q-k-1) mod R from rank q-1.
 *
 * Conventions shared by every entry point:
 *   - Return value: CCR_OK, or an error code with a message available from
 *     ccr_last_error() on the same thread.  No entry point aborts or prints.
 *   - Device pointers are caller-owned, must stay valid and unmodified until
 *     the work enqueued on `stream` completes, and must be 16-byte aligned.
 *     A buffer the call reads or writes zero bytes of is never accessed and
 *     may be NULL (an empty tensor).
 *     Host arrays of pointers or counts are read during the call only.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous unless stated otherwise: they return
 *     once the work is enqueued; any side stream the library uses is joined
 *     back into `stream` before return, so later work on `stream` sees the
 *     results (HOCCL §3.2: communication keeps operator order on the stream).
 *   - A count of zero is a successful no-op.
 *   - A context is bound to one device and must not be used from two host
 *     threads at once.
 *   - Some calls work through context-owned device scratch: the bf16
 *     all-reduce / reduce-scatter with fp32 partials, ccr_sendrecv (staging
 *     slots) and ccr_moe_plan (count scratch).  Two such calls on one
 *     context that are enqueued on different streams with nothing ordering
 *     them may run at the same time and race on that scratch; keep them on
 *     one stream or order the streams with events.  Every other call keeps
 *     no device state between launches.
 *   - That scratch grows on demand: the first call that needs more than the
 *     context holds allocates it, and when it replaces a smaller buffer it
 *     synchronises the device first (work still in flight may use the old
 *     one).  The fused MoE calls cycle through 4 segment-table slots and
 *     block the host until the call that last used their slot has finished.
 *     Warm a context up with its largest call before timing or capturing
 *     work around it.
 *   - HIP graphs: a call made of kernel launches only can be captured on a
 *     capturing stream and replayed (the ring collectives with kernel copies
 *     and per-hop bf16, with or without slices or overlap; ccr_alltoall,
 *     ccr_alltoall_rows, ccr_moe_dispatch and ccr_moe_combine with kernel
 *     copies; ccr_permute_rows; ccr_moe_topk).  A replay reuses the device
 *     pointers given at capture time.  Calls that would depend on context
 *     scratch that may be reallocated, on host memory copied at launch, or
 *     on the DMA proxy (SDMA copies, fp32 partials, ccr_sendrecv,
 *     ccr_sendrecv_batch, ccr_moe_plan, the fused MoE calls) return
 *     CCR_ERR_UNSUPPORTED while `stream` is capturing, and enqueue nothing;
 *     so does every call of a context with a CU budget, because a replay
 *     runs the captured kernels on the replaying stream's hardware queue,
 *     without the budget's CU mask.
 */
#ifndef CCR_H
#define CCR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CCR_OK = 0,
    CCR_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment, dtype, aliasing */
    CCR_ERR_UNSUPPORTED = 2, /* valid request the library cannot run        */
    CCR_ERR_HIP = 3,         /* a HIP runtime call failed                     */
    CCR_ERR_OOM = 4,         /* device or pinned-host allocation failed       */
    CCR_ERR_TIMEOUT = 5      /* a bounded wait expired                        */
} ccr_status_t;

typedef enum { CCR_F32 = 0, CCR_BF16 = 1 } ccr_dtype_t;

/* How copy hops (all-gather, staging, exchange) move bytes.
 * KERNEL: a compute-unit copy kernel on the caller's (or the CU-masked)
 * stream.  SDMA: the SDMA engines, no compute unit touches the data (HOCCL
 * Fig. 1c: DMA engine instead of SMs).  The copies are issued on the
 * device's SDMA engines by a CPU proxy thread that the stream hands each
 * operation to when it reaches it (HOCCL §3.2: the CPU takes over the
 * stream's coordination, with an explicit start request, finish and
 * acknowledgement); see ccr_dma_sync_t. */
typedef enum { CCR_COPY_KERNEL = 0, CCR_COPY_SDMA = 1 } ccr_copy_mode_t;

/* How an SDMA operation is tied to the stream (HOCCL §3.2: the CPU takes
 * over when the stream reaches the communication point, and the stream
 * continues once the copies are done).
 * HOST_FUNC (default): a hipLaunchHostFunc gate; the gate announces that
 *   the stream has arrived and returns when the proxy releases it after
 *   the copies, and the stream waits on the gate's completion without any
 *   GPU-side polling.
 * STREAM_FLAGS: stream memory operations on words in coherent host memory:
 *   the stream writes the operation's sequence number into a request word
 *   (hipStreamWriteValue32) and waits until the proxy's done word reaches
 *   it (hipStreamWaitValue32, >=); numbers only grow, so nothing is reset
 *   and nothing is acknowledged.  This HIP runtime executes those operations
 *   as kernels, and a stream waiting in hipStreamWaitValue32 for the length
 *   of a DMA slows concurrent compute by tens of percent, so it is kept for
 *   comparison only. */
typedef enum { CCR_DMA_SYNC_HOST_FUNC = 0, CCR_DMA_SYNC_STREAM_FLAGS = 1 } ccr_dma_sync_t;

/* bf16 reduce-scatter accumulation.  PER_HOP: every hop computes
 * bf16_rne(float(a) + float(b)); bf16 travels between ranks.
 * FP32_PARTIALS: the running partial travels in fp32 and is rounded to
 * bf16 once, at the last hop (R > 2; R = 2 has one hop, the same as
 * PER_HOP).  The context keeps 2 x R x chunk fp32 of scratch for the
 * partials; a hop then moves 8-10 bytes per element instead of 6. */
typedef enum { CCR_BF16_ACC_PER_HOP = 0, CCR_BF16_ACC_FP32_PARTIALS = 1 } ccr_bf16_acc_t;

typedef struct {
    int32_t copy_mode;           /* ccr_copy_mode_t                                 */
    int32_t cu_budget;           /* compute units the collective may use; 0 = all   */
    int32_t slices;              /* S >= 1 pipeline slices per ring chunk; they
                                    run separately only in an all-reduce whose
                                    all-gather overlaps (overlap = 1 or SDMA
                                    copies); otherwise a hop's slices run as one
                                    launch, with the same per-element order     */
    int32_t overlap;             /* 1: all-gather of slice s runs on a second stream
                                    while reduce-scatter continues with slice s+1   */
    int64_t staging_chunk_bytes; /* P2P staging chunk (multiple of 16)              */
    int32_t staging_slots;       /* number of staging slots (>= 1)                  */
    int32_t bf16_acc;            /* ccr_bf16_acc_t                                  */
    int32_t dma_stripe;          /* SDMA: engines each staging fill/drain is striped
                                    over; 0 = half the engines                      */
    int64_t dma_chunk_bytes;     /* SDMA: all-to-all flows are cut into chunks of at
                                    most this size (multiple of 16); 0 = automatic;
                                    raised if a job would need over 64 Ki chunks    */
    int32_t dma_sync;            /* ccr_dma_sync_t                                  */
    int32_t dma_engines;         /* SDMA: engines one call may use, 1..16 (the first
                                    of the usable ones); 0 = all.  Fewer engines
                                    move the copies at a lower rate: longer
                                    collectives, less traffic beside concurrent
                                    compute at any moment                          */
    int32_t graph_cache;         /* 1 (default): a ring collective of at most 2 MiB
                                    per rank and at least 12 hops (an all-reduce
                                    over 8 or more ranks, a reduce-scatter or
                                    all-gather over 13 or more) made of kernel
                                    launches only (kernel copies, no CU budget,
                                    no overlap, no fp32 partials) is captured
                                    into a HIP graph on its second call with the
                                    same buffers, count, dtype and operation,
                                    and replayed from then on (one host call
                                    instead of one launch per hop); arguments
                                    are still checked on every call.  0: always
                                    launch eagerly.  The context keeps up to 32
                                    graphs; replacing one of a full cache,
                                    ccr_ctx_set_config and ccr_ctx_destroy
                                    synchronise the device before destroying
                                    graphs.  See ccr_graph_cache_stats.        */
    int32_t dma_deadline_us;     /* SDMA: time one call's copies may take, in us;
                                    > 0: the call uses the fewest engines whose
                                    measured rate moves its copy bytes within
                                    that time (ccr_dma_pace; never more than
                                    dma_engines when that is set).  A staged
                                    ccr_sendrecv, once the context has completed
                                    one, uses the fewest engines for which
                                    chunks x (measured cost per chunk step +
                                    chunk / (stripe x rate)) fits, or all
                                    allowed engines when none does.  The rate is
                                    the engines' rate with nothing else running,
                                    so under concurrent load the copies can take
                                    longer.  0 (default): dma_engines alone
                                    decides                                    */
} ccr_config_t;

typedef struct ccr_ctx *ccr_ctx_t;

/* Fill *cfg with the defaults (kernel copies, all CUs, S = 1, no overlap,
 * 4 MiB x 2 staging slots, per-hop bf16, automatic SDMA striping and
 * chunking), then apply the environment overrides CCR_COPY_MODE
 * (kernel|sdma), CCR_CU_BUDGET, CCR_SLICES, CCR_OVERLAP, CCR_STAGING_CHUNK,
 * CCR_STAGING_SLOTS, CCR_BF16_ACC (per_hop|fp32_partials), CCR_DMA_STRIPE,
 * CCR_DMA_CHUNK, CCR_DMA_SYNC (host_func|stream_flags), CCR_DMA_ENGINES,
 * CCR_GRAPH_CACHE (0|1), CCR_DMA_DEADLINE_US.  HOCCL §4 switches backends by an
 * environment variable; this mirrors that.  (Read once per process and not part
 * of the configuration: CCR_NONTEMPORAL forces the streaming kernels' load mode,
 * 0 every access temporal, 1 every load and store non-temporal, 2 the incoming
 * operand's load non-temporal; unset, each call takes 2 when the buffers it
 * touches exceed the 256 MB last-level cache and 0 otherwise.) */
ccr_status_t ccr_config_default(ccr_config_t *cfg);

/* Create a context on HIP device `device`.  cfg NULL = ccr_config_default().
 * The context owns its side streams, events, staging slots, small device
 * scratch and -- from the first SDMA use on -- the DMA proxy thread and its
 * engine list (every engine is warmed with a small copy when the proxy
 * starts).  Side streams are CU-masked streams, each with a hardware queue
 * of its own (HOCCL §3.2: the stream manager runs communication on streams
 * of its own): the budgeted stream is made with the context when cu_budget
 * is set; a second one only when a call first overlaps an all-gather with
 * the next slice's reduce-scatter (overlap, or SDMA copies with slices > 1).
 * A context that needs neither holds no hardware queue of its own.  Makes
 * `device` current on the calling thread. */
ccr_status_t ccr_ctx_create(int device, const ccr_config_t *cfg, ccr_ctx_t *out);
/* Waits for the context's streams and SDMA operations, then frees
 * everything it owns.  An SDMA operation whose stream has not reached it
 * within CCR_DESTROY_TIMEOUT_MS (environment, default 10000) is abandoned:
 * its stream, when it gets there, goes on without the copies, and the call
 * returns CCR_ERR_TIMEOUT.  Copies still running after as long again are
 * left to finish: their streams are released, the memory they may write
 * (the staging slots) is kept, and CCR_ERR_TIMEOUT is returned.  The
 * context is gone in every case. */
ccr_status_t ccr_ctx_destroy(ccr_ctx_t ctx);
/* Replace the configuration.  Synchronises the context's streams first. */
ccr_status_t ccr_ctx_set_config(ccr_ctx_t ctx, const ccr_config_t *cfg);
ccr_status_t ccr_ctx_get_config(ccr_ctx_t ctx, ccr_config_t *cfg);

/* ----------------------------------------------------------------------
 * Ring schedule (host only, no device work).
 *
 * HOCCL §2.1 and Figure 1: the ring all-reduce as R-1 reduce-scatter steps
 * and R-1 all-gather steps, each rank sending one chunk to the next rank per
 * step; §3.3.1 cuts a chunk into slices (chunk pipelining).
 * One record per (hop, rank): the operation rank dst_rank performs in that
 * hop, on elements [lo, hi) of chunk `chunk`, reading rank src_rank's buffer.
 * phase 0 = reduce-scatter (dst += src), 1 = all-gather (dst = src).
 * Chunks are 16-byte aligned: with V = 16 / element size,
 * Lc = align_up(ceil(count / R), V), chunk c = [min(count, c*Lc),
 * min(count, (c+1)*Lc)); a chunk of length l is cut into S slices with
 * Ls = align_up(ceil(l / S), V) the same way.  Records come slice-major: for
 * each slice, the R-1 reduce-scatter hops, then the R-1 all-gather hops.
 * which: 0 = all-reduce, 1 = reduce-scatter only, 2 = all-gather only.
 * Writes at most max_ops records; *n_ops receives the full count (query the
 * size with ops = NULL, max_ops = 0).
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t phase, slice, step, dst_rank, src_rank, chunk;
    int64_t lo, hi;
} ccr_ring_op_t;

ccr_status_t ccr_ring_schedule(int R, int64_t count, int slices, int dtype, int which,
                               ccr_ring_op_t *ops, int64_t max_ops, int64_t *n_ops);

/* The workgroups of one ring-hop launch, as the kernel maps them (host only,
 * no device work; the kernel's index arithmetic, computed by the same
 * function on the host, for tests): one step of the ring of HOCCL §2.1,
 * Figure 1, as the device runs it.  Hop `step` of `phase` (0 = reduce-
 * scatter, 1 = all-gather) on slice `slice`, over the partition above.  The
 * launch has one workgroup per 2 x 256 16-byte vectors of each rank's
 * piece; per workgroup five int64: source rank, destination rank, byte
 * offset and byte length of its piece (the same in every rank buffer), and
 * the tile index within the piece.  Writes at most max_wg rows (rows holds
 * 5 * max_wg values); *n_wg receives the workgroup count (query with
 * rows = NULL, max_wg = 0).  CCR_ERR_UNSUPPORTED when the ring-hop kernel
 * does not take the hop (it then runs from a piece table). */
ccr_status_t ccr_ring_hop_layout(int R, int64_t count, int slices, int dtype, int phase, int step,
                                 int slice, int64_t *rows, int64_t max_wg, int64_t *n_wg);

/* ----------------------------------------------------------------------
 * Stage schedule of a collective's traffic (host only, no device work).
 *
 * HOCCL §3.4 (Collective Scheduler, Figure 6).  A collective over G GPUs is
 * an origin traffic matrix C: C[u*G + v] = bytes GPU u sends to GPU v
 * (int64, >= 0, at most 2^40; the diagonal is ignored).  node[u] (>= 0)
 * names u's scale-up domain; flows between nodes go over RDMA.  peer[u] is
 * u's symmetric peer in the same node (Figure 6 pairs 0-1 and 2-3; peers are
 * mutual: peer[peer[u]] == u), or -1 for none: an inter-node flow u -> v is sent as a forwarding copy on the
 * scale-up edge (u, peer[u]), the RDMA transfer, and a forwarding copy on
 * (peer[v], v) (Eq. 2).  1 <= G <= 256.  All arrays are host memory, read
 * during the call only.
 *
 * ccr_traffic_matrix: T = C with the forwarding copies added, T[u][peer u]
 *   = C[u][peer u] + (u's inter-node bytes) + (peer u's incoming inter-node
 *   bytes), T = C elsewhere, diagonal 0 (Eq. 3-5).  T: G*G int64.
 * ccr_schedule_stages: Algorithm 1 (Birkhoff-like decomposition).  Each
 *   stage takes a greedy matching of the inter-node flows with bytes left
 *   (by decreasing remainder, ties by (src, dst); at most one outgoing and
 *   one incoming per GPU, Eq. 8), moves the least remainder x on every
 *   matched flow, adds its forwarding copies, and fills the scale-up edges
 *   up to max(floor(x * bw_scaleup / bw_rdma), the largest forwarding load)
 *   with native components, which are greedy matchings peeled off each
 *   node's native traffic beforehand.  Native traffic left over forms
 *   further stages.  The stages sum to T (Eq. 7).  Bandwidths are integers
 *   in [1, 2^20] (any common unit, e.g. GB/s).
 *   entries: one record per (stage, kind, src, dst) with bytes > 0, sorted
 *   by those keys; kind 0 = RDMA flow, 1 = forwarding copy, 2 = native
 *   scale-up flow.  times[s]: the stage time of Eq. 9-10 as the exact ratio
 *   load / bw of the slowest domain.  At most max_entries / max_stages
 *   records are written; *n_entries and *n_stages receive the full counts
 *   (query them with NULL arrays and zero maxima).
 * Errors: CCR_ERR_INVALID_ARG for NULL arrays, G out of range, negative or
 * oversized bytes, a node id < 0, or a peer that is not -1 or another GPU of
 * the same node whose own peer is u.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t stage, kind, src, dst;
    int64_t bytes;
} ccr_stage_entry_t;

typedef struct {
    int64_t load, bw;
} ccr_stage_time_t;

ccr_status_t ccr_traffic_matrix(const int64_t *C, int G, const int32_t *node,
                                const int32_t *peer, int64_t *T);
ccr_status_t ccr_schedule_stages(const int64_t *C, int G, const int32_t *node,
                                 const int32_t *peer, int64_t bw_scaleup, int64_t bw_rdma,
                                 ccr_stage_entry_t *entries, int64_t max_entries,
                                 int64_t *n_entries, ccr_stage_time_t *times,
                                 int64_t max_stages, int64_t *n_stages);

/* ----------------------------------------------------------------------
 * Ring collectives, in place over R virtual ranks.
 * bufs: host array of R device pointers, each to `count` elements of dtype
 * (CCR_F32 or CCR_BF16); the R buffers must not overlap.  1 <= R <= 64.
 *
 * HOCCL composes every collective from point-to-point flows (§3.4,
 * Collective Scheduler, Fig. 6) and runs the reductions on the GPU cores
 * (§5 Limitations: reduction operators need core-side execution); the
 * pages describe no ring, so the ring here is the textbook one named at
 * the top of this file, each hop a pass over every rank's chunk.
 *
 * ccr_allreduce: every rank ends with the element-wise sum over all ranks.
 *   Element i of chunk c is reduced in the order the partial travels round
 *   the ring: ((x[c+1] + x[c+2]) + ... + x[c+R-1]) + x[c] (ranks mod R), so
 *   fp32 results are deterministic and independent of S, the CU budget and
 *   the copy mode.  bf16 follows the context's bf16_acc.
 * ccr_reduce_scatter: afterwards chunk r of bufs[r] holds the reduced chunk
 *   r; the other chunks hold partial sums.
 * ccr_all_gather: on entry chunk r of bufs[r] is rank r's contribution;
 *   afterwards every buffer holds all R chunks.  A pure copy (HOCCL §6.2,
 *   Fig. 8a-b measures AllGather as a DMA copy workload).
 * Errors: CCR_ERR_INVALID_ARG for a NULL or misaligned pointer, a buffer
 * that does not hold count elements, overlapping ranks, R or dtype out of
 * range; CCR_ERR_UNSUPPORTED for a call that cannot be captured while
 * `stream` is capturing (see the conventions above); CCR_ERR_HIP / OOM for
 * runtime failures.  Nothing is enqueued when an error is returned.
 * ---------------------------------------------------------------------- */
ccr_status_t ccr_allreduce(ccr_ctx_t ctx, void *const *bufs, int R, int64_t count,
                           int dtype, void *stream);
ccr_status_t ccr_reduce_scatter(ccr_ctx_t ctx, void *const *bufs, int R, int64_t count,
                                int dtype, void *stream);
ccr_status_t ccr_all_gather(ccr_ctx_t ctx, void *const *bufs, int R, int64_t count,
                            int dtype, void *stream);

/* ----------------------------------------------------------------------
 * Point-to-point transfers through the context's staging pool (HOCCL
 * §3.3.1 DMA-RNIC chunk pipelining; the slot states of Fig. 4).  A transfer
 * is cut into staging_chunk_bytes chunks; chunk i (counted over all of the
 * call's transfers in order) is copied into slot i mod staging_slots
 * (filling) and out of it (draining), and a slot is refilled only after it
 * has drained.  SDMA copies: the DMA proxy runs each slot's state machine,
 * fills and drains on different engines, so they overlap.  Kernel copies:
 * rounds of staging_slots chunks on one stream; one launch drains each
 * slot's chunk of the previous round to the receiver and refills the slot
 * with this round's chunk (each thread reads its part of the slot before
 * overwriting it), so a transfer of T chunks takes ceil(T / staging_slots)
 * + 1 launches (both stages share the compute units and HBM, so running
 * them apart would overlap nothing).  The buffers of one call must not
 * overlap.  The staging slots are context scratch (see the conventions).
 *
 * ccr_sendrecv: the ring shift over R ranks (HOCCL §3.4 group Send/Recv):
 *   recv[(r + 1) % R] <- send[r] for every r, `count` elements of dtype
 *   each, transfers in the order r = 0..R-1.  R = 2 is a pipeline pair
 *   exchanging in both directions.  send, recv: host arrays of R device
 *   pointers.  count * element size must be a multiple of 16.
 * ccr_sendrecv_batch: n transfers in one direction, recv[m] <- send[m],
 *   nbytes each (a multiple of 16), in the order m = 0..n-1: the micro-
 *   batches one pipeline stage sends the next.
 * Errors as for the ring collectives; CCR_ERR_OOM when the staging pool
 * cannot be allocated (nothing is enqueued; a smaller pool works again).
 * ---------------------------------------------------------------------- */
ccr_status_t ccr_sendrecv(ccr_ctx_t ctx, const void *const *send, void *const *recv, int R,
                          int64_t count, int dtype, void *stream);
ccr_status_t ccr_sendrecv_batch(ccr_ctx_t ctx, const void *const *send, void *const *recv, int n,
                                int64_t nbytes, void *stream);
/* ccr_sendrecv_batch for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * transfers, arguments, order and errors, but the staging slots live in a
 * fixed device array of 16 MiB per GPU that the library holds from its
 * first context on that GPU until the process ends, so the call allocates
 * no device or pinned memory and creates no stream or event.  Limits:
 * staging_slots x staging_chunk_bytes <= 16 MiB (CCR_ERR_INVALID_ARG
 * otherwise); kernel copies only (CCR_ERR_UNSUPPORTED with copy_mode SDMA,
 * whose proxy allocates when it starts).  It may be captured into a graph.
 * Every call on one GPU, from any context, shares that GPU's array: calls
 * that can overlap on the GPU (different streams with nothing ordering
 * them) race on it.  The array keeps the last call's contents; no call
 * needs it cleared. */
ccr_status_t ccr_sendrecv_batch_noalloc(ccr_ctx_t ctx, const void *const *send,
                                        void *const *recv, int n, int64_t nbytes, void *stream);

/* ----------------------------------------------------------------------
 * All-to-all over R ranks (HOCCL §6.2, Fig. 8c-d All-to-All; §2.1: the
 * expert-parallel dispatch and combine are all-to-all traffic).  Every
 * (source, destination) segment is its own flow; with SDMA copies the
 * flows are cut into chunks interleaved by size (§3.4).
 *
 * ccr_alltoall: send[r] holds `count` elements of dtype, its segments for
 *   d = 0..R-1 contiguous in destination order; recv[d] receives its
 *   segments contiguously in source order r = 0..R-1.  counts: host int64
 *   [R*R], counts[r*R + d] = elements r sends to d (each row summing to
 *   count), or NULL for count / R to every rank.  Every segment must be a
 *   whole number of 16-byte vectors, and recv[d] must hold the elements it
 *   receives (count, when counts is NULL).
 * ccr_alltoall_rows: the same exchange counted in rows of row_bytes (a
 *   multiple of 16): counts[r*R + d] rows from r to d (the form the MoE
 *   calls use, rows being tokens).
 * Errors as for the ring collectives, and CCR_ERR_INVALID_ARG for a negative
 * count, a row of counts that does not sum to count, or a ragged segment.
 * ---------------------------------------------------------------------- */
ccr_status_t ccr_alltoall(ccr_ctx_t ctx, const void *const *send, void *const *recv, int R,
                          int64_t count, const int64_t *counts, int dtype, void *stream);
ccr_status_t ccr_alltoall_rows(ccr_ctx_t ctx, const void *const *send, void *const *recv, int R,
                               const int64_t *counts, int64_t row_bytes, void *stream);

/* dst row i = src row d_idx[i], for i < nrows (the row gather of the MoE
 * pack and unpack: tokens placed by destination and expert before the
 * all-to-all, HOCCL §2.1).  d_idx: device int32, each entry in [0, nsrc);
 * nsrc, the rows src holds, bounds the indices, and an out-of-range entry
 * leaves that dst row unwritten (the indices live on the device, so no
 * error is returned for it).  dst must not overlap src. */
ccr_status_t ccr_permute_rows(ccr_ctx_t ctx, void *dst, const void *src, const int32_t *d_idx,
                              int64_t nrows, int64_t nsrc, int64_t row_bytes, void *stream);

/* ----------------------------------------------------------------------
 * Expert-parallel MoE dispatch and combine over R ranks (HOCCL §2.1: EP
 * dispatch/combine are all-to-all traffic).  Expert e lives on rank
 * e / (E/R) as local expert e % (E/R).
 *
 * ccr_moe_topk: topk[t*K + k] = the K experts with the largest logits of
 *   token t (device fp32 [T x E]), by decreasing logit, ties to the lower
 *   expert id.  Softmax is monotone, so this is also the top-K of the
 *   softmax.  E <= 1024, K <= min(E, 16).
 * ccr_moe_plan: one source rank's dispatch plan from its topk.  Rows are
 *   packed in (destination rank, local expert, token) order.
 *   src_tok[j] (device int32 [T*K]) = token carried by packed row j;
 *   slot[t*K + k] (device int32 [T*K]) = packed row that carries (t, k);
 *   h_ecnt (host int64 [E]) = rows for each expert.  Blocking: the counts
 *   are copied back to the host, because the exchange is sized on the host
 *   (DMA engines are driven from the CPU, HOCCL §1, §2.3).
 * ccr_moe_dispatch: pack (send[r] row j = x[r] row src_tok[r][j]), exchange
 *   (all-to-all, segments by destination), unpack (exp[d] rows ordered by
 *   local expert, then source rank, then token).  h_ecnt: host int64
 *   [R*E] (row r = ccr_moe_plan's counts of rank r).  Every rank sends
 *   T*K rows of row_bytes; send/recv/exp[r] must each hold the rows it gets.
 *   A buffer the call writes (send, recv, exp) must not overlap any other
 *   buffer of the call, src_tok included.
 * ccr_moe_combine: the exact inverse; out[r] is [T x K x row_bytes] with
 *   out[r] row (t, k) = the expert row that carried token t's k-th choice.
 *   Written buffers (recv, send, out) must not overlap any other buffer of
 *   the call, slot included.
 * ---------------------------------------------------------------------- */
ccr_status_t ccr_moe_topk(ccr_ctx_t ctx, const float *logits, int32_t *topk, int64_t T, int E,
                          int K, void *stream);
ccr_status_t ccr_moe_plan(ccr_ctx_t ctx, const int32_t *topk, int64_t T, int E, int K, int R,
                          int32_t *src_tok, int32_t *slot, int64_t *h_ecnt, void *stream);
ccr_status_t ccr_moe_dispatch(ccr_ctx_t ctx, const void *const *x, const int32_t *const *src_tok,
                              const int64_t *h_ecnt, int R, int64_t T, int E, int K,
                              int64_t row_bytes, void *const *send, void *const *recv,
                              void *const *exp, void *stream);
ccr_status_t ccr_moe_combine(ccr_ctx_t ctx, const void *const *exp, const int32_t *const *slot,
                             const int64_t *h_ecnt, int R, int64_t T, int E, int K,
                             int64_t row_bytes, void *const *recv, void *const *send,
                             void *const *out, void *stream);

/* Fused variants: the same results without the packed send or receive
 * buffers.  Each row moves once, directly between x[r] (or out[r]) and its
 * place in the destination's expert-major buffer exp[d] -- the pack, the
 * exchange and the unpack in one gather on the compute units (a one-GPU
 * stand-in for writing each row straight into the peer's receive buffer,
 * HOCCL §3.3.2's direct path).  2 bytes of traffic per payload byte instead
 * of 6.  exp[d] holds the same rows in the same order as ccr_moe_dispatch
 * gives; ccr_moe_combine_fused's out equals ccr_moe_combine's.  The copy mode
 * does not apply (row gathers run on compute units).  A buffer the call
 * writes (exp for dispatch, out for combine) must not overlap any other
 * buffer of the call, the index arrays included.  The segment table (R records of 16 bytes and R*E of
 * 24) is copied to the device on `stream`.  Arguments and errors as for
 * ccr_moe_dispatch / ccr_moe_combine; indices out of range leave their row
 * unwritten. */
ccr_status_t ccr_moe_dispatch_fused(ccr_ctx_t ctx, const void *const *x,
                                    const int32_t *const *src_tok, const int64_t *h_ecnt, int R,
                                    int64_t T, int E, int K, int64_t row_bytes, void *const *exp,
                                    void *stream);
ccr_status_t ccr_moe_combine_fused(ccr_ctx_t ctx, const void *const *exp,
                                   const int32_t *const *slot, const int64_t *h_ecnt, int R,
                                   int64_t T, int E, int K, int64_t row_bytes, void *const *out,
                                   void *stream);

/* ----------------------------------------------------------------------
 * Diagnostics.
 * ---------------------------------------------------------------------- */
/* SDMA engines the context's DMA proxy uses (starts the proxy if needed):
 * *n = engine count, ids[0..*n) = HSA engine indices (ids may be NULL;
 * room for 16). */
ccr_status_t ccr_dma_info(ccr_ctx_t ctx, int32_t *n, int32_t *ids);

/* Slot transitions of the context's most recent SDMA staged transfer
 * (ccr_sendrecv with copy_mode SDMA), in the order the proxy made them:
 * out[3*i] = chunk, out[3*i+1] = slot, out[3*i+2] = new state (0 idle,
 * 1 filling, 2 draining).  Synchronises with the proxy first.  Writes at
 * most max_events records; *n receives the full count. */
ccr_status_t ccr_sendrecv_slot_log(ccr_ctx_t ctx, int32_t *out, int64_t max_events, int64_t *n);

/* Wait up to timeout_ms for all work enqueued on `stream` to complete.
 * Returns CCR_ERR_TIMEOUT if it has not (the work keeps running), or
 * CCR_ERR_HIP with the proxy's message if the DMA proxy reported an error. */
ccr_status_t ccr_stream_wait(ccr_ctx_t ctx, void *stream, int timeout_ms);

/* SDMA pacing from a time budget (host only, touches no device): the
 * fewest engines whose combined rate moves `bytes` within `deadline_us`,
 * ceil(bytes / (deadline_us * 1e-6 * engine_gbs * 1e9)), at least 1 and at
 * most max_engines.  Returns max_engines when deadline_us <= 0,
 * engine_gbs <= 0 or bytes <= 0 would leave nothing to pace, and 0 when
 * max_engines < 1.  HOCCL §3.3.1 spreads a transfer over several queues to
 * raise its rate; this picks how many from the time it may take, so that
 * copies that are not waited on keep their HBM traffic beside concurrent
 * compute low. */
int32_t ccr_dma_pace(int64_t bytes, int64_t deadline_us, double engine_gbs, int32_t max_engines);

/* The context's SDMA pacing figures.  *engine_gbs: one engine's
 * device-to-device copy rate in GB/s, measured when the DMA proxy starts (a
 * 16 MiB copy on the first usable engine, nothing else running).
 * *last_engines: the engines the context's most recent SDMA job was allowed
 * (0 before any).  Starts the DMA proxy if it is not running. */
ccr_status_t ccr_dma_rate(ccr_ctx_t ctx, double *engine_gbs, int32_t *last_engines);

/* Fault injection for watchdog tests: the DMA proxy holds every
 * operation's release for `us` microseconds after its copies complete
 * (0 = off).  The stream is always released in the end. */
ccr_status_t ccr_dma_hold_finish(ccr_ctx_t ctx, int us);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char *ccr_last_error(void);
/* Library version string. */
const char *ccr_version(void);
/* Launch nblocks one-wave workgroups on the context's compute stream (the
 * CU-masked one when cu_budget is set) and write, per workgroup, the
 * hardware ids of the compute unit it ran on: out[3*b] = XCC id,
 * out[3*b+1] = shader engine id, out[3*b+2] = CU id.  out: device int32
 * [3*nblocks].  Used to show which compute units a CU budget leaves to the
 * collective. */
ccr_status_t ccr_probe_cu_ids(ccr_ctx_t ctx, int32_t *out, int nblocks, void *stream);
/* Streams the context holds now: *masked = CU-masked side streams (each
 * with a hardware queue of its own), *plain = plain streams (sharing the
 * runtime's queue pool; the graph cache's capture stream).  Host only;
 * either pointer may be NULL. */
ccr_status_t ccr_ctx_streams(ccr_ctx_t ctx, int32_t *masked, int32_t *plain);
/* The context's graph cache (ccr_config_t.graph_cache): *graphs = captured
 * graphs it holds now, *replays = ring calls served by a replay since the
 * context was created.  Host only; either pointer may be NULL. */
ccr_status_t ccr_graph_cache_stats(ccr_ctx_t ctx, int64_t *graphs, int64_t *replays);

/* Per-launch timing of the collectives' own kernels and SDMA copies.
 * While enabled, every reduce launch, copy launch and SDMA copy issued by
 * the ring collectives, ccr_sendrecv and ccr_alltoall is bracketed by a pair
 * of timing events recorded on the stream it runs on.  ccr_profile_read
 * synchronises the context's streams and the device, then reports, for
 * `kind` (0 = reduce kernels, 1 = copy kernels, 2 = SDMA copies,
 * 3 = reduce-and-forward kernels, the last reduce-scatter hop of an
 * all-reduce, 4 = fused MoE gathers, 2 bytes per byte of
 * payload), the number of launches since the last
 * enable, the sum of their durations in milliseconds, and their algorithmic
 * bytes (a reduce moves 3 bytes per byte of payload: read local, read
 * incoming, write local; reduce-and-forward 4; a copy 2; a staging
 * drain-and-fill, counted with the copy kernels, 4).  Kernel launches
 * are timed by events attached to the launch itself (hipExtLaunchKernel),
 * SDMA copies by events recorded around them.  Enabling (on = 1) also
 * clears the counters. */
typedef struct {
    int64_t launches;
    int64_t bytes;
    double ms;
} ccr_kernel_stats_t;

ccr_status_t ccr_profile_enable(ccr_ctx_t ctx, int on);
ccr_status_t ccr_profile_read(ccr_ctx_t ctx, int kind, ccr_kernel_stats_t *out);

/* The timed launches of `kind` (as for ccr_profile_read) since profiling
 * was enabled, one record each, in issue order: start_ms[i] and end_ms[i]
 * relative to `ref_event` (a hipEvent_t with timing, recorded on the
 * context's device and complete), and cus[i] = the compute units the
 * launch can hold at once: one per workgroup, at most the CUs the context's
 * budget allows (0 for SDMA copies).  With the intervals of the compute
 * kernels, this gives HOCCL's contention rate (Eq. 1: compute units held by
 * communication while compute kernels run, over all compute units).
 * Synchronises the device first.  Any of the three arrays may be NULL;
 * at most max records are written; *n receives the full count. */
ccr_status_t ccr_profile_intervals(ccr_ctx_t ctx, int kind, void *ref_event, double *start_ms,
                                  double *end_ms, int32_t *cus, int64_t max, int64_t *n);

#ifdef __cplusplus
}
#endif
#endif /* CCR_H */
