// Host runtime of the ring all-reduce hot path: context, argument checks,
// the ring chunk scheduler, and the stream manager that orders reduce
// kernels, copy kernels and SDMA copies against the caller's stream.
//
// Method: "HOCCL: Offloading Collective Communication from GPU Cores to
// Accelerate Distributed Training".  What is taken from it:
//  - copies may run on DMA (SDMA) engines instead of compute units
//    (Fig. 1c; §2.3 DMA Engines), while reductions stay on the compute units
//    (§5 Limitations);
//  - communication keeps its place in the caller's stream order relative
//    to the kernels before and after it (§3.2 Stream Manager); here events
//    between the caller's stream and the library's side streams do this;
//  - P2P transfers are staged through a pool of chunk slots whose fill and
//    drain overlap, each slot going idle -> filling -> draining -> idle
//    (§3.3.1 DMA-RNIC chunk pipelining; Fig. 4 state machine);
//  - a collective is a schedule of P2P flows, cut into chunks (§3.4).
// The ring order itself is the textbook ring (the paper describes none).

#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

#include "../../include/ccr.h"
#include "ccr_dma.h"
#include "ccr_internal.h"
#include "ccr_schedule.h"

using namespace ccr;

// ------------------------------------------------------------------ errors
namespace {

thread_local std::string g_last_error;

ccr_status_t fail(ccr_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ccr_status_t hip_fail(hipError_t e, const char* what) {
  (void)hipGetLastError();  // clear the sticky per-thread error
  return fail(e == hipErrorOutOfMemory ? CCR_ERR_OOM : CCR_ERR_HIP, "%s failed: %s (%d)", what,
              hipGetErrorString(e), (int)e);
}

#define HIP_TRY(expr)                                  \
  do {                                                 \
    hipError_t _e = (expr);                            \
    if (_e != hipSuccess) return hip_fail(_e, #expr);  \
  } while (0)

// A roctx range around each entry point: `rocprofv3 --marker-trace` shows
// every call's host span next to the kernels and copies it enqueued.
struct Mark {
  explicit Mark(const char* name) { roctxRangePushA(name); }
  ~Mark() { roctxRangePop(); }
  Mark(const Mark&) = delete;
  Mark& operator=(const Mark&) = delete;
};
#define CCR_MARK(name) Mark ccr_mark_(name)

#define CCR_TRY(expr)                    \
  do {                                   \
    ccr_status_t _s = (expr);            \
    if (_s != CCR_OK) return _s;         \
  } while (0)

constexpr int kMaxRanks = 64;
static_assert(kMaxRanks <= kMaxPieces, "one hop of every rank fits one launch");

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align_up(int64_t a, int64_t v) { return ceil_div(a, v) * v; }
int wrap(int a, int m) { return ((a % m) + m) % m; }

int dtype_size(int dtype) { return dtype == CCR_F32 ? 4 : dtype == CCR_BF16 ? 2 : 0; }

}  // namespace

// ----------------------------------------------------------------- context
struct ccr_ctx {
  int device = 0;
  int num_cus = 0;
  ccr_config_t cfg{};
  bool masked = false;          // a CU budget is set: s_a / s_b carry its mask
  // Side streams, each created with a CU mask (a hardware queue of its own):
  // s_a when a CU budget is set (created with the context), or on first use
  // by the CU-id probe; s_b when a call first needs a second stream (an
  // overlapped or SDMA all-gather of several slices).  s_cap: a plain stream
  // the graph cache captures on, created on the first capture.
  hipStream_t s_a = nullptr;    // reduce / fill / exchange side stream
  hipStream_t s_b = nullptr;    // all-gather (overlap, SDMA handshake) side stream
  hipStream_t s_cap = nullptr;
  std::unique_ptr<DmaProxy> dma;  // SDMA engines + CPU proxy, started on first SDMA use
  int last_dma_engines = 0;     // engines the most recent SDMA job was allowed
  int64_t footprint = 0;        // bytes of the buffers the current call touches
  std::vector<hipEvent_t> ev;   // event pool, grown on demand
  char* staging = nullptr;      // staging_slots x staging_chunk_bytes
  int64_t staging_bytes = 0;
  int64_t* d_ecnt = nullptr;    // MoE plan counts scratch
  int64_t d_ecnt_len = 0;
  int64_t* h_pinned = nullptr;  // pinned mirror of d_ecnt
  float* partials = nullptr;    // fp32 partials: 2 (hop parity) x R x chunk
  int64_t partials_bytes = 0;
  // Small per-call tables (fused MoE segment tables) go to the device
  // through a ring of pinned host / device buffer pairs; a slot is reused
  // only after the work of its previous call has completed.
  struct TableSlot {
    char* dev = nullptr;
    char* host = nullptr;
    int64_t cap = 0;
    hipEvent_t done = nullptr;
  };
  static constexpr int kTableSlots = 4;
  TableSlot tables[kTableSlots];
  int next_table = 0;
  // Small ring calls made of kernel launches only are captured once into a
  // graph and replayed (run_ring): one host call instead of 2(R-1) launches.
  struct RingGraph {
    std::vector<void*> bufs;
    int64_t count = 0;
    int dtype = 0, which = 0;
    int uses = 0;                   // calls seen with this key; < 0: never capture it
    uint64_t last = 0;              // tick of the last use (least recently used is replaced)
    hipGraphExec_t exec = nullptr;
  };
  static constexpr size_t kMaxRingGraphs = 32;
  std::vector<RingGraph> graphs;
  uint64_t graph_tick = 0;
  int64_t graph_replays = 0;
  // per-launch timing (ccr_profile_enable): event pairs and payload bytes
  bool prof_on = false;
  struct Timed {
    int kind;
    hipEvent_t start, stop;
    int64_t bytes;
    int32_t cus;  // compute units the launch can hold (0 for SDMA copies)
  };
  std::vector<Timed> timed;
  std::vector<hipEvent_t> timing_pool;
  std::string scratch_error;  // why the fixed scratch's address could not be resolved
};

namespace {

ccr_status_t check_config(const ccr_config_t* c) {
  if (c->copy_mode != CCR_COPY_KERNEL && c->copy_mode != CCR_COPY_SDMA)
    return fail(CCR_ERR_INVALID_ARG, "copy_mode %d is not kernel (0) or sdma (1)", c->copy_mode);
  if (c->cu_budget < 0) return fail(CCR_ERR_INVALID_ARG, "cu_budget %d < 0", c->cu_budget);
  if (c->slices < 1 || c->slices > 1024)
    return fail(CCR_ERR_INVALID_ARG, "slices %d outside [1, 1024]", c->slices);
  if (c->overlap != 0 && c->overlap != 1)
    return fail(CCR_ERR_INVALID_ARG, "overlap %d is not 0 or 1", c->overlap);
  if (c->staging_chunk_bytes <= 0 || c->staging_chunk_bytes % 16 != 0)
    return fail(CCR_ERR_INVALID_ARG, "staging_chunk_bytes %lld is not a positive multiple of 16",
                (long long)c->staging_chunk_bytes);
  if (c->staging_slots < 1 || c->staging_slots > 64)
    return fail(CCR_ERR_INVALID_ARG, "staging_slots %d outside [1, 64]", c->staging_slots);
  if (c->bf16_acc != CCR_BF16_ACC_PER_HOP && c->bf16_acc != CCR_BF16_ACC_FP32_PARTIALS)
    return fail(CCR_ERR_INVALID_ARG, "bf16_acc %d is not per_hop (0) or fp32_partials (1)",
                c->bf16_acc);
  if (c->dma_stripe < 0 || c->dma_stripe > 16)
    return fail(CCR_ERR_INVALID_ARG, "dma_stripe %d outside [0, 16]", c->dma_stripe);
  if (c->dma_chunk_bytes < 0 || c->dma_chunk_bytes % 16 != 0)
    return fail(CCR_ERR_INVALID_ARG, "dma_chunk_bytes %lld is not a non-negative multiple of 16",
                (long long)c->dma_chunk_bytes);
  if (c->dma_sync != CCR_DMA_SYNC_HOST_FUNC && c->dma_sync != CCR_DMA_SYNC_STREAM_FLAGS)
    return fail(CCR_ERR_INVALID_ARG, "dma_sync %d is not host_func (0) or stream_flags (1)",
                c->dma_sync);
  if (c->dma_engines < 0 || c->dma_engines > 16)
    return fail(CCR_ERR_INVALID_ARG, "dma_engines %d outside [0, 16]", c->dma_engines);
  if (c->graph_cache != 0 && c->graph_cache != 1)
    return fail(CCR_ERR_INVALID_ARG, "graph_cache %d is not 0 or 1", c->graph_cache);
  if (c->dma_deadline_us < 0)
    return fail(CCR_ERR_INVALID_ARG, "dma_deadline_us %d is negative", c->dma_deadline_us);
  return CCR_OK;
}

// Compute units of the CU mask for a budget of B: mask bit i is handed to
// XCC (i mod num_xcc) by the kernel-mode GPU driver, so the lowest B bits spread the budget
// evenly over the XCDs.
std::vector<uint32_t> cu_mask_for_budget(int budget, int num_cus) {
  std::vector<uint32_t> mask((size_t)(num_cus + 31) / 32, 0u);
  for (int i = 0; i < budget && i < num_cus; i++) mask[(size_t)i / 32] |= 1u << (i % 32);
  return mask;
}

ccr_status_t destroy_streams(ccr_ctx* ctx) {
  for (hipStream_t* p : {&ctx->s_a, &ctx->s_b, &ctx->s_cap})
    if (*p) HIP_TRY(hipStreamSynchronize(*p));
  for (hipStream_t* p : {&ctx->s_a, &ctx->s_b, &ctx->s_cap}) {
    if (*p) HIP_TRY(hipStreamDestroy(*p));
    *p = nullptr;
  }
  ctx->masked = false;
  return CCR_OK;
}

// A CU-masked side stream: the lowest cu_budget CUs, or all CUs without a
// budget.  A CU-masked stream gets a hardware queue of its own.  Plain
// streams share the runtime's few hardware queues round-robin, and a
// handshake wait or a join parked in a shared in-order queue would stall
// unrelated work (a concurrent GEMM) queued behind it.  Every such queue
// counts against the GPU's hardware scheduler (with about twenty of them,
// even idle, a lone GEMM ran 1.65x slower on MI355X), so the side streams
// are made only when a call needs them.
ccr_status_t masked_stream(ccr_ctx* ctx, hipStream_t* s) {
  if (*s) return CCR_OK;
  const int budget = ctx->cfg.cu_budget;
  const bool limited = budget > 0 && budget < ctx->num_cus;
  std::vector<uint32_t> mask = cu_mask_for_budget(limited ? budget : ctx->num_cus, ctx->num_cus);
  HIP_TRY(hipExtStreamCreateWithCUMask(s, (uint32_t)mask.size(), mask.data()));
  return CCR_OK;
}

ccr_status_t side_a(ccr_ctx* ctx, hipStream_t* out) {
  CCR_TRY(masked_stream(ctx, &ctx->s_a));
  *out = ctx->s_a;
  return CCR_OK;
}

ccr_status_t side_b(ccr_ctx* ctx, hipStream_t* out) {
  CCR_TRY(masked_stream(ctx, &ctx->s_b));
  *out = ctx->s_b;
  return CCR_OK;
}

// Streams for the context's configuration: with a CU budget, the budgeted
// stream every call runs on is made now, so calls need not create it.
ccr_status_t make_streams(ccr_ctx* ctx) {
  CCR_TRY(destroy_streams(ctx));
  const int budget = ctx->cfg.cu_budget;
  ctx->masked = budget > 0 && budget < ctx->num_cus;
  if (ctx->masked) CCR_TRY(masked_stream(ctx, &ctx->s_a));
  return CCR_OK;
}

ccr_status_t events(ccr_ctx* ctx, size_t n) {
  while (ctx->ev.size() < n) {
    hipEvent_t e;
    HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    ctx->ev.push_back(e);
  }
  return CCR_OK;
}

// Make `to` wait for everything enqueued on `from` so far.
ccr_status_t order_after(ccr_ctx* ctx, size_t ev_index, hipStream_t from, hipStream_t to) {
  if (from == to) return CCR_OK;
  CCR_TRY(events(ctx, ev_index + 1));
  HIP_TRY(hipEventRecord(ctx->ev[ev_index], from));
  HIP_TRY(hipStreamWaitEvent(to, ctx->ev[ev_index], 0));
  return CCR_OK;
}

// A call whose work depends on context scratch that may be reallocated, on
// host memory copied at launch time, or on the DMA proxy (a job runs once)
// cannot be replayed from a graph: refuse it while `s` is being captured.
ccr_status_t refuse_capture(hipStream_t s, const char* what) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  HIP_TRY(hipStreamIsCapturing(s, &st));
  if (st != hipStreamCaptureStatusNone)
    return fail(CCR_ERR_UNSUPPORTED, "%s cannot be captured into a graph", what);
  return CCR_OK;
}

// The stream a call's kernels run on: the budgeted side stream when a CU
// budget is set, else the caller's.  A budgeted call is refused while the
// caller's stream is capturing: a graph replay runs the captured kernels on
// the replaying stream's hardware queue, without the budget's CU mask (a
// probe captured with a 16-CU budget reached all 256 CUs when replayed).
ccr_status_t work_stream(ccr_ctx* ctx, hipStream_t caller, hipStream_t* s) {
  if (!ctx->masked) {
    *s = caller;
    return CCR_OK;
  }
  CCR_TRY(refuse_capture(caller, "a call with a CU budget (a replay would run without the CU mask)"));
  *s = ctx->s_a;
  return CCR_OK;
}

ccr_status_t check_ctx(ccr_ctx* ctx) {
  if (!ctx) return fail(CCR_ERR_INVALID_ARG, "ctx is NULL");
  HIP_TRY(hipSetDevice(ctx->device));
  return CCR_OK;
}

// A 16-byte aligned device pointer on this context's device whose next
// nbytes bytes lie inside one HIP allocation.
ccr_status_t check_dev_ptr(ccr_ctx* ctx, const void* p, int64_t nbytes, const char* what,
                           int index) {
  if (nbytes == 0) return CCR_OK;  // never dereferenced (an empty tensor may even be NULL)
  if (!p) return fail(CCR_ERR_INVALID_ARG, "%s[%d] is NULL", what, index);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(CCR_ERR_INVALID_ARG, "%s[%d] = %p is not 16-byte aligned", what, index, p);
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(CCR_ERR_INVALID_ARG, "%s[%d] = %p is not HIP memory", what, index, p);
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(CCR_ERR_INVALID_ARG, "%s[%d] = %p is not device memory", what, index, p);
  if (attr.device != ctx->device)
    return fail(CCR_ERR_INVALID_ARG, "%s[%d] = %p lives on device %d, not %d", what, index, p,
                attr.device, ctx->device);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(CCR_ERR_INVALID_ARG, "%s[%d] = %p: allocation range unknown", what, index, p);
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
  if (q < b || (uint64_t)nbytes > (uint64_t)(b + size - q))
    return fail(CCR_ERR_INVALID_ARG, "%s[%d] = %p: %lld bytes run past the end of its allocation",
                what, index, p, (long long)nbytes);
  return CCR_OK;
}

struct Range {
  uintptr_t lo, hi;
  int id;
};

ccr_status_t check_disjoint(std::vector<Range> r, const char* what) {
  // an empty range touches no byte and cannot conflict
  r.erase(std::remove_if(r.begin(), r.end(), [](const Range& x) { return x.hi <= x.lo; }), r.end());
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < r.size(); i++)
    if (r[i].lo < r[i - 1].hi)
      return fail(CCR_ERR_INVALID_ARG, "%s: buffers %d and %d overlap", what, r[i - 1].id,
                  r[i].id);
  return CCR_OK;
}

// ----------------------------------------------------------- ring schedule
// Chunk c of `count` elements over R ranks, 16-byte aligned (V elements).
void chunk_range(int64_t count, int R, int V, int c, int64_t* lo, int64_t* hi) {
  const int64_t L = align_up(ceil_div(count, R), V);
  *lo = std::min<int64_t>(count, (int64_t)c * L);
  *hi = std::min<int64_t>(count, (int64_t)(c + 1) * L);
}

// Slice s of the element range [clo, chi), cut into S aligned slices.
void slice_range(int64_t clo, int64_t chi, int S, int V, int s, int64_t* lo, int64_t* hi) {
  const int64_t len = chi - clo;
  const int64_t L = align_up(ceil_div(len, S), V);
  *lo = clo + std::min<int64_t>(len, (int64_t)s * L);
  *hi = clo + std::min<int64_t>(len, (int64_t)(s + 1) * L);
}

enum { kRS = 0, kAG = 1 };

// The R operations of one hop: rank q works on chunk (q-k-2) mod R for a
// reduce-scatter hop and chunk (q-k-1) mod R for an all-gather hop, reading
// rank q-1 (mod R).  Within a hop no chunk of any rank is both read and
// written, so the R operations run as one launch.
void hop_ops(int phase, int k, int s, int R, int64_t count, int S, int V,
             std::vector<ccr_ring_op_t>* out) {
  for (int q = 0; q < R; q++) {
    const int c = wrap(q - k - (phase == kRS ? 2 : 1), R);
    int64_t clo, chi, lo, hi;
    chunk_range(count, R, V, c, &clo, &chi);
    slice_range(clo, chi, S, V, s, &lo, &hi);
    out->push_back(ccr_ring_op_t{phase, s, k, q, wrap(q - 1, R), c, lo, hi});
  }
}

enum { kWhichAllreduce = 0, kWhichRS = 1, kWhichAG = 2 };

void ring_schedule(int R, int64_t count, int S, int V, int which,
                   std::vector<ccr_ring_op_t>* out) {
  for (int s = 0; s < S; s++) {
    if (which != kWhichAG)
      for (int k = 0; k + 1 < R; k++) hop_ops(kRS, k, s, R, count, S, V, out);
    if (which != kWhichRS)
      for (int k = 0; k + 1 < R; k++) hop_ops(kAG, k, s, R, count, S, V, out);
  }
}

LaunchTuning tuning() {
  // Overridable for tuning sweeps; defaults chosen by measurement.
  static LaunchTuning t = [] {
    // 2 x 16 B per operand per thread (best of 1/2/4/8 on gfx950); the
    // non-temporal mode is chosen per call (call_tuning) unless forced
    LaunchTuning x{2, -1, 0};
    if (const char* e = getenv("CCR_UNROLL")) x.unroll = atoi(e);
    if (const char* e = getenv("CCR_NONTEMPORAL")) x.nontemporal = atoi(e);
    if (const char* e = getenv("CCR_GRID")) x.grid = atoi(e);
    return x;
  }();
  return t;
}

// Load mode of a call's first reduce-scatter hop, whose operands were last
// written the longest time before (-1: the call's mode, as every other hop).
int first_hop_nontemporal() {
  static const int m = [] {
    const char* e = getenv("CCR_FIRST_HOP_NT");
    return e && *e ? atoi(e) : -1;
  }();
  return m;
}

// The MI355X's last-level cache (MALL, Infinity Cache) in front of HBM.
constexpr int64_t kMallBytes = int64_t(256) << 20;

// The launch tuning of one call.  A hop's incoming operand is read once and
// is dead afterwards.  When the call's buffers cannot stay in the MALL
// anyway, that load is non-temporal, so it does not displace the result,
// which the next hop reads (every hop kind of the 400 MiB bucket 5-8%
// faster).  When they fit, every access is temporal: the buffers stay
// cached from one call to the next, which a non-temporal load would undo
// (an 8-rank 4 MiB-per-rank all-reduce ran a third slower with it).
LaunchTuning call_tuning(const ccr_ctx* ctx) {
  LaunchTuning t = tuning();
  if (t.nontemporal < 0) t.nontemporal = ctx->footprint > kMallBytes ? 2 : 0;
  return t;
}

enum { kProfReduce = 0, kProfCopyKernel = 1, kProfSdma = 2, kProfReduceFwd = 3, kProfGather = 4 };

ccr_status_t timing_event(ccr_ctx* ctx, hipEvent_t* e) {
  if (!ctx->timing_pool.empty()) {
    *e = ctx->timing_pool.back();
    ctx->timing_pool.pop_back();
    return CCR_OK;
  }
  HIP_TRY(hipEventCreate(e));
  return CCR_OK;
}

// Bracket one launch with timing events when profiling is on.
struct TimedScope {
  ccr_ctx* ctx;
  hipStream_t s;
  int kind;
  int64_t bytes;
  hipEvent_t start = nullptr;
  ccr_status_t begin() {
    if (!ctx->prof_on) return CCR_OK;
    CCR_TRY(timing_event(ctx, &start));
    HIP_TRY(hipEventRecord(start, s));
    return CCR_OK;
  }
  ccr_status_t end() {
    if (!ctx->prof_on) return CCR_OK;
    hipEvent_t stop;
    CCR_TRY(timing_event(ctx, &stop));
    HIP_TRY(hipEventRecord(stop, s));
    ctx->timed.push_back(ccr_ctx::Timed{kind, start, stop, bytes, 0});  // SDMA: no compute unit
    return CCR_OK;
  }
};

// Compute units a launch of `workgroups` workgroups can hold at once: one
// per workgroup, at most the CUs the context's mask allows.
int32_t cus_held(const ccr_ctx* ctx, int64_t workgroups) {
  const int64_t allowed = ctx->cfg.cu_budget > 0 ? std::min(ctx->cfg.cu_budget, ctx->num_cus)
                                                 : ctx->num_cus;
  return (int32_t)std::max<int64_t>(0, std::min(allowed, workgroups));
}

int64_t payload(const Piece* p, size_t n) {
  int64_t b = 0;
  for (size_t i = 0; i < n; i++) b += p[i].nbytes;
  return b;
}

// A kernel launch; when profiling, its start/stop events are stamped by the
// dispatch itself (hipExtLaunchKernelGGL), so they time the kernel alone.
ccr_status_t launch_timed(ccr_ctx* ctx, HopKind kind, const Piece* p, int n, hipStream_t s,
                          int nt_override = -1) {
  LaunchTuning tune = call_tuning(ctx);
  if (nt_override >= 0) tune.nontemporal = nt_override;
  if (!ctx->prof_on) {
    HIP_TRY(launch_pieces(kind, p, n, tune, s));
    return CCR_OK;
  }
  const bool fwd = kind == HopKind::kReduceFwdF32 || kind == HopKind::kReduceFwdBf16;
  const bool reduce = fwd || kind == HopKind::kReduceF32 || kind == HopKind::kReduceBf16;
  const bool drain_fill = kind == HopKind::kDrainFill;
  hipEvent_t start, stop;
  CCR_TRY(timing_event(ctx, &start));
  CCR_TRY(timing_event(ctx, &stop));
  HIP_TRY(launch_pieces(kind, p, n, tune, s, start, stop));
  // algorithmic bytes: reduce reads 2 and writes 1 (forwarding writes 2),
  // copy reads 1 and writes 1, drain-and-fill reads 2 and writes 2, per byte
  // of payload
  // workgroups: one per kBlock x unroll 16-byte vectors of each piece
  const int64_t per_wg = (int64_t)kBlock * std::max(1, tune.unroll) * 16;
  int64_t wgs = 0;
  for (int i = 0; i < n; i++) wgs += (p[i].nbytes + per_wg - 1) / per_wg;
  if (tune.grid > 0) wgs = std::min<int64_t>(wgs, tune.grid);
  ctx->timed.push_back(ccr_ctx::Timed{fwd ? kProfReduceFwd : reduce ? kProfReduce : kProfCopyKernel,
                                      start, stop,
                                      payload(p, (size_t)n) * (fwd || drain_fill ? 4 : reduce ? 3 : 2),
                                      cus_held(ctx, wgs)});
  return CCR_OK;
}

// Ring hops go through launch_ring_hop (rank base addresses, one chunk
// geometry) unless CCR_RING_HOPS=table asks for the piece-table launch.
bool ring_hops_from_bases() {
  static const bool on = [] {
    const char* e = getenv("CCR_RING_HOPS");
    return !(e && strcmp(e, "table") == 0);
  }();
  return on;
}

// Hop k of `phase` on slice s as a RingHop: the operations hop_ops lists
// by rank, listed by chunk.  Rank q works on chunk c = q - k - 2 (reduce-
// scatter) or q - k - 1 (all-gather) and reads rank q - 1, so chunk c goes
// from rank c + k + 1 (resp. c + k) to the rank after it.  Chunks below
// count / L are whole and share slice s's offsets within a chunk; the chunk
// after them holds the ragged end (or nothing).
RingHop ring_hop_desc(int phase, int k, int s, int R, int64_t count, int S, int V, int esize,
                      void* const* bufs) {
  RingHop h;
  h.R = R;
  h.shift = (phase == kRS ? k + 1 : k) % R;
  const int64_t L = align_up(ceil_div(count, R), V);
  h.stride = L * esize;
  h.nfull = L > 0 ? (int)std::min<int64_t>(R, count / L) : 0;
  int64_t lo, hi;
  slice_range(0, L, S, V, s, &lo, &hi);
  h.full_off = lo * esize;
  h.full_len = (hi - lo) * esize;
  if (h.nfull < R) {
    int64_t clo, chi;
    chunk_range(count, R, V, h.nfull, &clo, &chi);
    slice_range(clo, chi, S, V, s, &lo, &hi);
    h.rag_c = h.nfull;
    h.rag_off = lo * esize;
    h.rag_len = (hi - lo) * esize;
  }
  // Full chunks in destination-rank order, as hop_ops lists them: from the
  // chunk the previous hop wrote last, whose tiles the caches most likely
  // still hold (on MI355X the bf16 bucket's all-reduce 2% faster than from
  // chunk 0; walking every other hop backwards instead was slower still).
  const int first = (2 * R - h.shift - 1) % R;
  h.rot = first < h.nfull ? first : 0;
  h.base = bufs;
  return h;
}

// One ring hop in the base-address form, timed like launch_timed; *done is
// false (and nothing is launched) when the form does not take the hop under
// the call's tuning, and the caller launches its pieces instead.
ccr_status_t ring_hop_timed(ccr_ctx* ctx, HopKind kind, const RingHop& h, hipStream_t s,
                            int nt_override, bool* done) {
  LaunchTuning tune = call_tuning(ctx);
  if (nt_override >= 0) tune.nontemporal = nt_override;
  *done = false;
  if (!ring_hops_from_bases() || tune.unroll != 2 || tune.grid > 0 ||
      !ring_hop_supported(h, kind, tune.nontemporal))
    return CCR_OK;
  *done = true;
  if (!ctx->prof_on) {
    HIP_TRY(launch_ring_hop(kind, h, tune.nontemporal, s));
    return CCR_OK;
  }
  const bool fwd = kind == HopKind::kReduceFwdF32 || kind == HopKind::kReduceFwdBf16;
  const bool reduce = fwd || kind == HopKind::kReduceF32 || kind == HopKind::kReduceBf16;
  hipEvent_t start, stop;
  CCR_TRY(timing_event(ctx, &start));
  CCR_TRY(timing_event(ctx, &stop));
  HIP_TRY(launch_ring_hop(kind, h, tune.nontemporal, s, start, stop));
  const int64_t payload_bytes = (int64_t)h.nfull * h.full_len + h.rag_len;
  ctx->timed.push_back(ccr_ctx::Timed{fwd ? kProfReduceFwd : reduce ? kProfReduce : kProfCopyKernel,
                                      start, stop, payload_bytes * (fwd ? 4 : reduce ? 3 : 2),
                                      cus_held(ctx, ring_hop_workgroups(h))});
  return CCR_OK;
}

// ------------------------------------------------------------- SDMA path
ccr_status_t ensure_dma(ccr_ctx* ctx) {
  if (ctx->dma) return CCR_OK;
  auto d = std::make_unique<DmaProxy>();
  std::string err;
  if (!d->start(ctx->device, &err)) return fail(CCR_ERR_HIP, "SDMA proxy: %s", err.c_str());
  ctx->dma = std::move(d);
  return CCR_OK;
}

// Engines one call that moves `bytes` over SDMA may use: the configured
// number, at most the usable ones, and with a deadline only as many as
// that time needs at the proxy's measured per-engine rate.
int dma_engine_limit(ccr_ctx* ctx, int64_t bytes) {
  const int n = ctx->dma->engine_count();
  int e = ctx->cfg.dma_engines > 0 ? std::min(ctx->cfg.dma_engines, n) : n;
  if (ctx->cfg.dma_deadline_us > 0)
    e = ccr_dma_pace(bytes, ctx->cfg.dma_deadline_us, ctx->dma->engine_gbs(), e);
  ctx->last_dma_engines = e;
  return e;
}

// All-gather links go to the least-loaded engine when issued, unless
// CCR_DMA_PLACE=static asks for the fixed placement.
bool any_engine_placement() {
  const char* place = getenv("CCR_DMA_PLACE");
  return !(place && strcmp(place, "static") == 0);
}

// Engines for a staged transfer of `chunks` chunks under the context's
// deadline, once a staged job has shown its fixed cost per chunk step: a
// transfer takes about chunks x (step cost + chunk / (stripe x rate)), its
// fills and drains each striped over `stripe` engines of their own (twice
// that when there are too few engines for both and they share them).  The
// fewest engines whose time fits, or every allowed one when none does; never
// fewer than ccr_dma_pace's count for the same bytes.
int staged_engines(ccr_ctx* ctx, int64_t chunks) {
  const ccr_config_t& c = ctx->cfg;
  const int n = ctx->dma->engine_count();
  const int emax = c.dma_engines > 0 ? std::min(c.dma_engines, n) : n;
  const double rate = ctx->dma->engine_gbs(), step = ctx->dma->staged_step_us();
  int e = emax;
  for (int k = 1; k <= emax && rate > 0; k++) {
    const int stripe = c.dma_stripe > 0 ? std::min(c.dma_stripe, k) : std::max(1, k / 2);
    const double share = k >= 2 * stripe ? 1.0 : 2.0;
    const double t_us =
        (double)chunks * share * (step + (double)c.staging_chunk_bytes / (stripe * rate * 1e3));
    if (t_us <= (double)c.dma_deadline_us) {
      e = k;
      break;
    }
  }
  ctx->last_dma_engines = e;
  return e;
}

ccr_status_t dma_submit(ccr_ctx* ctx, std::vector<DmaCopy> copies, hipStream_t s,
                        int max_engines = 0) {
  std::string err;
  if (!ctx->dma->submit_copies(std::move(copies), s, (DmaSync)ctx->cfg.dma_sync, &err, max_engines))
    return fail(CCR_ERR_HIP, "SDMA proxy: %s", err.c_str());
  return CCR_OK;
}

// Flow-size-aware chunk schedule (HOCCL §3.4): every flow is cut into
// chunks of at most C bytes and the chunks of all flows are interleaved so
// that each flow's share of engine service follows its size -- chunk j of a
// flow of n chunks gets the key (j + 0.5) / n and chunks are issued in key
// order, round-robin over the engines.  All flows progress together and
// finish together instead of a large flow holding an engine to the end.
// (Issued all at once, the key-ordered chunks are balanced by the round
// robin: placing each on the least-loaded engine instead made the 8-rank
// MoE exchange ~3% slower.)
std::vector<DmaCopy> flow_chunks(const std::vector<Piece>& flows, int64_t C, int engines) {
  struct Key {
    double key;
    size_t flow;
    int64_t j;
  };
  std::vector<Key> keys;
  for (size_t f = 0; f < flows.size(); f++) {
    const int64_t n = (flows[f].nbytes + C - 1) / C;
    for (int64_t j = 0; j < n; j++) keys.push_back(Key{(j + 0.5) / (double)n, f, j});
  }
  std::stable_sort(keys.begin(), keys.end(),
                   [](const Key& a, const Key& b) { return a.key < b.key; });
  std::vector<DmaCopy> out;
  out.reserve(keys.size());
  for (size_t i = 0; i < keys.size(); i++) {
    const Piece& f = flows[keys[i].flow];
    const int64_t lo = keys[i].j * C, hi = std::min<int64_t>(f.nbytes, lo + C);
    out.push_back(DmaCopy{f.dst + lo, f.src + lo, hi - lo, -1, (int32_t)(i % (size_t)engines)});
  }
  return out;
}

// Automatic chunk size for a DMA job: about 8 chunks per engine, kept
// within [256 KiB, 16 MiB].
int64_t auto_chunk(int64_t total, int engines) {
  int64_t c = total / std::max(1, 8 * engines);
  c = std::max<int64_t>(256 << 10, std::min<int64_t>(16 << 20, c));
  return (c + 15) & ~int64_t(15);
}

// fp32-partials hop; algorithmic bytes per element: read local bf16 (2) and
// incoming (2 bf16 / 4 fp32), write the partial (4 fp32) or the result
// (2 bf16, twice when forwarding).
ccr_status_t launch_partials_timed(ccr_ctx* ctx, PartialKind kind, const PartialPiece* p, int n,
                                   hipStream_t s) {
  // the first hop's operands stream like the other hops' incoming ones when
  // the call's buffers exceed the MALL
  const bool nt_first = call_tuning(ctx).nontemporal != 0;
  if (!ctx->prof_on) {
    HIP_TRY(launch_partials(kind, p, n, nt_first, s));
    return CCR_OK;
  }
  int64_t elems = 0;
  for (int i = 0; i < n; i++) elems += p[i].n;
  const int per = kind == PartialKind::kFirst ? 8 : kind == PartialKind::kMid ? 10
                  : kind == PartialKind::kLast ? 8 : 10;
  hipEvent_t start, stop;
  CCR_TRY(timing_event(ctx, &start));
  CCR_TRY(timing_event(ctx, &stop));
  HIP_TRY(launch_partials(kind, p, n, nt_first, s, start, stop));
  ctx->timed.push_back(ccr_ctx::Timed{kProfReduce, start, stop, elems * per,
                                      cus_held(ctx, (elems + 8 * kBlock * 2 - 1) / (8 * kBlock * 2))});
  return CCR_OK;
}

ccr_status_t ensure_partials(ccr_ctx* ctx, int64_t bytes) {
  if (ctx->partials && ctx->partials_bytes >= bytes) return CCR_OK;
  if (ctx->partials) {
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipFree(ctx->partials));
    ctx->partials = nullptr;
    ctx->partials_bytes = 0;
  }
  HIP_TRY(hipMalloc(reinterpret_cast<void**>(&ctx->partials), (size_t)bytes));
  ctx->partials_bytes = bytes;
  return CCR_OK;
}

// Copy `n` pieces on `s` with the copy kernel, kMaxPieces per launch.
ccr_status_t copy_pieces(ccr_ctx* ctx, const Piece* p, size_t n, hipStream_t s) {
  for (size_t i = 0; i < n; i += kMaxPieces) {
    const int m = (int)std::min<size_t>(kMaxPieces, n - i);
    CCR_TRY(launch_timed(ctx, HopKind::kCopy, p + i, m, s));
  }
  return CCR_OK;
}

// The all-gather of slice s as DMA copies.  Chunk c's copies form a chain
// (rank c -> c+1 -> ... -> c-1, one hop each).  Each chain is cut into m
// sub-chains over equal byte ranges (fewer if pieces would drop below
// 256 KiB).  By default (any_engine) m = ceil(E / R), just enough chains to
// keep the E engines busy, or more where links would exceed 8 MiB (so the
// last links of a large call leave no engine idle for long), and the DMA
// proxy issues each link on the
// least-loaded engine when it becomes ready: every SDMA copy carries a fixed
// cost of several microseconds on its engine, so fewer, larger links placed
// where an engine is free beat many small ones on fixed engines.  With fixed
// placement (CCR_DMA_PLACE=static) m = E / gcd(R, E), so the R*m chains
// spread evenly, and chain i runs on engine i mod E.  Hops before first_hop
// are already done (an all-reduce's last reduce-scatter hop forwards, which
// is hop 0).  Copies are listed hop by hop; each waits for the previous link
// of its chain, and the DMA proxy issues it when that link completes.
std::vector<DmaCopy> ag_chains(void* const* bufs, int R, int64_t count, int S, int s, int V,
                               int esize, int engines, int first_hop, bool any_engine) {
  const int E = std::max(1, engines);
  std::vector<int64_t> lo((size_t)R), hi((size_t)R);
  int64_t widest = 0;
  for (int c = 0; c < R; c++) {
    int64_t clo, chi;
    chunk_range(count, R, V, c, &clo, &chi);
    slice_range(clo, chi, S, V, s, &lo[(size_t)c], &hi[(size_t)c]);
    widest = std::max(widest, (hi[(size_t)c] - lo[(size_t)c]) * esize);
  }
  constexpr int64_t kMaxLink = int64_t(8) << 20;  // past this a link's fixed cost is ~1% of it
  int m = any_engine ? std::max<int64_t>((E + R - 1) / R, (widest + kMaxLink - 1) / kMaxLink)
                     : E / std::gcd(R, E);
  if (const char* e = getenv("CCR_DMA_SPLIT"); e && atoi(e) > 0) m = atoi(e);
  while (m > 1 && widest / m < (256 << 10)) m--;
  std::vector<DmaCopy> out;
  std::vector<int32_t> prev((size_t)R * m, -1);
  for (int k = first_hop; k + 1 < R; k++) {
    for (int c = 0; c < R; c++) {
      const int q = (c + 1 + k) % R, p = (q + R - 1) % R;
      const int64_t b0 = lo[(size_t)c] * esize, nb = (hi[(size_t)c] - lo[(size_t)c]) * esize;
      const int64_t part = ((nb + m - 1) / m + 15) & ~int64_t(15);
      for (int j = 0; j < m; j++) {
        const int64_t a = std::min(nb, j * part), z = std::min(nb, (j + 1) * part);
        if (z <= a) continue;
        const size_t chain = (size_t)c * m + j;
        out.push_back(DmaCopy{static_cast<char*>(bufs[q]) + b0 + a,
                              static_cast<const char*>(bufs[p]) + b0 + a, z - a, prev[chain],
                              any_engine ? -1 : (int32_t)(chain % (size_t)E)});
        prev[chain] = (int32_t)(out.size() - 1);
      }
    }
  }
  return out;
}

ccr_status_t enqueue_ring(ccr_ctx* ctx, void* const* bufs, int R, int64_t count, int dtype,
                          int which, hipStream_t caller);

// A graph replay has a fixed cost of its own on this runtime, so it pays only
// for a call of many small launches: measured on fp32 and bf16 rings, an
// 8-rank all-reduce (13 launches) at 0.5-2 MiB per rank takes 39-42 us per
// call instead of 46-49 (32-35 instead of 42-45 back to back), a 16-rank one
// at 0.5 MiB 80 instead of 96; with 5-7 launches, or from 4 MiB per rank on,
// replays are as slow as eager launches or slower.
constexpr int64_t kGraphMaxRankBytes = int64_t(2) << 20;
constexpr int kGraphMinLaunches = 12;

// A ring call is replayed from a graph when it is made of at least
// kGraphMinLaunches small launches on the caller's stream only (kernel
// copies, no CU budget, no overlap, no fp32 partials), is not profiled, and
// is not itself being captured.
bool ring_graph_eligible(ccr_ctx* ctx, int R, int64_t rank_bytes, int dtype, int which,
                         hipStream_t caller) {
  const ccr_config_t& c = ctx->cfg;
  const int launches = which == kWhichAllreduce ? 2 * R - 3 : R - 1;  // one per hop
  if (!c.graph_cache || ctx->prof_on || ctx->masked || c.overlap || rank_bytes > kGraphMaxRankBytes ||
      launches < kGraphMinLaunches)
    return false;
  if (c.copy_mode == CCR_COPY_SDMA && which != kWhichRS) return false;
  if (dtype == CCR_BF16 && which != kWhichAG && c.bf16_acc == CCR_BF16_ACC_FP32_PARTIALS) return false;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &st) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return st == hipStreamCaptureStatusNone;
}

// A graph is destroyed only after the device has drained: its last replay
// may still be running on any caller stream (an event recorded after every
// replay would cost each replay a gap on the GPU).  Replacing an entry of a
// full cache therefore synchronises the device once.
void drop_graph(ccr_ctx::RingGraph* g) {
  if (g->exec) {
    (void)hipDeviceSynchronize();
    (void)hipGraphExecDestroy(g->exec);
  }
  g->exec = nullptr;
}

void flush_graphs(ccr_ctx* ctx) {
  bool any = false;
  for (auto& g : ctx->graphs) any |= g.exec != nullptr;
  if (any) (void)hipDeviceSynchronize();
  for (auto& g : ctx->graphs)
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
  ctx->graphs.clear();
}

// The first call with a given (buffers, count, dtype, operation) runs
// eagerly; the second is captured on the context's own stream (the legacy
// default stream cannot be captured) and every call from then on replays
// the graph on the caller's stream.  Kernel arguments are captured by value,
// so a replay repeats exactly the launches of an eager call.
ccr_status_t run_ring_graph(ccr_ctx* ctx, void* const* bufs, int R, int64_t count, int dtype,
                            int which, hipStream_t caller, bool* launched) {
  ccr_ctx::RingGraph* g = nullptr;
  for (auto& e : ctx->graphs)
    if (e.count == count && e.dtype == dtype && e.which == which && (int)e.bufs.size() == R &&
        std::equal(e.bufs.begin(), e.bufs.end(), bufs)) {
      g = &e;
      break;
    }
  if (!g) {
    if (ctx->graphs.size() < ccr_ctx::kMaxRingGraphs) {
      ctx->graphs.emplace_back();
      g = &ctx->graphs.back();
    } else {
      g = &*std::min_element(ctx->graphs.begin(), ctx->graphs.end(),
                             [](const ccr_ctx::RingGraph& a, const ccr_ctx::RingGraph& b) {
                               return a.last < b.last;
                             });
      drop_graph(g);
      *g = ccr_ctx::RingGraph();
    }
    g->bufs.assign(bufs, bufs + R);
    g->count = count;
    g->dtype = dtype;
    g->which = which;
  }
  g->last = ++ctx->graph_tick;
  if (!g->exec && g->uses >= 0 && ++g->uses >= 2) {
    // A capture that the runtime refuses or cannot instantiate leaves this
    // key to eager launches for good (uses < 0); the call itself goes on.
    if (!ctx->s_cap && hipStreamCreateWithFlags(&ctx->s_cap, hipStreamNonBlocking) != hipSuccess) {
      (void)hipGetLastError();
      ctx->s_cap = nullptr;
      g->uses = -1;
      return CCR_OK;
    }
    hipStream_t cs = ctx->s_cap;
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      (void)hipGetLastError();
      g->uses = -1;
      return CCR_OK;
    }
    const ccr_status_t st = enqueue_ring(ctx, bufs, R, count, dtype, which, cs);
    const hipError_t e = hipStreamEndCapture(cs, &graph);
    if (st != CCR_OK || e != hipSuccess ||
        hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0) != hipSuccess) {
      (void)hipGetLastError();
      g->exec = nullptr;
      g->uses = -1;
    }
    if (graph) (void)hipGraphDestroy(graph);
  }
  if (!g->exec) return CCR_OK;  // first sight, or not capturable: the caller launches eagerly
  HIP_TRY(hipGraphLaunch(g->exec, caller));
  ctx->graph_replays++;
  *launched = true;
  return CCR_OK;
}

ccr_status_t run_ring(ccr_ctx* ctx, void* const* bufs, int R, int64_t count, int dtype,
                      int which, hipStream_t caller) {
  CCR_TRY(check_ctx(ctx));
  if (!bufs) return fail(CCR_ERR_INVALID_ARG, "bufs is NULL");
  if (R < 1 || R > kMaxRanks) return fail(CCR_ERR_INVALID_ARG, "R = %d outside [1, %d]", R, kMaxRanks);
  if (count < 0) return fail(CCR_ERR_INVALID_ARG, "count %lld < 0", (long long)count);
  const int esize = dtype_size(dtype);
  if (!esize) return fail(CCR_ERR_INVALID_ARG, "dtype %d is not f32 (0) or bf16 (1)", dtype);
  if (count == 0) return CCR_OK;
  std::vector<Range> ranges;
  for (int q = 0; q < R; q++) {
    CCR_TRY(check_dev_ptr(ctx, bufs[q], count * esize, "bufs", q));
    const uintptr_t p = reinterpret_cast<uintptr_t>(bufs[q]);
    ranges.push_back(Range{p, p + (uintptr_t)(count * esize), q});
  }
  CCR_TRY(check_disjoint(ranges, "bufs"));
  if (R == 1) return CCR_OK;
  if (ring_graph_eligible(ctx, R, count * esize, dtype, which, caller)) {
    bool launched = false;
    CCR_TRY(run_ring_graph(ctx, bufs, R, count, dtype, which, caller, &launched));
    if (launched) return CCR_OK;
  }
  return enqueue_ring(ctx, bufs, R, count, dtype, which, caller);
}

// The launches of a validated ring call, on `caller` (and the context's side
// streams, SDMA engines or scratch as the configuration asks).
ccr_status_t enqueue_ring(ccr_ctx* ctx, void* const* bufs, int R, int64_t count, int dtype,
                          int which, hipStream_t caller) {
  const int esize = dtype_size(dtype);
  const int V = 16 / esize;
  ctx->footprint = (int64_t)R * count * esize;
  const HopKind reduce = dtype == CCR_F32 ? HopKind::kReduceF32 : HopKind::kReduceBf16;
  const HopKind reduce_fwd = dtype == CCR_F32 ? HopKind::kReduceFwdF32 : HopKind::kReduceFwdBf16;
  // An all-reduce's last reduce-scatter hop also forwards the reduced chunk
  // to the next rank (rank q writes chunk q into bufs[q] and bufs[q+1] in
  // one pass), which is all-gather hop 0; with either copy mode the
  // all-gather then starts at hop 1.  Within that hop each forwarded element
  // is written only by the thread that read the same element, and no other
  // operation of the hop touches it.
  const bool fuse = which == kWhichAllreduce;
  // bf16 with the running partial carried in fp32 between ranks (R = 2 has a
  // single hop, identical to per-hop rounding).  Partials live in context
  // scratch, double-buffered by hop parity, indexed by offset in the chunk.
  const bool partials = dtype == CCR_BF16 && which != kWhichAG && R > 2 &&
                        ctx->cfg.bf16_acc == CCR_BF16_ACC_FP32_PARTIALS;
  const int64_t Lc = align_up(ceil_div(count, R), V);
  // Reduce-scatter runs on the CU-masked stream when a budget is set, else
  // directly on the caller's stream.  All-gather follows it on the same
  // stream, or, with several slices, on the second side stream when overlap
  // is on.  With SDMA copies the all-gather of each slice is one DMA job;
  // with several slices its handshake sits on the second side stream, so
  // the reduce-scatter of the next slice keeps going while the engines copy.
  const bool sdma = ctx->cfg.copy_mode == CCR_COPY_SDMA && which != kWhichRS;
  if (sdma) CCR_TRY(refuse_capture(caller, "a ring collective with SDMA copies"));
  if (partials) CCR_TRY(refuse_capture(caller, "a bf16 ring collective with fp32 partials"));
  if (partials) CCR_TRY(ensure_partials(ctx, 2 * (int64_t)R * Lc * 4));
  if (sdma) CCR_TRY(ensure_dma(ctx));
  // Slices exist so that one slice's all-gather can run while the next
  // slice's reduce-scatter does.  When nothing runs beside them (a single
  // phase, or both phases on one stream), the slices of a hop are adjacent
  // ranges of each chunk and run as one launch over whole chunks: every
  // element sees the same operations in the same order.
  const bool pipelined = which == kWhichAllreduce && (ctx->cfg.overlap || sdma);
  const int S = pipelined ? ctx->cfg.slices : 1;
  hipStream_t rs;
  CCR_TRY(work_stream(ctx, caller, &rs));
  // A second stream only when there is something to overlap: with a single
  // slice the all-gather (kernel copies or the SDMA job's gate) follows the
  // reduce-scatter on its stream, which saves two cross-stream waits (each
  // ~27 us of host time on this runtime when the work is still running).
  hipStream_t ag = rs;
  if (S > 1 && (ctx->cfg.overlap || sdma)) CCR_TRY(side_b(ctx, &ag));
  const size_t ev_fork = 0, ev_join_rs = 1, ev_join_ag = 2, ev_slice0 = 3;
  CCR_TRY(events(ctx, ev_slice0 + (size_t)S));
  if (rs != caller || ag != caller) {
    HIP_TRY(hipEventRecord(ctx->ev[ev_fork], caller));
    if (rs != caller) HIP_TRY(hipStreamWaitEvent(rs, ctx->ev[ev_fork], 0));
    if (ag != caller && ag != rs) HIP_TRY(hipStreamWaitEvent(ag, ctx->ev[ev_fork], 0));
  }

  std::vector<ccr_ring_op_t> ops;
  ops.reserve((size_t)R);
  std::vector<Piece> pieces((size_t)R);
  auto to_pieces = [&](int* n, bool forward) {
    *n = 0;
    for (const ccr_ring_op_t& o : ops) {
      if (o.hi <= o.lo) continue;
      Piece pc{static_cast<char*>(bufs[o.dst_rank]) + o.lo * esize,
               static_cast<const char*>(bufs[o.src_rank]) + o.lo * esize, (o.hi - o.lo) * esize};
      if (forward) pc.dst2 = static_cast<char*>(bufs[(o.dst_rank + 1) % R]) + o.lo * esize;
      pieces[(size_t)(*n)++] = pc;
    }
  };
  std::vector<PartialPiece> pp((size_t)R);
  for (int s = 0; s < S; s++) {
    if (which != kWhichAG) {
      for (int k = 0; k + 1 < R; k++) {
        const bool forward = fuse && k == R - 2;
        const int nt_hop = k == 0 ? first_hop_nontemporal() : -1;
        if (!partials) {
          bool done;
          CCR_TRY(ring_hop_timed(ctx, forward ? reduce_fwd : reduce,
                                 ring_hop_desc(kRS, k, s, R, count, S, V, esize, bufs), rs, nt_hop, &done));
          if (done) continue;
        }
        ops.clear();
        hop_ops(kRS, k, s, R, count, S, V, &ops);
        if (partials) {
          int n = 0;
          for (const ccr_ring_op_t& o : ops) {
            if (o.hi <= o.lo) continue;
            int64_t clo, chi;
            chunk_range(count, R, V, o.chunk, &clo, &chi);
            const int64_t off = o.lo - clo;
            char* mine = static_cast<char*>(bufs[o.dst_rank]) + o.lo * esize;
            PartialPiece pc;
            pc.loc = mine;
            pc.in = k == 0 ? static_cast<const char*>(bufs[o.src_rank]) + o.lo * esize
                           : reinterpret_cast<const char*>(
                                 ctx->partials + ((int64_t)((k - 1) % 2) * R + o.src_rank) * Lc + off);
            pc.out = k == R - 2 ? mine
                                : reinterpret_cast<char*>(
                                      ctx->partials + ((int64_t)(k % 2) * R + o.dst_rank) * Lc + off);
            pc.out2 = forward ? static_cast<char*>(bufs[(o.dst_rank + 1) % R]) + o.lo * esize : nullptr;
            pc.n = o.hi - o.lo;
            pp[(size_t)n++] = pc;
          }
          const PartialKind pk = k == 0 ? PartialKind::kFirst
                                 : k < R - 2 ? PartialKind::kMid
                                 : forward ? PartialKind::kLastFwd : PartialKind::kLast;
          CCR_TRY(launch_partials_timed(ctx, pk, pp.data(), n, rs));
          continue;
        }
        int n;
        to_pieces(&n, forward);
        CCR_TRY(launch_timed(ctx, forward ? reduce_fwd : reduce, pieces.data(), n, rs, nt_hop));
      }
    }
    if (which != kWhichRS && sdma) {
      CCR_TRY(order_after(ctx, ev_slice0 + (size_t)s, rs, ag));
      // every all-gather hop copies one chunk per rank: count elements over
      // the R-1 hops (R-2 when the last reduce hop forwarded), all slices
      const int64_t call_bytes = (int64_t)(R - 1 - (fuse ? 1 : 0)) * count * esize;
      const int E = dma_engine_limit(ctx, call_bytes);
      CCR_TRY(dma_submit(ctx, ag_chains(bufs, R, count, S, s, V, esize, E, fuse ? 1 : 0,
                                        any_engine_placement()),
                         ag, E));
    } else if (which != kWhichRS) {
      if (ag != rs) CCR_TRY(order_after(ctx, ev_slice0 + (size_t)s, rs, ag));
      for (int k = fuse ? 1 : 0; k + 1 < R; k++) {
        bool done;
        CCR_TRY(ring_hop_timed(ctx, HopKind::kCopy, ring_hop_desc(kAG, k, s, R, count, S, V, esize, bufs),
                               ag, -1, &done));
        if (done) continue;
        ops.clear();
        hop_ops(kAG, k, s, R, count, S, V, &ops);
        int n;
        to_pieces(&n, false);
        CCR_TRY(copy_pieces(ctx, pieces.data(), (size_t)n, ag));
      }
    }
  }
  CCR_TRY(order_after(ctx, ev_join_rs, rs, caller));
  if (ag != rs) CCR_TRY(order_after(ctx, ev_join_ag, ag, caller));
  return CCR_OK;
}

ccr_status_t ensure_staging(ccr_ctx* ctx) {
  const int64_t need = ctx->cfg.staging_chunk_bytes * ctx->cfg.staging_slots;
  if (ctx->staging && ctx->staging_bytes >= need) return CCR_OK;
  if (ctx->staging) {
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipFree(ctx->staging));
    ctx->staging = nullptr;
  }
  HIP_TRY(hipMalloc(reinterpret_cast<void**>(&ctx->staging), (size_t)need));
  ctx->staging_bytes = need;
  return CCR_OK;
}

ccr_status_t run_alltoall(ccr_ctx* ctx, const void* const* send, void* const* recv, int R,
                          const int64_t* counts, int64_t row_bytes, hipStream_t s) {
  std::vector<Piece> p;
  p.reserve((size_t)R * R);
  std::vector<int64_t> roff((size_t)R, 0);
  for (int r = 0; r < R; r++) {
    int64_t soff = 0;
    for (int d = 0; d < R; d++) {
      const int64_t c = counts[(size_t)r * R + d];
      if (c > 0)
        p.push_back(Piece{static_cast<char*>(recv[d]) + roff[(size_t)d] * row_bytes,
                          static_cast<const char*>(send[r]) + soff * row_bytes, c * row_bytes});
      soff += c;
      roff[(size_t)d] += c;
    }
  }
  if (ctx->cfg.copy_mode != CCR_COPY_SDMA) return copy_pieces(ctx, p.data(), p.size(), s);
  // SDMA: one DMA job; the segments are independent flows, chunked and
  // interleaved by size over the engines.
  CCR_TRY(ensure_dma(ctx));
  int64_t total = 0;
  for (const Piece& x : p) total += x.nbytes;
  const int E = dma_engine_limit(ctx, total);
  int64_t C = ctx->cfg.dma_chunk_bytes > 0 ? ctx->cfg.dma_chunk_bytes : auto_chunk(total, E);
  // at most ~64 Ki chunks per job, whatever chunk size was asked for
  C = std::max(C, (ceil_div(total, int64_t(1) << 16) + 15) & ~int64_t(15));
  return dma_submit(ctx, flow_chunks(p, C, E), s);
}

int64_t env_int(const char* name, int64_t dflt) {
  const char* e = getenv(name);
  return e && *e ? strtoll(e, nullptr, 0) : dflt;
}

}  // namespace

// ================================================================== C ABI
extern "C" {

const char* ccr_last_error(void) { return g_last_error.c_str(); }

const char* ccr_version(void) { return "ccr 0.1.0 gfx950"; }

ccr_status_t ccr_config_default(ccr_config_t* cfg) {
  if (!cfg) return fail(CCR_ERR_INVALID_ARG, "cfg is NULL");
  cfg->copy_mode = CCR_COPY_KERNEL;
  cfg->cu_budget = 0;
  cfg->slices = 1;
  cfg->overlap = 0;
  cfg->staging_chunk_bytes = 4 << 20;
  cfg->staging_slots = 2;
  cfg->bf16_acc = CCR_BF16_ACC_PER_HOP;
  cfg->dma_stripe = 0;
  cfg->dma_chunk_bytes = 0;
  cfg->dma_sync = CCR_DMA_SYNC_HOST_FUNC;
  if (const char* e = getenv("CCR_DMA_SYNC"); e && *e)
    cfg->dma_sync = strcmp(e, "stream_flags") == 0 ? CCR_DMA_SYNC_STREAM_FLAGS
                                                   : CCR_DMA_SYNC_HOST_FUNC;
  if (const char* e = getenv("CCR_COPY_MODE"); e && *e)
    cfg->copy_mode = strcmp(e, "sdma") == 0 ? CCR_COPY_SDMA : CCR_COPY_KERNEL;
  if (const char* e = getenv("CCR_BF16_ACC"); e && *e)
    cfg->bf16_acc = strcmp(e, "fp32_partials") == 0 ? CCR_BF16_ACC_FP32_PARTIALS
                                                    : CCR_BF16_ACC_PER_HOP;
  cfg->cu_budget = (int32_t)env_int("CCR_CU_BUDGET", cfg->cu_budget);
  cfg->slices = (int32_t)env_int("CCR_SLICES", cfg->slices);
  cfg->overlap = (int32_t)env_int("CCR_OVERLAP", cfg->overlap);
  cfg->staging_chunk_bytes = env_int("CCR_STAGING_CHUNK", cfg->staging_chunk_bytes);
  cfg->staging_slots = (int32_t)env_int("CCR_STAGING_SLOTS", cfg->staging_slots);
  cfg->dma_stripe = (int32_t)env_int("CCR_DMA_STRIPE", cfg->dma_stripe);
  cfg->dma_chunk_bytes = env_int("CCR_DMA_CHUNK", cfg->dma_chunk_bytes);
  cfg->dma_engines = (int32_t)env_int("CCR_DMA_ENGINES", 0);
  cfg->graph_cache = (int32_t)env_int("CCR_GRAPH_CACHE", 1);
  cfg->dma_deadline_us = (int32_t)env_int("CCR_DMA_DEADLINE_US", 0);
  return check_config(cfg);
}

ccr_status_t ccr_ctx_create(int device, const ccr_config_t* cfg, ccr_ctx_t* out) {
  if (!out) return fail(CCR_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  ccr_config_t c;
  if (cfg) {
    c = *cfg;
    CCR_TRY(check_config(&c));
  } else {
    CCR_TRY(ccr_config_default(&c));
  }
  int ndev = 0;
  HIP_TRY(hipGetDeviceCount(&ndev));
  if (device < 0 || device >= ndev)
    return fail(CCR_ERR_INVALID_ARG, "device %d outside [0, %d)", device, ndev);
  HIP_TRY(hipSetDevice(device));
  ccr_ctx* ctx = new ccr_ctx();
  ctx->device = device;
  ctx->cfg = c;
  hipError_t e = hipDeviceGetAttribute(&ctx->num_cus, hipDeviceAttributeMultiprocessorCount, device);
  ccr_status_t st = e == hipSuccess ? make_streams(ctx) : hip_fail(e, "hipDeviceGetAttribute");
  if (st == CCR_OK) st = events(ctx, 8);
  if (st == CCR_OK) {
    // the device's fixed scratch (the no-allocation entry points): resolved
    // here, with the device current, once per device
    const hipError_t se = resolve_scratch(device);
    if (se != hipSuccess) {
      (void)hipGetLastError();
      ctx->scratch_error = std::string("hipGetSymbolAddress: ") + hipGetErrorString(se);
    }
  }
  if (st != CCR_OK) {
    std::string msg = g_last_error;
    ccr_ctx_destroy(ctx);
    g_last_error = msg;
    return st;
  }
  *out = ctx;
  return CCR_OK;
}

ccr_status_t ccr_ctx_destroy(ccr_ctx_t ctx) {
  if (!ctx) return CCR_OK;
  (void)hipSetDevice(ctx->device);
  // Stop the DMA proxy: wait for its jobs (CCR_DESTROY_TIMEOUT_MS, default
  // 10 s), then abandon those whose streams have not reached them (each such
  // stream is released without the copies, whenever it gets there), then
  // wait as long again for copies that are running.
  DmaClose how = DmaClose::kClean;
  if (ctx->dma) {
    const double t = (double)env_int("CCR_DESTROY_TIMEOUT_MS", 10000) * 1e-3;
    how = ctx->dma->close(t > 0 ? t : 0.0);
    if (how != DmaClose::kInFlight) ctx->dma.reset();
    else (void)ctx->dma.release();  // its engines may still complete copies: keep its state
  }
  flush_graphs(ctx);
  ccr_status_t st = destroy_streams(ctx);
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
  for (auto& t : ctx->timed) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  for (hipEvent_t e : ctx->timing_pool) (void)hipEventDestroy(e);
  // An SDMA staging copy may still write the slots if the proxy gave up.
  if (ctx->staging && how != DmaClose::kInFlight) (void)hipFree(ctx->staging);
  if (ctx->d_ecnt) (void)hipFree(ctx->d_ecnt);
  if (ctx->partials) (void)hipFree(ctx->partials);
  if (ctx->h_pinned) (void)hipHostFree(ctx->h_pinned);
  for (auto& t : ctx->tables) {
    if (t.done) (void)hipEventSynchronize(t.done);
    if (t.dev) (void)hipFree(t.dev);
    if (t.host) (void)hipHostFree(t.host);
    if (t.done) (void)hipEventDestroy(t.done);
  }
  delete ctx;
  if (how == DmaClose::kAbandoned)
    return fail(CCR_ERR_TIMEOUT, "SDMA operations whose streams had not reached them were abandoned "
                                 "(their streams go on without the copies)");
  if (how == DmaClose::kInFlight)
    return fail(CCR_ERR_TIMEOUT, "SDMA copies still running at shutdown; their streams were released "
                                 "and the memory they write is kept");
  return st;
}

ccr_status_t ccr_ctx_set_config(ccr_ctx_t ctx, const ccr_config_t* cfg) {
  CCR_TRY(check_ctx(ctx));
  if (!cfg) return fail(CCR_ERR_INVALID_ARG, "cfg is NULL");
  CCR_TRY(check_config(cfg));
  const bool restream = cfg->cu_budget != ctx->cfg.cu_budget;
  for (hipStream_t x : {ctx->s_a, ctx->s_b})
    if (x) HIP_TRY(hipStreamSynchronize(x));
  flush_graphs(ctx);
  ctx->cfg = *cfg;
  if (restream) CCR_TRY(make_streams(ctx));
  return CCR_OK;
}

ccr_status_t ccr_ctx_get_config(ccr_ctx_t ctx, ccr_config_t* cfg) {
  if (!ctx || !cfg) return fail(CCR_ERR_INVALID_ARG, "ctx or cfg is NULL");
  *cfg = ctx->cfg;
  return CCR_OK;
}

ccr_status_t ccr_ring_schedule(int R, int64_t count, int slices, int dtype, int which,
                               ccr_ring_op_t* ops, int64_t max_ops, int64_t* n_ops) {
  if (!n_ops) return fail(CCR_ERR_INVALID_ARG, "n_ops is NULL");
  if (R < 1 || R > kMaxRanks) return fail(CCR_ERR_INVALID_ARG, "R = %d outside [1, %d]", R, kMaxRanks);
  if (count < 0 || slices < 1 || slices > 1024 || max_ops < 0)
    return fail(CCR_ERR_INVALID_ARG, "bad count, slices or max_ops");
  if (which < 0 || which > 2) return fail(CCR_ERR_INVALID_ARG, "which %d outside [0, 2]", which);
  const int esize = dtype_size(dtype);
  if (!esize) return fail(CCR_ERR_INVALID_ARG, "dtype %d is not f32 (0) or bf16 (1)", dtype);
  std::vector<ccr_ring_op_t> v;
  ring_schedule(R, count, slices, 16 / esize, which, &v);
  *n_ops = (int64_t)v.size();
  if (ops) std::copy(v.begin(), v.begin() + std::min<int64_t>(max_ops, (int64_t)v.size()), ops);
  return CCR_OK;
}

ccr_status_t ccr_ring_hop_layout(int R, int64_t count, int slices, int dtype, int phase, int step,
                                 int slice, int64_t* rows, int64_t max_wg, int64_t* n_wg) {
  if (!n_wg) return fail(CCR_ERR_INVALID_ARG, "n_wg is NULL");
  if (R < 1 || R > kMaxRanks) return fail(CCR_ERR_INVALID_ARG, "R = %d outside [1, %d]", R, kMaxRanks);
  if (count < 0 || slices < 1 || slices > 1024 || max_wg < 0)
    return fail(CCR_ERR_INVALID_ARG, "bad count, slices or max_wg");
  if (phase != kRS && phase != kAG) return fail(CCR_ERR_INVALID_ARG, "phase %d is not 0 or 1", phase);
  if (step < 0 || step >= R - 1 || slice < 0 || slice >= slices)
    return fail(CCR_ERR_INVALID_ARG, "step %d or slice %d out of range", step, slice);
  const int esize = dtype_size(dtype);
  if (!esize) return fail(CCR_ERR_INVALID_ARG, "dtype %d is not f32 (0) or bf16 (1)", dtype);
  if (max_wg > 0 && !rows) return fail(CCR_ERR_INVALID_ARG, "rows is NULL");
  const std::vector<void*> none((size_t)R, nullptr);  // the layout reads no base address
  const RingHop h = ring_hop_desc(phase, step, slice, R, count, slices, 16 / esize, esize, none.data());
  if (!ring_hop_supported(h, HopKind::kCopy, 0))
    return fail(CCR_ERR_UNSUPPORTED, "the ring-hop kernel does not take this hop");
  *n_wg = ring_hop_layout(h, rows, rows ? max_wg : 0);
  return CCR_OK;
}

ccr_status_t ccr_traffic_matrix(const int64_t* C, int G, const int32_t* node, const int32_t* peer,
                                int64_t* T) {
  CCR_MARK("ccr_traffic_matrix");
  ScheduleProblem p;
  p.G = G;
  p.C = C;
  p.node = node;
  p.peer = peer;
  const std::string bad = check_schedule_problem(p, false);
  if (!bad.empty()) return fail(CCR_ERR_INVALID_ARG, "%s", bad.c_str());
  if (!T) return fail(CCR_ERR_INVALID_ARG, "T is NULL");
  build_traffic_matrix(p, T);
  return CCR_OK;
}

ccr_status_t ccr_schedule_stages(const int64_t* C, int G, const int32_t* node, const int32_t* peer,
                                 int64_t bw_scaleup, int64_t bw_rdma, ccr_stage_entry_t* entries,
                                 int64_t max_entries, int64_t* n_entries, ccr_stage_time_t* times,
                                 int64_t max_stages, int64_t* n_stages) {
  CCR_MARK("ccr_schedule_stages");
  ScheduleProblem p;
  p.G = G;
  p.C = C;
  p.node = node;
  p.peer = peer;
  p.bw_scaleup = bw_scaleup;
  p.bw_rdma = bw_rdma;
  const std::string bad = check_schedule_problem(p, true);
  if (!bad.empty()) return fail(CCR_ERR_INVALID_ARG, "%s", bad.c_str());
  if (!n_entries || !n_stages) return fail(CCR_ERR_INVALID_ARG, "n_entries or n_stages is NULL");
  if (max_entries < 0 || max_stages < 0) return fail(CCR_ERR_INVALID_ARG, "negative maximum");
  std::vector<StageEntry> e;
  std::vector<StageTime> t;
  decompose_stages(p, &e, &t);
  *n_entries = (int64_t)e.size();
  *n_stages = (int64_t)t.size();
  if (entries) {
    const int64_t n = std::min<int64_t>(max_entries, (int64_t)e.size());
    for (int64_t i = 0; i < n; i++)
      entries[i] = {e[(size_t)i].stage, e[(size_t)i].kind, e[(size_t)i].src, e[(size_t)i].dst,
                    e[(size_t)i].bytes};
  }
  if (times) {
    const int64_t n = std::min<int64_t>(max_stages, (int64_t)t.size());
    for (int64_t i = 0; i < n; i++) times[i] = {t[(size_t)i].load, t[(size_t)i].bw};
  }
  return CCR_OK;
}

ccr_status_t ccr_allreduce(ccr_ctx_t ctx, void* const* bufs, int R, int64_t count, int dtype,
                           void* stream) {
  CCR_MARK("ccr_allreduce");
  return run_ring(ctx, bufs, R, count, dtype, kWhichAllreduce, static_cast<hipStream_t>(stream));
}

ccr_status_t ccr_reduce_scatter(ccr_ctx_t ctx, void* const* bufs, int R, int64_t count, int dtype,
                                void* stream) {
  CCR_MARK("ccr_reduce_scatter");
  return run_ring(ctx, bufs, R, count, dtype, kWhichRS, static_cast<hipStream_t>(stream));
}

ccr_status_t ccr_all_gather(ccr_ctx_t ctx, void* const* bufs, int R, int64_t count, int dtype,
                            void* stream) {
  CCR_MARK("ccr_all_gather");
  return run_ring(ctx, bufs, R, count, dtype, kWhichAG, static_cast<hipStream_t>(stream));
}


}  // extern "C"

namespace {

// Transfers m = 0..n-1, each nbytes from send[m] to recv[m], in order,
// through staging slots (the batch and ring-shift forms of the staged
// send/recv).  fixed_slots: NULL = the context's staging slots (allocated
// on demand); otherwise slots in memory the caller guarantees is large
// enough, used with kernel copies only and with nothing allocated.
ccr_status_t run_sendrecv(ccr_ctx* ctx, const void* const* send, void* const* recv, int n,
                          int64_t nbytes, hipStream_t caller, char* fixed_slots = nullptr) {
  CCR_TRY(check_ctx(ctx));
  if (n < 0 || nbytes < 0) return fail(CCR_ERR_INVALID_ARG, "n or nbytes < 0");
  if (nbytes % 16 != 0) return fail(CCR_ERR_INVALID_ARG, "%lld bytes per transfer is not a multiple of 16", (long long)nbytes);
  if (n == 0 || nbytes == 0) return CCR_OK;
  if (!send || !recv) return fail(CCR_ERR_INVALID_ARG, "send or recv is NULL");
  std::vector<Range> ranges;
  for (int m = 0; m < n; m++) {
    CCR_TRY(check_dev_ptr(ctx, send[m], nbytes, "send", m));
    CCR_TRY(check_dev_ptr(ctx, recv[m], nbytes, "recv", m));
    const uintptr_t a = reinterpret_cast<uintptr_t>(send[m]), b = reinterpret_cast<uintptr_t>(recv[m]);
    ranges.push_back(Range{a, a + (uintptr_t)nbytes, 2 * m});
    ranges.push_back(Range{b, b + (uintptr_t)nbytes, 2 * m + 1});
  }
  CCR_TRY(check_disjoint(ranges, "send/recv"));
  ctx->footprint = 2 * (int64_t)n * nbytes + ctx->cfg.staging_chunk_bytes * ctx->cfg.staging_slots;
  if (!fixed_slots) {
    CCR_TRY(refuse_capture(caller, "a staged send/recv (context staging slots)"));
    CCR_TRY(ensure_staging(ctx));
  }
  char* const slots_mem = fixed_slots ? fixed_slots : ctx->staging;
  if (ctx->cfg.copy_mode == CCR_COPY_SDMA && !fixed_slots) {
    // One DMA job: the proxy runs the slot state machine itself, each fill
    // and drain striped over several engines.
    CCR_TRY(ensure_dma(ctx));
    StagedPlan plan;
    for (int m = 0; m < n; m++) {
      plan.src.push_back(static_cast<const char*>(send[m]));
      plan.dst.push_back(static_cast<char*>(recv[m]));
    }
    plan.nbytes = nbytes;
    plan.chunk = ctx->cfg.staging_chunk_bytes;
    plan.slots = ctx->cfg.staging_slots;
    plan.slot_mem = ctx->staging;
    plan.engines = dma_engine_limit(ctx, 2 * (int64_t)n * nbytes);  // a fill and a drain per byte
    if (ctx->cfg.dma_deadline_us > 0 && ctx->dma->staged_step_us() > 0)
      plan.engines = staged_engines(ctx, (int64_t)n * ceil_div(nbytes, ctx->cfg.staging_chunk_bytes));
    plan.stripe = ctx->cfg.dma_stripe > 0 ? ctx->cfg.dma_stripe : std::max(1, plan.engines / 2);
    std::string err;
    if (!ctx->dma->submit_staged(plan, caller, (DmaSync)ctx->cfg.dma_sync, &err))
      return fail(CCR_ERR_HIP, "SDMA proxy: %s", err.c_str());
    return CCR_OK;
  }
  // Compute-unit copies on one stream, in rounds of P chunks (chunk c, over
  // all transfers in order, uses slot c mod P).  Round r hands slot p's
  // chunk (r-1)P+p to the receiver and refills the slot with chunk rP+p in
  // the same launch: each thread reads its part of the slot before it
  // overwrites it, so every slot still goes idle -> filling -> draining ->
  // idle and is refilled only after its chunk has drained, with one launch
  // per round instead of a fill launch and a drain launch.  Bytes of one
  // chunk that the other does not cover (a short last chunk of a transfer,
  // or no chunk left to fill) go to a plain copy launch: those byte ranges
  // are disjoint from the fused ones.  Filling and draining are both
  // compute-unit copies sharing HBM, so running them on two streams would
  // gain nothing on one GPU -- and a cross-stream wait costs ~27 us of host
  // time on this runtime.
  hipStream_t s;
  CCR_TRY(work_stream(ctx, caller, &s));
  CCR_TRY(order_after(ctx, 0, caller, s));
  const int P = ctx->cfg.staging_slots;
  const int64_t C = ctx->cfg.staging_chunk_bytes;
  const int64_t per = ceil_div(nbytes, C), T = per * n, rounds = ceil_div(T, (int64_t)P);
  // chunk c: transfer c / per, byte offset (c % per) * C
  auto chunk_len = [&](int64_t c) { return std::min<int64_t>(C, nbytes - (c % per) * C); };
  auto chunk_src = [&](int64_t c) { return static_cast<const char*>(send[c / per]) + (c % per) * C; };
  auto chunk_dst = [&](int64_t c) { return static_cast<char*>(recv[c / per]) + (c % per) * C; };
  std::vector<Piece> fused, copies;
  for (int64_t r = 0; r <= rounds; r++) {
    fused.clear();
    copies.clear();
    for (int p = 0; p < P; p++) {
      const int64_t a = (r - 1) * P + p, b = r * P + p;  // chunk drained, chunk filled
      char* slot = slots_mem + (int64_t)p * C;
      const bool drain = r >= 1 && a < T, fill = r < rounds && b < T;
      char* to = drain ? chunk_dst(a) : nullptr;
      const char* from = fill ? chunk_src(b) : nullptr;
      const int64_t la = drain ? chunk_len(a) : 0, lb = fill ? chunk_len(b) : 0;
      const int64_t both = std::min(la, lb);
      if (both > 0) fused.push_back(Piece{slot, from, both, to});
      if (la > both) copies.push_back(Piece{to + both, slot + both, la - both});
      if (lb > both) copies.push_back(Piece{slot + both, from + both, lb - both});
    }
    for (size_t i = 0; i < fused.size(); i += kMaxPieces) {
      const int m = (int)std::min<size_t>(kMaxPieces, fused.size() - i);
      if (fixed_slots)  // no timing events: they would be created on demand
        HIP_TRY(launch_pieces(HopKind::kDrainFill, fused.data() + i, m, call_tuning(ctx), s));
      else
        CCR_TRY(launch_timed(ctx, HopKind::kDrainFill, fused.data() + i, m, s));
    }
    if (fixed_slots) {
      for (size_t i = 0; i < copies.size(); i += kMaxPieces) {
        const int m = (int)std::min<size_t>(kMaxPieces, copies.size() - i);
        HIP_TRY(launch_pieces(HopKind::kCopy, copies.data() + i, m, call_tuning(ctx), s));
      }
    } else {
      CCR_TRY(copy_pieces(ctx, copies.data(), copies.size(), s));
    }
  }
  CCR_TRY(order_after(ctx, 1, s, caller));
  return CCR_OK;
}


// All-to-all of row segments: counts[r*R + d] rows of row_bytes from rank r
// to rank d; send[r] in destination order, recv[d] in source order.
ccr_status_t run_alltoall_rows(ccr_ctx* ctx, const void* const* send, void* const* recv, int R,
                               const int64_t* counts, int64_t row_bytes, hipStream_t caller) {
  CCR_TRY(check_ctx(ctx));
  if (R < 1 || R > kMaxRanks) return fail(CCR_ERR_INVALID_ARG, "R = %d outside [1, %d]", R, kMaxRanks);
  if (!send || !recv || !counts) return fail(CCR_ERR_INVALID_ARG, "send, recv or counts is NULL");
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(CCR_ERR_INVALID_ARG, "row_bytes %lld is not a positive multiple of 16", (long long)row_bytes);
  std::vector<int64_t> sent((size_t)R, 0), got((size_t)R, 0);
  for (int r = 0; r < R; r++)
    for (int d = 0; d < R; d++) {
      const int64_t c = counts[(size_t)r * R + d];
      if (c < 0) return fail(CCR_ERR_INVALID_ARG, "counts[%d][%d] < 0", r, d);
      sent[(size_t)r] += c;
      got[(size_t)d] += c;
    }
  std::vector<Range> ranges;
  for (int r = 0; r < R; r++) {
    if (sent[(size_t)r] > 0) {
      CCR_TRY(check_dev_ptr(ctx, send[r], sent[(size_t)r] * row_bytes, "send", r));
      const uintptr_t a = reinterpret_cast<uintptr_t>(send[r]);
      ranges.push_back(Range{a, a + (uintptr_t)(sent[(size_t)r] * row_bytes), r});
    }
    if (got[(size_t)r] > 0) {
      CCR_TRY(check_dev_ptr(ctx, recv[r], got[(size_t)r] * row_bytes, "recv", r));
      const uintptr_t b = reinterpret_cast<uintptr_t>(recv[r]);
      ranges.push_back(Range{b, b + (uintptr_t)(got[(size_t)r] * row_bytes), R + r});
    }
  }
  CCR_TRY(check_disjoint(ranges, "send/recv"));
  ctx->footprint = 0;
  for (int r = 0; r < R; r++) ctx->footprint += (sent[(size_t)r] + got[(size_t)r]) * row_bytes;
  if (ctx->cfg.copy_mode == CCR_COPY_SDMA)
    CCR_TRY(refuse_capture(caller, "an all-to-all with SDMA copies"));
  hipStream_t s;
  CCR_TRY(work_stream(ctx, caller, &s));
  CCR_TRY(order_after(ctx, 0, caller, s));
  CCR_TRY(run_alltoall(ctx, send, recv, R, counts, row_bytes, s));
  CCR_TRY(order_after(ctx, 1, s, caller));
  return CCR_OK;
}


}  // namespace

extern "C" {

ccr_status_t ccr_sendrecv(ccr_ctx_t ctx, const void* const* send, void* const* recv, int R,
                          int64_t count, int dtype, void* stream) {
  CCR_MARK("ccr_sendrecv");
  CCR_TRY(check_ctx(ctx));
  if (R < 1 || R > kMaxRanks) return fail(CCR_ERR_INVALID_ARG, "R = %d outside [1, %d]", R, kMaxRanks);
  if (count < 0) return fail(CCR_ERR_INVALID_ARG, "count %lld < 0", (long long)count);
  const int esize = dtype_size(dtype);
  if (!esize) return fail(CCR_ERR_INVALID_ARG, "dtype %d is not f32 (0) or bf16 (1)", dtype);
  if (count == 0) return CCR_OK;
  if (count * esize % 16 != 0)
    return fail(CCR_ERR_INVALID_ARG, "count %lld is not a whole number of 16-byte vectors",
                (long long)count);
  if (!send || !recv) return fail(CCR_ERR_INVALID_ARG, "send or recv is NULL");
  // rank r's transfer lands in the buffer of its ring successor
  std::vector<void*> to((size_t)R);
  for (int r = 0; r < R; r++) to[(size_t)r] = recv[(r + 1) % R];
  return run_sendrecv(ctx, send, to.data(), R, count * esize, static_cast<hipStream_t>(stream));
}

ccr_status_t ccr_sendrecv_batch(ccr_ctx_t ctx, const void* const* send, void* const* recv, int n,
                                int64_t nbytes, void* stream) {
  CCR_MARK("ccr_sendrecv_batch");
  return run_sendrecv(ctx, send, recv, n, nbytes, static_cast<hipStream_t>(stream));
}

ccr_status_t ccr_sendrecv_batch_noalloc(ccr_ctx_t ctx, const void* const* send, void* const* recv,
                                        int n, int64_t nbytes, void* stream) {
  CCR_MARK("ccr_sendrecv_batch_noalloc");
  CCR_TRY(check_ctx(ctx));
  const int64_t need = ctx->cfg.staging_chunk_bytes * ctx->cfg.staging_slots;
  if (need > kScratchBytes)
    return fail(CCR_ERR_INVALID_ARG,
                "staging_slots x staging_chunk_bytes = %lld bytes exceeds the %lld bytes of fixed "
                "scratch this entry point stages through", (long long)need, (long long)kScratchBytes);
  if (ctx->cfg.copy_mode != CCR_COPY_KERNEL)
    return fail(CCR_ERR_UNSUPPORTED, "the no-allocation send/recv runs on kernel copies only "
                                     "(the SDMA proxy allocates when it starts)");
  char* slots = scratch_address(ctx->device);
  if (!slots)
    return fail(CCR_ERR_HIP, "the device address of the fixed scratch was not resolved (%s)",
                ctx->scratch_error.c_str());
  return run_sendrecv(ctx, send, recv, n, nbytes, static_cast<hipStream_t>(stream), slots);
}

ccr_status_t ccr_alltoall(ccr_ctx_t ctx, const void* const* send, void* const* recv, int R,
                          int64_t count, const int64_t* counts, int dtype, void* stream) {
  CCR_MARK("ccr_alltoall");
  CCR_TRY(check_ctx(ctx));
  if (R < 1 || R > kMaxRanks) return fail(CCR_ERR_INVALID_ARG, "R = %d outside [1, %d]", R, kMaxRanks);
  if (count < 0) return fail(CCR_ERR_INVALID_ARG, "count %lld < 0", (long long)count);
  const int esize = dtype_size(dtype);
  if (!esize) return fail(CCR_ERR_INVALID_ARG, "dtype %d is not f32 (0) or bf16 (1)", dtype);
  const int64_t V = 16 / esize;  // elements per 16-byte vector
  // segments as rows of one 16-byte vector each
  std::vector<int64_t> rows((size_t)R * R);
  if (!counts) {
    if (count % ((int64_t)R * V) != 0)
      return fail(CCR_ERR_INVALID_ARG,
                  "count %lld does not split into %d segments of whole 16-byte vectors", (long long)count, R);
    std::fill(rows.begin(), rows.end(), count / R / V);
  } else {
    for (int r = 0; r < R; r++) {
      int64_t sent = 0;
      for (int d = 0; d < R; d++) {
        const int64_t c = counts[(size_t)r * R + d];
        if (c < 0) return fail(CCR_ERR_INVALID_ARG, "counts[%d][%d] < 0", r, d);
        if (c % V != 0)
          return fail(CCR_ERR_INVALID_ARG, "counts[%d][%d] = %lld is not a whole number of 16-byte vectors",
                      r, d, (long long)c);
        rows[(size_t)r * R + d] = c / V;
        sent += c;
      }
      if (sent != count)
        return fail(CCR_ERR_INVALID_ARG, "rank %d sends %lld elements, not count = %lld", r,
                    (long long)sent, (long long)count);
    }
  }
  return run_alltoall_rows(ctx, send, recv, R, rows.data(), 16, static_cast<hipStream_t>(stream));
}

ccr_status_t ccr_alltoall_rows(ccr_ctx_t ctx, const void* const* send, void* const* recv, int R,
                               const int64_t* counts, int64_t row_bytes, void* stream) {
  CCR_MARK("ccr_alltoall_rows");
  return run_alltoall_rows(ctx, send, recv, R, counts, row_bytes, static_cast<hipStream_t>(stream));
}

ccr_status_t ccr_permute_rows(ccr_ctx_t ctx, void* dst, const void* src, const int32_t* d_idx,
                              int64_t nrows, int64_t nsrc, int64_t row_bytes, void* stream) {
  CCR_MARK("ccr_permute_rows");
  CCR_TRY(check_ctx(ctx));
  if (nrows < 0 || nsrc < 0) return fail(CCR_ERR_INVALID_ARG, "nrows or nsrc < 0");
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(CCR_ERR_INVALID_ARG, "row_bytes %lld is not a positive multiple of 16", (long long)row_bytes);
  if (nrows == 0) return CCR_OK;
  CCR_TRY(check_dev_ptr(ctx, dst, nrows * row_bytes, "dst", 0));
  CCR_TRY(check_dev_ptr(ctx, d_idx, nrows * 4, "d_idx", 0));
  if (nsrc > 0) CCR_TRY(check_dev_ptr(ctx, src, nsrc * row_bytes, "src", 0));
  std::vector<Range> ranges{{reinterpret_cast<uintptr_t>(dst),
                             reinterpret_cast<uintptr_t>(dst) + (uintptr_t)(nrows * row_bytes), 0},
                            {reinterpret_cast<uintptr_t>(src),
                             reinterpret_cast<uintptr_t>(src) + (uintptr_t)(nsrc * row_bytes), 1}};
  CCR_TRY(check_disjoint(ranges, "dst/src"));
  hipStream_t caller = static_cast<hipStream_t>(stream);
  hipStream_t s;
  CCR_TRY(work_stream(ctx, caller, &s));
  CCR_TRY(order_after(ctx, 0, caller, s));
  HIP_TRY(launch_permute_rows(static_cast<char*>(dst), static_cast<const char*>(src), d_idx, nrows,
                              nsrc, row_bytes, s));
  CCR_TRY(order_after(ctx, 1, s, caller));
  return CCR_OK;
}

ccr_status_t ccr_moe_topk(ccr_ctx_t ctx, const float* logits, int32_t* topk, int64_t T, int E,
                          int K, void* stream) {
  CCR_MARK("ccr_moe_topk");
  CCR_TRY(check_ctx(ctx));
  if (T < 0 || E < 1 || E > 1024 || K < 1 || K > 16 || K > E)
    return fail(CCR_ERR_INVALID_ARG, "need T >= 0, 1 <= E <= 1024, 1 <= K <= min(E, 16)");
  if (T == 0) return CCR_OK;
  CCR_TRY(check_dev_ptr(ctx, logits, T * E * 4, "logits", 0));
  CCR_TRY(check_dev_ptr(ctx, topk, T * K * 4, "topk", 0));
  HIP_TRY(launch_moe_topk(logits, topk, T, E, K, static_cast<hipStream_t>(stream)));
  return CCR_OK;
}

ccr_status_t ccr_moe_plan(ccr_ctx_t ctx, const int32_t* topk, int64_t T, int E, int K, int R,
                          int32_t* src_tok, int32_t* slot, int64_t* h_ecnt, void* stream) {
  CCR_MARK("ccr_moe_plan");
  CCR_TRY(check_ctx(ctx));
  if (T < 0 || T > INT32_MAX / 16 || E < 1 || E > 1024 || K < 1 || K > 16 || K > E || R < 1 ||
      R > kMaxRanks || E % R != 0)
    return fail(CCR_ERR_INVALID_ARG, "need 0 <= T, 1 <= K <= min(E, 16), E <= 1024, R | E");
  if (!h_ecnt) return fail(CCR_ERR_INVALID_ARG, "h_ecnt is NULL");
  CCR_TRY(refuse_capture(static_cast<hipStream_t>(stream), "ccr_moe_plan (blocking)"));
  if (T > 0) {
    CCR_TRY(check_dev_ptr(ctx, topk, T * K * 4, "topk", 0));
    CCR_TRY(check_dev_ptr(ctx, src_tok, T * K * 4, "src_tok", 0));
    CCR_TRY(check_dev_ptr(ctx, slot, T * K * 4, "slot", 0));
  }
  if (ctx->d_ecnt_len < E) {
    if (ctx->d_ecnt) HIP_TRY(hipFree(ctx->d_ecnt));
    if (ctx->h_pinned) HIP_TRY(hipHostFree(ctx->h_pinned));
    ctx->d_ecnt = nullptr;
    ctx->h_pinned = nullptr;
    ctx->d_ecnt_len = 0;
    HIP_TRY(hipMalloc(reinterpret_cast<void**>(&ctx->d_ecnt), sizeof(int64_t) * 1024));
    HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&ctx->h_pinned), sizeof(int64_t) * 1024,
                          hipHostMallocDefault));
    ctx->d_ecnt_len = 1024;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_TRY(launch_moe_plan(topk, T, E, K, E / R, ctx->d_ecnt, src_tok, slot, s));
  HIP_TRY(hipMemcpyAsync(ctx->h_pinned, ctx->d_ecnt, sizeof(int64_t) * E, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  memcpy(h_ecnt, ctx->h_pinned, sizeof(int64_t) * E);
  return CCR_OK;
}

namespace {

struct MoeShape {
  int R, E, K, eloc;
  int64_t T, row_bytes;
  std::vector<int64_t> cnt;  // cnt[r*R + d]: rows r -> d
};

ccr_status_t moe_shape(ccr_ctx* ctx, const int64_t* h_ecnt, int R, int64_t T, int E, int K,
                       int64_t row_bytes, MoeShape* m) {
  CCR_TRY(check_ctx(ctx));
  if (R < 1 || R > kMaxRanks || E < 1 || E % R != 0 || K < 1 || K > E || T < 0)
    return fail(CCR_ERR_INVALID_ARG, "need 1 <= R <= %d, R | E, 1 <= K <= E, T >= 0", kMaxRanks);
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(CCR_ERR_INVALID_ARG, "row_bytes %lld is not a positive multiple of 16", (long long)row_bytes);
  if (!h_ecnt) return fail(CCR_ERR_INVALID_ARG, "h_ecnt is NULL");
  m->R = R; m->E = E; m->K = K; m->eloc = E / R; m->T = T; m->row_bytes = row_bytes;
  m->cnt.assign((size_t)R * R, 0);
  for (int r = 0; r < R; r++) {
    int64_t tot = 0;
    for (int e = 0; e < E; e++) {
      const int64_t c = h_ecnt[(size_t)r * E + e];
      if (c < 0) return fail(CCR_ERR_INVALID_ARG, "h_ecnt[%d][%d] < 0", r, e);
      m->cnt[(size_t)r * R + e / m->eloc] += c;
      tot += c;
    }
    if (tot != T * K)
      return fail(CCR_ERR_INVALID_ARG, "rank %d's expert counts sum to %lld, not T*K = %lld", r,
                  (long long)tot, (long long)(T * K));
  }
  return CCR_OK;
}

// The unpack of rank d as block copies: for local expert l, for source r,
// the rows of r's segment that go to expert (d, l) land contiguously.
void unpack_pieces(const MoeShape& m, const int64_t* h_ecnt, void* const* recv, void* const* exp,
                   bool inverse, std::vector<Piece>* out) {
  const int R = m.R, E = m.E, eloc = m.eloc;
  for (int d = 0; d < R; d++) {
    std::vector<int64_t> seg((size_t)R, 0);  // start of r's segment in recv[d]
    for (int r = 1; r < R; r++) seg[(size_t)r] = seg[(size_t)r - 1] + m.cnt[(size_t)(r - 1) * R + d];
    int64_t pos = 0;
    for (int l = 0; l < eloc; l++) {
      for (int r = 0; r < R; r++) {
        int64_t start = seg[(size_t)r];
        for (int ll = 0; ll < l; ll++) start += h_ecnt[(size_t)r * E + d * eloc + ll];
        const int64_t c = h_ecnt[(size_t)r * E + d * eloc + l];
        if (c > 0) {
          char* rp = static_cast<char*>(recv[d]) + start * m.row_bytes;
          char* ep = static_cast<char*>(exp[d]) + pos * m.row_bytes;
          out->push_back(inverse ? Piece{rp, ep, c * m.row_bytes} : Piece{ep, rp, c * m.row_bytes});
        }
        pos += c;
      }
    }
  }
}

ccr_status_t launch_copies(const ccr_ctx* ctx, const std::vector<Piece>& p, hipStream_t s) {
  const LaunchTuning tune = call_tuning(ctx);
  for (size_t i = 0; i < p.size(); i += kMaxPieces) {
    const int n = (int)std::min<size_t>(kMaxPieces, p.size() - i);
    HIP_TRY(launch_pieces(HopKind::kCopy, p.data() + i, n, tune, s));
  }
  return CCR_OK;
}

// Per-rank device pointers; nbytes[r] (or nbytes[0] for all ranks when
// per_rank is false) bytes must fit behind each.
ccr_status_t check_rank_ptrs(ccr_ctx* ctx, const void* const* p, int R, const int64_t* nbytes,
                             bool per_rank, const char* what) {
  if (!p) return fail(CCR_ERR_INVALID_ARG, "%s is NULL", what);
  for (int r = 0; r < R; r++) CCR_TRY(check_dev_ptr(ctx, p[r], nbytes[per_rank ? r : 0], what, r));
  return CCR_OK;
}

// The buffers of a call, each marked written or read-only.  No written
// buffer may overlap any other buffer of the call (read-only buffers may
// overlap each other); empty buffers are ignored.
struct CallBuf {
  uintptr_t lo, hi;
  bool written;
  const char* what;
  int rank;
};

void add_bufs(std::vector<CallBuf>* b, const void* const* p, int R, const int64_t* nbytes,
              bool per_rank, bool written, const char* what) {
  for (int r = 0; r < R; r++) {
    const int64_t n = nbytes[per_rank ? r : 0];
    if (n <= 0) continue;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p[r]);
    b->push_back(CallBuf{a, a + (uintptr_t)n, written, what, r});
  }
}

ccr_status_t check_writes_disjoint(const std::vector<CallBuf>& b) {
  for (size_t i = 0; i < b.size(); i++)
    for (size_t j = i + 1; j < b.size(); j++)
      if ((b[i].written || b[j].written) && b[i].lo < b[j].hi && b[j].lo < b[i].hi)
        return fail(CCR_ERR_INVALID_ARG, "%s[%d] and %s[%d] overlap", b[i].what, b[i].rank,
                    b[j].what, b[j].rank);
  return CCR_OK;
}

}  // namespace

ccr_status_t ccr_moe_dispatch(ccr_ctx_t ctx, const void* const* x, const int32_t* const* src_tok,
                              const int64_t* h_ecnt, int R, int64_t T, int E, int K,
                              int64_t row_bytes, void* const* send, void* const* recv,
                              void* const* exp, void* stream) {
  CCR_MARK("ccr_moe_dispatch");
  MoeShape m;
  CCR_TRY(moe_shape(ctx, h_ecnt, R, T, E, K, row_bytes, &m));
  if (T == 0) return CCR_OK;
  const int64_t xb = T * row_bytes, sb = T * K * row_bytes, ib = T * K * 4;
  std::vector<int64_t> rb((size_t)R, 0);
  for (int d = 0; d < R; d++)
    for (int r = 0; r < R; r++) rb[(size_t)d] += m.cnt[(size_t)r * R + d] * row_bytes;
  CCR_TRY(check_rank_ptrs(ctx, x, R, &xb, false, "x"));
  CCR_TRY(check_rank_ptrs(ctx, reinterpret_cast<const void* const*>(src_tok), R, &ib, false, "src_tok"));
  CCR_TRY(check_rank_ptrs(ctx, send, R, &sb, false, "send"));
  CCR_TRY(check_rank_ptrs(ctx, recv, R, rb.data(), true, "recv"));
  CCR_TRY(check_rank_ptrs(ctx, exp, R, rb.data(), true, "exp"));
  std::vector<CallBuf> bufs;
  add_bufs(&bufs, x, R, &xb, false, false, "x");
  add_bufs(&bufs, reinterpret_cast<const void* const*>(src_tok), R, &ib, false, false, "src_tok");
  add_bufs(&bufs, send, R, &sb, false, true, "send");
  add_bufs(&bufs, recv, R, rb.data(), true, true, "recv");
  add_bufs(&bufs, exp, R, rb.data(), true, true, "exp");
  CCR_TRY(check_writes_disjoint(bufs));
  ctx->footprint = 0;
  for (const CallBuf& b : bufs) ctx->footprint += (int64_t)(b.hi - b.lo);
  hipStream_t caller = static_cast<hipStream_t>(stream);
  if (ctx->cfg.copy_mode == CCR_COPY_SDMA)
    CCR_TRY(refuse_capture(caller, "ccr_moe_dispatch with SDMA copies"));
  hipStream_t s;
  CCR_TRY(work_stream(ctx, caller, &s));
  CCR_TRY(order_after(ctx, 0, caller, s));
  // pack: send[r] row j = x[r] row src_tok[r][j]
  for (int r = 0; r < R; r++)
    HIP_TRY(launch_permute_rows(static_cast<char*>(send[r]), static_cast<const char*>(x[r]),
                                src_tok[r], T * K, T, row_bytes, s));
  // exchange
  CCR_TRY(run_alltoall(ctx, const_cast<const void* const*>(send), recv, R, m.cnt.data(), row_bytes, s));
  // unpack to (local expert, source rank, token)
  std::vector<Piece> p;
  unpack_pieces(m, h_ecnt, recv, exp, false, &p);
  CCR_TRY(launch_copies(ctx, p, s));
  CCR_TRY(order_after(ctx, 1, s, caller));
  return CCR_OK;
}

ccr_status_t ccr_moe_combine(ccr_ctx_t ctx, const void* const* exp, const int32_t* const* slot,
                             const int64_t* h_ecnt, int R, int64_t T, int E, int K,
                             int64_t row_bytes, void* const* recv, void* const* send,
                             void* const* out, void* stream) {
  CCR_MARK("ccr_moe_combine");
  MoeShape m;
  CCR_TRY(moe_shape(ctx, h_ecnt, R, T, E, K, row_bytes, &m));
  if (T == 0) return CCR_OK;
  const int64_t sb = T * K * row_bytes, ib = T * K * 4;
  std::vector<int64_t> rb((size_t)R, 0);
  for (int d = 0; d < R; d++)
    for (int r = 0; r < R; r++) rb[(size_t)d] += m.cnt[(size_t)r * R + d] * row_bytes;
  CCR_TRY(check_rank_ptrs(ctx, exp, R, rb.data(), true, "exp"));
  CCR_TRY(check_rank_ptrs(ctx, reinterpret_cast<const void* const*>(slot), R, &ib, false, "slot"));
  CCR_TRY(check_rank_ptrs(ctx, recv, R, rb.data(), true, "recv"));
  CCR_TRY(check_rank_ptrs(ctx, send, R, &sb, false, "send"));
  CCR_TRY(check_rank_ptrs(ctx, out, R, &sb, false, "out"));
  std::vector<CallBuf> bufs;
  add_bufs(&bufs, exp, R, rb.data(), true, false, "exp");
  add_bufs(&bufs, reinterpret_cast<const void* const*>(slot), R, &ib, false, false, "slot");
  add_bufs(&bufs, recv, R, rb.data(), true, true, "recv");
  add_bufs(&bufs, send, R, &sb, false, true, "send");
  add_bufs(&bufs, out, R, &sb, false, true, "out");
  CCR_TRY(check_writes_disjoint(bufs));
  ctx->footprint = 0;
  for (const CallBuf& b : bufs) ctx->footprint += (int64_t)(b.hi - b.lo);
  hipStream_t caller = static_cast<hipStream_t>(stream);
  if (ctx->cfg.copy_mode == CCR_COPY_SDMA)
    CCR_TRY(refuse_capture(caller, "ccr_moe_combine with SDMA copies"));
  hipStream_t s;
  CCR_TRY(work_stream(ctx, caller, &s));
  CCR_TRY(order_after(ctx, 0, caller, s));
  // inverse unpack: expert-major rows back to source-segment order
  std::vector<Piece> p;
  unpack_pieces(m, h_ecnt, recv, const_cast<void* const*>(exp), true, &p);
  CCR_TRY(launch_copies(ctx, p, s));
  // reverse exchange: rank d returns to r what it received from r
  std::vector<int64_t> back((size_t)R * R);
  for (int r = 0; r < R; r++)
    for (int d = 0; d < R; d++) back[(size_t)d * R + r] = m.cnt[(size_t)r * R + d];
  CCR_TRY(run_alltoall(ctx, const_cast<const void* const*>(recv), send, R, back.data(), row_bytes, s));
  // out[r] row (t, k) = send[r] row slot[r][t*K + k]
  for (int r = 0; r < R; r++)
    HIP_TRY(launch_permute_rows(static_cast<char*>(out[r]), static_cast<const char*>(send[r]),
                                slot[r], T * K, T * K, row_bytes, s));
  CCR_TRY(order_after(ctx, 1, s, caller));
  return CCR_OK;
}

namespace {

// Copy `bytes` of host data to a device table for work about to be enqueued
// on `s`; the caller records the slot's `done` event on `s` after that work.
ccr_status_t upload_table(ccr_ctx* ctx, const void* data, int64_t bytes, hipStream_t s,
                          ccr_ctx::TableSlot** slot) {
  ccr_ctx::TableSlot& t = ctx->tables[ctx->next_table];
  ctx->next_table = (ctx->next_table + 1) % ccr_ctx::kTableSlots;
  if (!t.done) HIP_TRY(hipEventCreateWithFlags(&t.done, hipEventDisableTiming));
  HIP_TRY(hipEventSynchronize(t.done));  // the slot's previous call is done with it
  if (t.cap < bytes) {
    if (t.dev) HIP_TRY(hipFree(t.dev));
    if (t.host) HIP_TRY(hipHostFree(t.host));
    t.dev = t.host = nullptr;
    t.cap = 0;
    const int64_t cap = std::max<int64_t>(bytes, 64 << 10);
    HIP_TRY(hipMalloc(reinterpret_cast<void**>(&t.dev), (size_t)cap));
    HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&t.host), (size_t)cap, hipHostMallocDefault));
    t.cap = cap;
  }
  memcpy(t.host, data, (size_t)bytes);
  HIP_TRY(hipMemcpyAsync(t.dev, t.host, (size_t)bytes, hipMemcpyHostToDevice, s));
  *slot = &t;
  return CCR_OK;
}

// One gather per row between each source rank's rows and the expert-major
// buffers, with the placement of the three-stage path: for destination d,
// local expert l, source r, r's rows for expert d*eloc + l, in pack order.
ccr_status_t moe_gather(ccr_ctx* ctx, int combine, const MoeShape& m, const int64_t* h_ecnt,
                        void* const* own, const int32_t* const* idx, void* const* exp,
                        hipStream_t caller) {
  const int R = m.R, E = m.E, eloc = m.eloc;
  const int64_t rows = m.T * m.K;
  // table: R MoeRank records, then R*E MoeSeg records
  std::vector<char> tab(sizeof(MoeRank) * (size_t)R + sizeof(MoeSeg) * (size_t)R * E);
  MoeRank* rk = reinterpret_cast<MoeRank*>(tab.data());
  MoeSeg* sg = reinterpret_cast<MoeSeg*>(tab.data() + sizeof(MoeRank) * (size_t)R);
  for (int r = 0; r < R; r++) {
    rk[r] = MoeRank{static_cast<char*>(own[r]), idx[r]};
    int64_t start = 0;  // pack position of r's first row for expert e
    for (int e = 0; e < E; e++) {
      sg[(size_t)r * E + e] = MoeSeg{start, 0, static_cast<char*>(exp[e / eloc])};
      start += h_ecnt[(size_t)r * E + e];
    }
  }
  for (int d = 0; d < R; d++) {  // exp[d] holds (local expert, source rank) blocks in order
    int64_t row = 0;
    for (int l = 0; l < eloc; l++)
      for (int r = 0; r < R; r++) {
        const int e = d * eloc + l;
        sg[(size_t)r * E + e].exp_row = row;
        row += h_ecnt[(size_t)r * E + e];
      }
  }
  CCR_TRY(refuse_capture(caller, "a fused MoE call (segment table copied from host memory)"));
  hipStream_t s;
  CCR_TRY(work_stream(ctx, caller, &s));
  CCR_TRY(order_after(ctx, 0, caller, s));
  ccr_ctx::TableSlot* slot = nullptr;
  CCR_TRY(upload_table(ctx, tab.data(), (int64_t)tab.size(), s, &slot));
  const MoeRank* d_rk = reinterpret_cast<const MoeRank*>(slot->dev);
  const MoeSeg* d_sg = reinterpret_cast<const MoeSeg*>(slot->dev + sizeof(MoeRank) * (size_t)R);
  const int64_t limit = combine ? rows : m.T;
  // the combine reads every expert row once (non-temporal when the call's
  // buffers exceed the MALL); the dispatch reads each token row once per
  // chosen expert, so its loads stay temporal
  ctx->footprint = (int64_t)R * ((combine ? rows : m.T) + rows) * m.row_bytes;
  const bool nt_load = combine && call_tuning(ctx).nontemporal != 0;
  if (ctx->prof_on) {
    hipEvent_t start, stop;
    CCR_TRY(timing_event(ctx, &start));
    CCR_TRY(timing_event(ctx, &stop));
    HIP_TRY(launch_moe_gather(combine, d_rk, d_sg, R, E, rows, limit, m.row_bytes, nt_load, s, start,
                              stop));
    ctx->timed.push_back(ccr_ctx::Timed{kProfGather, start, stop, 2 * R * rows * m.row_bytes,
                                        cus_held(ctx, R * ((rows + 7) / 8))});
  } else {
    HIP_TRY(launch_moe_gather(combine, d_rk, d_sg, R, E, rows, limit, m.row_bytes, nt_load, s));
  }
  HIP_TRY(hipEventRecord(slot->done, s));
  CCR_TRY(order_after(ctx, 1, s, caller));
  return CCR_OK;
}

}  // namespace

ccr_status_t ccr_moe_dispatch_fused(ccr_ctx_t ctx, const void* const* x,
                                    const int32_t* const* src_tok, const int64_t* h_ecnt, int R,
                                    int64_t T, int E, int K, int64_t row_bytes, void* const* exp,
                                    void* stream) {
  CCR_MARK("ccr_moe_dispatch_fused");
  MoeShape m;
  CCR_TRY(moe_shape(ctx, h_ecnt, R, T, E, K, row_bytes, &m));
  if (T == 0) return CCR_OK;
  const int64_t xb = T * row_bytes, ib = T * K * 4;
  std::vector<int64_t> rb((size_t)R, 0);
  for (int d = 0; d < R; d++)
    for (int r = 0; r < R; r++) rb[(size_t)d] += m.cnt[(size_t)r * R + d] * row_bytes;
  CCR_TRY(check_rank_ptrs(ctx, x, R, &xb, false, "x"));
  CCR_TRY(check_rank_ptrs(ctx, reinterpret_cast<const void* const*>(src_tok), R, &ib, false, "src_tok"));
  CCR_TRY(check_rank_ptrs(ctx, exp, R, rb.data(), true, "exp"));
  std::vector<CallBuf> bufs;
  add_bufs(&bufs, x, R, &xb, false, false, "x");
  add_bufs(&bufs, reinterpret_cast<const void* const*>(src_tok), R, &ib, false, false, "src_tok");
  add_bufs(&bufs, exp, R, rb.data(), true, true, "exp");
  CCR_TRY(check_writes_disjoint(bufs));
  return moe_gather(ctx, 0, m, h_ecnt, const_cast<void* const*>(x), src_tok, exp,
                    static_cast<hipStream_t>(stream));
}

ccr_status_t ccr_moe_combine_fused(ccr_ctx_t ctx, const void* const* exp, const int32_t* const* slot,
                                   const int64_t* h_ecnt, int R, int64_t T, int E, int K,
                                   int64_t row_bytes, void* const* out, void* stream) {
  CCR_MARK("ccr_moe_combine_fused");
  MoeShape m;
  CCR_TRY(moe_shape(ctx, h_ecnt, R, T, E, K, row_bytes, &m));
  if (T == 0) return CCR_OK;
  const int64_t ob = T * K * row_bytes, ib = T * K * 4;
  std::vector<int64_t> rb((size_t)R, 0);
  for (int d = 0; d < R; d++)
    for (int r = 0; r < R; r++) rb[(size_t)d] += m.cnt[(size_t)r * R + d] * row_bytes;
  CCR_TRY(check_rank_ptrs(ctx, exp, R, rb.data(), true, "exp"));
  CCR_TRY(check_rank_ptrs(ctx, reinterpret_cast<const void* const*>(slot), R, &ib, false, "slot"));
  CCR_TRY(check_rank_ptrs(ctx, out, R, &ob, false, "out"));
  std::vector<CallBuf> bufs;
  add_bufs(&bufs, exp, R, rb.data(), true, false, "exp");
  add_bufs(&bufs, reinterpret_cast<const void* const*>(slot), R, &ib, false, false, "slot");
  add_bufs(&bufs, out, R, &ob, false, true, "out");
  CCR_TRY(check_writes_disjoint(bufs));
  return moe_gather(ctx, 1, m, h_ecnt, out, slot, const_cast<void* const*>(exp),
                    static_cast<hipStream_t>(stream));
}

ccr_status_t ccr_profile_enable(ccr_ctx_t ctx, int on) {
  CCR_TRY(check_ctx(ctx));
  HIP_TRY(hipDeviceSynchronize());
  for (auto& t : ctx->timed) {
    ctx->timing_pool.push_back(t.start);
    ctx->timing_pool.push_back(t.stop);
  }
  ctx->timed.clear();
  if (ctx->dma) {
    ctx->dma->drain(30.0);
    ctx->dma->reset_stats();
  }
  ctx->prof_on = on != 0;
  return CCR_OK;
}

ccr_status_t ccr_profile_intervals(ccr_ctx_t ctx, int kind, void* ref_event, double* start_ms,
                                  double* end_ms, int32_t* cus, int64_t max, int64_t* n) {
  CCR_TRY(check_ctx(ctx));
  if (!n || !ref_event) return fail(CCR_ERR_INVALID_ARG, "n or ref_event is NULL");
  if (kind < 0 || kind > 4) return fail(CCR_ERR_INVALID_ARG, "kind %d outside [0, 4]", kind);
  if (max < 0) return fail(CCR_ERR_INVALID_ARG, "max < 0");
  HIP_TRY(hipDeviceSynchronize());
  if (ctx->dma) ctx->dma->drain(30.0);
  hipEvent_t ref = static_cast<hipEvent_t>(ref_event);
  int64_t k = 0;
  for (const auto& t : ctx->timed) {
    if (t.kind != kind) continue;
    if (k < max) {
      float a = 0.f, b = 0.f;
      HIP_TRY(hipEventElapsedTime(&a, ref, t.start));
      HIP_TRY(hipEventElapsedTime(&b, ref, t.stop));
      if (start_ms) start_ms[k] = a;
      if (end_ms) end_ms[k] = b;
      if (cus) cus[k] = t.cus;
    }
    k++;
  }
  *n = k;
  return CCR_OK;
}

ccr_status_t ccr_ctx_streams(ccr_ctx_t ctx, int32_t* masked, int32_t* plain) {
  if (!ctx) return fail(CCR_ERR_INVALID_ARG, "ctx is NULL");
  if (masked) *masked = (ctx->s_a ? 1 : 0) + (ctx->s_b ? 1 : 0);
  if (plain) *plain = ctx->s_cap ? 1 : 0;
  return CCR_OK;
}

ccr_status_t ccr_graph_cache_stats(ccr_ctx_t ctx, int64_t* graphs, int64_t* replays) {
  if (!ctx) return fail(CCR_ERR_INVALID_ARG, "ctx is NULL");
  int64_t n = 0;
  for (const auto& g : ctx->graphs) n += g.exec != nullptr;
  if (graphs) *graphs = n;
  if (replays) *replays = ctx->graph_replays;
  return CCR_OK;
}

int32_t ccr_dma_pace(int64_t bytes, int64_t deadline_us, double engine_gbs, int32_t max_engines) {
  if (max_engines < 1) return 0;
  if (deadline_us <= 0 || !(engine_gbs > 0) || bytes <= 0) return max_engines;
  const double per_engine = (double)deadline_us * 1e-6 * engine_gbs * 1e9;  // bytes in the deadline
  const double need = std::ceil((double)bytes / per_engine);
  return need >= (double)max_engines ? max_engines : std::max<int32_t>(1, (int32_t)need);
}

ccr_status_t ccr_dma_rate(ccr_ctx_t ctx, double* engine_gbs, int32_t* last_engines) {
  CCR_TRY(check_ctx(ctx));
  if (!engine_gbs || !last_engines) return fail(CCR_ERR_INVALID_ARG, "engine_gbs or last_engines is NULL");
  CCR_TRY(ensure_dma(ctx));
  *engine_gbs = ctx->dma->engine_gbs();
  *last_engines = ctx->last_dma_engines;
  return CCR_OK;
}

ccr_status_t ccr_dma_info(ccr_ctx_t ctx, int32_t* n, int32_t* ids) {
  CCR_TRY(check_ctx(ctx));
  if (!n) return fail(CCR_ERR_INVALID_ARG, "n is NULL");
  CCR_TRY(ensure_dma(ctx));
  *n = ctx->dma->engine_count();
  if (ids)
    for (int i = 0; i < *n; i++) ids[i] = ctx->dma->engine_id(i);
  return CCR_OK;
}

ccr_status_t ccr_sendrecv_slot_log(ccr_ctx_t ctx, int32_t* out, int64_t max_events, int64_t* n) {
  CCR_TRY(check_ctx(ctx));
  if (!n || max_events < 0) return fail(CCR_ERR_INVALID_ARG, "n is NULL or max_events < 0");
  *n = 0;
  if (!ctx->dma) return CCR_OK;
  if (!ctx->dma->drain(30.0)) return fail(CCR_ERR_TIMEOUT, "SDMA operations still running after 30 s");
  const std::vector<SlotEvent> log = ctx->dma->last_slot_log();
  *n = (int64_t)log.size();
  for (int64_t i = 0; out && i < std::min<int64_t>(max_events, *n); i++) {
    out[3 * i] = log[(size_t)i].chunk;
    out[3 * i + 1] = log[(size_t)i].slot;
    out[3 * i + 2] = log[(size_t)i].state;
  }
  return CCR_OK;
}

ccr_status_t ccr_stream_wait(ccr_ctx_t ctx, void* stream, int timeout_ms) {
  CCR_TRY(check_ctx(ctx));
  if (timeout_ms < 0) return fail(CCR_ERR_INVALID_ARG, "timeout_ms < 0");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    const hipError_t e = hipStreamQuery(s);
    if (e == hipSuccess) break;
    if (e != hipErrorNotReady) return hip_fail(e, "hipStreamQuery");
    const double ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (ms > timeout_ms)
      return fail(CCR_ERR_TIMEOUT, "stream work not complete after %d ms", timeout_ms);
    std::this_thread::sleep_for(std::chrono::microseconds(50));
  }
  if (ctx->dma) {
    const std::string e = ctx->dma->take_error();
    if (!e.empty()) return fail(CCR_ERR_HIP, "SDMA proxy: %s", e.c_str());
  }
  return CCR_OK;
}

ccr_status_t ccr_dma_hold_finish(ccr_ctx_t ctx, int us) {
  CCR_TRY(check_ctx(ctx));
  if (us < 0 || us > 10000000) return fail(CCR_ERR_INVALID_ARG, "us outside [0, 10 s]");
  CCR_TRY(ensure_dma(ctx));
  ctx->dma->set_finish_delay_us(us);
  return CCR_OK;
}


ccr_status_t ccr_profile_read(ccr_ctx_t ctx, int kind, ccr_kernel_stats_t* out) {
  CCR_TRY(check_ctx(ctx));
  if (!out || kind < 0 || kind > 4) return fail(CCR_ERR_INVALID_ARG, "out is NULL or kind outside [0, 4]");
  HIP_TRY(hipDeviceSynchronize());
  ccr_kernel_stats_t st{0, 0, 0.0};
  if (kind == kProfSdma) {
    if (ctx->dma) {
      ctx->dma->drain(30.0);
      const DmaStats d = ctx->dma->stats();
      *out = ccr_kernel_stats_t{d.jobs, d.bytes, d.ms};
    } else {
      *out = st;
    }
    return CCR_OK;
  }
  for (const auto& t : ctx->timed) {
    if (t.kind != kind) continue;
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, t.start, t.stop));
    st.launches++;
    st.bytes += t.bytes;
    st.ms += ms;
  }
  *out = st;
  return CCR_OK;
}

ccr_status_t ccr_probe_cu_ids(ccr_ctx_t ctx, int32_t* out, int nblocks, void* stream) {
  CCR_TRY(check_ctx(ctx));
  if (nblocks < 0 || nblocks > (1 << 20)) return fail(CCR_ERR_INVALID_ARG, "nblocks outside [0, 2^20]");
  if (nblocks == 0) return CCR_OK;
  CCR_TRY(check_dev_ptr(ctx, out, (int64_t)nblocks * 12, "out", 0));
  hipStream_t caller = static_cast<hipStream_t>(stream);
  hipStream_t s;
  if (ctx->masked) CCR_TRY(work_stream(ctx, caller, &s));
  else CCR_TRY(side_a(ctx, &s));
  CCR_TRY(order_after(ctx, 0, caller, s));
  HIP_TRY(launch_probe_cu_ids(out, nblocks, s));
  CCR_TRY(order_after(ctx, 1, s, caller));
  return CCR_OK;
}

}  // extern "C"
