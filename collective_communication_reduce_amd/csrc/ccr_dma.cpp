// SDMA engines driven by a CPU proxy thread; see ccr_dma.h.

#include "ccr_dma.h"

#include <immintrin.h>

#include <atomic>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace ccr {
namespace {

constexpr int kFlagSlots = 256;            // flag-word slots in the process (jobs in flight at once)
constexpr int kFlagStride = 32;            // words between flag words (one 128-byte line each)
// Engines gfx950 offers for device-to-device copies when the runtime cannot
// report them itself (engines 0 and 1 serve host transfers).
constexpr uint32_t kFallbackEngineMask = 0xfffcu;

using clk = std::chrono::steady_clock;

// The process's flag words: coherent pinned host memory, allocated on first
// use and kept until the process ends (a stream may read a slot's done word
// long after the proxy that used the slot is gone), shared by every proxy.
FlagWords* flag_words(std::string* err) {
  static std::mutex mu;
  static FlagWords* pool = nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (pool) return pool;
  uint32_t* mem = nullptr;
  const size_t bytes = sizeof(uint32_t) * kFlagStride * 2 * kFlagSlots;
  if (hipHostMalloc(reinterpret_cast<void**>(&mem), bytes, hipHostMallocCoherent | hipHostMallocMapped) !=
      hipSuccess) {
    (void)hipGetLastError();
    *err = "hipHostMalloc of the flag words failed";
    return nullptr;
  }
  memset(mem, 0, bytes);
  pool = new FlagWords(mem, kFlagSlots, kFlagStride);
  return pool;
}

double seconds_since(clk::time_point t) {
  return std::chrono::duration<double>(clk::now() - t).count();
}

struct AgentSearch {
  uint32_t bus_dev;  // (bus << 5) | device
  uint32_t domain;
  int want_index;    // fallback: the n-th GPU agent
  int seen = 0;
  hsa_agent_t by_bdf{}, by_index{};
  bool bdf_ok = false, index_ok = false;
};

hsa_status_t match_agent(hsa_agent_t a, void* data) {
  auto* s = static_cast<AgentSearch*>(data);
  hsa_device_type_t t;
  if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) != HSA_STATUS_SUCCESS ||
      t != HSA_DEVICE_TYPE_GPU)
    return HSA_STATUS_SUCCESS;
  if (s->seen++ == s->want_index) {
    s->by_index = a;
    s->index_ok = true;
  }
  uint32_t bdf = 0, dom = 0;
  if (hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_BDFID, &bdf) ==
          HSA_STATUS_SUCCESS &&
      hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_DOMAIN, &dom) ==
          HSA_STATUS_SUCCESS &&
      (bdf >> 3) == s->bus_dev && dom == s->domain && !s->bdf_ok) {
    s->by_bdf = a;
    s->bdf_ok = true;
  }
  return HSA_STATUS_SUCCESS;
}

int64_t align16(int64_t x) { return (x + 15) & ~int64_t(15); }

}  // namespace

struct DmaProxy::Job {
  enum Kind { kCopies, kStaged } kind = kCopies;
  enum State { kQueued, kRunning } state = kQueued;
  DmaSync sync = DmaSync::kHostFunc;
  GateBlock* gate = nullptr;  // kHostFunc: shared with the stream's host function
  FlagWords* flags = nullptr;  // kStreamFlags: the slot and sequence number
  int flag = -1;
  uint32_t seq = 0;
  bool aborted = false;  // hand-over only partly enqueued: release without copying
  bool failed = false;   // an issue call failed: stop issuing, drain what was issued
  clk::time_point t0;
  int64_t bytes = 0, ncopies = 0;
  // kCopies
  std::vector<DmaCopy> copies;
  int max_engines = 0;             // engines a copy with engine -1 may use; 0 = all
  std::vector<int32_t> eng;        // per copy: the engine it was issued on
  std::vector<hsa_signal_t> sig;   // per copy; handle 0 until issued
  std::vector<int32_t> kid_start;  // copies that wait for copy i: kids[kid_start[i] .. kid_start[i+1])
  std::vector<int32_t> kids;
  std::vector<int32_t> inflight;   // issued, not yet seen complete
  int64_t ndone = 0;
  // kStaged
  StagedPlan plan;
  struct Slot {
    int state = 0;
    int64_t chunk = -1;
    std::vector<hsa_signal_t> sigs;
  };
  std::vector<Slot> slots;
  int64_t next_chunk = 0, done_chunks = 0, total_chunks = 0, chunks_per_transfer = 0;
  std::vector<SlotEvent> log;
};

DmaProxy::~DmaProxy() { (void)close(10.0); }

DmaClose DmaProxy::close(double timeout_s) {
  if (!started_ || closed_) return DmaClose::kClean;
  closed_ = true;
  DmaClose how = DmaClose::kClean;
  if (!drain(timeout_s)) {
    // Streams that never reached their jobs (e.g. held behind other work):
    // drop those jobs, releasing each stream for whenever it gets there.
    abandon_queued_.store(true);
    if (!drain(timeout_s)) {
      std::lock_guard<std::mutex> lk(mu_);
      give_up_ = true;
      how = DmaClose::kInFlight;
    }
  }
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_ = true;
    if (how == DmaClose::kClean && abandoned_ > 0) how = DmaClose::kAbandoned;
  }
  cv_.notify_all();
  if (thread_.joinable()) thread_.join();
  // Signals of copies still in flight belong to jobs that were given up
  // (leaked with them); the pool holds only completed ones.
  for (hsa_signal_t s : signal_pool_) hsa_signal_destroy(s);
  signal_pool_.clear();
  return how;
}

void DmaProxy::note_error(const std::string& e) {
  std::lock_guard<std::mutex> lk(mu_);
  if (error_.empty()) error_ = e;
}

std::string DmaProxy::take_error() {
  std::lock_guard<std::mutex> lk(mu_);
  std::string e;
  e.swap(error_);
  return e;
}

bool DmaProxy::start(int device, std::string* err) {
  if (started_) return true;
  if (hsa_init() != HSA_STATUS_SUCCESS) {
    *err = "hsa_init failed";
    return false;
  }
  int bus = 0, dev = 0, dom = 0;
  if (hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, device) != hipSuccess ||
      hipDeviceGetAttribute(&dev, hipDeviceAttributePciDeviceId, device) != hipSuccess ||
      hipDeviceGetAttribute(&dom, hipDeviceAttributePciDomainId, device) != hipSuccess) {
    (void)hipGetLastError();
    *err = "cannot read the device's PCI location";
    return false;
  }
  AgentSearch s;
  s.bus_dev = ((uint32_t)bus << 5) | (uint32_t)dev;
  s.domain = (uint32_t)dom;
  s.want_index = device;
  hsa_iterate_agents(match_agent, &s);
  if (!s.bdf_ok && !s.index_ok) {
    *err = "no HSA GPU agent for the device";
    return false;
  }
  agent_ = s.bdf_ok ? s.by_bdf : s.by_index;

  uint32_t mask = 0;
  if (hsa_amd_memory_copy_engine_status(agent_, agent_, &mask) != HSA_STATUS_SUCCESS || mask == 0)
    mask = kFallbackEngineMask;

  // Warm every engine: the first copy on an engine sets up its queue and is
  // slow (milliseconds); keep only engines whose warm-up copy completes.
  char* scratch = nullptr;
  if (hipMalloc(reinterpret_cast<void**>(&scratch), 8192) != hipSuccess) {
    (void)hipGetLastError();
    *err = "hipMalloc of the engine warm-up buffer failed";
    return false;
  }
  (void)hipMemset(scratch, 0, 8192);
  (void)hipDeviceSynchronize();
  bool any_stuck = false;
  for (int e = 0; e < 16; e++) {
    if (!(mask & (1u << e))) continue;
    hsa_signal_t sg;
    if (hsa_signal_create(1, 0, nullptr, &sg) != HSA_STATUS_SUCCESS) continue;
    const hsa_status_t st = hsa_amd_memory_async_copy_on_engine(
        scratch + 4096, agent_, scratch, agent_, 4096, 0, nullptr, sg,
        (hsa_amd_sdma_engine_id_t)(1u << e), true);
    bool ok = st == HSA_STATUS_SUCCESS;
    if (ok) {
      const auto t = clk::now();
      while (hsa_signal_load_scacquire(sg) > 0) {
        if (seconds_since(t) > 20.0) {
          ok = false;
          any_stuck = true;
          break;
        }
        std::this_thread::yield();
      }
    }
    if (ok) engines_.push_back(e);
    if (!any_stuck) hsa_signal_destroy(sg);
  }
  if (!any_stuck) (void)hipFree(scratch);  // else an engine may still write it
  if (engines_.empty()) {
    *err = "no usable SDMA engine for device-to-device copies";
    return false;
  }
  load_.assign(engines_.size(), 0);
  measure_engine_rate();
  thread_ = std::thread(&DmaProxy::loop, this);
  started_ = true;
  return true;
}

// A staged job moves chunk after chunk through its slots; beyond its bytes
// at the engines' rate, each chunk step costs a fixed time (copy issue and
// completion, the slot hand-over).  Keep that per-step cost of the last
// completed job, for pacing staged transfers by a deadline.
void DmaProxy::note_staged(const Job& j, double elapsed_s) {
  const StagedPlan& p = j.plan;
  const int n_eng = p.engines > 0 ? std::min(p.engines, (int)engines_.size()) : (int)engines_.size();
  const int stripe = std::max(1, std::min(p.stripe, n_eng));
  if (!(engine_gbs_ > 0) || j.total_chunks <= 0) return;
  const double step_us = elapsed_s * 1e6 / (double)j.total_chunks;
  const double copy_us = (double)p.chunk / ((double)stripe * engine_gbs_ * 1e3);
  staged_step_us_.store(std::max(0.0, step_us - copy_us));
}

// One engine's device-to-device rate, for pacing calls by a deadline: a
// 16 MiB copy on the first usable engine (already warm), nothing else
// running.  Left at 0 (no pacing) if the copy cannot be made or timed.
void DmaProxy::measure_engine_rate() {
  constexpr int64_t kBytes = int64_t(16) << 20;
  char* buf = nullptr;
  if (hipMalloc(reinterpret_cast<void**>(&buf), (size_t)(2 * kBytes)) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  (void)hipMemset(buf, 0, (size_t)(2 * kBytes));
  (void)hipDeviceSynchronize();
  hsa_signal_t sg;
  if (hsa_signal_create(1, 0, nullptr, &sg) != HSA_STATUS_SUCCESS) {
    (void)hipFree(buf);
    return;
  }
  const auto t = clk::now();
  bool ok = hsa_amd_memory_async_copy_on_engine(buf + kBytes, agent_, buf, agent_, (size_t)kBytes, 0,
                                                nullptr, sg,
                                                (hsa_amd_sdma_engine_id_t)(1u << engines_[0]),
                                                true) == HSA_STATUS_SUCCESS;
  bool stuck = false;
  while (ok && hsa_signal_load_scacquire(sg) > 0) {
    if (seconds_since(t) > 20.0) {
      stuck = ok = false;
      break;
    }
  }
  const double s = seconds_since(t);
  if (ok && s > 0) engine_gbs_ = (double)kBytes / s * 1e-9;
  if (!stuck) {  // else the engine may still write the buffer
    hsa_signal_destroy(sg);
    (void)hipFree(buf);
  }
}

// The host-function gate: runs on the runtime's callback thread when the
// stream reaches it and holds the stream until the proxy releases it (or
// returns at once for a job the proxy has abandoned).
void DmaProxy::gate(void* p) { (void)GateBlock::arrive_and_wait(static_cast<GateBlock*>(p)); }

bool DmaProxy::submit(Job* j, hipStream_t stream, std::string* err) {
  if (j->sync == DmaSync::kHostFunc) {
    j->gate = GateBlock::make();
    const hipError_t e = hipLaunchHostFunc(stream, &DmaProxy::gate, j->gate);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      *err = std::string("hipLaunchHostFunc failed: ") + hipGetErrorString(e);
      (void)GateBlock::abandon(j->gate);  // the job's reference
      (void)GateBlock::arrive_and_wait(j->gate);  // the callback's, which will never run
      delete j;
      return false;
    }
  } else {
    j->flags = flag_words(err);
    if (!j->flags) {
      delete j;
      return false;
    }
    if (!j->flags->take(&j->flag, &j->seq, std::chrono::seconds(30))) {
      *err = "no free flag slot within 30 s (DMA operations are not completing)";
      delete j;
      return false;
    }
    hipError_t e = hipStreamWriteValue32(stream, j->flags->req(j->flag), j->seq, 0);
    if (e != hipSuccess) {  // nothing enqueued
      (void)hipGetLastError();
      *err = std::string("hipStreamWriteValue32 failed: ") + hipGetErrorString(e);
      j->flags->complete(j->flag, j->seq);
      delete j;
      return false;
    }
    e = hipStreamWaitValue32(stream, j->flags->done(j->flag), j->seq, hipStreamWaitValueGte,
                             0xffffffffu);
    if (e != hipSuccess) {
      // the request is enqueued: hand the job over marked aborted, so the
      // proxy answers the request without copying
      (void)hipGetLastError();
      *err = std::string("hipStreamWaitValue32 failed: ") + hipGetErrorString(e);
      j->aborted = true;
      note_error(*err);
    }
  }
  const bool aborted = j->aborted;
  {
    std::lock_guard<std::mutex> lk(mu_);
    incoming_.push_back(j);
    pending_++;
  }
  cv_.notify_one();
  return !aborted;
}

bool DmaProxy::submit_copies(std::vector<DmaCopy> copies, hipStream_t stream, DmaSync sync,
                             std::string* err, int max_engines) {
  if (copies.empty()) return true;
  Job* j = new Job();
  j->kind = Job::kCopies;
  j->sync = sync;
  j->max_engines = max_engines;
  for (const DmaCopy& c : copies) j->bytes += c.bytes;
  j->ncopies = (int64_t)copies.size();
  j->copies = std::move(copies);
  return submit(j, stream, err);
}

bool DmaProxy::submit_staged(const StagedPlan& plan, hipStream_t stream, DmaSync sync,
                             std::string* err) {
  if (plan.src.empty() || plan.nbytes == 0) return true;
  Job* j = new Job();
  j->kind = Job::kStaged;
  j->sync = sync;
  j->plan = plan;
  j->chunks_per_transfer = (plan.nbytes + plan.chunk - 1) / plan.chunk;
  j->total_chunks = j->chunks_per_transfer * (int64_t)plan.src.size();
  j->bytes = 2 * plan.nbytes * (int64_t)plan.src.size();
  return submit(j, stream, err);
}

bool DmaProxy::drain(double timeout_s) {
  std::unique_lock<std::mutex> lk(mu_);
  return freed_.wait_for(lk, std::chrono::duration<double>(timeout_s), [&] { return pending_ == 0; });
}

DmaStats DmaProxy::stats() {
  std::lock_guard<std::mutex> lk(mu_);
  return stats_;
}

void DmaProxy::reset_stats() {
  std::lock_guard<std::mutex> lk(mu_);
  stats_ = DmaStats();
}

std::vector<SlotEvent> DmaProxy::last_slot_log() {
  std::lock_guard<std::mutex> lk(mu_);
  return slot_log_;
}

hsa_signal_t DmaProxy::get_signal() {
  hsa_signal_t s;
  if (!signal_pool_.empty()) {
    s = signal_pool_.back();
    signal_pool_.pop_back();
  } else if (hsa_signal_create(1, 0, nullptr, &s) != HSA_STATUS_SUCCESS) {
    s.handle = 0;
    return s;
  }
  hsa_signal_store_relaxed(s, 1);
  return s;
}

void DmaProxy::put_signal(hsa_signal_t s) {
  if (s.handle) signal_pool_.push_back(s);
}

bool DmaProxy::issue(char* dst, const char* src, int64_t bytes, hsa_signal_t done, int engine) {
  if (!done.handle) return false;
  const int e = engines_[(size_t)engine % engines_.size()];
  return hsa_amd_memory_async_copy_on_engine(dst, agent_, src, agent_, (size_t)bytes, 0, nullptr,
                                             done, (hsa_amd_sdma_engine_id_t)(1u << e),
                                             true) == HSA_STATUS_SUCCESS;
}

// The allowed engine with the fewest bytes outstanding (the lowest index on
// a tie).
int DmaProxy::least_loaded(int max_engines) const {
  const int n = max_engines > 0 ? std::min(max_engines, (int)engines_.size()) : (int)engines_.size();
  int best = 0;
  for (int e = 1; e < n; e++)
    if (load_[(size_t)e] < load_[(size_t)best]) best = e;
  return best;
}

bool DmaProxy::start_copy(Job& j, int32_t i) {
  const DmaCopy& c = j.copies[(size_t)i];
  const int e = c.engine >= 0 ? c.engine % (int)engines_.size() : least_loaded(j.max_engines);
  hsa_signal_t s = get_signal();
  if (!issue(c.dst, c.src, c.bytes, s, e)) {
    put_signal(s);
    j.failed = true;
    note_error("an SDMA copy could not be issued");
    return false;
  }
  j.sig[(size_t)i] = s;
  j.eng[(size_t)i] = e;
  load_[(size_t)e] += c.bytes;
  j.inflight.push_back(i);
  return true;
}

// A copy job starts with the copies that wait for nothing; the proxy issues
// each remaining copy once the copy it waits for has completed.  Chains are
// kept on the host on purpose: expressed as HSA dependency signals, a chain
// makes its engine wait on the signal itself, and with chains on many
// engines at once that waiting slowed a concurrent GEMM by 2x and the
// copies themselves by two orders of magnitude on gfx950.
void DmaProxy::begin(Job& j) {
  if (j.kind == Job::kCopies) {
    const size_t n = j.copies.size();
    j.sig.assign(n, hsa_signal_t{0});
    j.eng.assign(n, 0);
    j.kid_start.assign(n + 1, 0);
    for (size_t i = 0; i < n; i++) {
      const int32_t a = j.copies[i].after;
      if (a >= (int32_t)i) {  // a copy can only wait for an earlier one
        j.failed = true;
        note_error("an SDMA copy waits for a later copy of its job");
        return;
      }
      if (a >= 0) j.kid_start[(size_t)a + 1]++;
    }
    for (size_t i = 0; i < n; i++) j.kid_start[i + 1] += j.kid_start[i];
    j.kids.assign((size_t)j.kid_start[n], 0);
    std::vector<int32_t> fill(j.kid_start.begin(), j.kid_start.end() - 1);
    for (size_t i = 0; i < n; i++)
      if (const int32_t a = j.copies[i].after; a >= 0) j.kids[(size_t)fill[(size_t)a]++] = (int32_t)i;
    for (size_t i = 0; i < n && !j.failed; i++)
      if (j.copies[i].after < 0) start_copy(j, (int32_t)i);
    return;
  }
  j.slots.assign((size_t)j.plan.slots, Job::Slot());
}

// Progress a running job; true once every issued copy has completed and
// nothing is left to issue.
bool DmaProxy::advance(Job& j) {
  if (j.kind == Job::kCopies) {
    std::vector<int32_t> running;
    running.swap(j.inflight);
    for (size_t k = 0; k < running.size(); k++) {
      const int32_t i = running[k];
      if (hsa_signal_load_scacquire(j.sig[(size_t)i]) > 0) {
        j.inflight.push_back(i);
        continue;
      }
      j.ndone++;
      load_[(size_t)j.eng[(size_t)i]] -= j.copies[(size_t)i].bytes;
      for (int32_t q = j.kid_start[(size_t)i]; q < j.kid_start[(size_t)i + 1] && !j.failed; q++)
        start_copy(j, j.kids[(size_t)q]);
    }
    if (j.failed) return j.inflight.empty();  // finish once nothing issued is running
    return j.ndone == (int64_t)j.copies.size();
  }
  // Staged transfer: the per-slot state machine (idle -> filling ->
  // draining -> idle); chunk i always uses slot i mod slots.
  const StagedPlan& p = j.plan;
  const int n_eng = p.engines > 0 ? std::min(p.engines, (int)engines_.size()) : (int)engines_.size();
  const int stripe = std::max(1, std::min(p.stripe, n_eng));
  const int drain_base = n_eng >= 2 * stripe ? n_eng / 2 : 0;
  auto all_done = [](const std::vector<hsa_signal_t>& v) {
    for (hsa_signal_t s : v)
      if (hsa_signal_load_scacquire(s) > 0) return false;
    return true;
  };
  auto striped = [&](Job::Slot& sl, char* dst, const char* src, int64_t len, int base) {
    const int64_t part = align16((len + stripe - 1) / stripe);
    for (int k = 0; k < stripe && !j.failed; k++) {
      const int64_t lo = std::min<int64_t>(len, k * part), hi = std::min<int64_t>(len, (k + 1) * part);
      if (hi <= lo) break;
      hsa_signal_t s = get_signal();
      if (!issue(dst + lo, src + lo, hi - lo, s, base + k)) {
        put_signal(s);
        j.failed = true;
        note_error("an SDMA staging copy could not be issued");
        break;
      }
      sl.sigs.push_back(s);
      j.ncopies++;
    }
  };
  auto chunk_io = [&](int64_t c, int64_t* m, int64_t* off, int64_t* len) {
    *m = c / j.chunks_per_transfer;
    *off = (c % j.chunks_per_transfer) * p.chunk;
    *len = std::min<int64_t>(p.chunk, p.nbytes - *off);
  };
  for (int s = 0; s < p.slots; s++) {
    Job::Slot& sl = j.slots[(size_t)s];
    if (sl.state == 0 || !all_done(sl.sigs)) continue;
    for (hsa_signal_t x : sl.sigs) put_signal(x);
    sl.sigs.clear();
    if (sl.state == 1) {  // filled -> draining
      sl.state = 2;
      j.log.push_back(SlotEvent{(int32_t)sl.chunk, s, 2});
      if (!j.failed) {
        int64_t m, off, len;
        chunk_io(sl.chunk, &m, &off, &len);
        striped(sl, p.dst[(size_t)m] + off, p.slot_mem + (int64_t)s * p.chunk, len, drain_base);
      }
    } else {  // drained -> idle
      sl.state = 0;
      j.log.push_back(SlotEvent{(int32_t)sl.chunk, s, 0});
      j.done_chunks++;
    }
  }
  while (!j.failed && j.next_chunk < j.total_chunks) {
    const int s = (int)(j.next_chunk % p.slots);
    Job::Slot& sl = j.slots[(size_t)s];
    if (sl.state != 0) break;  // chunks fill in order; wait for this slot
    sl.state = 1;
    sl.chunk = j.next_chunk++;
    j.log.push_back(SlotEvent{(int32_t)sl.chunk, s, 1});
    int64_t m, off, len;
    chunk_io(sl.chunk, &m, &off, &len);
    striped(sl, p.slot_mem + (int64_t)s * p.chunk, p.src[(size_t)m] + off, len, 0);
  }
  if (j.failed) {  // finish once nothing issued is still running
    for (const Job::Slot& sl : j.slots)
      if (!all_done(sl.sigs)) return false;
    return true;
  }
  return j.done_chunks == j.total_chunks;
}

// Has the job's stream reached the communication point?
bool DmaProxy::arrived(Job& j) {
  return j.sync == DmaSync::kStreamFlags ? j.flags->requested(j.flag, j.seq) : j.gate->state() == 1;
}

// Drop a job whose stream has not arrived (shutdown); false if it has.
bool DmaProxy::try_abandon(Job& j) {
  if (j.sync == DmaSync::kStreamFlags) {
    if (j.flags->requested(j.flag, j.seq)) return false;
    j.flags->abandon(j.flag);  // the stream passes whenever it gets there; slot retired
    return true;
  }
  return GateBlock::abandon(j.gate);
}

// Let the job's stream go on.  `abandoned`: its copies may not have run
// (shutdown), so a flag slot is retired rather than reused.
void DmaProxy::release(Job& j, bool abandoned) {
  if (j.sync == DmaSync::kStreamFlags) {
    if (abandoned) j.flags->abandon(j.flag);
    else j.flags->complete(j.flag, j.seq);
  } else {
    GateBlock::release(j.gate);
  }
}

void DmaProxy::loop() {
  int idle = 0;  // polls in a row without progress
  for (;;) {
    {
      std::unique_lock<std::mutex> lk(mu_);
      while (!incoming_.empty()) {
        active_.push_back(incoming_.front());
        incoming_.pop_front();
      }
      if (give_up_) {
        // Shutdown after the timeouts: release every stream still held.
        // Jobs with copies in flight are leaked with their signals (an
        // engine may still complete them).
        for (Job* j : active_) {
          if (j->state == Job::kQueued) {
            if (try_abandon(*j)) {
              abandoned_++;
              delete j;
              continue;
            }
          }
          release(*j, true);
        }
        active_.clear();
        pending_ = 0;
        freed_.notify_all();
        return;
      }
      if (active_.empty()) {
        if (stop_) return;
        cv_.wait_for(lk, std::chrono::milliseconds(20));
        continue;
      }
    }
    const bool abandon = abandon_queued_.load();
    bool progress = false;
    for (auto it = active_.begin(); it != active_.end();) {
      Job& j = **it;
      bool finished = false;
      if (j.state == Job::kQueued) {
        if (arrived(j)) {
          j.t0 = clk::now();
          if (!j.aborted) begin(j);
          j.state = Job::kRunning;
          progress = true;
        } else if (abandon && try_abandon(j)) {
          std::lock_guard<std::mutex> lk(mu_);
          abandoned_++;
          finished = true;
        }
      }
      if (!finished && j.state == Job::kRunning && (j.aborted || advance(j))) {
        if (j.kind == Job::kStaged && !j.aborted && !j.failed) note_staged(j, seconds_since(j.t0));
        if (const int d = finish_delay_us_.load(); d > 0)
          std::this_thread::sleep_for(std::chrono::microseconds(d));
        {
          std::lock_guard<std::mutex> lk(mu_);
          if (!j.aborted && !j.failed) {
            stats_.jobs++;
            stats_.copies += j.kind == Job::kCopies ? (int64_t)j.sig.size() : j.ncopies;
            stats_.bytes += 2 * j.bytes;
            stats_.ms += 1e3 * seconds_since(j.t0);
          }
          if (j.kind == Job::kStaged) slot_log_ = j.log;
        }
        for (hsa_signal_t x : j.sig)
          if (x.handle) put_signal(x);
        j.sig.clear();
        release(j, false);
        finished = true;
      }
      if (finished) {
        {
          std::lock_guard<std::mutex> lk(mu_);
          pending_--;
        }
        freed_.notify_all();
        delete &j;
        it = active_.erase(it);
        progress = true;
        continue;
      }
      ++it;
    }
    // Spin while copies are short; on a long one, give the core away between
    // polls (after ~4096 idle polls) so the proxy does not hold a CPU busy.
    if (progress) idle = 0;
    else if (++idle < 4096) _mm_pause();
    else std::this_thread::yield();
  }
}

}  // namespace ccr
