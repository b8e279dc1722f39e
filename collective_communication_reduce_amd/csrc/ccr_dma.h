// SDMA engines driven by a CPU proxy thread, synchronised with HIP streams.
//
// Method: "HOCCL: Offloading Collective Communication from GPU Cores to
// Accelerate Distributed Training".  When a stream reaches a communication
// point, the CPU takes over: a proxy thread drives the DMA engines and lets
// the stream continue once the copies are done, so communication keeps its
// place in the stream order (§3.2 Stream Manager, Fig. 4).  Staging slots
// move through a three-state machine, and chunks are spread over several
// engines so more than one is in flight (§3.3.1 chunk pipelining and
// multi-QP striping; §3.4 flow-size-aware chunk schedule).
//
// On gfx950 the copies run on the SDMA engines through
// hsa_amd_memory_async_copy_on_engine(force_copy_on_sdma = true): no compute
// unit touches the data.  Two ways tie a job to the stream (ccr_handoff.h):
//  - kHostFunc (default): the stream reaches a hipLaunchHostFunc gate, which
//    announces the arrival and blocks until the proxy releases it; the
//    stream waits on the host function's completion signal, with no
//    GPU-side polling.
//  - kStreamFlags: the stream writes a request word with
//    hipStreamWriteValue32 and waits with hipStreamWaitValue32 until the
//    proxy's done word reaches the job's sequence number.  This HIP runtime
//    runs those operations as kernels, and a stream parked in
//    hipStreamWaitValue32 for the length of a DMA slows a concurrent GEMM by
//    tens of percent, so it is an option, not the default.
#pragma once

#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <list>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "ccr_handoff.h"

namespace ccr {

// One copy of a job.  `after` indexes an earlier copy of the same job that
// must have finished before this one starts (-1: none); the proxy issues the
// copy when that one completes.  `engine` indexes the proxy's engine list;
// -1 lets the proxy issue the copy, when it is ready, on whichever of the
// job's engines has the fewest bytes outstanding.
struct DmaCopy {
  char* dst;
  const char* src;
  int64_t bytes;
  int32_t after;
  int32_t engine;
};

// Point-to-point transfers through the slot pool: transfer m moves nbytes
// from src[m] to dst[m]; chunk i (over all transfers in order) uses slot
// i mod slots.  Each fill / drain is striped over `stripe` engines.
struct StagedPlan {
  std::vector<const char*> src;
  std::vector<char*> dst;
  int64_t nbytes = 0;
  int64_t chunk = 0;
  int slots = 0;
  char* slot_mem = nullptr;
  int stripe = 1;
  int engines = 0;  // engines the job may use (the first of the proxy's list); 0 = all
};

// One slot transition of a staged job: state 0 idle, 1 filling, 2 draining.
struct SlotEvent {
  int32_t chunk, slot, state;
};

struct DmaStats {
  int64_t jobs = 0, copies = 0, bytes = 0;
  double ms = 0;  // sum over jobs of (start acknowledged -> last copy done)
};

enum class DmaSync { kHostFunc = 0, kStreamFlags = 1 };

// How a proxy's shutdown went: every job done; some jobs abandoned before
// their streams reached them (their streams are released without copies,
// nothing else is affected); or copies possibly still in flight after the
// timeouts (their streams were released, and the memory they write --
// caller buffers, staging slots -- must be kept).
enum class DmaClose { kClean = 0, kAbandoned = 1, kInFlight = 2 };

class DmaProxy {
 public:
  DmaProxy() = default;
  DmaProxy(const DmaProxy&) = delete;
  DmaProxy& operator=(const DmaProxy&) = delete;
  ~DmaProxy();

  // Find HIP device `device`'s HSA agent and its SDMA engines, warm every
  // engine with a small copy, start the thread.
  bool start(int device, std::string* err);
  // Stop the proxy: wait up to timeout_s for the submitted jobs; then
  // abandon the jobs whose streams have not arrived and wait as long again
  // for the running ones; then release every stream that still waits and
  // stop.  Idempotent (the destructor calls it with 10 s).
  DmaClose close(double timeout_s);
  int engine_count() const { return (int)engines_.size(); }
  int engine_id(int i) const { return engines_[(size_t)i]; }
  // One engine's device-to-device copy rate measured at start (GB/s; 0 if
  // it could not be measured).
  double engine_gbs() const { return engine_gbs_; }
  // Fixed time per chunk step of the last completed staged job, beyond its
  // bytes at engine_gbs() (microseconds; 0 before any).
  double staged_step_us() const { return staged_step_us_.load(); }

  // Enqueue on `stream` the hand-over of a job and give the job to the
  // proxy.  Returns false (with *err) if nothing could be enqueued.
  // max_engines: the engines (the first of the proxy's list) that copies
  // with engine -1 may go to; 0 = all.
  bool submit_copies(std::vector<DmaCopy> copies, hipStream_t stream, DmaSync sync,
                     std::string* err, int max_engines = 0);
  bool submit_staged(const StagedPlan& plan, hipStream_t stream, DmaSync sync, std::string* err);

  // Wait until every submitted job has completed and released its stream;
  // false on timeout.
  bool drain(double timeout_s);

  DmaStats stats();
  void reset_stats();
  std::vector<SlotEvent> last_slot_log();
  // First error the proxy thread ran into since the last call ("" if none).
  std::string take_error();

  // Test hook: hold every job's release for this long after its copies
  // complete (simulates a slow engine, for the watchdog test).
  void set_finish_delay_us(int us) { finish_delay_us_.store(us); }

 private:
  struct Job;
  static void gate(void* block);
  bool submit(Job* j, hipStream_t stream, std::string* err);
  void loop();
  bool arrived(Job& j);
  bool try_abandon(Job& j);
  void release(Job& j, bool abandoned);
  void begin(Job& j);
  bool advance(Job& j);
  bool issue(char* dst, const char* src, int64_t bytes, hsa_signal_t done, int engine);
  bool start_copy(Job& j, int32_t i);
  int least_loaded(int max_engines) const;
  hsa_signal_t get_signal();
  void put_signal(hsa_signal_t s);
  void note_error(const std::string& e);
  void measure_engine_rate();
  void note_staged(const Job& j, double elapsed_s);

  hsa_agent_t agent_{};
  std::vector<int> engines_;  // HSA SDMA engine indices (bit positions)
  std::vector<int64_t> load_;  // per engine: bytes of copy-job copies issued, not yet seen done
  double engine_gbs_ = 0;     // one engine's measured copy rate
  std::atomic<double> staged_step_us_{0};  // written by the proxy thread
  std::list<Job*> active_;    // owned by the proxy thread
  std::deque<Job*> incoming_;
  std::vector<hsa_signal_t> signal_pool_;
  std::mutex mu_;
  std::condition_variable cv_;       // incoming work / shutdown
  std::condition_variable freed_;    // a job finished
  std::thread thread_;
  bool stop_ = false;                // under mu_: the thread returns once nothing is active
  bool give_up_ = false;             // under mu_: release every stream still held and return
  std::atomic<bool> abandon_queued_{false};  // jobs whose streams have not arrived are dropped
  bool started_ = false;
  bool closed_ = false;
  int64_t pending_ = 0;  // submitted, not yet released
  int64_t abandoned_ = 0;
  DmaStats stats_;
  std::vector<SlotEvent> slot_log_;
  std::string error_;
  std::atomic<int> finish_delay_us_{0};
};

}  // namespace ccr
