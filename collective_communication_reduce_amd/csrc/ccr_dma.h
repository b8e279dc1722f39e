// SDMA engines driven by a CPU proxy thread, synchronised with HIP streams
// through a start/finish flag handshake.
//
// Method: "HOCCL: Offloading Collective Communication from GPU Cores to
// Accelerate Distributed Training".  The stream manager keeps one start and
// one finish flag in host memory per in-flight operation; the GPU stream
// raises the start flag when it reaches the communication point and waits
// until the CPU has acknowledged it (reset it to zero), then waits for the
// finish flag and acknowledges it in turn, while a CPU proxy thread polls
// the start flag, acknowledges it, drives the DMA engine and raises the
// finish flag (§3.2, Listing 1, Fig. 4).  Staging slots move through a
// three-state machine, and chunks are spread over several engines so more
// than one is in flight (§3.3.1 chunk pipelining and multi-QP striping;
// §3.4 flow-size-aware chunk schedule).
//
// On gfx950 the copies run on the SDMA engines through
// hsa_amd_memory_async_copy_on_engine(force_copy_on_sdma = true): no compute
// unit touches the data.  Two ways tie a job to the stream:
//  - kHostFunc (default): the stream reaches a hipLaunchHostFunc gate; the
//    gate hands the job to the proxy (the start request) and blocks until
//    the proxy reports the copies done (the finish), and the stream resumes
//    when the gate returns; the proxy frees the job once the gate has
//    returned (the final acknowledgement).  The stream waits on the host
//    function's completion signal, with no GPU-side polling.
//  - kStreamFlags: the literal flag handshake with hipStreamWriteValue32 /
//    hipStreamWaitValue32 on host flags.  This HIP runtime runs those as
//    kernels, and a stream parked in hipStreamWaitValue32 for the length of
//    a DMA slows a concurrent GEMM by tens of percent, so it is an option,
//    not the default.
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

class DmaProxy {
 public:
  DmaProxy() = default;
  DmaProxy(const DmaProxy&) = delete;
  DmaProxy& operator=(const DmaProxy&) = delete;
  ~DmaProxy();

  // Find HIP device `device`'s HSA agent and its SDMA engines, warm every
  // engine with a small copy, allocate the flag pool, start the thread.
  bool start(int device, std::string* err);
  int engine_count() const { return (int)engines_.size(); }
  int engine_id(int i) const { return engines_[(size_t)i]; }
  // One engine's device-to-device copy rate measured at start (GB/s; 0 if
  // it could not be measured).
  double engine_gbs() const { return engine_gbs_; }
  // Fixed time per chunk step of the last completed staged job, beyond its
  // bytes at engine_gbs() (microseconds; 0 before any).
  double staged_step_us() const { return staged_step_us_.load(); }

  // Enqueue on `stream` the handshake around a job and hand the job to the
  // proxy.  Returns false (with *err) if no flag pair frees up in time.
  // max_engines: the engines (the first of the proxy's list) that copies
  // with engine -1 may go to; 0 = all.
  bool submit_copies(std::vector<DmaCopy> copies, hipStream_t stream, DmaSync sync,
                     std::string* err, int max_engines = 0);
  bool submit_staged(const StagedPlan& plan, hipStream_t stream, DmaSync sync, std::string* err);

  // Wait until every submitted job has completed its handshake; false on
  // timeout.
  bool drain(double timeout_s);

  DmaStats stats();
  void reset_stats();
  std::vector<SlotEvent> last_slot_log();
  // First error the proxy thread ran into since the last call ("" if none).
  std::string take_error();

  // Test hook: hold every job's finish flag for this long after its copies
  // complete (simulates a slow engine, for the watchdog test).
  void set_finish_delay_us(int us) { finish_delay_us_.store(us); }

 private:
  struct Job;
  static void gate(void* job);
  bool submit(Job* j, hipStream_t stream, std::string* err);
  bool take_flag(int* f, std::string* err);
  bool enqueue_handshake(int f, hipStream_t stream, std::string* err);
  void loop();
  bool begin(Job& j);
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
  uint32_t* flags_ = nullptr;  // pinned host: start flag of pair f at word 2f*stride, finish at (2f+1)*stride
  std::vector<int> free_flags_;
  std::list<Job*> active_;    // owned by the proxy thread
  std::deque<Job*> incoming_;
  std::vector<hsa_signal_t> signal_pool_;
  std::mutex mu_;
  std::condition_variable cv_;       // incoming work / shutdown
  std::condition_variable freed_;    // a flag pair was released / a job finished
  std::mutex gate_mu_;
  std::condition_variable gate_cv_;  // host-function gates wait here for their job
  std::thread thread_;
  bool stop_ = false;
  bool started_ = false;
  int64_t pending_ = 0;  // submitted, not yet released
  DmaStats stats_;
  std::vector<SlotEvent> slot_log_;
  std::string error_;
  std::atomic<int> finish_delay_us_{0};
};

}  // namespace ccr
