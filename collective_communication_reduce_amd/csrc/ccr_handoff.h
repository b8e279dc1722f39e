// How a stream hands an SDMA job to the CPU proxy and gets it back -- the
// host-side state of the two ways a job is tied to a stream.  Plain C++
// (no HIP), so the state machines can be exercised on the CPU alone.
//
// Method: "HOCCL: Offloading Collective Communication from GPU Cores to
// Accelerate Distributed Training", §3.2 (Stream Manager): when the stream
// reaches the communication point the CPU takes over, runs the copies, and
// lets the stream continue once they are done, so that communication keeps
// its place in the stream order.
//
//  - Gate (a host function the stream runs at that point): the stream
//    arrives, and waits until the proxy releases it.  The gate's state lives
//    in a GateBlock shared by the proxy's job and the callback, freed by
//    whichever lets go last, so neither side depends on the other's lifetime:
//    a proxy torn down before the stream arrives releases the block first
//    (the callback then returns at once), and a callback still returning
//    after the proxy is gone touches only the block.
//  - Flag words (stream memory operations on coherent host memory): each
//    slot is a pair of words, `req` and `done`, and hands out increasing
//    sequence numbers.  A job with sequence number q: the stream writes
//    req = q (the request) and waits until done >= q; the proxy starts the
//    copies once it reads req == q and writes done = q when they are done.
//    Nothing is ever reset and no acknowledgement is needed: done only
//    grows, so a wait for q is also met by any later job's value, and the
//    slot is free again as soon as the proxy has written done.  A job the
//    proxy abandons before its stream arrives gets done = kPoison (larger
//    than every sequence number), which releases the stream whenever it
//    arrives; that slot is never used again.
#pragma once

#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <mutex>
#include <vector>

namespace ccr {

class GateBlock {
 public:
  // States: 0 the stream has not reached the gate, 1 the stream waits at
  // the gate, 2 released (copies done, or the job abandoned).
  static GateBlock* make() { return new GateBlock(); }

  // The stream side (the host function): announce arrival, wait for the
  // release, drop this side's reference.  Returns true when the job was
  // abandoned before the stream arrived (no copy ran for it).
  static bool arrive_and_wait(GateBlock* g) {
    bool abandoned;
    {
      std::unique_lock<std::mutex> lk(g->mu_);
      int expect = 0;
      abandoned = !g->state_.compare_exchange_strong(expect, 1);
      if (!abandoned) g->cv_.wait(lk, [&] { return g->state_.load() == 2; });
    }
    unref(g);
    return abandoned;
  }

  // The proxy side.
  int state() const { return state_.load(std::memory_order_acquire); }
  // Copies done: let the stream go on, drop the job's reference.
  static void release(GateBlock* g) {
    {
      std::lock_guard<std::mutex> lk(g->mu_);
      g->state_.store(2);
    }
    g->cv_.notify_all();
    unref(g);
  }
  // Abandon a job whose stream has not arrived: true (and the job's
  // reference dropped) if the stream was not at the gate; false if it
  // already waits there (the job must then run, or be released).
  static bool abandon(GateBlock* g) {
    {
      std::lock_guard<std::mutex> lk(g->mu_);
      int expect = 0;
      if (!g->state_.compare_exchange_strong(expect, 2)) return false;
    }
    unref(g);
    return true;
  }

  // Blocks alive in the process (for tests).
  static int live() { return live_.load(); }

 private:
  GateBlock() { live_++; }
  ~GateBlock() { live_--; }
  static void unref(GateBlock* g) {
    if (g->refs_.fetch_sub(1) == 1) delete g;
  }
  std::mutex mu_;
  std::condition_variable cv_;
  std::atomic<int> state_{0};
  std::atomic<int> refs_{2};  // the proxy's job and the stream's callback
  static inline std::atomic<int> live_{0};
};

// A pool of flag-word slots over caller-provided memory that both the CPU
// and the GPU's stream operations can read and write (coherent host
// memory).  Slot f's words are at words[2 f stride] (req) and
// words[(2 f + 1) stride] (done), one cache line apart.
class FlagWords {
 public:
  static constexpr uint32_t kPoison = 0x7fffffffu;
  static constexpr uint32_t kMaxSeq = 0x7ffffff0u;  // below kPoison, below 2^31

  FlagWords(uint32_t* words, int slots, int stride) : w_(words), stride_(stride), seq_((size_t)slots, 0) {
    for (int f = slots - 1; f >= 0; f--) free_.push_back(f);
  }

  uint32_t* req(int f) const { return w_ + (size_t)(2 * f) * stride_; }
  uint32_t* done(int f) const { return w_ + (size_t)(2 * f + 1) * stride_; }

  // Take a free slot and its next sequence number; false if none frees up
  // within the timeout.
  template <class Dur>
  bool take(int* f, uint32_t* seq, Dur timeout) {
    std::unique_lock<std::mutex> lk(mu_);
    if (!cv_.wait_for(lk, timeout, [&] { return !free_.empty(); })) return false;
    *f = free_.back();
    free_.pop_back();
    *seq = ++seq_[(size_t)*f];
    return true;
  }

  // The proxy: has the stream of job (f, seq) made its request?
  bool requested(int f, uint32_t seq) const { return load(req(f)) == seq; }

  // The proxy: copies of job (f, seq) done -- release the stream and free
  // the slot (a slot whose numbers ran out is retired instead).
  void complete(int f, uint32_t seq) {
    store(done(f), seq);
    std::lock_guard<std::mutex> lk(mu_);
    if (seq_[(size_t)f] < kMaxSeq) free_.push_back(f);
    cv_.notify_one();
  }

  // The proxy: abandon job (f, seq) -- its stream is released whenever it
  // arrives, and the slot is retired.
  void abandon(int f) { store(done(f), kPoison); }

  // The stream side, for callers that stand in for the GPU (tests).
  void stream_request(int f, uint32_t seq) { store(req(f), seq); }
  bool stream_may_pass(int f, uint32_t seq) const { return load(done(f)) >= seq; }

  int free_slots() {
    std::lock_guard<std::mutex> lk(mu_);
    return (int)free_.size();
  }

 private:
  static uint32_t load(const uint32_t* p) { return __atomic_load_n(p, __ATOMIC_ACQUIRE); }
  static void store(uint32_t* p, uint32_t v) { __atomic_store_n(p, v, __ATOMIC_RELEASE); }
  uint32_t* w_;
  int stride_;
  std::vector<uint32_t> seq_;  // last sequence number handed out, per slot
  std::vector<int> free_;
  std::mutex mu_;
  std::condition_variable cv_;
};

}  // namespace ccr
