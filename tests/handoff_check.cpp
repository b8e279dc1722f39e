// CPU check of the stream/proxy hand-over state (ccr_handoff.h): host
// threads stand in for the stream's host function and the GPU's stream
// memory operations.  Exits 0 when every scenario holds; prints the first
// that does not and exits 1.
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

#include "../collective_communication_reduce_amd/csrc/ccr_handoff.h"

using namespace ccr;
using namespace std::chrono_literals;

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "%s:%d: %s failed\n", __FILE__, __LINE__, #cond); \
      failures++;                                                     \
    }                                                                 \
  } while (0)

static void gate_scenarios() {
  // 1. the stream arrives first and waits; the proxy sees it and releases
  {
    GateBlock* g = GateBlock::make();
    bool abandoned = true;
    std::thread stream([&] { abandoned = GateBlock::arrive_and_wait(g); });
    while (g->state() != 1) std::this_thread::yield();
    CHECK(!GateBlock::abandon(g));  // arrived: cannot be abandoned
    std::this_thread::sleep_for(2ms);
    GateBlock::release(g);          // the proxy lets go of its reference here
    stream.join();
    CHECK(!abandoned);
  }
  // 2. the proxy abandons the job before the stream arrives; the stream,
  //    arriving later, passes at once and frees the block
  {
    GateBlock* g = GateBlock::make();
    CHECK(GateBlock::abandon(g));
    bool abandoned = false;
    std::thread stream([&] { abandoned = GateBlock::arrive_and_wait(g); });
    stream.join();
    CHECK(abandoned);
  }
  // 3. release racing the arrival, many times over
  for (int i = 0; i < 2000; i++) {
    GateBlock* g = GateBlock::make();
    std::thread stream([&] { (void)GateBlock::arrive_and_wait(g); });
    while (g->state() != 1) std::this_thread::yield();
    GateBlock::release(g);
    stream.join();
  }
  // 4. abandon racing the arrival: exactly one side decides
  for (int i = 0; i < 2000; i++) {
    GateBlock* g = GateBlock::make();
    bool abandoned = false;
    std::thread stream([&] { abandoned = GateBlock::arrive_and_wait(g); });
    if (!GateBlock::abandon(g)) {  // the stream got there first: run and release
      GateBlock::release(g);
      stream.join();
      CHECK(!abandoned);
    } else {
      stream.join();
      CHECK(abandoned);
    }
  }
  CHECK(GateBlock::live() == 0);
}

static void flag_scenarios() {
  constexpr int kSlots = 4, kStride = 32;
  std::vector<uint32_t> mem(2 * kSlots * kStride, 0);
  FlagWords fw(mem.data(), kSlots, kStride);
  // sequence numbers grow per slot; a request is seen only for its own job
  int f;
  uint32_t q;
  CHECK(fw.take(&f, &q, 10ms) && q == 1);
  CHECK(!fw.requested(f, q) && !fw.stream_may_pass(f, q));
  fw.stream_request(f, q);
  CHECK(fw.requested(f, q) && !fw.stream_may_pass(f, q));
  fw.complete(f, q);
  CHECK(fw.stream_may_pass(f, q));
  // the slot comes back with the next number; the old job's wait stays met
  int f2;
  uint32_t q2;
  for (int i = 0; i < kSlots; i++) {
    CHECK(fw.take(&f2, &q2, 10ms));
    if (f2 == f) break;
  }
  CHECK(f2 == f && q2 == q + 1);
  CHECK(!fw.requested(f2, q2) && fw.stream_may_pass(f, q) && !fw.stream_may_pass(f2, q2));
  fw.stream_request(f2, q2);
  fw.complete(f2, q2);
  CHECK(fw.stream_may_pass(f, q) && fw.stream_may_pass(f2, q2));
  // an abandoned job releases its stream whenever it arrives, and its slot
  // is never handed out again
  int free_before = fw.free_slots();
  int f3;
  uint32_t q3;
  CHECK(fw.take(&f3, &q3, 10ms));
  fw.abandon(f3);
  fw.stream_request(f3, q3);  // the stream arrives late
  CHECK(fw.stream_may_pass(f3, q3) && fw.stream_may_pass(f3, q3 + 1000000));
  CHECK(fw.free_slots() == free_before - 1);
}

// Many streams and one proxy thread run jobs through the flag words and
// gates at once; every stream must get past every job it submitted.
static void concurrent_scenario() {
  constexpr int kSlots = 8, kStride = 32, kStreams = 6, kJobs = 300;
  std::vector<uint32_t> mem(2 * kSlots * kStride, 0);
  FlagWords fw(mem.data(), kSlots, kStride);
  struct Job {
    int f;
    uint32_t q;
    GateBlock* g;
  };
  std::mutex mu;
  std::vector<Job> queue;
  std::atomic<int> done_streams{0};
  std::thread proxy([&] {
    std::vector<Job> active;
    while (done_streams.load() < kStreams || !active.empty()) {
      {
        std::lock_guard<std::mutex> lk(mu);
        for (auto& j : queue) active.push_back(j);
        queue.clear();
      }
      for (size_t i = 0; i < active.size();) {
        Job& j = active[i];
        const bool ready = j.g ? j.g->state() == 1 : fw.requested(j.f, j.q);
        if (ready) {
          if (j.g) GateBlock::release(j.g);
          else fw.complete(j.f, j.q);
          active[i] = active.back();
          active.pop_back();
        } else {
          i++;
        }
      }
      std::this_thread::yield();
    }
  });
  std::vector<std::thread> streams;
  for (int s = 0; s < kStreams; s++)
    streams.emplace_back([&, s] {
      std::mt19937 rng(s);
      for (int k = 0; k < kJobs; k++) {
        Job j{-1, 0, nullptr};
        if (rng() & 1) {
          j.g = GateBlock::make();
        } else if (!fw.take(&j.f, &j.q, 5s)) {
          std::fprintf(stderr, "no flag slot\n");
          std::abort();
        }
        {
          std::lock_guard<std::mutex> lk(mu);
          queue.push_back(j);
        }
        if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
        if (j.g) {
          (void)GateBlock::arrive_and_wait(j.g);
        } else {
          fw.stream_request(j.f, j.q);
          const auto t0 = std::chrono::steady_clock::now();
          while (!fw.stream_may_pass(j.f, j.q)) {
            if (std::chrono::steady_clock::now() - t0 > 10s) {
              std::fprintf(stderr, "stream %d stuck on job %d\n", s, k);
              std::abort();
            }
            std::this_thread::yield();
          }
        }
      }
      done_streams++;
    });
  for (auto& t : streams) t.join();
  proxy.join();
  CHECK(fw.free_slots() == kSlots);
  CHECK(GateBlock::live() == 0);
}

int main() {
  gate_scenarios();
  flag_scenarios();
  concurrent_scenario();
  if (failures) return 1;
  std::printf("handoff: ok\n");
  return 0;
}
