// Topology-aware stage decomposition of a collective's traffic (host only).
//
// Method: "HOCCL: Offloading Collective Communication from GPU Cores to
// Accelerate Distributed Training", §3.4 Collective Scheduler (Figure 6,
// Eq. 2-11, Algorithm 1).  A collective is an origin traffic matrix C of
// logical flows between G GPUs.  An inter-node flow u -> v also costs a
// forwarding copy on the scale-up edge (u, ū) and one on (v̄, v), where ū is
// u's symmetric peer; T is C with those copies added.  The scheduler cuts T
// into stages: each stage holds at most one outgoing and one incoming
// inter-node flow per GPU, moves the same amount on each of them, carries
// their forwarding copies, and packs native scale-up traffic into whatever
// scale-up time the inter-node transfer leaves.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace ccr {

enum StageKind : int32_t { kStageRdma = 0, kStageForward = 1, kStageNative = 2 };

struct StageEntry {
  int32_t stage, kind, src, dst;
  int64_t bytes;
};

// Stage time tau = load / bw of the stage's slowest domain.
struct StageTime {
  int64_t load, bw;
};

struct ScheduleProblem {
  int G = 0;
  const int64_t* C = nullptr;     // G x G row-major, bytes; the diagonal is ignored
  const int32_t* node = nullptr;  // node (scale-up domain) of each GPU
  const int32_t* peer = nullptr;  // symmetric peer, -1 = none
  int64_t bw_scaleup = 1, bw_rdma = 1;
};

constexpr int kMaxScheduleGpus = 256;
constexpr int64_t kMaxFlowBytes = int64_t(1) << 40;
constexpr int64_t kMaxBandwidth = int64_t(1) << 20;

// "" when the problem is well formed, else what is wrong with it.
std::string check_schedule_problem(const ScheduleProblem& p, bool need_bandwidths);

// Eq. 2-5.  T: G x G row-major.
void build_traffic_matrix(const ScheduleProblem& p, int64_t* T);

// Algorithm 1.  Entries come sorted by (stage, kind, src, dst), one per
// distinct key; times[s] is stage s's (L, B).
void decompose_stages(const ScheduleProblem& p, std::vector<StageEntry>* entries,
                      std::vector<StageTime>* times);

}  // namespace ccr
