// Stage decomposition of a traffic matrix: HOCCL §3.4, Algorithm 1.
//
// Readings of the steps the paper leaves open (integer arithmetic
// throughout, so every decision is exact):
//  - a matching (the native components; each stage's contention-free
//    inter-node set) is greedy: flows with bytes left, by decreasing remainder,
//    ties by (src, dst); a flow joins if neither its sender nor its receiver
//    is taken yet.  Native traffic is peeled node by node.
//  - the portion a stage removes is the least remainder in the matching,
//    the Birkhoff-von Neumann coefficient, so each stage empties a flow.
//  - each moved portion x of u -> v adds x on (u, ū) and on (v̄, v).
//  - scale-up slack: an edge may carry up to
//    cap = max(floor(x * B_up / B_rdma), the largest forwarding load) in the
//    stage; native components, nodes in increasing id and components in
//    peel order, each move min(remainder, least room on their edges).
//  - native traffic left once inter-node traffic is done forms a tail of
//    stages; tail stage i takes the first unfinished component of each node.

#include "ccr_schedule.h"

#include <algorithm>
#include <cstdio>

namespace ccr {
namespace {

struct Flow {
  int32_t src, dst;
  int64_t left;
};

struct Component {
  std::vector<int32_t> src, dst;
  int64_t left;
};

// Flows with bytes left, kept in matching order: decreasing remainder, then
// (src, dst).  A stage subtracts the same amount from every matched flow,
// which keeps the matched flows in order among themselves, so the order is
// restored by one merge with the untouched flows instead of a sort.  Flows
// are stored in that order, so every pass is a linear walk over memory.
class Residual {
 public:
  Residual(std::vector<Flow> flows, int G) : out_((size_t)G, 0), in_((size_t)G, 0), G_(G) {
    for (const Flow& f : flows)
      if (f.left > 0) f_.push_back(f);
    std::sort(f_.begin(), f_.end(), before);
  }

  // Greedy matching: walk the order, take a flow if its sender and its
  // receiver are both still free; once G flows are taken every sender is.
  // Positions come in matching order.
  const std::vector<int>& match() {
    epoch_++;
    picked_.clear();
    for (int i = 0; i < (int)f_.size() && (int)picked_.size() < G_; i++) {
      const Flow& f = f_[(size_t)i];
      if (out_[(size_t)f.src] == epoch_ || in_[(size_t)f.dst] == epoch_) continue;
      out_[(size_t)f.src] = in_[(size_t)f.dst] = epoch_;
      picked_.push_back(i);
    }
    return picked_;
  }

  // Subtract x from every flow of the last matching; drop emptied flows.
  void take(int64_t x) {
    moved_.clear();
    size_t w = 0, k = 0;
    for (size_t i = 0; i < f_.size(); i++) {
      if (k < picked_.size() && (size_t)picked_[k] == i) {
        k++;
        Flow f = f_[i];
        f.left -= x;
        if (f.left > 0) moved_.push_back(f);
      } else {
        f_[w++] = f_[i];
      }
    }
    tmp_.resize(w + moved_.size());
    std::merge(moved_.begin(), moved_.end(), f_.begin(), f_.begin() + (std::ptrdiff_t)w,
               tmp_.begin(), before);
    f_.swap(tmp_);
  }

  const Flow& flow(int i) const { return f_[(size_t)i]; }

 private:
  static bool before(const Flow& x, const Flow& y) {
    if (x.left != y.left) return x.left > y.left;
    if (x.src != y.src) return x.src < y.src;
    return x.dst < y.dst;
  }

  std::vector<Flow> f_, moved_, tmp_;
  std::vector<int> picked_;
  std::vector<uint32_t> out_, in_;  // == epoch_: sender / receiver taken
  int G_;
  uint32_t epoch_ = 0;
};

// One stage under construction: bytes per (kind, cell), with the cells each
// kind touched, and the bytes each scale-up cell carries over all kinds.
struct StageBuilder {
  int G;
  std::vector<int64_t> bytes[3];     // per kind, G*G
  std::vector<int32_t> touched[3];   // per kind, cells with nonzero bytes
  std::vector<int64_t> cell;         // scale-up load (forwarding + native)
  int64_t rdma_max = 0;

  explicit StageBuilder(int g) : G(g), cell((size_t)g * g, 0) {
    for (auto& b : bytes) b.assign((size_t)g * g, 0);
  }

  void add(int32_t kind, int32_t u, int32_t v, int64_t b) {
    const int32_t c = u * G + v;
    int64_t& k = bytes[kind][(size_t)c];
    if (k == 0) touched[kind].push_back(c);
    k += b;
    if (kind == kStageRdma) {
      rdma_max = std::max(rdma_max, k);
      return;
    }
    cell[(size_t)c] += b;
  }
  int64_t load(int32_t u, int32_t v) const { return cell[(size_t)u * G + v]; }
  bool empty() const { return touched[0].empty() && touched[1].empty() && touched[2].empty(); }

  // Append the stage's entries, ordered by (kind, src, dst), and its time;
  // then reset.
  void emit(int32_t s, const ScheduleProblem& p, std::vector<StageEntry>* out,
            std::vector<StageTime>* times) {
    int64_t up = 0;
    for (int32_t kind = 0; kind < 3; kind++) {
      std::vector<int32_t>& t = touched[kind];
      std::sort(t.begin(), t.end());  // cell = src * G + dst: (src, dst) order
      for (int32_t c : t) {
        out->push_back({s, kind, c / G, c % G, bytes[kind][(size_t)c]});
        bytes[kind][(size_t)c] = 0;
        if (kind != kStageRdma) {
          up = std::max(up, cell[(size_t)c]);
          cell[(size_t)c] = 0;
        }
      }
      t.clear();
    }
    // Eq. 9, 10: the slowest domain sets the stage time.  All scale-up
    // domains share one bandwidth, so the largest scale-up cell of any node
    // stands for them all.
    const __int128 rd_t = (__int128)rdma_max * p.bw_scaleup;
    const __int128 up_t = (__int128)up * p.bw_rdma;
    times->push_back(rd_t >= up_t ? StageTime{rdma_max, p.bw_rdma} : StageTime{up, p.bw_scaleup});
    rdma_max = 0;
  }
};

}  // namespace

std::string check_schedule_problem(const ScheduleProblem& p, bool need_bandwidths) {
  char msg[160];
  if (p.G < 1 || p.G > kMaxScheduleGpus) {
    snprintf(msg, sizeof msg, "G = %d outside [1, %d]", p.G, kMaxScheduleGpus);
    return msg;
  }
  if (!p.C || !p.node || !p.peer) return "C, node or peer is NULL";
  if (need_bandwidths && (p.bw_scaleup < 1 || p.bw_scaleup > kMaxBandwidth || p.bw_rdma < 1 ||
                          p.bw_rdma > kMaxBandwidth)) {
    snprintf(msg, sizeof msg, "bandwidths must lie in [1, %lld]", (long long)kMaxBandwidth);
    return msg;
  }
  for (int u = 0; u < p.G; u++) {
    if (p.node[u] < 0) {
      snprintf(msg, sizeof msg, "node[%d] = %d < 0", u, p.node[u]);
      return msg;
    }
  }
  for (int u = 0; u < p.G; u++) {
    const int32_t w = p.peer[u];
    if (w == -1) continue;
    if (w < 0 || w >= p.G || w == u || p.node[w] != p.node[u]) {
      snprintf(msg, sizeof msg, "peer[%d] = %d is not -1 or another GPU of the same node", u, w);
      return msg;
    }
    if (p.peer[w] != u) {  // Eq. 4 charges both copies of the pair to the edge (u, peer u)
      snprintf(msg, sizeof msg, "peer[%d] = %d but peer[%d] = %d: peers must be mutual", u, w, w,
               p.peer[w]);
      return msg;
    }
  }
  for (int64_t i = 0; i < (int64_t)p.G * p.G; i++) {
    if (p.C[i] < 0 || p.C[i] > kMaxFlowBytes) {
      snprintf(msg, sizeof msg, "C[%lld][%lld] = %lld outside [0, 2^40]", (long long)(i / p.G),
               (long long)(i % p.G), (long long)p.C[i]);
      return msg;
    }
  }
  return "";
}

void build_traffic_matrix(const ScheduleProblem& p, int64_t* T) {
  const int G = p.G;
  std::vector<int64_t> send_fwd((size_t)G, 0), recv_fwd((size_t)G, 0);  // A_u, B_v (Eq. 3)
  for (int u = 0; u < G; u++) {
    for (int v = 0; v < G; v++) {
      const int64_t f = p.C[(size_t)u * G + v];
      T[(size_t)u * G + v] = u == v ? 0 : f;
      if (u == v || f == 0 || p.node[u] == p.node[v]) continue;
      if (p.peer[u] >= 0) send_fwd[(size_t)u] += f;
      if (p.peer[v] >= 0) recv_fwd[(size_t)v] += f;
    }
  }
  // Eq. 4: the edge to the symmetric peer carries the sender-side copies of
  // u's inter-node flows and the receiver-side copies of ū's.
  for (int u = 0; u < G; u++) {
    const int32_t w = p.peer[u];
    if (w >= 0) T[(size_t)u * G + w] += send_fwd[(size_t)u] + recv_fwd[(size_t)w];
  }
}

void decompose_stages(const ScheduleProblem& p, std::vector<StageEntry>* entries,
                      std::vector<StageTime>* times) {
  const int G = p.G;
  entries->clear();
  times->clear();

  // Node ids in increasing order.
  std::vector<int32_t> nodes(p.node, p.node + G);
  std::sort(nodes.begin(), nodes.end());
  nodes.erase(std::unique(nodes.begin(), nodes.end()), nodes.end());

  // Peel native components node by node.
  std::vector<std::vector<Component>> comps(nodes.size());
  for (size_t n = 0; n < nodes.size(); n++) {
    std::vector<Flow> native;
    for (int u = 0; u < G; u++) {
      if (p.node[u] != nodes[n]) continue;
      for (int v = 0; v < G; v++) {
        const int64_t f = p.C[(size_t)u * G + v];
        if (v != u && f > 0 && p.node[v] == nodes[n]) native.push_back({u, v, f});
      }
    }
    Residual res(std::move(native), G);
    for (;;) {
      const std::vector<int>& m = res.match();
      if (m.empty()) break;
      Component c;
      c.left = res.flow(m[0]).left;
      for (int i : m) {
        c.left = std::min(c.left, res.flow(i).left);
        c.src.push_back(res.flow(i).src);
        c.dst.push_back(res.flow(i).dst);
      }
      res.take(c.left);
      comps[n].push_back(std::move(c));
    }
  }

  // The inter-node part of the residual matrix.
  std::vector<Flow> cross;
  for (int u = 0; u < G; u++)
    for (int v = 0; v < G; v++) {
      const int64_t f = p.C[(size_t)u * G + v];
      if (f > 0 && p.node[u] != p.node[v]) cross.push_back({u, v, f});
    }
  Residual rdma(std::move(cross), G);

  StageBuilder st(G);
  int32_t s = 0;
  for (;;) {
    const std::vector<int>& m = rdma.match();
    if (m.empty()) break;
    int64_t x = rdma.flow(m[0]).left;
    for (int i : m) x = std::min(x, rdma.flow(i).left);
    int64_t fwd_max = 0;
    for (int i : m) {
      const Flow& f = rdma.flow(i);
      st.add(kStageRdma, f.src, f.dst, x);
      if (p.peer[f.src] >= 0) {  // sender-side copy on (u, ū)
        st.add(kStageForward, f.src, p.peer[f.src], x);
        fwd_max = std::max(fwd_max, st.load(f.src, p.peer[f.src]));
      }
      if (p.peer[f.dst] >= 0) {  // receiver-side copy on (v̄, v)
        st.add(kStageForward, p.peer[f.dst], f.dst, x);
        fwd_max = std::max(fwd_max, st.load(p.peer[f.dst], f.dst));
      }
    }
    rdma.take(x);
    const int64_t cap = std::max(x * p.bw_scaleup / p.bw_rdma, fwd_max);
    for (auto& node_comps : comps) {          // fill the scale-up slack
      size_t keep = 0;                        // drop finished components as we go
      for (size_t ci = 0; ci < node_comps.size(); ci++) {
        Component& c = node_comps[ci];
        int64_t amount = c.left;
        for (size_t k = 0; k < c.src.size() && amount > 0; k++)
          amount = std::min(amount, cap - st.load(c.src[k], c.dst[k]));
        if (amount > 0) {
          for (size_t k = 0; k < c.src.size(); k++) st.add(kStageNative, c.src[k], c.dst[k], amount);
          c.left -= amount;
        }
        if (c.left > 0) {
          if (keep != ci) node_comps[keep] = std::move(c);
          keep++;
        }
      }
      node_comps.resize(keep);
    }
    st.emit(s++, p, entries, times);
  }

  // Native traffic that did not fit into the inter-node stages.
  // Only unfinished components are left, in peel order.
  for (size_t i = 0;; i++) {
    for (auto& node_comps : comps) {
      if (i >= node_comps.size()) continue;
      const Component& c = node_comps[i];
      for (size_t k = 0; k < c.src.size(); k++) st.add(kStageNative, c.src[k], c.dst[k], c.left);
    }
    if (st.empty()) break;
    st.emit(s++, p, entries, times);
  }
}

}  // namespace ccr
