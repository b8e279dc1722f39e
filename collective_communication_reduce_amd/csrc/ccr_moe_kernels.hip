// Device kernels of the expert-parallel MoE path, written for gfx950
// (CDNA4: wave64, 256 CUs in 8 XCDs, HBM3E): routing (top-K), the dispatch
// plan (per-expert counts and stable compaction), row permutes, and the
// fused gather that moves every row once between a source rank and its
// place in the destination's expert-major buffer.
//
// Method: "HOCCL: Offloading Collective Communication from GPU Cores to
// Accelerate Distributed Training".  Expert-parallel dispatch and combine
// are all-to-all traffic (§2.1); the exchange itself runs in the host
// runtime (compute-unit copies or SDMA engines).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <stdint.h>

#include "ccr_internal.h"

namespace ccr {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- permute
// dst row i = src row idx[i].  One workgroup moves RPB rows; thread t moves
// 16-byte column t (and t + kBlock, ...) of each, with the RPB loads of a
// column issued together.
template <int RPB>
__global__ __launch_bounds__(kBlock) void permute_rows_kernel(u32x4* dst, const u32x4* src,
                                                              const int32_t* idx, int64_t nrows,
                                                              int64_t nsrc, int64_t vpr) {
  const int64_t r0 = (int64_t)blockIdx.x * RPB;
  int64_t from[RPB];
#pragma unroll
  for (int j = 0; j < RPB; j++) {
    const int64_t r = r0 + j;
    const int64_t s = r < nrows ? (int64_t)idx[r] : -1;
    from[j] = (s >= 0 && s < nsrc) ? s : -1;
  }
  for (int64_t c = threadIdx.x; c < vpr; c += kBlock) {
    u32x4 v[RPB];
#pragma unroll
    for (int j = 0; j < RPB; j++)
      if (from[j] >= 0) v[j] = src[from[j] * vpr + c];
#pragma unroll
    for (int j = 0; j < RPB; j++)
      if (from[j] >= 0) dst[(r0 + j) * vpr + c] = v[j];
  }
}

// ------------------------------------------------------- fused MoE gather
// One workgroup moves RPB consecutive rows of one source rank's T*K rows.
// Lane j of the first wave resolves row j (its index, then the expert whose
// segment holds the pack position, by binary search over the segment
// starts) and leaves the row's source and destination in LDS, so the RPB
// lookups run side by side; then every thread moves 16-byte column c of
// all RPB rows, loads first.  The expert of a pack position is the last
// expert whose segment starts at or before it (an empty segment shares its
// start with the next one, so the search lands on the segment that holds
// the position).
template <int RPB, bool NTL>
__global__ __launch_bounds__(kBlock) void moe_gather_kernel(const MoeRank* ranks,
                                                            const MoeSeg* segs, int E,
                                                            int64_t rows, int64_t idx_limit,
                                                            int64_t vpr, int64_t blocks_per_rank,
                                                            int combine) {
  static_assert(RPB <= 64, "one lane per row of the first wave");
  __shared__ const u32x4* s_from[RPB];
  __shared__ u32x4* s_to[RPB];
  const int64_t r = blockIdx.x / blocks_per_rank;
  const int64_t q0 = (int64_t)(blockIdx.x % blocks_per_rank) * RPB;
  if (threadIdx.x < RPB) {
    const MoeRank rk = ranks[r];
    const MoeSeg* sg = segs + r * E;
    const int64_t q = q0 + threadIdx.x;
    const u32x4* from = nullptr;
    u32x4* to = nullptr;
    const int64_t i = q < rows ? (int64_t)rk.idx[q] : -1;
    if (i >= 0 && i < idx_limit) {
      const int64_t pos = combine ? i : q;  // pack position
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sg[mid].pack_start <= pos) lo = mid; else hi = mid - 1;
      }
      const MoeSeg g = sg[lo];
      u32x4* e = reinterpret_cast<u32x4*>(g.exp) + (g.exp_row + (pos - g.pack_start)) * vpr;
      u32x4* own = reinterpret_cast<u32x4*>(rk.rows) + (combine ? q : i) * vpr;
      from = combine ? e : own;
      to = combine ? own : e;
    }
    s_from[threadIdx.x] = from;
    s_to[threadIdx.x] = to;
  }
  __syncthreads();
  const u32x4* from[RPB];
  u32x4* to[RPB];
#pragma unroll
  for (int j = 0; j < RPB; j++) {
    from[j] = s_from[j];
    to[j] = s_to[j];
  }
  for (int64_t c = threadIdx.x; c < vpr; c += kBlock) {
    u32x4 v[RPB];
#pragma unroll
    for (int j = 0; j < RPB; j++)
      if (from[j]) {
        if constexpr (NTL) v[j] = __builtin_nontemporal_load(from[j] + c);
        else v[j] = from[j][c];
      }
#pragma unroll
    for (int j = 0; j < RPB; j++)
      if (to[j]) to[j][c] = v[j];
  }
}

// ------------------------------------------------------------------- topk
// One wave per token: lane l holds the logits of experts l, l+64, ...
// Each of the K rounds takes the largest remaining logit (lowest expert id
// among equals) with a butterfly reduction over the wave.
constexpr int kTopkMaxPerLane = 16;  // E <= 1024

__global__ __launch_bounds__(kBlock) void topk_kernel(const float* logits, int32_t* topk,
                                                      int64_t T, int E, int K) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + t * E;
  float v[kTopkMaxPerLane];
  uint32_t avail = 0;  // bit j: expert j*64+lane exists and is not yet taken
#pragma unroll
  for (int j = 0; j < kTopkMaxPerLane; j++) {
    const int e = j * 64 + lane;
    v[j] = e < E ? row[e] : 0.0f;
    if (e < E) avail |= 1u << j;
  }
  for (int k = 0; k < K; k++) {
    float bv = 0.0f;
    int be = -1;
#pragma unroll
    for (int j = 0; j < kTopkMaxPerLane; j++)
      if (((avail >> j) & 1u) && (be < 0 || v[j] > bv)) {
        bv = v[j];
        be = j * 64 + lane;
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (oe >= 0 && (be < 0 || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
      }
    }
    if (be >= 0 && lane == (be & 63)) avail &= ~(1u << (be >> 6));
    if (lane == 0) topk[t * K + k] = be;
  }
}

// ------------------------------------------------------------------- plan
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Workgroup e counts the (token, choice) pairs routed to expert e.
__global__ __launch_bounds__(kBlock) void plan_count_kernel(const int32_t* topk, int64_t T, int K,
                                                            int64_t* ecnt) {
  __shared__ int part[kBlock / 64];
  const int e = blockIdx.x;
  int n = 0;
  for (int64_t t = threadIdx.x; t < T; t += kBlock)
    for (int k = 0; k < K; k++) n += topk[t * K + k] == e;
  n = wave_sum(n);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t s = 0;
    for (int w = 0; w < kBlock / 64; w++) s += part[w];
    ecnt[e] = s;
  }
}

// Workgroup e writes expert e's rows: they start after all rows of experts
// < e (pack order (destination, local expert, token) is expert order), and
// tokens keep their order through a workgroup-wide stable compaction.
__global__ __launch_bounds__(kBlock) void plan_fill_kernel(const int32_t* topk, int64_t T, int K,
                                                           const int64_t* ecnt, int32_t* src_tok,
                                                           int32_t* slot) {
  __shared__ int64_t s_base;
  __shared__ int wcount[kBlock / 64];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    int64_t b = 0;
    for (int x = 0; x < e; x++) b += ecnt[x];
    s_base = b;
  }
  __syncthreads();
  int64_t base = s_base;
  for (int64_t t0 = 0; t0 < T; t0 += kBlock) {
    const int64_t t = t0 + threadIdx.x;
    int kk = -1;
    if (t < T)
      for (int k = 0; k < K; k++)
        if (topk[t * K + k] == e) kk = k;
    const uint64_t mask = __ballot(kk >= 0);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wcount[wave] = __popcll(mask);
    __syncthreads();
    int wbase = 0, total = 0;
    for (int w = 0; w < kBlock / 64; w++) {
      if (w < wave) wbase += wcount[w];
      total += wcount[w];
    }
    if (kk >= 0) {
      const int64_t j = base + wbase + before;
      src_tok[j] = (int32_t)t;
      slot[t * K + kk] = (int32_t)j;
    }
    base += total;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_permute_rows(char* dst, const char* src, const int32_t* idx, int64_t nrows,
                               int64_t nsrc, int64_t row_bytes, hipStream_t stream) {
  if (nrows <= 0 || row_bytes <= 0) return hipSuccess;
  constexpr int kRpb = 4;
  const int64_t grid = (nrows + kRpb - 1) / kRpb;
  if (grid > kMaxGridWorkgroups) return hipErrorInvalidValue;
  permute_rows_kernel<kRpb><<<(unsigned)grid, kBlock, 0, stream>>>(
      reinterpret_cast<u32x4*>(dst), reinterpret_cast<const u32x4*>(src), idx, nrows, nsrc,
      row_bytes >> 4);
  return hipGetLastError();
}

template <int RPB, bool NTL>
hipError_t launch_gather_rpb(int combine, const MoeRank* ranks, const MoeSeg* segs, int R, int E,
                             int64_t rows_per_rank, int64_t idx_limit, int64_t row_bytes,
                             hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int64_t per_rank = (rows_per_rank + RPB - 1) / RPB;
  const int64_t grid = per_rank * R;
  if (grid > kMaxGridWorkgroups) return hipErrorInvalidValue;
  if (start && stop)
    hipExtLaunchKernelGGL(moe_gather_kernel<RPB, NTL>, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                          start, stop, 0, ranks, segs, E, rows_per_rank, idx_limit, row_bytes >> 4,
                          per_rank, combine);
  else
    moe_gather_kernel<RPB, NTL><<<(unsigned)grid, kBlock, 0, stream>>>(
        ranks, segs, E, rows_per_rank, idx_limit, row_bytes >> 4, per_rank, combine);
  return hipGetLastError();
}

template <int RPB>
hipError_t launch_gather_nt(int combine, const MoeRank* ranks, const MoeSeg* segs, int R, int E,
                            int64_t rows_per_rank, int64_t idx_limit, int64_t row_bytes,
                            bool nt_load, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  return nt_load ? launch_gather_rpb<RPB, true>(combine, ranks, segs, R, E, rows_per_rank, idx_limit,
                                                row_bytes, stream, start, stop)
                 : launch_gather_rpb<RPB, false>(combine, ranks, segs, R, E, rows_per_rank,
                                                 idx_limit, row_bytes, stream, start, stop);
}

hipError_t launch_moe_gather(int combine, const MoeRank* ranks, const MoeSeg* segs, int R, int E,
                             int64_t rows_per_rank, int64_t idx_limit, int64_t row_bytes,
                             bool nt_load, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (R <= 0 || E <= 0 || rows_per_rank <= 0 || row_bytes <= 0) return hipSuccess;
  // rows per workgroup: overridable for tuning sweeps
  static const int rpb = [] {
    const char* e = getenv("CCR_GATHER_RPB");
    const int v = e ? atoi(e) : 8;
    return (v == 4 || v == 16) ? v : 8;
  }();
  switch (rpb) {
    case 4:
      return launch_gather_nt<4>(combine, ranks, segs, R, E, rows_per_rank, idx_limit, row_bytes,
                                 nt_load, stream, start, stop);
    case 16:
      return launch_gather_nt<16>(combine, ranks, segs, R, E, rows_per_rank, idx_limit,
                                  row_bytes, nt_load, stream, start, stop);
    default:
      return launch_gather_nt<8>(combine, ranks, segs, R, E, rows_per_rank, idx_limit, row_bytes,
                                 nt_load, stream, start, stop);
  }
}

hipError_t launch_moe_topk(const float* logits, int32_t* topk, int64_t T, int E, int K,
                           hipStream_t stream) {
  if (T <= 0 || K <= 0) return hipSuccess;
  if (E > 64 * kTopkMaxPerLane) return hipErrorInvalidValue;
  const int64_t grid = (T + kBlock / 64 - 1) / (kBlock / 64);
  if (grid > kMaxGridWorkgroups) return hipErrorInvalidValue;
  topk_kernel<<<(unsigned)grid, kBlock, 0, stream>>>(logits, topk, T, E, K);
  return hipGetLastError();
}

hipError_t launch_moe_plan(const int32_t* topk, int64_t T, int E, int K, int eloc, int64_t* ecnt,
                           int32_t* src_tok, int32_t* slot, hipStream_t stream) {
  (void)eloc;
  if (E <= 0) return hipSuccess;
  plan_count_kernel<<<E, kBlock, 0, stream>>>(topk, T, K, ecnt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || T <= 0 || K <= 0) return err;
  plan_fill_kernel<<<E, kBlock, 0, stream>>>(topk, T, K, ecnt, src_tok, slot);
  return hipGetLastError();
}

}  // namespace ccr
