// Ring hops launched from the rank buffers' base addresses (gfx950).
//
// A reduce-scatter or all-gather hop of the ring moves one chunk per rank:
// chunk c goes from rank (c + shift) mod R to the next rank (HOCCL: "HOCCL:
// Offloading Collective Communication from GPU Cores to Accelerate
// Distributed Training", §2.1 and Fig. 1, the ring algorithm's steps).  The
// chunks of a call are equal except the last non-empty one, so a hop is
// described by the R base addresses and one chunk geometry instead of a
// table of pieces: each workgroup finds its chunk by one division and its
// ranks by adding the shift, then fetches their base addresses with one
// scalar load.  The table form's workgroups search a table and then load
// their piece before the first data access; on MI355X the 32-rank fp32
// reduce-scatter + all-gather (1 MiB chunks) runs 7% faster in this form.
//
// This file is built with kernel-argument preloading: the leading scalar
// arguments arrive in registers, so a workgroup's first scalar memory access
// is the load of its base addresses.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ccr_device.h"
#include "ccr_internal.h"

namespace ccr {
namespace {

using namespace dev;

// The part of a hop's description read from memory: the ragged chunk's piece
// (only its workgroups read it) and the base addresses.  base[R] and
// base[R + 1] repeat base[0] and base[1], so a hop's source, destination and
// forwarding target are consecutive entries, fetched by one scalar load.
template <int NB>
struct RingRest {
  int64_t rag_off;  // byte offset of the ragged chunk's piece in each rank buffer
  int64_t rag_len;  // its length in bytes (0: none)
  int32_t rag_c;    // its chunk index
  int32_t pad;
  char* base[NB + 2];
};

// Workgroup b works on the tile ring_tile gives it.  Source rank (c + shift)
// mod R, destination the next rank, forwarding to the one after.  The
// RingLaunch fields arrive as separate scalars: only scalar arguments are
// preloaded into registers, a by-value struct would be read from memory.
template <HopKind K, int NTM, int NB>
__global__ __launch_bounds__(kBlock) void ring_hop_kernel(int32_t R, int32_t shift, int32_t tpp,
                                                          int32_t nfull, int32_t stride_v, int32_t off_v,
                                                          int32_t len_v, int32_t rot, RingRest<NB> a) {
  const RingLaunch g{tpp, nfull, stride_v, off_v, len_v, rot};
  const RingTile t = ring_tile(blockIdx.x, g, a.rag_c, a.rag_off, a.rag_len);
  int s = t.c + shift;  // c < R and shift < R
  s = s >= R ? s - R : s;
  char* const* const ranks = a.base + s;  // source, destination, the rank after
  char* dst2 = nullptr;
  if constexpr (forwards<K>()) dst2 = ranks[2] + t.off;
  hop_tile<K, 2, NTM>(ranks[1] + t.off, ranks[0] + t.off, dst2, t.len, t.tile);
}

constexpr int64_t kTileBytes = (int64_t)kBlock * 2 * 16;

RingLaunch ring_launch(const RingHop& h) {
  RingLaunch g;
  g.tpp = (int32_t)((h.full_len + kTileBytes - 1) / kTileBytes);
  g.nfull = h.nfull;
  g.stride_v = (int32_t)(h.stride >> 4);
  g.off_v = (int32_t)(h.full_off >> 4);
  g.len_v = (int32_t)(h.full_len >> 4);
  g.rot = h.rot;
  return g;
}

template <HopKind K, int NTM, int NB>
hipError_t launch_nb(const RingHop& h, unsigned grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  RingRest<NB> a{};
  a.rag_off = h.rag_off;
  a.rag_len = h.rag_len;
  a.rag_c = h.rag_c;
  for (int r = 0; r < h.R + 2; r++) a.base[r] = static_cast<char*>(h.base[r % h.R]);
  const RingLaunch g = ring_launch(h);
  if (start && stop)
    hipExtLaunchKernelGGL(ring_hop_kernel<K, NTM, NB>, dim3(grid), dim3(kBlock), 0, s, start, stop, 0,
                          h.R, h.shift, g.tpp, g.nfull, g.stride_v, g.off_v, g.len_v, g.rot, a);
  else
    ring_hop_kernel<K, NTM, NB><<<grid, kBlock, 0, s>>>(h.R, h.shift, g.tpp, g.nfull, g.stride_v, g.off_v,
                                                        g.len_v, g.rot, a);
  return hipGetLastError();
}

template <HopKind K, int NTM>
hipError_t launch_ntm(const RingHop& h, unsigned grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (h.R <= 8) return launch_nb<K, NTM, 8>(h, grid, s, start, stop);
  if (h.R <= 16) return launch_nb<K, NTM, 16>(h, grid, s, start, stop);
  if (h.R <= 32) return launch_nb<K, NTM, 32>(h, grid, s, start, stop);
  return launch_nb<K, NTM, 64>(h, grid, s, start, stop);
}

template <HopKind K>
hipError_t launch_kind(const RingHop& h, int ntm, unsigned grid, hipStream_t s, hipEvent_t start,
                       hipEvent_t stop) {
  switch (ntm) {
    case 2: return launch_ntm<K, 2>(h, grid, s, start, stop);
    case 3: return launch_ntm<K, 3>(h, grid, s, start, stop);
    default: return launch_ntm<K, 0>(h, grid, s, start, stop);
  }
}

}  // namespace

bool ring_hop_supported(const RingHop& h, HopKind kind, int ntm) {
  const bool kind_ok = kind == HopKind::kReduceF32 || kind == HopKind::kReduceBf16 ||
                       kind == HopKind::kReduceFwdF32 || kind == HopKind::kReduceFwdBf16 ||
                       kind == HopKind::kCopy;
  if (!kind_ok || (ntm != 0 && ntm != 2 && ntm != 3)) return false;
  if (h.R < 1 || h.R > kRingHopMaxRanks || h.shift < 0 || h.shift >= h.R) return false;
  if (h.nfull < 0 || h.nfull > h.R || h.rag_len < 0 || h.full_len < 0) return false;
  if (h.rag_len > 0 && (h.rag_c < h.nfull || h.rag_c >= h.R)) return false;
  if (h.rot < 0 || (h.rot > 0 && h.rot >= h.nfull)) return false;
  // full pieces: whole 16-byte vectors, offsets and lengths in int32 vectors
  if ((h.stride | h.full_off | h.full_len) & 15) return false;
  if ((h.stride >> 4) > INT32_MAX || ((h.full_off + h.full_len) >> 4) > INT32_MAX) return false;
  // one workgroup per tile, within one dispatch's grid (the piece-table
  // launch, whose workgroups loop over tiles, takes larger hops)
  const int64_t tpp = (h.full_len + kTileBytes - 1) / kTileBytes;
  const int64_t rag_tiles = (h.rag_len + kTileBytes - 1) / kTileBytes;
  return (int64_t)h.nfull * tpp + rag_tiles <= kMaxGridWorkgroups;
}

int64_t ring_hop_workgroups(const RingHop& h) {
  const int64_t tpp = (h.full_len + kTileBytes - 1) / kTileBytes;
  return (int64_t)h.nfull * tpp + (h.rag_len + kTileBytes - 1) / kTileBytes;
}

hipError_t launch_ring_hop(HopKind kind, const RingHop& h, int ntm, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop) {
  if (!ring_hop_supported(h, kind, ntm)) return hipErrorInvalidValue;
  const int64_t grid = ring_hop_workgroups(h);
  if (grid == 0) return hipSuccess;
  switch (kind) {
    case HopKind::kReduceF32:
      return launch_kind<HopKind::kReduceF32>(h, ntm, (unsigned)grid, stream, start, stop);
    case HopKind::kReduceBf16:
      return launch_kind<HopKind::kReduceBf16>(h, ntm, (unsigned)grid, stream, start, stop);
    case HopKind::kReduceFwdF32:
      return launch_kind<HopKind::kReduceFwdF32>(h, ntm, (unsigned)grid, stream, start, stop);
    case HopKind::kReduceFwdBf16:
      return launch_kind<HopKind::kReduceFwdBf16>(h, ntm, (unsigned)grid, stream, start, stop);
    default:
      return launch_kind<HopKind::kCopy>(h, ntm, (unsigned)grid, stream, start, stop);
  }
}

int64_t ring_hop_layout(const RingHop& h, int64_t* rows, int64_t max_wg) {
  const int64_t n = ring_hop_workgroups(h);
  const RingLaunch g = ring_launch(h);
  for (int64_t b = 0; b < n && b < max_wg; b++) {
    const RingTile t = ring_tile((int)b, g, h.rag_c, h.rag_off, h.rag_len);
    const int s = (t.c + h.shift) % h.R;
    int64_t* row = rows + 5 * b;
    row[0] = s;
    row[1] = (s + 1) % h.R;
    row[2] = t.off;
    row[3] = t.len;
    row[4] = t.tile;
  }
  return n;
}

}  // namespace ccr
