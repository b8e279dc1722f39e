// Device kernels of the ring all-reduce hot path, written for gfx950
// (CDNA4: wave64, 256 CUs in 8 XCDs, HBM3E).
//
// Every hot step here is a streaming pass over HBM (one fp32 add per 12
// bytes moved, one bf16 add per 6), so the kernels are built for bandwidth:
// 16-byte vector loads/stores, consecutive lanes on consecutive 16-byte
// vectors (a wave moves 1 KiB per instruction), several independent vectors
// in flight per thread, and no LDS or MFMA.  Batches of pieces are passed by
// value in the kernel arguments, so a hop needs no table upload.
//
// Method: "HOCCL: Offloading Collective Communication from GPU Cores to
// Accelerate Distributed Training".  The reduction stays on the compute
// units (§5 Limitations); copies have a compute-unit kernel here and an SDMA
// path in the host runtime (Fig. 1c, §2.3).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <stdint.h>

#include "ccr_device.h"
#include "ccr_internal.h"

namespace ccr {
namespace {

using namespace dev;

// The pieces of one launch, by value in the kernel arguments.  NP slots: a
// launch of up to 8, 16 or 32 pieces (one ring hop of R <= 32 ranks) uses a
// smaller table, because a launch's host cost grows with its argument block
// (on gfx950, ~2.3 us for 32 bytes, ~4.7 us for the 2.6 KB of 64 slots).
template <int NP>
struct PieceArgs {
  Piece p[NP];
  int32_t tile_start[NP + 1];  // first workgroup of each piece
  int32_t n;
};

// Piece of workgroup tile b: the number of pieces after the first whose
// first tile is <= b.  Unused slots hold the total tile count (> b), so the
// count runs over the whole table with no bound on n: the table's entries
// are independent scalar loads issued together, instead of the dependent
// chain of loads a binary search makes every workgroup wait through.
template <int NP>
__device__ __forceinline__ int piece_of(const int32_t* tile_start, int b) {
  int lo = 0;
#pragma unroll
  for (int i = 1; i < NP; i++) lo += tile_start[i] <= b ? 1 : 0;
  return lo;
}

// Workgroup b processes tiles b, b + gridDim.x, ... (one tile when the grid
// has one workgroup per tile), each found in the piece table.
template <HopKind K, int U, int NTM, int NP>
__global__ __launch_bounds__(kBlock) void pieces_kernel(PieceArgs<NP> a) {
  const int ntiles = a.tile_start[NP];
  for (int b = blockIdx.x; b < ntiles; b += gridDim.x) {
    const int lo = piece_of<NP>(a.tile_start, b);  // tile_start[lo] <= b < tile_start[lo + 1]
    hop_tile<K, U, NTM>(a.p[lo].dst, a.p[lo].src, a.p[lo].dst2, a.p[lo].nbytes, b - a.tile_start[lo]);
  }
}

struct Timing {
  hipEvent_t start, stop;
};

template <HopKind K, int U, int NTM, int NP>
hipError_t launch_one(const PieceArgs<NP>& a, hipStream_t s, Timing t, int grid_cap) {
  int grid = a.tile_start[a.n];
  if (grid_cap > 0 && grid > grid_cap) grid = grid_cap;
  if (grid > kMaxGridWorkgroups) grid = (int)kMaxGridWorkgroups;  // the workgroups loop over the rest
  if (t.start && t.stop)
    hipExtLaunchKernelGGL(pieces_kernel<K, U, NTM, NP>, dim3(grid), dim3(kBlock), 0, s, t.start,
                          t.stop, 0, a);
  else
    pieces_kernel<K, U, NTM, NP><<<grid, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

template <HopKind K, int U>
hipError_t launch_kind(const PieceArgs<kMaxPieces>& a, int ntm, hipStream_t s, Timing t, int g) {
  switch (ntm) {
    case 1: return launch_one<K, U, 1>(a, s, t, g);
    case 2: return launch_one<K, U, 2>(a, s, t, g);
    case 3: return launch_one<K, U, 3>(a, s, t, g);
    default: return launch_one<K, U, 0>(a, s, t, g);
  }
}

// Every tuning variant exists for the full table; the small tables exist for
// 2 vectors per operand per thread with temporal accesses or non-temporal
// loads (incoming only, or both operands).
template <HopKind K, int NP>
hipError_t launch_unroll(const PieceArgs<NP>& a, int unroll, int nt, hipStream_t s, Timing t,
                         int g) {
  if constexpr (NP != kMaxPieces) {
    (void)unroll;
    switch (nt) {
      case 2: return launch_one<K, 2, 2>(a, s, t, g);
      case 3: return launch_one<K, 2, 3>(a, s, t, g);
      default: return launch_one<K, 2, 0>(a, s, t, g);
    }
  } else {
    switch (unroll) {
      case 1: return launch_kind<K, 1>(a, nt, s, t, g);
      case 2: return launch_kind<K, 2>(a, nt, s, t, g);
      case 8: return launch_kind<K, 8>(a, nt, s, t, g);
      default: return launch_kind<K, 4>(a, nt, s, t, g);
    }
  }
}

// ---------------------------------------------------------- fp32 partials
template <int NP>
struct PartialArgs {
  PartialPiece p[NP];
  int32_t tile_start[NP + 1];
  int32_t n;
};

constexpr int kPartialUnroll = 2;  // 8-element groups per thread per tile

__device__ __forceinline__ void unpack_bf16x8(u32x4 w, float* f) {
#pragma unroll
  for (int j = 0; j < 4; j++) {
    f[2 * j] = bf16_lo(w[j]);
    f[2 * j + 1] = bf16_hi(w[j]);
  }
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float* f) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    f32x2 v = {f[2 * j], f[2 * j + 1]};
    r[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  return r;
}

// One group of 8 elements: out = in + float(loc).  The loads and the
// stores are split so that a tile issues all its loads before its first
// store (the compiler may not move a load above a store that could alias).
// NT: the first hop's two bf16 operands, both last written long before and
// dead after this hop, are loaded non-temporally (the bucket's first hop
// 39.3 -> 35.8 us); every other load is temporal: a non-temporal load of the
// incoming partial made the 8-rank bucket's all-reduce in this mode 9% slower.
template <PartialKind K, bool NT>
__device__ __forceinline__ void partial_load(const PartialPiece& pc, int64_t g, u32x4* loc,
                                             f32x4* in) {
  constexpr bool nt_first = NT && K == PartialKind::kFirst;
  *loc = load16<nt_first>(reinterpret_cast<const u32x4*>(pc.loc) + g);
  if constexpr (K == PartialKind::kFirst) {
    float f[8];
    unpack_bf16x8(load16<nt_first>(reinterpret_cast<const u32x4*>(pc.in) + g), f);
    in[0] = f32x4{f[0], f[1], f[2], f[3]};
    in[1] = f32x4{f[4], f[5], f[6], f[7]};
  } else {
    in[0] = reinterpret_cast<const f32x4*>(pc.in)[2 * g];
    in[1] = reinterpret_cast<const f32x4*>(pc.in)[2 * g + 1];
  }
}

template <PartialKind K>
__device__ __forceinline__ void partial_store(const PartialPiece& pc, int64_t g, u32x4 locw,
                                              const f32x4* in) {
  float loc[8], acc[8];
  unpack_bf16x8(locw, loc);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    acc[j] = in[0][j] + loc[j];
    acc[4 + j] = in[1][j] + loc[4 + j];
  }
  if constexpr (K == PartialKind::kFirst || K == PartialKind::kMid) {
    reinterpret_cast<f32x4*>(pc.out)[2 * g] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    reinterpret_cast<f32x4*>(pc.out)[2 * g + 1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    const u32x4 r = pack_bf16x8(acc);
    reinterpret_cast<u32x4*>(pc.out)[g] = r;
    if constexpr (K == PartialKind::kLastFwd) reinterpret_cast<u32x4*>(pc.out2)[g] = r;
  }
}

template <PartialKind K>
__device__ __forceinline__ void partial_one(const PartialPiece& pc, int64_t i) {
  const float loc = bf16_lo(reinterpret_cast<const uint16_t*>(pc.loc)[i]);
  const float in = K == PartialKind::kFirst ? bf16_lo(reinterpret_cast<const uint16_t*>(pc.in)[i])
                                            : reinterpret_cast<const float*>(pc.in)[i];
  const float acc = in + loc;
  if constexpr (K == PartialKind::kFirst || K == PartialKind::kMid) {
    reinterpret_cast<float*>(pc.out)[i] = acc;
  } else {
    const uint16_t r = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc));
    reinterpret_cast<uint16_t*>(pc.out)[i] = r;
    if constexpr (K == PartialKind::kLastFwd) reinterpret_cast<uint16_t*>(pc.out2)[i] = r;
  }
}

template <PartialKind K, int NP, bool NT>
__global__ __launch_bounds__(kBlock) void partial_kernel(PartialArgs<NP> a) {
  const int b = blockIdx.x;
  const int lo = piece_of<NP>(a.tile_start, b);
  const PartialPiece pc = a.p[lo];
  const int64_t ngroups = pc.n >> 3;
  const int64_t tile = b - a.tile_start[lo];
  const int64_t first = tile * (int64_t)(kBlock * kPartialUnroll);
  if (first + kBlock * kPartialUnroll <= ngroups) {  // whole tile in range (uniform)
    u32x4 loc[kPartialUnroll];
    f32x4 in[kPartialUnroll][2];
#pragma unroll
    for (int u = 0; u < kPartialUnroll; u++)
      partial_load<K, NT>(pc, first + u * kBlock + threadIdx.x, &loc[u], in[u]);
#pragma unroll
    for (int u = 0; u < kPartialUnroll; u++)
      partial_store<K>(pc, first + u * kBlock + threadIdx.x, loc[u], in[u]);
  } else {
#pragma unroll
    for (int u = 0; u < kPartialUnroll; u++) {
      const int64_t g = first + u * kBlock + threadIdx.x;
      if (g < ngroups) {
        u32x4 loc;
        f32x4 in[2];
        partial_load<K, NT>(pc, g, &loc, in);
        partial_store<K>(pc, g, loc, in);
      }
    }
  }
  const int tail = (int)(pc.n & 7);
  if (tail > 0 && tile == ngroups / (kBlock * kPartialUnroll) && (int)threadIdx.x < tail)
    partial_one<K>(pc, (ngroups << 3) + threadIdx.x);
}

// ------------------------------------------------------------------ probe
__global__ __launch_bounds__(64) void probe_cu_ids_kernel(int32_t* out) {
  unsigned hw, xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  if (threadIdx.x == 0) {
    out[3 * blockIdx.x] = (int32_t)(xcc & 0xfu);
    out[3 * blockIdx.x + 1] = (int32_t)((hw >> 13) & 0x7u);
    out[3 * blockIdx.x + 2] = (int32_t)((hw >> 8) & 0xfu);
  }
}

}  // namespace

namespace {

template <int NP>
hipError_t launch_pieces_np(HopKind kind, const Piece* pieces, int n, LaunchTuning tune, int unroll,
                            hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  PieceArgs<NP> a;
  const int64_t per_tile = (int64_t)kBlock * unroll;
  int64_t tiles = 0;
  a.n = n;
  for (int i = 0; i < n; i++) {
    a.p[i] = pieces[i];
    a.tile_start[i] = (int32_t)tiles;
    const int64_t nvec = pieces[i].nbytes >> 4;
    const int64_t units = nvec + ((pieces[i].nbytes & 15) ? 1 : 0);
    tiles += (units + per_tile - 1) / per_tile;
    // tile indices and a workgroup's next tile (b + gridDim.x) stay in int32
    if (tiles > INT32_MAX - kMaxGridWorkgroups) return hipErrorInvalidValue;
  }
  for (int i = n; i <= NP; i++) a.tile_start[i] = (int32_t)tiles;
  if (tiles == 0) return hipSuccess;
  const int nt = tune.nontemporal >= 1 && tune.nontemporal <= 3 ? tune.nontemporal : 0;
  const Timing t{start, stop};
  const int g = tune.grid;
  switch (kind) {
    case HopKind::kReduceF32: return launch_unroll<HopKind::kReduceF32>(a, unroll, nt, stream, t, g);
    case HopKind::kReduceBf16: return launch_unroll<HopKind::kReduceBf16>(a, unroll, nt, stream, t, g);
    case HopKind::kReduceFwdF32:
      return launch_unroll<HopKind::kReduceFwdF32>(a, unroll, nt, stream, t, g);
    case HopKind::kReduceFwdBf16:
      return launch_unroll<HopKind::kReduceFwdBf16>(a, unroll, nt, stream, t, g);
    case HopKind::kDrainFill: return launch_unroll<HopKind::kDrainFill>(a, unroll, nt, stream, t, g);
    default: return launch_unroll<HopKind::kCopy>(a, unroll, nt, stream, t, g);
  }
}

}  // namespace

hipError_t launch_pieces(HopKind kind, const Piece* pieces, int n, LaunchTuning tune,
                         hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (n <= 0) return hipSuccess;
  if (n > kMaxPieces) return hipErrorInvalidValue;
  const int unroll = (tune.unroll == 1 || tune.unroll == 2 || tune.unroll == 8) ? tune.unroll : 4;
  const bool small_ok = unroll == 2 && tune.nontemporal != 1;
  if (small_ok && n <= 8)
    return launch_pieces_np<8>(kind, pieces, n, tune, unroll, stream, start, stop);
  if (small_ok && n <= 16)
    return launch_pieces_np<16>(kind, pieces, n, tune, unroll, stream, start, stop);
  if (small_ok && n <= 32)
    return launch_pieces_np<32>(kind, pieces, n, tune, unroll, stream, start, stop);
  return launch_pieces_np<kMaxPieces>(kind, pieces, n, tune, unroll, stream, start, stop);
}

namespace {

template <int NP>
hipError_t launch_partials_np(PartialKind kind, const PartialPiece* pieces, int n, bool nt_first,
                              hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  PartialArgs<NP> a;
  const int64_t per_tile = (int64_t)kBlock * kPartialUnroll;
  int64_t tiles = 0;
  a.n = n;
  for (int i = 0; i < n; i++) {
    a.p[i] = pieces[i];
    a.tile_start[i] = (int32_t)tiles;
    const int64_t units = (pieces[i].n >> 3) + ((pieces[i].n & 7) ? 1 : 0);
    tiles += (units + per_tile - 1) / per_tile;
    if (tiles > kMaxGridWorkgroups) return hipErrorInvalidValue;  // one workgroup per tile
  }
  for (int i = n; i <= NP; i++) a.tile_start[i] = (int32_t)tiles;
  if (tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)tiles), block(kBlock);
  auto go = [&](auto kernel) {
    if (start && stop) hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, a);
    else kernel<<<grid, block, 0, stream>>>(a);
  };
  switch (kind) {
    case PartialKind::kFirst:
      if (nt_first) go(partial_kernel<PartialKind::kFirst, NP, true>);
      else go(partial_kernel<PartialKind::kFirst, NP, false>);
      break;
    case PartialKind::kMid: go(partial_kernel<PartialKind::kMid, NP, false>); break;
    case PartialKind::kLast: go(partial_kernel<PartialKind::kLast, NP, false>); break;
    default: go(partial_kernel<PartialKind::kLastFwd, NP, false>); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partials(PartialKind kind, const PartialPiece* pieces, int n, bool nt_first,
                           hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (n <= 0) return hipSuccess;
  if (n > kMaxPieces) return hipErrorInvalidValue;
  if (n <= 16) return launch_partials_np<16>(kind, pieces, n, nt_first, stream, start, stop);
  return launch_partials_np<kMaxPieces>(kind, pieces, n, nt_first, stream, start, stop);
}

hipError_t launch_probe_cu_ids(int32_t* out, int nblocks, hipStream_t stream) {
  if (nblocks <= 0) return hipSuccess;
  probe_cu_ids_kernel<<<nblocks, 64, 0, stream>>>(out);
  return hipGetLastError();
}

}  // namespace ccr
