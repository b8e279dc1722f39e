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

#include "ccr_internal.h"

namespace ccr {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct PieceArgs {
  Piece p[kMaxPieces];
  int32_t tile_start[kMaxPieces + 1];  // first workgroup of each piece
  int32_t n;
};

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__device__ __forceinline__ void store16(u32x4* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// Eight bf16 hops at once: fp32 add, then round to nearest even with
// gfx950's v_cvt_pk_bf16_f32 (two results per instruction).  The fp32 sum of
// two bf16 values rounded to bf16 is the correctly rounded bf16 sum.
__device__ __forceinline__ u32x4 add_bf16x8(u32x4 a, u32x4 b) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    f32x2 fa = {bf16_lo(a[j]), bf16_hi(a[j])};
    f32x2 fb = {bf16_lo(b[j]), bf16_hi(b[j])};
    r[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(fa + fb, bf16x2));
  }
  return r;
}

__device__ __forceinline__ u32x4 add_f32x4(u32x4 a, u32x4 b) {
  f32x4 s = __builtin_bit_cast(f32x4, a) + __builtin_bit_cast(f32x4, b);
  return __builtin_bit_cast(u32x4, s);
}

template <HopKind K>
constexpr bool is_f32() {
  return K == HopKind::kReduceF32 || K == HopKind::kReduceFwdF32;
}
template <HopKind K>
constexpr bool is_bf16() {
  return K == HopKind::kReduceBf16 || K == HopKind::kReduceFwdBf16;
}
template <HopKind K>
constexpr bool forwards() {
  return K == HopKind::kReduceFwdF32 || K == HopKind::kReduceFwdBf16;
}

template <HopKind K>
__device__ __forceinline__ u32x4 apply16(u32x4 local, u32x4 incoming) {
  if constexpr (is_f32<K>()) return add_f32x4(local, incoming);
  else if constexpr (is_bf16<K>()) return add_bf16x8(local, incoming);
  else return incoming;
}

// The last (ragged) few elements of a piece, one element per thread.
template <HopKind K>
__device__ __forceinline__ void apply_tail(char* dst, const char* src, char* dst2, int unit) {
  if constexpr (is_f32<K>()) {
    float* d = reinterpret_cast<float*>(dst) + unit;
    const float r = *d + reinterpret_cast<const float*>(src)[unit];
    *d = r;
    if constexpr (forwards<K>()) reinterpret_cast<float*>(dst2)[unit] = r;
  } else if constexpr (is_bf16<K>()) {
    uint16_t* d = reinterpret_cast<uint16_t*>(dst) + unit;
    const float s = bf16_lo(*d) + bf16_lo(reinterpret_cast<const uint16_t*>(src)[unit]);
    const uint16_t r = __builtin_bit_cast(uint16_t, static_cast<__bf16>(s));
    *d = r;
    if constexpr (forwards<K>()) reinterpret_cast<uint16_t*>(dst2)[unit] = r;
  } else {
    reinterpret_cast<uint16_t*>(dst)[unit] = reinterpret_cast<const uint16_t*>(src)[unit];
  }
}

template <HopKind K>
constexpr int tail_unit_bytes() {
  return is_f32<K>() ? 4 : 2;
}

// One tile = kBlock * U consecutive 16-byte vectors of one piece.  Thread t
// handles vectors first + u * kBlock + t, u < U, so every load instruction
// of a wave covers 1 KiB of contiguous memory.  All loads of a tile are
// issued before the first add, so 2U vectors per thread are in flight.
// Workgroup b processes tiles b, b + gridDim.x, ... (one tile when the grid
// has one workgroup per tile).
template <HopKind K, int U, bool NT>
__global__ __launch_bounds__(kBlock) void pieces_kernel(PieceArgs a) {
  const int ntiles = a.tile_start[a.n];
  for (int b = blockIdx.x; b < ntiles; b += gridDim.x) {
    int lo = 0, hi = a.n;  // tile_start[lo] <= b < tile_start[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tile_start[mid] <= b) lo = mid;
      else hi = mid;
    }
    char* const dst = a.p[lo].dst;
    char* const dst2 = a.p[lo].dst2;
    const char* const src = a.p[lo].src;
    const int64_t nbytes = a.p[lo].nbytes;
    const int64_t nvec = nbytes >> 4;
    const int64_t tile = b - a.tile_start[lo];
    const int64_t first = tile * (int64_t)(kBlock * U);  // first vector of the tile
    const int64_t v0 = first + threadIdx.x;
    u32x4* const d16 = reinterpret_cast<u32x4*>(dst);
    u32x4* const f16 = reinterpret_cast<u32x4*>(dst2);
    const u32x4* const s16 = reinterpret_cast<const u32x4*>(src);

    if (first + kBlock * U <= nvec) {  // whole tile in range (uniform): no bounds checks
      u32x4 in[U];
      u32x4 loc[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        in[u] = load16<NT>(s16 + v0 + u * kBlock);
        if constexpr (K != HopKind::kCopy) loc[u] = load16<NT>(d16 + v0 + u * kBlock);
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const u32x4 r = apply16<K>(loc[u], in[u]);
        store16<NT>(d16 + v0 + u * kBlock, r);
        if constexpr (forwards<K>()) store16<NT>(f16 + v0 + u * kBlock, r);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int64_t v = v0 + u * kBlock;
        if (v < nvec) {
          u32x4 loc = {0, 0, 0, 0};
          if constexpr (K != HopKind::kCopy) loc = load16<NT>(d16 + v);
          const u32x4 r = apply16<K>(loc, load16<NT>(s16 + v));
          store16<NT>(d16 + v, r);
          if constexpr (forwards<K>()) store16<NT>(f16 + v, r);
        }
      }
    }
    // Ragged end: the bytes past the last whole vector belong to the tile
    // that would hold vector index nvec (never a whole in-range tile).
    const int tail_units = (int)(nbytes & 15) / tail_unit_bytes<K>();
    if (tail_units > 0 && tile == nvec / (kBlock * U) && (int)threadIdx.x < tail_units)
      apply_tail<K>(dst + (nvec << 4), src + (nvec << 4), dst2 + (forwards<K>() ? (nvec << 4) : 0),
                    threadIdx.x);
  }
}

struct Timing {
  hipEvent_t start, stop;
};

template <HopKind K, int U, bool NT>
hipError_t launch_one(const PieceArgs& a, hipStream_t s, Timing t, int grid_cap) {
  int grid = a.tile_start[a.n];
  if (grid_cap > 0 && grid > grid_cap) grid = grid_cap;
  if (t.start && t.stop)
    hipExtLaunchKernelGGL(pieces_kernel<K, U, NT>, dim3(grid), dim3(kBlock), 0, s, t.start, t.stop,
                          0, a);
  else
    pieces_kernel<K, U, NT><<<grid, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

template <HopKind K, int U>
hipError_t launch_kind(const PieceArgs& a, bool nt, hipStream_t s, Timing t, int g) {
  return nt ? launch_one<K, U, true>(a, s, t, g) : launch_one<K, U, false>(a, s, t, g);
}

template <HopKind K>
hipError_t launch_unroll(const PieceArgs& a, int unroll, bool nt, hipStream_t s, Timing t, int g) {
  switch (unroll) {
    case 1: return launch_kind<K, 1>(a, nt, s, t, g);
    case 2: return launch_kind<K, 2>(a, nt, s, t, g);
    case 8: return launch_kind<K, 8>(a, nt, s, t, g);
    default: return launch_kind<K, 4>(a, nt, s, t, g);
  }
}

// ---------------------------------------------------------- fp32 partials
struct PartialArgs {
  PartialPiece p[kMaxPieces];
  int32_t tile_start[kMaxPieces + 1];
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

// One group of 8 elements: out = in + float(loc).
template <PartialKind K>
__device__ __forceinline__ void partial_group(const PartialPiece& pc, int64_t g) {
  float loc[8], in[8], acc[8];
  unpack_bf16x8(reinterpret_cast<const u32x4*>(pc.loc)[g], loc);
  if constexpr (K == PartialKind::kFirst) {
    unpack_bf16x8(reinterpret_cast<const u32x4*>(pc.in)[g], in);
  } else {
    const f32x4 a = reinterpret_cast<const f32x4*>(pc.in)[2 * g];
    const f32x4 b = reinterpret_cast<const f32x4*>(pc.in)[2 * g + 1];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      in[j] = a[j];
      in[4 + j] = b[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 8; j++) acc[j] = in[j] + loc[j];
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

template <PartialKind K>
__global__ __launch_bounds__(kBlock) void partial_kernel(PartialArgs a) {
  const int b = blockIdx.x;
  int lo = 0, hi = a.n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tile_start[mid] <= b) lo = mid;
    else hi = mid;
  }
  const PartialPiece pc = a.p[lo];
  const int64_t ngroups = pc.n >> 3;
  const int64_t tile = b - a.tile_start[lo];
  const int64_t first = tile * (int64_t)(kBlock * kPartialUnroll);
#pragma unroll
  for (int u = 0; u < kPartialUnroll; u++) {
    const int64_t g = first + u * kBlock + threadIdx.x;
    if (g < ngroups) partial_group<K>(pc, g);
  }
  const int tail = (int)(pc.n & 7);
  if (tail > 0 && tile == ngroups / (kBlock * kPartialUnroll) && (int)threadIdx.x < tail)
    partial_one<K>(pc, (ngroups << 3) + threadIdx.x);
}

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
template <int RPB>
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
      if (from[j]) v[j] = from[j][c];
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

hipError_t launch_pieces(HopKind kind, const Piece* pieces, int n, LaunchTuning tune,
                         hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (n <= 0) return hipSuccess;
  if (n > kMaxPieces) return hipErrorInvalidValue;
  PieceArgs a;
  const int unroll = (tune.unroll == 1 || tune.unroll == 2 || tune.unroll == 8) ? tune.unroll : 4;
  const int64_t per_tile = (int64_t)kBlock * unroll;
  int64_t tiles = 0;
  a.n = n;
  for (int i = 0; i < n; i++) {
    a.p[i] = pieces[i];
    a.tile_start[i] = (int32_t)tiles;
    const int64_t nvec = pieces[i].nbytes >> 4;
    const int64_t units = nvec + ((pieces[i].nbytes & 15) ? 1 : 0);
    tiles += (units + per_tile - 1) / per_tile;
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
  }
  a.tile_start[n] = (int32_t)tiles;
  for (int i = n + 1; i <= kMaxPieces; i++) a.tile_start[i] = (int32_t)tiles;
  if (tiles == 0) return hipSuccess;
  const bool nt = tune.nontemporal != 0;
  const Timing t{start, stop};
  const int g = tune.grid;
  switch (kind) {
    case HopKind::kReduceF32: return launch_unroll<HopKind::kReduceF32>(a, unroll, nt, stream, t, g);
    case HopKind::kReduceBf16: return launch_unroll<HopKind::kReduceBf16>(a, unroll, nt, stream, t, g);
    case HopKind::kReduceFwdF32:
      return launch_unroll<HopKind::kReduceFwdF32>(a, unroll, nt, stream, t, g);
    case HopKind::kReduceFwdBf16:
      return launch_unroll<HopKind::kReduceFwdBf16>(a, unroll, nt, stream, t, g);
    default: return launch_unroll<HopKind::kCopy>(a, unroll, nt, stream, t, g);
  }
}

hipError_t launch_partials(PartialKind kind, const PartialPiece* pieces, int n, hipStream_t stream,
                           hipEvent_t start, hipEvent_t stop) {
  if (n <= 0) return hipSuccess;
  if (n > kMaxPieces) return hipErrorInvalidValue;
  PartialArgs a;
  const int64_t per_tile = (int64_t)kBlock * kPartialUnroll;
  int64_t tiles = 0;
  a.n = n;
  for (int i = 0; i < n; i++) {
    a.p[i] = pieces[i];
    a.tile_start[i] = (int32_t)tiles;
    const int64_t units = (pieces[i].n >> 3) + ((pieces[i].n & 7) ? 1 : 0);
    tiles += (units + per_tile - 1) / per_tile;
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
  }
  for (int i = n; i <= kMaxPieces; i++) a.tile_start[i] = (int32_t)tiles;
  if (tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)tiles), block(kBlock);
  auto go = [&](auto kernel) {
    if (start && stop) hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, a);
    else kernel<<<grid, block, 0, stream>>>(a);
  };
  switch (kind) {
    case PartialKind::kFirst: go(partial_kernel<PartialKind::kFirst>); break;
    case PartialKind::kMid: go(partial_kernel<PartialKind::kMid>); break;
    case PartialKind::kLast: go(partial_kernel<PartialKind::kLast>); break;
    default: go(partial_kernel<PartialKind::kLastFwd>); break;
  }
  return hipGetLastError();
}

hipError_t launch_permute_rows(char* dst, const char* src, const int32_t* idx, int64_t nrows,
                               int64_t nsrc, int64_t row_bytes, hipStream_t stream) {
  if (nrows <= 0 || row_bytes <= 0) return hipSuccess;
  constexpr int kRpb = 4;
  const int64_t grid = (nrows + kRpb - 1) / kRpb;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  permute_rows_kernel<kRpb><<<(unsigned)grid, kBlock, 0, stream>>>(
      reinterpret_cast<u32x4*>(dst), reinterpret_cast<const u32x4*>(src), idx, nrows, nsrc,
      row_bytes >> 4);
  return hipGetLastError();
}

template <int RPB>
hipError_t launch_gather_rpb(int combine, const MoeRank* ranks, const MoeSeg* segs, int R, int E,
                             int64_t rows_per_rank, int64_t idx_limit, int64_t row_bytes,
                             hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int64_t per_rank = (rows_per_rank + RPB - 1) / RPB;
  const int64_t grid = per_rank * R;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (start && stop)
    hipExtLaunchKernelGGL(moe_gather_kernel<RPB>, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                          start, stop, 0, ranks, segs, E, rows_per_rank, idx_limit, row_bytes >> 4,
                          per_rank, combine);
  else
    moe_gather_kernel<RPB><<<(unsigned)grid, kBlock, 0, stream>>>(
        ranks, segs, E, rows_per_rank, idx_limit, row_bytes >> 4, per_rank, combine);
  return hipGetLastError();
}

hipError_t launch_moe_gather(int combine, const MoeRank* ranks, const MoeSeg* segs, int R, int E,
                             int64_t rows_per_rank, int64_t idx_limit, int64_t row_bytes,
                             hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (R <= 0 || E <= 0 || rows_per_rank <= 0 || row_bytes <= 0) return hipSuccess;
  // rows per workgroup: overridable for tuning sweeps
  static const int rpb = [] {
    const char* e = getenv("CCR_GATHER_RPB");
    const int v = e ? atoi(e) : 8;
    return (v == 4 || v == 16) ? v : 8;
  }();
  switch (rpb) {
    case 4:
      return launch_gather_rpb<4>(combine, ranks, segs, R, E, rows_per_rank, idx_limit, row_bytes,
                                  stream, start, stop);
    case 16:
      return launch_gather_rpb<16>(combine, ranks, segs, R, E, rows_per_rank, idx_limit,
                                   row_bytes, stream, start, stop);
    default:
      return launch_gather_rpb<8>(combine, ranks, segs, R, E, rows_per_rank, idx_limit, row_bytes,
                                  stream, start, stop);
  }
}

hipError_t launch_moe_topk(const float* logits, int32_t* topk, int64_t T, int E, int K,
                           hipStream_t stream) {
  if (T <= 0 || K <= 0) return hipSuccess;
  if (E > 64 * kTopkMaxPerLane) return hipErrorInvalidValue;
  const int64_t grid = (T + kBlock / 64 - 1) / (kBlock / 64);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
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

hipError_t launch_probe_cu_ids(int32_t* out, int nblocks, hipStream_t stream) {
  if (nblocks <= 0) return hipSuccess;
  probe_cu_ids_kernel<<<nblocks, 64, 0, stream>>>(out);
  return hipGetLastError();
}

}  // namespace ccr
