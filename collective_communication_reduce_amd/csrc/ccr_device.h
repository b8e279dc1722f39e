// Device-side building blocks shared by the streaming kernels (the piece
// table kernels and the ring-hop kernels): 16-byte vector loads and stores,
// the fp32 and bf16 adds of a hop, and the work of one tile of a piece.
// gfx950 only; included by the .hip sources, never by host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ccr_internal.h"

namespace ccr {
namespace dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
  } else if constexpr (K == HopKind::kDrainFill) {
    uint16_t* d = reinterpret_cast<uint16_t*>(dst) + unit;
    const uint16_t old = *d;
    reinterpret_cast<uint16_t*>(dst2)[unit] = old;
    *d = reinterpret_cast<const uint16_t*>(src)[unit];
  } else {
    reinterpret_cast<uint16_t*>(dst)[unit] = reinterpret_cast<const uint16_t*>(src)[unit];
  }
}

template <HopKind K>
constexpr int tail_unit_bytes() {
  return is_f32<K>() ? 4 : 2;
}


// One tile of a piece (dst op src over nbytes): kBlock * U consecutive
// 16-byte vectors.  Thread t handles vectors first + u * kBlock + t, u < U,
// so every load instruction of a wave covers 1 KiB of contiguous memory.
// All loads of a tile are issued before the first add, so 2U vectors per
// thread are in flight.  The tile holding vector index nvec also handles the
// bytes past the last whole vector (the ragged end of a buffer).
//
// NTM: 0 = every access temporal; 1 = every load and store non-temporal;
// 2 = only the incoming operand's load non-temporal (it is read once and
// is dead afterwards, so it need not displace the result, which the next
// hop reads, from the caches)
// 3 = both loads non-temporal, the store temporal (the local operand is
// overwritten by the result, and only the result is read again)
template <HopKind K, int U, int NTM>
__device__ __forceinline__ void hop_tile(char* const dst, const char* const src, char* const dst2,
                                         const int64_t nbytes, const int64_t tile) {
  constexpr bool NT = NTM == 1;
  constexpr bool NTI = NTM != 0;
  constexpr bool NTL = NTM == 1 || NTM == 3;
  const int64_t nvec = nbytes >> 4;
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
      in[u] = load16<NTI>(s16 + v0 + u * kBlock);
      if constexpr (K != HopKind::kCopy) loc[u] = load16<NTL>(d16 + v0 + u * kBlock);
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const u32x4 r = apply16<K>(loc[u], in[u]);
      if constexpr (K == HopKind::kDrainFill) store16<NT>(f16 + v0 + u * kBlock, loc[u]);
      store16<NT>(d16 + v0 + u * kBlock, r);
      if constexpr (forwards<K>()) store16<NT>(f16 + v0 + u * kBlock, r);
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int64_t v = v0 + u * kBlock;
      if (v < nvec) {
        u32x4 loc = {0, 0, 0, 0};
        if constexpr (K != HopKind::kCopy) loc = load16<NTL>(d16 + v);
        const u32x4 r = apply16<K>(loc, load16<NTI>(s16 + v));
        if constexpr (K == HopKind::kDrainFill) store16<NT>(f16 + v, loc);
        store16<NT>(d16 + v, r);
        if constexpr (forwards<K>()) store16<NT>(f16 + v, r);
      }
    }
  }
  // Ragged end: the bytes past the last whole vector belong to the tile
  // that would hold vector index nvec (never a whole in-range tile).
  const int tail_units = (int)(nbytes & 15) / tail_unit_bytes<K>();
  if (tail_units > 0 && tile == nvec / (kBlock * U) && (int)threadIdx.x < tail_units)
    apply_tail<K>(dst + (nvec << 4), src + (nvec << 4),
                  dst2 + (forwards<K>() || K == HopKind::kDrainFill ? (nvec << 4) : 0), threadIdx.x);
}

}  // namespace dev
}  // namespace ccr
