// Internal interface between the host runtime (ccr_api.cpp) and the device
// kernels (the .hip sources).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ccr {

// One contiguous piece of work of a batched launch: `dst` (op) `src` over
// nbytes bytes.  For a reduce, dst = dst + src element-wise; for a copy,
// dst = src.  Pointers and nbytes are 16-byte multiples except for the tail
// of the very last piece of a buffer, whose length is a multiple of the
// element size.
struct Piece {
  char* dst;
  const char* src;
  int64_t nbytes;
  char* dst2 = nullptr;  // reduce-and-forward: second copy of the result;
                         // drain-and-fill: where dst's old contents go
};

// Up to kMaxPieces pieces go into one launch, passed by value as kernel
// arguments (no device-side table, no upload per call).
constexpr int kMaxPieces = 64;

// Threads per workgroup of the streaming kernels: four wave64 wavefronts.
constexpr int kBlock = 256;

// A dispatch counts its grid in work-items, in 32 bits, so one launch of
// kBlock-thread workgroups takes at most this many of them (2^24 - 1).
constexpr int64_t kMaxGridWorkgroups = int64_t(UINT32_MAX) / kBlock;

// kReduce*: dst = dst + src.  kReduceFwd*: the same, and the result is also
// written to dst2 (the last reduce-scatter hop forwarding the reduced chunk
// to the next rank, which replaces the first all-gather hop).  kCopy:
// dst = src.  kDrainFill: dst2 = dst, then dst = src, element by element in
// the same thread (a staging slot handing its chunk to the receiver and
// taking the sender's next chunk in one pass).
enum class HopKind : int {
  kReduceF32 = 0,
  kReduceBf16 = 1,
  kCopy = 2,
  kReduceFwdF32 = 3,
  kReduceFwdBf16 = 4,
  kDrainFill = 5
};

struct LaunchTuning {
  int unroll;       // 16-byte vectors per thread per pass: 1, 2, 4 or 8
  int nontemporal;  // 1 = streaming (non-temporal) loads and stores; 2 = only
                    // the incoming operand's load non-temporal
  int grid;         // 0 = one workgroup per tile; > 0 = that many workgroups
                    // looping over the tiles
};

// bf16 reduce-scatter with the running partial carried in fp32.  Per
// piece: out = in + float(loc) over n elements, where `in` is bf16 (the
// first hop) or fp32 (a partial), and `out` is fp32 (a partial) or bf16
// (the last hop, rounded to nearest even; also written to out2 when
// forwarding).  Pointers are 16-byte aligned; element groups of 8.
struct PartialPiece {
  char* out;
  const char* in;
  const char* loc;
  char* out2;
  int64_t n;
};

enum class PartialKind : int { kFirst = 0, kMid = 1, kLast = 2, kLastFwd = 3 };

// nt_first: the first hop (kFirst) loads its two bf16 operands non-temporally.
hipError_t launch_partials(PartialKind kind, const PartialPiece* pieces, int n, bool nt_first,
                           hipStream_t stream, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// Enqueue one batched launch over `n` pieces (n <= kMaxPieces).  With
// start/stop events, the launch goes through hipExtLaunchKernelGGL so that
// the events carry the kernel's own start and end timestamps.
hipError_t launch_pieces(HopKind kind, const Piece* pieces, int n, LaunchTuning tune,
                         hipStream_t stream, hipEvent_t start = nullptr,
                         hipEvent_t stop = nullptr);

// One ring hop over R rank buffers: chunk c moves from rank (c + shift) mod R
// to the next rank (kReduce*: added into it; kReduceFwd*: also written to
// the rank after; kCopy: copied).  Chunks 0..nfull-1 start `stride` bytes
// apart and the hop touches full_len bytes at full_off within each; chunk
// rag_c (>= nfull), if rag_len > 0, touches rag_len bytes at absolute byte
// offset rag_off.  stride, full_off and full_len are 16-byte multiples;
// rag_off too, and rag_len a multiple of the element size.  The full chunks
// are taken in the order rot, rot + 1, ..., nfull - 1, 0, ..., rot - 1.
struct RingHop {
  int R = 0;
  int shift = 0;
  int rot = 0;
  int64_t stride = 0;
  int nfull = 0;
  int64_t full_off = 0, full_len = 0;
  int rag_c = 0;
  int64_t rag_off = 0, rag_len = 0;
  void* const* base = nullptr;  // R rank buffers
};
constexpr int kRingHopMaxRanks = 64;

// The scalar arguments of a ring-hop launch (16-byte vectors, int32): tiles
// per full-chunk piece, full chunks, their stride, the slice's offset and
// length inside a full chunk, and the rotation of the walk.
struct RingLaunch {
  int32_t tpp, nfull, stride_v, off_v, len_v, rot;
};

// Where workgroup b of a ring-hop launch works: chunk c, the tile of the
// chunk's piece, and that piece's byte offset and length in every rank
// buffer.  Workgroups below nfull * tpp take full chunks in the order rot,
// rot + 1, ..., nfull - 1, 0, ..., rot - 1; the ones after them the ragged
// chunk's piece.  Used by the kernel and, on the host, by ring_hop_layout.
struct RingTile {
  int c;
  int64_t tile, off, len;
};
__host__ __device__ inline RingTile ring_tile(int b, const RingLaunch& g, int rag_c, int64_t rag_off,
                                              int64_t rag_len) {
  RingTile t;
  const int nf = g.nfull * g.tpp;
  if (b < nf) {
    const int j = b / g.tpp;
    t.tile = b - j * g.tpp;
    const int c = j + g.rot;
    t.c = c >= g.nfull ? c - g.nfull : c;
    t.off = ((int64_t)t.c * g.stride_v + g.off_v) << 4;
    t.len = (int64_t)g.len_v << 4;
  } else {
    t.c = rag_c;
    t.tile = b - nf;
    t.off = rag_off;
    t.len = rag_len;
  }
  return t;
}

// Whether launch_ring_hop takes this hop (hop kinds of the ring, load modes
// 0, 2 and 3, R <= 64, full-piece offsets within 2^31 vectors, at most
// kMaxGridWorkgroups tiles).
bool ring_hop_supported(const RingHop& h, HopKind kind, int ntm);
// Workgroups of its launch: one per 2 x kBlock 16-byte vectors of a piece.
int64_t ring_hop_workgroups(const RingHop& h);
// One launch for the hop (2 vectors per operand per thread, load mode ntm as
// in LaunchTuning::nontemporal); start/stop as for launch_pieces.
hipError_t launch_ring_hop(HopKind kind, const RingHop& h, int ntm, hipStream_t stream,
                           hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// The launch's workgroups as the kernel maps them, on the host: per
// workgroup b, rows[5b..5b+4] = source rank, destination rank, byte offset
// and byte length of its piece, tile index.  Returns the workgroup count
// (rows written for at most max_wg of them).
int64_t ring_hop_layout(const RingHop& h, int64_t* rows, int64_t max_wg);

// Fused MoE dispatch / combine (one gather per row).  Per source rank r:
// `rows` is x[r] (dispatch) or out[r] (combine) and `idx` is src_tok[r]
// (pack position -> token) or slot[r] ((t, k) -> pack position).  Per
// (r, expert e): the pack position where e's rows start, and where they sit
// in the destination's expert-major buffer `exp` (row exp_row onwards).
struct MoeRank {
  char* rows;
  const int32_t* idx;
};
struct MoeSeg {
  int64_t pack_start;
  int64_t exp_row;
  char* exp;
};
// ranks: device [R]; segs: device [R * E], pack_start increasing in e with
// pack_start[r][0] = 0.  rows_per_rank = T * K.  combine = 0: exp row of
// pack position p <- x row idx[p] (idx < T); combine = 1: out row q <- exp
// row of pack position idx[q] (idx < T * K).  Out-of-range indices skip the
// row.
// nt_load: load the rows non-temporally (rows that are read once).
hipError_t launch_moe_gather(int combine, const MoeRank* ranks, const MoeSeg* segs, int R, int E,
                             int64_t rows_per_rank, int64_t idx_limit, int64_t row_bytes,
                             bool nt_load, hipStream_t stream, hipEvent_t start = nullptr,
                             hipEvent_t stop = nullptr);
// dst row i = src row idx[i] for i < nrows; rows of row_bytes (multiple of
// 16); entries outside [0, nsrc) are skipped.
hipError_t launch_permute_rows(char* dst, const char* src, const int32_t* idx, int64_t nrows,
                               int64_t nsrc, int64_t row_bytes, hipStream_t stream);

// Top-K expert ids per token (E <= 1024, K <= 16).
hipError_t launch_moe_topk(const float* logits, int32_t* topk, int64_t T, int E, int K,
                           hipStream_t stream);

// Dispatch plan of one rank: ecnt[E] rows per expert, src_tok[T*K], slot[T*K].
hipError_t launch_moe_plan(const int32_t* topk, int64_t T, int E, int K, int eloc,
                           int64_t* ecnt, int32_t* src_tok, int32_t* slot, hipStream_t stream);

// One wave64 workgroup per block; writes (XCC id, SE id, CU id) per block.
hipError_t launch_probe_cu_ids(int32_t* out, int nblocks, hipStream_t stream);

// Fixed device scratch of the entry points that allocate nothing: one
// array of kScratchBytes per GPU, held until the process ends (its device
// address is resolved once per device, with that device current, by
// resolve_scratch; scratch_address returns it, or NULL before that).
constexpr int64_t kScratchBytes = int64_t(16) << 20;
hipError_t resolve_scratch(int device);
char* scratch_address(int device);

}  // namespace ccr
