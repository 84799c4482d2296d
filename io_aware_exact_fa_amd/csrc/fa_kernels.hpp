// Host-side declarations of the kernel launchers (one per dtype x head dim x
// causal instance).  Every launcher only enqueues work on `stream` and
// returns hipGetLastError(); argument checks live in fa_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// An open side of the attention window (no limit on j - i or i - j).
constexpr int kNoLimit = 1 << 30;

// Dropout on P: element (query i, key j) of head b H + h is kept iff its 16-bit
// uniform is below keep_t (keep_t = 65536: no dropout); kept elements are
// scaled by `scale` = 65536 / keep_t.  The uniform of (i, j) is half number
// (j % 16) / 2 (low half of word 0 first) of Philox4x32-10 with counter
// (i, 2 (j / 16) + j % 2, b H + h, offset) and key (seed_lo, seed_hi).
struct Dropout {
  uint32_t keep_t = 65536;
  float scale = 1.f;
  uint32_t seed_lo = 0, seed_hi = 0, offset = 0;
};

// Block-sparse mask: blocks of kBlockQ queries x kBlockK keys (positions in the
// sequence); block (qb, kb) of query head h is mask[(h % heads) * nbq * nbk +
// qb * nbk + kb], nonzero = computed.  Every workgroup of every kernel lies in
// one block row (at most kBlockQ query rows) or one block column (kBlockK keys).
constexpr int kBlockQ = 256, kBlockK = 128;
struct BlockMask {
  const uint8_t* mask = nullptr;   // null: every block is computed
  int heads = 1, nbq = 0, nbk = 0;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N;    // H query heads; K and V have H / G heads
  float scale;
  int G = 1;      // query heads per K/V head
  // Packed variable-length batch when non-null: [B + 1] token offsets of the
  // sequences in tensors laid out [heads, total, d]; N is then the longest
  // length (the grid and the LSE rows per (sequence, head)).
  const int* cu_seqlens = nullptr;
  int total = 0;
  // Window: key j is visible to query i iff i - wl <= j <= i + wr (positions in
  // the sequence; wl, wr >= 0 or kNoLimit).  Causal launches take wr = 0.
  int wl = kNoLimit, wr = kNoLimit;
  Dropout drop;
  BlockMask bm;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;   // workspace [B,H,Np]: D_i = rowsum(dO_i * O_i), 0 past N
  float* l2;      // workspace [B,H,Np]: LSE_i * log2(e), +inf past N
  // Workspace [B,H,Np,d] float32 of the one-pass backward: dS K summed over the
  // key tiles by atomic adds (null: the two-pass backward, dQ by its own pass).
  // The preprocess zeroes it when set.
  float* dqacc = nullptr;
  int B, H, N;
  int Np;         // N rounded up to a multiple of 64
  float scale;
  int G = 1;      // query heads per K/V head (K, V, dK, dV have H / G heads)
  const int* cu_seqlens = nullptr;   // as in FwdArgs; workspace and LSE rows per
  int total = 0;                     // (sequence, head) stay Np and N
  int wl = kNoLimit, wr = kNoLimit;  // as in FwdArgs
  Dropout drop;                      // as in FwdArgs
  BlockMask bm;                      // as in FwdArgs
};

// Active tiles along one block row (forward, dQ: key tiles of one query block)
// or block column (dK/dV: query tiles of one key block) of a block mask, tpb
// tiles per block.  Blocks are scanned 64 at a time, one byte load per lane and
// a ballot; everything else is uniform (scalar).
struct BlockSkip {
  const uint8_t* base = nullptr;   // block x of the row/column at base[x * stride]; null: all
  int stride = 1, nblk = 0, tpb = 1;
  int chunk = -1;
  uint64_t bits = 0;
  // The first active tile >= t, or some tile >= end if there is none below end.
  __device__ int next(int t, int end, int lane) {
    if (__builtin_expect(!base, 1)) return t;   // no block mask: the loops' straight path
    while (t < end) {
      const int blk = t / tpb, c = blk >> 6;
      if (c != chunk) {
        chunk = c;
        const int x = (c << 6) + lane;
        bits = __ballot(x < nblk && base[(size_t)x * stride] != 0);
      }
      const uint64_t m = bits >> (blk & 63);
      if (m & 1ull) return t;
      t = m ? (blk + __builtin_ctzll(m)) * tpb : ((c + 1) << 6) * tpb;
    }
    return t;
  }
};

// Whether block (q / kBlockQ, k / kBlockK) of query head `head` is computed
// (the register-staged kernels test tiles one by one instead of skipping).
template <class Args>
__device__ inline bool block_on(const Args& a, int head, int q, int k) {
  if (!a.bm.mask) return true;
  return a.bm.mask[(size_t)((head % a.H) % a.bm.heads) * a.bm.nbq * a.bm.nbk +
                   (size_t)(q / kBlockQ) * a.bm.nbk + k / kBlockK] != 0;
}

// The workgroup's next tiles: t[0] the current one, t[1..3] the following active
// ones (copied ahead), s the step count (buffer parity of the 4-wave kernels).
struct TileQueue {
  int t[4];
  int s;
  __device__ void start(BlockSkip& sk, int lo, int end, int lane) {
    t[0] = sk.next(lo, end, lane);
#pragma unroll
    for (int k = 1; k < 4; ++k) t[k] = sk.next(t[k - 1] + 1, end, lane);
    s = 0;
  }
  __device__ void advance(BlockSkip& sk, int end, int lane) {
    t[0] = t[1];
    t[1] = t[2];
    t[2] = t[3];
    t[3] = sk.next(t[3] + 1, end, lane);
    ++s;
  }
};

// The skip of one workgroup: a row of the mask (forward, dQ: query block qb,
// key tiles of `tile` keys) or a column (dK/dV: key block kb, query tiles).
template <class Args>
__device__ inline BlockSkip block_row(const Args& a, int head, int qb, int tile) {
  BlockSkip sk;
  if (a.bm.mask) {
    sk.base = a.bm.mask + (size_t)((head % a.H) % a.bm.heads) * a.bm.nbq * a.bm.nbk +
              (size_t)qb * a.bm.nbk;
    sk.stride = 1;
    sk.nblk = a.bm.nbk;
    sk.tpb = kBlockK / tile;
  }
  return sk;
}
template <class Args>
__device__ inline BlockSkip block_col(const Args& a, int head, int kb, int tile) {
  BlockSkip sk;
  if (a.bm.mask) {
    sk.base = a.bm.mask + (size_t)((head % a.H) % a.bm.heads) * a.bm.nbq * a.bm.nbk + kb;
    sk.stride = a.bm.nbk;
    sk.nblk = a.bm.nbq;
    sk.tpb = kBlockQ / tile;
  }
  return sk;
}

// Tile ranges of one workgroup under the window: rows [ra, rb] of the outer
// operand (queries in the forward and dQ, keys in dK/dV) need inner tiles
// (BI rows each, `n` rows in all) [lo, hi); of these, [ml, mu) need no mask in
// any outer row (every element inside the window and below n), [lo, ml) and
// [mu, hi) do.  The inner rows visible to outer row r are [r - back, r + fwd],
// with back >= 0 and fwd >= 0 (or kNoLimit).  `full_tail`: inner rows past n
// need no mask (the dK/dV kernels, whose padding rows contribute zero).
struct TileRange {
  int lo, ml, mu, hi;
};
__device__ inline TileRange tile_range(int ra, int rb, int n, int back, int fwd, int BI,
                                       bool full_tail) {
  TileRange t;
  const int first = max(0, ra - back), last = min(n - 1, rb + fwd);
  t.lo = first / BI;
  t.hi = last / BI + 1;
  // [ml, mu): tiles whose first row is >= rb - back and whose last row is <= ra + fwd.
  t.ml = rb - back <= 0 ? t.lo : min(t.hi, (rb - back + BI - 1) / BI);
  t.ml = max(t.ml, t.lo);
  int mu = min(t.hi, (ra + fwd + 1) / BI);
  if (!full_tail) mu = min(mu, n / BI);
  t.mu = max(mu, t.ml);
  return t;
}

// Rows of the (sequence, query head) pair hd = b H + h in the row-major
// tensors: the first row of its query slab (q, o, dout, dq), of its K/V head's
// slab (k, v, dk, dv), the row distance between consecutive query heads, and
// the number of rows.  Dense: slab hd of N rows.  Packed: rows cu[b] .. cu[b+1]
// of head h's slab of `total` rows; offsets are clamped into [0, total] and the
// length to N, so any offsets stay inside the tensors.
struct Span {
  size_t q, kv, hs;
  int n;
};
// Packed batches: the work order's linear head index is taken head-major
// (lin = h B + b), so that the contiguous range of heads that one XCD receives
// spans every sequence and the XCDs get equal shares of long and short ones;
// returns the (sequence, head) index b Hx + h.  Dense launches keep lin.
template <class Args>
__device__ inline int packed_head(const Args& a, int lin, int Hx) {
  if (!a.cu_seqlens) return lin;
  const int h = lin / a.B;
  return (lin - h * a.B) * Hx + h;
}

template <class Args>
__device__ inline Span span_of(const Args& a, int hd) {
  if (!a.cu_seqlens)
    return Span{(size_t)hd * a.N, (size_t)(hd / a.G) * a.N, (size_t)a.N, a.N};
  const int b = hd / a.H, h = hd - b * a.H;
  const int s0 = min(max(a.cu_seqlens[b], 0), a.total);
  const int s1 = min(max(a.cu_seqlens[b + 1], s0), a.total);
  return Span{(size_t)h * a.total + s0, (size_t)(h / a.G) * a.total + s0, (size_t)a.total,
              min(s1 - s0, a.N)};
}

enum class Dt { f32 = 0, f16 = 1, bf16 = 2 };

hipError_t launch_fwd(Dt dt, int d, bool causal, const FwdArgs& a, hipStream_t s);
// The forward with 64 query rows per wave (fa_fwd64.hip): 16-bit types,
// d = 128, no dropout.
hipError_t launch_fwd64(Dt dt, int d, bool causal, const FwdArgs& a, hipStream_t s);
// The backward in three launches: D; dK and dV; dQ.  Only the fields each step
// reads or writes need to be set.
hipError_t launch_bwd_pre(Dt dt, int d, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv(Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq(Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s);
// The one-pass backward (16-bit types without dropout): dK, dV and the atomic
// dQ accumulation in one launch, then dq = scale * accumulator.
hipError_t launch_bwd_dkdvq(Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dqfin(Dt dt, int d, const BwdArgs& a, hipStream_t s);

// Backward instances per dtype (T = float, _Float16, __bf16) and head dimension
// (D = 64, 128), defined in one translation unit each (fa_bwd_<dtype>_d<D>.hip).
enum class BwdStep { pre, dkdv, dq, dkdvq, dqfin };
template <typename T, int D>
hipError_t launch_bwd_inst(BwdStep st, bool causal, const BwdArgs& a, hipStream_t s);
#define FA_BWD_EXTERN(T, D) \
  extern template hipError_t launch_bwd_inst<T, D>(BwdStep, bool, const BwdArgs&, hipStream_t);
FA_BWD_EXTERN(float, 64)
FA_BWD_EXTERN(float, 128)
FA_BWD_EXTERN(_Float16, 64)
FA_BWD_EXTERN(_Float16, 128)
FA_BWD_EXTERN(__bf16, 64)
FA_BWD_EXTERN(__bf16, 128)
#undef FA_BWD_EXTERN

}  // namespace fa
