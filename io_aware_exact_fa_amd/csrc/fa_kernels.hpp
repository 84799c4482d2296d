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
  int B, H, N;
  int Np;         // N rounded up to a multiple of 64
  float scale;
  int G = 1;      // query heads per K/V head (K, V, dK, dV have H / G heads)
  const int* cu_seqlens = nullptr;   // as in FwdArgs; workspace and LSE rows per
  int total = 0;                     // (sequence, head) stay Np and N
  int wl = kNoLimit, wr = kNoLimit;  // as in FwdArgs
  Dropout drop;                      // as in FwdArgs
};

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
// The backward in three launches: D; dK and dV; dQ.  Only the fields each step
// reads or writes need to be set.
hipError_t launch_bwd_pre(Dt dt, int d, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv(Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq(Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s);

// Backward instances per dtype (T = float, _Float16, __bf16) and head dimension
// (D = 64, 128), defined in one translation unit each (fa_bwd_<dtype>_d<D>.hip).
enum class BwdStep { pre, dkdv, dq };
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
