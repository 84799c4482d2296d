// Device helpers shared by the gfx950 attention kernels: MFMA fragments,
// LDS operand loads (plain and transposing), wave64 half exchanges, exp2.
//
// Register layouts used throughout (CDNA4 MFMA, 64-lane wavefront; lane l,
// col = l % 32, half h = l / 32):
//   v_mfma_f32_32x32x16_{bf16,f16}: A operand A[col][8h + e], B operand
//     B[8h + e][col] (e = 0..7); result element i (0..15) is
//     C[8*(i/4) + 4h + i%4][col].
//   v_mfma_f32_32x32x2_f32: the same with one k value per lane (k = h).
// So a 32x32 result keeps one column per lane and spreads the rows over the
// 16 result registers and the two lane halves.  A result tile can therefore
// feed a later MFMA straight from registers whenever that MFMA contracts
// over the tile's rows: the contraction index is free to be permuted, and
// the "slot" order below is the one the result registers already have.
//
// Slot order of a transposed operand: for MFMA step u over a block of 32 rows
// (16-bit types: u = 0..1, 16 rows per step; f32: u = 0..15, 2 rows per step),
// lane (col, h) supplies, in slot t, row
//     16-bit: 16u + 8(t/4) + 4h + t%4   (t = 0..7)
//     f32:    8(u/4) + 4h + u%4
// of the block, which is exactly result element i = 8u + t (16-bit) or
// i = u (f32) of the same lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
// Calls f(std::integral_constant<int, I>{}) for I = B, ..., E - 1 in order, so
// that each call sees its index as a compile-time constant.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// s_waitcnt operand that waits for every outstanding vector-memory load and
// leaves the other counters alone (vmcnt = 0, expcnt = 7, lgkmcnt = 15).
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  static constexpr int KPL = 8;      // k values per lane per MFMA
  typedef bf16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<_Float16> {
  static constexpr int KPL = 8;
  typedef f16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Steps (MFMAs) needed to contract over a block of 32 rows.
template <typename T> constexpr int steps32() { return 32 / (2 * Mfma<T>::KPL); }

// ---------------------------------------------------------------- fragments

// Plain operand: KPL consecutive elements starting at p (16-byte aligned for 16-bit types).
template <typename T>
__device__ inline typename Mfma<T>::frag load_frag(const T* p) {
  return *reinterpret_cast<const typename Mfma<T>::frag*>(p);
}

// Transposed operand from a row-major LDS matrix M (row pitch `pitch`
// elements): slot t of lane (col, h) gets M[rb + row(u, t, h)][cb + col], with
// the slot order described at the top of this file.
template <typename T>
__device__ inline typename Mfma<T>::frag load_frag_tr(const T* M, int pitch, int rb, int u, int cb,
                                                      int lane);

template <>
__device__ inline float load_frag_tr<float>(const float* M, int pitch, int rb, int u, int cb,
                                            int lane) {
  const int row = rb + 8 * (u >> 2) + 4 * (lane >> 5) + (u & 3);
  return M[row * pitch + cb + (lane & 31)];
}

// 16-bit: two ds_read_b64_tr_b16.  Within each group of 16 lanes, lane 4a+e
// receives element e of the 8-byte rows addressed by lanes a, a+4, a+8, a+12.
// Each lane therefore addresses row rb + 16u + 8q + 4h + (lane%16)/4 at
// column cb + 16((lane/16)%2) + 4(lane%4); read q yields slots 4q..4q+3.
__device__ inline s16x8 load_tr16_pair(const void* M, int pitch, int rb, int u, int cb, int lane) {
  const int row = rb + 16 * u + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int colx = cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const short* base = reinterpret_cast<const short*>(M) + row * pitch + colx;
  s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
  s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * pitch));
  return __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <>
__device__ inline bf16x8 load_frag_tr<__bf16>(const __bf16* M, int pitch, int rb, int u, int cb,
                                              int lane) {
  return __builtin_bit_cast(bf16x8, load_tr16_pair(M, pitch, rb, u, cb, lane));
}

template <>
__device__ inline f16x8 load_frag_tr<_Float16>(const _Float16* M, int pitch, int rb, int u, int cb,
                                               int lane) {
  return __builtin_bit_cast(f16x8, load_tr16_pair(M, pitch, rb, u, cb, lane));
}

// Pack result elements 8u..8u+7 (16-bit) or element u (f32) of a 32x32 result
// tile into an operand fragment, rounding to T (nearest even).
template <typename T>
__device__ inline typename Mfma<T>::frag pack_frag(const f32x16& c, int u);

template <>
__device__ inline float pack_frag<float>(const f32x16& c, int u) { return c[u]; }

template <>
__device__ inline bf16x8 pack_frag<__bf16>(const f32x16& c, int u) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (__bf16)c[8 * u + t];
  return r;
}

template <>
__device__ inline f16x8 pack_frag<_Float16>(const f32x16& c, int u) {
  f16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (_Float16)c[8 * u + t];
  return r;
}

// ps[x] += elements 2x and 2x + 1 of a 16-bit fragment, as they stand in the
// fragment (rounded): one dot-2 instruction against (1, 1) per pair, products
// exact, accumulated in f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ inline void frag_sum4(const typename Mfma<T>::frag& f, float (&ps)[4]);

template <>
__device__ inline void frag_sum4<__bf16>(const bf16x8& f, float (&ps)[4]) {
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int x = 0; x < 4; ++x)
    ps[x] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[2 * x], f[2 * x + 1]}, one, ps[x], false);
}

template <>
__device__ inline void frag_sum4<_Float16>(const f16x8& f, float (&ps)[4]) {
  const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
  for (int x = 0; x < 4; ++x)
    ps[x] = __builtin_amdgcn_fdot2(f16x2{f[2 * x], f[2 * x + 1]}, one, ps[x], false);
}

// Negate every element of a fragment (exact).
template <typename T>
__device__ inline typename Mfma<T>::frag neg_frag(typename Mfma<T>::frag a) { return -a; }

// ---------------------------------------------------------------- lane halves

// Combine a value with the same lane of the other 32-lane half.
__device__ inline float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- AGPR accumulators

// acc += A B on a 32 x 32 x 16 MFMA whose accumulator lives in AGPRs.  Issued
// as inline assembly, so the compiler's hazard recognizer does not see it; the
// kernels that use it keep the hazards on their side: nothing but these MFMAs
// touches the accumulators between agpr_settle() calls, and A and B are VGPRs
// the compiler waits for (LDS reads) or that were written many instructions
// earlier (packed P~, P, dS).  Successive MFMAs on one accumulator (full
// overlap of the source C with the previous result) need no wait states.
template <typename T> __device__ inline void mma_agpr(f32x16& acc, const typename Mfma<T>::frag& a,
                                                      const typename Mfma<T>::frag& b);
template <> __device__ inline void mma_agpr<__bf16>(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <> __device__ inline void mma_agpr<_Float16>(f32x16& acc, const f16x8& a, const f16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last mma_agpr and a VALU access (read or write) of
// its accumulators, and between a VALU write of them and the next mma_agpr:
// 20 (a 32 x 32 MFMA's result is readable 18 wait states after it issues).
__device__ inline void agpr_settle(f32x16 (&acc)[2][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                 "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]));
}
__device__ inline void agpr_settle(f32x16 (&acc)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[1][0]), "+a"(acc[1][1]));
}

// ---------------------------------------------------------------- register transposes

// Four rows of 16 bytes (rows = consecutive keys or queries, 16 bytes = 16/sizeof(T)
// consecutive columns) -> for each column e, the four row values packed in 8
// (16-bit) or 16 (f32) bytes, ready for one LDS store into a transposed tile.
__device__ inline void transpose4_16bit(const uint4 (&x)[4], uint2 (&out)[8]) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(&x[0]);
  const uint32_t* b = reinterpret_cast<const uint32_t*>(&x[1]);
  const uint32_t* c = reinterpret_cast<const uint32_t*>(&x[2]);
  const uint32_t* d = reinterpret_cast<const uint32_t*>(&x[3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // v_perm_b32 selectors: low halves (0x05040100) or high halves (0x07060302) of (S1, S0).
    out[2 * w] = uint2{__builtin_amdgcn_perm(b[w], a[w], 0x05040100u),
                       __builtin_amdgcn_perm(d[w], c[w], 0x05040100u)};
    out[2 * w + 1] = uint2{__builtin_amdgcn_perm(b[w], a[w], 0x07060302u),
                           __builtin_amdgcn_perm(d[w], c[w], 0x07060302u)};
  }
}

__device__ inline void transpose4_32bit(const uint4 (&x)[4], uint4 (&out)[4]) {
  out[0] = uint4{x[0].x, x[1].x, x[2].x, x[3].x};
  out[1] = uint4{x[0].y, x[1].y, x[2].y, x[3].y};
  out[2] = uint4{x[0].z, x[1].z, x[2].z, x[3].z};
  out[3] = uint4{x[0].w, x[1].w, x[2].w, x[3].w};
}

// Store the transpose of a 4-row x (16/sizeof(T))-column block: row r (0..3),
// column e goes to dst[e * pitch + r].  dst must be 8-byte (16-bit T) or
// 16-byte (f32) aligned, pitch in elements.
template <typename T>
__device__ inline void store_transposed4(T* dst, int pitch, const uint4 (&x)[4]) {
  if constexpr (sizeof(T) == 2) {
    uint2 t[8];
    transpose4_16bit(x, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<uint2*>(dst + e * pitch) = t[e];
  } else {
    uint4 t[4];
    transpose4_32bit(x, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<uint4*>(dst + e * pitch) = t[e];
  }
}

// Row permutation inside each group of 16 result rows that swaps bit 2 (the
// lane half) and bit 3 of the row index.  If the A operand of an MFMA that
// produces a 32x32 tile supplies row perm16(r) in place of row r, then the
// eight result elements 8u..8u+7 of lane half h hold rows 16u + 8h + t
// (t = 0..7): a later MFMA that contracts over these rows can read its
// other operand as 8 consecutive rows of a transposed tile (one 16-byte
// load).  Only used for 16-bit types (8 k values per lane).
__device__ inline int perm16(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// ---------------------------------------------------------------- transposed LDS tiles

// Index of element (row, col) in a transposed LDS tile whose rows (one per head
// dimension) hold 64 consecutive keys or queries.  The 16-byte chunks of each
// row are XOR-swizzled by the row so that (a) the transposed stores of the
// 4-row x 16-byte register groups and (b) the 16-byte operand reads of 32
// consecutive rows both hit distinct LDS banks (64 banks x 4 bytes).  Pitch:
// kTrPitch elements.
constexpr int kTrCols = 64;
constexpr int kTrPitch = kTrCols + 8;

template <typename T>
__device__ inline int tr_index(int row, int col) {
  constexpr int KPC = 16 / sizeof(T);                      // elements per 16-byte chunk
  const int swz = sizeof(T) == 2 ? (row >> 4) & 7 : (row >> 2) & 15;
  return row * kTrPitch + ((col / KPC) ^ swz) * KPC + (col % KPC);
}

// A [64 x D] tile (rows = keys or queries) staged global -> registers by NT threads
// in groups of 4 rows x 16 bytes (group g: column chunk g % CPR, rows 4 (g / CPR) .. +3), then
// stored row-major and/or transposed into LDS.  Rows past `nvalid` are clamped to
// the last valid row (callers mask their contribution).
template <typename T, int D, int NT>
struct TileStage {
  static constexpr int E16 = 16 / sizeof(T);
  static constexpr int CPR = D / E16;
  static constexpr int NG = (kTrCols / 4) * CPR;
  static constexpr int GPT = (NG + NT - 1) / NT;
  uint4 x[GPT][4];

  __device__ inline void load(const T* src, int row0, int nvalid, int tid) {
#pragma unroll
    for (int r = 0; r < GPT; ++r) {
      const int g = tid + NT * r;
      const int dg = g % CPR, rg = g / CPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = min(row0 + 4 * rg + i, nvalid - 1);
        if (g < NG) x[r][i] = *reinterpret_cast<const uint4*>(src + (size_t)row * D + dg * E16);
      }
    }
  }
  // Row-major copy: element (row, c) at dst[row * pitch + c].
  __device__ inline void store_rows(T* dst, int pitch, int tid) const {
#pragma unroll
    for (int r = 0; r < GPT; ++r) {
      const int g = tid + NT * r;
      const int dg = g % CPR, rg = g / CPR;
      if (g < NG) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint4*>(dst + (4 * rg + i) * pitch + dg * E16) = x[r][i];
      }
    }
  }
  // Transposed copy: element (row, c) at dst[tr_index(c, row)].
  __device__ inline void store_transposed(T* dst, int tid) const;
};

// Work index of this workgroup: workgroups are dealt to the 8 XCDs round-robin
// by linear id; give each XCD a contiguous range so that the tiles of one head
// share their K/V (or Q/dO) through one L2.
__device__ inline int xcd_work_index() {
  const int nwork = gridDim.x * gridDim.y * gridDim.z;
  int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  if ((nwork & 7) == 0) lin = (lin & 7) * (nwork >> 3) + (lin >> 3);
  return lin;
}

// Tile rank (position in its head's range) and head of this workgroup, for a
// grid of nt tiles per head.  Without HEAVY_FIRST: xcd_work_index order.  With
// it (causal launches, whose tiles differ in cost by rank): each XCD still
// takes a contiguous range of heads, and walks them in groups of up to
// kHeavyGroup heads, each group rank-major, rank 0 (the heaviest) of every
// head of the group first, so that the shortest workgroups come last in each
// group and fill the gaps of the next.  A group rather than all of the XCD's
// heads: the workgroups that run together then stream the K/V (or Q/dO) tiles
// of only a few heads, which stay in the XCD's L2 (walking all 16 heads of an
// XCD at once made the causal kernels fetch 5-6x their algorithmic bytes;
// groups of 4 measured 4-6 % faster than 16 or 8 on B4 H32 N4096, and than 1
// or 2).  Inside an XCD, workgroups go to its shader engines in turn
// (measured: the i-th one of an XCD lands on engine i mod 4 whatever the
// engines' load), so within a rank the heads of a group are rotated by the
// rank: each engine then gets every head's tiles in turn instead of a fixed
// share of the heads, which matters when heads differ in length (packed
// batches).
constexpr int kHeavyGroup = 4;
template <bool HEAVY_FIRST>
__device__ inline void work_item(int nt, int& rank, int& head) {
  const int nwork = gridDim.x * gridDim.y * gridDim.z;
  const int nheads = nwork / nt;
  if (HEAVY_FIRST && (nheads & 7) == 0) {
    const int id = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int hpx = nheads >> 3, li = id >> 3;
    const int gs = hpx < kHeavyGroup ? hpx : kHeavyGroup;
    const int grp = li / (gs * nt), within = li - grp * (gs * nt);
    // The last group of an XCD holds fewer heads when gs does not divide hpx;
    // within a group of gn heads, `within` runs over gn nt (rank, head) pairs.
    const int gn = min(gs, hpx - grp * gs);
    rank = within / gn;
    head = (id & 7) * hpx + grp * gs + (within + rank) % gn;
  } else {
    const int lin = xcd_work_index();
    head = lin / nt;
    rank = lin % nt;
  }
}

// ---------------------------------------------------------------- dropout

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): ten rounds of two 32 x 32 -> 64-bit products mixed
// with the other counter words and the key, the key bumped by two Weyl
// constants between rounds.
__device__ inline void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                     uint32_t k0, uint32_t k1, uint32_t (&w)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  w[0] = c0;
  w[1] = c1;
  w[2] = c2;
  w[3] = c3;
}

// The eight 16-bit uniforms of one call (query q, 16-key group g, key parity
// par): those of keys 16 g + par + 2 t, t = 0..7, half t of the output.
template <class Drop>
__device__ inline void drop_call(const Drop& d, int head, int q, int g, int par, uint32_t (&w)[4]) {
  philox4x32_10((uint32_t)q, (uint32_t)(2 * g + par), (uint32_t)head, d.offset, d.seed_lo,
                d.seed_hi, w);
}

// Keep decision of one element (query q, key k) from its own call.
template <class Drop>
__device__ inline bool drop_keep(const Drop& d, int head, int q, int k) {
  uint32_t w[4];
  drop_call(d, head, q, k >> 4, k & 1, w);
  const int t = (k & 15) >> 1;
  const uint32_t x = (t >> 1) == 0 ? w[0] : (t >> 1) == 1 ? w[1] : (t >> 1) == 2 ? w[2] : w[3];
  return ((t & 1) ? (x >> 16) : (x & 0xFFFFu)) < d.keep_t;
}

// Keep masks of the halves of 4 packed dwords (element 2 k in the low half of
// dword k, 2 k + 1 in the high half) from one call: 0xFFFF where kept.
template <class Drop>
__device__ inline void drop_masks(const Drop& d, const uint32_t (&w)[4], uint32_t (&m)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
    m[k] = ((w[k] & 0xFFFFu) < d.keep_t ? 0xFFFFu : 0u) | ((w[k] >> 16) < d.keep_t ? 0xFFFF0000u : 0u);
}

// Row of a 32-row block (queries or keys) that supplies result row m of an MFMA
// whose A operand is read from a row-major tile (m = 8a + 4h + s -> 8a + 2s + h):
// the 4 rows that one transposing read gathers for a later MFMA are then 2 apart.
__device__ constexpr int row_pi(int m) { return (m & ~7) | ((m & 3) << 1) | ((m >> 2) & 1); }

// ---------------------------------------------------------------- copies into LDS

// Byte address in LDS of a pointer into a __shared__ array.
__device__ inline uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource of the byte range [base, base + bytes): raw addressing
// (stride 0), 32-bit elements, every access checked against the range.
__device__ inline i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Copy 4 bytes per lane from a buffer straight into LDS: lane i reads the dword
// at byte soff + voff_i of the range of rsrc (soff wave-uniform, voff_i per
// lane) and it lands at LDS byte address lds + 4 i (lds wave-uniform).  A dword
// at or past the end of the range is not read and lands as zero, so rows past
// the end of a matrix need no clamping.  Issued as inline assembly so that the compiler adds no waits of its
// own for it: the caller waits with s_waitcnt vmcnt before the data is read,
// and before the barrier that hands it to the other waves.  The instruction
// offset is left at zero: it would move the LDS address as well.  Expects every
// lane of the wave active.
//
// The compiler does not look inside inline assembly for hazards, so the wait
// states before each copy are this code's business: one (s_nop 0) after the
// SALU write of M0 that the compiler places just before the copy, and five
// after any VALU write of an SGPR the copy reads (v_readlane of a spilled
// descriptor, v_readfirstlane).  The second is not paid on every copy: the
// compiler rarely puts such a write there, and the build checks every copy of
// the linked library for it (a descriptor reloaded right before a copy gave a
// garbage base address and a memory fault).  SAFE pays it (s_nop 4, five wait
// states), for instances whose register pressure makes the compiler spill
// copy descriptors to VGPR lanes.
template <bool SAFE = false>
__device__ inline void copy_to_lds(const i32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  if constexpr (SAFE) {
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                 "{m0}"(lds)
                 : "memory");
  } else {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                 "{m0}"(lds)
                 : "memory");
  }
}

// Copy 16 bytes per lane from a buffer straight into LDS: lane i reads bytes
// soff + voff_i .. + 15 of the range of rsrc and they land at LDS byte address
// lds + 16 i, so one copy fills 1 KB of LDS.  Range checking, waits, the
// instruction offset and the leading wait states (SAFE) as for copy_to_lds.
// Expects every lane active.
template <bool SAFE = false>
__device__ inline void copy16_to_lds(const i32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  if constexpr (SAFE)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(soff), "{m0}"(lds)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(soff), "{m0}"(lds)
                 : "memory");
}

// Copy NG row groups of one matrix (1 KB each, 64 lanes x 16 bytes) that lie
// 1 KB apart in global memory and STEP bytes apart in LDS, in one block: the
// compiler sets M0 (the first group's LDS address) once, the scalar offset is
// shared, and the instruction offset g STEP moves both addresses of group g.
// Lane voff[g] makes up the difference of the two strides: with the
// resource's base moved back by copy16_shift(NG, STEP) bytes, voff[g] = the
// lane's offset in a group + copy16_shift - g (STEP - 1024), never negative.
// Wait states and range checking as for copy16_to_lds.
__host__ __device__ constexpr int copy16_shift(int NG, int STEP) { return (NG - 1) * (STEP - 1024); }

template <int NG, int STEP, bool SAFE = false>
__device__ inline void copy16_groups(const i32x4& rsrc, const uint32_t (&voff)[NG], uint32_t soff,
                                     uint32_t lds) {
  static_assert((NG == 2 || NG == 4) && STEP >= 1024 && (NG - 1) * STEP < 4096,
                "two or four groups within the 12-bit instruction offset");
  if constexpr (NG == 2) {
    asm volatile("s_nop %4\n\t"
                 "buffer_load_dwordx4 %0, %2, %3 offen lds\n\t"
                 "buffer_load_dwordx4 %1, %2, %3 offen offset:%5 lds"
                 ::"v"(voff[0]), "v"(voff[1]), "s"(rsrc), "s"(soff), "n"(SAFE ? 4 : 0), "n"(STEP),
                 "{m0}"(lds)
                 : "memory");
  } else {
    asm volatile("s_nop %6\n\t"
                 "buffer_load_dwordx4 %0, %4, %5 offen lds\n\t"
                 "buffer_load_dwordx4 %1, %4, %5 offen offset:%7 lds\n\t"
                 "buffer_load_dwordx4 %2, %4, %5 offen offset:%8 lds\n\t"
                 "buffer_load_dwordx4 %3, %4, %5 offen offset:%9 lds"
                 ::"v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(rsrc), "s"(soff),
                 "n"(SAFE ? 4 : 0), "n"(STEP), "n"(2 * STEP), "n"(3 * STEP), "{m0}"(lds)
                 : "memory");
  }
}

// ------------------------------------------------- tile layouts of the 16-bit kernels
//
// A tile holds rows of 2D bytes (D 16-bit elements) in LDS.  Two reads use it:
// A-operand reads (16 bytes: 8 consecutive elements of one row; the 32 lanes of
// a lane half read rows row_pi(0..31) of a 32-row block, all at the same
// 16-byte chunk) and transposing reads (8 bytes per lane; a lane half reads
// rows 2s + h, s = 0..3, of an 8-row step, 64 bytes each).  Both layouts below
// keep every 16-lane quarter of an A read and every lane half of a
// transposing read on distinct banks, and are filled one group of rows (1 KB,
// 64 lanes x 16 bytes) per copy.  Offsets between rows that are a multiple of
// ROWS_PER_COPY apart are (rows) * PB in both.
//
// d = 64: 8-row groups of 1 KB, dense (rows 128 bytes apart).  Row r = 8 g + x
// sits at row slot slot(x, g & 1) = 2 x0 + (x1 ^ g0) + 4 x2 of its group, its
// 16-byte chunk c at chunk c ^ x (x0..x2, g0: bits of x and g).  The rows of a
// quarter-wave A read then cover bank groups 8 (x1 ^ g0) + (c ^ x) once each,
// and so do the 4 rows x 4 chunks of a half-wave transposing read.
// d = 128: 4-row groups of 1 KB (rows 256 bytes apart), groups 1152 bytes
// apart; chunk c of row r at chunk c ^ swz(r), swz(r) = r0 | r3 << 1 | r1 << 2
// (bits of r).
template <int D> struct TileLds;

template <> struct TileLds<64> {
  static constexpr int PB = 128;             // per row, for multiples of 8 rows
  static constexpr int ROWS_PER_COPY = 8;
  __device__ static constexpr int slot(int x, int g0) {
    return 2 * (x & 1) + (((x >> 1) & 1) ^ g0) + 4 * (x >> 2);
  }
  // Byte address of chunk c of row r (from the start of the tile).
  __device__ static constexpr int at(int r, int c) {
    return (r >> 3) * 1024 + 128 * slot(r & 7, (r >> 3) & 1) + 16 * ((c ^ r) & 7);
  }
  // Lane offsets: A reads of k step ks at a[ks]; transposing reads of the
  // 8-row step with bit 3 of its rows = rp at t[rp][db] (the caller adds the
  // step's rows * PB); group copies of groups g with g & 1 = x from global byte
  // offset c[x] (relative to the group's first row).
  int a[4], t[2][2], c[2];
  __device__ TileLds(int lane) {
    const int col = lane & 31, h = lane >> 5;
    const int ts = (lane >> 2) & 3, ta = lane & 3, tg = (lane >> 4) & 1;
    const int ra = row_pi(col);
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = at(ra, 2 * k + h);
#pragma unroll
    for (int rp = 0; rp < 2; ++rp)
#pragma unroll
      for (int db = 0; db < 2; ++db)
        t[rp][db] = at(2 * ts + h + 8 * rp, 4 * db + 2 * tg + (ta >> 1)) - 1024 * rp + 8 * (ta & 1);
    // Lane i fills row slot i >> 3, chunk slot i & 7 of the group.
    const int s = lane >> 3;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = ((s >> 1) & 1) | (((s & 1) ^ x) << 1) | ((s >> 2) << 2);
      c[x] = 128 * r + 16 * ((lane & 7) ^ r);
    }
  }
  __device__ int A(int ks) const { return a[ks]; }
  __device__ int T(int rp, int db) const { return t[rp][db & 1]; }
};

// A 64-column tile written from registers rather than copied (the dS^T buffers
// of the one-pass backward): rows 160 bytes apart (128 + 32 of padding), the
// 16-byte chunk c of row r at chunk c ^ ((r >> 3) & 1); reads as in TileLds.
struct RowLds64 {
  static constexpr int PB = 160;
  int t[2];
  __device__ RowLds64(int lane) {
    const int h = lane >> 5;
    const int ts = (lane >> 2) & 3, ta = lane & 3, tg = (lane >> 4) & 1;
#pragma unroll
    for (int x = 0; x < 2; ++x) t[x] = (2 * ts + h) * PB + 16 * ((2 * tg + (ta >> 1)) ^ x) + 8 * (ta & 1);
  }
  __device__ int T(int rp, int db) const { return t[rp] + 64 * db; }
};

template <> struct TileLds<128> {
  static constexpr int PB = 288;             // per row, for multiples of 4 rows
  static constexpr int ROWS_PER_COPY = 4;
  __device__ static constexpr int row(int r) { return (r >> 2) * 4 * PB + (r & 3) * 256; }
  __device__ static constexpr int swz(int r) {
    return (r & 1) | (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2);
  }
  // Lane offsets: A reads of k step ks at a[ks & 3] + 128 (ks >> 2);
  // transposing reads at t[rp][db & 1] + 128 (db >> 1); group copies of groups
  // q with (q >> 1) & 1 = x from global byte offset c[x] (relative to the
  // group's first row).
  int a[4], t[2][2], c[2];
  __device__ TileLds(int lane) {
    const int col = lane & 31, h = lane >> 5;
    const int ts = (lane >> 2) & 3, ta = lane & 3, tg = (lane >> 4) & 1;
    const int ra = row_pi(col);
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = row(ra) + 16 * ((2 * k + h) ^ swz(ra));
    // Rows 2 ts + h (+ 8 rp + multiples of 16): swz = h | rp << 1 | (ts & 1) << 2.
#pragma unroll
    for (int rp = 0; rp < 2; ++rp)
#pragma unroll
      for (int d0 = 0; d0 < 2; ++d0)
        t[rp][d0] = row(2 * ts + h) + 16 * ((2 * tg + (ta >> 1)) ^ (2 * rp + h)) + 8 * (ta & 1) +
                    64 * (d0 ^ (ts & 1));
    // Lane i fills chunk i & 15 of row i >> 4 of the group.
    const int gr = lane >> 4;
#pragma unroll
    for (int x = 0; x < 2; ++x)
      c[x] = gr * 256 + 16 * ((lane & 15) ^ ((gr & 1) | (x << 1) | (((gr >> 1) & 1) << 2)));
  }
  __device__ int A(int ks) const { return a[ks & 3] + 128 * (ks >> 2); }
  __device__ int T(int rp, int db) const { return t[rp][db & 1] + 128 * (db >> 1); }
};

// s_waitcnt operand that waits until at most n vector-memory loads are
// outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima).
__host__ __device__ constexpr int wait_vmcnt(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// ---------------------------------------------------------------- stores

// Store 4 consecutive values (rounded to T) at p.
template <typename T> __device__ inline void store4(T* p, float a, float b, float c, float d);

template <> __device__ inline void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

template <> __device__ inline void store4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}

template <>
__device__ inline void store4<_Float16>(_Float16* p, float a, float b, float c, float d) {
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<f16x4*>(p) = f16x4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
}

template <typename T> __device__ inline float to_f32(T x) { return (float)x; }

template <typename T, int D, int NT>
__device__ inline void TileStage<T, D, NT>::store_transposed(T* dst, int tid) const {
#pragma unroll
  for (int r = 0; r < GPT; ++r) {
    const int g = tid + NT * r;
    const int dg = g % CPR, rg = g / CPR;
    if (g < NG) {
      const int c0 = dg * E16;
      // The E16 transposed rows c0..c0+E16-1 share one swizzle (it changes every
      // 16 rows for 16-bit types and every 4 rows for f32), so one base index
      // serves all of them.
      store_transposed4<T>(dst + tr_index<T>(c0, 4 * rg), kTrPitch, x[r]);
    }
  }
}

}  // namespace fa
