// Forward attention kernels for gfx950.
//
// One workgroup computes a tile of query rows of one (batch, head); each wave
// owns 32 rows (the queries are split across waves, so the softmax of a row
// never leaves its wave).  The workgroup loops over key/value tiles of 64 keys.
// Two kernels:
//   fwd16_kernel (16-bit types, d = 128): 8 waves (256 rows); tiles copied
//     from global memory straight into LDS, read as 8-byte rows (K) and by
//     transposing reads (V^T); each tile one fixed MFMA stream.
//   fwd_kernel (fp32, and 16-bit d = 64): 8 waves for 16-bit, 4 for fp32;
//     tiles staged global -> registers -> LDS, V stored transposed.
// Per tile and wave:
//   S^T = K_j Q^T            MFMA, fp32 accumulation (32 queries x 64 keys);
//   mask                     only on tiles crossing the causal diagonal or N;
//   m_new = max(m, rowmax)   per-lane max, then one exchange between halves;
//   P~ = 2^(c S - m_new)     c = |scale| log2(e), so the largest P~ of a row is 1;
//   l = l 2^(m - m_new) + rowsum P~   (kept per lane; the halves are added once
//                                       at the end);
//   O^T = 2^(m - m_new) O^T + V_j^T P~^T   MFMA, P~ rounded to the input type.
// After the last tile O = O^T / l is stored once and LSE = ln2 (m + log2 l).
//
// The computation order is the query-tile-outer loop with the unnormalized
// accumulator and a single division at the end ("FlashAttention-2: Faster
// Attention with Better Parallelism and Work Partitioning", sections
// "결과: FlashAttention-2 Forward 알고리즘" and "개선 1"), whose per-row state and
// merge rule are those of "FlashAttention 원 논문 해부", section
// "두 tile을 한 row로 합치는 식".  Splitting query rows across waves follows the
// same FlashAttention-2 page ("Work Partitioning Between Warps", split-Q).
// Causal key tiles above the diagonal are never loaded (FlashAttention-2 page,
// "Causal Masking 최적화"); with the causal mask the heavier query tiles (more
// key tiles) are launched first.
//
// Computing S^T instead of S puts one query per lane (the MFMA result keeps
// one column per lane), so the row max and sum are in-register reductions
// plus one exchange between the two 32-lane halves, and the rescale factor
// is a per-lane scalar for the O^T accumulator.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <typename T, int D>
struct FwdTile {
  // 16-bit types: 8 waves x 32 query rows, so each K/V tile streamed from L2
  // serves 256 rows (the tile traffic, not the MFMA work, bounded 4-wave tiles);
  // f32 (1 wave per SIMD for registers) keeps 4 waves.
  static constexpr int NW = sizeof(T) == 2 ? 8 : 4;
  static constexpr int BR = 32 * NW;             // query rows per workgroup
  static constexpr int BC = 64;                  // keys per tile
  static constexpr int NT = 64 * NW;             // threads per workgroup
  static constexpr int KPL = Mfma<T>::KPL;
  static constexpr int KM = 2 * KPL;             // MFMA k depth
  static constexpr int NKS = D / KM;             // MFMAs per 32x32 block of S
  static constexpr int NU = steps32<T>();        // MFMAs per 32 keys of P V
  static constexpr int E16 = 16 / sizeof(T);     // elements per 16-byte chunk
  static constexpr int KP = D + E16;             // K row pitch (elements)
  static constexpr int VP = BC + 8;              // V^T row pitch (elements)
  static constexpr int CPR = D / E16;            // 16-byte chunks per K row
  static constexpr int KCPT = BC * CPR / NT;     // K chunks per thread per tile
  static constexpr int VGRP = (BC / 4) * CPR;    // 4-key x 16-byte V groups per tile
  static constexpr int VGPT = (VGRP + NT - 1) / NT;
  static constexpr int WAVES_PER_SIMD = sizeof(T) == 2 ? 2 : 1;
  static constexpr int KS_EL = BC * KP;          // one K buffer, elements
  static constexpr int VS_EL = D * VP;           // one V^T buffer, elements
  static_assert(BC * CPR % NT == 0, "K tile must split evenly over the threads");
};

// V^T tile layout: row d (head dimension) holds the tile's keys, in 16-byte
// chunks whose order is XOR-swizzled by the row, so that both the transposed
// stores (each lane writes 4 keys of one row) and the 16-byte operand reads
// (32 consecutive rows, one chunk each) hit distinct LDS banks.
template <typename T>
__device__ inline int vt_index(int d, int key) {
  constexpr int KPC = 16 / sizeof(T);                      // keys per 16-byte chunk
  constexpr int SW = sizeof(T) == 2 ? 7 : 15;
  const int swz = sizeof(T) == 2 ? (d >> 4) & SW : (d >> 2) & SW;
  return ((key / KPC) ^ swz) * KPC + (key % KPC);
}

// BSPARSE: a block mask is given and tiles of dropped blocks are skipped one by
// one; without it the per-tile test is compiled out (it costs this kernel 8-12 %).
template <typename T, int D, bool CAUSAL, bool DROP, bool BSPARSE>
__global__ __launch_bounds__((FwdTile<T, D>::NT), (FwdTile<T, D>::WAVES_PER_SIMD))
void fwd_kernel(FwdArgs a) {
  using C = FwdTile<T, D>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr bool kPerm = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) T Ks[2][C::KS_EL];
  __shared__ __attribute__((aligned(16))) T Vt[2][C::VS_EL];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, col = lane & 31, h = lane >> 5;

  // Workgroup -> (head, query tile).  Workgroups are dealt to the 8 XCDs
  // round-robin by linear id; give each XCD a contiguous range of (head, tile)
  // pairs so the tiles of one head share their K/V through one L2.  Under the
  // causal mask the tiles of a head run heaviest (most key tiles) first.
  const int ntq = gridDim.x;
  const int nwork = ntq * gridDim.y * gridDim.z;
  int lin = blockIdx.x + ntq * (blockIdx.y + gridDim.y * blockIdx.z);
  if ((nwork & 7) == 0) lin = (lin & 7) * (nwork >> 3) + (lin >> 3);
  const size_t head = (size_t)packed_head(a, lin / ntq, a.H);
  const Span sp = span_of(a, (int)head);
  const int N = sp.n;
  // Causal: the tile with the most keys first (counted in this sequence's tiles).
  const int ntq_own = (N + C::BR - 1) / C::BR;
  const int qt = CAUSAL ? ntq_own - 1 - (lin % ntq) : (lin % ntq);
  if (qt < 0 || qt >= ntq_own) return;   // a tile past the end of a shorter sequence
  const int q0 = qt * C::BR;
  const T* Q = static_cast<const T*>(a.q) + sp.q * D;
  const T* K = static_cast<const T*>(a.k) + sp.kv * D;   // the head's K/V head
  const T* V = static_cast<const T*>(a.v) + sp.kv * D;
  T* O = static_cast<T*>(a.o) + sp.q * D;
  float* L = a.lse + head * a.N;

  const int qw = q0 + 32 * w;   // first query row of this wave
  const int myq = qw + col;     // the query row of this lane

  // Q^T operand, held for the whole kernel.  Rows past N read row N-1 (their
  // results are never stored).  A negative scale is folded into Q (exact sign
  // flip) so that c > 0 and max(c S) = c max(S).
  const float c = fabsf(a.scale) * kLog2e;
  frag qf[C::NKS];
  {
    const T* qrow = Q + (size_t)min(myq, N - 1) * D + C::KPL * h;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const frag f = load_frag<T>(qrow + ks * C::KM);
      qf[ks] = (a.scale < 0.f) ? neg_frag<T>(f) : f;
    }
  }

  // Window: keys [myq - wl, myq + wr] of this lane's row are visible.
  const int wl = a.wl, wr = CAUSAL ? min(a.wr, 0) : a.wr;
  // Key tiles of the workgroup: [j0, ntiles).
  const TileRange tr = tile_range(q0, min(q0 + C::BR, N) - 1, N, wl, wr, C::BC, false);
  const int j0 = tr.lo, ntiles = tr.hi;
  // Tiles this wave needs: [wfirst, wlast]; wlast = -1 if the wave holds no
  // row below N.
  const int wfirst = max(0, qw - wl) / C::BC;
  const int wlast = (qw >= N) ? -1 : min(qw + 31 + wr, N - 1) / C::BC;

  // This lane's K row inside each 32-key block (permuted for 16-bit types, so
  // that lane half h ends up holding keys 16u + 8h + t of the P~ operand).
  const int krow = kPerm ? perm16(col) : col;
  // Key (inside a 32-key block) of result element i of this lane: key0_of(i) + hoff,
  // with key0_of(i) the key of lane half 0 (a compile-time constant per i).
  const int hoff = kPerm ? 8 * h : 4 * h;
  auto key0_of = [](int i) {
    const int r = 8 * (i >> 2) + (i & 3);
    return kPerm ? perm16(r) : r;
  };

  // Staging registers: K of tile j+2 and V of tile j+1 while tile j is computed.
  // Rows past N are clamped to row N-1: their scores are masked to -inf and their
  // P~ set to 0.
  uint4 kst[C::KCPT];
  uint4 vst[C::VGPT][4];
  auto gload_k = [&](int j) {
    const int key0 = j * C::BC;
#pragma unroll
    for (int r = 0; r < C::KCPT; ++r) {
      const int ch = tid + r * C::NT, row = ch / C::CPR, cc = ch % C::CPR;
      kst[r] = *reinterpret_cast<const uint4*>(K + (size_t)min(key0 + row, N - 1) * D + cc * C::E16);
    }
  };
  auto gload_v = [&](int j) {
    const int key0 = j * C::BC;
#pragma unroll
    for (int r = 0; r < C::VGPT; ++r) {
      const int g = tid + r * C::NT;
      const int dg = g % C::CPR, kg = g / C::CPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = min(key0 + 4 * kg + i, N - 1);
        if (g < C::VGRP) vst[r][i] = *reinterpret_cast<const uint4*>(V + (size_t)key * D + dg * C::E16);
      }
    }
  };
  auto sstore_k = [&](int buf) {
#pragma unroll
    for (int r = 0; r < C::KCPT; ++r) {
      const int ch = tid + r * C::NT, row = ch / C::CPR, cc = ch % C::CPR;
      *reinterpret_cast<uint4*>(&Ks[buf][row * C::KP + cc * C::E16]) = kst[r];
    }
  };
  auto sstore_v = [&](int buf) {
#pragma unroll
    for (int r = 0; r < C::VGPT; ++r) {
      const int g = tid + r * C::NT;
      if (g < C::VGRP) {
        const int dg = g % C::CPR, kg = g / C::CPR;
        const int d0 = dg * C::E16;
        // The E16 rows d0..d0+E16-1 share one swizzle (it changes every 4 or 16 rows).
        store_transposed4<T>(&Vt[buf][d0 * C::VP + vt_index<T>(d0, 4 * kg)], C::VP, vst[r]);
      }
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;   // running max of c*S (log2 units)
  float l_run = 0.f;         // this lane's share of the running normalizer

  // S^T of one 64-key tile (two 32-key blocks) from K buffer `kbuf`.
  auto s_tile = [&](int kbuf, f32x16 (&sn)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const T* krowp = &Ks[kbuf][(kb * 32 + krow) * C::KP + C::KPL * h];
      frag kf[C::NKS];
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) kf[ks] = load_frag<T>(krowp + ks * C::KM);
      sn[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) sn[kb] = M::mma(kf[ks], qf[ks], sn[kb]);
    }
  };
  // P~ = 2^(c S - m) for the tile with reference max m_use, row-sum partials.
  // DROP: the sum takes every P~, the P~V operand only the kept ones (each
  // element's keep bit from its own generator call).
  auto exp_tile = [&](f32x16 (&sc)[2], float m_use, bool masked, int key0) {
    const float nm = -m_use;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = sc[kb][i];
        float p = exp2_fast(fmaf(x, c, nm));
        if (masked) p = (x == -INFINITY) ? 0.f : p;   // exact also for c == 0
        ps[i & 3] += p;
        if constexpr (DROP)
          if (!drop_keep(a.drop, (int)head, myq, key0 + kb * 32 + key0_of(i) + hoff)) p = 0.f;
        sc[kb][i] = p;
      }
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };
  auto tile_max = [&](const f32x16 (&sc)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
    mx = half_max(mx);
    return (mx == -INFINITY) ? -INFINITY : mx * c;
  };

  // Software pipeline: during iteration j the matrix core computes S of tile j+1
  // while the vector unit computes the softmax of tile j, then P~_j V_j is
  // issued.  K therefore runs one tile ahead of V in LDS (two buffers each, one
  // barrier per iteration): iteration j reads K_{j+1} and V_j and writes
  // K_{j+2} and V_{j+1}.
  gload_k(j0);
  gload_v(j0);
  sstore_k(j0 & 1);
  sstore_v(j0 & 1);
  if (j0 + 1 < ntiles) {
    gload_k(j0 + 1);
    sstore_k((j0 + 1) & 1);
  }
  __syncthreads();
  // Tiles this wave computes: inside its range and in an active block of a block
  // mask (the whole workgroup lies in one block row).
  auto proc = [&](int j) {
    if constexpr (BSPARSE)
      return j < ntiles && j >= wfirst && j <= wlast && block_on(a, (int)head, q0, j * C::BC);
    else
      return j >= wfirst && j <= wlast;
  };
  f32x16 sc[2];
  if (proc(j0)) s_tile(j0 & 1, sc);
  // Iteration j0 overwrites the K buffer read just above with K of tile j0 + 2.
  __syncthreads();
  for (int j = j0; j < ntiles; ++j) {
    if (j + 2 < ntiles) gload_k(j + 2);
    if (j + 1 < ntiles) gload_v(j + 1);
    // A wave that skips this tile but computes the next one takes its S now
    // (without a block mask: the wave's first tile is the next one).
    const bool pj = proc(j);
    if (BSPARSE ? (!pj && proc(j + 1)) : (j + 1 == wfirst && wfirst <= wlast))
      s_tile((j + 1) & 1, sc);
    if (pj) {
      const int key0 = j * C::BC;
      const bool masked = (key0 + C::BC - 1 > qw + wr) || (key0 < qw + 31 - wl) || (key0 + C::BC > N);
      f32x16 sn[2];
      float m_new, lsum;
      if (!masked) {
        // One scheduling region: the 16 MFMAs of S_{j+1} interleaved with the
        // softmax of tile j.  (When j is the last tile the S_{j+1} result is unused;
        // the reads stay inside the LDS buffers.)
        s_tile((j + 1) & 1, sn);
        m_new = fmaxf(m_run, tile_max(sc));
        lsum = exp_tile(sc, m_new, false, key0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // 8 LDS reads (K operands)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // 6 VALU
          }
        }
      } else {
        // Visible keys of this lane's row: [myq - wl, myq + wr] and below N.
        const int lim = min(myq + wr, N - 1) - key0 - hoff, low = myq - wl - key0 - hoff;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * 32 + key0_of(i) > lim || kb * 32 + key0_of(i) < low) sc[kb][i] = -INFINITY;
        const float mt = tile_max(sc);
        m_new = (mt == -INFINITY) ? m_run : fmaxf(m_run, mt);
        lsum = exp_tile(sc, (m_new == -INFINITY) ? 0.f : m_new, true, key0);
        s_tile((j + 1) & 1, sn);
      }
      // Rescale the accumulator only when the max of some row of the wave grew.  The
      // max is tracked exactly so that the largest P~ of a row is exactly 1 and its
      // rounding to the 16-bit operand type costs nothing (it dominates peaked rows).
      if (__any(m_new > m_run)) {
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
      }
      m_run = m_new;
      l_run += lsum;
      // O^T += V_j^T P~^T: A operand = 8 consecutive keys of one head-dim row of V^T.
      const T* Vb = Vt[j & 1];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
          const frag pf = pack_frag<T>(sc[kb], u);
          const int kofs = kb * 32 + (kPerm ? 16 * u + 8 * h : 8 * (u >> 2) + 4 * h + (u & 3));
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const int d = db * 32 + col;
            acc[db] = M::mma(load_frag<T>(&Vb[d * C::VP + vt_index<T>(d, kofs)]), pf, acc[db]);
          }
        }
      sc[0] = sn[0];
      sc[1] = sn[1];
    }
    if (j + 2 < ntiles) sstore_k(j & 1);
    if (j + 1 < ntiles) sstore_v((j + 1) & 1);
    __syncthreads();
  }

  const float l = half_sum(l_run);
  if (myq < N) {
    // Dropout scales the kept weights by the inverse keep probability.
    const float inv = l > 0.f ? (DROP ? a.drop.scale : 1.f) / l : 0.f;
    T* orow = O + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        store4<T>(orow + db * 32 + 8 * r + 4 * h, acc[db][4 * r] * inv, acc[db][4 * r + 1] * inv,
                  acc[db][4 * r + 2] * inv, acc[db][4 * r + 3] * inv);
    if (h == 0) L[myq] = l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------------------ 16-bit types


// The forward for 16-bit types.  K and V tiles are copied from global memory
// straight into LDS (global_load_lds), four buffers deep, into row-major tiles
// whose rows are padded to D + 16 elements with the 8-byte slots of row r
// XOR-ed in their low two bits by (r >> 3) & 3.  S^T = K Q^T takes its A
// operand from K rows (two 8-byte reads, rows in the order row_pi) and Q from
// registers; O^T += V^T P~^T takes V^T through transposing LDS reads
// (ds_read_b64_tr_b16), which gather the 4 keys of each lane's P~ elements.
// Each tile is one fixed MFMA stream: S of the next tile with the softmax of
// this tile spread between its MFMAs, then P~ V of this tile; the accumulator
// is rescaled in between, only when the max of some row of the wave grew.
// 8 waves x 32 query rows per workgroup.
// Growth of a row max (log2 units) that fwd16_kernel absorbs without
// rescaling its accumulator: the exponentials are taken against a reference
// that may lag the true row max by up to this much, so P~ <= 2^8.  Softmax is
// unchanged by the choice of reference (it cancels between O and l).
constexpr float kMaxSlack = 8.f;

// NW = 8: one workgroup of 8 waves per CU, four K/V buffers, the K/V tiles
// copied three tiles ahead (waves 0-3 copy K, 4-7 V).  NW = 4: two workgroups
// of 4 waves per CU, two buffers, K copied two tiles and V one tile ahead by
// every wave; 128 query rows per workgroup balance causal work better.
template <int D, int NW_>
struct Fwd16 {
  static constexpr int NW = NW_;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;             // query rows per workgroup
  static constexpr int BC = 64;                  // keys per tile
  static constexpr int PB = TileLds<D>::PB;      // bytes per row (4-row multiples)
  static constexpr int TILE = BC * PB;
  static constexpr int BUF = 2 * TILE;           // K, V
  static constexpr int NB = NW == 8 ? 4 : 2;     // K/V buffers
  static constexpr int NKS = D / 16;
  static constexpr int NS = 2 * NKS;             // S MFMAs per tile (two 32-key blocks)
  static constexpr int NV = 4 * (D / 32);        // P~V MFMAs per tile
  static constexpr int NM = NS + NV;
  static constexpr int NLD = 2 * BC / NW / TileLds<D>::ROWS_PER_COPY;   // copies per wave per tile
  static constexpr int NA = NS / 2;              // slots of the row max
};

template <typename T, int D, bool CAUSAL, int NW, bool DROP>
__global__ __launch_bounds__(64 * NW, 2) void fwd16_kernel(FwdArgs a) {
  using C = Fwd16<D, NW>;
  static_assert((D == 64 || D == 128) && (NW == 4 || NW == 8), "fwd16_kernel: d = 64 or 128");
  // Row groups (one copy each) per wave and matrix: 16 rows of RPC each, STEP
  // bytes apart in LDS (see copy16_groups).
  constexpr int RPC = TileLds<D>::ROWS_PER_COPY, GPW = 16 / RPC, STEP = RPC * C::PB;
  constexpr int SHIFT = copy16_shift(GPW, STEP);
  using M = Mfma<T>;
  using frag = typename M::frag;
  __shared__ __attribute__((aligned(16))) char smem[C::NB * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntq = gridDim.x;
  int rank, hd;
  work_item<CAUSAL>(ntq, rank, hd);
  hd = packed_head(a, hd, a.H);
  const size_t head = (size_t)hd;
  const Span sp = span_of(a, hd);
  const int N = sp.n;
  // Causal: the last query tiles (most keys) first, counted in this sequence's tiles.
  const int ntq_own = (N + C::BR - 1) / C::BR;
  const int qt = CAUSAL ? ntq_own - 1 - rank : rank;
  if (qt < 0 || qt >= ntq_own) return;   // a tile past the end of a shorter sequence
  const int q0 = qt * C::BR;
  const T* Q = static_cast<const T*>(a.q) + sp.q * D;
  const T* K = static_cast<const T*>(a.k) + sp.kv * D;   // the head's K/V head
  const T* V = static_cast<const T*>(a.v) + sp.kv * D;
  T* O = static_cast<T*>(a.o) + sp.q * D;
  float* L = a.lse + head * a.N;

  const int qw = q0 + 32 * w;
  const int myq = qw + col;
  // A negative scale is folded into Q (exact sign flip) so that c > 0.
  const float c = fabsf(a.scale) * kLog2e;
  frag qf[C::NKS];
  {
    const T* qrow = Q + (size_t)min(myq, N - 1) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const frag f = load_frag<T>(qrow + ks * 16);
      qf[ks] = (a.scale < 0.f) ? neg_frag<T>(f) : f;
    }
  }
  // Visible keys of this lane's row: klo .. khi (window, causal and N).
  const int wr = CAUSAL ? min(a.wr, 0) : a.wr;
  const int khi = min(myq + wr, N - 1), klo = myq - a.wl;
  // Key tiles of the workgroup: [lo, hi), of which [ml, mu) need no mask.
  const TileRange tr = tile_range(q0, min(q0 + C::BR, N) - 1, N, a.wl, wr, C::BC, false);
  // The tiles to visit, in order: consecutive, or the active ones of the
  // workgroup's row of a block mask.
  BlockSkip sk = block_row(a, hd, q0 / kBlockQ, C::BC);
  TileQueue tq;
  tq.start(sk, tr.lo, tr.hi, lane);

  // Lane parts of the LDS addresses (bytes from the start of a buffer).
  const TileLds<D> lay(lane);
  // Copy of the GPW row groups of 16 rows starting at row r0 (a multiple of 16)
  // of K (mat 0) or V (mat 1) of key tile t into buffer b, in one block.  Rows
  // past N read as zero (and are masked through khi).  The resources start
  // SHIFT bytes before K and V.
  const i32x4 rsk = buffer_rsrc(reinterpret_cast<const char*>(K) - SHIFT, (uint32_t)N * (2 * D) + SHIFT);
  const i32x4 rsv = buffer_rsrc(reinterpret_cast<const char*>(V) - SHIFT, (uint32_t)N * (2 * D) + SHIFT);
  uint32_t voff[GPW];
#pragma unroll
  for (int g = 0; g < GPW; ++g) voff[g] = lay.c[((RPC * g) >> 3) & 1] + SHIFT - g * (STEP - 1024);
  auto copy_rows = [&](int b, int mat, int t, int r0) {
    copy16_groups<GPW, STEP>(mat ? rsv : rsk, voff, (uint32_t)(t * C::BC + r0) * (2 * D),
                             lds_address(smem) + b * C::BUF + mat * C::TILE + r0 * C::PB);
  };
  // S^T MFMA m of a tile (m < NS): key block kb = m & 1, k step ks = m >> 1.
  auto opS = [&](int kboff, int m) -> frag {
    const int off = kboff + (m & 1) * 32 * C::PB;
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(smem + lay.A(m >> 1) + off));
  };
  // P~V MFMA r of a tile (r < NV): key block kb, 16-key step u, head-dim block db.
  auto opV = [&](int vboff, int r) -> frag {
    const int kb = r / (2 * (D / 32)), u = (r / (D / 32)) & 1, db = r % (D / 32);
    s16x4 v[2];
#pragma unroll
    for (int rp = 0; rp < 2; ++rp) {
      const int off = vboff + C::TILE + (kb * 32 + 16 * u + 8 * rp) * C::PB;
      v[rp] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + lay.T(rp, db) + off));
    }
    return __builtin_bit_cast(frag, s16x8{v[0][0], v[0][1], v[0][2], v[0][3],
                                          v[1][0], v[1][1], v[1][2], v[1][3]});
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;   // running max of c S (log2 units)
  // This lane's share of the running normalizer: the sum of P~ as rounded to T
  // for the MFMA, so that the weights of O sum to 1 exactly as used.
  float l_run = 0.f;
  float nm_run = 0.f;            // -m_run, 0 while m_run is -inf
  float thr_run = -INFINITY;     // m_run + kMaxSlack

  // Prologue (queue tiles t0, t1, t2): NW = 8: t0, t1, t2 into buffers 0, 1, 2
  // (wave w copies the groups of rows 16 (w & 3) .. + 15 of K (w < 4) or V);
  // NW = 4: K and V of t0 into buffer 0 and K of t1 into buffer 1 (wave w
  // copies the groups of rows 16 w .. + 15 of each).  Then S of t0.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if constexpr (NW == 8) {
#pragma unroll
    for (int t = 0; t < 3; ++t) copy_rows(t, w >> 2, tq.t[t], 16 * (w & 3));
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(C::NLD));   // t2 may still be in flight
  } else {
    copy_rows(0, 0, tq.t[0], 16 * w);
    copy_rows(0, 1, tq.t[0], 16 * w);
    copy_rows(1, 0, tq.t[1], 16 * w);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  __syncthreads();
  // S of the current tile and of the next one; the two trade places every tile
  // (the loops run two tiles per trip), so no tile copies them.
  f32x16 sA[2], sB[2];
  sA[0] = f32x16{};
  sA[1] = f32x16{};
#pragma unroll
  for (int m = 0; m < C::NS; ++m) sA[m & 1] = M::mma(opS(0, m), qf[m >> 1], sA[m & 1]);

  constexpr int NS = C::NS, NV = C::NV, NM = C::NM, NA = C::NA;
  constexpr int PD = 4;
  // Slots of the softmax of the current tile (element e = 16 kb + i):
  // row max over slots [0, NA), the exchange between lane halves at NA, the
  // exponentials of key block 0 in (NA, NS) and of key block 1 in the first
  // half of the P~V MFMAs (before its P~ operands are needed).
  constexpr auto max_slot = [](int e) { return (e * NA) / 32; };
  constexpr auto exp_slot = [](int kb, int i) {
    return kb == 0 ? NA + 1 + (i * (NS - NA - 1)) / 16 : NS + (i * (NV / 2)) / 16;
  };
  // NW = 8: the wave's block of queue tile t3 as the P~V MFMAs start; NW = 4:
  // the step's blocks (K of t2, V of t1) early in the stream, since they must
  // land before its end.
  constexpr auto copy_slot = [](int k) { return NW == 8 ? NS : 1 + 2 * k; };

  int b0 = 0;   // buffer of tile t0 (NW = 8)
  // One step: S of queue tile t1 (into sn) with the softmax of t0 (S in sc),
  // then P~V of t0.  MASK: some row of the wave crosses an edge of the window,
  // the causal diagonal or N in t0.  NW = 4 buffers alternate by step.
  auto iteration = [&](const TileQueue& q, auto maskc, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    const int key0 = q.t[0] * C::BC;
    const int bk = NW == 8 ? (b0 + 1) & 3 : (q.s + 1) & 1, bc = (b0 + 3) & 3;
    const int kboff = bk * C::BUF, vboff = (NW == 8 ? b0 : q.s & 1) * C::BUF;
    frag pf[2][2];
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    float mx = -INFINITY, m_new;   // m_new: set and used only when grow
    bool grow = false;
    // Masked tiles: visible element offsets (key - key0 - h) of this lane's row.
    const int rlo = klo - key0 - h;
    const uint32_t rspan = (uint32_t)(khi - klo);   // khi >= klo for rows below N
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
    frag opq[PD];
    auto operand = [&](int m) -> frag { return m < NS ? opS(kboff, m) : opV(vboff, m - NS); };
#pragma unroll
    for (int m = 0; m < PD; m += 2) {
      opq[m + 1] = operand(m + 1);
      asm volatile("" ::: "memory");
      opq[m] = operand(m);
    }
    // One slot of the tile's stream: MFMA m (S of tile t1, or P~V of tile t0)
    // and the softmax / copy work placed on that slot.
    auto slot = [&](auto mc, auto maskc) {
      constexpr int m = decltype(mc)::value;
      constexpr bool MASK = decltype(maskc)::value;
      // Operands are read in pairs at odd slots, the odd one first, so that the
      // wait for the even one covers both.
      const frag x = opq[m % PD];
      if constexpr ((m & 1) && m + PD - 1 < NM) {
        opq[(m + PD) % PD] = operand(m + PD);
        asm volatile("" ::: "memory");   // keeps the two operands' reads apart
        opq[(m + PD - 1) % PD] = operand(m + PD - 1);
      }
      if constexpr (m < NS) {
        sn[m & 1] = M::mma(x, qf[m >> 1], sn[m & 1]);
      } else {
        constexpr int r = m - NS, kb = r / (2 * (D / 32)), u = (r / (D / 32)) & 1, db = r % (D / 32);
        acc[db] = M::mma(x, pf[kb][u], acc[db]);
      }
#pragma unroll
      for (int k = 0; k < (NW == 8 ? 1 : 2); ++k)
        if (m == copy_slot(k)) {
          if constexpr (NW == 8) copy_rows(bc, w >> 2, q.t[3], 16 * (w & 3));
          else if (k == 0) copy_rows(q.s & 1, 0, q.t[2], 16 * w);
          else copy_rows((q.s + 1) & 1, 1, q.t[1], 16 * w);
        }
#pragma unroll
      for (int e = 0; e < 32; ++e)
        if (m == max_slot(e)) {
          const int kb = e >> 4, i = e & 15;
          if constexpr (MASK) {
            // Visible iff rlo <= ke <= rhi, as one unsigned compare.
            const int ke = kb * 32 + 8 * (i / 4) + 2 * (i % 4);   // key - key0 - h
            if ((uint32_t)(ke - rlo) > rspan) sc[kb][i] = -INFINITY;
          }
          mx = fmaxf(mx, sc[kb][i]);
        }
      if constexpr (m == NA) {
        // The reference max of the exponentials moves only when the max of
        // some row of the wave grew by more than kMaxSlack (log2 units), so
        // P~ <= 2^kMaxSlack and most tiles skip the rescale.  The test runs
        // per lane, on its half of the row (c > 0: the same decision as on the
        // exchanged row max); the exchange and the new reference only when
        // some row grew.  Both rare branches are marked unlikely, so the
        // common path runs straight through (a taken branch costs the wave
        // its instruction fetch).
        grow = __builtin_amdgcn_ballot_w64(mx * c > thr_run) != 0;
        if (__builtin_expect(grow, 0)) {
          const float mh = half_max(mx);
          const float mt = (mh == -INFINITY) ? -INFINITY : mh * c;
          m_new = fmaxf(m_run, mt);
          nm_run = (m_new == -INFINITY) ? 0.f : -m_new;
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (m == exp_slot(kb, i)) {
            const float xs = sc[kb][i];
            float p = exp2_fast(fmaf(xs, c, nm_run));
            if constexpr (MASK) p = (xs == -INFINITY) ? 0.f : p;
            sc[kb][i] = p;
            if ((i + 1) % 8 == 0) {
              pf[kb][i / 8] = pack_frag<T>(sc[kb], i / 8);
              frag_sum4<T>(pf[kb][i / 8], ps);
              if constexpr (DROP) {
                // The 8 keys of this fragment, key0 + 32 kb + 16 (i / 8) + h + 2 t,
                // are exactly the keys of one generator call: the row sum above
                // took them all, the P~V operand keeps the kept ones.
                uint32_t wv[4], mk[4];
                drop_call(a.drop, hd, myq, (key0 + 32 * kb) / 16 + i / 8, h, wv);
                drop_masks(a.drop, wv, mk);
                i32x4 pv = __builtin_bit_cast(i32x4, pf[kb][i / 8]);
#pragma unroll
                for (int k = 0; k < 4; ++k) pv[k] &= (int)mk[k];
                pf[kb][i / 8] = __builtin_bit_cast(frag, pv);
              }
              // Pin the fragment (and the exponentials behind it) to this slot: the
              // results are only used after the rescale branch, and the compiler
              // would otherwise sink the whole computation past it.
              asm volatile("" : "+v"(pf[kb][i / 8]));
              asm volatile("" : "+v"(ps[0]), "+v"(ps[1]), "+v"(ps[2]), "+v"(ps[3]));
            }
          }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto rescale = [&]() {
      if (__builtin_expect(grow, 0)) {
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
        m_run = m_new;
        thr_run = m_new + kMaxSlack;
      }
    };
    // With two waves on a SIMD (8-wave workgroups), the wave in the S half of
    // its stream (S of the next tile, the softmax of this one) issues first;
    // the other wave's P~V MFMAs and exponentials fill in around it (measured
    // 1-2 % faster; the 4-wave causal workgroups gain nothing from it).
    if constexpr (NW == 8) __builtin_amdgcn_s_setprio(1);
    static_for<0, NS>([&](auto mc) { slot(mc, maskc); });
    if constexpr (NW == 8) __builtin_amdgcn_s_setprio(0);
    rescale();
    static_for<NS, NM>([&](auto mc) { slot(mc, maskc); });
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // NW = 8: t2 (copied during the previous step) must have landed, the copies
    // of t3 may still be in flight.  NW = 4: K of t2 and V of t1 must have landed.
    __builtin_amdgcn_s_waitcnt(NW == 8 ? wait_vmcnt(C::NLD) : kWaitVmcnt0);
    __syncthreads();
    b0 = (b0 + 1) & 3;
  };
  // Tiles [lo, ml) and [mu, hi) need masks in some row of the workgroup (the
  // window's edges, the causal diagonal, N); [ml, mu) none.  Each range runs in
  // a loop of its own, so that each loop body keeps its own register
  // allocation; after an odd tile the S registers are handed over by copy.
  // The queue skips the inactive tiles of a block mask.
  auto step = [&](auto maskc, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    iteration(tq, maskc, sc, sn);
    tq.advance(sk, tr.hi, lane);
  };
  while (tq.t[1] < tr.ml) {
    step(std::true_type{}, sA, sB);
    step(std::true_type{}, sB, sA);
  }
  if (tq.t[0] < tr.ml) {
    step(std::true_type{}, sA, sB);
    sA[0] = sB[0];
    sA[1] = sB[1];
  }
  while (tq.t[1] < tr.mu) {
    step(std::false_type{}, sA, sB);
    step(std::false_type{}, sB, sA);
  }
  if (tq.t[0] < tr.mu) {
    step(std::false_type{}, sA, sB);
    sA[0] = sB[0];
    sA[1] = sB[1];
  }
  while (tq.t[1] < tr.hi) {
    step(std::true_type{}, sA, sB);
    step(std::true_type{}, sB, sA);
  }
  if (tq.t[0] < tr.hi) step(std::true_type{}, sA, sB);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  const float l = half_sum(l_run);
  if (myq < N) {
    // Dropout scales the kept weights by the inverse keep probability.
    const float inv = l > 0.f ? (DROP ? a.drop.scale : 1.f) / l : 0.f;
    T* orow = O + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        store4<T>(orow + db * 32 + 8 * r + 4 * h, acc[db][4 * r] * inv, acc[db][4 * r + 1] * inv,
                  acc[db][4 * r + 2] * inv, acc[db][4 * r + 3] * inv);
    if (h == 0) L[myq] = l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  // Under the causal mask at d = 128, 128 query rows per workgroup (two per
  // CU) balance the triangle better; without it one 256-row workgroup per CU
  // copies half as much.
  const bool drop = a.drop.keep_t < 65536;
  [[maybe_unused]] constexpr Dt dt = std::is_same<T, __bf16>::value ? Dt::bf16 : Dt::f16;
  if constexpr (sizeof(T) == 2 && D == 128 && !CAUSAL) {
    // Without the causal mask and dropout, and with enough key tiles per
    // workgroup (measured: 2 % faster at N = 8192, 2 % slower at N = 1024):
    // 64 query rows per wave.
    if (!drop && a.N >= 2048) return launch_fwd64(dt, 128, false, a, s);
  }
  // 16-bit types otherwise (d = 128 causal or short, d = 64, dropout): 32 query
  // rows per wave, two waves per SIMD.  At d = 64 this measured 9-10 % faster
  // than 64 rows per wave (same-process A/B on b8h16n1024d64-f16 and
  // b1h16n16384d64-f16 causal), the other wave hiding the softmax, which at
  // d = 64 is twice the arithmetic per MFMA of d = 128.
  if constexpr (sizeof(T) == 2) {
    constexpr int NW = CAUSAL ? 4 : 8;
    using C = Fwd16<D, NW>;
    dim3 grid((a.N + C::BR - 1) / C::BR, a.H, a.B);
    if (drop)
      hipLaunchKernelGGL((fwd16_kernel<T, D, CAUSAL, NW, true>), grid, dim3(C::NT), 0, s, a);
    else
      hipLaunchKernelGGL((fwd16_kernel<T, D, CAUSAL, NW, false>), grid, dim3(C::NT), 0, s, a);
  } else {
    using C = FwdTile<T, D>;
    dim3 grid((a.N + C::BR - 1) / C::BR, a.H, a.B);
    if (drop && a.bm.mask)
      hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, true, true>), grid, dim3(C::NT), 0, s, a);
    else if (drop)
      hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, true, false>), grid, dim3(C::NT), 0, s, a);
    else if (a.bm.mask)
      hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, false, true>), grid, dim3(C::NT), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, false, false>), grid, dim3(C::NT), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_c(bool causal, const FwdArgs& a, hipStream_t s) {
  return causal ? launch_fwd_t<T, D, true>(a, s) : launch_fwd_t<T, D, false>(a, s);
}

template <typename T>
static hipError_t launch_fwd_d(int d, bool causal, const FwdArgs& a, hipStream_t s) {
  return d == 64 ? launch_fwd_c<T, 64>(causal, a, s) : launch_fwd_c<T, 128>(causal, a, s);
}

hipError_t launch_fwd(Dt dt, int d, bool causal, const FwdArgs& a, hipStream_t s) {
  switch (dt) {
    case Dt::f32: return launch_fwd_d<float>(d, causal, a, s);
    case Dt::f16: return launch_fwd_d<_Float16>(d, causal, a, s);
    case Dt::bf16: return launch_fwd_d<__bf16>(d, causal, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
