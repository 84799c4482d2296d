// Forward attention kernel for gfx950.
//
// One workgroup of 4 wavefronts computes a tile of BR = 128 query rows of one
// (batch, head): each wave owns 32 rows (the queries are split across waves,
// so the softmax of a row never leaves its wave).  The workgroup loops over
// key/value tiles of BC = 64 keys, staged global -> registers -> LDS with the
// next tile's global loads in flight while the current tile is computed.
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

template <typename T, int D, bool CAUSAL>
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
  const int N = a.N;

  // Workgroup -> (head, query tile).  Workgroups are dealt to the 8 XCDs
  // round-robin by linear id; give each XCD a contiguous range of (head, tile)
  // pairs so the tiles of one head share their K/V through one L2.  Under the
  // causal mask the tiles of a head run heaviest (most key tiles) first.
  const int ntq = gridDim.x;
  const int nwork = ntq * gridDim.y * gridDim.z;
  int lin = blockIdx.x + ntq * (blockIdx.y + gridDim.y * blockIdx.z);
  if ((nwork & 7) == 0) lin = (lin & 7) * (nwork >> 3) + (lin >> 3);
  const int qt = CAUSAL ? ntq - 1 - (lin % ntq) : (lin % ntq);
  const int q0 = qt * C::BR;
  const size_t head = (size_t)(lin / ntq);
  const T* Q = static_cast<const T*>(a.q) + head * N * D;
  const T* K = static_cast<const T*>(a.k) + head * N * D;
  const T* V = static_cast<const T*>(a.v) + head * N * D;
  T* O = static_cast<T*>(a.o) + head * N * D;
  float* L = a.lse + head * N;

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

  const int ntiles_all = (N + C::BC - 1) / C::BC;
  const int qlast = min(q0 + C::BR, N) - 1;
  const int ntiles = CAUSAL ? min(ntiles_all, qlast / C::BC + 1) : ntiles_all;
  // Last tile this wave needs; -1 if the wave holds no row below N.
  const int wlast = (qw >= N) ? -1 : (CAUSAL ? min(qw + 31, N - 1) / C::BC : ntiles - 1);

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
  auto exp_tile = [&](f32x16 (&sc)[2], float m_use, bool masked) {
    const float nm = -m_use;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = sc[kb][i];
        float p = exp2_fast(fmaf(x, c, nm));
        if (masked) p = (x == -INFINITY) ? 0.f : p;   // exact also for c == 0
        sc[kb][i] = p;
        ps[i & 3] += p;
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
  gload_k(0);
  gload_v(0);
  sstore_k(0);
  sstore_v(0);
  if (ntiles > 1) {
    gload_k(1);
    sstore_k(1);
  }
  __syncthreads();
  f32x16 sc[2];
  if (wlast >= 0) s_tile(0, sc);
  // Iteration 0 overwrites K buffer 0 (read just above) with K_2.
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    if (j + 2 < ntiles) gload_k(j + 2);
    if (j + 1 < ntiles) gload_v(j + 1);
    if (j <= wlast) {
      const int key0 = j * C::BC;
      const bool masked = (CAUSAL && key0 + C::BC - 1 > qw) || (key0 + C::BC > N);
      f32x16 sn[2];
      float m_new, lsum;
      if (!masked) {
        // One scheduling region: the 16 MFMAs of S_{j+1} interleaved with the
        // softmax of tile j.  (When j is the last tile the S_{j+1} result is unused;
        // the reads stay inside the LDS buffers.)
        s_tile((j + 1) & 1, sn);
        m_new = fmaxf(m_run, tile_max(sc));
        lsum = exp_tile(sc, m_new, false);
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
        // Visible keys of this lane's row: key <= myq (causal) and key < N.
        const int lim = (CAUSAL ? min(myq, N - 1) : N - 1) - key0 - hoff;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * 32 + key0_of(i) > lim) sc[kb][i] = -INFINITY;
        const float mt = tile_max(sc);
        m_new = (mt == -INFINITY) ? m_run : fmaxf(m_run, mt);
        lsum = exp_tile(sc, (m_new == -INFINITY) ? 0.f : m_new, true);
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
    const float inv = l > 0.f ? 1.f / l : 0.f;
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
  using C = FwdTile<T, D>;
  dim3 grid((a.N + C::BR - 1) / C::BR, a.H, a.B);
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL>), grid, dim3(C::NT), 0, s, a);
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
