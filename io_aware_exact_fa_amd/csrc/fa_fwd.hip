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
  static constexpr int BR = 128;                 // query rows per workgroup
  static constexpr int BC = 64;                  // keys per tile
  static constexpr int NT = 256;                 // threads per workgroup
  static constexpr int KPL = Mfma<T>::KPL;
  static constexpr int KM = 2 * KPL;             // MFMA k depth
  static constexpr int NKS = D / KM;             // MFMAs per 32x32 block of S
  static constexpr int NU = steps32<T>();        // MFMAs per 32 keys of P V
  static constexpr int E16 = 16 / sizeof(T);     // elements per 16-byte chunk
  static constexpr int PITCH = D + E16;          // LDS row pitch (16 B pad)
  static constexpr int CPR = D / E16;            // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / NT;      // chunks per thread per tile
  static_assert(BC * CPR % NT == 0, "tile must split evenly over the threads");
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  using C = FwdTile<T, D>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  __shared__ __attribute__((aligned(16))) T Ks[C::BC * C::PITCH];
  __shared__ __attribute__((aligned(16))) T Vs[C::BC * C::PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, col = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int qt = CAUSAL ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const int q0 = qt * C::BR;
  const size_t head = (size_t)blockIdx.z * a.H + blockIdx.y;
  const T* Q = static_cast<const T*>(a.q) + head * N * D;
  const T* K = static_cast<const T*>(a.k) + head * N * D;
  const T* V = static_cast<const T*>(a.v) + head * N * D;
  T* O = static_cast<T*>(a.o) + head * N * D;
  float* L = a.lse + head * N;

  const int qw = q0 + 32 * w;   // first query row of this wave
  const int myq = qw + col;     // the query row of this lane

  // Q^T operand, held for the whole kernel.  A negative scale is folded into Q
  // (exact sign flip) so that c > 0 and max(c S) = c max(S).
  const float c = fabsf(a.scale) * kLog2e;
  frag qf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    frag f = {};
    if (myq < N) f = load_frag<T>(Q + (size_t)myq * D + ks * C::KM + C::KPL * h);
    qf[ks] = (a.scale < 0.f) ? neg_frag<T>(f) : f;
  }

  const int ntiles_all = (N + C::BC - 1) / C::BC;
  const int qlast = min(q0 + C::BR, N) - 1;
  const int ntiles = CAUSAL ? min(ntiles_all, qlast / C::BC + 1) : ntiles_all;
  // Last tile this wave needs; -1 if the wave holds no row below N.
  const int wlast = (qw >= N) ? -1 : (CAUSAL ? min(qw + 31, N - 1) / C::BC : ntiles - 1);

  uint4 kst[C::CPT], vst[C::CPT];
  auto gload = [&](int j) {
    const int key0 = j * C::BC;
#pragma unroll
    for (int r = 0; r < C::CPT; ++r) {
      const int ch = tid + r * C::NT, row = ch / C::CPR, cc = ch % C::CPR;
      if (key0 + row < N) {
        const size_t off = (size_t)(key0 + row) * D + cc * C::E16;
        kst[r] = *reinterpret_cast<const uint4*>(K + off);
        vst[r] = *reinterpret_cast<const uint4*>(V + off);
      } else {
        kst[r] = uint4{0, 0, 0, 0};   // keys past N: masked scores, zero values
        vst[r] = uint4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int r = 0; r < C::CPT; ++r) {
      const int ch = tid + r * C::NT, row = ch / C::CPR, cc = ch % C::CPR;
      *reinterpret_cast<uint4*>(&Ks[row * C::PITCH + cc * C::E16]) = kst[r];
      *reinterpret_cast<uint4*>(&Vs[row * C::PITCH + cc * C::E16]) = vst[r];
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;   // running max of c*S (log2 units)
  float l_run = 0.f;         // this lane's share of the running normalizer

  gload(0);
  sstore();
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    if (j + 1 < ntiles) gload(j + 1);
    if (j <= wlast) {
      const int key0 = j * C::BC;
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks)
          s[kb] = M::mma(load_frag<T>(&Ks[(kb * 32 + col) * C::PITCH + ks * C::KM + C::KPL * h]),
                         qf[ks], s[kb]);
      }
      const bool masked = (CAUSAL && key0 + C::BC - 1 > qw) || (key0 + C::BC > N);
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key >= N || (CAUSAL && key > myq)) s[kb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = half_max(mx);
      const float m_new = (mx == -INFINITY) ? m_run : fmaxf(m_run, mx * c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      float lsum = 0.f;
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x = s[kb][i];
            const float p = (x == -INFINITY) ? 0.f : exp2_fast(fmaf(x, c, -m_use));
            s[kb][i] = p;
            lsum += p;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = exp2_fast(fmaf(s[kb][i], c, -m_use));
            s[kb][i] = p;
            lsum += p;
          }
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      if (alpha != 1.f) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
      }
      frag pf[2][C::NU];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < C::NU; ++u) pf[kb][u] = pack_frag<T>(s[kb], u);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < C::NU; ++u)
            acc[db] = M::mma(load_frag_tr<T>(Vs, C::PITCH, kb * 32, u, db * 32, lane), pf[kb][u],
                             acc[db]);
    }
    __syncthreads();
    if (j + 1 < ntiles) sstore();
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
