// Backward attention kernels for gfx950.
//
// Three launches on the caller's stream:
//   1. bwd_pre_kernel: D_i = rowsum(dO_i * O_i) in fp32, and zero the fp32 dQ
//      accumulator row (a fill kernel, not a memset, so the sequence can be
//      captured in a graph).  HBM-bound.
//   2. bwd_kernel: one workgroup of 4 wavefronts per (batch, head, tile of 128
//      keys); each wave owns 32 keys and keeps K, V of those keys and its dK,
//      dV accumulators in registers.  The workgroup loops over query tiles of
//      BQ rows (Q, dO, LSE, D staged in LDS) and per tile computes
//        S  = Q K^T,  P = 2^(c S - LSE log2 e)           (recomputed from LSE)
//        dP = dO V^T, dS = P * (dP - D)
//        dV += P^T dO,  dK += dS^T Q                    (registers)
//        dQacc += dS K                                  (fp32 atomics, via dS in LDS)
//      and stores dK * scale and dV once at the end.
//   3. bwd_dq_kernel: dq = scale * dQacc rounded to the input type.
//
// Sources: the gradients dV = P^T dO, dP = dO V^T, dS = P (dP - D),
// D_i = sum_j P_ij dP_ij, dQ = dS K, dK = dS^T Q ("FlashAttention-2: Faster
// Attention with Better Parallelism and Work Partitioning", section
// "Standard Attention Implementation / Backward Pass"; the factor scale on dQ
// and dK comes from S = scale Q K^T by the chain rule); D precomputed as
// rowsum(dO * O), P recomputed from the stored L, the key/value-tile-outer
// order and dQ accumulated across workgroups (same page, sections
// "Backward Pass" and "Parallelism: 시퀀스 길이 차원 병렬화"); S and P are never
// stored, only regenerated per tile ("FlashAttention 원 논문 해부", section
// "forward가 끝난 뒤 backward는 무엇을 저장하고 무엇을 다시 계산하는가").
//
// Register orientation: S and dP are computed as Q K^T and dO V^T, so each
// lane holds one key (column) and the query rows sit in the result registers.
// dV = P^T dO and dK = dS^T Q contract over queries, i.e. over the result rows,
// so P and dS feed those MFMAs from registers; dO and Q enter as transposed
// operands read from row-major LDS tiles with ds_read_b64_tr_b16.  dQ = dS K
// contracts over keys, so dS goes through LDS once (stored as dS^T, read back
// transposed).
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

// ------------------------------------------------------------------ preprocess

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, long rows) {
  constexpr int E16 = 16 / sizeof(T);
  constexpr int LPR = D / E16;          // lanes per row
  constexpr int RPB = 256 / LPR;        // rows per block
  const int sub = threadIdx.x % LPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  float part = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + sub * E16;
    const T* o = static_cast<const T*>(a.o) + off;
    const T* g = static_cast<const T*>(a.dout) + off;
#pragma unroll
    for (int e = 0; e < E16; ++e) part = fmaf(to_f32(o[e]), to_f32(g[e]), part);
    float* acc = a.dq_acc + off;
#pragma unroll
    for (int e = 0; e < E16; e += 4) *reinterpret_cast<f32x4*>(acc + e) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) part += __shfl_xor(part, m, LPR);
  if (row < rows && sub == 0) a.delta[row] = part;
}

// ------------------------------------------------------------------ main

template <typename T, int D>
struct BwdTile {
  static constexpr int BKC = 128;                          // keys per workgroup
  static constexpr int BQ = sizeof(T) == 4 ? 32 : 64;      // queries per tile
  static constexpr int NT = 256;
  static constexpr int KPL = Mfma<T>::KPL;
  static constexpr int KM = 2 * KPL;
  static constexpr int NKS = D / KM;
  static constexpr int NU = steps32<T>();
  static constexpr int E16 = 16 / sizeof(T);
  static constexpr int PITCH = D + E16;                    // Q, dO, K rows
  static constexpr int SPITCH = BQ + E16;                  // dS^T rows (keys)
  static constexpr int CPR = D / E16;
  static constexpr int NQB = BQ / 32;                      // 32-query blocks per tile
  static constexpr int NDQ = NQB * (D / 32);               // 32x32 dQ blocks per tile
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdArgs a) {
  using C = BwdTile<T, D>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  __shared__ __attribute__((aligned(16))) T Ks[C::BKC * C::PITCH];
  __shared__ __attribute__((aligned(16))) T Qs[C::BQ * C::PITCH];
  __shared__ __attribute__((aligned(16))) T dOs[C::BQ * C::PITCH];
  __shared__ __attribute__((aligned(16))) T dSt[C::BKC * C::SPITCH];
  __shared__ __attribute__((aligned(16))) float lse2s[C::BQ];
  __shared__ __attribute__((aligned(16))) float dls[C::BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, col = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int k0 = blockIdx.x * C::BKC;
  const size_t head = (size_t)blockIdx.z * a.H + blockIdx.y;
  const size_t hoff = head * N * D;
  const T* Q = static_cast<const T*>(a.q) + hoff;
  const T* K = static_cast<const T*>(a.k) + hoff;
  const T* V = static_cast<const T*>(a.v) + hoff;
  const T* dO = static_cast<const T*>(a.dout) + hoff;
  const float* LSE = a.lse + head * N;
  const float* Dl = a.delta + head * N;
  float* dQacc = a.dq_acc + hoff;
  const float c = a.scale * kLog2e;

  const int kw = k0 + 32 * w;   // first key of this wave
  const int myk = kw + col;     // the key of this lane (column of S)

  // K tile of the workgroup in LDS (read transposed by the dQ product).
  for (int ch = tid; ch < C::BKC * C::CPR; ch += C::NT) {
    const int row = ch / C::CPR, cc = ch % C::CPR;
    uint4 x = uint4{0, 0, 0, 0};
    if (k0 + row < N) x = *reinterpret_cast<const uint4*>(K + (size_t)(k0 + row) * D + cc * C::E16);
    *reinterpret_cast<uint4*>(&Ks[row * C::PITCH + cc * C::E16]) = x;
  }
  // K and V operands of this lane's key, held for the whole kernel.
  frag kf[C::NKS], vf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    kf[ks] = frag{};
    vf[ks] = frag{};
    if (myk < N) {
      kf[ks] = load_frag<T>(K + (size_t)myk * D + ks * C::KM + C::KPL * h);
      vf[ks] = load_frag<T>(V + (size_t)myk * D + ks * C::KM + C::KPL * h);
    }
  }
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dv[db] = f32x16{};
    dk[db] = f32x16{};
  }

  const int nqt = (N + C::BQ - 1) / C::BQ;
  const int qt0 = CAUSAL ? k0 / C::BQ : 0;   // earlier query tiles see none of these keys
  for (int qt = qt0; qt < nqt; ++qt) {
    const int qi0 = qt * C::BQ;
    __syncthreads();   // previous tile's LDS reads are done
    for (int ch = tid; ch < C::BQ * C::CPR; ch += C::NT) {
      const int row = ch / C::CPR, cc = ch % C::CPR;
      uint4 xq = uint4{0, 0, 0, 0}, xo = uint4{0, 0, 0, 0};
      if (qi0 + row < N) {
        const size_t off = (size_t)(qi0 + row) * D + cc * C::E16;
        xq = *reinterpret_cast<const uint4*>(Q + off);
        xo = *reinterpret_cast<const uint4*>(dO + off);
      }
      *reinterpret_cast<uint4*>(&Qs[row * C::PITCH + cc * C::E16]) = xq;
      *reinterpret_cast<uint4*>(&dOs[row * C::PITCH + cc * C::E16]) = xo;
    }
    for (int r = tid; r < C::BQ; r += C::NT) {
      const int qq = qi0 + r;
      float l2 = INFINITY, dd = 0.f;   // rows past N (or with no visible key) get P = 0
      if (qq < N) {
        const float lse = LSE[qq];
        if (lse != -INFINITY) l2 = lse * kLog2e;
        dd = Dl[qq];
      }
      lse2s[r] = l2;
      dls[r] = dd;
    }
    __syncthreads();

    const bool idle = CAUSAL && (qi0 + C::BQ - 1 < kw);   // every query of the tile precedes every key
    if (idle) {
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store4<T>(&dSt[(32 * w + col) * C::SPITCH + qb * 32 + 8 * r + 4 * h], 0.f, 0.f, 0.f, 0.f);
    } else {
      f32x16 p[C::NQB], ds[C::NQB];
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          const int off = (qb * 32 + col) * C::PITCH + ks * C::KM + C::KPL * h;
          s = M::mma(load_frag<T>(&Qs[off]), kf[ks], s);
          dp = M::mma(load_frag<T>(&dOs[off]), vf[ks], dp);
        }
        const bool mask = (myk >= N) || (CAUSAL && qi0 + qb * 32 < kw + 31);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[qb * 32 + 8 * r + 4 * h]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dls[qb * 32 + 8 * r + 4 * h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * r + e;
            float pv = exp2_fast(fmaf(s[i], c, -l4[e]));
            if (mask) {
              const int qq = qi0 + qb * 32 + 8 * r + 4 * h + e;
              if (myk >= N || (CAUSAL && qq < myk)) pv = 0.f;
            }
            p[qb][i] = pv;
            ds[qb][i] = pv * (dp[i] - d4[e]);
          }
        }
      }
      // dV += P^T dO and dK += dS^T Q  (contraction over the tile's queries)
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
          const frag pa = pack_frag<T>(p[qb], u);
          const frag sa = pack_frag<T>(ds[qb], u);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            dv[db] = M::mma(pa, load_frag_tr<T>(dOs, C::PITCH, qb * 32, u, db * 32, lane), dv[db]);
            dk[db] = M::mma(sa, load_frag_tr<T>(Qs, C::PITCH, qb * 32, u, db * 32, lane), dk[db]);
          }
        }
      // dS^T (keys x queries) to LDS for the dQ product.
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store4<T>(&dSt[(32 * w + col) * C::SPITCH + qb * 32 + 8 * r + 4 * h], ds[qb][4 * r],
                    ds[qb][4 * r + 1], ds[qb][4 * r + 2], ds[qb][4 * r + 3]);
    }
    __syncthreads();

    // dQacc[tile] += dS K over the workgroup's 128 keys; 32x32 blocks split over waves.
    for (int bi = w; bi < C::NDQ; bi += 4) {
      const int qb = bi / (D / 32), db = bi % (D / 32);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kb = 0; kb < C::BKC / 32; ++kb)
#pragma unroll
        for (int u = 0; u < C::NU; ++u)
          acc = M::mma(load_frag_tr<T>(dSt, C::SPITCH, kb * 32, u, qb * 32, lane),
                       load_frag_tr<T>(Ks, C::PITCH, kb * 32, u, db * 32, lane), acc);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qq = qi0 + qb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (qq < N) unsafeAtomicAdd(&dQacc[(size_t)qq * D + db * 32 + col], acc[i]);
      }
    }
  }

  // Epilogue: dK = scale * dS^T Q, dV; lane (col = d, h) holds keys 8(i/4) + 4h + i%4.
  T* dK = static_cast<T*>(a.dk) + hoff;
  T* dV = static_cast<T*>(a.dv) + hoff;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw + 8 * (i >> 2) + 4 * h + (i & 3);
      if (key < N) {
        const size_t off = (size_t)key * D + db * 32 + col;
        dK[off] = (T)(dk[db][i] * a.scale);
        dV[off] = (T)dv[db][i];
      }
    }
}

// ------------------------------------------------------------------ dQ finalize

template <typename T>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a, long n4) {
  const float* acc = a.dq_acc;
  T* dq = static_cast<T*>(a.dq);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(acc + 4 * i);
    store4<T>(dq + 4 * i, x[0] * a.scale, x[1] * a.scale, x[2] * a.scale, x[3] * a.scale);
  }
}

// ------------------------------------------------------------------ launchers

enum class Step { pre, main, fin };

template <typename T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(Step step, const BwdArgs& a, hipStream_t s) {
  using C = BwdTile<T, D>;
  const long rows = (long)a.B * a.H * a.N;
  if (step == Step::pre) {
    constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
    const long blocks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a, rows);
  } else if (step == Step::main) {
    dim3 grid((a.N + C::BKC - 1) / C::BKC, a.H, a.B);
    hipLaunchKernelGGL((bwd_kernel<T, D, CAUSAL>), grid, dim3(C::NT), 0, s, a);
  } else {
    const long n4 = rows * D / 4;
    const long blocks = n4 / 256 < 8192 ? (n4 + 255) / 256 : 8192;
    hipLaunchKernelGGL((bwd_dq_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, s, a, n4);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_bwd_c(Step st, bool causal, const BwdArgs& a, hipStream_t s) {
  return causal ? launch_bwd_t<T, D, true>(st, a, s) : launch_bwd_t<T, D, false>(st, a, s);
}

template <typename T>
static hipError_t launch_bwd_d(Step st, int d, bool causal, const BwdArgs& a, hipStream_t s) {
  return d == 64 ? launch_bwd_c<T, 64>(st, causal, a, s) : launch_bwd_c<T, 128>(st, causal, a, s);
}

static hipError_t launch_step(Step st, Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s) {
  switch (dt) {
    case Dt::f32: return launch_bwd_d<float>(st, d, causal, a, s);
    case Dt::f16: return launch_bwd_d<_Float16>(st, d, causal, a, s);
    case Dt::bf16: return launch_bwd_d<__bf16>(st, d, causal, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_pre(Dt dt, int d, const BwdArgs& a, hipStream_t s) {
  return launch_step(Step::pre, dt, d, false, a, s);
}

hipError_t launch_bwd_main(Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s) {
  return launch_step(Step::main, dt, d, causal, a, s);
}

hipError_t launch_bwd_fin(Dt dt, int d, const BwdArgs& a, hipStream_t s) {
  return launch_step(Step::fin, dt, d, false, a, s);
}

}  // namespace fa
