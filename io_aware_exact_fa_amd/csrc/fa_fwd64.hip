// Forward attention for 16-bit types: 64 query rows per wave, one wave per
// SIMD (d = 64 and 128).
//
// One workgroup of 4 waves computes 256 query rows of one (batch, head); wave
// w owns rows q0 + 64 w .. + 63 as two 32-row blocks A and B.  Per key tile of
// 64 keys each operand read from LDS feeds two MFMAs, one per block: a K row
// fragment the S^T = K Q^T products of A and B, a V^T fragment (transposing
// read) their O^T += V^T P~^T products.  That halves the LDS reads per MFMA of
// a 32-row wave, and with one wave per SIMD the instruction stream is this
// wave's alone.  The O^T accumulators of both blocks (4 D registers) live in
// AGPRs, the rest (S^T, read by the softmax) in VGPRs: the P~V MFMAs are
// issued as inline assembly with AGPR accumulators (mma_agpr below), the S^T
// MFMAs by the compiler in their VGPR form.
//
// The method per row is the one of fwd16_kernel (fa_fwd.hip): running max
// m with a reference that moves only when a row max of the wave grew by more
// than 2^8, P~ = 2^(c S - m), l summed from P~ as rounded for the P~V product,
// one division by l at the end, LSE = ln2 (m + log2 l) ("FlashAttention-2:
// Faster Attention with Better Parallelism and Work Partitioning", sections
// "결과: FlashAttention-2 Forward 알고리즘" and "개선 1"; per-row state and merge
// rule: "FlashAttention 원 논문 해부", section "두 tile을 한 row로 합치는 식";
// rows split across waves: the FlashAttention-2 page, "Work Partitioning Between
// Warps", split-Q).  Tiles are copied global -> LDS four buffers deep (the
// copies of tile t + 3 in two blocks, K and V, among tile t's first MFMAs,
// as soon as the barrier has freed their buffer; each block one M0 and
// scalar offset for all the wave's row groups), visited
// through the tile queue (window edges and N need masks; a block mask skips
// tiles).
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <int D_>
struct Fwd64 {
  static constexpr int D = D_;
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 64 * NW;             // query rows per workgroup
  static constexpr int BC = 64;                  // keys per tile
  static constexpr int PB = TileLds<D>::PB;
  static constexpr int TILE = BC * PB;
  static constexpr int BUF = 2 * TILE;           // K, V
  static constexpr int NB = 4;
  static constexpr int NKS = D / 16;             // k steps of one 32 x 32 block of S^T
  static constexpr int NDB = D / 32;             // head-dim blocks of O^T
  static constexpr int NS = 2 * 2 * NKS;         // S^T MFMAs per tile: 2 key blocks x 2 query blocks
  static constexpr int NV = 2 * 2 * NDB * 2;     // P~V MFMAs: key block x step x head-dim block x query block
  static constexpr int NM = NS + NV;
  static constexpr int RPC = TileLds<D>::ROWS_PER_COPY;
  static constexpr int NLD = 2 * BC / NW / RPC;  // copies per wave per tile
  static constexpr int NG = NLD / 2;             // row groups per wave per matrix
  static constexpr int STEP = RPC * PB;          // LDS bytes between row groups
  static constexpr int SHIFT = copy16_shift(NG, STEP);
  static constexpr int NA = NS / 2;              // slots of the row max
};

// Growth of a row max (log2 units) absorbed without rescaling (as fwd16_kernel).
constexpr float kMaxSlack64 = 8.f;

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd64_kernel(FwdArgs a) {
  using C = Fwd64<D>;
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
  const int ntq_own = (N + C::BR - 1) / C::BR;
  // Under the causal mask the last query tiles see the most keys and come first.
  const int qt = CAUSAL ? ntq_own - 1 - rank : rank;
  if (qt < 0 || qt >= ntq_own) return;   // a tile past the end of a shorter sequence
  const int q0 = qt * C::BR;
  const T* Q = static_cast<const T*>(a.q) + sp.q * D;
  const T* K = static_cast<const T*>(a.k) + sp.kv * D;
  const T* V = static_cast<const T*>(a.v) + sp.kv * D;
  T* O = static_cast<T*>(a.o) + sp.q * D;
  float* L = a.lse + head * a.N;

  const int qw = q0 + 64 * w;
  int myq[2];
  myq[0] = qw + col;
  myq[1] = qw + 32 + col;
  const float c = fabsf(a.scale) * kLog2e;
  // Q^T operands of both query blocks (a negative scale folded into Q).
  frag qf[2][C::NKS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const T* qrow = Q + (size_t)min(myq[qb], N - 1) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const frag f = load_frag<T>(qrow + ks * 16);
      qf[qb][ks] = (a.scale < 0.f) ? neg_frag<T>(f) : f;
    }
  }
  // Q stays in AGPRs (the S^T MFMAs read their B operand from there).
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) asm volatile("" : "+a"(qf[qb][ks]));
  const int wr = CAUSAL ? min(a.wr, 0) : a.wr;
  int khi[2], klo[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    khi[qb] = min(myq[qb] + wr, N - 1);
    klo[qb] = myq[qb] - a.wl;
  }
  const TileRange tr = tile_range(q0, min(q0 + C::BR, N) - 1, N, a.wl, wr, C::BC, false);
  BlockSkip sk = block_row(a, hd, q0 / kBlockQ, C::BC);
  TileQueue tq;
  tq.start(sk, tr.lo, tr.hi, lane);

  const TileLds<D> lay(lane);
  // The resources start SHIFT bytes before K and V (see copy16_groups).
  const i32x4 rsk = buffer_rsrc(reinterpret_cast<const char*>(K) - C::SHIFT, (uint32_t)N * (2 * D) + C::SHIFT);
  const i32x4 rsv = buffer_rsrc(reinterpret_cast<const char*>(V) - C::SHIFT, (uint32_t)N * (2 * D) + C::SHIFT);
  // Lane offsets of the wave's row groups g (rows 16 w + RPC g ..).
  uint32_t voff[C::NG];
#pragma unroll
  for (int g = 0; g < C::NG; ++g) voff[g] = lay.c[((C::RPC * g) >> 3) & 1] + C::SHIFT - g * (C::STEP - 1024);
  // Copy of matrix mat (0: K, 1: V) of key tile t into buffer b: the wave's
  // NG row groups, rows 16 w .. 16 w + 15.
  auto copy_op = [&](int b, int t, int mat) {
    copy16_groups<C::NG, C::STEP>(mat ? rsv : rsk, voff, (uint32_t)(t * C::BC + 16 * w) * (2 * D),
                                  lds_address(smem) + b * C::BUF + mat * C::TILE + 16 * w * C::PB);
  };
  // Operand of MFMA pair p (two MFMAs, query blocks A and B): p < NS / 2: K
  // fragment of k step p / 2, key block p % 2; else V^T fragment of pair
  // pr = p - NS / 2: key block pr / (2 NDB), 16-key step (pr / NDB) % 2,
  // head-dim block pr % NDB.
  auto opS = [&](int kboff, int p) -> frag {
    const int off = kboff + (p & 1) * 32 * C::PB;
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(smem + lay.A(p >> 1) + off));
  };
  auto opV = [&](int vboff, int pr) -> frag {
    const int kb = pr / (2 * C::NDB), u = (pr / C::NDB) & 1, db = pr % C::NDB;
    s16x4 v[2];
#pragma unroll
    for (int rp = 0; rp < 2; ++rp) {
      const int off = vboff + C::TILE + (kb * 32 + 16 * u + 8 * rp) * C::PB;
      v[rp] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + lay.T(rp, db) + off));
    }
    return __builtin_bit_cast(frag, s16x8{v[0][0], v[0][1], v[0][2], v[0][3],
                                          v[1][0], v[1][1], v[1][2], v[1][3]});
  };

  f32x16 acc[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[qb][db] = f32x16{};
  agpr_settle(acc);
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  float nm_run[2] = {0.f, 0.f};                  // -m_run, 0 while m_run is -inf
  float thr_run[2] = {-INFINITY, -INFINITY};     // m_run + slack

  // Prologue: queue tiles t0, t1, t2 into buffers 0, 1, 2; then S^T of t0.
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) copy_op(t, tq.t[t], mat);
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(C::NLD));   // t2 may still be in flight
  __syncthreads();
  // S^T of the current tile and of the next one, [query block][key block];
  // they trade places every tile (two tiles per loop trip).
  f32x16 sA[2][2], sB[2][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sA[qb][kb] = f32x16{};
#pragma unroll
  for (int p = 0; p < C::NS / 2; ++p) {
    const frag x = opS(0, p);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) sA[qb][p & 1] = M::mma(x, qf[qb][p >> 1], sA[qb][p & 1]);
  }

  constexpr int NS = C::NS, NM = C::NM, NA = C::NA;
  constexpr int PD = 3;   // operand pairs read ahead
  // Slots (MFMA indices) of the softmax of the current tile, element e =
  // 32 qb + 16 kb + i: row max over slots [0, NA), the exchange at NA, then
  // the exponentials of the four P~ fragments of each query block in the
  // order the P~V MFMAs use them, each group of 16 (one fragment of both
  // query blocks) spread evenly up to the slot before its first use:
  // fragment f = (kb, u) = 2 kb + u first feeds slot NS + 2 NDB f.
  constexpr int NF = 2 * C::NDB;                  // P~V slots per fragment
  constexpr auto max_slot = [](int e) { return (e * NA) / 64; };
  constexpr auto exp_slot = [](int qb, int kb, int i) {
    const int f = 2 * kb + i / 8;                 // fragment (kb, u), in order of use
    const int j = 8 * qb + (i % 8);               // 0..15 within the group
    const int first = NA + 1 + (f * (NM - NF - NA - 1)) / 4;   // groups overlap evenly
    const int last = NS + NF * f - 1;             // the slot before the first use
    return first + (j * (last - first)) / 16;
  };
  // Copies of K and of V of the tile three ahead, early in the tile so that
  // they have the most time to land (the barrier at the end of the previous
  // tile freed their buffer).
  constexpr auto copy_slot = [](int mat) { return 2 + 8 * mat; };

  int b0 = 0;   // buffer of tile t0
  auto iteration = [&](const TileQueue& q, auto maskc, f32x16 (&sc)[2][2], f32x16 (&sn)[2][2]) {
    const int key0 = q.t[0] * C::BC;
    const int kboff = ((b0 + 1) & 3) * C::BUF, vboff = b0 * C::BUF, bc = (b0 + 3) & 3;
    frag pf[2][2][2];   // [query block][key block][16-key step]
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sn[qb][kb] = f32x16{};
    float mx[2] = {-INFINITY, -INFINITY}, m_new[2];   // m_new: set and used only when grow
    bool grow = false;
    int rlo[2];
    uint32_t rspan[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      rlo[qb] = klo[qb] - key0 - h;
      rspan[qb] = (uint32_t)(khi[qb] - klo[qb]);
    }
    float ps[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    frag opq[PD];
    auto operand = [&](int p) -> frag { return p < NS / 2 ? opS(kboff, p) : opV(vboff, p - NS / 2); };
#pragma unroll
    for (int p = 0; p < PD; ++p) opq[p] = operand(p);
    auto slot = [&](auto mc, auto maskc2) {
      constexpr int m = decltype(mc)::value;
      constexpr bool MASK = decltype(maskc2)::value;
      constexpr int p = m >> 1, qb = m & 1;
      const frag x = opq[p % PD];
      if constexpr (qb == 1 && p + PD < NM / 2) opq[p % PD] = operand(p + PD);
      if constexpr (m < NS) {
        sn[qb][p & 1] = M::mma(x, qf[qb][p >> 1], sn[qb][p & 1]);
      } else {
        constexpr int pr = p - NS / 2, kb = pr / NF, u = (pr / C::NDB) & 1, db = pr % C::NDB;
        mma_agpr<T>(acc[qb][db], x, pf[qb][kb][u]);
      }
#pragma unroll
      for (int mat = 0; mat < 2; ++mat)
        if (m == copy_slot(mat)) copy_op(bc, q.t[3], mat);
#pragma unroll
      for (int e = 0; e < 64; ++e)
        if (m == max_slot(e)) {
          const int eq = e >> 5, kb = (e >> 4) & 1, i = e & 15;
          if constexpr (MASK) {
            const int ke = kb * 32 + 8 * (i / 4) + 2 * (i % 4);   // key - key0 - h
            if ((uint32_t)(ke - rlo[eq]) > rspan[eq]) sc[eq][kb][i] = -INFINITY;
          }
          mx[eq] = fmaxf(mx[eq], sc[eq][kb][i]);
        }
      // The growth test per lane (its half of the row against m + slack; c >
      // 0, so the same decision as on the exchanged row max); the exchange
      // and the new reference only when some row of the wave grew.  Both
      // rare branches are marked unlikely, so the common path runs straight
      // through (a taken branch costs this single wave per SIMD its fetch).
      if constexpr (m == NA) {
        grow = __builtin_amdgcn_ballot_w64((mx[0] * c > thr_run[0]) || (mx[1] * c > thr_run[1])) != 0;
        if (__builtin_expect(grow, 0)) {
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const float mh = half_max(mx[e2]);
            const float mt = (mh == -INFINITY) ? -INFINITY : mh * c;
            m_new[e2] = fmaxf(m_run[e2], mt);
            nm_run[e2] = (m_new[e2] == -INFINITY) ? 0.f : -m_new[e2];
          }
        }
      }
#pragma unroll
      for (int eq = 0; eq < 2; ++eq)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (m == exp_slot(eq, kb, i)) {
              const float xs = sc[eq][kb][i];
              float pv = exp2_fast(fmaf(xs, c, nm_run[eq]));
              if constexpr (MASK) pv = (xs == -INFINITY) ? 0.f : pv;
              sc[eq][kb][i] = pv;
              if ((i + 1) % 8 == 0) {
                pf[eq][kb][i / 8] = pack_frag<T>(sc[eq][kb], i / 8);
                frag_sum4<T>(pf[eq][kb][i / 8], ps[eq]);
                asm volatile("" : "+v"(pf[eq][kb][i / 8]));
                asm volatile("" : "+v"(ps[eq][0]), "+v"(ps[eq][1]), "+v"(ps[eq][2]), "+v"(ps[eq][3]));
              }
            }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto rescale = [&]() {
      if (__builtin_expect(grow, 0)) {
        agpr_settle(acc);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float alpha = (m_new[qb] == -INFINITY) ? 1.f : exp2_fast(m_run[qb] - m_new[qb]);
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) acc[qb][db] *= alpha;
          m_run[qb] = m_new[qb];
          thr_run[qb] = m_new[qb] + kMaxSlack64;
        }
        agpr_settle(acc);
      }
    };
    static_for<0, NS>([&](auto mc) { slot(mc, maskc); });
    rescale();
    static_for<NS, NM>([&](auto mc) { slot(mc, maskc); });
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) l_run[qb] += (ps[qb][0] + ps[qb][1]) + (ps[qb][2] + ps[qb][3]);
    // t2 (copied during the previous step) must have landed; t3 may be in flight.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(C::NLD));
    __syncthreads();
    b0 = (b0 + 1) & 3;
  };
  auto step = [&](auto maskc, f32x16 (&sc)[2][2], f32x16 (&sn)[2][2]) {
    iteration(tq, maskc, sc, sn);
    tq.advance(sk, tr.hi, lane);
  };
  auto hand_over = [&]() {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sA[qb][kb] = sB[qb][kb];
  };
  while (tq.t[1] < tr.ml) {
    step(std::true_type{}, sA, sB);
    step(std::true_type{}, sB, sA);
  }
  if (tq.t[0] < tr.ml) {
    step(std::true_type{}, sA, sB);
    hand_over();
  }
  while (tq.t[1] < tr.mu) {
    step(std::false_type{}, sA, sB);
    step(std::false_type{}, sB, sA);
  }
  if (tq.t[0] < tr.mu) {
    step(std::false_type{}, sA, sB);
    hand_over();
  }
  while (tq.t[1] < tr.hi) {
    step(std::true_type{}, sA, sB);
    step(std::true_type{}, sB, sA);
  }
  if (tq.t[0] < tr.hi) step(std::true_type{}, sA, sB);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  agpr_settle(acc);

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = half_sum(l_run[qb]);
    if (myq[qb] < N) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      T* orow = O + (size_t)myq[qb] * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store4<T>(orow + db * 32 + 8 * r + 4 * h, acc[qb][db][4 * r] * inv,
                    acc[qb][db][4 * r + 1] * inv, acc[qb][db][4 * r + 2] * inv,
                    acc[qb][db][4 * r + 3] * inv);
      if (h == 0) L[myq[qb]] = l > 0.f ? (m_run[qb] + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <typename T, int D>
static hipError_t launch_fwd64_t(bool causal, const FwdArgs& a, hipStream_t s) {
  using C = Fwd64<D>;
  dim3 grid((a.N + C::BR - 1) / C::BR, a.H, a.B);
  if (causal)
    hipLaunchKernelGGL((fwd64_kernel<T, D, true>), grid, dim3(C::NT), 0, s, a);
  else
    hipLaunchKernelGGL((fwd64_kernel<T, D, false>), grid, dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

// Instantiated at d = 128 only: at d = 64 the two-wave-per-SIMD fwd16_kernel
// is faster (the kernel itself is written for both).
template <typename T>
static hipError_t launch_fwd64_d(int d, bool causal, const FwdArgs& a, hipStream_t s) {
  if (d == 128) return launch_fwd64_t<T, 128>(causal, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd64(Dt dt, int d, bool causal, const FwdArgs& a, hipStream_t s) {
  if (dt == Dt::bf16) return launch_fwd64_d<__bf16>(d, causal, a, s);
  if (dt == Dt::f16) return launch_fwd64_d<_Float16>(d, causal, a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
