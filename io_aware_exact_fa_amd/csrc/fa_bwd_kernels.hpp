// Backward attention kernels for gfx950.
//
// Three launches on the caller's stream, no atomics and no fp32 accumulator
// in device memory:
//   1. bwd_pre_kernel: D_i = rowsum(dO_i * O_i) and L2_i = LSE_i log2(e) in
//      fp32, padded per head to whole 64-row tiles (HBM-bound).
//   2. dK, dV (bwd_dkdv16_kernel for 16-bit types, bwd_dkdv_kernel for fp32):
//      one workgroup per (batch, head, 128-key tile); each wave owns 32 keys.
//      For every query tile, recompute
//        S = Q K^T, P = 2^(c S - L2), dP = dO V^T, dS = P (dP - D)
//      and accumulate dV += P^T dO, dK += dS^T Q in registers; dk = scale dK.
//   3. dQ (bwd_dq16_kernel / bwd_dq_kernel): one workgroup per (batch, head,
//      query tile), the forward's loop order: for every key tile, recompute
//      S^T, P, dP^T, dS and accumulate dQ^T += K^T dS^T in registers;
//      dq = scale dQ at the end.
// dQ is computed by its own pass instead of being summed across key-tile
// workgroups: the two GEMMs it recomputes cost less than the fp32 atomic
// traffic they replace, and every output is written exactly once (bitwise
// repeatable).
//
// Sources: the gradients dV = P^T dO, dP = dO V^T, dS = P (dP - D),
// D_i = sum_j P_ij dP_ij, dQ = dS K, dK = dS^T Q ("FlashAttention-2: Faster
// Attention with Better Parallelism and Work Partitioning", section
// "Standard Attention Implementation / Backward Pass"; the factor scale on dQ
// and dK comes from S = scale Q K^T by the chain rule); D precomputed as
// rowsum(dO * O), P recomputed from the stored L, the key/value-tile-outer
// order for dK/dV and a separate reduction for dQ (same page, sections
// "Backward Pass" and "Parallelism: 시퀀스 길이 차원 병렬화"); S and P are never
// stored, only regenerated per tile ("FlashAttention 원 논문 해부", section
// "forward가 끝난 뒤 backward는 무엇을 저장하고 무엇을 다시 계산하는가").
//
// Operands: every MFMA reads one operand from registers (a result tile of an
// earlier MFMA, or rows held for the whole kernel) and the other from LDS.
// The 16-bit kernels keep each tile in LDS once, row-major and swizzled, copied
// there straight from global memory, and read it two ways (8-byte reads of
// rows, transposing reads of columns); the fp32 kernels stage tiles through
// registers into a row-major and a transposed copy read with 16-byte reads.
#pragma once

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
  // Workspace row (head, q) with q < Np; rows q >= N are padding.
  const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  const long head = row / a.Np;
  const int q = (int)(row - head * a.Np);
  const Span sp = row < rows ? span_of(a, (int)head) : Span{0, 0, 0, 0};
  const bool live = q < sp.n;
  float part = 0.f;
  if (live) {
    const size_t off = (sp.q + q) * D + sub * E16;
    const T* o = static_cast<const T*>(a.o) + off;
    const T* g = static_cast<const T*>(a.dout) + off;
#pragma unroll
    for (int e = 0; e < E16; ++e) part = fmaf(to_f32(o[e]), to_f32(g[e]), part);
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) part += __shfl_xor(part, m, LPR);
  if (a.dqacc && row < rows) {
    // One-pass backward: this lane's E16 floats of the row's dQ accumulator start at 0.
    f32x4* z = reinterpret_cast<f32x4*>(a.dqacc + (size_t)row * D + sub * E16);
#pragma unroll
    for (int e = 0; e < E16 / 4; ++e) z[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (row < rows && sub == 0) {
    float l2 = INFINITY;   // P = exp2(-inf) = 0 on padding rows and rows that see no key
    if (live) {
      const float lse = a.lse[(size_t)head * a.N + q];
      if (lse != -INFINITY) l2 = lse * kLog2e;
    }
    a.delta[row] = part;
    a.l2[row] = l2;
  }
}


// dq = -scale * (accumulated -dS K) of the one-pass backward, rounded to T;
// one thread per 8 consecutive elements of a row (rows of every head; rows
// past a sequence's length are not written).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dqfin_kernel(BwdArgs a, long rows) {
  constexpr int TPR = D / 8;   // threads per row
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t / TPR;
  if (row >= rows) return;
  const int sub = (int)(t - row * TPR);
  const long head = row / a.Np;
  const int q = (int)(row - head * a.Np);
  const Span sp = span_of(a, (int)head);
  if (q >= sp.n) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(a.dqacc + (size_t)row * D + sub * 8);
  const f32x4 x0 = src[0], x1 = src[1];
  const float f = -a.scale;   // the accumulator holds -dS K (see the one-pass kernel)
  T* dst = static_cast<T*>(a.dq) + (sp.q + q) * D + sub * 8;
  store4<T>(dst, x0[0] * f, x0[1] * f, x0[2] * f, x0[3] * f);
  store4<T>(dst + 4, x1[0] * f, x1[1] * f, x1[2] * f, x1[3] * f);
}

// ------------------------------------------------------------------ dQ

template <typename T, int D>
struct DqTile {
  // 16-bit types: 8 waves x 32 queries, so each K/V tile streamed from L2 serves
  // 256 query rows; f32 keeps 4 waves (1 wave per SIMD for registers).
  static constexpr int NW = sizeof(T) == 2 ? 8 : 4;
  static constexpr int NT = 64 * NW;
  static constexpr int WAVES_PER_SIMD = sizeof(T) == 2 ? 2 : 1;
  static constexpr int BR = 32 * NW;             // queries per workgroup
  static constexpr int BC = kTrCols;             // keys per tile (64)
  static constexpr int KPL = Mfma<T>::KPL;
  static constexpr int KM = 2 * KPL;
  static constexpr int NKS = D / KM;
  static constexpr int NU = steps32<T>();
  static constexpr int E16 = 16 / sizeof(T);
  static constexpr int KP = D + E16;             // row pitch of the K and V tiles
};

template <typename T, int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__((DqTile<T, D>::NT), (DqTile<T, D>::WAVES_PER_SIMD))
void bwd_dq_kernel(BwdArgs a) {
  using C = DqTile<T, D>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr bool kPerm = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) T Ks[C::BC * C::KP];
  __shared__ __attribute__((aligned(16))) T Vs[C::BC * C::KP];
  __shared__ __attribute__((aligned(16))) T Kt[D * kTrPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, col = lane & 31, h = lane >> 5;
  const int ntq = gridDim.x;
  const int lin = xcd_work_index();
  const size_t head = (size_t)packed_head(a, lin / ntq, a.H);
  const Span sp = span_of(a, (int)head);
  const int N = sp.n;
  const int ntq_own = (N + C::BR - 1) / C::BR;
  const int qt = CAUSAL ? ntq_own - 1 - (lin % ntq) : (lin % ntq);
  if (qt < 0 || qt >= ntq_own) return;   // a tile past the end of a shorter sequence
  const int q0 = qt * C::BR;
  const T* Q = static_cast<const T*>(a.q) + sp.q * D;
  const T* K = static_cast<const T*>(a.k) + sp.kv * D;   // the head's K/V head
  const T* V = static_cast<const T*>(a.v) + sp.kv * D;
  const T* dO = static_cast<const T*>(a.dout) + sp.q * D;
  T* dQ = static_cast<T*>(a.dq) + sp.q * D;
  const float c = a.scale * kLog2e;

  const int qw = q0 + 32 * w;
  const int myq = qw + col;
  const int qrow = min(myq, N - 1);
  // Q^T and dO^T operands of this lane's query, held for the whole kernel.
  frag qf[C::NKS], gf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    qf[ks] = load_frag<T>(Q + (size_t)qrow * D + ks * C::KM + C::KPL * h);
    gf[ks] = load_frag<T>(dO + (size_t)qrow * D + ks * C::KM + C::KPL * h);
  }
  // Row statistics of this lane's query.  A row with no visible key (LSE = -inf)
  // has P = 0: use +inf as its log2-domain LSE.
  const float lse = a.lse[head * a.N + qrow];
  const float l2 = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
  const float dl = a.delta[head * a.Np + qrow];

  // Window: keys [myq - wl, myq + wr] of this lane's row are visible.
  const int wl = a.wl, wr = CAUSAL ? min(a.wr, 0) : a.wr;
  const TileRange tr = tile_range(q0, min(q0 + C::BR, N) - 1, N, wl, wr, C::BC, false);
  const int j0 = tr.lo, ntiles = tr.hi;
  // Tiles this wave needs: [wfirst, wlast] (none if it holds no row below N).
  const int wfirst = max(0, qw - wl) / C::BC;
  const int wlast = (qw >= N) ? -1 : min(qw + 31 + wr, N - 1) / C::BC;
  const int krow = kPerm ? perm16(col) : col;
  const int hoff = kPerm ? 8 * h : 4 * h;
  auto key0_of = [](int i) {
    const int r = 8 * (i >> 2) + (i & 3);
    return kPerm ? perm16(r) : r;
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  TileStage<T, D, C::NT> ks_stage, vs_stage;
  ks_stage.load(K, j0 * C::BC, N, tid);
  vs_stage.load(V, j0 * C::BC, N, tid);
  for (int j = j0; j < ntiles; ++j) {
    ks_stage.store_rows(Ks, C::KP, tid);
    ks_stage.store_transposed(Kt, tid);
    vs_stage.store_rows(Vs, C::KP, tid);
    __syncthreads();
    if (j + 1 < ntiles) {
      ks_stage.load(K, (j + 1) * C::BC, N, tid);
      vs_stage.load(V, (j + 1) * C::BC, N, tid);
    }
    if (j >= wfirst && j <= wlast && block_on(a, (int)head, q0, j * C::BC)) {
      const int key0 = j * C::BC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T and dP^T for 32 keys x 32 queries.
        f32x16 s = f32x16{}, dp = f32x16{};
        const T* kr = &Ks[(kb * 32 + krow) * C::KP + C::KPL * h];
        const T* vr = &Vs[(kb * 32 + krow) * C::KP + C::KPL * h];
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          s = M::mma(load_frag<T>(kr + ks * C::KM), qf[ks], s);
          dp = M::mma(load_frag<T>(vr + ks * C::KM), gf[ks], dp);
        }
        const int kb0 = key0 + kb * 32;
        const bool masked = (kb0 + 31 > qw + wr) || (kb0 < qw + 31 - wl) || (kb0 + 32 > N);
        const int lim = min(myq + wr, N - 1) - kb0 - hoff, low = myq - wl - kb0 - hoff;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = exp2_fast(fmaf(s[i], c, -l2));
          if (masked && (key0_of(i) > lim || key0_of(i) < low)) p = 0.f;
          float dpi = dp[i];
          if constexpr (DROP)   // dP through the kept entries and their scale
            dpi = drop_keep(a.drop, (int)head, myq, kb0 + key0_of(i) + hoff) ? dpi * a.drop.scale : 0.f;
          s[i] = p * (dpi - dl);                       // dS
        }
        // dQ^T += K^T dS^T: A operand = 8 consecutive keys of one head-dim row of K^T.
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
          const frag sf = pack_frag<T>(s, u);
          const int kofs = kb * 32 + (kPerm ? 16 * u + 8 * h : 8 * (u >> 2) + 4 * h + (u & 3));
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            acc[db] = M::mma(load_frag<T>(&Kt[tr_index<T>(db * 32 + col, kofs)]), sf, acc[db]);
        }
      }
    }
    __syncthreads();
  }

  if (myq < N) {
    T* orow = dQ + (size_t)myq * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        store4<T>(orow + db * 32 + 8 * r + 4 * h, acc[db][4 * r] * sc, acc[db][4 * r + 1] * sc,
                  acc[db][4 * r + 2] * sc, acc[db][4 * r + 3] * sc);
  }
}

// ------------------------------------------------------------------ dK, dV

template <typename T, int D>
struct DkvTile {
  static constexpr int BKC = 128;                // keys per workgroup (32 per wave)
  static constexpr int BQ = kTrCols;             // queries per tile (64)
  static constexpr int KPL = Mfma<T>::KPL;
  static constexpr int KM = 2 * KPL;
  static constexpr int NKS = D / KM;
  static constexpr int NU = steps32<T>();
  static constexpr int E16 = 16 / sizeof(T);
  static constexpr int QP = D + E16;             // row pitch of the Q and dO tiles
  // Two LDS buffers (one barrier per query tile) when they fit beside each other.
  static constexpr int BUF_BYTES = (2 * BQ * QP + 2 * D * kTrPitch) * (int)sizeof(T) + 2 * BQ * 4;
  static constexpr int NBUF = 2 * BUF_BYTES <= 160 * 1024 ? 2 : 1;
};

template <typename T, int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using C = DkvTile<T, D>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr bool kPerm = sizeof(T) == 2;
  // Double-buffered query tiles: row-major Q and dO (A operands of S and dP),
  // transposed Q^T and dO^T (B operands of dK and dV), LSE and D.
  __shared__ __attribute__((aligned(16))) T Qs[C::NBUF][C::BQ * C::QP];
  __shared__ __attribute__((aligned(16))) T Gs[C::NBUF][C::BQ * C::QP];      // dO
  __shared__ __attribute__((aligned(16))) T Qt[C::NBUF][D * kTrPitch];
  __shared__ __attribute__((aligned(16))) T Gt[C::NBUF][D * kTrPitch];
  __shared__ __attribute__((aligned(16))) float lse2s[C::NBUF][C::BQ];
  __shared__ __attribute__((aligned(16))) float dls[C::NBUF][C::BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, col = lane & 31, h = lane >> 5;
  const int ntk = gridDim.x;
  int kt, hd;
  // Under the causal mask the key tiles near the start see the most queries and
  // come first.
  work_item<CAUSAL>(ntk, kt, hd);
  hd = packed_head(a, hd, a.H / a.G);
  const int k0 = kt * C::BKC;
  // hd is a K/V head; its query heads hd G .. hd G + G - 1 run one after another.
  const size_t kvhead = (size_t)hd;
  const Span sp = span_of(a, hd * a.G);
  const int N = sp.n;
  if (k0 >= N) return;   // a tile past the end of a shorter sequence
  const T* K = static_cast<const T*>(a.k) + sp.kv * D;
  const T* V = static_cast<const T*>(a.v) + sp.kv * D;
  const T *Q = nullptr, *dO = nullptr;
  const float *LSE = nullptr, *Dl = nullptr;
  int qhead = 0;   // query head of the current pass (dropout's generator counter)
  const float c = a.scale * kLog2e;

  const int kw = k0 + 32 * w;    // first key of this wave
  const int myk = kw + col;      // this lane's key (column of S)
  const int kg = min(myk, N - 1);
  // K and V operands (B of S = Q K^T and of dP = dO V^T) of this lane's key.
  frag kf[C::NKS], vf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    kf[ks] = load_frag<T>(K + (size_t)kg * D + ks * C::KM + C::KPL * h);
    vf[ks] = load_frag<T>(V + (size_t)kg * D + ks * C::KM + C::KPL * h);
  }
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dv[db] = f32x16{};
    dk[db] = f32x16{};
  }
  // Query (inside a 32-query block) of result element i of this lane:
  // qoff_of(i) + hoff (rows of the Q and dO operands are permuted for 16-bit types).
  const int qrow = kPerm ? perm16(col) : col;
  const int hoff = kPerm ? 8 * h : 4 * h;
  auto qoff_of = [](int i) {
    const int r = 8 * (i >> 2) + (i & 3);
    return kPerm ? perm16(r) : r;
  };

  // Window: queries [myk - wr, myk + wl] see this lane's key.  Query tiles of
  // the workgroup: [qt0, nqt) (qt0 < nqt because k0 < N).
  const int wl = a.wl, wr = CAUSAL ? min(a.wr, 0) : a.wr;
  const TileRange tr = tile_range(k0, k0 + C::BKC - 1, N, wr, wl, C::BQ, true);
  const int qt0 = tr.lo, nqt = tr.hi;
  // Staging of a query tile (Q and dO, 64 rows each) through registers, as
  // 2 NGM units of 4 rows x 16 bytes: thread tid owns units tid + 256 u, which
  // belong to Q (mat 0) or dO (mat 1).  The work is split into single
  // operations (st_op / ld_op) with no branches, so that the tile loop can
  // place them between its MFMAs; addresses are clamped to row N - 1, so a
  // tile past the end is loaded (and stored) harmlessly.
  constexpr int E16 = 16 / (int)sizeof(T), CPR = D / E16, NGM = (C::BQ / 4) * CPR;
  constexpr int UPT = 2 * NGM / 256;
  static_assert(2 * NGM % 256 == 0, "units must divide among the threads");
  uint4 stx[UPT][4];
  float lse_st, d_st;   // LSE and D of query row (tile start + lane) of the staged tile
  auto unit = [&](int u, int& mat, int& dg, int& rg) {
    const int gu = tid + 256 * u;
    mat = gu / NGM;
    dg = (gu % NGM) % CPR;
    rg = (gu % NGM) / CPR;
  };
  // Loads: 4 per unit (one row each), then LSE and D.
  constexpr int NLD = 4 * UPT + 1;
  auto ld_op = [&](int qt, int j) {
    if (j < 4 * UPT) {
      const int u = j / 4, i = j % 4;
      int mat, dg, rg;
      unit(u, mat, dg, rg);
      const int row = min(qt * C::BQ + 4 * rg + i, N - 1);
      const T* src = mat ? dO : Q;
      stx[u][i] = *reinterpret_cast<const uint4*>(src + (size_t)row * D + dg * E16);
    } else {
      const int qq = min(qt * C::BQ + lane, N - 1);
      lse_st = LSE[qq];
      d_st = Dl[qq];
    }
  };
  // Stores: per unit 4 row-major rows, then the transposed block in 4 parts;
  // last LSE and D (every wave writes the same 64 values).
  constexpr int NST = 8 * UPT + 1;
  auto st_op = [&](int buf, int qt, int j) {
    if (j < 8 * UPT) {
      const int u = j / 8, o = j % 8;
      int mat, dg, rg;
      unit(u, mat, dg, rg);
      if (o < 4) {
        T* dst = mat ? Gs[buf] : Qs[buf];
        *reinterpret_cast<uint4*>(dst + (4 * rg + o) * C::QP + dg * E16) = stx[u][o];
      } else {
        // Rows dg E16 .. dg E16 + E16 - 1 of the transposed tile share one swizzle.
        T* dst = (mat ? Gt[buf] : Qt[buf]) + tr_index<T>(dg * E16, 4 * rg);
        const int wd = o - 4;   // dword of the 16-byte rows
        const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&stx[u][0]);
        const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&stx[u][1]);
        const uint32_t* x2 = reinterpret_cast<const uint32_t*>(&stx[u][2]);
        const uint32_t* x3 = reinterpret_cast<const uint32_t*>(&stx[u][3]);
        if constexpr (sizeof(T) == 2) {
          // Dword wd holds columns 2 wd and 2 wd + 1 of the 4 rows.
          *reinterpret_cast<uint2*>(dst + (2 * wd) * kTrPitch) =
              uint2{__builtin_amdgcn_perm(x1[wd], x0[wd], 0x05040100u),
                    __builtin_amdgcn_perm(x3[wd], x2[wd], 0x05040100u)};
          *reinterpret_cast<uint2*>(dst + (2 * wd + 1) * kTrPitch) =
              uint2{__builtin_amdgcn_perm(x1[wd], x0[wd], 0x07060302u),
                    __builtin_amdgcn_perm(x3[wd], x2[wd], 0x07060302u)};
        } else {
          *reinterpret_cast<uint4*>(dst + wd * kTrPitch) = uint4{x0[wd], x1[wd], x2[wd], x3[wd]};
        }
      }
    } else {
      // Rows past N, and rows that see no key at all, get P = exp2(-inf) = 0.
      const bool live = qt * C::BQ + lane < N && lse_st != -INFINITY;
      lse2s[buf][lane] = live ? lse_st * kLog2e : INFINITY;
      dls[buf][lane] = live ? d_st : 0.f;
    }
  };
  // Staging operation k of a tile's sequence: unit 0's stores, unit 0's loads,
  // unit 1's stores, ...; then the LSE/D store and load.  Returns the operation
  // kind (0 none, 1 store j, 2 load j).
  constexpr int NSTAGE = NST + NLD;
  constexpr auto stage_seq = [](int k, int& j) {
    if (k < 12 * UPT) {
      const int u = k / 12, o = k % 12;
      j = o < 8 ? 8 * u + o : 4 * u + (o - 8);
      return o < 8 ? 1 : 2;
    }
    if (k == 12 * UPT) { j = 8 * UPT; return 1; }
    if (k == 12 * UPT + 1) { j = 4 * UPT; return 2; }
    return 0;
  };
  auto stage_all = [&](int buf, int qt_st, int qt_ld) {
#pragma unroll
    for (int k = 0; k < NSTAGE; ++k) {
      int j = 0;
      const int kind = stage_seq(k, j);
      if (kind == 1) st_op(buf, qt_st, j);
      if (kind == 2) ld_op(qt_ld, j);
    }
  };
  // One query head of the group: stage its first tiles, then the tile loop.
  auto use_head = [&](int g) {
    const size_t head = kvhead * a.G + g;
    qhead = (int)head;
    Q = static_cast<const T*>(a.q) + (sp.q + g * sp.hs) * D;
    dO = static_cast<const T*>(a.dout) + (sp.q + g * sp.hs) * D;
    LSE = a.lse + head * a.N;
    Dl = a.delta + head * a.Np;
    // The K/V fragments must have landed before the loop, whose waits then
    // cover only the loads issued inside it.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
    for (int j = 0; j < NLD; ++j) ld_op(qt0, j);
    stage_all(0, qt0, qt0 + 1);
    __syncthreads();
  };

  // One query tile is a fixed stream of NM MFMAs, in issue order:
  //   [0, NS)            S = Q K^T and dP = dO V^T of block 0 (32 queries)
  //   [NS, 2NS)          the same for block 1
  //   [2NS, 2NS+NV)      dV += P^T dO and dK += dS^T Q of block 0
  //   [2NS+NV, NM)       the same for block 1
  // The LDS operand of MFMA m (a Q / dO row fragment, or 8 consecutive queries
  // of one head-dim row of dO^T / Q^T) is read PD slots ahead, and the P / dS
  // arithmetic of a block, one element at a time, fills the slots between its
  // S/dP MFMAs and its dV/dK MFMAs, so one wave keeps the matrix unit busy.
  constexpr int NS = 2 * C::NKS;
  constexpr int NVB = 2 * (D / 32);
  constexpr int NV = C::NU * NVB;
  constexpr int NM = 2 * NS + 2 * NV;
  static_assert(C::NBUF == 1 || NSTAGE + 1 <= NM, "every staging operation needs a slot");
  constexpr int PD = 4;
  constexpr int EPU = 16 / C::NU;   // elements of P (and dS) per packed fragment
  // Slot that computes element i of P/dS of block b (blocks overlap S/dP of
  // block 1 and dV/dK of block 0 respectively).
  constexpr auto elem_slot = [](int b, int i) {
    return b == 0 ? NS + 2 + (i * (NS - 2)) / 16 : 2 * NS + 2 + (i * (NV - 2)) / 16;
  };
  auto lds_opnd = [&](int buf, int m) -> frag {
    if (m < 2 * NS) {
      const int qb = m / NS, ks = (m % NS) / 2;
      const T* base = (m & 1) ? Gs[buf] : Qs[buf];
      return load_frag<T>(&base[(qb * 32 + qrow) * C::QP + C::KPL * h + ks * C::KM]);
    }
    const int r = m - 2 * NS, qb = r / NV, u = (r % NV) / NVB, db = (r % NVB) / 2;
    const int qofs = qb * 32 + (kPerm ? 16 * u + 8 * h : 8 * (u >> 2) + 4 * h + (u & 3));
    const T* base = (r & 1) ? Qt[buf] : Gt[buf];
    return load_frag<T>(&base[tr_index<T>(db * 32 + col, qofs)]);
  };

  for (int g = 0; g < a.G; ++g) {
  use_head(g);
  for (int qt = qt0; qt < nqt; ++qt) {
    const int qi0 = qt * C::BQ;
    const bool tact = block_on(a, qhead, qi0, k0);   // block of a block mask computed
    const int buf = C::NBUF == 2 ? (qt - qt0) & 1 : 0;
    f32x16 s[2], dp[2], p[2], ds[2];
    frag pa[2][C::NU], sa[2][C::NU];
    f32x4 l4[2][4], d4[2][4];   // lse2 and D of 4 consecutive queries, per element group
    frag opq[PD];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x16{};
      dp[b] = f32x16{};
    }
#pragma unroll
    for (int m = 0; m < PD; ++m) opq[m] = lds_opnd(buf, m);
    static_for<0, NM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      // LSE / D reads, PD slots before the first element of their group.
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (m == elem_slot(b, 4 * g) - PD) {
            const int row = b * 32 + qoff_of(4 * g) + hoff;
            l4[b][g] = *reinterpret_cast<const f32x4*>(&lse2s[buf][row]);
            d4[b][g] = *reinterpret_cast<const f32x4*>(&dls[buf][row]);
          }
      const frag x = opq[m % PD];
      if constexpr (m + PD < NM) opq[m % PD] = lds_opnd(buf, m + PD);
      if constexpr (m < 2 * NS) {
        constexpr int qb = m / NS, ks = (m % NS) / 2;
        if constexpr (m & 1) dp[qb] = M::mma(x, vf[ks], dp[qb]);
        else s[qb] = M::mma(x, kf[ks], s[qb]);
      } else {
        constexpr int r = m - 2 * NS, qb = r / NV, u = (r % NV) / NVB, db = (r % NVB) / 2;
        if constexpr (r & 1) dk[db] = M::mma(sa[qb][u], x, dk[db]);
        else dv[db] = M::mma(pa[qb][u], x, dv[db]);
      }
      // Staging of tile qt + 1 into the other buffer (free since the previous
      // barrier) and loads of tile qt + 2, one operation per slot from slot 1.
      if constexpr (C::NBUF == 2 && m >= 1 && m - 1 < NSTAGE) {
        int j = 0;
        constexpr int k = m - 1;
        const int kind = stage_seq(k, j);
        if (kind == 1) st_op(buf ^ 1, qt + 1, j);
        if (kind == 2) ld_op(qt + 2, j);
      }
      // P = exp2(S c - lse2), dS = P (dP - D); keys past N need no mask (their
      // results are never stored), rows past N have lse2 = +inf.
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (m == elem_slot(b, i)) {
            const int qo = b * 32 + qoff_of(i) + hoff;
            float e = exp2_fast(fmaf(s[b][i], c, -l4[b][i / 4][i % 4]));
            if (!tact || qi0 + qo < myk - wr || qi0 + qo > myk + wl) e = 0.f;
            float pe = e, dpi = dp[b][i];
            if constexpr (DROP) {   // dV's P and dP through the kept entries
              const bool keep = drop_keep(a.drop, qhead, qi0 + qo, myk);
              pe = keep ? e * a.drop.scale : 0.f;
              dpi = keep ? dpi * a.drop.scale : 0.f;
            }
            p[b][i] = pe;
            ds[b][i] = e * (dpi - d4[b][i / 4][i % 4]);
            if ((i + 1) % EPU == 0) {
              pa[b][i / EPU] = pack_frag<T>(p[b], i / EPU);
              sa[b][i / EPU] = pack_frag<T>(ds[b], i / EPU);
            }
          }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (C::NBUF == 2) {
      __syncthreads();
    } else {
      __syncthreads();
      stage_all(0, qt + 1, qt + 2);
      __syncthreads();
    }
  }
  }

  // Epilogue: lane (col = d, h) holds keys kw + 8(i/4) + 4h + i%4.
  T* dK = static_cast<T*>(a.dk) + sp.kv * D;
  T* dV = static_cast<T*>(a.dv) + sp.kv * D;
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

// ------------------------------------------------------------------ dQ (16-bit types)


// The dQ kernel for 16-bit types, on the same LDS layout as the 16-bit dK/dV
// kernel (rows padded to D + 16 elements, 8-byte slot XOR (r >> 3) & 3):
// K and V tiles are copied straight into LDS, three buffers deep; S^T = K Q^T
// and dP^T = V dO^T take their A operand from K / V rows (two 8-byte reads,
// rows in the order row_pi) and Q / dO from registers; dQ^T += K^T dS^T takes
// K^T through transposing reads.  8 waves x 32 queries per workgroup.
// NW = 8: one workgroup of 8 waves per CU, three K/V buffers, tiles copied two
// ahead (waves 0-3 copy K, 4-7 V).  NW = 4 (d = 128): two workgroups of 4 waves
// per CU, two buffers, each tile copied one ahead by every wave; 128 query rows
// per workgroup balance causal work better.
template <int D, int NW_>
struct Dq16 {
  static constexpr int NW = NW_;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;             // queries per workgroup
  static constexpr int BC = 64;                  // keys per tile
  static constexpr int PB = TileLds<D>::PB;      // bytes per row (multiples of RPC rows)
  static constexpr int TILE = BC * PB;
  static constexpr int BUF = 2 * TILE;           // K, V
  static constexpr int NB = NW == 8 ? 3 : 2;
  static constexpr int RPC = TileLds<D>::ROWS_PER_COPY;
  static constexpr int NKS = D / 16;
  static constexpr int NS = 2 * NKS;             // S/dP MFMAs per 32-key block
  static constexpr int NQ = 2 * (D / 32);        // dQ MFMAs per 32-key block
  static constexpr int NM = 2 * NS + 2 * NQ;     // MFMAs per tile
  static constexpr int NLD = 2 * BC / NW / RPC;  // copies per wave per tile
};

// BSPARSE as for the dK/dV kernel: the tile queue only in the block-sparse
// instance, plain consecutive tiles otherwise.
template <typename T, int D, bool CAUSAL, int NW, bool DROP, bool BSPARSE>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq16_kernel(BwdArgs a) {
  using C = Dq16<D, NW>;
  static_assert(NW == 8 || (NW == 4 && D == 128), "4-wave dQ workgroups are built for d = 128");
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
  // Under the causal mask the last query tiles see the most keys: start them
  // first (counted in this sequence's tiles).
  const int ntq_own = (N + C::BR - 1) / C::BR;
  const int qt = CAUSAL ? ntq_own - 1 - rank : rank;
  if (qt < 0 || qt >= ntq_own) return;   // a tile past the end of a shorter sequence
  const int q0 = qt * C::BR;
  const T* Q = static_cast<const T*>(a.q) + sp.q * D;
  const T* K = static_cast<const T*>(a.k) + sp.kv * D;   // the head's K/V head
  const T* V = static_cast<const T*>(a.v) + sp.kv * D;
  const T* dO = static_cast<const T*>(a.dout) + sp.q * D;
  T* dQ = static_cast<T*>(a.dq) + sp.q * D;
  const float c = a.scale * kLog2e;

  const int qw = q0 + 32 * w;
  const int myq = qw + col;
  const int qrow = min(myq, N - 1);
  // Q and dO operands (B of S^T = K Q^T and of dP^T = V dO^T) of this lane's
  // query, held in registers for the whole kernel.
  frag qf[C::NKS], gf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    qf[ks] = load_frag<T>(Q + (size_t)qrow * D + ks * 16 + 8 * h);
    gf[ks] = load_frag<T>(dO + (size_t)qrow * D + ks * 16 + 8 * h);
  }
  const float l2 = a.l2[head * a.Np + qrow];       // LSE log2(e), +inf if no visible key
  const float dl = a.delta[head * a.Np + qrow];
  // The dP^T accumulators start at -D (every element of a lane is this lane's
  // query), so that they end at dP - D and dS = P (dP - D) is one multiply.
  // Not in the d = 128 dropout instances, whose registers would spill.
  constexpr bool DINIT = !DROP || D == 64;
  f32x16 dinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) dinit[i] = DINIT ? -dl : 0.f;
  // Under dropout the kept dP is scaled: dS = P (scale (acc + D) - D) =
  // P (scale acc + D (scale - 1)) for kept elements, -P D for dropped ones.
  const float dls = DROP ? dl * (a.drop.scale - 1.f) : 0.f;
  // Visible keys of this lane's row: klo .. khi (window, causal and N).
  const int wr = CAUSAL ? min(a.wr, 0) : a.wr;
  const int khi = min(myq + wr, N - 1), klo = myq - a.wl;
  // Key tiles of the workgroup: [lo, hi), of which [ml, mu) need no mask.
  const TileRange tr = tile_range(q0, min(q0 + C::BR, N) - 1, N, a.wl, wr, C::BC, false);
  // The key tiles to visit: consecutive, or the active ones of the
  // workgroup's row of a block mask.
  BlockSkip sk;
  TileQueue tq;
  if constexpr (BSPARSE) {
    sk = block_row(a, hd, q0 / kBlockQ, C::BC);
    tq.start(sk, tr.lo, tr.hi, lane);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) tq.t[t] = tr.lo + t;
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  // Lane parts of the LDS addresses (bytes from the start of a buffer).
  const TileLds<D> lay(lane);
  // Copy op j of key tile kt into buffer b, one group of RPC rows (4 at
  // d = 128, 8 at d = 64) starting at row r0.  NW = 8: waves 0-3 copy K, 4-7
  // copy V, wave w rows 16 (w & 3) + RPC j ..  NW = 4: wave w copies rows
  // 16 w + 4 j .. of K (j < 4) and 16 w + 4 (j - 4) .. of V.  Rows past N read
  // as zero (and are masked through khi).
  const i32x4 rsk = buffer_rsrc(K, (uint32_t)N * (2 * D));
  const i32x4 rsv = buffer_rsrc(V, (uint32_t)N * (2 * D));
  auto copy_op = [&](int b, int kt, int j) {
    const int mat = NW == 8 ? w >> 2 : j >> 2;
    const i32x4& rsrc = mat ? rsv : rsk;
    const uint32_t base = lds_address(smem) + b * C::BUF + mat * C::TILE;
    const int r0 = NW == 8 ? 16 * (w & 3) + C::RPC * j : 16 * w + C::RPC * (j & 3);
    copy16_to_lds(rsrc, lay.c[(r0 >> 3) & 1], (uint32_t)(kt * C::BC + r0) * (2 * D), base + r0 * C::PB);
  };

  // Prologue: queue tiles t0 and t1 (NW = 8) or t0 (NW = 4).  The copies go
  // out while the Q / dO fragments and L2 / D are still loading; the wait after
  // them covers both.
#pragma unroll
  for (int t = 0; t < C::NB - 1; ++t)
#pragma unroll
    for (int j = 0; j < C::NLD; ++j) copy_op(t, tq.t[t], j);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  // The MFMA stream of one key tile: S^T/dP^T of key blocks 0 and 1 (32 keys
  // each), then dQ^T of blocks 0 and 1; the dS arithmetic of block 0 runs
  // beside the S/dP MFMAs of block 1, that of block 1 beside dQ of block 0.
  constexpr int NS = C::NS, NQ = C::NQ, NM = C::NM;
  constexpr int PD = 4;
  // Element i of block b: its exponential at elem_slot(b, i), the rest of its
  // arithmetic one slot later, so that no instruction waits on the
  // exponential's result in the slot that computes it.
  constexpr auto elem_slot = [](int b, int i) {
    return b == 0 ? NS + 2 + (i * (NS - 3)) / 16 : 2 * NS + 1 + (i * (NQ - 3)) / 16;
  };
  // NW = 8: copies of queue tile t2 spread over the stream; NW = 4: copies of
  // t1 early in the stream, since they must land before its end.
  constexpr auto copy_slot = [](int k) { return NW == 8 ? 1 + (k * (NM - 6)) / C::NLD : 1 + 2 * k; };
  int bcur = 0;
  // One key tile.  MASK: some key of the tile is past N or, under the causal
  // mask, after some query of the workgroup.
  auto tile = [&](int kt, int tnext, auto maskc) {
    constexpr bool MASK = decltype(maskc)::value;
    const int key0 = kt * C::BC;
    const int rlo = klo - key0 - h;                 // masked tiles: offsets rlo ..
    const uint32_t rspan = (uint32_t)(khi - klo);   // rlo + rspan are visible
    uint32_t kbits[2] = {0u, 0u};                   // dropout: keep bit of element i of block b
    const int b1 = bcur == C::NB - 1 ? 0 : bcur + 1;
    const int b2 = b1 == C::NB - 1 ? 0 : b1 + 1;
    const int boff = bcur * C::BUF;
    auto operand = [&](int m) -> frag {
      if (m < 2 * NS) {
        const int kb = m / NS, ks = (m % NS) / 2, mat = m & 1;   // K for S, V for dP
        const int off = boff + mat * C::TILE + kb * 32 * C::PB;
        return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(smem + lay.A(ks) + off));
      }
      const int r = m - 2 * NS, kb = r / NQ, u = (r % NQ) / (D / 32), db = r % (D / 32);
      s16x4 v[2];
#pragma unroll
      for (int rp = 0; rp < 2; ++rp) {
        const int off = boff + (kb * 32 + 16 * u + 8 * rp) * C::PB;
        v[rp] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(smem + lay.T(rp, db) + off));
      }
      return __builtin_bit_cast(frag, s16x8{v[0][0], v[0][1], v[0][2], v[0][3],
                                            v[1][0], v[1][1], v[1][2], v[1][3]});
    };
    f32x16 s[2], dp[2], ds[2];
    frag sa[2][2];
    frag opq[PD];
#pragma unroll
    for (int m = 0; m < PD; m += 2) {
      opq[m + 1] = operand(m + 1);
      asm volatile("" ::: "memory");   // keeps the two operands' reads apart
      opq[m] = operand(m);
    }
    auto slot = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
#pragma unroll
      for (int k = 0; k < C::NLD; ++k)
        if (m == copy_slot(k)) copy_op(C::NB == 3 ? b2 : b1, tnext, k);
      // Operands are read in pairs at odd slots, the odd one first, so that the
      // wait for the even one covers both.
      const frag x = opq[m % PD];
      if constexpr ((m & 1) && m + PD - 1 < NM) {
        opq[(m + PD) % PD] = operand(m + PD);
        asm volatile("" ::: "memory");
        opq[(m + PD - 1) % PD] = operand(m + PD - 1);
      }
      if constexpr (m < 2 * NS) {
        constexpr int kb = m / NS, ks = (m % NS) / 2;
        if constexpr (m & 1) dp[kb] = M::mma(x, gf[ks], ks == 0 ? (DINIT ? dinit : f32x16{}) : dp[kb]);
        else s[kb] = M::mma(x, qf[ks], ks == 0 ? f32x16{} : s[kb]);
      } else {
        constexpr int r = m - 2 * NS, kb = r / NQ, u = (r % NQ) / (D / 32), db = r % (D / 32);
        acc[db] = M::mma(x, sa[kb][u], acc[db]);
      }
      // P = exp2(S c - L2), dS = P (dP - D); element i of lane half h is key
      // 8 (i / 4) + 2 (i % 4) + h of its block.
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (m == elem_slot(b, i)) ds[b][i] = exp2_fast(fmaf(s[b][i], c, -l2));
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (m == elem_slot(b, i) + 1) {
            float e = ds[b][i];
            if (MASK) {
              // Visible iff klo <= key <= khi, as one unsigned compare.
              const int ke = b * 32 + 8 * (i / 4) + 2 * (i % 4);   // key - key0 - h
              if ((uint32_t)(ke - rlo) > rspan) e = 0.f;
            }
            if constexpr (DROP) {
              // Elements 8 u .. 8 u + 7 are keys key0 + 32 b + 16 u + h + 2 t: one
              // generator call, made at the first of them.
              if (i % 8 == 0) {
                uint32_t wv[4];
                drop_call(a.drop, hd, myq, (key0 + 32 * b) / 16 + i / 8, h, wv);
                uint32_t bits = 0;
#pragma unroll
                for (int t = 0; t < 8; ++t)
                  bits |= (((t & 1) ? (wv[t >> 1] >> 16) : (wv[t >> 1] & 0xFFFFu)) < a.drop.keep_t ? 1u : 0u) << t;
                kbits[b] = (kbits[b] & ~(0xFFu << i)) | (bits << i);
              }
              if constexpr (DINIT)
                ds[b][i] = e * (((kbits[b] >> i) & 1u) ? fmaf(a.drop.scale, dp[b][i], dls) : -dl);
              else
                ds[b][i] = e * ((((kbits[b] >> i) & 1u) ? dp[b][i] * a.drop.scale : 0.f) - dl);
            } else {
              ds[b][i] = e * dp[b][i];
            }
            if ((i + 1) % 8 == 0) sa[b][i / 8] = pack_frag<T>(ds[b], i / 8);
          }
      __builtin_amdgcn_sched_barrier(0);
    };
    // Two waves share a SIMD: the wave in the S / dP half of its stream issues
    // first, the other wave's dQ MFMAs and dS arithmetic fill in around it
    // (measured 1-2 % faster than equal priorities).
    __builtin_amdgcn_s_setprio(1);
    static_for<0, 2 * NS>(slot);
    __builtin_amdgcn_s_setprio(0);
    static_for<2 * NS, NM>(slot);
    // The tile copied during the previous tile (NW = 8) or this one (NW = 4)
    // must have landed.
    __builtin_amdgcn_s_waitcnt(NW == 8 ? wait_vmcnt(C::NLD) : kWaitVmcnt0);
    __syncthreads();
    bcur = b1;
  };
  // Tiles [lo, ml) and [mu, hi) need masks in some row (the window's edges,
  // the causal diagonal, N); [ml, mu) none.  Separate loops, each with its own
  // register allocation.
  if constexpr (BSPARSE) {
    // The queue skips the inactive tiles of the block mask; tnext is the tile
    // copied during this one.
    for (; tq.t[0] < tr.ml; tq.advance(sk, tr.hi, lane)) tile(tq.t[0], tq.t[C::NB - 1], std::true_type{});
    for (; tq.t[0] < tr.mu; tq.advance(sk, tr.hi, lane)) tile(tq.t[0], tq.t[C::NB - 1], std::false_type{});
    for (; tq.t[0] < tr.hi; tq.advance(sk, tr.hi, lane)) tile(tq.t[0], tq.t[C::NB - 1], std::true_type{});
  } else {
    int kt = tr.lo;
    for (; kt < tr.ml; ++kt) tile(kt, kt + C::NB - 1, std::true_type{});
    // Two tiles per trip of the unmasked loop: one taken branch per two tiles
    // (about 0.3 % of dQ's time on the offset workload).
    for (; kt + 1 < tr.mu; kt += 2) {
      tile(kt, kt + C::NB - 1, std::false_type{});
      tile(kt + 1, kt + C::NB, std::false_type{});
    }
    for (; kt < tr.mu; ++kt) tile(kt, kt + C::NB - 1, std::false_type{});
    for (; kt < tr.hi; ++kt) tile(kt, kt + C::NB - 1, std::true_type{});
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  if (myq < N) {
    // Lane (col = query, h) holds dQ^T rows d = 32 db + 8 (i / 4) + 4 h + i % 4.
    T* orow = dQ + (size_t)myq * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        store4<T>(orow + db * 32 + 8 * r + 4 * h, acc[db][4 * r] * sc, acc[db][4 * r + 1] * sc,
                  acc[db][4 * r + 2] * sc, acc[db][4 * r + 3] * sc);
  }
}

// ------------------------------------------------------------------ dK, dV (16-bit types)

// Layout of the 16-bit dK/dV kernel.  Query tiles (Q and dO, 64 rows) live in
// LDS only row-major, with rows padded to D + 16 elements and the 8-byte slots
// of row r permuted by XOR-ing the low two slot bits with (r >> 3) & 3.  With
// the A-operand rows of S taken in the order pi (below), both kinds of operand
// read touch 32 distinct 8-byte bank pairs per half wave (no bank conflicts):
//   S = Q K^T, dP = dO V^T: A operand = two 8-byte reads from one Q / dO row;
//   dV += P^T dO, dK += dS^T Q: B operand = two transposing reads
//     (ds_read_b64_tr_b16), each gathering 4 queries of one head-dim column.
// Tiles are copied from global memory straight into LDS (global_load_lds),
// three buffers deep, so the copy of tile t + 2 runs during tile t.
template <int D>
struct Dkv16 {
  static constexpr int BKC = 128;                // keys per workgroup (32 per wave)
  static constexpr int BQ = 64;                  // queries per tile
  static constexpr int PB = TileLds<D>::PB;      // bytes per row (multiples of RPC rows)
  static constexpr int TILE = BQ * PB;           // bytes of one Q or dO tile
  static constexpr int BUF = 2 * TILE + 2 * BQ * 4;   // Q, dO, L2, D
  static constexpr int NB = 3;
  static constexpr int RPC = TileLds<D>::ROWS_PER_COPY;   // rows per copy
  static constexpr int NKS = D / 16;             // k steps of S and dP
  static constexpr int NS = 2 * NKS;             // S/dP MFMAs per 32-query block
  static constexpr int NVB = 2 * (D / 32);       // dV/dK MFMAs per 16 queries
  static constexpr int NV = 2 * NVB;             // dV/dK MFMAs per block
  static constexpr int NM = 2 * NS + 2 * NV;     // MFMAs per tile
  static constexpr int NLD = 2 * BQ / 4 / RPC + 2;   // copies per wave per tile: Q, dO; L2, D
};

// BSPARSE: a block mask is given (the tile queue skips its dropped blocks);
// without it the tiles are consecutive and the loops step plainly, which
// keeps this kernel's code as small as before the queue (1-2 % faster).
//
// DQ (the one-pass backward): the workgroup also adds its key tile's share of
// dQ, dS K over its 128 keys, into the float32 accumulator a.dqacc by atomic
// adds ("FlashAttention-2: Faster Attention with Better Parallelism and Work
// Partitioning", section "Parallelism: 시퀀스 길이 차원 병렬화": dQ by atomic adds
// across the key-tile workgroups).  Each wave stores its rounded dS (as dS^T,
// keys x queries) into LDS; after the tile's barrier, during the next tile,
// wave w reads the whole 128-key dS^T of the tile and multiplies it with K
// (held in registers for the whole kernel) for its part of the 64 x D dQ
// tile: D = 128: head-dim block w of both 32-query blocks; D = 64: query block
// w / 2, head-dim block w % 2.  Rows past N land in the accumulator's padding
// rows (their dS is 0).  Not with dropout (its LDS area does not fit beside
// the two dS^T buffers).
template <typename T, int D, bool CAUSAL, bool DROP, bool BSPARSE, bool DQ = false>
__global__ __launch_bounds__(256, 1) void bwd_dkdv16_kernel(BwdArgs a) {
  using C = Dkv16<D>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  static_assert(!(DQ && DROP), "the one-pass backward has no dropout instance");
  // Dropout: per wave and 32-query block, the 16-bit uniforms of its 32 x 32
  // (query, key) elements, 2 KB, after the tile buffers.
  constexpr int DSCR = 2048;
  // DQ: two dS^T buffers (128 keys x 64 queries, the 64-column tile layout).
  using LayS = RowLds64;
  constexpr int DST = C::BKC * LayS::PB;
  constexpr int DSB = C::NB * C::BUF;   // first dS^T buffer
  __shared__ __attribute__((aligned(16))) char smem[C::NB * C::BUF + (DROP ? 8 * DSCR : 0) +
                                                    (DQ ? 2 * DST : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntk = gridDim.x;
  int kt, hd;
  // Under the causal mask the key tiles near the start see the most queries and
  // come first.
  work_item<CAUSAL>(ntk, kt, hd);
  hd = packed_head(a, hd, a.H / a.G);
  const int k0 = kt * C::BKC;
  // hd is a K/V head; its query heads hd G .. hd G + G - 1 run one after another.
  const size_t kvhead = (size_t)hd;
  const Span sp = span_of(a, hd * a.G);
  const int N = sp.n;
  if (k0 >= N) return;   // a tile past the end of a shorter sequence
  const T* K = static_cast<const T*>(a.k) + sp.kv * D;
  const T* V = static_cast<const T*>(a.v) + sp.kv * D;
  const float c = a.scale * kLog2e;

  const int kw = k0 + 32 * w;    // first key of this wave
  const int myk = kw + col;      // this lane's key (column of S)
  const int kg = min(myk, N - 1);
  // K and V operands (B of S = Q K^T and of dP = dO V^T) of this lane's key.
  // V is negated (exact): the dP accumulators start at D and end at D - dP,
  // so dS = -P (D - dP) needs one multiply, and the sign goes into dK's scale.
  frag kf[C::NKS], vf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    kf[ks] = load_frag<T>(K + (size_t)kg * D + ks * 16 + 8 * h);
    vf[ks] = neg_frag<T>(load_frag<T>(V + (size_t)kg * D + ks * 16 + 8 * h));
  }
  // K and V stay in AGPRs (MFMA reads its B operand from there); the VGPRs
  // hold the accumulators, which the VALU reads directly.
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    asm volatile("" : "+a"(kf[ks]));
    asm volatile("" : "+a"(vf[ks]));
  }
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dv[db] = f32x16{};
    dk[db] = f32x16{};
  }
  // DQ: this wave's dQ blocks (query block qbq + j, j < NQB; head-dim block dbq).
  constexpr int NQB = D / 64;
  const int dbq = D == 128 ? w : (w & 1), qbq = D == 128 ? 0 : (w >> 1);
  const LayS lays(lane);
  frag kq[DQ ? C::BKC / 16 : 1];
  // Window: queries [myk - wr, myk + wl] see this lane's key.  Query tiles of
  // the workgroup: [lo, hi), of which [ml, mu) need no mask.
  const int wl = a.wl, wr = CAUSAL ? min(a.wr, 0) : a.wr;
  const TileRange tr = tile_range(k0, k0 + C::BKC - 1, N, wr, wl, C::BQ, true);

  // Lane parts of the LDS addresses (bytes from the start of a buffer).
  const TileLds<D> lay(lane);
  // Copy op j of tile qt into buffer b: j < NROW: rows of Q (first half of
  // the ops) or dO, wave w taking rows 16 w .. 16 w + 15 in groups of RPC rows
  // (16 w + RPC jj ..); j = NROW, NROW + 1: the tile's L2 and
  // D, lane p holding query row_pi(p) of the tile (the order of a lane half's
  // P elements).  Every wave copies the same L2 and D.  Rows past N read as
  // zero (the padding rows of L2 are +inf, so their P is 0; past Np all of Q,
  // dO, L2 and D read as zero, and P dO and P (dP - D) vanish with dO).
  i32x4 rsq, rsg, rsl, rsd;   // Q, dO, L2 and D of the current query head
  int qhead = 0;              // its index b H + h (dropout's generator counter)
  constexpr int NROW = C::NLD - 2;
  // Copies of one tile into one buffer.  Wave w's rows are 16 w .. 16 w + 15, so
  // with the per-tile bases below (LDS address of the wave's first row, global
  // byte offset of that row, LDS address of the buffer, byte offset of the
  // tile's L2 and D) every copy adds only constants.  The bases pass through an
  // empty asm so that the compiler computes them per tile instead of keeping one
  // sum per copy live in scalar registers.
  struct Bases { uint32_t row_lds, row_glb, buf_lds, ld_glb; };
  auto bases = [&](int b, int qt) {
    Bases x{lds_address(smem) + b * C::BUF + 16 * w * C::PB, (uint32_t)(qt * C::BQ + 16 * w) * (2 * D),
            lds_address(smem) + b * C::BUF, (uint32_t)(qt * C::BQ) * 4};
    asm volatile("" : "+s"(x.row_lds), "+s"(x.row_glb), "+s"(x.buf_lds), "+s"(x.ld_glb));
    return x;
  };
  // The dropout instances (the most registers of all) pay the full wait states
  // before every copy rather than rely on where the compiler reloads spilled
  // descriptors.
  constexpr bool SAFE = DROP;
  auto copy_op = [&](const Bases& x, int j) {
    if (j < NROW) {
      const int mat = j / (NROW / 2), r = C::RPC * (j % (NROW / 2));
      copy16_to_lds<SAFE>(mat ? rsg : rsq, lay.c[(r >> 3) & 1], x.row_glb + r * (2 * D),
                          x.row_lds + mat * C::TILE + r * C::PB);
    } else {
      copy_to_lds<SAFE>(j == NROW ? rsl : rsd, 4 * row_pi(lane), x.ld_glb,
                        x.buf_lds + 2 * C::TILE + (j - NROW) * C::BQ * 4);
    }
  };

  // The query tiles to visit for the current query head: consecutive, or the
  // active ones of the workgroup's column of its block mask.
  BlockSkip sk;
  TileQueue tq;
  // Start query head g of the group: its resources and tile queue, then queue
  // tiles t0 and t1 into buffers 0 and 1.
  auto use_head = [&](int g) {
    const size_t head = kvhead * a.G + g;
    qhead = (int)head;
    if constexpr (BSPARSE) {
      sk = block_col(a, qhead, k0 / kBlockK, C::BQ);
      tq.start(sk, tr.lo, tr.hi, lane);
    } else {
      tq.t[0] = tr.lo;
      tq.t[1] = tr.lo + 1;
    }
    rsq = buffer_rsrc(static_cast<const T*>(a.q) + (sp.q + g * sp.hs) * D, (uint32_t)N * (2 * D));
    rsg = buffer_rsrc(static_cast<const T*>(a.dout) + (sp.q + g * sp.hs) * D, (uint32_t)N * (2 * D));
    rsl = buffer_rsrc(a.l2 + head * a.Np, (uint32_t)a.Np * 4);
    rsd = buffer_rsrc(a.delta + head * a.Np, (uint32_t)a.Np * 4);
    // The copies go out while the K / V fragments are still loading (first
    // head); the wait after them covers both (1 % on short causal workgroups).
    const Bases x0 = bases(0, tq.t[0]), x1 = bases(1, tq.t[1]);
#pragma unroll
    for (int j = 0; j < C::NLD; ++j) copy_op(x0, j);
#pragma unroll
    for (int j = 0; j < C::NLD; ++j) copy_op(x1, j);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };

  // The MFMA stream of one tile: S/dP of blocks 0 and 1 (32 queries each), then
  // dV/dK of blocks 0 and 1; each LDS operand is read PD slots ahead, and the
  // P/dS arithmetic of a block fills the slots between its S/dP and dV/dK MFMAs.
  constexpr int NS = C::NS, NV = C::NV, NVB = C::NVB, NM = C::NM;
  constexpr int PD = 4;
  // Element i of block b: the first 8 (P and dS for the first half of the
  // block's dV/dK MFMAs) done before those start, the last 8 overlapping
  // them, before the second half starts.
  // The exponential of each element at elem_slot(b, i), the rest of its
  // arithmetic one slot later (nothing waits on the exponential in its slot).
  constexpr auto elem_slot = [](int b, int i) {
    return (b == 0 ? NS : 2 * NS) + 2 + (i * (NS + NVB - 3)) / 16;
  };
  // Slot of copy k of the next-but-one tile.
  constexpr auto copy_slot = [](int k) { return 1 + (k * (NM - 6)) / C::NLD; };
  int bcur = 0;
  // DQ: the dS^T buffer the current tile writes, the tile whose dS^T the other
  // buffer holds (-1: none), and this lane's row and swizzle in a dS^T buffer.
  int dpar = 0, dprev = -1;
  const int dsrow = (32 * w + col) * LayS::PB, dsswz = (col >> 3) & 1;
  // dQ of query tile qtp of the current query head from dS^T buffer par: this
  // wave's blocks, 8 MFMAs each over the 128 keys, added into the accumulator.
  // Element i of lane (col, h) is accumulator row 32 qb + 16 (i / 8) + 8 h +
  // 2 (i % 4) + (i / 4) % 2 of the tile (the query of logical slot
  // 8 (i / 4) + 4 h + i % 4 of block qb), column 32 dbq + col.
  auto dq_flush = [&](int par, int qtp) {
    if constexpr (DQ) {
      float* base = a.dqacc + ((size_t)qhead * a.Np + (size_t)qtp * C::BQ + 8 * h) * D + dbq * 32 + col;
      const char* dsb = smem + DSB + par * DST;
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        const int qb = qbq + j;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::BKC / 16; ++ks) {
          s16x4 v[2];
#pragma unroll
          for (int rp = 0; rp < 2; ++rp)
            v[rp] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(dsb + lays.T(rp, qb) + (16 * ks + 8 * rp) * LayS::PB));
          acc = M::mma(__builtin_bit_cast(frag, s16x8{v[0][0], v[0][1], v[0][2], v[0][3],
                                                      v[1][0], v[1][1], v[1][2], v[1][3]}),
                       kq[ks], acc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
          unsafeAtomicAdd(base + (32 * qb + 16 * (i >> 3) + 2 * (i & 3) + ((i >> 2) & 1)) * D, acc[i]);
      }
    }
  };
  // One query tile (tnext: the tile copied meanwhile).  MASK: some query of the
  // tile lies outside the window of some key of the workgroup.
  auto tile = [&](int qt, int tnext, auto maskc) {
    constexpr bool MASK = decltype(maskc)::value;
    const int qi0 = qt * C::BQ;
    // DQ: the previous tile's dQ (its dS^T was written before the last barrier).
    if constexpr (DQ)
      if (dprev >= 0) dq_flush(dpar ^ 1, dprev);
    // Masked tiles: query offsets (q - qi0 - h) rlo .. rlo + rspan see this
    // lane's key (sides of kNoLimit keep the sums below 2^31).
    const int rlo = myk - wr - qi0 - h;
    const uint32_t rspan = (uint32_t)wl + (uint32_t)wr;
    const int b1 = bcur == 2 ? 0 : bcur + 1;
    const int b2 = b1 == 2 ? 0 : b1 + 1;
    const int boff = bcur * C::BUF;
    auto operand = [&](int m) -> frag {
      if (m < 2 * NS) {
        const int qb = m / NS, ks = (m % NS) / 2, mat = m & 1;
        const int off = boff + mat * C::TILE + qb * 32 * C::PB;
        return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(smem + lay.A(ks) + off));
      }
      const int r = m - 2 * NS, qb = r / NV, u = (r % NV) / NVB, db = (r % NVB) / 2;
      const int mat = (r & 1) ? 0 : 1;         // dK reads Q, dV reads dO
      s16x4 v[2];
#pragma unroll
      for (int rp = 0; rp < 2; ++rp) {
        const int off = boff + mat * C::TILE + (qb * 32 + 16 * u + 8 * rp) * C::PB;
        v[rp] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(smem + lay.T(rp, db) + off));
      }
      return __builtin_bit_cast(frag, s16x8{v[0][0], v[0][1], v[0][2], v[0][3],
                                            v[1][0], v[1][1], v[1][2], v[1][3]});
    };
    f32x16 s[2], dp[2], p[2], ds[2];
    frag pa[2][2], sa[2][2];
    f32x4 l4[2][4];
    frag opq[PD];
    // D of the 16 queries of this lane's elements of block b, in element order.
    auto load_d = [&](int b) -> f32x16 {
      const float* dl = reinterpret_cast<const float*>(smem + boff + 2 * C::TILE) + C::BQ + b * 32 + 4 * h;
      f32x16 r;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 q = *reinterpret_cast<const f32x4*>(dl + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 * g + e] = q[e];
      }
      return r;
    };
    dp[0] = load_d(0);
#pragma unroll
    for (int b = 0; b < 2; ++b) s[b] = f32x16{};
#pragma unroll
    for (int m = 0; m < PD; m += 2) {
      opq[m + 1] = operand(m + 1);
      asm volatile("" ::: "memory");   // keeps the two operands' reads apart
      opq[m] = operand(m);
    }
    const Bases xc = bases(b2, tnext);
    // Dropout keep bits of this lane's key column, bit i of block b for query
    // 8 (i / 4) + 2 (i % 4) + h of the block.  A generator call serves the 8
    // keys 16 p + par + 2 t of one query, which sit in 8 lanes here: lane (col,
    // h) makes the calls of query col and key half p = h (both parities) into
    // the wave's LDS area, then reads the uniforms of its own key back.
    uint32_t kbits[2] = {0u, 0u};
    float d4[2][4][4];   // D of 4 queries per element group (dropout only)
    if constexpr (DROP) {
      const int kgrp = (kw >> 4) + h;   // 16-key group of the calls this lane makes
      char* scr = smem + C::NB * C::BUF + w * 2 * DSCR;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          uint32_t wv[4];
          drop_call(a.drop, qhead, qi0 + 32 * b + col, kgrp, par, wv);
          *reinterpret_cast<uint4*>(scr + b * DSCR + ((col * 2 + h) * 2 + par) * 16) =
              uint4{wv[0], wv[1], wv[2], wv[3]};
        }
      __builtin_amdgcn_wave_barrier();
      const int kp = col >> 4, kpar = col & 1, kt = (col & 15) >> 1;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = 8 * (i / 4) + 2 * (i % 4) + h;
          const uint16_t u = *reinterpret_cast<const uint16_t*>(
              scr + b * DSCR + ((ql * 2 + kp) * 2 + kpar) * 16 + 2 * kt);
          kbits[b] |= ((uint32_t)u < a.drop.keep_t ? 1u : 0u) << i;
        }
      __builtin_amdgcn_wave_barrier();
    }
    static_for<0, NM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
#pragma unroll
      for (int k = 0; k < C::NLD; ++k)
        if (m == copy_slot(k)) copy_op(xc, k);
      // L2 of 4 queries (one element group), PD slots before first use; D of
      // block 1 well before its first dP MFMA.
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (m == elem_slot(b, 4 * g) - PD) {
            const float* l2 = reinterpret_cast<const float*>(smem + boff + 2 * C::TILE);
            l4[b][g] = *reinterpret_cast<const f32x4*>(&l2[b * 32 + 8 * g + 4 * h]);
            if constexpr (DROP) {
              const f32x4 dd = *reinterpret_cast<const f32x4*>(&l2[C::BQ + b * 32 + 8 * g + 4 * h]);
#pragma unroll
              for (int e = 0; e < 4; ++e) d4[b][g][e] = dd[e];
            }
          }
      if constexpr (m == NS / 2) dp[1] = load_d(1);
      // Operands are read in pairs at odd slots, the odd one first, so that the
      // wait for the even one covers both.
      const frag x = opq[m % PD];
      if constexpr ((m & 1) && m + PD - 1 < NM) {
        opq[(m + PD) % PD] = operand(m + PD);
        asm volatile("" ::: "memory");
        opq[(m + PD - 1) % PD] = operand(m + PD - 1);
      }
      if constexpr (m < 2 * NS) {
        constexpr int qb = m / NS, ks = (m % NS) / 2;
        if constexpr (m & 1) dp[qb] = M::mma(x, vf[ks], dp[qb]);
        else s[qb] = M::mma(x, kf[ks], s[qb]);
      } else {
        constexpr int r = m - 2 * NS, qb = r / NV, u = (r % NV) / NVB, db = (r % NVB) / 2;
        if constexpr (r & 1) dk[db] = M::mma(sa[qb][u], x, dk[db]);
        else dv[db] = M::mma(pa[qb][u], x, dv[db]);
      }
      // P = exp2(S c - L2), -dS = P (D - dP).  Element i of lane half h is
      // query 8 (i / 4) + 2 (i % 4) + h of its block; keys past N need no mask
      // (their results are never stored).
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (m == elem_slot(b, i)) p[b][i] = exp2_fast(fmaf(s[b][i], c, -l4[b][i / 4][i % 4]));
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (m == elem_slot(b, i) + 1) {
            float e = p[b][i];
            if (MASK) {
              // Visible iff myk - wr <= q <= myk + wl, as one unsigned compare.
              const int qe = b * 32 + 8 * (i / 4) + 2 * (i % 4);   // q - qi0 - h
              if ((uint32_t)(qe - rlo) > rspan) e = 0.f;
            }
            if constexpr (DROP) {
              // dV takes the kept P scaled; -dS = P (D - dP') with dP' the kept,
              // scaled dP = D - (accumulator), as the accumulator holds D - dP.
              const bool keep = (kbits[b] >> i) & 1u;
              const float dd = d4[b][i / 4][i % 4];
              p[b][i] = keep ? e * a.drop.scale : 0.f;
              ds[b][i] = e * (keep ? fmaf(a.drop.scale, dp[b][i] - dd, dd) : dd);
            } else {
              p[b][i] = e;
              ds[b][i] = e * dp[b][i];
            }
            if ((i + 1) % 8 == 0) {
              pa[b][i / 8] = pack_frag<T>(p[b], i / 8);
              sa[b][i / 8] = pack_frag<T>(ds[b], i / 8);
              if constexpr (DQ) {
                // dS^T row 32 w + col (this lane's key); logical query slots
                // 32 b + 16 u + 8 h + t hold queries 32 b + 16 u + 8 (t / 4) +
                // 2 (t % 4) + h, the elements of this fragment in order.
                *reinterpret_cast<s16x8*>(smem + DSB + dpar * DST + dsrow +
                                          16 * ((4 * b + 2 * (i / 8) + h) ^ dsswz)) =
                    __builtin_bit_cast(s16x8, sa[b][i / 8]);
              }
            }
          }
      __builtin_amdgcn_sched_barrier(0);
    });
    // Tile qt + 1 (copied during the previous tile) must have landed; the
    // copies of tile tnext may still be in flight.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(C::NLD));
    __syncthreads();
    bcur = b1;
    if constexpr (DQ) {
      dprev = qt;
      dpar ^= 1;
    }
  };
  // Tiles [lo, ml) and [mu, hi) need masks in some key column (the causal
  // diagonal and the window's near edge, its far edge); [ml, mu) none, rows past
  // N included (their L2 is +inf).  Separate loops, each with its own register
  // allocation.
  if constexpr (DQ) {
    // K rows k0 .. k0 + 127 into buffer 2 (rows past N land as zero), read back
    // as the B operands of dQ: lane (col, h) of k step ks holds K[k0 + 16 ks +
    // 8 rp + 2 s + h][32 dbq + col] (rp < 2, s < 4), the keys that the dS^T
    // reads of the same step give it.  Held in AGPRs for the whole kernel.
    const i32x4 rsk = buffer_rsrc(K, (uint32_t)N * (2 * D));
    const uint32_t kbuf = lds_address(smem) + 2 * C::BUF;
#pragma unroll
    for (int j = 0; j < 32 / C::RPC; ++j) {
      const int r = 32 * w + C::RPC * j;   // first row of the group
      copy16_to_lds(rsk, lay.c[(r >> 3) & 1], (uint32_t)(k0 + r) * (2 * D), kbuf + r * C::PB);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // Lane offsets of head-dim block dbq, selected rather than indexed (a
    // runtime index into the layout's offset array would move it to memory).
    int tq[2];
#pragma unroll
    for (int rp = 0; rp < 2; ++rp)
      tq[rp] = ((dbq & 1) ? lay.T(rp, 1) : lay.T(rp, 0)) + (dbq >> 1) * (lay.T(rp, 2) - lay.T(rp, 0));
#pragma unroll
    for (int ks = 0; ks < C::BKC / 16; ++ks) {
      s16x4 v[2];
#pragma unroll
      for (int rp = 0; rp < 2; ++rp)
        v[rp] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(smem + 2 * C::BUF + tq[rp] + (16 * ks + 8 * rp) * C::PB));
      kq[ks] = __builtin_bit_cast(frag, s16x8{v[0][0], v[0][1], v[0][2], v[0][3],
                                              v[1][0], v[1][1], v[1][2], v[1][3]});
      asm volatile("" : "+a"(kq[ks]));
    }
    // (Buffer 2 is next written by the first tile's copies, after use_head's
    // barrier, which every wave reaches only with these reads done.)
  }
  for (int g = 0; g < a.G; ++g) {
    use_head(g);
    bcur = 0;
    if constexpr (BSPARSE) {
      // The queue skips the inactive tiles of the block mask; the tile copied
      // during tile t0 is t2.
      for (; tq.t[0] < tr.ml; tq.advance(sk, tr.hi, lane)) tile(tq.t[0], tq.t[2], std::true_type{});
      for (; tq.t[0] < tr.mu; tq.advance(sk, tr.hi, lane)) tile(tq.t[0], tq.t[2], std::false_type{});
      for (; tq.t[0] < tr.hi; tq.advance(sk, tr.hi, lane)) tile(tq.t[0], tq.t[2], std::true_type{});
    } else {
      int qt = tr.lo;
      for (; qt < tr.ml; ++qt) tile(qt, qt + 2, std::true_type{});
      // Two tiles per trip of the unmasked loop: one taken branch per two
      // tiles, which this single wave per SIMD pays in full (1 % of the
      // kernel's time on the offset workload).
      for (; qt + 1 < tr.mu; qt += 2) {
        tile(qt, qt + 2, std::false_type{});
        tile(qt + 1, qt + 3, std::false_type{});
      }
      for (; qt < tr.mu; ++qt) tile(qt, qt + 2, std::false_type{});
      for (; qt < tr.hi; ++qt) tile(qt, qt + 2, std::true_type{});
    }
    // No copy may still be writing LDS when the next head starts or the
    // workgroup ends, and every wave is done with the buffers.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // DQ: the head's last tile (its dS^T is complete after that barrier).
    if constexpr (DQ) {
      if (dprev >= 0) dq_flush(dpar ^ 1, dprev);
      dprev = -1;
    }
  }

  // Epilogue: lane (col = d, h) holds keys kw + 8(i/4) + 4h + i%4, so its
  // values of a row are 2 bytes wide and 256 bytes apart.  They go through
  // LDS (the buffers are free now), this wave's 32 rows of dK and of dV
  // row-major with rows ERS bytes apart (rows 4 apart, the two lane halves of
  // a write, then fall on opposite bank halves), and come back as 16-byte
  // row chunks: 16 stores of 1 KB per wave at d = 128 instead of 128 of 128
  // bytes.  (On the causal B4 H32 N4096 workload, whose workgroups are short,
  // the stores take 4.6 % of this kernel's time; staged, 4.0 %: the rest is
  // the wait for the written bytes before the workgroup's slot frees.)
  T* dK = static_cast<T*>(a.dk) + sp.kv * D;
  T* dV = static_cast<T*>(a.dv) + sp.kv * D;
  constexpr int ERS = 2 * D + 16;
  constexpr int CPR = 2 * D / 16;                // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                  // rows per read / store
  static_assert(4 * 2 * 32 * ERS <= (int)sizeof(smem), "epilogue staging fits the buffers");
  __syncthreads();                               // DQ: every wave is past its last dS^T read
  char* st = smem + w * 2 * 32 * ERS;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + 4 * h + (i & 3);
      *reinterpret_cast<T*>(st + r * ERS + 2 * (db * 32 + col)) = (T)(dk[db][i] * -a.scale);   // dk holds -dS^T Q
      *reinterpret_cast<T*>(st + (32 + r) * ERS + 2 * (db * 32 + col)) = (T)dv[db][i];
    }
  // (A wave's LDS accesses complete in order: its reads below see its writes.)
#pragma unroll
  for (int mat = 0; mat < 2; ++mat) {
    T* dst = mat ? dV : dK;
#pragma unroll
    for (int j = 0; j < 32 / RPI; ++j) {
      const int r = RPI * j + lane / CPR, c = lane % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(st + (32 * mat + r) * ERS + 16 * c);
      if (kw + r < N) *reinterpret_cast<uint4*>(dst + (size_t)(kw + r) * D + 8 * c) = v;
    }
  }
}

// dK/dV for 16-bit types with the tile stream pipelined across query tiles.
//
// The work split and data flow are those of bwd_dkdv16_kernel (4 waves x 32
// keys; K and V of the lane's key in registers; the Q, dO, L2 and D tiles of
// 64 queries copied straight into LDS; P recomputed from L2, dS = P (dP - D);
// "FlashAttention-2: Faster Attention with Better Parallelism and Work
// Partitioning", section "Backward Pass").  Three things differ:
//   * The stream of query tile t runs four phases of MFMAs: A, S and dP of its
//     query block 0; D', dV and dK of block 1 of tile t - 1; B, S and dP of its
//     block 1; C, dV and dK of its block 0.  The P / dS arithmetic of block 1
//     of tile t - 1 runs beside A and that of block 0 beside D' and B, so the
//     vector work spreads over the whole tile instead of crowding its second
//     half.
//   * dK and dV accumulate in AGPRs (mma_agpr), which leaves the VGPRs to the
//     S / dP of both blocks and to the state carried into the next tile.
//   * Four buffers (tile t - 1 is still read during tile t), copies two tiles
//     ahead, and the barrier before phase C.  Past it the first operands and
//     D of tile t + 1 are read while tile t still runs, so a tile starts
//     without waiting for LDS.
// A run of tiles with one mask flag starts with a tile without phase D' and
// ends with phase D' alone (drain).  The launcher takes it at d = 64, where a
// tile has half the MFMAs per element of P of d = 128 and the spread-out
// arithmetic pays; at d = 128 it measured slower than bwd_dkdv16_kernel.
template <typename T, int D, bool CAUSAL, bool DROP, bool BSPARSE>
__global__ __launch_bounds__(256, 1) void bwd_dkdv16p_kernel(BwdArgs a) {
  using C = Dkv16<D>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int NB = 4;
  // Dropout: per wave, the 16-bit uniforms of the 32 x 32 (query, key)
  // elements of one 32-query block, 2 KB, after the tile buffers (the two
  // blocks of a tile use it in turn).
  constexpr int DSCR = 2048;
  __shared__ __attribute__((aligned(16))) char smem[NB * C::BUF + (DROP ? 4 * DSCR : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntk = gridDim.x;
  int kt, hd;
  // Under the causal mask the key tiles near the start see the most queries and
  // come first.
  work_item<CAUSAL>(ntk, kt, hd);
  hd = packed_head(a, hd, a.H / a.G);
  const int k0 = kt * C::BKC;
  // hd is a K/V head; its query heads hd G .. hd G + G - 1 run one after another.
  const size_t kvhead = (size_t)hd;
  const Span sp = span_of(a, hd * a.G);
  const int N = sp.n;
  if (k0 >= N) return;   // a tile past the end of a shorter sequence
  const T* K = static_cast<const T*>(a.k) + sp.kv * D;
  const T* V = static_cast<const T*>(a.v) + sp.kv * D;
  const float c = a.scale * kLog2e;

  const int kw = k0 + 32 * w;    // first key of this wave
  const int myk = kw + col;      // this lane's key (column of S)
  const int kg = min(myk, N - 1);
  // K and V operands (B of S = Q K^T and of dP = dO V^T) of this lane's key,
  // pinned in AGPRs.  V is negated (exact): the dP accumulators start at D
  // and end at D - dP, so dS = -P (D - dP) needs one multiply, and the sign
  // goes into dK's scale.
  frag kf[C::NKS], vf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    kf[ks] = load_frag<T>(K + (size_t)kg * D + ks * 16 + 8 * h);
    vf[ks] = neg_frag<T>(load_frag<T>(V + (size_t)kg * D + ks * 16 + 8 * h));
  }
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    asm volatile("" : "+a"(kf[ks]));
    asm volatile("" : "+a"(vf[ks]));
  }
  // dV (acc[0]) and dK (acc[1]) of the lane's key, in AGPRs.
  f32x16 acc[2][D / 32];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[j][db] = f32x16{};
  agpr_settle(acc);
  // Window: queries [myk - wr, myk + wl] see this lane's key.  Query tiles of
  // the workgroup: [lo, hi), of which [ml, mu) need no mask.
  const int wl = a.wl, wr = CAUSAL ? min(a.wr, 0) : a.wr;
  const TileRange tr = tile_range(k0, k0 + C::BKC - 1, N, wr, wl, C::BQ, true);
  const uint32_t rspan = (uint32_t)wl + (uint32_t)wr;

  const TileLds<D> lay(lane);
  // Copies as in bwd_dkdv16_kernel: op j < NROW a group of RPC rows of Q (first
  // half of the ops) or dO, wave w taking rows 16 w ..; ops NROW, NROW + 1 the
  // tile's L2 and D, lane p holding query row_pi(p).
  i32x4 rsq, rsg, rsl, rsd;
  int qhead = 0;
  constexpr int NROW = C::NLD - 2;
  struct Bases { uint32_t row_lds, row_glb, buf_lds, ld_glb; };
  auto bases = [&](int b, int qt) {
    Bases x{lds_address(smem) + b * C::BUF + 16 * w * C::PB, (uint32_t)(qt * C::BQ + 16 * w) * (2 * D),
            lds_address(smem) + b * C::BUF, (uint32_t)(qt * C::BQ) * 4};
    asm volatile("" : "+s"(x.row_lds), "+s"(x.row_glb), "+s"(x.buf_lds), "+s"(x.ld_glb));
    return x;
  };
  constexpr bool SAFE = DROP;
  auto copy_op = [&](const Bases& x, int j) {
    if (j < NROW) {
      const int mat = j / (NROW / 2), r = C::RPC * (j % (NROW / 2));
      copy16_to_lds<SAFE>(mat ? rsg : rsq, lay.c[(r >> 3) & 1], x.row_glb + r * (2 * D),
                          x.row_lds + mat * C::TILE + r * C::PB);
    } else {
      copy_to_lds<SAFE>(j == NROW ? rsl : rsd, 4 * row_pi(lane), x.ld_glb,
                        x.buf_lds + 2 * C::TILE + (j - NROW) * C::BQ * 4);
    }
  };

  BlockSkip sk;
  TileQueue tq;
  // Start query head g of the group: resources and tile queue, then copy tiles
  // t0 and t1 into buffers 0 and 1.
  auto use_head = [&](int g) {
    const size_t head = kvhead * a.G + g;
    qhead = (int)head;
    if constexpr (BSPARSE) {
      sk = block_col(a, qhead, k0 / kBlockK, C::BQ);
      tq.start(sk, tr.lo, tr.hi, lane);
    } else {
      tq.t[0] = tr.lo;
      tq.t[1] = tr.lo + 1;
    }
    rsq = buffer_rsrc(static_cast<const T*>(a.q) + (sp.q + g * sp.hs) * D, (uint32_t)N * (2 * D));
    rsg = buffer_rsrc(static_cast<const T*>(a.dout) + (sp.q + g * sp.hs) * D, (uint32_t)N * (2 * D));
    rsl = buffer_rsrc(a.l2 + head * a.Np, (uint32_t)a.Np * 4);
    rsd = buffer_rsrc(a.delta + head * a.Np, (uint32_t)a.Np * 4);
    const Bases x0 = bases(0, tq.t[0]), x1 = bases(1, tq.t[1]);
#pragma unroll
    for (int j = 0; j < C::NLD; ++j) copy_op(x0, j);
#pragma unroll
    for (int j = 0; j < C::NLD; ++j) copy_op(x1, j);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };

  constexpr int NS = C::NS, NV = C::NV, NVB = C::NVB, NM = C::NM;
  constexpr int PD = 4;                           // operands read ahead (slots)
  // Phase starts (MFMA slots of one tile).
  constexpr int P_D = NS, P_B = NS + NV, P_C = 2 * NS + NV;
  constexpr int XB = P_C - 2;                     // the tile's barrier
  // Element i of block 1 of the previous tile (its P and dS) at e1_slot(i):
  // elements 0..7 before phase D' starts, 8..15 before its second half.
  constexpr auto e1_slot = [](int i) { return (i * (NS + NVB - 2)) / 16; };
  // D (the dP accumulator's start) of block 1 of this tile, after the previous
  // tile's block 1 is done with the registers.
  constexpr int DRL1 = NS + NVB - 1;
  // Element i of block 0 of this tile: 0..7 before phase C, 8..15 before its
  // second half.
  constexpr int E0S = NS + NVB;
  constexpr auto e0_slot = [](int i) { return E0S + (i * (P_C + NVB - 2 - E0S)) / 16; };
  // D of block 0 of the next tile (past the barrier and past this tile's
  // block 0 arithmetic), and L2 (with D under dropout) of block 1 of this tile
  // for the next tile's arithmetic.
  constexpr int DRL0 = e0_slot(15) + 2 > XB + 1 ? e0_slot(15) + 2 : XB + 1;
  constexpr int L1S = P_C;
  // Copy k of the tile two ahead, all before the barrier.
  constexpr auto copy_slot = [](int k) { return 1 + (k * (XB - 3)) / C::NLD; };

  // Carried from tile to tile: S and D - dP of both blocks (block 1's are the
  // previous tile's until DRL1), the packed P and dS, L2 / D / keep bits of
  // the previous tile's block 1, the operands read ahead.
  f32x16 s[2], dp[2];
  frag pa[2][2], sa[2][2];
  f32x4 l4p[4];
  float d4p[4][4];
  uint32_t kb[2] = {0u, 0u};
  frag opq[PD];
  int step = 0, qprev = 0;

  auto l2_at = [&](int boff) { return reinterpret_cast<const float*>(smem + boff + 2 * C::TILE); };
  // D of the 16 queries of this lane's elements of block b, in element order.
  auto load_d = [&](int boff, int b) -> f32x16 {
    const float* dl = l2_at(boff) + C::BQ + b * 32 + 4 * h;
    f32x16 r;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(dl + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) r[4 * g + e] = q[e];
    }
    return r;
  };
  // A operand of S (mat 0: Q rows) or dP (mat 1: dO rows), k step ks, query
  // block qb, from the buffer at boff.
  auto opA = [&](int boff, int qb, int ks, int mat) -> frag {
    const int off = boff + mat * C::TILE + qb * 32 * C::PB;
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(smem + lay.A(ks) + off));
  };
  // B operand of dV (mat 1: dO^T) or dK (mat 0: Q^T): 16-query step u, head-dim
  // block db, query block qb; two transposing reads.
  auto opT = [&](int boff, int qb, int u, int db, int mat) -> frag {
    s16x4 v[2];
#pragma unroll
    for (int rp = 0; rp < 2; ++rp) {
      const int off = boff + mat * C::TILE + (qb * 32 + 16 * u + 8 * rp) * C::PB;
      v[rp] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + lay.T(rp, db) + off));
    }
    return __builtin_bit_cast(frag, s16x8{v[0][0], v[0][1], v[0][2], v[0][3],
                                          v[1][0], v[1][1], v[1][2], v[1][3]});
  };
  // P and dS of element i of one block: e = 2^(c S - L2) (zero outside the
  // window when MASK), P = e (dropped and scaled under dropout), and -dS = P
  // (D - dP) from the accumulator that holds D - dP.  Element i of lane half h
  // is query 8 (i / 4) + 2 (i % 4) + h of its block.
  auto elem = [&](auto maskc, int b, int i, float sv, float dpv, float l2v, float ddv, uint32_t kbits,
                  int rl, f32x16& pv, f32x16& dsv) {
    constexpr bool MASK = decltype(maskc)::value;
    float e = exp2_fast(fmaf(sv, c, -l2v));
    if (MASK) {
      const int qe = b * 32 + 8 * (i / 4) + 2 * (i % 4);   // q - qi0 - h
      if ((uint32_t)(qe - rl) > rspan) e = 0.f;
    }
    if constexpr (DROP) {
      const bool keep = (kbits >> i) & 1u;
      pv[i] = keep ? e * a.drop.scale : 0.f;
      dsv[i] = e * (keep ? fmaf(a.drop.scale, dpv - ddv, ddv) : ddv);
    } else {
      pv[i] = e;
      dsv[i] = e * dpv;
    }
  };
  // Dropout keep bits of both blocks of query tile qi0 for this lane's key, bit
  // i of block b for query 8 (i / 4) + 2 (i % 4) + h of the block (as in
  // bwd_dkdv16_kernel: each lane makes the generator calls of one query and
  // key half into the wave's LDS area and reads its own key column back).
  auto keep_bits = [&](int qi0) {
    if constexpr (DROP) {
      const int kgrp = (kw >> 4) + h;
      char* scr = smem + NB * C::BUF + w * DSCR;
      const int kp = col >> 4, kpar = col & 1, kt2 = (col & 15) >> 1;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          uint32_t wv[4];
          drop_call(a.drop, qhead, qi0 + 32 * b + col, kgrp, par, wv);
          *reinterpret_cast<uint4*>(scr + ((col * 2 + h) * 2 + par) * 16) = uint4{wv[0], wv[1], wv[2], wv[3]};
        }
        __builtin_amdgcn_wave_barrier();
        uint32_t bits = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = 8 * (i / 4) + 2 * (i % 4) + h;
          const uint16_t u = *reinterpret_cast<const uint16_t*>(scr + ((ql * 2 + kp) * 2 + kpar) * 16 + 2 * kt2);
          bits |= ((uint32_t)u < a.drop.keep_t ? 1u : 0u) << i;
        }
        kb[b] = bits;
        __builtin_amdgcn_wave_barrier();
      }
    }
  };
  // L2 (and D under dropout) of block 1 of the tile in buffer boff.
  auto load_l4p = [&](int boff) {
    const float* l2 = l2_at(boff);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      l4p[g] = *reinterpret_cast<const f32x4*>(&l2[32 + 8 * g + 4 * h]);
      if constexpr (DROP) {
        const f32x4 dd = *reinterpret_cast<const f32x4*>(&l2[C::BQ + 32 + 8 * g + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) d4p[g][e] = dd[e];
      }
    }
  };

  // One query tile: qt at queue step `step` (buffer step & 3), tnext the tile
  // two steps ahead (copied meanwhile).  PREV: phase D' and the arithmetic of
  // block 1 of the previous tile (qprev) run in it.
  auto tile = [&](int qt, int tnext, auto maskc, auto prevc) {
    constexpr bool PREV = decltype(prevc)::value;
    const int qi0 = qt * C::BQ;
    const int bc = step & 3;
    const int boff = bc * C::BUF, bpoff = ((step + 3) & 3) * C::BUF, bnoff = ((step + 1) & 3) * C::BUF;
    const int rlo = myk - wr - qi0 - h, rlop = myk - wr - qprev * C::BQ - h;
    const Bases xc = bases((step + 2) & 3, tnext);
    const uint32_t kbp = kb[1];
    keep_bits(qi0);
    f32x4 l4[4];
    float d40[4][4];
    f32x16 p1, ds1, p0, ds0;
    // Operand of slot m (m >= NM: slot m - NM of the next tile).
    auto operand = [&](auto mc2) -> frag {
      constexpr int mm = decltype(mc2)::value;
      if constexpr (mm >= NM) {
        return opA(bnoff, 0, (mm - NM) / 2, (mm - NM) & 1);
      } else if constexpr (mm < P_D) {
        return opA(boff, 0, mm / 2, mm & 1);
      } else if constexpr (mm < P_B) {
        if constexpr (PREV) {
          constexpr int r = mm - P_D;
          return opT(bpoff, 1, r / NVB, (r % NVB) / 2, (r & 1) ? 0 : 1);
        } else {
          return frag{};
        }
      } else if constexpr (mm < P_C) {
        return opA(boff, 1, (mm - P_B) / 2, (mm - P_B) & 1);
      } else {
        constexpr int r = mm - P_C;
        return opT(boff, 0, r / NVB, (r % NVB) / 2, (r & 1) ? 0 : 1);
      }
    };
    static_for<0, NM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
#pragma unroll
      for (int k = 0; k < C::NLD; ++k)
        if (m == copy_slot(k)) copy_op(xc, k);
      if constexpr (m == XB) {
        // Tile t + 1 (copied during the previous tile) must have landed; the
        // copies of t + 2 may still be in flight.  Past the barrier every wave
        // is done with tile t - 1 and may read tile t + 1.
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(C::NLD));
        __syncthreads();
      }
      // L2 of one element group of block 0, PD slots before first use.
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (m == e0_slot(4 * g) - PD) {
          const float* l2 = l2_at(boff);
          l4[g] = *reinterpret_cast<const f32x4*>(&l2[8 * g + 4 * h]);
          if constexpr (DROP) {
            const f32x4 dd = *reinterpret_cast<const f32x4*>(&l2[C::BQ + 8 * g + 4 * h]);
#pragma unroll
            for (int e = 0; e < 4; ++e) d40[g][e] = dd[e];
          }
        }
      if constexpr (m == DRL1) dp[1] = load_d(boff, 1);
      if constexpr (m == L1S) load_l4p(boff);
      if constexpr (m == DRL0) dp[0] = load_d(bnoff, 0);
      const frag x = opq[m % PD];
      if constexpr ((m & 1) && m + PD - 1 < NM + PD) {
        opq[(m + PD) % PD] = operand(std::integral_constant<int, m + PD>{});
        asm volatile("" ::: "memory");
        opq[(m + PD - 1) % PD] = operand(std::integral_constant<int, m + PD - 1>{});
      }
      if constexpr (m < P_D) {
        constexpr int ks = m / 2;
        if constexpr (m & 1) dp[0] = M::mma(x, vf[ks], dp[0]);
        else s[0] = M::mma(x, kf[ks], ks == 0 ? f32x16{} : s[0]);
      } else if constexpr (m < P_B) {
        if constexpr (PREV) {
          constexpr int r = m - P_D, u = r / NVB, db = (r % NVB) / 2;
          if constexpr (r & 1) mma_agpr<T>(acc[1][db], sa[1][u], x);
          else mma_agpr<T>(acc[0][db], pa[1][u], x);
        }
      } else if constexpr (m < P_C) {
        constexpr int ks = (m - P_B) / 2;
        if constexpr ((m - P_B) & 1) dp[1] = M::mma(x, vf[ks], dp[1]);
        else s[1] = M::mma(x, kf[ks], ks == 0 ? f32x16{} : s[1]);
      } else {
        constexpr int r = m - P_C, u = r / NVB, db = (r % NVB) / 2;
        if constexpr (r & 1) mma_agpr<T>(acc[1][db], sa[0][u], x);
        else mma_agpr<T>(acc[0][db], pa[0][u], x);
      }
      if constexpr (PREV) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (m == e1_slot(i)) {
            elem(maskc, 1, i, s[1][i], dp[1][i], l4p[i / 4][i % 4], DROP ? d4p[i / 4][i % 4] : 0.f, kbp,
                 rlop, p1, ds1);
            if ((i + 1) % 8 == 0) {
              pa[1][i / 8] = pack_frag<T>(p1, i / 8);
              sa[1][i / 8] = pack_frag<T>(ds1, i / 8);
            }
          }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (m == e0_slot(i)) {
          elem(maskc, 0, i, s[0][i], dp[0][i], l4[i / 4][i % 4], DROP ? d40[i / 4][i % 4] : 0.f, kb[0], rlo,
               p0, ds0);
          if ((i + 1) % 8 == 0) {
            pa[0][i / 8] = pack_frag<T>(p0, i / 8);
            sa[0][i / 8] = pack_frag<T>(ds0, i / 8);
          }
        }
      __builtin_amdgcn_sched_barrier(0);
    });
    qprev = qt;
    ++step;
  };
  // Phase D' of the last tile of a run, with its block 1 arithmetic first.
  auto drain = [&](auto maskc) {
    const int bpoff = ((step + 3) & 3) * C::BUF;
    const int rlop = myk - wr - qprev * C::BQ - h;
    f32x16 p1, ds1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      elem(maskc, 1, i, s[1][i], dp[1][i], l4p[i / 4][i % 4], DROP ? d4p[i / 4][i % 4] : 0.f, kb[1], rlop,
           p1, ds1);
      if ((i + 1) % 8 == 0) {
        pa[1][i / 8] = pack_frag<T>(p1, i / 8);
        sa[1][i / 8] = pack_frag<T>(ds1, i / 8);
      }
    }
    // The packs stay above this point, and an MFMA reads a VGPR no sooner
    // than two wait states after a VALU instruction wrote it.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 1");
    static_for<0, NV>([&](auto mc) {
      constexpr int r = decltype(mc)::value, u = r / NVB, db = (r % NVB) / 2;
      const frag x = opT(bpoff, 1, u, db, (r & 1) ? 0 : 1);
      if constexpr (r & 1) mma_agpr<T>(acc[1][db], sa[1][u], x);
      else mma_agpr<T>(acc[0][db], pa[1][u], x);
    });
  };
  // A run of tiles [.., end) with one mask flag, the queue at its first tile.
  auto run = [&](int end, auto maskc) {
    if constexpr (BSPARSE) {
      if (tq.t[0] >= end) return;
      tile(tq.t[0], tq.t[2], maskc, std::false_type{});
      tq.advance(sk, tr.hi, lane);
      for (; tq.t[0] < end; tq.advance(sk, tr.hi, lane)) tile(tq.t[0], tq.t[2], maskc, std::true_type{});
    } else {
      int qt = tq.t[0];
      if (qt >= end) return;
      tile(qt, qt + 2, maskc, std::false_type{});
      for (++qt; qt < end; ++qt) tile(qt, qt + 2, maskc, std::true_type{});
      tq.t[0] = qt;
    }
    drain(maskc);
  };

  for (int g = 0; g < a.G; ++g) {
    use_head(g);
    step = 0;
    // The first tile's first operands and D.
    static_for<0, PD>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      opq[m] = opA(0, 0, m / 2, m & 1);
    });
    dp[0] = load_d(0, 0);
    // Tiles [lo, ml) and [mu, hi) need masks in some key column (the causal
    // diagonal and the window's near edge, its far edge); [ml, mu) none, rows
    // past N included (their L2 is +inf).
    run(tr.ml, std::true_type{});
    run(tr.mu, std::false_type{});
    run(tr.hi, std::true_type{});
    // No copy may still be writing LDS when the next head starts or the
    // workgroup ends, and every wave is done with the buffers.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }

  // Epilogue: lane (col = d, h) holds keys kw + 8(i/4) + 4h + i%4.
  agpr_settle(acc);
  T* dK = static_cast<T*>(a.dk) + sp.kv * D;
  T* dV = static_cast<T*>(a.dv) + sp.kv * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw + 8 * (i >> 2) + 4 * h + (i & 3);
      if (key < N) {
        const size_t off = (size_t)key * D + db * 32 + col;
        dK[off] = (T)(acc[1][db][i] * -a.scale);   // holds -dS^T Q
        dV[off] = (T)acc[0][db][i];
      }
    }
}

// ------------------------------------------------------------------ launchers

template <typename T, int D, bool CAUSAL, bool DROP>
static hipError_t launch_bwd_t(BwdStep step, const BwdArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.H * a.Np;
  if (step == BwdStep::pre) {
    constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
    const long blocks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a, rows);
  } else if (step == BwdStep::dkdv) {
    if constexpr (sizeof(T) == 2) {
      dim3 grid((a.N + Dkv16<D>::BKC - 1) / Dkv16<D>::BKC, a.H / a.G, a.B);
      // d = 64: the pipelined kernel (same-process A/B on one MI355X: 11 %
      // faster on b8h16n1024d64 and b1h16n16384d64 causal).  d = 128 keeps
      // the single-tile stream, which measured 2 % faster than the pipelined
      // one on b2h32n8192d128 and b4h32n4096d128 causal, except with dropout.
      if constexpr (D == 64 || DROP) {
        if (a.bm.mask)
          hipLaunchKernelGGL((bwd_dkdv16p_kernel<T, D, CAUSAL, DROP, true>), grid, dim3(256), 0, s, a);
        else
          hipLaunchKernelGGL((bwd_dkdv16p_kernel<T, D, CAUSAL, DROP, false>), grid, dim3(256), 0, s, a);
      } else {
        if (a.bm.mask)
          hipLaunchKernelGGL((bwd_dkdv16_kernel<T, D, CAUSAL, DROP, true>), grid, dim3(256), 0, s, a);
        else
          hipLaunchKernelGGL((bwd_dkdv16_kernel<T, D, CAUSAL, DROP, false>), grid, dim3(256), 0, s, a);
      }
    } else {
      dim3 grid((a.N + DkvTile<T, D>::BKC - 1) / DkvTile<T, D>::BKC, a.H / a.G, a.B);
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, DROP>), grid, dim3(256), 0, s, a);
    }
  } else if (step == BwdStep::dkdvq) {
    // The one-pass backward: 16-bit types without dropout only (the host
    // never asks for anything else).
    if constexpr (sizeof(T) == 2 && !DROP) {
      dim3 grid((a.N + Dkv16<D>::BKC - 1) / Dkv16<D>::BKC, a.H / a.G, a.B);
      if (a.bm.mask)
        hipLaunchKernelGGL((bwd_dkdv16_kernel<T, D, CAUSAL, false, true, true>), grid, dim3(256), 0,
                           s, a);
      else
        hipLaunchKernelGGL((bwd_dkdv16_kernel<T, D, CAUSAL, false, false, true>), grid, dim3(256), 0,
                           s, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (step == BwdStep::dqfin) {
    const long threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_dqfin_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, s, a, rows);
  } else if constexpr (sizeof(T) == 2) {
    // Causal d = 128: 128-row workgroups, two per CU, balance the triangle.
    constexpr int NW = CAUSAL && D == 128 ? 4 : 8;
    using C = Dq16<D, NW>;
    dim3 grid((a.N + C::BR - 1) / C::BR, a.H, a.B);
    if (a.bm.mask)
      hipLaunchKernelGGL((bwd_dq16_kernel<T, D, CAUSAL, NW, DROP, true>), grid, dim3(C::NT), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq16_kernel<T, D, CAUSAL, NW, DROP, false>), grid, dim3(C::NT), 0, s, a);
  } else {
    dim3 grid((a.N + DqTile<T, D>::BR - 1) / DqTile<T, D>::BR, a.H, a.B);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, DROP>), grid, dim3(DqTile<T, D>::NT), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_inst(BwdStep st, bool causal, const BwdArgs& a, hipStream_t s) {
  if (a.drop.keep_t < 65536)
    return causal ? launch_bwd_t<T, D, true, true>(st, a, s) : launch_bwd_t<T, D, false, true>(st, a, s);
  return causal ? launch_bwd_t<T, D, true, false>(st, a, s) : launch_bwd_t<T, D, false, false>(st, a, s);
}

}  // namespace fa
