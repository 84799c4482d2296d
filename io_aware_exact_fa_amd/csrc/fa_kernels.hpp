// Host-side declarations of the kernel launchers (one per dtype x head dim x
// causal instance).  Every launcher only enqueues work on `stream` and
// returns hipGetLastError(); argument checks live in fa_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N;    // H query heads; K and V have H / G heads
  float scale;
  int G = 1;      // query heads per K/V head
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
};

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
