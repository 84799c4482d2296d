// Backward entry points of the kernel layer: dispatch on dtype and head
// dimension to the instances in fa_bwd_<dtype>_d<D>.hip; the kernels
// themselves are in fa_bwd_kernels.hpp.
#include "fa_kernels.hpp"

namespace fa {

template <typename T>
static hipError_t launch_d(BwdStep st, int d, bool causal, const BwdArgs& a, hipStream_t s) {
  return d == 64 ? launch_bwd_inst<T, 64>(st, causal, a, s) : launch_bwd_inst<T, 128>(st, causal, a, s);
}

static hipError_t launch_step(BwdStep st, Dt dt, int d, bool causal, const BwdArgs& a,
                              hipStream_t s) {
  switch (dt) {
    case Dt::f32: return launch_d<float>(st, d, causal, a, s);
    case Dt::f16: return launch_d<_Float16>(st, d, causal, a, s);
    case Dt::bf16: return launch_d<__bf16>(st, d, causal, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_pre(Dt dt, int d, const BwdArgs& a, hipStream_t s) {
  return launch_step(BwdStep::pre, dt, d, false, a, s);
}

hipError_t launch_bwd_dkdv(Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s) {
  return launch_step(BwdStep::dkdv, dt, d, causal, a, s);
}

hipError_t launch_bwd_dq(Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s) {
  return launch_step(BwdStep::dq, dt, d, causal, a, s);
}

hipError_t launch_bwd_dkdvq(Dt dt, int d, bool causal, const BwdArgs& a, hipStream_t s) {
  return launch_step(BwdStep::dkdvq, dt, d, causal, a, s);
}

hipError_t launch_bwd_dqfin(Dt dt, int d, const BwdArgs& a, hipStream_t s) {
  return launch_step(BwdStep::dqfin, dt, d, false, a, s);
}

}  // namespace fa
