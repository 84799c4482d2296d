// Backward kernels instantiated for __bf16, head dimension 64 (one translation
// unit per instance so that they compile in parallel).
#include "fa_bwd_kernels.hpp"

namespace fa {
template hipError_t launch_bwd_inst<__bf16, 64>(BwdStep, bool, const BwdArgs&, hipStream_t);
}  // namespace fa
