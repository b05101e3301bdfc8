// fa_bwd_kernel_d64.hip -- the D = 64 instances of the backward kernels
// (fa_bwd_kernels.h), in a translation unit of their own so that the build
// can schedule them with LLVM's max-ILP strategy (faster at D = 64, slower
// at D = 128).
#include "fa_bwd_kernels.h"

namespace fa {
namespace bwd {

int launch_backward_d64(const BwdArgs &a, int B, bool causal, hipStream_t stream)
{
    return causal ? launch_bwd<64, true>(a, B, stream) : launch_bwd<64, false>(a, B, stream);
}

}  // namespace bwd
}  // namespace fa
