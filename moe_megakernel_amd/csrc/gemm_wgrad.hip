// Kernel launchers of the weight-gradient GEMMs, in a translation unit of their own so
// that they take LLVM's max-ilp instruction scheduling (moe_megakernel_amd/build.py),
// which measured faster for them than the default.
#include <hip/hip_runtime.h>

#include "gemm.hpp"

namespace moe {
namespace gemm {

template <int FC, bool MG16, bool SHORT>
void launch_wgrad(dim3 grid, hipStream_t st, const WgradArgs& a) {
  hipLaunchKernelGGL((k_wgrad<FC, MG16, SHORT>), grid, dim3(TL_WG<MG16, SHORT>::NTH), 0, st, a);
}
template void launch_wgrad<1, true, false>(dim3, hipStream_t, const WgradArgs&);
template void launch_wgrad<1, false, true>(dim3, hipStream_t, const WgradArgs&);
template void launch_wgrad<1, false, false>(dim3, hipStream_t, const WgradArgs&);
template void launch_wgrad<2, true, false>(dim3, hipStream_t, const WgradArgs&);
template void launch_wgrad<2, false, true>(dim3, hipStream_t, const WgradArgs&);
template void launch_wgrad<2, false, false>(dim3, hipStream_t, const WgradArgs&);

}  // namespace gemm
}  // namespace moe
