// Kernel launchers of the token-dimension GEMMs (FC1 + SwiGLU, FC2, SwiGLU backward, FC1
// data gradient; BF16 routed weights in two shape sets, and MXFP8), in a translation unit
// of their own: the weight gradients' unit takes another instruction-scheduling strategy
// (moe_megakernel_amd/build.py).
#include <hip/hip_runtime.h>

#include "gemm.hpp"

namespace moe {
namespace gemm {

template <bool MX, bool WIDE>
void launch_fc1(dim3 grid, hipStream_t st, const Fc1Args& a) {
  hipLaunchKernelGGL((k_fc1_swiglu<MX, WIDE>), grid, dim3(ShapesOf<MX, WIDE>::FC1::NTH), 0, st, a);
}
template <int BMODE, bool MX, bool WIDE>
void launch_plain(dim3 grid, hipStream_t st, const PlainArgs& a) {
  hipLaunchKernelGGL((k_gemm_plain<BMODE, MX, WIDE>), grid, dim3(TL_PLAIN<BMODE, MX, WIDE>::NTH), 0, st, a);
}
template <bool MX, bool WIDE>
void launch_dgrad_swiglu(dim3 grid, hipStream_t st, const DgradSwigluArgs& a) {
  hipLaunchKernelGGL((k_dgrad_swiglu<MX, WIDE>), grid, dim3(ShapesOf<MX, WIDE>::DG2::NTH), 0, st, a);
}

template void launch_fc1<false, false>(dim3, hipStream_t, const Fc1Args&);
template void launch_fc1<false, true>(dim3, hipStream_t, const Fc1Args&);
template void launch_fc1<true, false>(dim3, hipStream_t, const Fc1Args&);
template void launch_plain<KC, false, false>(dim3, hipStream_t, const PlainArgs&);
template void launch_plain<KC, false, true>(dim3, hipStream_t, const PlainArgs&);
template void launch_plain<KC, true, false>(dim3, hipStream_t, const PlainArgs&);
template void launch_plain<RC, false, false>(dim3, hipStream_t, const PlainArgs&);
template void launch_plain<RC, false, true>(dim3, hipStream_t, const PlainArgs&);
template void launch_plain<RC, true, false>(dim3, hipStream_t, const PlainArgs&);
template void launch_dgrad_swiglu<false, false>(dim3, hipStream_t, const DgradSwigluArgs&);
template void launch_dgrad_swiglu<false, true>(dim3, hipStream_t, const DgradSwigluArgs&);
template void launch_dgrad_swiglu<true, false>(dim3, hipStream_t, const DgradSwigluArgs&);

}  // namespace gemm
}  // namespace moe
