// Kernel launchers of the token-dimension GEMMs (FC1 + SwiGLU, FC2, SwiGLU backward, FC1
// data gradient; BF16 and MXFP8 routed weights), in a translation unit of their own:
// the weight gradients' unit takes another instruction-scheduling strategy
// (moe_megakernel_amd/build.py).
#include <hip/hip_runtime.h>

#include "gemm.hpp"

namespace moe {
namespace gemm {

template <>
void launch_fc1<false>(dim3 grid, hipStream_t st, const Fc1Args& a) {
  hipLaunchKernelGGL(k_fc1_swiglu<false>, grid, dim3(Shapes<false>::FC1::NTH), 0, st, a);
}
template <>
void launch_plain<KC, false>(dim3 grid, hipStream_t st, const PlainArgs& a) {
  hipLaunchKernelGGL((k_gemm_plain<KC, false>), grid, dim3(TL_PLAIN<KC, false>::NTH), 0, st, a);
}
template <>
void launch_dgrad_swiglu<false>(dim3 grid, hipStream_t st, const DgradSwigluArgs& a) {
  hipLaunchKernelGGL(k_dgrad_swiglu<false>, grid, dim3(Shapes<false>::DG2::NTH), 0, st, a);
}
template <>
void launch_plain<RC, false>(dim3 grid, hipStream_t st, const PlainArgs& a) {
  hipLaunchKernelGGL((k_gemm_plain<RC, false>), grid, dim3(TL_PLAIN<RC, false>::NTH), 0, st, a);
}
template <>
void launch_fc1<true>(dim3 grid, hipStream_t st, const Fc1Args& a) {
  hipLaunchKernelGGL(k_fc1_swiglu<true>, grid, dim3(Shapes<true>::FC1::NTH), 0, st, a);
}
template <>
void launch_plain<KC, true>(dim3 grid, hipStream_t st, const PlainArgs& a) {
  hipLaunchKernelGGL((k_gemm_plain<KC, true>), grid, dim3(TL_PLAIN<KC, true>::NTH), 0, st, a);
}
template <>
void launch_dgrad_swiglu<true>(dim3 grid, hipStream_t st, const DgradSwigluArgs& a) {
  hipLaunchKernelGGL(k_dgrad_swiglu<true>, grid, dim3(Shapes<true>::DG2::NTH), 0, st, a);
}
template <>
void launch_plain<RC, true>(dim3 grid, hipStream_t st, const PlainArgs& a) {
  hipLaunchKernelGGL((k_gemm_plain<RC, true>), grid, dim3(TL_PLAIN<RC, true>::NTH), 0, st, a);
}

}  // namespace gemm
}  // namespace moe
