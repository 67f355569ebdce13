// MXFP8 weight gradients of the expert MLP as K-grouped GroupGemms on the
// block-scaled MFMA: for each expert, C_e = A_e^T B_e with the reduction over
// the group's rows, both operands read from transposed MXFP8 copies in the
// K-tiled layout (dW1 from the copies of Xg and dgu, dW2 from those of y and
// dY2), fp32 output.  One kernel per pair of element formats (e4m3 / e5m2).
#include "internal.hpp"

namespace moe {

template <int AT>
static void launch_wgm(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((group_gemm_kernel<EPI_WGRAD, BL_NK, AT>), dim3(grid),
                     dim3(64 * gm_waves(EPI_WGRAD, BL_NK, AT)), 0, s, a);
}

moe_status_t launch_group_gemm_wgrad_mx(const GemmArgs& a, bool a_e5, bool b_e5, int grid,
                                        hipStream_t s) {
  if (grid < 1) return MOE_OK;    // no experts: nothing to write
  if (a_e5 && b_e5) launch_wgm<AT_MX_AB5>(a, grid, s);
  else if (a_e5) launch_wgm<AT_MX_A5>(a, grid, s);
  else if (b_e5) launch_wgm<AT_MX_B5>(a, grid, s);
  else launch_wgm<AT_MX>(a, grid, s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
