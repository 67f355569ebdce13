// The block-scaled MXFP8 x MXFP8 GroupGemm + Quantize on
// v_mfma_scale_f32_32x32x64_f8f6f4: activations quantised row-wise along K
// (e4m3, or e5m2 for a gradient), the weight quantised along K (e4m3) and
// tile-blocked offline.  (FC1 + GLU with
// MXFP8 operands is in gemm_act_fwd.hip.)
#include "internal.hpp"

namespace moe {

moe_status_t launch_group_gemm_mx(const GemmArgs& a, bool a_e5, int grid, hipStream_t s) {
  if (a_e5)
    hipLaunchKernelGGL((group_gemm_kernel<EPI_STORE, BL_PACKED, AT_MX_A5>), dim3(grid), dim3(64 * gm_waves(EPI_STORE, BL_PACKED, AT_MX_A5)), 0,
                       s, a);
  else
    hipLaunchKernelGGL((group_gemm_kernel<EPI_STORE, BL_PACKED, AT_MX>), dim3(grid), dim3(64 * gm_waves(EPI_STORE, BL_PACKED, AT_MX)), 0,
                       s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
