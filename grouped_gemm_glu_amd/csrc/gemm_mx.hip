// The block-scaled MXFP8 x MXFP8 GroupGemm + Quantize on
// v_mfma_scale_f32_32x32x64_f8f6f4: activations quantised row-wise along K,
// the weight quantised along K and tile-blocked offline.  (FC1 + GLU with
// MXFP8 operands is in gemm_act_fwd.hip.)
#include "internal.hpp"

namespace moe {

moe_status_t launch_group_gemm_mx(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((group_gemm_kernel<EPI_STORE, BL_PACKED, AT_MX>), dim3(grid), dim3(GM_NT), 0,
                     s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
