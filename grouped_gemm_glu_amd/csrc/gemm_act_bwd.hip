// dgrad + dGLU kernels for one activation (MOE_ACT, a moe_act_t value given
// on the compile line; the build compiles this file once per activation):
// W2 read as W2^T from the packed copy or from the K-contiguous [I][H], each
// with and without the bias / row-scale gradients; and the non-gated form.
#include "internal.hpp"

#ifndef MOE_ACT
#error "compile once per activation with -DMOE_ACT=<0..3>"
#endif

#define MOE_CAT_(a, b) a##b
#define MOE_CAT(a, b) MOE_CAT_(a, b)

namespace moe {

template <int EPI, int BLAY>
static void launch_dglu(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((group_gemm_kernel<EPI, BLAY, AT_BF16, MOE_ACT>), dim3(grid), dim3(64 * gm_waves(EPI, BLAY, AT_BF16)), 0, s, a);
}

moe_status_t MOE_CAT(launch_act_bwd_, MOE_ACT)(int kind, const GemmArgs& a, int grid,
                                               hipStream_t s) {
  switch (kind) {
    case KIND_DGLU_PACKED: launch_dglu<EPI_DGLU, BL_PACKED>(a, grid, s); break;
    case KIND_DGLU_NK: launch_dglu<EPI_DGLU, BL_NK>(a, grid, s); break;
    case KIND_DGLU_G_PACKED: launch_dglu<EPI_DGLU_G, BL_PACKED>(a, grid, s); break;
    case KIND_DGLU_G_NK: launch_dglu<EPI_DGLU_G, BL_NK>(a, grid, s); break;
    case KIND_DACT_PACKED: launch_dglu<EPI_DACT, BL_PACKED>(a, grid, s); break;
    case KIND_DACT_NK: launch_dglu<EPI_DACT, BL_NK>(a, grid, s); break;
    default: return MOE_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
