// FC1 + GLU kernels for one activation (MOE_ACT, a moe_act_t value given on
// the compile line; the build compiles this file once per activation): bf16
// or MXFP8 operands on the packed W1, with or without MXFP8 outputs; and the
// non-gated form on the plain packed W1.
#include "internal.hpp"

#ifndef MOE_ACT
#error "compile once per activation with -DMOE_ACT=<0..3>"
#endif

#define MOE_CAT_(a, b) a##b
#define MOE_CAT(a, b) MOE_CAT_(a, b)

namespace moe {

template <int EPI, int AT>
static void launch_glu(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((group_gemm_kernel<EPI, BL_PACKED, AT, MOE_ACT>), dim3(grid), dim3(64 * gm_waves(EPI, BL_PACKED, AT)), 0, s,
                     a);
}

moe_status_t MOE_CAT(launch_act_fwd_, MOE_ACT)(int kind, const GemmArgs& a, int grid,
                                               hipStream_t s) {
  switch (kind) {
    case KIND_GLU: launch_glu<EPI_GLU, AT_BF16>(a, grid, s); break;
    case KIND_GLU_MXO: launch_glu<EPI_GLU_MX, AT_BF16>(a, grid, s); break;
    case KIND_MXIN_GLU: launch_glu<EPI_GLU, AT_MX>(a, grid, s); break;
    case KIND_MXIN_GLU_MXO: launch_glu<EPI_GLU_MX, AT_MX>(a, grid, s); break;
    case KIND_ACT: launch_glu<EPI_ACT, AT_BF16>(a, grid, s); break;
    default: return MOE_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
