// Host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "group_gemm.hpp"
#include "moe_glu.h"

namespace moe {

// Launch one persistent grouped-GEMM kernel instantiation; each returns
// MOE_ERR_UNSUPPORTED for a combination its translation unit does not hold.
moe_status_t launch_group_gemm_fwd(int epi, int blay, const GemmArgs& args, int grid,
                                   hipStream_t stream);
moe_status_t launch_group_gemm_bwd(int epi, int blay, const GemmArgs& args, int grid,
                                   hipStream_t stream);
// MXFP8 x MXFP8 GroupGemm (packed MXFP8 weight, bf16 output)
moe_status_t launch_group_gemm_mx(const GemmArgs& args, int grid, hipStream_t stream);
// FC1 + GLU with MXFP8 inputs (epi: EPI_GLU or EPI_GLU_MX)
moe_status_t launch_group_gemm_mx_glu(const GemmArgs& args, int epi, int grid, hipStream_t stream);
// K-grouped weight gradient (fp32 output)
moe_status_t launch_group_gemm_wgrad(const GemmArgs& args, int grid, hipStream_t stream);

}  // namespace moe
