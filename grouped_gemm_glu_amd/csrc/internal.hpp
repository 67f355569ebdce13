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
// MXFP8 x MXFP8 GroupGemm (packed MXFP8 weight, bf16 output); a_e5: A holds
// e5m2 codes
moe_status_t launch_group_gemm_mx(const GemmArgs& args, bool a_e5, int grid, hipStream_t stream);

// Kernels whose epilogue applies the activation exist once per activation
// (gemm_act_fwd.hip and gemm_act_bwd.hip are compiled once per value of
// MOE_ACT); launch_activation_kernel picks the one for args.ep.act.
enum {
  KIND_GLU = 0,          // FC1 + GLU, bf16 operands, packed W1
  KIND_GLU_MXO,          // the same with MXFP8 outputs
  KIND_MXIN_GLU,         // FC1 + GLU, MXFP8 operands
  KIND_MXIN_GLU_MXO,     // the same with MXFP8 outputs
  KIND_ACT,              // FC1 + non-gated activation, packed plain W1
  KIND_DGLU_PACKED,      // dgrad + dGLU, packed W2 (this and the kinds below: backward)
  KIND_DGLU_NK,          // dgrad + dGLU, W2 as [I][H]
  KIND_DGLU_G_PACKED,    // the same two adding d(bias) and d(row_scale)
  KIND_DGLU_G_NK,
  KIND_DACT_PACKED,      // dgrad + non-gated activation derivative
  KIND_DACT_NK
};
moe_status_t launch_activation_kernel(int kind, const GemmArgs& args, int grid, hipStream_t stream);
#define MOE_DECLARE_ACT_LAUNCHERS(n)                                                              \
  moe_status_t launch_act_fwd_##n(int kind, const GemmArgs& args, int grid, hipStream_t stream); \
  moe_status_t launch_act_bwd_##n(int kind, const GemmArgs& args, int grid, hipStream_t stream);
MOE_DECLARE_ACT_LAUNCHERS(0)
MOE_DECLARE_ACT_LAUNCHERS(1)
MOE_DECLARE_ACT_LAUNCHERS(2)
MOE_DECLARE_ACT_LAUNCHERS(3)
#undef MOE_DECLARE_ACT_LAUNCHERS
// K-grouped weight gradient (fp32 output)
moe_status_t launch_group_gemm_wgrad(const GemmArgs& args, int grid, hipStream_t stream);
// the same on K-tiled MXFP8 column copies; a_e5 / b_e5: e5m2 codes
moe_status_t launch_group_gemm_wgrad_mx(const GemmArgs& args, bool a_e5, bool b_e5, int grid,
                                        hipStream_t stream);

}  // namespace moe
