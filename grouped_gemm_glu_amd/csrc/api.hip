// C ABI of the MoE GroupGEMM + GLU library: argument checking, the cached
// device properties and the launches.  Every entry point validates what the
// host can see and returns before any launch on error; nothing here
// allocates, synchronises or reads device memory back.
#include <math.h>
#include <string.h>

#include "aux_kernels.hpp"
#include "internal.hpp"

using namespace moe;

namespace {

constexpr int kMaxDevices = 64;
int g_num_cus[kMaxDevices];  // 0 = not initialised

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

moe_status_t ensure_init(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  if (g_num_cus[dev] == 0) {
    moe_status_t st = moe_init(dev);
    if (st != MOE_OK) return st;
  }
  *cus = g_num_cus[dev];
  return MOE_OK;
}

moe_status_t check_groups(const moe_groups_t* g) {
  if (!g || !g->counts) return MOE_ERR_NULL;
  if (g->E < 1 || g->E > kMaxExperts || g->M_cap < 0) return MOE_ERR_SHAPE;
  if (!aligned4(g->counts) || (g->offsets_out && !aligned4(g->offsets_out)) ||
      (g->status_out && !aligned4(g->status_out)))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

moe_status_t check_mx(const moe_mx_out_t* mx) {
  if (!mx) return MOE_OK;
  if ((mx->row_q == nullptr) != (mx->row_s == nullptr)) return MOE_ERR_NULL;
  if ((mx->col_q == nullptr) != (mx->col_s == nullptr)) return MOE_ERR_NULL;
  if (mx->e5m2 != 0 && mx->e5m2 != 1) return MOE_ERR_UNSUPPORTED;
  if (mx->col_blocked != 0 && mx->col_blocked != 1) return MOE_ERR_UNSUPPORTED;
  if (mx->col_blocked && mx->col_q && !aligned16(mx->col_q)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

moe_status_t fill_epilogue(const moe_epilogue_t* ep, EpiParams* out) {
  if (!ep) return MOE_ERR_NULL;
  if (ep->act < MOE_ACT_SWIGLU || ep->act > MOE_ACT_SRELU) return MOE_ERR_UNSUPPORTED;
  if (ep->bias && !aligned16(ep->bias)) return MOE_ERR_ALIGN;
  if (ep->row_scale && !aligned4(ep->row_scale)) return MOE_ERR_ALIGN;
  if (isnan(ep->alpha) || isnan(ep->gate_lo) || isnan(ep->gate_hi) || isnan(ep->up_lo) ||
      isnan(ep->up_hi) || isnan(ep->up_offset))
    return MOE_ERR_SHAPE;
  out->act = ep->act;
  out->alpha = ep->alpha;
  out->gate_lo = ep->gate_lo;
  out->gate_hi = ep->gate_hi;
  out->up_lo = ep->up_lo;
  out->up_hi = ep->up_hi;
  out->up_offset = ep->up_offset;
  out->bias = static_cast<const uint16_t*>(ep->bias);
  out->row_scale = ep->row_scale;
  if (ep->amax_out && !aligned4(ep->amax_out)) return MOE_ERR_ALIGN;
  out->amax_out = ep->amax_out;
  out->rht_signs = ep->rht_signs & 0xFFFFu;
  if ((ep->dbias_out && !aligned4(ep->dbias_out)) || (ep->drow_scale_out && !aligned4(ep->drow_scale_out)))
    return MOE_ERR_ALIGN;
  out->dbias_out = ep->dbias_out;
  out->drs_out = ep->drow_scale_out;
  return MOE_OK;
}

void fill_groups(GemmArgs* a, const moe_groups_t* g) {
  a->counts = g->counts;
  a->E = g->E;
  a->M_cap = g->M_cap;
  a->offsets_out = g->offsets_out;
  a->status_out = g->status_out;
}

void fill_mx(GemmArgs* a, const moe_mx_out_t* mx, int cols, const moe_groups_t* g) {
  a->row_q = mx ? mx->row_q : nullptr;
  a->row_s = mx ? mx->row_s : nullptr;
  a->col_q = mx ? mx->col_q : nullptr;
  a->col_s = mx ? mx->col_s : nullptr;
  a->mx_cols = cols;
  a->mx_e5 = mx ? mx->e5m2 : 0;
  a->col_blocked = mx ? mx->col_blocked : 0;
  a->col_s_ld = a->col_blocked ? 4 * ((g->M_cap + 127) / 128 + g->E) : (g->M_cap + 31) / 32 + g->E;
}

// Persistent grid: one workgroup per usable CU (the kernel holds a CU's LDS),
// capped by an upper bound on the tile count (each expert adds at most one
// partial m-tile).
int persistent_grid(int cus, int cu_margin, int M_cap, int E, int ntiles_n) {
  int usable = cus - (cu_margin > 0 ? cu_margin : 0);
  if (usable < 1) usable = 1;
  long long bound = ((long long)(M_cap + GM_BM - 1) / GM_BM + E) * ntiles_n;
  if (bound < 1) bound = 1;
  return (int)(bound < usable ? bound : usable);
}

}  // namespace

namespace moe {

moe_status_t launch_activation_kernel(int kind, const GemmArgs& a, int grid, hipStream_t s) {
  const bool bwd = kind >= KIND_DGLU_PACKED;
  switch (a.ep.act) {
    case ACT_SWIGLU: return bwd ? launch_act_bwd_0(kind, a, grid, s) : launch_act_fwd_0(kind, a, grid, s);
    case ACT_GEGLU: return bwd ? launch_act_bwd_1(kind, a, grid, s) : launch_act_fwd_1(kind, a, grid, s);
    case ACT_GEGLU_TANH:
      return bwd ? launch_act_bwd_2(kind, a, grid, s) : launch_act_fwd_2(kind, a, grid, s);
    case ACT_SRELU: return bwd ? launch_act_bwd_3(kind, a, grid, s) : launch_act_fwd_3(kind, a, grid, s);
    default: return MOE_ERR_UNSUPPORTED;
  }
}

}  // namespace moe

extern "C" {

moe_status_t moe_init(int device) {
  if (device < 0 || device >= kMaxDevices) return MOE_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return MOE_ERR_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_DEVICE;
  g_num_cus[device] = prop.multiProcessorCount;
  return MOE_OK;
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or not a supported multiple";
    case MOE_ERR_ALIGN: return "a pointer is not suitably aligned";
    case MOE_ERR_UNSUPPORTED: return "unsupported option combination";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_DEVICE: return "no usable gfx950 device";
  }
  return "unknown status";
}

size_t moe_packed_weight_bytes(int E, int N, int K) {
  if (E <= 0 || N <= 0 || K <= 0) return 0;
  return (size_t)E * (size_t)((N + 255) / 256) * 256 * (size_t)K * 2;
}

size_t moe_packed_w1_bytes(int E, int H, int I) {
  if (I <= 0) return 0;
  return moe_packed_weight_bytes(E, 2 * I, H);
}

static moe_status_t launch_pack(const void* src, void* dst, int E, int N, int K, int mode, int I,
                                void* stream) {
  int cus;
  moe_status_t st = ensure_init(&cus);
  if (st != MOE_OK) return st;
  dim3 grid(K / 64, (N + 255) / 256, E);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), N, K, mode, I);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t moe_pack_weight(const void* src, int E, int N, int K, int src_layout, void* dst,
                             void* stream) {
  if (!src || !dst) return MOE_ERR_NULL;
  if (E < 1 || N < 64 || N % 64 != 0 || K < 64 || K % 64 != 0) return MOE_ERR_SHAPE;
  if (src_layout != MOE_B_NK && src_layout != MOE_B_KN) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_ALIGN;
  return launch_pack(src, dst, E, N, K, src_layout == MOE_B_NK ? PACK_NK : PACK_KN, 0, stream);
}

size_t moe_packed_mx_weight_bytes(int E, int N, int K) {
  if (E <= 0 || N <= 0 || K <= 0) return 0;
  return (size_t)E * (size_t)((N + 255) / 256) * 256 * (size_t)K;
}

size_t moe_packed_mx_scale_bytes(int E, int N, int K) {
  return moe_packed_mx_weight_bytes(E, N, K) / 32;
}

moe_status_t moe_pack_weight_mx(const void* src, int E, int N, int K, int src_layout, void* dst_q,
                                void* dst_s, void* stream) {
  if (!src || !dst_q || !dst_s) return MOE_ERR_NULL;
  if (E < 1 || N < 64 || N % 64 != 0 || K < 128 || K % 128 != 0) return MOE_ERR_SHAPE;
  if (src_layout != MOE_B_NK && src_layout != MOE_B_KN) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(dst_q) || !aligned16(dst_s)) return MOE_ERR_ALIGN;
  int cus;
  moe_status_t st = ensure_init(&cus);
  if (st != MOE_OK) return st;
  dim3 grid(K / 128, (N + 255) / 256, E);
  hipLaunchKernelGGL(pack_mx_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint16_t*>(src), static_cast<uint8_t*>(dst_q),
                     static_cast<uint8_t*>(dst_s), N, K, src_layout == MOE_B_KN ? 1 : 0, 0);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t moe_repack_gate_up_mx(const void* w1, int E, int H, int I, void* dst_q, void* dst_s,
                                   void* stream) {
  if (!w1 || !dst_q || !dst_s) return MOE_ERR_NULL;
  if (E < 1 || H < 128 || H % 128 != 0 || I < 64 || I % 64 != 0) return MOE_ERR_SHAPE;
  if (!aligned16(w1) || !aligned16(dst_q) || !aligned16(dst_s)) return MOE_ERR_ALIGN;
  int cus;
  moe_status_t st = ensure_init(&cus);
  if (st != MOE_OK) return st;
  dim3 grid(H / 128, (2 * I + 255) / 256, E);
  hipLaunchKernelGGL(pack_mx_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint16_t*>(w1), static_cast<uint8_t*>(dst_q),
                     static_cast<uint8_t*>(dst_s), 2 * I, H, 1, I);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t moe_repack_gate_up(const void* w1, int E, int H, int I, void* w1_packed,
                                void* stream) {
  if (!w1 || !w1_packed) return MOE_ERR_NULL;
  if (E < 1 || H < 64 || H % 64 != 0 || I < 64 || I % 64 != 0) return MOE_ERR_SHAPE;
  if (!aligned16(w1) || !aligned16(w1_packed)) return MOE_ERR_ALIGN;
  return launch_pack(w1, w1_packed, E, 2 * I, H, PACK_GATEUP, I, stream);
}

moe_status_t moe_unpack_gate_up(const void* w1_packed, int E, int H, int I, void* w1,
                                void* stream) {
  if (!w1 || !w1_packed) return MOE_ERR_NULL;
  if (E < 1 || H < 64 || H % 64 != 0 || I < 64 || I % 64 != 0) return MOE_ERR_SHAPE;
  if (!aligned16(w1) || !aligned16(w1_packed)) return MOE_ERR_ALIGN;
  return launch_pack(w1_packed, w1, E, 2 * I, H, UNPACK_GATEUP, I, stream);
}

moe_status_t moe_route_group(const float* logits, const int32_t* topk_ids, int T, int E, int k,
                             int32_t* topk_ids_out, int32_t* counts, int32_t* offsets,
                             int32_t* dst, int32_t* src, const void* x, int H, void* xg,
                             void* stream) {
  if ((logits == nullptr) == (topk_ids == nullptr)) return MOE_ERR_NULL;
  if (!topk_ids_out || !counts || !offsets || !dst || !src) return MOE_ERR_NULL;
  if ((x == nullptr) != (xg == nullptr)) return MOE_ERR_NULL;
  if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > 16 || k > E) return MOE_ERR_SHAPE;
  if ((long long)T * k >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (x && (H < 8 || H % 8 != 0)) return MOE_ERR_SHAPE;
  if (x && (!aligned16(x) || !aligned16(xg))) return MOE_ERR_ALIGN;
  int cus;
  moe_status_t st = ensure_init(&cus);
  if (st != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int TK = T * k;
  if (logits) {
    if (T > 0) {
      // one token per 16, 32 or 64 lanes
      const int L = E <= 16 ? 16 : (E <= 32 ? 32 : 64);
      const int per_block = 4 * (64 / L);
      const dim3 grid((T + per_block - 1) / per_block);
      if (L == 16)
        hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, s, logits, T, E, k, topk_ids_out);
      else if (L == 32)
        hipLaunchKernelGGL(topk_kernel<32>, grid, dim3(256), 0, s, logits, T, E, k, topk_ids_out);
      else
        hipLaunchKernelGGL(topk_kernel<64>, grid, dim3(256), 0, s, logits, T, E, k, topk_ids_out);
    }
  } else if (topk_ids != topk_ids_out && TK > 0) {
    if (hipMemcpyAsync(topk_ids_out, topk_ids, (size_t)TK * 4, hipMemcpyDeviceToDevice, s) !=
        hipSuccess)
      return MOE_ERR_LAUNCH;
  }
  // chunks of C pairs (C >= 2E, so that the per-chunk counts fit in src; see
  // group_count_kernel)
  int C = 1024;
  while (C < 2 * E) C *= 2;
  const int nchunks = (TK + C - 1) / C;
  if (nchunks > 1) {
    hipLaunchKernelGGL(group_count_kernel, dim3(nchunks), dim3(256), 0, s, topk_ids_out, TK, E, C, src);
    hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), 0, s, nchunks, E, src, counts, offsets);
  }
  // (with no pairs the single rank workgroup still writes zero counts)
  hipLaunchKernelGGL(group_rank_kernel, dim3(nchunks > 1 ? nchunks : 1), dim3(256), 0, s,
                     topk_ids_out, TK, E, C, nchunks > 1 ? src : nullptr, dst, counts, offsets);
  if (TK > 0) {
    const int grid = min((TK + 3) / 4, cus * 32);   // 4 pairs (one per wave) per workgroup step
    hipLaunchKernelGGL(group_scatter_kernel, dim3(grid), dim3(256), 0, s, topk_ids_out, TK, k, E, dst,
                       offsets, src, static_cast<const uint16_t*>(x), H, static_cast<uint16_t*>(xg));
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t moe_group_gemm_glu_fwd(const void* xg, const moe_groups_t* groups,
                                    const void* w1_packed, int H, int I,
                                    const moe_epilogue_t* ep, void* y, void* preact,
                                    const moe_mx_out_t* mx, int cu_margin, void* stream) {
  moe_status_t st = check_groups(groups);
  if (st != MOE_OK) return st;
  if (!xg || !w1_packed || !ep) return MOE_ERR_NULL;
  if ((st = check_mx(mx)) != MOE_OK) return st;
  if (H < 64 || H % 64 != 0 || I < 64 || I % 64 != 0) return MOE_ERR_SHAPE;
  if (ep->gated != 0 && ep->gated != 1) return MOE_ERR_UNSUPPORTED;
  const bool gated = ep->gated == 1;
  if (!aligned16(xg) || !aligned16(w1_packed) || (y && !aligned16(y)) ||
      (preact && !aligned16(preact)))
    return MOE_ERR_ALIGN;
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = fill_epilogue(ep, &a.ep)) != MOE_OK) return st;
  int cus;
  if ((st = ensure_init(&cus)) != MOE_OK) return st;
  fill_groups(&a, groups);
  a.A = static_cast<const uint16_t*>(xg);
  a.B = static_cast<const uint16_t*>(w1_packed);
  // gated: the gate/up-repacked W1 (N = 2I packed columns); non-gated: W1
  // [E][H][I] packed by moe_pack_weight (N = I plain columns)
  a.b_estride = gated ? (long long)moe_packed_w1_bytes(1, H, I) / 2
                      : (long long)moe_packed_weight_bytes(1, I, H) / 2;
  a.ldb = H;
  a.N = gated ? 2 * I : I;
  a.K = H;
  a.I = I;
  a.C = static_cast<uint16_t*>(y);
  a.preact = static_cast<uint16_t*>(preact);
  fill_mx(&a, mx, I, groups);
  a.ntiles_n = (a.N + GM_BN - 1) / GM_BN;
  int grid = persistent_grid(cus, cu_margin, groups->M_cap, groups->E, a.ntiles_n);
  const int kind = !gated ? KIND_ACT : (a.row_q || a.col_q) ? KIND_GLU_MXO : KIND_GLU;
  return launch_activation_kernel(kind, a, grid, (hipStream_t)stream);
}

moe_status_t moe_group_gemm_glu_fwd_mx(const moe_operand_t* xg, const moe_groups_t* groups,
                                       const moe_operand_t* w1, int H, int I,
                                       const moe_epilogue_t* ep, void* y, void* preact,
                                       const moe_mx_out_t* mx, int cu_margin, void* stream) {
  moe_status_t st = check_groups(groups);
  if (st != MOE_OK) return st;
  if (!xg || !w1 || !ep || !xg->data || !xg->scales || !w1->data || !w1->scales) return MOE_ERR_NULL;
  if ((st = check_mx(mx)) != MOE_OK) return st;
  if (H < 128 || H % 128 != 0 || I < 64 || I % 64 != 0) return MOE_ERR_SHAPE;
  if (ep->gated != 1 || xg->dtype != MOE_DT_MXFP8 || w1->dtype != MOE_DT_MXFP8 ||
      w1->layout != MOE_B_PACKED)
    return MOE_ERR_UNSUPPORTED;
  if (!aligned16(xg->data) || !aligned16(xg->scales) || !aligned16(w1->data) ||
      !aligned16(w1->scales) || (y && !aligned16(y)) || (preact && !aligned16(preact)))
    return MOE_ERR_ALIGN;
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = fill_epilogue(ep, &a.ep)) != MOE_OK) return st;
  int cus;
  if ((st = ensure_init(&cus)) != MOE_OK) return st;
  fill_groups(&a, groups);
  a.A = static_cast<const uint16_t*>(xg->data);
  a.a_scales = xg->scales;
  a.B = static_cast<const uint16_t*>(w1->data);
  a.b_scales = w1->scales;
  a.b_estride = (long long)moe_packed_mx_weight_bytes(1, 2 * I, H);   // bytes = elements
  a.ldb = H;
  a.N = 2 * I;
  a.K = H;
  a.I = I;
  a.C = static_cast<uint16_t*>(y);
  a.preact = static_cast<uint16_t*>(preact);
  fill_mx(&a, mx, I, groups);
  a.ntiles_n = (2 * I + GM_BN - 1) / GM_BN;
  int grid = persistent_grid(cus, cu_margin, groups->M_cap, groups->E, a.ntiles_n);
  return launch_activation_kernel((a.row_q || a.col_q) ? KIND_MXIN_GLU_MXO : KIND_MXIN_GLU, a,
                                  grid, (hipStream_t)stream);
}

moe_status_t moe_group_gemm_dglu_bwd(const void* dy2, const moe_operand_t* w2, int H, int I,
                                     const moe_groups_t* groups, const void* preact,
                                     const moe_epilogue_t* ep, void* dgu,
                                     const moe_mx_out_t* mx, int cu_margin, void* stream) {
  moe_status_t st = check_groups(groups);
  if (st != MOE_OK) return st;
  if (!dy2 || !w2 || !w2->data || !preact || !ep) return MOE_ERR_NULL;
  if ((st = check_mx(mx)) != MOE_OK) return st;
  if (H < 64 || H % 64 != 0 || I < 64 || I % 64 != 0) return MOE_ERR_SHAPE;
  if ((ep->gated != 0 && ep->gated != 1) || w2->dtype != MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
  const bool gated = ep->gated == 1;
  if (!gated && (ep->dbias_out || ep->drow_scale_out)) return MOE_ERR_UNSUPPORTED;
  if (w2->layout != MOE_B_NK && w2->layout != MOE_B_PACKED) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(dy2) || !aligned16(w2->data) || !aligned16(preact) || (dgu && !aligned16(dgu)))
    return MOE_ERR_ALIGN;
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = fill_epilogue(ep, &a.ep)) != MOE_OK) return st;
  a.ep.bias = nullptr;
  int cus;
  if ((st = ensure_init(&cus)) != MOE_OK) return st;
  fill_groups(&a, groups);
  a.A = static_cast<const uint16_t*>(dy2);
  a.B = static_cast<const uint16_t*>(w2->data);  // W2_e [I][H] = W2_e^T stored [N=I][K=H]
  const bool w2_packed = w2->layout == MOE_B_PACKED;
  a.b_estride = w2_packed ? (long long)moe_packed_weight_bytes(1, I, H) / 2 : (long long)I * H;
  a.ldb = H;
  a.N = I;
  a.K = H;
  a.I = I;
  a.C = static_cast<uint16_t*>(dgu);
  a.preact = const_cast<uint16_t*>(static_cast<const uint16_t*>(preact));
  fill_mx(&a, mx, gated ? 2 * I : I, groups);
  a.ntiles_n = (I + GM_BN - 1) / GM_BN;
  int grid = persistent_grid(cus, cu_margin, groups->M_cap, groups->E, a.ntiles_n);
  const bool grads = a.ep.dbias_out || a.ep.drs_out;
  const int kind = !gated ? (w2_packed ? KIND_DACT_PACKED : KIND_DACT_NK)
                   : grads ? (w2_packed ? KIND_DGLU_G_PACKED : KIND_DGLU_G_NK)
                           : (w2_packed ? KIND_DGLU_PACKED : KIND_DGLU_NK);
  return launch_activation_kernel(kind, a, grid, (hipStream_t)stream);
}

moe_status_t moe_group_gemm_quant(const moe_operand_t* a_op, const moe_operand_t* b_op, int N,
                                  int K, const moe_groups_t* groups, void* c_bf16,
                                  const moe_mx_out_t* mx, int cu_margin, void* stream) {
  moe_status_t st = check_groups(groups);
  if (st != MOE_OK) return st;
  if (!a_op || !b_op || !a_op->data || !b_op->data) return MOE_ERR_NULL;
  if ((st = check_mx(mx)) != MOE_OK) return st;
  if (N < 64 || N % 64 != 0 || K < 64 || K % 64 != 0) return MOE_ERR_SHAPE;
  const bool a_e5 = a_op->dtype == MOE_DT_MXFP8_E5M2;
  const bool mx_in = a_op->dtype == MOE_DT_MXFP8 || a_e5 || b_op->dtype != MOE_DT_BF16;
  if (mx_in) {   // MXFP8 (A e4m3 or e5m2) x MXFP8 e4m3 only, weight from moe_pack_weight_mx
    if ((a_op->dtype != MOE_DT_MXFP8 && !a_e5) || b_op->dtype != MOE_DT_MXFP8 ||
        b_op->layout != MOE_B_PACKED)
      return MOE_ERR_UNSUPPORTED;
    if (!a_op->scales || !b_op->scales) return MOE_ERR_NULL;
    if (K % 128 != 0) return MOE_ERR_SHAPE;
    if (!aligned16(a_op->scales) || !aligned16(b_op->scales)) return MOE_ERR_ALIGN;
  } else if (a_op->dtype != MOE_DT_BF16 || b_op->dtype != MOE_DT_BF16) {
    return MOE_ERR_UNSUPPORTED;
  }
  if (!aligned16(a_op->data) || !aligned16(b_op->data) || (c_bf16 && !aligned16(c_bf16)))
    return MOE_ERR_ALIGN;
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  int cus;
  if ((st = ensure_init(&cus)) != MOE_OK) return st;
  fill_groups(&a, groups);
  a.A = static_cast<const uint16_t*>(a_op->data);
  a.B = static_cast<const uint16_t*>(b_op->data);
  a.N = N;
  a.K = K;
  a.C = static_cast<uint16_t*>(c_bf16);
  fill_mx(&a, mx, N, groups);
  a.ntiles_n = (N + GM_BN - 1) / GM_BN;
  if (mx_in) {
    a.a_scales = static_cast<const uint8_t*>(a_op->scales);
    a.b_scales = static_cast<const uint8_t*>(b_op->scales);
    a.ldb = K;
    a.b_estride = (long long)moe_packed_mx_weight_bytes(1, N, K);   // bytes = elements
    int grid = persistent_grid(cus, cu_margin, groups->M_cap, groups->E, a.ntiles_n);
    return launch_group_gemm_mx(a, a_e5, grid, (hipStream_t)stream);
  }
  int blay;
  switch (b_op->layout) {
    case MOE_B_KN: blay = BL_KN; a.ldb = N; a.b_estride = (long long)K * N; break;
    case MOE_B_NK: blay = BL_NK; a.ldb = K; a.b_estride = (long long)N * K; break;
    case MOE_B_PACKED:
      blay = BL_PACKED; a.ldb = K; a.b_estride = (long long)moe_packed_weight_bytes(1, N, K) / 2;
      break;
    default: return MOE_ERR_UNSUPPORTED;
  }
  int grid = persistent_grid(cus, cu_margin, groups->M_cap, groups->E, a.ntiles_n);
  if (blay == BL_PACKED) return launch_group_gemm_bwd(EPI_STORE, blay, a, grid, (hipStream_t)stream);
  return launch_group_gemm_fwd(EPI_STORE, blay, a, grid, (hipStream_t)stream);
}

moe_status_t moe_group_gemm_wgrad(const void* a, const void* b, int P, int Q,
                                  const moe_groups_t* groups, float* c, int accumulate,
                                  int cu_margin, void* stream) {
  moe_status_t st = check_groups(groups);
  if (st != MOE_OK) return st;
  if (!a || !b || !c) return MOE_ERR_NULL;
  if (P < 64 || P % 64 != 0 || Q < 64 || Q % 64 != 0) return MOE_ERR_SHAPE;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return MOE_ERR_ALIGN;
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  int cus;
  if ((st = ensure_init(&cus)) != MOE_OK) return st;
  fill_groups(&g, groups);
  g.A = static_cast<const uint16_t*>(a);
  g.B = static_cast<const uint16_t*>(b);
  g.ldb = Q;
  g.N = Q;
  g.K = 64;                       // unused: each tile reduces over its group's rows
  g.wg_P = P;
  g.ntiles_m = (P + GM_BM - 1) / GM_BM;
  g.ntiles_n = (Q + GM_BN - 1) / GM_BN;
  g.Cf = c;
  g.accumulate = accumulate ? 1 : 0;
  int usable = cus - (cu_margin > 0 ? cu_margin : 0);
  if (usable < 1) usable = 1;
  const long long tiles = (long long)groups->E * g.ntiles_m * g.ntiles_n;
  const int grid = (int)(tiles < usable ? tiles : usable);
  return launch_group_gemm_wgrad(g, grid, (hipStream_t)stream);
}

moe_status_t moe_group_gemm_wgrad_mx(const moe_operand_t* a, const moe_operand_t* b, int P, int Q,
                                     const moe_groups_t* groups, float* c, int accumulate,
                                     int cu_margin, void* stream) {
  moe_status_t st = check_groups(groups);
  if (st != MOE_OK) return st;
  if (!a || !b || !c || !a->data || !b->data || !a->scales || !b->scales) return MOE_ERR_NULL;
  auto is_mx = [](int dt) { return dt == MOE_DT_MXFP8 || dt == MOE_DT_MXFP8_E5M2; };
  if (!is_mx(a->dtype) || !is_mx(b->dtype)) return MOE_ERR_UNSUPPORTED;
  if (P < 64 || P % 64 != 0 || Q < 64 || Q % 64 != 0) return MOE_ERR_SHAPE;
  if (!aligned16(a->data) || !aligned16(b->data) || !aligned4(a->scales) || !aligned4(b->scales) ||
      !aligned16(c))
    return MOE_ERR_ALIGN;
  const int S = 4 * ((groups->M_cap + 127) / 128 + groups->E);   // slots per copied column
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  int cus;
  if ((st = ensure_init(&cus)) != MOE_OK) return st;
  fill_groups(&g, groups);
  g.A = static_cast<const uint16_t*>(a->data);
  g.B = static_cast<const uint16_t*>(b->data);
  g.a_scales = a->scales;
  g.b_scales = b->scales;
  g.K = 32 * S;                   // bytes per copied column (row of each operand)
  g.ldb = 32 * S;
  g.N = Q;
  g.wg_P = P;
  g.ntiles_m = (P + GM_BM - 1) / GM_BM;
  g.ntiles_n = (Q + GM_BN - 1) / GM_BN;
  g.Cf = c;
  g.accumulate = accumulate ? 1 : 0;
  int usable = cus - (cu_margin > 0 ? cu_margin : 0);
  if (usable < 1) usable = 1;
  const long long tiles = (long long)groups->E * g.ntiles_m * g.ntiles_n;
  const int grid = (int)(tiles < usable ? tiles : usable);
  return launch_group_gemm_wgrad_mx(g, a->dtype == MOE_DT_MXFP8_E5M2, b->dtype == MOE_DT_MXFP8_E5M2,
                                    grid, (hipStream_t)stream);
}

moe_status_t moe_glu_unfused(const void* z, const moe_groups_t* groups, int I,
                             const moe_epilogue_t* ep, void* y, void* stream) {
  moe_status_t st = check_groups(groups);
  if (st != MOE_OK) return st;
  if (!z || !y || !ep) return MOE_ERR_NULL;
  if (I < 64 || I % 64 != 0) return MOE_ERR_SHAPE;
  if (ep->gated != 1) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(z) || !aligned16(y)) return MOE_ERR_ALIGN;
  EpiParams e;
  if ((st = fill_epilogue(ep, &e)) != MOE_OK) return st;
  int cus;
  if ((st = ensure_init(&cus)) != MOE_OK) return st;
  hipLaunchKernelGGL(glu_unfused_kernel, dim3(cus * 8), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint16_t*>(z), groups->counts, groups->E, groups->M_cap, I,
                     e, static_cast<uint16_t*>(y));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t moe_dglu_unfused(const void* g, const void* z, const moe_groups_t* groups, int I,
                              const moe_epilogue_t* ep, void* dgu, void* stream) {
  moe_status_t st = check_groups(groups);
  if (st != MOE_OK) return st;
  if (!g || !z || !dgu || !ep) return MOE_ERR_NULL;
  if (I < 64 || I % 64 != 0) return MOE_ERR_SHAPE;
  if (ep->gated != 1) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(g) || !aligned16(z) || !aligned16(dgu)) return MOE_ERR_ALIGN;
  EpiParams e;
  if ((st = fill_epilogue(ep, &e)) != MOE_OK) return st;
  int cus;
  if ((st = ensure_init(&cus)) != MOE_OK) return st;
  hipLaunchKernelGGL(dglu_unfused_kernel, dim3(cus * 8), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(z), groups->counts,
                     groups->E, groups->M_cap, I, e, static_cast<uint16_t*>(dgu));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t moe_mxfp8_quantize(const void* v, int R, int C, const moe_groups_t* groups,
                                const moe_mx_out_t* mx, void* stream) {
  if (!v || !mx) return MOE_ERR_NULL;
  moe_status_t st = check_mx(mx);
  if (st != MOE_OK) return st;
  if (groups && (st = check_groups(groups)) != MOE_OK) return st;
  if (groups && groups->M_cap != R) return MOE_ERR_SHAPE;
  if (R < 0 || C < 32 || C % 32 != 0) return MOE_ERR_SHAPE;
  if (!aligned16(v)) return MOE_ERR_ALIGN;
  int cus;
  if ((st = ensure_init(&cus)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int* counts = groups ? groups->counts : nullptr;
  const int E = groups ? groups->E : 0;
  if (mx->row_q && R > 0) {
    hipLaunchKernelGGL(mx_rows_kernel, dim3(cus * 8), dim3(256), 0, s,
                       static_cast<const uint16_t*>(v), R, C, counts, E, mx->row_q, mx->row_s,
                       mx->e5m2);
  }
  if (mx->col_q && R > 0) {
    const int Eg = groups ? E : 0;
    int s_ld = mx->col_blocked ? 4 * ((R + 127) / 128 + Eg) : (R + 31) / 32 + Eg;
    if (mx->col_blocked) {   // LDS-staged, 256 rows x 64 columns per item
      const long long items = (long long)((R + 255) / 256 + Eg) * ((C + 63) / 64);
      const int grid = (int)(items < (long long)cus * 6 ? items : (long long)cus * 6);
      hipLaunchKernelGGL(mx_cols_ktiled_kernel, dim3(grid), dim3(256), 0, s,
                         static_cast<const uint16_t*>(v), R, C, counts, E, mx->col_q, mx->col_s, s_ld,
                         mx->e5m2);
    } else {
      long long by = s_ld;
      int gy = (int)(by < 65535 ? by : 65535);
      hipLaunchKernelGGL(mx_cols_kernel, dim3((C + 255) / 256, gy), dim3(256), 0, s,
                         static_cast<const uint16_t*>(v), R, C, counts, E, mx->col_q, mx->col_s, s_ld,
                         mx->e5m2, mx->col_blocked);
    }
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // extern "C"
