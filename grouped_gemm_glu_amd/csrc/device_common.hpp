// Device helpers shared by the library's kernels (gfx950 / CDNA4, wave64):
// bf16 and e4m3fn encoders, the E8M0 block-scale rule, the GLU activations and
// their derivatives, and the per-workgroup scan of the device-resident expert
// counts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMxBlock = 32;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; overflow rounds to +-inf and
// NaN stays NaN (gfx950 converts in hardware: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- MXFP8
// Block-scale exponent for a block maximum (OCP MX, E8M0 scale): the smallest
// E with amax / 2^E <= vmax = 1.75 * 2^vexp, the largest element value (e4m3fn:
// 448, vexp 8; e5m2: 57344, vexp 15), clamped to [-127, 127]: amax = 1.f *
// 2^e needs 2^(e - vexp) when f <= 1.75, else 2^(e - vexp + 1).  Zero or an
// fp32 subnormal amax gives -127, a non-finite one 128 (NaN scale).
__device__ __forceinline__ int mx_scale_exponent(float amax, int vexp = 8) {
  uint32_t u = __float_as_uint(amax) & 0x7FFFFFFFu;
  if (u >= 0x7F800000u) return 128;
  uint32_t ebits = u >> 23;
  if (ebits == 0) return -127;                 // zero or subnormal: ceil(log2(amax/vmax)) < -127
  int E = static_cast<int>(ebits) - 127 - vexp + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

__device__ __forceinline__ uint8_t e8m0_byte(int E) {
  return E >= 128 ? static_cast<uint8_t>(0xFF) : static_cast<uint8_t>(E + 127);
}

// fp32 -> e4m3fn code, round to nearest, ties to even, saturating at 448; the
// sign bit is kept (also on zero).  Integer arithmetic on the fp32 bits: the
// three kept mantissa bits are rounded on the 20 dropped ones; below 2^-6 the
// value is a multiple of the subnormal quantum 2^-9, rounded by rintf (RNE).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;    // NaN
  uint32_t code;
  if (a < 0x3C800000u) {                       // |x| < 2^-6
    code = static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.0f));  // 0..8, 8 == 2^-6
  } else {
    uint32_t e = (a >> 23) - 120u;             // biased e4m3 exponent (bias 7)
    uint32_t keep = (a >> 20) & 7u;
    uint32_t rem = a & 0xFFFFFu;
    uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (keep & 1u));
    code = (e << 3) + keep + up;
    if (code > 0x7Eu || e > 15u) code = 0x7Eu;
  }
  return sign | code;
}

// Four fp32 values -> four e4m3fn codes (byte k = value k) with the hardware
// conversion v_cvt_pk_fp8_f32 (round to nearest even; identical to
// f32_to_e4m3 for |x| <= 448, checked exhaustively over the bf16 values).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// Four fp32 values -> four e5m2 codes (byte k = value k) with v_cvt_pk_bf8_f32
// (round to nearest even; the callers keep |x| <= 57344).
__device__ __forceinline__ uint32_t e5m2x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_bf8_f32(c, d, lo, true));
}

// Quantises one 32-value MX block (nvalid of the values real; the others must
// be finite and are encoded too) to e4m3fn or, with e5, e5m2 codes (4 per
// word of w) and returns its E8M0 scale byte.  A NaN among the valid values
// makes the whole block NaN (scale 0xFF, every code 0x7F).
__device__ __forceinline__ uint8_t mx_quant32(const float* v, int nvalid, uint32_t* w, bool e5) {
  float amax = 0.0f;
  bool has_nan = false;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (i < nvalid) {
      amax = fmaxf(amax, fabsf(v[i]));   // fmaxf drops NaN: tracked separately
      if (v[i] != v[i]) has_nan = true;
    }
  const int E = has_nan ? 128 : mx_scale_exponent(amax, e5 ? 15 : 8);
  if (E == 128) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0x7F7F7F7Fu;
    return 0xFF;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = ldexpf(v[4 * i], -E), b = ldexpf(v[4 * i + 1], -E);
    const float c = ldexpf(v[4 * i + 2], -E), d = ldexpf(v[4 * i + 3], -E);
    w[i] = e5 ? e5m2x4(a, b, c, d) : e4m3x4(a, b, c, d);
  }
  return e8m0_byte(E);
}

// One slot of the K-tiled transposed layout: 32 codes to a 16-byte aligned
// dst, the codes of rows from nvalid on (past the group's last row) zero.
// NT: with the non-temporal hint (for callers whose neighbouring lanes write
// the neighbouring slots, so that the lines are written whole).
template <bool NT = false>
__device__ __forceinline__ void store_codes32_slot(uint8_t* dst, const uint32_t* w, int nvalid) {
  uint32_t m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = nvalid - 4 * i;   // valid bytes of word i
    m[i] = k >= 4 ? w[i] : (k <= 0 ? 0u : (w[i] & ((1u << (8 * k)) - 1u)));
  }
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  v4u* d = reinterpret_cast<v4u*>(dst);
  const v4u lo = {m[0], m[1], m[2], m[3]}, hi = {m[4], m[5], m[6], m[7]};
  if constexpr (NT) {
    __builtin_nontemporal_store(lo, d);
    __builtin_nontemporal_store(hi, d + 1);
  } else {
    d[0] = lo;
    d[1] = hi;
  }
}

// 32 codes to a 16-byte aligned dst with the non-temporal hint (row-wise
// copies, where 8 neighbouring lanes write one 256-byte run).
__device__ __forceinline__ void store_codes32_aligned_nt(uint8_t* dst, const uint32_t* w) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  v4u* d = reinterpret_cast<v4u*>(dst);
  const v4u lo = {w[0], w[1], w[2], w[3]}, hi = {w[4], w[5], w[6], w[7]};
  __builtin_nontemporal_store(lo, d);
  __builtin_nontemporal_store(hi, d + 1);
}

// 32 codes (w, little-endian) to dst, which has any alignment.  A full block
// at a non-4-byte-aligned address (a transposed block starting at a group's
// first row) goes out as h = 4 - (dst % 4) head bytes, 7 aligned dwords
// (each two neighbouring words of w funnel-shifted by h bytes) and 4 - h tail
// bytes, instead of 32 byte stores; a partial block (a group's last) byte by
// byte.
__device__ __forceinline__ void store_codes32(uint8_t* dst, const uint32_t* w, int nvalid) {
  uintptr_t a = reinterpret_cast<uintptr_t>(dst);
  auto byte = [&](int i) { return static_cast<uint8_t>(w[i >> 2] >> (8 * (i & 3))); };
  if (nvalid == 32 && (a & 15) == 0) {
    uint4* d = reinterpret_cast<uint4*>(dst);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else if (nvalid == 32 && (a & 3) == 0) {
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = w[i];
  } else if (nvalid == 32) {
    const int h = 4 - (int)(a & 3);   // 1..3
    for (int i = 0; i < h; ++i) dst[i] = byte(i);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + h);
    const uint32_t sr = 8u * (uint32_t)h, sl = 32u - sr;
#pragma unroll
    for (int k = 0; k < 7; ++k) d[k] = (w[k] >> sr) | (w[k + 1] << sl);
    for (int i = h + 28; i < 32; ++i) dst[i] = byte(i);
  } else {
    for (int i = 0; i < nvalid; ++i) dst[i] = byte(i);
  }
}

// ---------------------------------------------------------------- activations
enum { ACT_SWIGLU = 0, ACT_GEGLU = 1, ACT_GEGLU_TANH = 2, ACT_SRELU = 3 };

// 1 / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp each;
// the results are rounded to bf16).
__device__ __forceinline__ float sigmoidf_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// The Gaussian CDF as 0.5 erfc(-g / sqrt 2) and the tanh form's 0.5 (1 +
// tanh u) as sigmoid(2u): the same functions as 0.5 (1 + erf) and 0.5 (1 +
// tanh), but without their cancellation for negative g, so a(g) and a'(g)
// keep their relative accuracy in the tail (they set MXFP8 block scales of
// the outputs, which follow the block's largest value, however small).
__device__ __forceinline__ float gauss_cdf(float g) { return 0.5f * erfcf(g * -0.70710678118654752f); }
__device__ __forceinline__ float gelu_tanh_u(float g) {
  return 0.79788456080286536f * (g + 0.044715f * g * g * g);
}

// a(g) for a compile-time activation (epilogues dispatch once per launch,
// not per element).
template <int ACT>
__device__ __forceinline__ float act_fwd_t(float g, float alpha) {
  if constexpr (ACT == ACT_SWIGLU) {
    return g * sigmoidf_fast(alpha * g);
  } else if constexpr (ACT == ACT_GEGLU) {
    return g * gauss_cdf(g);
  } else if constexpr (ACT == ACT_GEGLU_TANH) {
    return g * sigmoidf_fast(2.0f * gelu_tanh_u(g));
  } else {
    const float r = fmaxf(g, 0.0f);
    return r * r;
  }
}

__device__ __forceinline__ float act_fwd(int act, float g, float alpha) {
  switch (act) {
    case ACT_SWIGLU: return act_fwd_t<ACT_SWIGLU>(g, alpha);
    case ACT_GEGLU: return act_fwd_t<ACT_GEGLU>(g, alpha);
    case ACT_GEGLU_TANH: return act_fwd_t<ACT_GEGLU_TANH>(g, alpha);
    default: return act_fwd_t<ACT_SRELU>(g, alpha);
  }
}

// a(g) and a'(g) for a compile-time activation.
template <int ACT>
__device__ __forceinline__ void act_fwd_bwd_t(float g, float alpha, float& a, float& da) {
  if constexpr (ACT == ACT_SWIGLU) {
    const float s = sigmoidf_fast(alpha * g);
    a = g * s;
    da = s * (1.0f + alpha * g * (1.0f - s));
  } else if constexpr (ACT == ACT_GEGLU) {
    const float cdf = gauss_cdf(g);
    const float pdf = 0.39894228040143268f * __expf(-0.5f * g * g);
    a = g * cdf;
    da = cdf + g * pdf;
  } else if constexpr (ACT == ACT_GEGLU_TANH) {
    // a = g s, s = sigmoid(2u) = (1 + tanh u) / 2; 1 - tanh^2 u = 4 s (1 - s)
    const float s = sigmoidf_fast(2.0f * gelu_tanh_u(g));
    const float du = 0.79788456080286536f * (1.0f + 3.0f * 0.044715f * g * g);
    a = g * s;
    da = s + 2.0f * g * s * (1.0f - s) * du;
  } else {
    const float r = fmaxf(g, 0.0f);
    a = r * r;
    da = 2.0f * r;
  }
}

// a(g) and a'(g) together (the backward epilogue needs both).
__device__ __forceinline__ void act_fwd_bwd(int act, float g, float alpha, float& a, float& da) {
  switch (act) {
    case ACT_SWIGLU: act_fwd_bwd_t<ACT_SWIGLU>(g, alpha, a, da); break;
    case ACT_GEGLU: act_fwd_bwd_t<ACT_GEGLU>(g, alpha, a, da); break;
    case ACT_GEGLU_TANH: act_fwd_bwd_t<ACT_GEGLU_TANH>(g, alpha, a, da); break;
    default: act_fwd_bwd_t<ACT_SRELU>(g, alpha, a, da); break;
  }
}

struct EpiParams {
  int act;
  float alpha;
  float gate_lo, gate_hi, up_lo, up_hi, up_offset;
  const uint16_t* bias;      // plain [E][2I] or null
  const float* row_scale;    // [M_cap] or null
  float* amax_out;           // raised atomically to an amax, or null
  uint32_t rht_signs;        // row signs of the 16-point rotation (bit i: row i)
  float* dbias_out;          // backward: [E][2I] += column sums of dgu, or null
  float* drs_out;            // backward: [M_cap] += d(row_scale), or null
};

// ---------------------------------------------------------------- group scan
// Per-workgroup view of the device-resident expert counts.  Every workgroup
// rebuilds it in LDS at kernel start (E <= 1024, a few hundred cycles), so no
// extra launch and no host readback is needed.  Counts are clamped: negative
// counts become 0 (status bit 0) and rows past M_cap are dropped (bit 1).
struct GroupScan {
  int row_off[kMaxExperts + 1];   // o_e of the clamped counts
  int tile_off[kMaxExperts + 1];  // prefix of full-height m-tiles per expert
  int half_off[kMaxExperts + 1];  // prefix of half-height m-tiles (0 or 1 per expert)
  int mxs_off[kMaxExperts + 1];   // MX column-scale slot of each group's first block
  long long wave_tmp[16];
  long long total_raw;
};

// Block-wide inclusive scan of one value per thread (NT threads, NT % 64 == 0).
template <int NT, typename T>
__device__ __forceinline__ T block_incl_scan(T v, long long* wave_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    T o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) wave_tmp[wave] = static_cast<long long>(v);
  __syncthreads();
  T add = 0;
  for (int w = 0; w < wave; ++w) add += static_cast<T>(wave_tmp[w]);
  __syncthreads();
  return v + add;
}

// Fills gs from counts[0..E) for m-tiles of BM rows.  With half_rows > 0 an
// expert's last m-tile counts as a half-height tile (half_off) when it holds
// 1 .. half_rows rows, else as a full one (tile_off); half_rows = 0 makes every
// m-tile full.  mxs_off: the first column-scale slot of each group, ceil(m/32)
// slots per group, or with mx_blocked 4 ceil(m/128) (the K-tiled layout).  NT threads, each owning up to kMaxExperts/NT consecutive
// experts.  The writer workgroup also stores the clamped offsets and the
// status bits.  gs is valid after the final barrier.
template <int NT>
__device__ void build_group_scan(GroupScan& gs, const int* __restrict__ counts, int E, int M_cap,
                                 int BM, int half_rows, int* offsets_out, int* status_out,
                                 bool writer, bool mx_blocked = false) {
  const int t = threadIdx.x;
  constexpr int PER = (kMaxExperts + NT - 1) / NT;
  int c[PER];
  long long raw_sum = 0;
  int bad_neg = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int e = t * PER + i;
    int v = (e < E) ? counts[e] : 0;
    if (v < 0) { bad_neg = 1; v = 0; }
    c[i] = v;
    raw_sum += v;
  }
  long long incl = block_incl_scan<NT, long long>(raw_sum, gs.wave_tmp);
  long long run = incl - raw_sum;  // exclusive prefix of the non-negative counts
  int mt_sum = 0, hf_sum = 0, mx_sum = 0;
  int mloc[PER];
  auto n_half = [&](int m) { const int r = m % BM; return (half_rows > 0 && r > 0 && r <= half_rows) ? 1 : 0; };
  auto n_full = [&](int m) { return (m + BM - 1) / BM - n_half(m); };
  auto n_mx = [&](int m) { return mx_blocked ? 4 * ((m + 127) >> 7) : (m + kMxBlock - 1) / kMxBlock; };
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int e = t * PER + i;
    long long room = (long long)M_cap - run;
    if (room < 0) room = 0;
    int m = (long long)c[i] < room ? c[i] : (int)room;
    mloc[i] = m;
    if (e < E) gs.row_off[e] = run < M_cap ? (int)run : M_cap;
    run += c[i];
    mt_sum += n_full(m);
    hf_sum += n_half(m);
    mx_sum += n_mx(m);
  }
  if (t == NT - 1) gs.total_raw = run;
  int mt_incl = block_incl_scan<NT, int>(mt_sum, gs.wave_tmp);
  int hf_incl = block_incl_scan<NT, int>(hf_sum, gs.wave_tmp);
  int mx_incl = block_incl_scan<NT, int>(mx_sum, gs.wave_tmp);
  int mt_run = mt_incl - mt_sum, hf_run = hf_incl - hf_sum, mx_run = mx_incl - mx_sum;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int e = t * PER + i;
    if (e < E) {
      gs.tile_off[e] = mt_run;
      gs.half_off[e] = hf_run;
      gs.mxs_off[e] = mx_run;
    }
    mt_run += n_full(mloc[i]);
    hf_run += n_half(mloc[i]);
    mx_run += n_mx(mloc[i]);
  }
  if (t == NT - 1) {
    gs.tile_off[E] = mt_run;
    gs.half_off[E] = hf_run;
    gs.mxs_off[E] = mx_run;
  }
  int neg_any = __syncthreads_or(bad_neg);
  if (t == 0) gs.row_off[E] = gs.total_raw < M_cap ? (int)gs.total_raw : M_cap;
  __syncthreads();
  if (writer) {
    if (offsets_out)
      for (int e = t; e <= E; e += NT) offsets_out[e] = gs.row_off[e];
    if (status_out && t == 0) {
      int st = (neg_any ? 1 : 0) | (gs.total_raw > M_cap ? 2 : 0);
      if (st) atomicOr(status_out, st);
    }
  }
}

}  // namespace moe
