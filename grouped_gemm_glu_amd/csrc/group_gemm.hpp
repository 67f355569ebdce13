// Persistent grouped GEMM for gfx950 with fused epilogues.
//
// One launch covers every expert.  The group sizes exist only in device
// memory ("Boosting MoE Training Throughput with Advanced Fusion Kernels",
// section "Eliminando la sincronización host-device"): each workgroup scans
// counts[E] into LDS, then walks global tile ids t = slot, slot + P, ... and
// decodes each into (expert, m-tile, n-tile) by binary search over the tile
// prefix.  Rows of one expert are contiguous ([MEGA] §4.3); the last m-tile of
// a group is partial and handled by clamped loads and masked stores ([MEGA]
// §5.3).
//
// Tile 256 x 256 x 64.  Every kernel but the weight gradients (gm_waves)
// runs 8 waves (two per SIMD) in a 4 x 2 grid of 64 x 128 sub-tiles: FC1,
// FC2, dX and dgrad + dGLU (with or without the parameter gradients), and
// the non-gated forms, on packed or K-contiguous plain weights as 4 x 8
// blocks of v_mfma_f32_16x16x32_bf16 (the dGLU's 128 x 128 quarter tiles:
// 32 x 64 per wave, 1 x 2 blocks of v_mfma_f32_32x32x16_bf16), the
// GroupGemm on N-contiguous plain weights as 2 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, MXFP8 operands as 2 x 4 blocks of the
// block-scaled 32 x 32 x 64; the weight gradients 4 waves in a 2 x 2 grid of
// 128 x 128 sub-tiles.  Operands are
// staged in LDS as [rows][128 bytes] (64 bf16 or 128 fp8 values), with the
// 16-byte chunk index XOR-swizzled by row bits 0..4 (swz_key) so that the
// fragment reads of both MFMA shapes are free of bank conflicts.  Two LDS
// stages filled by direct global -> LDS loads (buffer_load ... lds): the DMA
// of K-tile t + 2 is issued right after the barrier that frees its stage,
// spread over the MFMAs of the last k-step of K-tile t, whose fragments are
// already in registers, so the barrier does not drain the MFMA pipe.
//
// Epilogues (fused; the accumulators never go to HBM in fp32):
//   EPI_GLU   FC1: bias, clamp, activation * up, row scale -> bf16 y; optional
//             bf16 pre-activation; optional MXFP8 row-wise / transposed copies.
//   EPI_STORE plain bf16 output (FC2, dX) with optional MXFP8 copies.
//   EPI_DGLU  backward: reads the saved pre-activation, writes d(gate | up).
// Output tiles are staged in LDS and written with 16-byte coalesced stores.
#pragma once

#include <utility>

#include "device_common.hpp"

namespace moe {

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): loop
// bodies whose indices must be compile-time constants.
template <typename F, int... G>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, G...>) {
  (f(std::integral_constant<int, G>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

constexpr int GM_BM = 256;
constexpr int GM_BN = 256;
constexpr int GM_BK = 64;
constexpr int GM_TILE_BYTES = GM_BM * GM_BK * 2;              // one operand tile: 32 KB
constexpr int GM_STAGE_BYTES = 2 * GM_TILE_BYTES;             // A + B
constexpr int GM_MAIN_BYTES = 2 * GM_STAGE_BYTES;             // two stages: 128 KB
constexpr int GM_STG_LD_256 = 264;                            // staged row, 256 cols (+16 B pad)
constexpr int GM_STG_LD_128 = 136;                            // staged row, 128 cols (+16 B pad)
// Each of the two LDS stage arrays also holds one 128-row half of the staged
// output tile in the epilogue (rows 0..127 in array 0, 128..255 in array 1).
constexpr int GM_HALF_STG_BYTES = (GM_BM / 2) * GM_STG_LD_256 * 2;   // 66 KB
constexpr int GM_STAGE_ALLOC =
    GM_HALF_STG_BYTES > GM_STAGE_BYTES ? GM_HALF_STG_BYTES : GM_STAGE_BYTES;

// Staged output tile split over the two stage arrays by row halves: hr rows
// each (128 for a 256-row tile, 64 for a 128-row tile).
struct Stg {
  uint16_t* h0;
  uint16_t* h1;
  int ld;
  int hr = 128;
  __device__ __forceinline__ uint16_t* row(int r) const {
    return (r < hr ? h0 : h1) + (r < hr ? r : r - hr) * ld;
  }
  __device__ __forceinline__ int rows() const { return 2 * hr; }
};

// EPI_DGLU_G: EPI_DGLU that also adds the gradients of the epilogue's own
// parameters (bias, row scale); a kernel of its own, so that the plain
// backward epilogue keeps its register allocation.
// EPI_ACT / EPI_DACT: the non-gated activation (N = I columns, no gate/up
// pairs): forward y = a(z) * row_scale with z = acc + bias (z optionally
// saved), backward dz = G * row_scale * a'(z) from the saved z.
enum { EPI_GLU = 0, EPI_STORE = 1, EPI_DGLU = 2, EPI_GLU_MX = 3, EPI_WGRAD = 4, EPI_DGLU_G = 5,
       EPI_ACT = 6, EPI_DACT = 7 };
enum { BL_NK = 0, BL_KN = 1, BL_PACKED = 2 };
// operand element type: bf16, or MXFP8 (OCP e4m3 codes with one E8M0 scale
// per 32 consecutive K values, consumed by the block-scaled MFMA); AT_MX_A5:
// the same with e5m2 codes for A (a gradient) and e4m3 for B; AT_MX_B5 and
// AT_MX_AB5: e5m2 codes for B, or for both (weight gradients, where both
// operands are transposed MXFP8 copies of activations or gradients)
enum { AT_BF16 = 0, AT_MX = 1, AT_MX_A5 = 2, AT_MX_B5 = 3, AT_MX_AB5 = 4 };

// Waves per workgroup.  4: a 2 x 2 grid of waves, one per SIMD, each owning
// a 128 x 128 sub-tile.  8: a 4 x 2 grid of 64 x 128 sub-tiles, two waves per
// SIMD, so that one wave's MFMAs run while the other waits on its loads or at
// the stage barrier (the kernels on packed weights with bf16 or MXFP8 e4m3 /
// e5m2-A operands: 3-5% faster on the DeepSeek-V3-like share, same results
// bit for bit; the dGLU kernel with d(bias) / d(row_scale) 6.5% faster once
// its epilogue stopped spilling, the non-gated FC1 14% and its backward 3%;
// on K-contiguous plain weights, whose B DMA is row-strided like A's, dX 10%
// and dgrad's GEMM 3%; on N-contiguous ones FC2 3%).
// The weight gradients keep 4 waves: their 128 x 128 fp32 sub-tile per wave
// and its staging need the register file of one wave per SIMD (8 waves
// measured +-0.5%).
constexpr int gm_waves(int epi, int /*blay*/, int /*at*/) { return epi == EPI_WGRAD ? 4 : 8; }

struct GemmArgs {
  const uint16_t* A;        // [M_cap][K] grouped rows, K contiguous
  const uint16_t* B;        // expert e at B + e * b_estride
  long long b_estride;      // elements between experts
  int ldb;                  // elements between consecutive rows of the stored B
  int M_cap, N, K;          // N = GEMM output columns (FC1: 2I, packed order)
  int I;                    // GLU / dGLU intermediate size
  const int* counts;
  int E;
  int* offsets_out;
  int* status_out;
  EpiParams ep;
  uint16_t* C;              // GLU: y [M_cap][I]; STORE: [M_cap][N]; DGLU: dgu [M_cap][2I]
  uint16_t* preact;         // GLU: optional output; DGLU: input; [M_cap][2I] plain order
  uint8_t* row_q;
  uint8_t* row_s;
  uint8_t* col_q;
  uint8_t* col_s;
  int mx_cols;              // columns of the quantised output (row length of row_q)
  int mx_e5;                // 1: the quantised copies hold e5m2 codes, 0: e4m3fn
  int col_blocked;          // 1: transposed copy in the K-tiled layout (slots of 32 rows)
  int col_s_ld;             // slots per column: ceil(M_cap/32) + E, or 4 (ceil(M_cap/128) + E)
  int ntiles_n;
  // MXFP8 operands: A scales [M_cap][K/32]; B scales in the tile-blocked
  // order [E][ceil(N/256)][K/128][256][4] (4 consecutive K blocks per row)
  const uint8_t* a_scales;
  const uint8_t* b_scales;
  // weight gradient (K-grouped): C_e [wg_P][N] fp32 = A_e^T B_e over the
  // group's rows; A [M_cap][wg_P], B [M_cap][N] bf16
  int wg_P;
  int ntiles_m;             // ceil(wg_P / 256)
  float* Cf;                // [E][wg_P][N]
  int accumulate;           // 1: C += result
};

// Physical 16-byte chunk of logical chunk c in operand-tile row r.  The XOR
// key uses only row bits 0..4, so rows r and r + 32 share it and the four
// 32-row MFMA blocks of a wave are immediate offsets from one address.
// gfx950 serves a 16-byte LDS read in four passes of 16 lanes (64 banks x 4
// bytes each); a pass takes the lanes that agree in lane bit 5 and in the
// parity of lane bits 2..4 (measured with single-pair conflict probes).  Both
// fragment shapes read without conflicts under this key: the 16 x 16 x 32
// reads (lane: row bits 0..3, chunk bits 0..1) and the 32 x 32 reads (lane:
// row bits 0..4, chunk bit 0).  Row bit 3 moves key bit 1 and row bit 4 key
// bit 0; with bit 3 on key bit 0 instead, a 16 x 16 pass would put two rows
// on each 4-bank group (the conflict counter read 0.5 conflict cycles per
// active LDS cycle with that key, 0.01 with this one).
__device__ __forceinline__ int swz_hi(int t) { return ((t & 1) << 1) | ((t >> 1) & 1); }   // t = row bits 3..4
__device__ __forceinline__ int swz_key(int r) { return (r & 7) ^ swz_hi((r >> 3) & 3); }
__device__ __forceinline__ int swz_off(int r, int c) { return r * 128 + ((c ^ swz_key(r)) << 4); }

// Weight-gradient operand tiles keep their [reduction rows][columns] layout:
// 64 rows of 256 bf16 columns, 512 bytes per row, 16-byte chunk c of row r at
// chunk c ^ 4 (r % 4).  A transposed fragment read names 4 consecutive rows
// x 4 chunks per half wave; the key sends those 16 pieces to 16 different
// 16-byte bank groups.
__device__ __forceinline__ int wg_off(int r, int c) { return r * 512 + ((c ^ ((r & 3) << 2)) << 4); }

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// LDS transpose read (8 bytes per lane): lane j of each 16-lane group gets
// element j % 4 of the 4-element pieces named by lanes j/4 + 4 i of its group,
// i = 0..3, in that order.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// Raw buffer descriptor over [base, base + bytes) (bytes clamped to 2^32 - 1).
// gfx9 descriptor word 3: 32-bit data format, no swizzle, no stride.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long long bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0xFFFFFFFFll) bytes = 0xFFFFFFFFll;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(uint32_t)bytes, 0x00020000);
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes lds_wave_base + 16 l (the LDS base is wave-uniform, held in M0).
__device__ __forceinline__ void lds_dma16(const rsrc_t& rs, uint8_t* lds_wave_base,
                                          uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, soff, 0, 0);
}

// 16 bytes to global memory with the non-temporal hint: kernel outputs are
// not read again by the kernel, and streaming them keeps the L2 for the
// operand panels that the tiles running together share.  Used where a store
// instruction writes whole 128-byte lines (staged rows); FC1's 32-byte row
// pieces of y stay ordinary stores, which the L2 merges (with the hint they
// measured 3% slower on the GPT-OSS-like FC1).
__device__ __forceinline__ void store16_nt(void* dst, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(dst));
}

// A zero the compiler cannot see through.  Epilogue addressing is derived
// from it so that none of it is hoisted out of the tile loop, where it would
// stay live across the main loop and push loop values into scratch.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

// Wait until every vector memory operation of this wave has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------- MX helpers

// MXFP8 of a staged bf16 tile: stg[r][c] (row stride ld elements) holds rows
// [0, rows_valid) x cols [0, ncols) of the output, whose global position is
// grouped row grow0 + r, column col0 + c.  row-wise: blocks along the row;
// col-wise: blocks of 32 rows starting at the tile's first row (a tile always
// starts a block because tiles start at group row multiples of 256), scale
// column scol0 + r / 32.
// gcol(c): the global column of staged column c (a multiple of 32 apart from
// c's offset in its 32-column block), or -1 where the staged column is not
// output; ncols is a multiple of 32.
template <int NT, typename GCol>
__device__ __forceinline__ void mx_from_stage_map(const Stg& stg, int rows_valid, int ncols, int grow0,
                                                  const GemmArgs& p, int scol0, GCol gcol) {
  const int t = threadIdx.x + opaque_zero();
  if (p.row_q) {
    const bool rq_aligned = (reinterpret_cast<uintptr_t>(p.row_q) & 15) == 0;
    const int nb = ncols >> 5;
    for (int it = t; it < stg.rows() * nb; it += NT) {
      int r = it / nb, cb = it - r * nb;
      const int gc = gcol(cb * 32);
      if (r >= rows_valid || gc < 0) continue;
      float v[32];
      const uint4* s = reinterpret_cast<const uint4*>(stg.row(r) + cb * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 x = s[q];
        uint32_t ww[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * q + 2 * j] = __uint_as_float(ww[j] << 16);
          v[8 * q + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
        }
      }
      uint32_t w[8];
      uint8_t sb = mx_quant32(v, 32, w, p.mx_e5 != 0);
      long long grow = grow0 + r;
      // (rows are a multiple of 64 bytes and gc of 32: 16-byte aligned
      // whenever row_q is)
      if (rq_aligned) store_codes32_aligned_nt(p.row_q + grow * p.mx_cols + gc, w);
      else store_codes32(p.row_q + grow * p.mx_cols + gc, w, 32);
      p.row_s[grow * (p.mx_cols >> 5) + (gc >> 5)] = sb;
    }
  }
  if (p.col_q) {
    // items of two adjacent columns x 32 rows: one 4-byte LDS read per row;
    // the row blocks of a column pair are consecutive items, so neighbouring
    // lanes store neighbouring 32-byte pieces of a column.  K-tiled layout:
    // a group's last tile also fills its slots up to the next multiple of 4
    // (128 rows) with zero codes and scale byte 127.
    const int nrb = (rows_valid + 31) >> 5;
    const int npad = p.col_blocked ? 4 * ((rows_valid + 127) >> 7) : nrb;
    const int nc2 = ncols >> 1;
    const int nrbt = stg.rows() >> 5;
    const long long slot_bytes = 32LL * p.col_s_ld;   // K-tiled: one column's codes
    for (int it = t; it < nc2 * nrbt; it += NT) {
      const int rb = it % nrbt, c2 = it / nrbt;
      const long long gc = gcol(2 * c2);
      if (rb >= npad || gc < 0) continue;
      if (rb >= nrb) {   // K-tiled padding slot
        const uint32_t z[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        store_codes32_slot<true>(p.col_q + gc * slot_bytes + (scol0 + rb) * 32LL, z, 0);
        store_codes32_slot<true>(p.col_q + (gc + 1) * slot_bytes + (scol0 + rb) * 32LL, z, 0);
        p.col_s[gc * p.col_s_ld + scol0 + rb] = 127;
        p.col_s[(gc + 1) * p.col_s_ld + scol0 + rb] = 127;
        continue;
      }
      int nvalid = rows_valid - rb * 32;
      if (nvalid > 32) nvalid = 32;
      float v0[32], v1[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t w2 = *reinterpret_cast<const uint32_t*>(stg.row(rb * 32 + i) + 2 * c2);
        v0[i] = __uint_as_float(w2 << 16);
        v1[i] = __uint_as_float(w2 & 0xFFFF0000u);
      }
      uint32_t w[8];
      uint8_t sb = mx_quant32(v0, nvalid, w, p.mx_e5 != 0);
      if (p.col_blocked) store_codes32_slot<true>(p.col_q + gc * slot_bytes + (scol0 + rb) * 32LL, w, nvalid);
      else store_codes32(p.col_q + gc * p.M_cap + grow0 + rb * 32, w, nvalid);
      p.col_s[gc * p.col_s_ld + scol0 + rb] = sb;
      sb = mx_quant32(v1, nvalid, w, p.mx_e5 != 0);
      if (p.col_blocked)
        store_codes32_slot<true>(p.col_q + (gc + 1) * slot_bytes + (scol0 + rb) * 32LL, w, nvalid);
      else store_codes32(p.col_q + (gc + 1) * p.M_cap + grow0 + rb * 32, w, nvalid);
      p.col_s[(gc + 1) * p.col_s_ld + scol0 + rb] = sb;
    }
  }
}
// staged columns [0, ncols) are global columns col0 ..
template <int NT>
__device__ __forceinline__ void mx_from_stage(const Stg& stg, int rows_valid, int ncols, int grow0,
                                              int col0, const GemmArgs& p, int scol0) {
  mx_from_stage_map<NT>(stg, rows_valid, ncols, grow0, p, scol0, [=](int c) { return col0 + c; });
}

// Wave maximum of a non-negative float (no NaN), as its bits: for such
// values the float order is the order of their bits as unsigned integers.
// Swizzle in bitmask mode pairs lane ^ xm within each half of the wave; the
// result is wave-uniform (a scalar register).
__device__ __forceinline__ uint32_t wave_max_bits(float v) {
  uint32_t b = __float_as_uint(v);
  b = max(b, (uint32_t)__builtin_amdgcn_ds_swizzle((int)b, (1 << 10) | 0x1F));
  b = max(b, (uint32_t)__builtin_amdgcn_ds_swizzle((int)b, (2 << 10) | 0x1F));
  b = max(b, (uint32_t)__builtin_amdgcn_ds_swizzle((int)b, (4 << 10) | 0x1F));
  b = max(b, (uint32_t)__builtin_amdgcn_ds_swizzle((int)b, (8 << 10) | 0x1F));
  b = max(b, (uint32_t)__builtin_amdgcn_ds_swizzle((int)b, (16 << 10) | 0x1F));
  return max((uint32_t)__builtin_amdgcn_readlane((int)b, 0), (uint32_t)__builtin_amdgcn_readlane((int)b, 32));
}

// In-place Walsh-Hadamard butterflies of 16 values (Sylvester order, not
// normalised).
__device__ __forceinline__ void fwht16(float (&v)[16]) {
#pragma unroll
  for (int len = 1; len < 16; len <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & len) == 0) {
        const float a = v[i], b = v[i + len];
        v[i] = a + b;
        v[i + len] = a - b;
      }
}

// Largest |.| of the orthonormal 16-point Hadamard rotation of the transposed
// staged tile: every column (of the 64-column chunks whose bit is set in
// chunk_ok) is cut into runs of 16 consecutive rows starting at the tile's
// first row (tiles start at group row multiples of 256, so the runs restart
// at each group's first row); rows from rows_valid on count as zero, and row
// i of every run is negated first when bit i of signs is set.  One item is
// 4 columns x 16 rows, read as 16 conflict-free 8-byte rows.
template <int NT>
__device__ __forceinline__ float rht16_amax_stage(const Stg& stg, int rows_valid, uint32_t chunk_ok,
                                                  uint32_t signs) {
  const int t = threadIdx.x + opaque_zero();
  float amax = 0.0f;
  for (int it = t; it < (stg.rows() / 16) * 64; it += NT) {
    const int ch = it & 63, r0 = (it >> 6) * 16;
    if (r0 >= rows_valid || !((chunk_ok >> (ch >> 4)) & 1u)) continue;
    uint2 w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      w[i] = r0 + i < rows_valid ? *reinterpret_cast<const uint2*>(stg.row(r0 + i) + ch * 4)
                                 : make_uint2(0u, 0u);
      const uint32_t neg = ((signs >> i) & 1u) * 0x80008000u;
      w[i].x ^= neg;
      w[i].y ^= neg;
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      float lo[16], hi[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t x = d ? w[i].y : w[i].x;
        lo[i] = __uint_as_float(x << 16);
        hi[i] = __uint_as_float(x & 0xFFFF0000u);
      }
      fwht16(lo);
      fwht16(hi);
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(lo[i]), fabsf(hi[i])));
    }
  }
  return 0.25f * amax;   // the 1/4 of the orthonormal H16 (exact)
}

// Coalesced store of a staged bf16 tile (ncols % 8 == 0 assumed per 8-chunk validity).
template <int NT>
__device__ __forceinline__ void store_stage(const Stg& stg, int rows_valid,
                                            int ncols_valid, int ncols_tile, uint16_t* dst,
                                            long long dst_ld) {
  const int t = threadIdx.x + opaque_zero();
  const int cpr = ncols_tile >> 3;  // 16-byte chunks per row
  for (int it = t; it < stg.rows() * cpr; it += NT) {
    int r = it / cpr, ch = it - r * cpr;
    if (r < rows_valid && ch * 8 < ncols_valid) {
      const uint4 v = *reinterpret_cast<const uint4*>(stg.row(r) + ch * 8);
      store16_nt(dst + r * dst_ld + ch * 8, v);
    }
  }
}

// ---------------------------------------------------------------- the kernel
// ACT: the activation of the GLU and dGLU epilogues (one kernel per
// activation, so the epilogue holds no dispatch); unused by the others.
template <int EPI, int BLAY, int AT = AT_BF16, int ACT = ACT_SWIGLU>
__global__ __launch_bounds__(64 * gm_waves(EPI, BLAY, AT), 1) void group_gemm_kernel(GemmArgs p) {
  // Operand rows are staged as 128-byte K slices whatever the type: 64 bf16
  // (4 k-steps of v_mfma_f32_32x32x16_bf16 or 2 of v_mfma_f32_16x16x32_bf16)
  // or 128 e4m3 (2 k-steps of v_mfma_scale_f32_32x32x64_f8f6f4).  MXFP8
  // stages also carry the tile's E8M0 scales: 256 rows x 4 bytes for A and
  // for B after the two tiles.
  constexpr bool MXT = AT != AT_BF16;
  // block-scaled MFMA format codes (0 = e4m3, 1 = e5m2) of B (the first
  // source) and of A (the second source)
  constexpr int FMT_A = (AT == AT_MX_A5 || AT == AT_MX_AB5) ? 1 : 0;
  constexpr int FMT_B = (AT == AT_MX_B5 || AT == AT_MX_AB5) ? 1 : 0;
  constexpr int ESZ = MXT ? 1 : 2;            // operand element bytes
  constexpr int KSTEPS = MXT ? 2 : 4;         // k-steps per K-tile
  static_assert(!MXT || (BLAY == BL_PACKED && (EPI == EPI_STORE || EPI == EPI_GLU ||
                                                EPI == EPI_GLU_MX)) ||
                    (BLAY == BL_NK && EPI == EPI_WGRAD),
                "MXFP8 inputs: packed B with a plain store or GLU epilogue, or a weight gradient");
  static_assert(2 * GM_TILE_BYTES + 2048 <= GM_STAGE_ALLOC, "scale slots");
  // Weight gradients reduce over a group's rows.  bf16 (WGT): both operands
  // are stored [rows][columns] with the reduction dimension as the row index;
  // they go to LDS as they are (LDS-DMA, wg_off layout) and the MFMA
  // fragments come out of the LDS transpose read.  MXFP8 (WGM): both
  // operands are transposed copies in the K-tiled layout, [columns][slots of
  // 32 rows], so each is K-contiguous with its own block scales and takes
  // the ordinary MXFP8 path; group e's reduction is its 4 ceil(m_e/128) slots
  // from slot 4 sum_{j<e} ceil(m_j/128), whole 128-code K-tiles zero-padded
  // past the group's rows.  Other N-contiguous B operands go through a
  // register transpose.
  constexpr bool WG = EPI == EPI_WGRAD;
  constexpr bool WGM = WG && MXT;
  constexpr bool WGT = WG && !MXT;
  static_assert(!WG || (BLAY == BL_KN && !MXT) || (BLAY == BL_NK && MXT),
                "weight gradient: N-contiguous bf16 operands or K-tiled MXFP8 copies");
  constexpr bool KNR = BLAY == BL_KN && !WG;
  constexpr int NW = gm_waves(EPI, BLAY, AT);   // waves per workgroup (4 or 8)
  constexpr int NTH = 64 * NW;           // threads
  static_assert(NW == 4 || !WG, "8 waves: not the weight gradients");
  static_assert(64 * 32 % NTH == 0 && (NTH == 256 || NTH == 512), "N-contiguous B transpose: 4 or 8 waves");
  // Two distinct stage arrays: the compiler can then see that the LDS-DMA
  // writes of the next stage never alias the fragment reads of the current
  // one, and does not wait for the prefetch before computing.
  __shared__ __attribute__((aligned(16))) uint8_t lds0[GM_STAGE_ALLOC];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[GM_STAGE_ALLOC];
  __shared__ GroupScan gs;
  __shared__ float drs_lds[GM_BM];   // dGLU: per-row d(row_scale) of the tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;

  // (MXFP8 weight gradient: 128-row m-tiles, so tile_off[e] is the group's
  // first K-tile of the column copies)
  // A group's last m-tile with at most 128 rows always runs as a 128-row
  // tile; whether it is also scheduled apart, among the half tiles that take
  // the first ids, is per kernel.  The dGLU kernel (N = I: few tile rounds
  // per CU; with or without the parameter gradients) keeps that, since a
  // workgroup's share is then at most one half tile plus full ones.  The
  // other 8-wave kernels (FC1, FC2 and dX, bf16
  // or MXFP8; many rounds) schedule it in its expert's 4 x 8 block instead,
  // where it shares the B panels of the expert's other m-tiles in L2:
  // measured 2-9% faster on the DeepSeek-V3-like share, neutral on the
  // GPT-OSS-like FC1.
  constexpr bool HALF_FIRST = !WG && !(NW == 8 && EPI != EPI_DGLU && EPI != EPI_DGLU_G);
  // The dGLU kernels on packed or K-contiguous plain W2 (N = I = 2048 on the
  // DeepSeek-V3-like share: 2.2 full-tile units per CU) split each short
  // m-tile once more, into two 128 x 128 quarter tiles (column halves of
  // the n-tile): with F
  // full tiles and 2H quarter tiles on P workgroups every workgroup gets F / P
  // full tiles and at most one quarter, where a half tile left the workgroups
  // that drew one idle-free and the rest idle for its duration.
  constexpr bool QTILE = (EPI == EPI_DGLU || EPI == EPI_DGLU_G) && (BLAY == BL_PACKED || BLAY == BL_NK);
  static_assert(!QTILE || HALF_FIRST, "quarter tiles: short tiles first");
  build_group_scan<NTH>(gs, p.counts, p.E, p.M_cap, WGM ? 128 : GM_BM, HALF_FIRST ? GM_BM / 2 : 0,
                          p.offsets_out, p.status_out, blockIdx.x == 0, p.col_blocked != 0);
  if (WG) {
    // Every expert owns the same number of output tiles but its tiles cost
    // m_e: hand them out largest group first (ties: lower id), the order kept
    // in mxs_off (the MX scale prefix is not needed here).
    for (int ee = tid; ee < p.E; ee += NTH) {
      const int ce = gs.row_off[ee + 1] - gs.row_off[ee];
      int rank = 0;
      for (int j = 0; j < p.E; ++j) {
        const int cj = gs.row_off[j + 1] - gs.row_off[j];
        rank += (cj > ce) || (cj == ce && j < ee);
      }
      gs.mxs_off[rank] = ee;
    }
    __syncthreads();
  }
  // grouped GEMM: the half-height tiles (ids [0, n_half)) come first, then
  // the full ones, so that every workgroup's share is balanced: with F full
  // and H half tiles on P workgroups, H <= P gives each workgroup at most
  // ceil((H + F) / P) tiles of which the first may be a half one.
  // ids per short m-tile: one per n-tile, or with quarter tiles one per
  // 128-column half of I
  const int NHT = QTILE ? (p.N + 127) / 128 : p.ntiles_n;
  const int n_half = WG ? 0 : gs.half_off[p.E] * NHT;
  const int total_tiles =
      WG ? p.E * p.ntiles_m * p.ntiles_n : n_half + gs.tile_off[p.E] * p.ntiles_n;

  // XCD-aware slot: consecutive workgroups land on different XCDs (round
  // robin over 8), so give each XCD a contiguous run of tile ids per round.
  const int P = gridDim.x;
  const int slot = (P % 8 == 0) ? ((blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3)) : blockIdx.x;
  const int nk = p.K * ESZ / 128;             // K-tiles of 128 bytes per row
  const int NT = p.ntiles_n;

  // the amax epilogues' running wave maximum (bits of a non-negative float):
  // raised into amax_out with one atomic per wave after the last tile, not
  // once per tile, so no tile's main loop waits on a contended atomic
  uint32_t amax_bits = 0u;
  for (int tile = slot; tile < total_tiles; tile += P) {
    // ---- decode (expert, m-tile, n-tile).  Half tiles: expert e owns ids
    // [half_off[e] * NT, half_off[e+1] * NT), one per n-tile of its last
    // m-tile.  Full tiles: expert e owns ids n_half + [tile_off[e] * NT,
    // tile_off[e+1] * NT), in blocks of 4 m-tiles x 8 n-tiles (m fastest), so
    // the run of consecutive ids an XCD takes per round shares few A panels
    // and few B panels.
    int e, mt, nt;
    int nq = 0;   // quarter tiles: the n-tile's column half
    if (!WG && tile < n_half) {
      int lo = 0, hi = p.E;  // invariant: half_off[lo]*NHT <= tile < half_off[hi]*NHT
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (gs.half_off[mid] * NHT <= tile) lo = mid; else hi = mid;
      }
      e = lo;
      const int lq = tile - gs.half_off[e] * NHT;
      nt = QTILE ? lq >> 1 : lq;
      nq = QTILE ? lq & 1 : 0;
      mt = gs.tile_off[e + 1] - gs.tile_off[e];   // after the expert's full m-tiles
    } else {
      int local, MT;
      if (WG) {   // weight gradient: p.ntiles_m x NT output tiles per expert
        const int per = p.ntiles_m * NT;
        const int rank = tile / per;
        e = gs.mxs_off[rank];
        local = tile - rank * per;
        MT = p.ntiles_m;
      } else {
        const int ft = tile - n_half;
        int lo = 0, hi = p.E;  // invariant: tile_off[lo]*NT <= ft < tile_off[hi]*NT
        while (hi - lo > 1) {
          int mid = (lo + hi) >> 1;
          if (gs.tile_off[mid] * NT <= ft) lo = mid; else hi = mid;
        }
        e = lo;
        local = ft - gs.tile_off[e] * NT;
        MT = gs.tile_off[e + 1] - gs.tile_off[e];
      }
      constexpr int BHT = 4, BWT = 8;
      const int band = local / (BHT * NT);
      const int bh = min(BHT, MT - band * BHT);
      const int l2 = local - band * BHT * NT;
      const int nb = l2 / (bh * BWT);
      const int l3 = l2 - nb * bh * BWT;
      mt = band * BHT + l3 % bh;
      nt = nb * BWT + l3 / bh;
    }
    const int g_row0 = gs.row_off[e];
    const int m_e = gs.row_off[e + 1] - g_row0;
    // grouped GEMM: the tile's first grouped row; weight gradient: the
    // group's first row (the reduction runs over all m_e rows)
    // (MXFP8 weight gradient: A's rows are the output rows mt*256 ..)
    const int row0 = WGT ? g_row0 : (WGM ? mt * GM_BM : g_row0 + mt * GM_BM);
    const int rows_valid = WG ? min(GM_BM, p.wg_P - mt * GM_BM) : min(GM_BM, m_e - mt * GM_BM);
    const int n0 = nt * GM_BN + nq * (GM_BN / 2);
    const int nk_t = WGT ? (m_e + 63) / 64 : (WGM ? (m_e + 127) / 128 : nk);   // K-tiles of this tile
    const int kt0 = WGM ? gs.tile_off[e] : 0;        // first K-tile (MXFP8 weight gradient)

    // The tile body for MI 32-row MFMA blocks per wave, NW / 2 wave rows, and
    // NBW 32-column blocks per wave, 2 wave columns: the 256 x 256 tile (4
    // waves: MI = 4, waves 128 x 128; 8 waves: MI = 2, waves 64 x 128); a
    // group's last m-tile with at most 128 valid rows runs with half the MI as
    // a 128-row tile, half the MFMA work of the padded 256-row tile (the dGLU
    // kernels on packed W2: two 128 x 128 quarter tiles, NBW = 2).
    // Weight-gradient tiles are always full.
    auto tile_body = [&](auto mic, auto nbwc) {
    constexpr int MI = decltype(mic)::value;
    constexpr int NBW = decltype(nbwc)::value;  // 32-column MFMA blocks per wave (4; quarter tiles 2)
    constexpr int WBN = 32 * NBW;               // columns per wave
    constexpr int TBN = 2 * WBN;                // tile columns
    constexpr int HR = 32 * MI;                 // rows per wave row
    constexpr int TBM = (NW / 2) * HR;          // tile rows
    constexpr int SHR = TBM / 2;                // staged rows per LDS stage array

    // Per-tile opaque zero: main-loop addressing is recomputed for each tile,
    // so it is not live across the epilogue.
    const int zt = opaque_zero();
    const int lane_t = lane + zt;

    // ---- buffer descriptors: loads past the record count return zero, so
    // rows past the tile's valid rows (A) or past N (K-contiguous B) need no
    // clamping.  The A descriptor ends at the group's last row: the padding
    // rows of a group's last m-tile read zeros instead of the next group's
    // rows, which costs no memory traffic, and MFMAs on zero operands draw
    // less power on this power-limited chip.
    const uint32_t a_stride = WGT ? (uint32_t)p.wg_P * 2u : (uint32_t)p.K * ESZ;
    // weight gradient: only the group's rows (the next group's rows read zero)
    const long long a_bytes = (long long)(WGT ? m_e : rows_valid) * a_stride;
    const uint8_t* Ab = reinterpret_cast<const uint8_t*>(p.A);
    const rsrc_t rsA = make_rsrc(Ab + (long long)row0 * a_stride, a_bytes);
    const uint8_t* Bb = WGT ? reinterpret_cast<const uint8_t*>(p.B) + (long long)row0 * p.ldb * 2
                            : reinterpret_cast<const uint8_t*>(p.B) + (long long)e * p.b_estride * ESZ;
    const uint32_t b_stride = (uint32_t)p.ldb * ESZ;
    rsrc_t rsB;
    if (WGT)
      rsB = make_rsrc(Bb, (long long)m_e * b_stride);
    else if (BLAY == BL_NK)
      rsB = make_rsrc(Bb + (long long)n0 * b_stride, (long long)(p.N - n0) * b_stride);
    else if (BLAY == BL_PACKED)   // the n-tile's K/64 contiguous 32 KB blocks
      rsB = make_rsrc(Bb + (long long)nt * nk * GM_TILE_BYTES, (long long)nk * GM_TILE_BYTES);
    else
      rsB = make_rsrc(Bb, p.b_estride * ESZ);

    // MXFP8 scales of the tile: A rows row0.. (K/32 bytes each), B's blocked
    // 1 KB per K-tile (weight gradient: B rows n0.., K/32 bytes each)
    const uint32_t sa_stride = (uint32_t)p.K / 32u;
    const uint32_t sb_stride = (uint32_t)p.ldb / 32u;
    rsrc_t rsSA, rsSB;
    if (MXT) {
      rsSA = make_rsrc(p.a_scales + (long long)row0 * sa_stride, (long long)rows_valid * sa_stride);
      rsSB = WGM ? make_rsrc(p.b_scales + (long long)n0 * sb_stride, (long long)(p.N - n0) * sb_stride)
                 : make_rsrc(p.b_scales + ((long long)e * NT + nt) * nk * 1024, (long long)nk * 1024);
    }

    // N-contiguous B: n-chunk tid % 32 (8 columns), k-group tid / 32 (KR rows:
    // 8 with 256 threads, 4 with 512); the column chunk is clamped inside the
    // row so no load leaves the matrix.
    constexpr int KR = 64 * 32 / NTH;
    const int kn_c = (tid + zt) & 31, kn_g = (tid + zt) >> 5;
    const uint32_t kn_voff =
        (uint32_t)(kn_g * KR) * b_stride + (uint32_t)min(n0 + kn_c * 8, p.N - 8) * 2u;

    // bf16 on 8 waves (FC1, the plain GroupGemm, and dgrad + dGLU with or
    // without the parameter gradients on full and half tiles): the main
    // loop runs on v_mfma_f32_16x16x32_bf16 (its
    // accumulators are moved into the 32 x 32 layout below for the
    // epilogues; the results are bit-identical to the 32 x 32 loop's).  The
    // dGLU quarter tiles (64 columns per wave) and everything else run on
    // v_mfma_f32_32x32x16_bf16 or the block-scaled 32 x 32 x 64 form.  With
    // conflict-free 16 x 16 reads the dGLU kernel gains 0.4-0.7% (it measured
    // even while those reads had two-way bank conflicts).
    constexpr bool M16 = NW == 8 && !MXT && !WG && BLAY != BL_KN && ((EPI != EPI_DGLU && EPI != EPI_DGLU_G) || NBW == 4);
    constexpr bool MX8 = NW == 8 && MXT && !WG;
    static_assert(NBW == 4 || ((EPI == EPI_DGLU || EPI == EPI_DGLU_G) && !M16 && !MX8),
                  "narrow tiles: the dGLU kernels' 32 x 32 loop only");
    constexpr int MB = 2 * MI;                  // 16-row blocks per wave
    f32x16 acc[MI][4];
    f32x4 acc16[M16 ? MB : 1][8];
    if constexpr (M16) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc16[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    }

    // direct global -> LDS of one ROWS x 64 operand tile (swizzled layout).
    // Instruction j of wave w fills rows 8 (NJ w + j) .. + 7 (NJ = ROWS / 8 NW);
    // lane (rl, pc) lands on row 8 (NJ w + j) + rl, physical chunk pc, so it
    // fetches logical chunk pc ^ key(row), key = rl ^ swz_hi((NJ w + j) & 3).
    const int rl_t = lane_t >> 3, pc_t = lane_t & 7;
    auto issue_tile = [&](auto rowsc, const rsrc_t& rs, uint8_t* lds_tile, uint32_t stride,
                          uint32_t koff) {
      constexpr int NJ = decltype(rowsc)::value / (8 * NW);
      const uint32_t vrow = (uint32_t)(wave * 8 * NJ + rl_t) * stride;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = pc_t ^ (rl_t ^ swz_hi((wave * NJ + j) & 3));
        const uint32_t voff = vrow + (uint32_t)(j * 8) * stride + (uint32_t)(c << 4);
        lds_dma16(rs, lds_tile + (wave * NJ + j) * 1024, voff, koff);
      }
    };
    // K-tiles past the end are fetched through a descriptor with no records:
    // the loads return zeros, so the main loop needs no tail branch.
    const rsrc_t rsZ = make_rsrc(Ab, 0);
    // a packed 32 KB block is already in LDS order: each wave instruction
    // streams 1 KB contiguously
    // (a quarter tile takes rows nq * 128 .. + 127 of the block: the second
    // 16 KB, whose rows keep their swizzle, which depends on row bits 0..4)
    auto issue_block = [&](const rsrc_t& rs, uint8_t* lds_tile, uint32_t koff) {
      constexpr int NBK = TBN / (8 * NW);      // 1 KB pieces per wave
#pragma unroll
      for (int j = 0; j < NBK; ++j) {
        const int blk = wave * NBK + j;
        lds_dma16(rs, lds_tile + blk * 1024,
                  (uint32_t)(nq * (GM_TILE_BYTES / 2) + blk * 1024 + lane_t * 16), koff);
      }
    };
    // weight gradient: K-tile kt (rows kt*64 .. + 63 of the group) of an
    // operand stored [rows][columns], columns from byte col0b on, into the
    // wg_off layout.  Instruction j of wave w fills rows 2 (8 w + j) and the
    // next one; lane l lands on row + l / 32, physical chunk l % 32, so it
    // fetches logical chunk (l % 32) ^ 4 (row % 4).  The descriptor starts at
    // the K-tile's first row and ends at the group's last row, so rows past
    // the group read zero.  Columns past the matrix edge read other bytes of
    // the operand; they only reach output columns the epilogue drops.
    auto issue_wg = [&](const rsrc_t& rs, uint8_t* lds_tile, uint32_t stride, uint32_t col0b) {
      const int hr = lane_t >> 5, pw = lane_t & 31;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 2 * (8 * wave + j) + hr;
        const int c = pw ^ ((r & 3) << 2);
        lds_dma16(rs, lds_tile + (8 * wave + j) * 1024,
                  (uint32_t)r * stride + col0b + (uint32_t)(c << 4), 0u);
      }
    };
    auto issue_direct = [&](int kt, uint8_t* sa) {
      const bool in = kt < nk_t;
      if constexpr (WGT) {
        const long long r0 = (long long)kt * 64;
        const rsrc_t rak = in ? make_rsrc(Ab + ((long long)row0 + r0) * a_stride,
                                          ((long long)m_e - r0) * a_stride)
                              : rsZ;
        const rsrc_t rbk = in ? make_rsrc(Bb + r0 * b_stride, ((long long)m_e - r0) * b_stride) : rsZ;
        issue_wg(rak, sa, a_stride, (uint32_t)(mt * GM_BM) * 2u);
        issue_wg(rbk, sa + GM_TILE_BYTES, b_stride, (uint32_t)n0 * 2u);
        return;
      }
      const uint32_t kk = (uint32_t)(kt0 + kt);   // K-tile within the rows
      issue_tile(std::integral_constant<int, TBM>{}, in ? rsA : rsZ, sa, a_stride, kk * 128u);
      if (BLAY == BL_NK)   // the tile's TBN rows of B from n0 (a quarter tile's 128)
        issue_tile(std::integral_constant<int, TBN>{}, in ? rsB : rsZ, sa + GM_TILE_BYTES,
                   b_stride, kk * 128u);
      if (BLAY == BL_PACKED)
        issue_block(in ? rsB : rsZ, sa + GM_TILE_BYTES, (uint32_t)kt * GM_TILE_BYTES);
      if (MXT && NW == 4) {   // 4 scale bytes per row: one dword per lane, 64 rows per wave
        const uint32_t r = (uint32_t)(wave * 64 + lane_t);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            in ? rsSA : rsZ, (__attribute__((address_space(3))) void*)(sa + 2 * GM_TILE_BYTES + wave * 256),
            4, r * sa_stride, kk * 4u, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            in ? rsSB : rsZ,
            (__attribute__((address_space(3))) void*)(sa + 2 * GM_TILE_BYTES + 1024 + wave * 256), 4,
            WGM ? r * sb_stride : r * 4u, WGM ? kk * 4u : kk * 1024u, 0, 0);
      }
      if (MXT && NW == 8) {   // waves 0-3: A's scales, waves 4-7: B's (64 rows per wave)
        const bool ah = wave < 4;
        const uint32_t r = (uint32_t)((wave & 3) * 64 + lane_t);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            in ? (ah ? rsSA : rsSB) : rsZ,
            (__attribute__((address_space(3))) void*)(sa + 2 * GM_TILE_BYTES + (ah ? 0 : 1024) + (wave & 3) * 256),
            4, r * (ah ? sa_stride : 4u), kk * (ah ? 4u : 1024u), 0, 0);
      }
    };
    u32x4 rb[KR];
    auto kn_load = [&](int kt) {
      const bool in = kt < nk_t;
      const int ktc = in ? kt : 0;
      const long long krow = (long long)ktc * 64;
#pragma unroll
      for (int i = 0; i < KR; ++i)
        rb[i] = __builtin_amdgcn_raw_buffer_load_b128(in ? rsB : rsZ, kn_voff,
                                                      (uint32_t)((krow + i) * b_stride), 0);
    };
    // r[i] holds 8 columns at k = KR*kn_g + i; transposed to KR k-values per
    // column: a whole 16-byte chunk (KR = 8) or its half 8 (kn_g % 2) bytes in
    auto kn_put = [&](const u32x4 (&r)[KR], uint8_t* t) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t o[KR / 2];
#pragma unroll
        for (int q = 0; q < KR / 2; ++q) {
          const uint32_t lo = r[2 * q][j >> 1], hi = r[2 * q + 1][j >> 1];
          o[q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        if constexpr (KR == 8)
          *reinterpret_cast<uint4*>(t + swz_off(kn_c * 8 + j, kn_g)) = make_uint4(o[0], o[1], o[2], o[3]);
        else
          *reinterpret_cast<uint2*>(t + swz_off(kn_c * 8 + j, kn_g >> 1) + 8 * (kn_g & 1)) = make_uint2(o[0], o[1]);
      }
    };
    auto kn_store = [&](uint8_t* stage) { kn_put(rb, stage + GM_TILE_BYTES); };

    // Fragments are double-buffered one k-step ahead.  A K-tile is 4 k-steps
    // of 16 MFMAs per wave.  The barrier that hands a stage back to the DMA
    // sits before the LAST k-step of each K-tile: that k-step's fragments are
    // already in registers, so its 16 MFMAs keep the pipe busy while the next
    // stage's first fragments are read and the next DMA is issued.
    bf16x8 af[2][MI], bfr[2][4];                // bf16 fragments
    i32x8 afx[2][MI], bfx[2][4];                // e4m3 fragments (32 bytes per lane)
    uint32_t sca[2][MI], scb[2][4];             // E8M0 scales per stage set
    // reads in order of first use by the MFMA sequence (i outer, j inner).
    // bf16: lane half h = lane / 32 takes 16-byte chunk 2 ks + h of its row
    // (8 k values).  e4m3: the block-scaled MFMA takes, in lane half h, bytes
    // 0..15 = k 16 h .. + 15 of the step's first 32-block and bytes 16..31 =
    // k 32 + 16 h .. + 15 of its second, so chunks 4 ks + h and 4 ks + 2 + h;
    // the first block's scale comes from the lower-half lane of the row and
    // the second block's from the upper-half lane.  With k-step 0 an MXFP8
    // stage also yields its scales: the upper half shifts its dword down by
    // one byte, so both halves select byte 2 ks in the MFMA (block 2 ks + h).
    auto frag_load = [&](const uint8_t* sa, int ks, int buf, int sset) {
      const uint8_t* sb = sa + GM_TILE_BYTES;
      const int h = lane_t >> 5;
      const int ra = wm * HR + (lane_t & 31), rbw = wn * WBN + (lane_t & 31);
      if constexpr (WGT) {
        // lane l names row ks*16 + 8 (l/32) + 4 t + (l%16)/4 at column
        // c0 + 16 ((l/16) % 2) + 4 (l % 4) and so receives column c0 + l % 32
        // at rows ks*16 + 8 (l/32) + 4 t .. + 3: two reads (t = 0, 1) give
        // the 8 k values of the MFMA fragment
        // (each address is one byte offset from the stage base: a longer
        // chain of pointer steps hides from the compiler which stage array a
        // read touches, and it then waits for the other stage's DMA)
        const int rr = ks * 16 + 8 * h + ((lane_t & 15) >> 2);
        const int cl = 16 * ((lane_t >> 4) & 1) + 4 * (lane_t & 3);
        auto rd = [&](int tile, int c0) {
          const int c = c0 + cl;
          const int o = tile + wg_off(rr, c >> 3) + 2 * (c & 7);
          const s16x4 lo = lds_read_tr16(sa + o), hi = lds_read_tr16(sa + (o + 4 * 512));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        af[buf][0] = rd(0, wm * HR);
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[buf][j] = rd(GM_TILE_BYTES, wn * 128 + 32 * j);
#pragma unroll
        for (int i = 1; i < MI; ++i) af[buf][i] = rd(0, wm * HR + 32 * i);
      } else if constexpr (!MXT) {
        const int ch = ks * 2 + h;
        auto rd_a = [&](int i) {
          af[buf][i] = *reinterpret_cast<const bf16x8*>(sa + swz_off(ra + i * 32, ch));
        };
        auto rd_b = [&](int j) {
          bfr[buf][j] = *reinterpret_cast<const bf16x8*>(sb + swz_off(rbw + j * 32, ch));
        };
        rd_a(0);
#pragma unroll
        for (int j = 0; j < NBW; ++j) rd_b(j);
#pragma unroll
        for (int i = 1; i < MI; ++i) rd_a(i);
      } else {
        const int ch = ks * 4 + h;
        auto rd32 = [&](const uint8_t* t, int r) {
          const uint4 lo = *reinterpret_cast<const uint4*>(t + swz_off(r, ch));
          const uint4 hi = *reinterpret_cast<const uint4*>(t + swz_off(r, ch + 2));
          i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          return v;
        };
        if (ks == 0) {
          const uint32_t* ssa = reinterpret_cast<const uint32_t*>(sa + 2 * GM_TILE_BYTES);
          const uint32_t* ssb = reinterpret_cast<const uint32_t*>(sa + 2 * GM_TILE_BYTES + 1024);
#pragma unroll
          for (int i = 0; i < MI; ++i) sca[sset][i] = ssa[ra + i * 32];
#pragma unroll
          for (int j = 0; j < 4; ++j) scb[sset][j] = ssb[rbw + j * 32];
        }
        afx[buf][0] = rd32(sa, ra);
#pragma unroll
        for (int j = 0; j < 4; ++j) bfx[buf][j] = rd32(sb, rbw + j * 32);
#pragma unroll
        for (int i = 1; i < MI; ++i) afx[buf][i] = rd32(sa, ra + i * 32);
      }
    };
    // the 16 MFMAs of one k-step on fragment buffer buf (k-step ks of the
    // K-tile, scale set sset)
    auto mfmas = [&](int buf, int sset, int ks) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          if constexpr (!MXT) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][j], af[buf][i],
                                                                acc[i][j], 0, 0, 0);
          } else {
            const uint32_t sh = 8u * (uint32_t)(lane >> 5);
            const int sB = (int)(scb[sset][j] >> sh), sA = (int)(sca[sset][i] >> sh);
            if (ks == 0)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  bfx[buf][j], afx[buf][i], acc[i][j], FMT_B, FMT_A, 0, sB, 0, sA);
            else
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  bfx[buf][j], afx[buf][i], acc[i][j], FMT_B, FMT_A, 2, sB, 2, sA);
          }
        }
    };
    // LDS reads issued by the frag_load just before a k-step
    constexpr int DS_STEP = (MXT || WG) ? 2 * (MI + 4) : MI + NBW;
    constexpr int NMF = NBW * MI;               // MFMAs per k-step
    // NMF MFMAs; the LDS reads issued just before are spread over them from
    // the first MFMA on (two per MFMA where there are more reads than
    // MFMAs), so each has many MFMAs of cover before its use
    auto mfma_step = [&](int buf, int sset, int ks) {
      mfmas(buf, sset, ks);
      static_for<NMF>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        if constexpr (g < DS_STEP)
          __builtin_amdgcn_sched_group_barrier(0x100, g < DS_STEP - NMF ? 2 : 1, 0);   // DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                           // 1 MFMA
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    // The same with the next stage's DMA (NVM VMEM instructions per wave, 2
    // more with MXFP8 scales) spread over the MFMAs, one or two per MFMA:
    // issued as a burst right after the barrier, the waves' DMA
    // instructions queue at the address unit and hold up the MFMAs issued
    // behind them.
    constexpr int NVM = WGT ? 16 : (TBM + TBN) / (8 * NW);
    auto mfma_step_dma = [&](int buf, int sset, int ks) {
      if constexpr (NW == 8) __builtin_amdgcn_s_setprio(1);   // as in the 16x16 loop (dGLU: -0.7%)
      mfmas(buf, sset, ks);
      static_for<NMF>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        if constexpr (g < DS_STEP) __builtin_amdgcn_sched_group_barrier(0x100, (MXT || WG) ? 2 : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, NVM / NMF + (g < NVM % NMF ? 1 : 0), 0);  // DMA
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   // MFMA
      });
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NW == 8) __builtin_amdgcn_s_setprio(0);
    };
    // k-steps 0 .. KSTEPS-2 of the K-tile in stage sa (fragments of k-step 0
    // requested); the last k-step runs after the stage barrier
    auto first_steps = [&](const uint8_t* sa, int sset) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS - 1; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        frag_load(sa, ks + 1, (ks + 1) & 1, sset);
        mfma_step(ks & 1, sset, ks);
      }
    };
    // every wave's reads of a stage done and every wave's DMA into the other
    // stage landed: s_waitcnt vmcnt(0) lgkmcnt(0), then the barrier
    auto stage_barrier = [&]() {
      __builtin_amdgcn_s_waitcnt(0x0070);
      __syncthreads();
    };
    // Two K-tiles per iteration, stage arrays used in a fixed order so every
    // LDS access names its array directly.  With an odd tile count the last
    // K-tile (in lds0) runs after the loop, with no DMA (the loop's last
    // prefetch into lds1 reads zeros and is drained before the epilogue).
    if constexpr (M16) {
    // 16x16x32 main loop: a K-tile is 2 k-steps of 32; A fragments double
    // buffered, B fragments single and reloaded right after their last use
    bf16x8 aF[2][MB], bB[8];
    const int ch_l = lane_t >> 4;
    const int ra16 = wm * HR + (lane_t & 15), rb16 = wn * 128 + (lane_t & 15);
    auto rdA = [&](const uint8_t* sa, int ks, int i) {
      return *reinterpret_cast<const bf16x8*>(sa + swz_off(ra16 + 16 * i, 4 * ks + ch_l));
    };
    auto rdB = [&](const uint8_t* sa, int ks, int j) {
      return *reinterpret_cast<const bf16x8*>(sa + GM_TILE_BYTES + swz_off(rb16 + 16 * j, 4 * ks + ch_l));
    };
    constexpr int NJA = TBM / (8 * NW);           // == MB
    constexpr int NJB = 32 / NW;                  // 4
    static_assert(NJA == MB, "A DMA pieces");
    auto dmaA = [&](int kt, uint8_t* st, int j) {
      const bool in = kt < nk_t;
      const uint32_t vrow = (uint32_t)(wave * 8 * NJA + rl_t) * a_stride;
      const int c = pc_t ^ (rl_t ^ swz_hi((wave * NJA + j) & 3));
      lds_dma16(in ? rsA : rsZ, st + (wave * NJA + j) * 1024,
                vrow + (uint32_t)(j * 8) * a_stride + (uint32_t)(c << 4), (uint32_t)kt * 128u);
    };
    auto dmaB = [&](int kt, uint8_t* st, int j) {
      const bool in = kt < nk_t;
      const int blk = wave * NJB + j;
      if constexpr (BLAY == BL_NK) {   // K-contiguous plain B: row-strided, as A
        const uint32_t vrow = (uint32_t)(wave * 8 * NJB + rl_t) * b_stride;
        const int c = pc_t ^ (rl_t ^ swz_hi(blk & 3));
        lds_dma16(in ? rsB : rsZ, st + GM_TILE_BYTES + blk * 1024,
                  vrow + (uint32_t)(j * 8) * b_stride + (uint32_t)(c << 4), (uint32_t)kt * 128u);
      } else {                         // packed: each 1 KB piece contiguous
        lds_dma16(in ? rsB : rsZ, st + GM_TILE_BYTES + blk * 1024, (uint32_t)(blk * 1024 + lane_t * 16),
                  (uint32_t)kt * GM_TILE_BYTES);
      }
    };
    // one k-step, j (B block) outer: B fragment j is dead after its MB MFMAs
    // and is reloaded for the next k-step right away, so every reload has
    // most of the k-step to land; the next A fragments (MB of them, double
    // buffered) are read during the first MB blocks; the next stage's DMA
    // (when DMA) goes out one instruction per block.  The k-step that issues
    // the DMA (the first after a stage barrier) runs at raised wave priority:
    // of the two waves sharing a SIMD, the one that is behind keeps issuing
    // while the other, done first, has dropped back, so the pair reaches the
    // next barrier closer together (interleaved, same results: FC1 -0.8%,
    // FC2 -0.8%, dX -1.5%; the MXFP8 loop measured no gain and keeps one
    // priority).
    auto kstep = [&](auto curc, auto dmac, const uint8_t* nsa, int nks, int dkt, uint8_t* dst) {
      constexpr int cur = decltype(curc)::value;
      constexpr bool DMA = decltype(dmac)::value;
      if constexpr (DMA) __builtin_amdgcn_s_setprio(1);
      static_for<8>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j < MB) aF[cur ^ 1][j] = rdA(nsa, nks, j);
        if constexpr (DMA) {
          if constexpr (j < NJA) dmaA(dkt, dst, j);
          else if constexpr (j - NJA < NJB) dmaB(dkt, dst, j - NJA);
        }
        static_for<MB>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          acc16[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bB[j], aF[cur][i], acc16[i][j], 0, 0, 0);
        });
        bB[j] = rdB(nsa, nks, j);
        if constexpr (j < MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // A read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (DMA && j < NJA + NJB) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MB - 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                          // B reload
      });
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DMA) __builtin_amdgcn_s_setprio(0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using NoD = std::false_type;
    using D = std::true_type;
    issue_direct(0, lds0);
    stage_barrier();
    issue_direct(1, lds1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < MB; ++i) aF[0][i] = rdA(lds0, 0, i);
#pragma unroll
    for (int j = 0; j < 8; ++j) bB[j] = rdB(lds0, 0, j);
    const int nk_even16 = nk_t & ~1;
    for (int kt = 0; kt < nk_even16; kt += 2) {
      kstep(I0{}, NoD{}, lds0, 1, 0, nullptr);
      stage_barrier();
      kstep(I1{}, D{}, lds1, 0, kt + 2, lds0);
      kstep(I0{}, NoD{}, lds1, 1, 0, nullptr);
      stage_barrier();
      kstep(I1{}, D{}, lds0, 0, kt + 3, lds1);
    }
    if (nk_t & 1) {
      kstep(I0{}, NoD{}, lds0, 1, 0, nullptr);
      kstep(I1{}, NoD{}, lds0, 0, 0, nullptr);
    }
    } else if constexpr (MX8) {
    // MXFP8 operands on 8 waves: the same order on the block-scaled
    // v_mfma_scale_f32_32x32x64_f8f6f4.  A K-tile is 2 k-steps of 64 codes;
    // per k-step, B block j (outer) feeds its MI MFMAs and is re-read for the
    // next k-step at once (B single-buffered, A double-buffered), and a new
    // K-tile's scale dwords are read with its first fragments (two scale
    // sets, one per stage array).  Lane half h takes bytes 16h .. 16h + 15 of
    // each of the k-step's two 32-code blocks (chunks 4 ks + h, 4 ks + 2 + h);
    // the upper half's scale dword is shifted down one byte so that both
    // halves select byte 2 ks (block 2 ks + h).
    i32x8 aX[2][MI], bX[4];
    uint32_t sAx[2][MI], sBx[2][4];
    const int hx = lane_t >> 5;
    const int rax = wm * HR + (lane_t & 31), rbx = wn * 128 + (lane_t & 31);
    const uint32_t shx = 8u * (uint32_t)(lane >> 5);
    auto rd32x = [&](const uint8_t* t, int r, int ks) {
      const uint4 lo = *reinterpret_cast<const uint4*>(t + swz_off(r, 4 * ks + hx));
      const uint4 hi = *reinterpret_cast<const uint4*>(t + swz_off(r, 4 * ks + 2 + hx));
      i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      return v;
    };
    auto rdSAx = [&](const uint8_t* sa, int i) {
      return reinterpret_cast<const uint32_t*>(sa + 2 * GM_TILE_BYTES)[rax + 32 * i];
    };
    auto rdSBx = [&](const uint8_t* sa, int j) {
      return reinterpret_cast<const uint32_t*>(sa + 2 * GM_TILE_BYTES + 1024)[rbx + 32 * j];
    };
    constexpr int NJA = TBM / (8 * NW);           // A DMA pieces per K-tile (2 or 4)
    auto dmaA = [&](int kt, uint8_t* st, int j) {
      const bool in = kt < nk_t;
      const uint32_t vrow = (uint32_t)(wave * 8 * NJA + rl_t) * a_stride;
      const int c = pc_t ^ (rl_t ^ swz_hi((wave * NJA + j) & 3));
      lds_dma16(in ? rsA : rsZ, st + (wave * NJA + j) * 1024,
                vrow + (uint32_t)(j * 8) * a_stride + (uint32_t)(c << 4), (uint32_t)kt * 128u);
    };
    auto dmaB = [&](int kt, uint8_t* st, int j) {
      const bool in = kt < nk_t;
      const int blk = wave * 4 + j;
      lds_dma16(in ? rsB : rsZ, st + GM_TILE_BYTES + blk * 1024, (uint32_t)(blk * 1024 + lane_t * 16),
                (uint32_t)kt * GM_TILE_BYTES);
    };
    // (one instruction whose operands are selected per wave half: a branch
    // here would let the compiler sink the k-step's MFMAs past it)
    const bool sA_half = wave < 4;
    const rsrc_t rsS = sA_half ? rsSA : rsSB;
    const uint32_t s_voff = (uint32_t)((wave & 3) * 64 + lane_t) * (sA_half ? sa_stride : 4u);
    const uint32_t s_kmul = sA_half ? 4u : 1024u;
    const int s_lds = 2 * GM_TILE_BYTES + (sA_half ? 0 : 1024) + (wave & 3) * 256;
    auto dmaS = [&](int kt, uint8_t* st) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          kt < nk_t ? rsS : rsZ, (__attribute__((address_space(3))) void*)(st + s_lds), 4, s_voff,
          (uint32_t)kt * s_kmul, 0, 0);
    };
    // one k-step on A buffer CUR, scale set SET, k-step KS of its K-tile;
    // the next k-step's fragments come from (nsa, NKS), with its K-tile's
    // scales into set NSET when NEWT; DMA: K-tile dkt into dst, pieces
    // spread over the blocks (A pieces, B pieces, then the scale dword)
    auto kstepx = [&](auto curc, auto setc, auto ksc, auto dmac, auto nksc, auto nsetc, auto newtc,
                      const uint8_t* nsa, int dkt, uint8_t* dst) {
      constexpr int cur = decltype(curc)::value, set = decltype(setc)::value;
      constexpr int ks = decltype(ksc)::value, nks = decltype(nksc)::value;
      constexpr int nset = decltype(nsetc)::value;
      constexpr bool DMA = decltype(dmac)::value, NEWT = decltype(newtc)::value;
      static_for<4>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j < MI) {
          aX[cur ^ 1][j] = rd32x(nsa, rax + 32 * j, nks);
          if constexpr (NEWT) sAx[nset][j] = rdSAx(nsa, j);
        }
        if constexpr (DMA) {
          // 2 or 4 A pieces, 4 B pieces and one scale dword over 4 blocks
          if constexpr (NJA == 4) { dmaA(dkt, dst, j); dmaB(dkt, dst, j); }
          else {
            if constexpr (j < 2) dmaA(dkt, dst, j);
            dmaB(dkt, dst, j);
          }
          if constexpr (j == 3) dmaS(dkt, dst);
        }
        static_for<MI>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          const int sb = (int)(sBx[set][j] >> shx), sa_ = (int)(sAx[set][i] >> shx);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bX[j], aX[cur][i], acc[i][j], FMT_B, FMT_A, 2 * ks, sb, 2 * ks, sa_);
        });
        bX[j] = rd32x(nsa + GM_TILE_BYTES, rbx + 32 * j, nks);
        if constexpr (NEWT) sBx[nset][j] = rdSBx(nsa, j);
        if constexpr (j < MI) __builtin_amdgcn_sched_group_barrier(0x100, NEWT ? 3 : 2, 0);   // A reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (DMA) __builtin_amdgcn_sched_group_barrier(0x020, (NJA == 4 || j < 2 ? 2 : 1) + (j == 3 ? 1 : 0), 0);
        if constexpr (MI > 1) __builtin_amdgcn_sched_group_barrier(0x008, MI - 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NEWT ? 3 : 2, 0);                        // B reload
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using NoDx = std::false_type;
    using Dx = std::true_type;
    issue_direct(0, lds0);
    stage_barrier();
    issue_direct(1, lds1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      aX[0][i] = rd32x(lds0, rax + 32 * i, 0);
      sAx[0][i] = rdSAx(lds0, i);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bX[j] = rd32x(lds0 + GM_TILE_BYTES, rbx + 32 * j, 0);
      sBx[0][j] = rdSBx(lds0, j);
    }
    const int nk_evenx = nk_t & ~1;
    for (int kt = 0; kt < nk_evenx; kt += 2) {
      kstepx(C0{}, C0{}, C0{}, NoDx{}, C1{}, C0{}, std::false_type{}, lds0, 0, nullptr);
      stage_barrier();
      kstepx(C1{}, C0{}, C1{}, Dx{}, C0{}, C1{}, std::true_type{}, lds1, kt + 2, lds0);
      kstepx(C0{}, C1{}, C0{}, NoDx{}, C1{}, C1{}, std::false_type{}, lds1, 0, nullptr);
      stage_barrier();
      kstepx(C1{}, C1{}, C1{}, Dx{}, C0{}, C0{}, std::true_type{}, lds0, kt + 3, lds1);
    }
    if (nk_t & 1) {
      kstepx(C0{}, C0{}, C0{}, NoDx{}, C1{}, C0{}, std::false_type{}, lds0, 0, nullptr);
      kstepx(C1{}, C0{}, C1{}, NoDx{}, C0{}, C1{}, std::false_type{}, lds0, 0, nullptr);
    }
    } else {
    issue_direct(0, lds0);
    if (KNR) {
      kn_load(0);
      kn_store(lds0);
    }
    stage_barrier();
    issue_direct(1, lds1);
    if (KNR) kn_load(1);
    __builtin_amdgcn_sched_barrier(0);
    frag_load(lds0, 0, 0, 0);
    const int nk_even = nk_t & ~1;
    for (int kt = 0; kt < nk_even; kt += 2) {
      first_steps(lds0, 0);
      if (KNR) kn_store(lds1);
      stage_barrier();
      issue_direct(kt + 2, lds0);
      if (KNR) kn_load(kt + 2);
      frag_load(lds1, 0, 0, 1);
      mfma_step_dma(1, 0, KSTEPS - 1);   // last k-step of K-tile kt
      first_steps(lds1, 1);
      if (KNR) kn_store(lds0);
      stage_barrier();
      issue_direct(kt + 3, lds1);
      if (KNR) kn_load(kt + 3);
      frag_load(lds0, 0, 0, 0);
      mfma_step_dma(1, 1, KSTEPS - 1);   // last k-step of K-tile kt + 1
    }
    if (nk_t & 1) {   // the odd last K-tile, landed in lds0 (waited for in the loop)
      first_steps(lds0, 0);
      mfma_step(1, 0, KSTEPS - 1);
    }
    }   // neither M16 nor MX8
    // the loop leaves one DMA (a K-tile past the end: zeros) and one set of
    // fragment reads in flight; the epilogue reuses both stage arrays
    stage_barrier();
    if constexpr (M16) {
      // 16 x 16 block (2i + a, 2j + b) gives lane l rows 16a + l % 16 and
      // columns 16b + 4 (l / 16) + 0..3; the 32 x 32 block (i, j) wants lane L
      // to hold row L % 32 and columns 8q + 4 (L / 32) + 0..3.  In 16-lane rows
      // R: q = 2b takes [X0.R0, X1.R0, X0.R1, X1.R1] and q = 2b + 1 takes
      // [X0.R2, X1.R2, X0.R3, X1.R3] of the pair X_a = block (2i + a, 2j + b):
      // one v_permlane16_swap (odd rows of the first operand with even rows
      // of the second) and one v_permlane32_swap (upper half of the first with
      // lower half of the second) per register pair.
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc16[2 * i][2 * j + b][r]),
                                                                __float_as_uint(acc16[2 * i + 1][2 * j + b][r]),
                                                                false, false);
              const auto s32 = __builtin_amdgcn_permlane32_swap(s16[0], s16[1], false, false);
              acc[i][j][8 * b + r] = __uint_as_float(s32[0]);
              acc[i][j][8 * b + 4 + r] = __uint_as_float(s32[1]);
            }
    }

    // ================================================================ epilogues
    // The MFMAs compute D = W X^T per 32 x 32 block, so accumulator element r
    // of block (i, j) is
    //   tile row    m = wm*128 + 32 i + lane%32
    //   tile column n = wn*128 + 32 j + 8 (r/4) + 4 (lane/32) + r%4,
    // i.e. each lane holds runs of 4 consecutive columns of one row.
    const int z0 = opaque_zero();
    // this wave's rows (wm*HR ..) live in stage array 0 (tile rows below SHR)
    // or 1, from staged row slm - lm on
    uint16_t* wstg = reinterpret_cast<uint16_t*>(wm * HR >= SHR ? lds1 : lds0) + z0;
    const int lm = (lane & 31) + z0;
    const int slm = (wm * HR) % SHR + lm;
    const int ln = 4 * (lane >> 5) + z0;
    float rsc[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = wm * HR + 32 * i + lm;
      rsc[i] = (p.ep.row_scale && m < rows_valid) ? p.ep.row_scale[row0 + m] : 1.0f;
    }

    if constexpr (WG) {
      // fp32 C_e rows mt*256 + m, passed per 32-row block through the wave's
      // own 16.5 KB of the stage arrays (rows of 128 fp32 + 16 bytes of
      // padding) so that each store writes 2 rows x 512 contiguous bytes:
      // whole cache lines instead of 32 rows x 32 bytes, a quarter of the L2
      // write requests; with the non-temporal hint (aux bit 1 on gfx950), as
      // the output is not read again here.  Rows past wg_P are outside the descriptor and
      // dropped; columns past N are skipped; accumulate adds the current
      // contents first.
      if (!(p.accumulate && m_e == 0)) {
        constexpr int SLD = 128 * 4 + 16;               // staged row pitch (bytes)
        uint8_t* wst = (wm ? lds1 : lds0) + wn * (32 * SLD) + z0;
        const long long PQ = (long long)p.wg_P * p.N;
        const rsrc_t rsC = make_rsrc(p.Cf + (long long)e * PQ, PQ * 4);
        const int lh = (lane >> 5) + z0;
        const int q0 = n0 + wn * 128 + 4 * (lane & 31) + z0;   // read-back: chunk lane % 32
        const bool col_ok = q0 < p.N;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq)
              *reinterpret_cast<float4*>(wst + lm * SLD + (32 * j + 8 * rq + 4 * lh) * 4) =
                  make_float4(acc[i][j][4 * rq], acc[i][j][4 * rq + 1], acc[i][j][4 * rq + 2],
                              acc[i][j][4 * rq + 3]);
          const int row_base = mt * GM_BM + wm * HR + 32 * i;
#pragma unroll
          for (int s2 = 0; s2 < 16; ++s2) {
            const int r = 2 * s2 + lh;
            float4 v = *reinterpret_cast<const float4*>(wst + r * SLD + (lane & 31) * 16);
            const uint32_t off = ((uint32_t)(row_base + r) * (uint32_t)p.N + (uint32_t)q0) * 4u;
            if (col_ok) {
              if (p.accumulate) {
                const float4 o =
                    __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rsC, off, 0, 0));
                v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
              }
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsC, off, 0, 2);   // nt
            }
          }
        }
      }
      // the next tile's first DMA rewrites lds0: every wave's staging reads done
      __syncthreads();
    } else if (EPI == EPI_GLU || EPI == EPI_GLU_MX) {
      // y goes straight from registers to HBM, no LDS and no barrier.  Pair
      // wn of this tile: gate = blocks j = 0, 1; up = blocks j = 2, 3.  For
      // two column groups q = 2p, 2p + 1 a lane holds columns 8q + 4 (lane /
      // 32) .. + 3 of its row; one v_permlane32_swap per dword gives lane
      // l < 32 columns 16p .. 16p + 7 and lane l + 32 columns 16p + 8 .. 16p +
      // 15, so every lane stores 16 bytes and each row gets 32 contiguous
      // bytes per store.  Descriptors cover the tile's valid rows only: stores
      // of the rows past the group are dropped by the buffer range check.
      // The pre-activation (twice y's bytes) leaves through one staged round
      // of full-row stores instead.  With MXFP8 outputs, y is also staged (a
      // round before the pre-activation's) for the row-wise and transposed
      // quantisation.
      constexpr bool MXO = EPI == EPI_GLU_MX;
      const int cvalid_n = min(128, p.I - nt * 128);
      const bool wave_on = wn * 64 < cvalid_n;
      const long long ld2 = 2LL * p.I;
      const int lh = (lane >> 5) + z0;
      // bias of this lane's 16 gate and 16 up columns, loaded once per tile
      // (all loads in flight together)
      uint2 bgw[2][2][2], buw[2][2][2];
      const bool has_bias = p.ep.bias != nullptr;
      if (has_bias && wave_on) {
        const uint16_t* bias_e = p.ep.bias + (long long)e * ld2;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = nt * 128 + wn * 64 + 32 * jj + 8 * q + 4 * lh;
            bgw[jj][q >> 1][q & 1] = *reinterpret_cast<const uint2*>(bias_e + c);
            buw[jj][q >> 1][q & 1] = *reinterpret_cast<const uint2*>(bias_e + p.I + c);
          }
      }
      auto lo16 = [](uint32_t w) { return __uint_as_float(w << 16); };
      auto hi16 = [](uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); };
      // z = acc + bias for the 4 columns of column group q = 2 pp + h
      auto zcols = [&](int i, int jj, int pp, int h, float (&g)[4], float (&u)[4]) {
        const int q = 2 * pp + h;
        const uint2 vg = bgw[jj][pp][h], vu = buw[jj][pp][h];
        const float bg[4] = {lo16(vg.x), hi16(vg.x), lo16(vg.y), hi16(vg.y)};
        const float bu[4] = {lo16(vu.x), hi16(vu.x), lo16(vu.y), hi16(vu.y)};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          g[s2] = acc[i][jj][4 * q + s2] + (has_bias ? bg[s2] : 0.0f);
          u[s2] = acc[i][jj + 2][4 * q + s2] + (has_bias ? bu[s2] : 0.0f);
        }
      };
      // stage the pre-activation: gate at columns 0..127, up at 128..255
      auto stage_preact = [&](int i, int jj, int pp, int h, const float (&g)[4], const float (&u)[4]) {
        const int c = wn * 64 + 32 * jj + 8 * (2 * pp + h) + 4 * lh;
        uint16_t* srow = wstg + (32 * i + slm) * GM_STG_LD_256;
        *reinterpret_cast<uint2*>(srow + c) = make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]));
        *reinterpret_cast<uint2*>(srow + 128 + c) =
            make_uint2(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]));
      };
      const rsrc_t rsY = make_rsrc(p.C ? p.C + (long long)row0 * p.I : p.A,
                                   p.C ? (long long)rows_valid * p.I * 2 : 0);
      float ymax = 0.0f;                   // max |y| of this lane's valid rows
      auto body = [&]() {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            __builtin_amdgcn_sched_barrier(0);
            // byte offset of this lane's 16 bytes in row 0 of the tile
            const uint32_t ycol = (uint32_t)(wn * 64 + 32 * jj + 16 * pp + 8 * lh);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
              const int m = wm * HR + 32 * i + lm;
              uint32_t yw[2][2];
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                float o[4], g[4], u[4];
                zcols(i, jj, pp, h, g, u);
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                  const float gc = fminf(fmaxf(g[s2], p.ep.gate_lo), p.ep.gate_hi);
                  const float uc = fminf(fmaxf(u[s2], p.ep.up_lo), p.ep.up_hi) + p.ep.up_offset;
                  o[s2] = act_fwd_t<ACT>(gc, p.ep.alpha) * uc * rsc[i];
                }
                yw[h][0] = pack_bf16x2(o[0], o[1]);
                yw[h][1] = pack_bf16x2(o[2], o[3]);
                if (p.ep.amax_out && m < rows_valid) {
#pragma unroll
                  for (int w2 = 0; w2 < 2; ++w2)
                    ymax = fmaxf(ymax, fmaxf(fabsf(__uint_as_float(yw[h][w2] << 16)),
                                             fabsf(__uint_as_float(yw[h][w2] & 0xFFFF0000u))));
                }
                if (MXO) {   // y staged for the MXFP8 round (128 columns)
                  const int c = wn * 64 + 32 * jj + 8 * (2 * pp + h) + 4 * lh;
                  *reinterpret_cast<uint2*>(wstg + (32 * i + slm) * GM_STG_LD_128 + c) =
                      make_uint2(yw[h][0], yw[h][1]);
                } else if (p.preact) {
                  stage_preact(i, jj, pp, h, g, u);
                }
              }
              if (p.C) {
                const auto s0 = __builtin_amdgcn_permlane32_swap(yw[0][0], yw[1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(yw[0][1], yw[1][1], false, false);
                const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
                __builtin_amdgcn_raw_buffer_store_b128(
                    v, rsY, ((uint32_t)m * (uint32_t)p.I + (uint32_t)nt * 128 + ycol) * 2u, 0, 0);
              }
            }
          }
        }
      };
      // per row: gate columns nt*128 .. + 127 and up columns I + nt*128 ..
      // + 127, 256 contiguous bytes each, 16 bytes per lane
      auto store_preact = [&]() {
        __syncthreads();
        const Stg stg{reinterpret_cast<uint16_t*>(lds0) + z0, reinterpret_cast<uint16_t*>(lds1) + z0,
                      GM_STG_LD_256, SHR};
        uint16_t* prow0 = p.preact + (long long)row0 * ld2 + nt * 128;
        const int t = tid + z0;
#pragma unroll 4
        for (int it = t; it < TBM * 32; it += NTH) {
          const int r = it >> 5, ch = it & 31, cc = (ch & 15) * 8;
          if (r < rows_valid && cc < cvalid_n) {
            const uint4 v = *reinterpret_cast<const uint4*>(stg.row(r) + ch * 8);
            store16_nt(prow0 + r * ld2 + (ch < 16 ? 0 : p.I) + cc, v);
          }
        }
        __syncthreads();
      };
      // MXFP8 outputs: the pre-activation round first, so the accumulators
      // are dead by the time the quantisation runs
      if (MXO && p.preact) {
        if (wave_on) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
              for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  float g[4], u[4];
                  zcols(i, jj, pp, h, g, u);
                  stage_preact(i, jj, pp, h, g, u);
                }
        }
        store_preact();
      }
      if (wave_on) {
        body();
        if (p.ep.amax_out) amax_bits = max(amax_bits, wave_max_bits(ymax));   // NaN dropped by fmaxf
      }
      if (MXO) {
        __syncthreads();
        mx_from_stage<NTH>(Stg{reinterpret_cast<uint16_t*>(lds0) + z0, reinterpret_cast<uint16_t*>(lds1) + z0,
                          GM_STG_LD_128, SHR},
                      rows_valid, cvalid_n, row0, nt * 128, p, gs.mxs_off[e] + mt * 8);
        __syncthreads();
      } else if (p.preact) {
        store_preact();
      }
    } else if (EPI == EPI_ACT || EPI == EPI_DACT) {
      // Per element, from the accumulator of output column n (plain order):
      // forward  z = acc + bias[n], y = bf16(a(z) * rs), staged and stored like
      //          the plain GroupGemm output (with its MXFP8 copies), then z in
      //          a second staged round when the pre-activation is kept;
      // backward dz = bf16(acc * rs * a'(z)), z (bf16) read back 8 bytes per
      //          lane group, all 16 of a row block's loads in flight together.
      constexpr bool FWD = EPI == EPI_ACT;
      const int ld = GM_STG_LD_256;
      const Stg stg{reinterpret_cast<uint16_t*>(lds0) + z0, reinterpret_cast<uint16_t*>(lds1) + z0, ld, SHR};
      const int cvalid_n = min(GM_BN, p.N - n0);
      const uint16_t* bias_e = (FWD && p.ep.bias) ? p.ep.bias + (long long)e * p.N + n0 : nullptr;
      const rsrc_t rsZ = make_rsrc(p.preact + (long long)row0 * p.N,
                                   FWD ? 0 : (long long)rows_valid * p.N * 2);
      float ymax = 0.0f;
      auto stage_round = [&](auto rc) {   // 0: y (forward) or dz (backward); 1: z (forward)
        constexpr int RD = decltype(rc)::value;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int m = wm * HR + 32 * i + lm;
          uint2 zw[4][4];
          if constexpr (!FWD) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint32_t col = (uint32_t)(n0 + wn * 128 + 32 * j + 8 * q + ln);
                zw[j][q] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                    rsZ, ((uint32_t)m * (uint32_t)p.N + col) * 2u, 0, 0));
              }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int n = wn * 128 + 32 * j + 8 * q + ln;
              float o[4];
              if constexpr (FWD) {
                uint2 bw = make_uint2(0u, 0u);
                if (bias_e && n < cvalid_n) bw = *reinterpret_cast<const uint2*>(bias_e + n);
                const float bz[4] = {__uint_as_float(bw.x << 16), __uint_as_float(bw.x & 0xFFFF0000u),
                                     __uint_as_float(bw.y << 16), __uint_as_float(bw.y & 0xFFFF0000u)};
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                  const float z = acc[i][j][4 * q + s2] + bz[s2];
                  o[s2] = RD == 0 ? act_fwd_t<ACT>(z, p.ep.alpha) * rsc[i] : z;
                }
              } else {
                const float zv[4] = {__uint_as_float(zw[j][q].x << 16), __uint_as_float(zw[j][q].x & 0xFFFF0000u),
                                     __uint_as_float(zw[j][q].y << 16), __uint_as_float(zw[j][q].y & 0xFFFF0000u)};
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                  float a, da;
                  act_fwd_bwd_t<ACT>(zv[s2], p.ep.alpha, a, da);
                  o[s2] = acc[i][j][4 * q + s2] * rsc[i] * da;
                }
              }
              const uint2 w = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
              if (FWD && RD == 0 && p.ep.amax_out && m < rows_valid && n < cvalid_n)
                ymax = fmaxf(ymax, fmaxf(fmaxf(fabsf(__uint_as_float(w.x << 16)), fabsf(__uint_as_float(w.x & 0xFFFF0000u))),
                                         fmaxf(fabsf(__uint_as_float(w.y << 16)), fabsf(__uint_as_float(w.y & 0xFFFF0000u)))));
              *reinterpret_cast<uint2*>(wstg + (32 * i + slm) * ld + n) = w;
            }
        }
      };
      stage_round(std::integral_constant<int, 0>{});
      __syncthreads();
      if (p.C)
        store_stage<NTH>(stg, rows_valid, cvalid_n, GM_BN, p.C + (long long)row0 * p.N + n0, p.N);
      if (p.row_q || p.col_q) mx_from_stage<NTH>(stg, rows_valid, cvalid_n, row0, n0, p, gs.mxs_off[e] + mt * 8);
      if (!FWD && p.ep.amax_out) {   // rotated amax of dz^T over the tile's valid 64-column chunks
        uint32_t ok = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) ok |= (n0 + 64 * k < p.N ? 1u : 0u) << k;
        ymax = rht16_amax_stage<NTH>(stg, rows_valid, ok, p.ep.rht_signs);
      }
      __syncthreads();
      if (FWD && p.preact) {
        stage_round(std::integral_constant<int, 1>{});
        __syncthreads();
        store_stage<NTH>(stg, rows_valid, cvalid_n, GM_BN, p.preact + (long long)row0 * p.N + n0, p.N);
        __syncthreads();
      }
      if (p.ep.amax_out) amax_bits = max(amax_bits, wave_max_bits(ymax));
    } else if (EPI == EPI_STORE) {
      const int ld = GM_STG_LD_256;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_barrier(0);
            const int n = wn * 128 + 32 * j + 8 * q + ln;
            *reinterpret_cast<uint2*>(wstg + (32 * i + slm) * ld + n) =
                make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                           pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
          }
      }
      __syncthreads();
      const int cvalid_n = min(GM_BN, p.N - n0);
      if (p.C)
        store_stage<NTH>(Stg{reinterpret_cast<uint16_t*>(lds0) + z0, reinterpret_cast<uint16_t*>(lds1) + z0, ld, SHR},
                    rows_valid, cvalid_n, GM_BN, p.C + (long long)row0 * p.N + n0, p.N);
      if (p.row_q || p.col_q)
        mx_from_stage<NTH>(Stg{reinterpret_cast<uint16_t*>(lds0) + z0, reinterpret_cast<uint16_t*>(lds1) + z0, ld, SHR},
                      rows_valid, cvalid_n, row0, n0, p, gs.mxs_off[e] + mt * 8);
      __syncthreads();
    } else {  // EPI_DGLU: acc = G = dL/dy for columns n0 .. n0+255 of I
      const int ld = GM_STG_LD_256;
      const long long ld2 = 2LL * p.I;
      const int lh = (lane >> 5) + z0;
      // The saved pre-activation of this tile's rows comes in through a
      // descriptor over rows row0 .. row0 + rows_valid - 1 (rows past it read
      // zero; columns past I give values that are never stored).  Per column
      // block j all 16 loads of 16 bytes are in flight together; lane half h
      // loads columns 16p + 8h .. + 7 of the pair p, and one v_permlane32_swap
      // per dword turns that into the MFMA layout (columns 8q + 4h .. + 3).
      // Two rounds, each finishing half of every wave's columns (blocks j =
      // 2r, 2r + 1): the staged row holds [dg wn0 | dg wn1 | du wn0 | du wn1],
      // 64 columns each, and goes out as four 128-byte row segments.
      const rsrc_t rsPre = make_rsrc(p.preact + (long long)row0 * ld2,
                                     (long long)rows_valid * ld2 * 2);
      const Stg stg{reinterpret_cast<uint16_t*>(lds0) + z0, reinterpret_cast<uint16_t*>(lds1) + z0, ld, SHR};
      // d(row_scale): per block j and row block, each lane sums G * a(g_c) *
      // u_c (dL/dy times the unscaled y) over its 16 columns and adds that
      // to the row's LDS slot; after the tile one global atomic per row
      constexpr bool PG = EPI == EPI_DGLU_G;
      const bool want_drs = PG && p.ep.drs_out != nullptr;
      if (want_drs) {
        for (int r = tid; r < TBM; r += NTH) drs_lds[r] = 0.0f;
        __syncthreads();
      }
      auto do_block = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        // (a select, not a branch: the block stays one scheduling region)
        const bool drs_j = want_drs && n0 + wn * WBN + 32 * j < p.I;   // whole block (I % 64 == 0)
        u32x4 lg[MI][2], lu[MI][2];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const uint32_t rowb = (uint32_t)(wm * HR + 32 * i + lm) * (uint32_t)ld2 * 2u;
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const uint32_t col = (uint32_t)(n0 + wn * WBN + 32 * j + 16 * pp + 8 * lh);
            lg[i][pp] = __builtin_amdgcn_raw_buffer_load_b128(rsPre, rowb + col * 2u, 0, 0);
            lu[i][pp] = __builtin_amdgcn_raw_buffer_load_b128(
                rsPre, rowb + (col + (uint32_t)p.I) * 2u, 0, 0);
          }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          uint16_t* srow = wstg + (32 * i + slm) * ld;
          float drs_part = 0.0f;
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            // w[h2][d]: dword d (columns 2d, 2d+1) of column group q = 2pp + h2
            uint32_t gw[2][2], uw[2][2];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const auto sg = __builtin_amdgcn_permlane32_swap(lg[i][pp][d], lg[i][pp][d + 2], false, false);
              const auto su = __builtin_amdgcn_permlane32_swap(lu[i][pp][d], lu[i][pp][d + 2], false, false);
              gw[0][d] = sg[0]; gw[1][d] = sg[1];
              uw[0][d] = su[0]; uw[1][d] = su[1];
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const int q = 2 * pp + h2;
              const float gv[4] = {__uint_as_float(gw[h2][0] << 16), __uint_as_float(gw[h2][0] & 0xFFFF0000u),
                                   __uint_as_float(gw[h2][1] << 16), __uint_as_float(gw[h2][1] & 0xFFFF0000u)};
              const float uv[4] = {__uint_as_float(uw[h2][0] << 16), __uint_as_float(uw[h2][0] & 0xFFFF0000u),
                                   __uint_as_float(uw[h2][1] << 16), __uint_as_float(uw[h2][1] & 0xFFFF0000u)};
              float dg[4], du[4];
#pragma unroll
              for (int s2 = 0; s2 < 4; ++s2) {
                const float Gu = acc[i][j][4 * q + s2];
                const float G = Gu * rsc[i];
                const float g = gv[s2], u = uv[s2];
                const float gc = fminf(fmaxf(g, p.ep.gate_lo), p.ep.gate_hi);
                const float uc = fminf(fmaxf(u, p.ep.up_lo), p.ep.up_hi) + p.ep.up_offset;
                float a, da;
                act_fwd_bwd_t<ACT>(gc, p.ep.alpha, a, da);
                const bool gin = (g >= p.ep.gate_lo) && (g <= p.ep.gate_hi);
                const bool uin = (u >= p.ep.up_lo) && (u <= p.ep.up_hi);
                dg[s2] = gin ? G * uc * da : 0.0f;
                du[s2] = uin ? G * a : 0.0f;
                if constexpr (PG) drs_part += Gu * (a * uc);
              }
              // staged column: wave's 64-column half (j & 1) at chunk wn (dg) / 2 + wn (du)
              const int sc = wn * 64 + 32 * (j & 1) + 8 * q + ln;
              *reinterpret_cast<uint2*>(srow + sc) =
                  make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
              *reinterpret_cast<uint2*>(srow + 128 + sc) =
                  make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
            }
          }
          if (PG && drs_j) atomicAdd(&drs_lds[wm * HR + 32 * i + lm], drs_part);   // LDS add
        }
      };
      // (accumulator indices must stay compile-time constants, or the
      // accumulators move to scratch memory: every block index is a template
      // constant and both rounds are written out)
      auto stage_round = [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        __builtin_amdgcn_sched_barrier(0);
        do_block(std::integral_constant<int, 2 * R>{});
        __builtin_amdgcn_sched_barrier(0);
        do_block(std::integral_constant<int, 2 * R + 1>{});
        __builtin_amdgcn_sched_barrier(0);
      };
      float hmax = 0.0f;   // rotated amax of this thread's share of the tile
      constexpr int NROUND = NBW / 2;   // (quarter tiles: one round)
#pragma unroll NROUND
      for (int round = 0; round < NROUND; ++round) {
        if (round == 0) stage_round(std::integral_constant<int, 0>{});
        else if constexpr (NBW == 4) stage_round(std::integral_constant<int, 1>{});
        __syncthreads();
        // staged chunk k (64 columns): dg (k < 2) or du, of wave half wn = k & 1;
        // its first global column of I is n0 + WBN (k & 1) + 64 round
        auto chunk_col = [&](int k) { return n0 + WBN * (k & 1) + 64 * round; };
        if (p.ep.amax_out) {
          const uint32_t ok = (chunk_col(0) < p.I ? 5u : 0u) | (chunk_col(1) < p.I ? 10u : 0u);
          hmax = fmaxf(hmax, rht16_amax_stage<NTH>(stg, rows_valid, ok, p.ep.rht_signs));
        }
        if (PG && p.ep.dbias_out) {
          // d(bias): thread t of a 256-thread group sums staged column t
          // (chunk t / 64) over the tile's valid rows (bf16 values as
          // written), one atomic per column and group; with 8 waves the two
          // groups take one staged row half each
          constexpr int NGRP = NTH / 256;
          static_assert(NGRP == 1 || NGRP == 2, "d(bias) column sums: 4 or 8 waves");
          const int t = (tid + z0) & 255, grp_half = (tid + z0) >> 8;
          const int k = t >> 6, c = chunk_col(k) + (t & 63);
          if (c < p.I) {
            // 8 rows per step, 4 partial sums: the loads run ahead of the adds
            float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              if (NGRP == 2 && hh != grp_half) continue;
              const uint16_t* col = (hh ? stg.h1 : stg.h0) + k * 64 + (t & 63);
              const int nr = min(SHR, rows_valid - hh * SHR);
              int r = 0;
              for (; r + 8 <= nr; r += 8) {
#pragma unroll
                for (int u = 0; u < 8; ++u) s4[u & 3] += bf16_to_f32(col[(r + u) * ld]);
              }
              for (; r < nr; ++r) s4[0] += bf16_to_f32(col[r * ld]);
            }
            atomicAdd(p.ep.dbias_out + (long long)e * ld2 + (k < 2 ? 0 : p.I) + c,
                      (s4[0] + s4[1]) + (s4[2] + s4[3]));
          }
        }
        if (p.C) {
          const int t = tid + z0;
#pragma unroll 4
          for (int it = t; it < TBM * 32; it += NTH) {
            const int r = it >> 5, k = (it >> 3) & 3, pc = it & 7;
            const int c = chunk_col(k) + pc * 8;
            if (r < rows_valid && c < p.I) {
              const uint4 v = *reinterpret_cast<const uint4*>(stg.row(r) + k * 64 + pc * 8);
              store16_nt(p.C + (long long)(row0 + r) * ld2 + (k < 2 ? 0 : p.I) + c, v);
            }
          }
        }
        if (p.row_q || p.col_q) {
          // the four staged 64-column chunks in one pass: chunk k is output
          // column (k < 2 ? 0 : I) + chunk_col(k) on, if inside I (I % 64 == 0)
          const int g0 = chunk_col(0) < p.I ? chunk_col(0) : -1;
          const int g1 = chunk_col(1) < p.I ? chunk_col(1) : -1;
          const int g2 = g0 < 0 ? -1 : p.I + g0, g3 = g1 < 0 ? -1 : p.I + g1;
          mx_from_stage_map<NTH>(stg, rows_valid, 256, row0, p, gs.mxs_off[e] + mt * 8, [=](int c) {
            const int k = c >> 6;
            const int g = k == 0 ? g0 : (k == 1 ? g1 : (k == 2 ? g2 : g3));
            return g < 0 ? -1 : g + (c & 63);
          });
        }
        __syncthreads();
      }
      if (p.ep.amax_out) amax_bits = max(amax_bits, wave_max_bits(hmax));
      if (want_drs) {   // (the rounds end with a barrier: every LDS add is in)
        for (int r = tid; r < rows_valid; r += NTH) atomicAdd(p.ep.drs_out + row0 + r, drs_lds[r]);
        __syncthreads();
      }
    }
    };  // tile_body
    if constexpr (WG) {
      tile_body(std::integral_constant<int, 4>{}, std::integral_constant<int, 4>{});
    } else {
      using NB4 = std::integral_constant<int, 4>;
      if (rows_valid <= 128) {
        if constexpr (QTILE) tile_body(std::integral_constant<int, 8 / NW>{}, std::integral_constant<int, 2>{});
        else tile_body(std::integral_constant<int, 8 / NW>{}, NB4{});
      } else {
        tile_body(std::integral_constant<int, 16 / NW>{}, NB4{});
      }
    }
  }
  if (p.ep.amax_out && lane == 0) atomicMax(reinterpret_cast<unsigned int*>(p.ep.amax_out), amax_bits);
}

}  // namespace moe
