// Memory-bound kernels around the grouped GEMM: the offline gate/up repack,
// device routing and grouping, the unfused GLU pass and the standalone MXFP8
// quantize/transpose.  All are bandwidth kernels: 16-byte coalesced accesses,
// LDS only where a transpose needs it.
#pragma once

#include "device_common.hpp"

namespace moe {

// ---------------------------------------------------------------- weight packing
// Packed row of plain FC1 column j ("Boosting MoE Training Throughput…",
// section "Optimizando GLU…", Figure 2: one tile holds half a tile width of the
// gate and of the input/up columns).  128-row block p = gate columns 64p..64p+63
// then up columns I+64p..I+64p+63; this is the inverse map (packed row -> j).
__device__ __forceinline__ int plain_col_of_packed(int pr, int I) {
  const int pair = pr >> 7, s = pr & 127;
  return s < 64 ? pair * 64 + s : I + pair * 64 + (s - 64);
}

// 16-byte chunk key of the tile-blocked layout (include/moe_glu.h): the same
// XOR the GEMM uses for its LDS operand tiles.
__device__ __forceinline__ int pack_key(int r) { return (r & 7) ^ ((r >> 3) & 3); }

enum { PACK_NK = 0, PACK_KN = 1, PACK_GATEUP = 2, UNPACK_GATEUP = 3 };

// One workgroup per 256 x 64 destination block (grid: K/64, ceil(N/256), E).
// The block is assembled as tile[n][k] in LDS and then written in the
// blocked, swizzled order (or, for UNPACK_GATEUP, read in that order and
// scattered back to the plain [E][H][2I] layout).
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ src,
                                                   uint16_t* __restrict__ dst, int N, int K,
                                                   int mode, int I) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[256][72];
  const int kb = blockIdx.x, nb = blockIdx.y, e = blockIdx.z;
  const int t = threadIdx.x;
  const int KB = K >> 6;
  const long long pe = (long long)((N + 255) / 256) * 256 * K;       // packed expert stride
  uint16_t* pblk = (mode == UNPACK_GATEUP ? const_cast<uint16_t*>(src) : dst) + (long long)e * pe +
                   ((long long)nb * KB + kb) * 16384;
  if (mode == UNPACK_GATEUP) {
    for (int it = t; it < 2048; it += 256) {
      const int r = it >> 3, pc = it & 7, c = pc ^ pack_key(r);
      *reinterpret_cast<uint4*>(&tile[r][c * 8]) = reinterpret_cast<const uint4*>(pblk)[it];
    }
    __syncthreads();
    // plain W1 [E][H][2I]: row k = 64 kb + kk, 8 packed rows -> 8 consecutive plain columns
    uint16_t* w = dst + (long long)e * K * N;
    for (int it = t; it < 2048; it += 256) {
      const int kk = it >> 5, cc = it & 31, r0 = cc * 8, pr = nb * 256 + r0;
      if (pr >= N) continue;
      uint4 v;
      uint16_t* pv = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
      for (int q = 0; q < 8; ++q) pv[q] = tile[r0 + q][kk];
      *reinterpret_cast<uint4*>(w + (long long)(kb * 64 + kk) * N + plain_col_of_packed(pr, I)) = v;
    }
    return;
  }
  if (mode == PACK_NK) {
    const uint16_t* w = src + (long long)e * N * K;
    for (int it = t; it < 2048; it += 256) {
      const int r = it >> 3, c = it & 7, n = nb * 256 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < N) v = *reinterpret_cast<const uint4*>(w + (long long)n * K + kb * 64 + c * 8);
      *reinterpret_cast<uint4*>(&tile[r][c * 8]) = v;
    }
  } else {  // PACK_KN and PACK_GATEUP: source [K][N]-major rows, 8 consecutive n per chunk
    const uint16_t* w = src + (long long)e * K * N;
    for (int it = t; it < 2048; it += 256) {
      const int kk = it >> 5, cc = it & 31, r0 = cc * 8, pr = nb * 256 + r0;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (pr < N) {
        const int col = mode == PACK_GATEUP ? plain_col_of_packed(pr, I) : pr;
        v = *reinterpret_cast<const uint4*>(w + (long long)(kb * 64 + kk) * N + col);
      }
      const uint16_t* pv = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
      for (int q = 0; q < 8; ++q) tile[r0 + q][kk] = pv[q];
    }
  }
  __syncthreads();
  for (int it = t; it < 2048; it += 256) {
    const int r = it >> 3, pc = it & 7, c = pc ^ pack_key(r);
    reinterpret_cast<uint4*>(pblk)[it] = *reinterpret_cast<const uint4*>(&tile[r][c * 8]);
  }
}

// ---------------------------------------------------------------- routing
// Top-k of one token's logits ([MEGA] §2.1), ties to the lower expert id:
// a candidate enters when it beats the current k-th entry, or equals it with a
// lower id.  One thread per token.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int* __restrict__ ids_out) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float val[16];
  int id[16];
  for (int j = 0; j < 16; ++j) { val[j] = -INFINITY; id[j] = 0x7FFFFFFF; }
  const float* lg = logits + (long long)t * E;
  for (int e = 0; e < E; ++e) {
    float v = lg[e];
    bool better = (v > val[k - 1]) || (v == val[k - 1] && e < id[k - 1]);
    if (!better) continue;
    int pos = k - 1;
    while (pos > 0 && ((v > val[pos - 1]) || (v == val[pos - 1] && e < id[pos - 1]))) {
      val[pos] = val[pos - 1];
      id[pos] = id[pos - 1];
      --pos;
    }
    val[pos] = v;
    id[pos] = e;
  }
  for (int j = 0; j < k; ++j) ids_out[(long long)t * k + j] = id[j];
}

// Counting sort of the T*k (token, slot) pairs by expert, stable in (t, j)
// order ([MEGA] §4.3: rows for one expert contiguous).  One workgroup of 1024
// threads: LDS histogram, exclusive scan, then each wave ranks the pairs of
// its experts with ballots (order-independent of scheduling, so bit-exact).
__global__ __launch_bounds__(1024) void group_kernel(const int* __restrict__ ids, int TK, int k,
                                                     int E, int* __restrict__ counts,
                                                     int* __restrict__ offsets,
                                                     int* __restrict__ dst, int* __restrict__ src) {
  __shared__ int hist[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += 1024) hist[e] = 0;
  __syncthreads();
  for (int p = t; p < TK; p += 1024) {
    int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) { off[e] = run; run += hist[e]; }
    off[E] = run;
  }
  __syncthreads();
  for (int e = t; e < E; e += 1024) counts[e] = hist[e];
  for (int e = t; e <= E; e += 1024) offsets[e] = off[e];
  const int lane = t & 63, wave = t >> 6;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = wave; e < E; e += 16) {
    int base = off[e];
    for (int c = 0; c < TK; c += 64) {
      int p = c + lane;
      bool m = p < TK && ids[p] == e;
      unsigned long long mask = __ballot(m);
      if (m) {
        int r = base + __popcll(mask & below);
        dst[p] = r;
        src[r] = p / k;
      }
      base += __popcll(mask);
    }
  }
}

// xg[r] = x[src[r]]: one 16-byte chunk per thread.
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ x,
                                                     const int* __restrict__ src, int R, int H,
                                                     uint16_t* __restrict__ xg) {
  const int cpr = H >> 3;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long total = (long long)R * cpr;
  for (; i < total; i += (long long)gridDim.x * blockDim.x) {
    int r = (int)(i / cpr), ch = (int)(i - (long long)r * cpr);
    int s = src[r];
    *reinterpret_cast<uint4*>(xg + (long long)r * H + ch * 8) =
        *reinterpret_cast<const uint4*>(x + (long long)s * H + ch * 8);
  }
}

// ---------------------------------------------------------------- unfused GLU
// y = GLU epilogue of the plain-order FC1 output z [M_cap][2I] (+ bias), one
// 8-column chunk per thread per step; rows beyond the groups are skipped.
// Each workgroup scans the counts to find row ranges and experts.
__global__ __launch_bounds__(256) void glu_unfused_kernel(const uint16_t* __restrict__ z,
                                                          const int* __restrict__ counts, int E,
                                                          int M_cap, int I, EpiParams ep,
                                                          uint16_t* __restrict__ y) {
  __shared__ GroupScan gs;
  build_group_scan<256>(gs, counts, E, M_cap, 1, 0, nullptr, nullptr, false);
  const int M = gs.row_off[E];
  const int cpr = I >> 3;
  long long total = (long long)M * cpr;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (long long)gridDim.x * 256) {
    int r = (int)(i / cpr), ch = (int)(i - (long long)r * cpr);
    const uint16_t* zr = z + (long long)r * 2 * I;
    uint4 gv = *reinterpret_cast<const uint4*>(zr + ch * 8);
    uint4 uv = *reinterpret_cast<const uint4*>(zr + I + ch * 8);
    const uint16_t* g16 = reinterpret_cast<const uint16_t*>(&gv);
    const uint16_t* u16 = reinterpret_cast<const uint16_t*>(&uv);
    float bg[8] = {0, 0, 0, 0, 0, 0, 0, 0}, bu[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (ep.bias) {
      int lo = 0, hi = E;  // expert of row r: last e with row_off[e] <= r and rows in it
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (gs.row_off[mid] <= r) lo = mid; else hi = mid;
      }
      const uint16_t* b = ep.bias + (long long)lo * 2 * I;
      uint4 bgv = *reinterpret_cast<const uint4*>(b + ch * 8);
      uint4 buv = *reinterpret_cast<const uint4*>(b + I + ch * 8);
      const uint16_t* bg16 = reinterpret_cast<const uint16_t*>(&bgv);
      const uint16_t* bu16 = reinterpret_cast<const uint16_t*>(&buv);
#pragma unroll
      for (int q = 0; q < 8; ++q) { bg[q] = bf16_to_f32(bg16[q]); bu[q] = bf16_to_f32(bu16[q]); }
    }
    float rs = ep.row_scale ? ep.row_scale[r] : 1.0f;
    uint4 out;
    uint16_t* o16 = reinterpret_cast<uint16_t*>(&out);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float g = bf16_to_f32(g16[q]) + bg[q];
      float u = bf16_to_f32(u16[q]) + bu[q];
      float gc = fminf(fmaxf(g, ep.gate_lo), ep.gate_hi);
      float uc = fminf(fmaxf(u, ep.up_lo), ep.up_hi) + ep.up_offset;
      float v = act_fwd(ep.act, gc, ep.alpha) * uc;
      if (ep.row_scale) v *= rs;
      o16[q] = f32_to_bf16(v);
    }
    *reinterpret_cast<uint4*>(y + (long long)r * I + ch * 8) = out;
  }
}

// ---------------------------------------------------------------- MXFP8 quantize
__device__ __forceinline__ void store_q32(uint8_t* dst, const uint32_t* w, int nvalid) {
  uintptr_t a = reinterpret_cast<uintptr_t>(dst);
  if (nvalid == 32 && (a & 15) == 0) {
    uint4* d = reinterpret_cast<uint4*>(dst);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    for (int i = 0; i < nvalid; ++i) dst[i] = static_cast<uint8_t>(w[i >> 2] >> (8 * (i & 3)));
  }
}

// Row-wise: one thread per (row, 32-column block) over rows [0, R_used).
__global__ __launch_bounds__(256) void mx_rows_kernel(const uint16_t* __restrict__ v, int R, int C,
                                                      const int* __restrict__ counts, int E,
                                                      uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ s, int e5) {
  __shared__ GroupScan gs;
  int Ruse = R;
  if (counts) {
    build_group_scan<256>(gs, counts, E, R, 1, 0, nullptr, nullptr, false);
    Ruse = gs.row_off[E];
  }
  const int nb = C >> 5;
  long long total = (long long)Ruse * nb;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (long long)gridDim.x * 256) {
    int r = (int)(i / nb), cb = (int)(i - (long long)r * nb);
    const uint4* src = reinterpret_cast<const uint4*>(v + (long long)r * C + cb * 32);
    float x[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 u = src[c];
      uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * c + 2 * j] = __uint_as_float(ww[j] << 16);
        x[8 * c + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
      }
    }
    uint32_t w[8];
    uint8_t sb = mx_quant32(x, 32, w, e5 != 0);
    store_q32(q + (long long)r * C + cb * 32, w, 32);
    s[(long long)r * nb + cb] = sb;
  }
}

// Column-wise: one thread per (column, 32-row block); blocks restart at each
// group's first row (with counts) or run over all R rows (without).  Grid.y
// walks blocks; grid.x covers columns in 256-column chunks.
__global__ __launch_bounds__(256) void mx_cols_kernel(const uint16_t* __restrict__ v, int R, int C,
                                                      const int* __restrict__ counts, int E,
                                                      uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ s, int s_ld, int e5) {
  __shared__ GroupScan gs;
  int nblocks;
  if (counts) {
    build_group_scan<256>(gs, counts, E, R, 1, 0, nullptr, nullptr, false);
    nblocks = gs.mxs_off[E];
  } else {
    nblocks = (R + 31) >> 5;
  }
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  for (int b = blockIdx.y; b < nblocks; b += gridDim.y) {
    int r0, nvalid;
    if (counts) {
      int lo = 0, hi = E;  // group owning scale column b: last e with mxs_off[e] <= b
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (gs.mxs_off[mid] <= b) lo = mid; else hi = mid;
      }
      int blk = b - gs.mxs_off[lo];
      r0 = gs.row_off[lo] + blk * 32;
      nvalid = min(32, gs.row_off[lo + 1] - r0);
    } else {
      r0 = b * 32;
      nvalid = min(32, R - r0);
    }
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = (i < nvalid) ? bf16_to_f32(v[(long long)(r0 + i) * C + c]) : 0.0f;
    uint32_t w[8];
    uint8_t sb = mx_quant32(x, nvalid, w, e5 != 0);
    store_q32(q + (long long)c * R + r0, w, nvalid);
    s[(long long)c * s_ld + b] = sb;
  }
}

// ---------------------------------------------------------------- MXFP8 weight pack
// Offline quantisation of a bf16 weight to MXFP8 along K, written in the
// tile-blocked order the block-scaled GEMM streams: per expert, blocks of 256
// rows (output columns n) x 128 K bytes (32 KB), block (nb, kb) at
// (nb * K/128 + kb) * 32768 bytes, the 16-byte chunk c of row r at
// 16 * (c ^ key(r)); the four E8M0 scales of row r in block (nb, kb) form the
// dword at ((nb * K/128 + kb) * 256 + r) * 4 of the scale array (byte b: K
// values kb * 128 + 32 b .. + 31).  Rows past N are zero with scale byte 0.
// Grid (K/128, ceil(N/256), E), one thread per row.
// gate_up_I > 0: the packed rows are W1's gate/up-interleaved columns (row n
// of the packed order holds plain column plain_col_of_packed(n, I); src is
// [E][K = H][N = 2I]).
__global__ __launch_bounds__(256) void pack_mx_kernel(const uint16_t* __restrict__ src,
                                                      uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ sc, int N, int K,
                                                      int src_kn, int gate_up_I) {
  const int kb = blockIdx.x, nb = blockIdx.y, e = blockIdx.z;
  const int nk = gridDim.x, NB = gridDim.y;
  const int r = threadIdx.x, n_pk = nb * 256 + r;
  const int n = (gate_up_I > 0 && n_pk < N) ? plain_col_of_packed(n_pk, gate_up_I) : n_pk;
  const uint16_t* W = src + (long long)e * N * K;
  const long long blk = ((long long)e * NB + nb) * nk + kb;
  uint8_t* row = q + blk * 32768 + r * 128;
  uint32_t sword = 0;
  for (int b = 0; b < 4; ++b) {
    float v[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const long long k = (long long)kb * 128 + b * 32 + t;
      v[t] = n_pk < N ? bf16_to_f32(src_kn ? W[k * N + n] : W[(long long)n * K + k]) : 0.0f;
    }
    uint32_t w[8];
    sword |= (uint32_t)mx_quant32(v, 32, w, false) << (8 * b);
    *reinterpret_cast<uint4*>(row + (((2 * b) ^ pack_key(r)) << 4)) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(row + (((2 * b + 1) ^ pack_key(r)) << 4)) = make_uint4(w[4], w[5], w[6], w[7]);
  }
  reinterpret_cast<uint32_t*>(sc)[blk * 256 + r] = sword;
}

}  // namespace moe
