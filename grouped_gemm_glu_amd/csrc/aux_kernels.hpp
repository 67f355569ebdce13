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
__device__ __forceinline__ int pack_key(int r) { return (r & 7) ^ (((r >> 2) & 2) | ((r >> 4) & 1)); }

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
    // thread t: k rows 8 kg .. + 7 (kg = t / 32) x n chunk cc = t % 32 (8 values);
    // eight 16-byte loads (a wave reads 2 x 512 contiguous bytes per load),
    // an 8 x 8 transpose of the 16-bit values in registers, eight 16-byte
    // LDS writes tile[n][8 kg .. + 7]
    const uint16_t* w = src + (long long)e * K * N;
    const int kg = t >> 5, cc = t & 31, r0 = cc * 8, pr = nb * 256 + r0;
    uint32_t in[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (pr < N) {
        const int col = mode == PACK_GATEUP ? plain_col_of_packed(pr, I) : pr;
        v = *reinterpret_cast<const uint4*>(w + (long long)(kb * 64 + kg * 8 + i) * N + col);
      }
      in[i][0] = v.x; in[i][1] = v.y; in[i][2] = v.z; in[i][3] = v.w;
    }
    // out word d of n = r0 + j: k = 8 kg + 2d (low half), 8 kg + 2d + 1 (high)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = (in[2 * d][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const uint32_t hi = (in[2 * d + 1][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        o[d] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(&tile[r0 + j][kg * 8]) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  __syncthreads();
  for (int it = t; it < 2048; it += 256) {
    const int r = it >> 3, pc = it & 7, c = pc ^ pack_key(r);
    reinterpret_cast<uint4*>(pblk)[it] = *reinterpret_cast<const uint4*>(&tile[r][c * 8]);
  }
}

// ---------------------------------------------------------------- routing
// Top-k of one token's logits ([MEGA] §2.1), ties to the lower expert id.
// The order is (logit descending, id ascending) with NaN below every number
// (numpy's sort order).  One token per group of L lanes (64 / L tokens per
// wave); lane l of a group holds logits l, l + L, ... (at most 16, E <= 1024).
// Each of the k rounds takes every lane's best untaken value, reduces it over
// the group with xor shuffles, and marks the winner taken in its owner lane.
__device__ __forceinline__ bool topk_before(float v, int e, float w, int f) {
  const bool vn = v != v, wn = w != w;
  if (vn) return wn && e < f;
  if (wn) return true;
  return v > w || (v == w && e < f);
}
template <int L>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int* __restrict__ ids_out) {
  const int lane = threadIdx.x & 63;
  const int gl = lane % L;
  const long long tok = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / L) + lane / L;
  const bool tv = tok < T;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = gl + L * i;
    v[i] = (tv && e < E) ? logits[tok * E + e] : __builtin_nanf("");
  }
  uint32_t taken = 0;
  for (int j = 0; j < k; ++j) {
    float bv = __builtin_nanf("");
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = gl + L * i;
      const bool cand = e < E && !((taken >> i) & 1u) && topk_before(v[i], e, bv, be);
      bv = cand ? v[i] : bv;
      be = cand ? e : be;
    }
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      const bool b = topk_before(ov, oe, bv, be);
      bv = b ? ov : bv;
      be = b ? oe : be;
    }
    if (be % L == gl) taken |= 1u << (be / L);
    if (tv && gl == 0) ids_out[tok * k + j] = be;
  }
}

// Grouping: a counting sort of the T*k (token, slot) pairs by expert, stable in
// (t, j) order ([MEGA] §4.3: rows for one expert contiguous).  Pairs whose id
// is outside [0, E) are not grouped.  Chunks of C pairs (C = max(1024, a power
// of two >= 2E), one workgroup each):
//   group_count_kernel  per-chunk expert counts -> cnt[c][e]
//   group_scan_kernel   counts, offsets, and cnt[c][e] = the number of pairs
//                       of expert e in the chunks before c
//   group_rank_kernel   dst[p] = that base + the pair's rank among the chunk's
//                       earlier pairs of its expert
//   group_scatter_kernel src[dst[p]] = token of p, and the gathered rows
// A single chunk skips the first two: the rank kernel scans its own counts.
// With several chunks cnt lives in src, which holds T*k >= chunks x E entries
// (T*k > C (chunks - 1) >= 2E (chunks - 1)), and is overwritten only by the
// scatter, after the rank kernel has read it.  Ranks depend only on the pair
// order, so the result is bit-exact.
__global__ __launch_bounds__(256) void group_count_kernel(const int* __restrict__ ids, int TK,
                                                          int E, int C, int* __restrict__ cnt) {
  __shared__ int h[kMaxExperts];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int p1 = min(TK, (blockIdx.x + 1) * C);
  for (int p0 = blockIdx.x * C; p0 < p1; p0 += 2048) {
    int e8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + 256 * j + t;
      e8[j] = p < p1 ? ids[p] : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (e8[j] >= 0 && e8[j] < E) atomicAdd(&h[e8[j]], 1);
  }
  __syncthreads();
  for (int e = t; e < E; e += 256) cnt[(long long)blockIdx.x * E + e] = h[e];
}

__global__ __launch_bounds__(1024) void group_scan_kernel(int nchunks, int E, int* __restrict__ cnt,
                                                          int* __restrict__ counts,
                                                          int* __restrict__ offsets) {
  __shared__ long long wave_tmp[16];
  const int t = threadIdx.x;
  int tot = 0;
  if (t < E) {
    for (int c0 = 0; c0 < nchunks; c0 += 8) {   // 8 loads in flight
      int v8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v8[j] = c0 + j < nchunks ? cnt[(long long)(c0 + j) * E + t] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (c0 + j < nchunks) cnt[(long long)(c0 + j) * E + t] = tot;
        tot += v8[j];
      }
    }
  }
  const int incl = block_incl_scan<1024, int>(tot, wave_tmp);
  if (t < E) {
    counts[t] = tot;
    offsets[t] = incl - tot;
  }
  if (t == 1023) offsets[E] = incl;   // threads past E hold 0: incl is the total
}

// One chunk per workgroup of 4 waves; wave w ranks the chunk's quarter w, 64
// pairs at a time: a ballot loop over the distinct experts of the 64 pairs
// gives every lane its rank among the lanes below with the same expert and
// the lowest such lane (the leader) the 64 pairs' count of that expert; the
// leaders read and advance their experts' counters (distinct addresses) and
// every lane takes its leader's base by a lane permute.  The chunk's first row
// of expert e is offsets[e] + base[chunk][e]; base == nullptr: the only chunk,
// whose expert bases come from a scan of its own counts, which also gives
// counts and offsets.
__global__ __launch_bounds__(256) void group_rank_kernel(const int* __restrict__ ids, int TK, int E,
                                                         int C, const int* __restrict__ base,
                                                         int* __restrict__ dst, int* __restrict__ counts,
                                                         int* __restrict__ offsets) {
  __shared__ int ctr[4][kMaxExperts];
  __shared__ long long wave_tmp[16];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q = C / 4;
  const int s0 = min(TK, blockIdx.x * C + wave * q);
  const int s1 = min(TK, s0 + q);
  for (int i = t; i < 4 * kMaxExperts; i += 256) (&ctr[0][0])[i] = 0;
  __syncthreads();
  for (int p0 = s0; p0 < s1; p0 += 512) {
    int e8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + 64 * j + lane;
      e8[j] = p < s1 ? ids[p] : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (e8[j] >= 0 && e8[j] < E) atomicAdd(&ctr[wave][e8[j]], 1);
  }
  __syncthreads();
  if (base == nullptr) {
    // experts 4t .. 4t + 3: chunk totals, a block scan of their sums, and the
    // running prefix inside the thread's four
    int tot4[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * t + i;
      tot4[i] = e < E ? ctr[0][e] + ctr[1][e] + ctr[2][e] + ctr[3][e] : 0;
      sum += tot4[i];
    }
    const int incl = block_incl_scan<256, int>(sum, wave_tmp);
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * t + i;
      if (e < E) {
        counts[e] = tot4[i];
        offsets[e] = run;
        for (int w = 0; w < 4; ++w) {
          const int c = ctr[w][e];
          ctr[w][e] = run;
          run += c;
        }
      }
    }
    if (t == 255) offsets[E] = incl;
  } else {
    for (int e = t; e < E; e += 256) {   // per-wave bases from the chunk's base
      int run = offsets[e] + base[(long long)blockIdx.x * E + e];
      for (int w = 0; w < 4; ++w) {
        const int c = ctr[w][e];
        ctr[w][e] = run;
        run += c;
      }
    }
  }
  __syncthreads();
  int* my = ctr[wave];
  for (int p0 = s0; p0 < s1; p0 += 512) {
    int e8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + 64 * j + lane;
      e8[j] = p < s1 ? ids[p] : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + 64 * j + lane;
      const int e = e8[j];
      const bool valid = e >= 0 && e < E;
      unsigned long long pending = __ballot(valid);
      int rank = 0, leader = 0, n_e = 0;
      // (selects, not branches: the loop body stays one basic block)
      while (pending) {
        const int ld = __builtin_ctzll(pending);
        const int el = __builtin_amdgcn_readlane(e, ld);
        const bool in = e == el;
        const unsigned long long m = __ballot(in);
        pending &= ~m;
        const int rk = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        rank = in ? rk : rank;
        leader = in ? ld : leader;
        n_e = lane == ld ? __popcll(m) : n_e;
      }
      int b = 0;
      if (valid && lane == leader) {
        b = my[e];
        my[e] = b + n_e;
      }
      b = __shfl(b, leader, 64);
      if (valid) dst[p] = b + rank;
    }
  }
}

// src[dst[p]] = p / k for the grouped pairs p, and with x given the gathered
// row xg[dst[p]] = x[p / k]: one wave per pair, 16 bytes per lane.
__global__ __launch_bounds__(256) void group_scatter_kernel(const int* __restrict__ ids, int TK,
                                                            int k, int E, const int* __restrict__ dst,
                                                            const int* __restrict__ offsets,
                                                            int* __restrict__ src,
                                                            const uint16_t* __restrict__ x, int H,
                                                            uint16_t* __restrict__ xg) {
  const int lane = threadIdx.x & 63;
  const int cpr = H >> 3;
  // entries of src past the grouped rows (pairs with ids outside [0, E)) may
  // still hold the per-chunk counts of the earlier kernels: set them to -1
  for (int r = offsets[E] + blockIdx.x * 256 + threadIdx.x; r < TK; r += gridDim.x * 256) src[r] = -1;
  for (int p = blockIdx.x * 4 + (threadIdx.x >> 6); p < TK; p += gridDim.x * 4) {
    const int e = ids[p];
    if (e < 0 || e >= E) continue;
    const int r = dst[p], tok = p / k;
    if (lane == 0) src[r] = tok;
    if (x) {
      const uint4* __restrict__ srow = reinterpret_cast<const uint4*>(x + (long long)tok * H);
      uint4* __restrict__ drow = reinterpret_cast<uint4*>(xg + (long long)r * H);
#pragma unroll 8
      for (int c = lane; c < cpr; c += 64) drow[c] = srow[c];
    }
  }
}

// ---------------------------------------------------------------- unfused GLU
// The unfused baseline passes (B1): each workgroup scans the counts to find
// the routed rows (and a row's expert for the bias), then takes rows
// blockIdx.x, blockIdx.x + gridDim.x, ..., one 8-column chunk per thread.
__device__ __forceinline__ int expert_of_row(const GroupScan& gs, int E, int r) {
  int lo = 0, hi = E;   // last e with row_off[e] <= r (and rows in it)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (gs.row_off[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// y = GLU epilogue of the plain-order FC1 output z [M_cap][2I] (+ bias).
__global__ __launch_bounds__(256) void glu_unfused_kernel(const uint16_t* __restrict__ z,
                                                          const int* __restrict__ counts, int E,
                                                          int M_cap, int I, EpiParams ep,
                                                          uint16_t* __restrict__ y) {
  __shared__ GroupScan gs;
  build_group_scan<256>(gs, counts, E, M_cap, 1, 0, nullptr, nullptr, false);
  const int M = gs.row_off[E];
  const int cpr = I >> 3;
  for (int r = blockIdx.x; r < M; r += gridDim.x) {
    const uint16_t* zr = z + (long long)r * 2 * I;
    const uint16_t* b = ep.bias ? ep.bias + (long long)expert_of_row(gs, E, r) * 2 * I : nullptr;
    const float rs = ep.row_scale ? ep.row_scale[r] : 1.0f;
    for (int ch = threadIdx.x; ch < cpr; ch += 256) {
      uint4 gv = *reinterpret_cast<const uint4*>(zr + ch * 8);
      uint4 uv = *reinterpret_cast<const uint4*>(zr + I + ch * 8);
      const uint16_t* g16 = reinterpret_cast<const uint16_t*>(&gv);
      const uint16_t* u16 = reinterpret_cast<const uint16_t*>(&uv);
      float bg[8] = {0, 0, 0, 0, 0, 0, 0, 0}, bu[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (b) {
        uint4 bgv = *reinterpret_cast<const uint4*>(b + ch * 8);
        uint4 buv = *reinterpret_cast<const uint4*>(b + I + ch * 8);
        const uint16_t* bg16 = reinterpret_cast<const uint16_t*>(&bgv);
        const uint16_t* bu16 = reinterpret_cast<const uint16_t*>(&buv);
#pragma unroll
        for (int q = 0; q < 8; ++q) { bg[q] = bf16_to_f32(bg16[q]); bu[q] = bf16_to_f32(bu16[q]); }
      }
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
}

// d(gate | up) [M_cap][2I] from dL/dy G [M_cap][I] (bf16, the plain dgrad
// GroupGemm's output) and the saved pre-activation z [M_cap][2I]: the same
// arithmetic as the fused dGLU epilogue, on the bf16-rounded G.
__global__ __launch_bounds__(256) void dglu_unfused_kernel(const uint16_t* __restrict__ G,
                                                           const uint16_t* __restrict__ z,
                                                           const int* __restrict__ counts, int E,
                                                           int M_cap, int I, EpiParams ep,
                                                           uint16_t* __restrict__ dgu) {
  __shared__ GroupScan gs;
  build_group_scan<256>(gs, counts, E, M_cap, 1, 0, nullptr, nullptr, false);
  const int M = gs.row_off[E];
  const int cpr = I >> 3;
  for (int r = blockIdx.x; r < M; r += gridDim.x) {
    const uint16_t* zr = z + (long long)r * 2 * I;
    const uint16_t* gr = G + (long long)r * I;
    uint16_t* dr = dgu + (long long)r * 2 * I;
    const float rs = ep.row_scale ? ep.row_scale[r] : 1.0f;
    for (int ch = threadIdx.x; ch < cpr; ch += 256) {
      uint4 Gv = *reinterpret_cast<const uint4*>(gr + ch * 8);
      uint4 gv = *reinterpret_cast<const uint4*>(zr + ch * 8);
      uint4 uv = *reinterpret_cast<const uint4*>(zr + I + ch * 8);
      const uint16_t* G16 = reinterpret_cast<const uint16_t*>(&Gv);
      const uint16_t* g16 = reinterpret_cast<const uint16_t*>(&gv);
      const uint16_t* u16 = reinterpret_cast<const uint16_t*>(&uv);
      uint4 og, ou;
      uint16_t* og16 = reinterpret_cast<uint16_t*>(&og);
      uint16_t* ou16 = reinterpret_cast<uint16_t*>(&ou);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float Gq = bf16_to_f32(G16[q]) * rs;
        const float g = bf16_to_f32(g16[q]), u = bf16_to_f32(u16[q]);
        const float gc = fminf(fmaxf(g, ep.gate_lo), ep.gate_hi);
        const float uc = fminf(fmaxf(u, ep.up_lo), ep.up_hi) + ep.up_offset;
        float a, da;
        act_fwd_bwd(ep.act, gc, ep.alpha, a, da);
        const bool gin = (g >= ep.gate_lo) && (g <= ep.gate_hi);
        const bool uin = (u >= ep.up_lo) && (u <= ep.up_hi);
        og16[q] = f32_to_bf16(gin ? Gq * uc * da : 0.0f);
        ou16[q] = f32_to_bf16(uin ? Gq * a : 0.0f);
      }
      *reinterpret_cast<uint4*>(dr + ch * 8) = og;
      *reinterpret_cast<uint4*>(dr + I + ch * 8) = ou;
    }
  }
}

// ---------------------------------------------------------------- MXFP8 quantize

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
    store_codes32(q + (long long)r * C + cb * 32, w, 32);
    s[(long long)r * nb + cb] = sb;
  }
}

// Column-wise: one thread per (column, 32-row block); blocks restart at each
// group's first row (with counts) or run over all R rows (without).  Grid.y
// walks blocks (scale slots); grid.x covers columns in 256-column chunks.
// blocked: the K-tiled layout (slots of 32 bytes, each group a whole number
// of 4-slot K-tiles; slots past a group's rows get zero codes, scale 127).
__global__ __launch_bounds__(256) void mx_cols_kernel(const uint16_t* __restrict__ v, int R, int C,
                                                      const int* __restrict__ counts, int E,
                                                      uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ s, int s_ld, int e5,
                                                      int blocked) {
  __shared__ GroupScan gs;
  int nblocks;
  if (counts) {
    build_group_scan<256>(gs, counts, E, R, 1, 0, nullptr, nullptr, false, blocked != 0);
    nblocks = gs.mxs_off[E];
  } else {
    nblocks = blocked ? 4 * ((R + 127) >> 7) : (R + 31) >> 5;
  }
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  for (int b = blockIdx.y; b < nblocks; b += gridDim.y) {
    int r0, nvalid;
    if (counts) {
      int lo = 0, hi = E;  // group owning scale slot b: last e with mxs_off[e] <= b
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
    if (nvalid < 0) nvalid = 0;   // a padding slot of the K-tiled layout
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = (i < nvalid) ? bf16_to_f32(v[(long long)(r0 + i) * C + c]) : 0.0f;
    uint32_t w[8];
    uint8_t sb = nvalid > 0 ? mx_quant32(x, nvalid, w, e5 != 0) : (uint8_t)127;
    if (blocked) store_codes32_slot(q + ((long long)c * s_ld + b) * 32, w, nvalid);
    else store_codes32(q + (long long)c * R + r0, w, nvalid);
    s[(long long)c * s_ld + b] = sb;
  }
}

// The K-tiled transposed copy (blocked layout) with the tile staged in LDS:
// one work item is 256 rows (8 slots, two K-tiles) of one group x 64 columns.
// The item's rows are read as 128-byte row segments into LDS, each 16-byte
// chunk rotated by its row's 32-row block (chunk (c + r/32) % 8) so that the
// column reads of the quantisation step spread over the banks; lane (jp, k) of
// a wave then quantises slot k of the column pair jp (one 4-byte read per row)
// and writes their 32-code runs, 8 consecutive slots of a column (256
// contiguous bytes) per 8 lanes.  Slots
// of the group past its rows get zero codes and scale byte 127.  Persistent
// grid over (row chunk, column chunk), column chunk fastest.
__global__ __launch_bounds__(256) void mx_cols_ktiled_kernel(const uint16_t* __restrict__ v, int R, int C,
                                                             const int* __restrict__ counts, int E,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ s, int S, int e5) {
  __shared__ GroupScan gs;
  __shared__ __attribute__((aligned(16))) uint16_t tile[256 * 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int Eg = 1;
  if (counts) {
    build_group_scan<256>(gs, counts, E, R, 256, 0, nullptr, nullptr, false, true);
    Eg = E;
  } else {   // one group of R rows
    if (t == 0) {
      gs.row_off[0] = 0; gs.row_off[1] = R;
      gs.tile_off[0] = 0; gs.tile_off[1] = (R + 255) >> 8;
      gs.mxs_off[0] = 0; gs.mxs_off[1] = 4 * ((R + 127) >> 7);
    }
    __syncthreads();
  }
  const int ncb = (C + 63) >> 6;
  const long long items = (long long)gs.tile_off[Eg] * ncb;
  // item geometry: group, chunk within it, rows, slots, columns
  struct Item { int e, tc, r0, nrows, nsl, c0, ncols; };
  auto item_of = [&](long long it) {
    Item d;
    const int ch = (int)(it / ncb), cb = (int)(it - (long long)ch * ncb);
    int lo = 0, hi = Eg;   // the group of row chunk ch: last e with tile_off[e] <= ch
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (gs.tile_off[mid] <= ch) lo = mid; else hi = mid;
    }
    d.e = lo;
    d.tc = ch - gs.tile_off[lo];
    const int m_e = gs.row_off[lo + 1] - gs.row_off[lo];
    d.r0 = gs.row_off[lo] + 256 * d.tc;
    d.nrows = min(256, m_e - 256 * d.tc);
    d.nsl = min(8, 4 * ((m_e + 127) >> 7) - 8 * d.tc);
    d.c0 = cb * 64;
    d.ncols = min(64, C - d.c0);
    return d;
  };
  // this thread's 8 chunks of 8 columns (rows p*32 + t/8, chunk t%8); the
  // next item's loads go out before the current item is quantised
  uint4 buf[8];
  auto load_item = [&](const Item& d) {
#pragma unroll
    for (int pss = 0; pss < 8; ++pss) {
      const int rr = pss * 32 + (t >> 3), cc = t & 7;
      buf[pss] = make_uint4(0u, 0u, 0u, 0u);
      if (rr < d.nrows && cc * 8 < d.ncols)
        buf[pss] = *reinterpret_cast<const uint4*>(v + (long long)(d.r0 + rr) * C + d.c0 + cc * 8);
    }
  };
  long long it = blockIdx.x;
  Item cur;
  if (it < items) {
    cur = item_of(it);
    load_item(cur);
  }
  for (; it < items; it += gridDim.x) {
    const int e = cur.e, tc = cur.tc, nrows = cur.nrows, nsl = cur.nsl, c0 = cur.c0, ncols = cur.ncols;
    __syncthreads();   // the previous item's reads of the tile are done
#pragma unroll
    for (int pss = 0; pss < 8; ++pss) {
      const int rr = pss * 32 + (t >> 3), cc = t & 7;
      *reinterpret_cast<uint4*>(tile + rr * 64 + ((cc + (rr >> 5)) & 7) * 8) = buf[pss];
    }
    __syncthreads();
    if (it + gridDim.x < items) {
      cur = item_of(it + gridDim.x);
      load_item(cur);
    }
    // lane (column pair jp, slot k): one 4-byte LDS read per row gives both
    // columns' values
    {
      const int j = wave * 16 + 2 * (lane >> 3), k = lane & 7;
      if (j < ncols && k < nsl) {
        const int nv = max(0, min(32, nrows - 32 * k));
        const uint32_t* col = reinterpret_cast<const uint32_t*>(tile + (((j >> 3) + k) & 7) * 8 + (j & 7));
        float x0[32], x1[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t pr = col[(32 * k + i) * 32];
          x0[i] = __uint_as_float(pr << 16);
          x1[i] = __uint_as_float(pr & 0xFFFF0000u);
        }
        uint32_t w0[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u}, w1[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        const uint8_t sb0 = nv > 0 ? mx_quant32(x0, nv, w0, e5 != 0) : (uint8_t)127;
        const uint8_t sb1 = nv > 0 ? mx_quant32(x1, nv, w1, e5 != 0) : (uint8_t)127;
        const long long slot = (long long)(c0 + j) * S + gs.mxs_off[e] + 8 * tc + k;
        store_codes32_slot(q + slot * 32, w0, nv);
        store_codes32_slot(q + (slot + S) * 32, w1, nv);
        s[slot] = sb0;
        s[slot + S] = sb1;
      }
    }
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
