/*
 * moe_glu.h -- C ABI of the sync-free MoE expert-MLP library for AMD MI355X
 * (CDNA4, gfx950): grouped GEMM over per-expert token groups whose sizes live
 * only in device memory, with the GLU activation, its backward and an MXFP8
 * quantize/transpose fused into the GEMM epilogues.
 *
 * Sources ("the pages"):
 *   [BLOG] "Boosting MoE Training Throughput with Advanced Fusion Kernels"
 *          (Spanish translation).  Its kernel family: GroupGemm + Quantize,
 *          GroupGemm + Activation + Quantize/Transpose, GroupGemm +
 *          dActivation + Quantize/Transpose; activations SwiGLU, GeGLU,
 *          sReLU with clamping and scaling.
 *   [MEGA] DeepSeek MegaMoE / DeepGEMM walkthrough (hnwysp.cn), §2.1 routing,
 *          §4.3 grouped GEMM over contiguous per-expert rows, §5.3 tail tiles.
 *
 * Conventions shared by every call:
 *   - Pointers are DEVICE pointers unless marked (host).  bf16 tensors are
 *     passed as 16-bit storage, e4m3fn elements and E8M0 scales as bytes.
 *     Every device pointer must be 16-byte aligned, except the MX outputs.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  No call allocates, synchronises, or reads device data back to
 *     the host, so each is legal inside hipStreamBeginCapture.
 *   - The caller owns every buffer.  The library keeps no per-call state.
 *   - Errors a host can see (null required pointer, bad shape, misalignment,
 *     unsupported option) return a nonzero status BEFORE anything launches.
 *     A failed launch returns MOE_ERR_LAUNCH.  Errors only the device can see
 *     (a negative count, counts summing past M_cap) set bits in
 *     groups->status_out and the work is clamped to M_cap rows; nothing is
 *     read or written out of bounds and no kernel traps.
 *   - Grouped rows: expert e owns rows [o_e, o_e + m_e) of every [M_cap][*]
 *     operand, o_e = sum_{j<e} m_j ([MEGA] §4.3).  Rows >= sum m_e, and all
 *     rows of a zero-row expert, are never written.
 *   - Calls on different streams are independent and re-entrant.
 */
#ifndef MOE_GLU_H
#define MOE_GLU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,         /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,        /* a size is out of range or not a supported multiple */
  MOE_ERR_ALIGN = 3,        /* a pointer is not 16-byte aligned */
  MOE_ERR_UNSUPPORTED = 4,  /* an option combination the library does not implement */
  MOE_ERR_LAUNCH = 5,       /* the HIP runtime rejected a launch */
  MOE_ERR_DEVICE = 6        /* no usable gfx950 device */
} moe_status_t;

typedef enum {
  MOE_ACT_SWIGLU = 0,       /* a(g) = g * sigmoid(alpha * g) */
  MOE_ACT_GEGLU = 1,        /* a(g) = g * Phi(g), exact erf form */
  MOE_ACT_GEGLU_TANH = 2,   /* a(g) = tanh approximation of g * Phi(g) */
  MOE_ACT_SRELU = 3         /* a(g) = max(g, 0)^2 */
} moe_act_t;

/* GLU epilogue ([BLOG] "Optimizando GLU vía epílogos GEMM fusionados": the
 * GLU splits FC1's output into an input (up) half and a gate half; the fused
 * epilogue also does feature scaling, clamping and bias addition).
 * With z = FC1 output + bias, g = z[:, :I] (gate), u = z[:, I:] (up):
 *     y = a(clamp(g, gate_lo, gate_hi)) * (clamp(u, up_lo, up_hi) + up_offset)
 *         * row_scale[row]
 * rounded to bf16 (round-to-nearest-even).  (host struct) */
typedef struct {
  int32_t act;              /* moe_act_t */
  int32_t gated;            /* 1: the gated (GLU) form y = a(g_c) * u_c; 0: the non-gated form
                               y = a(z) over I columns (no clamps, no up_offset; sReLU's
                               plain form), see moe_group_gemm_glu_fwd */
  float alpha;              /* SwiGLU gate scale inside the sigmoid; 1 = plain SiLU */
  float gate_lo, gate_hi;   /* clamp bounds on g; -inf/+inf = off */
  float up_lo, up_hi;       /* clamp bounds on u; -inf/+inf = off */
  float up_offset;          /* added to the clamped up value; 0 = off */
  const void* bias;         /* nullable: bf16 [E][2I] in PLAIN order (gate | up); [E][I] when
                               non-gated */
  const float* row_scale;   /* nullable: fp32 [M_cap], multiplies y per row */
  /* Per-tensor amax for an NVFP4-style recipe ([BLOG] "Fusionando cuantización MXFP8 y
     NVFP4": the forward emits its output's amax, the backward the amax of the Hadamard
     rotation of its transposed output).  Nullable device float, 4-byte aligned, raised
     (atomic max) by the call, so the caller sets it to 0 (or a running max) first:
       moe_group_gemm_glu_fwd(_mx): max |y| over the routed rows, bf16 values as written;
       moe_group_gemm_dglu_bwd:     max |R d| over every column d of dgu = [dg | du] (bf16
         values as written) cut into runs of 16 consecutive rows that restart at each group's
         first row, the last run of a group padded with zero rows, and R = H16 S / 4: H16 the
         Sylvester Hadamard matrix of order 16 and S = diag(s_i), s_i = -1 where bit i of
         rht_signs is set (row i of the run), else +1.
     NaN values are skipped.  Other entry points ignore both fields. */
  float* amax_out;
  uint32_t rht_signs;       /* low 16 bits: the row signs of the backward rotation */
  /* Gradients of the epilogue's own parameters, written by moe_group_gemm_dglu_bwd only
     (nullable device fp32 buffers, 4-byte aligned, ADDED to atomically, so the caller zeroes
     them or passes running sums; the summation order is unspecified):
       dbias_out      [E][2I], plain (gate | up) order: per expert, the sum over its rows of
                      dgu (the bf16 values as written) = dL/d(bias) of the FC1 + GLU forward;
       drow_scale_out [M_cap]: for every routed row r, sum over j < I of G[r][j] a(g_c) u_c,
                      G = dY2 W2^T (= dL/dy) and a(g_c) u_c the unscaled GLU output in fp32 =
                      dL/d(row_scale[r]); rows past the routed ones are not touched. */
  float* dbias_out;
  float* drow_scale_out;
} moe_epilogue_t;

/* MXFP8 outputs ([BLOG] "Fusionando cuantización MXFP8 y NVFP4": the
 * quantised activation plus a transposed copy for back prop).  Blocks of 32
 * values share one E8M0 scale X = 2^E, E the smallest integer with
 * amax/X <= 448; elements are e4m3fn(v / X), round-to-nearest-even.
 * For an output of R = M_cap rows and C columns:
 *   row_q [R][C], row_s [R][C/32]          blocks along a row
 *   col_q [C][R], col_s [C][ceil(R/32)+E]  blocks of 32 rows of one column
 *                                          that restart at each group's first
 *                                          row; group e's scales start at column
 *                                          sum_{j<e} ceil(m_j/32)
 * Any pointer may be NULL (that copy is skipped); row_q/row_s and col_q/col_s
 * go in pairs.  No alignment requirement (col_blocked = 1: 16 bytes).
 * e5m2 = 1 selects OCP e5m2 elements instead (the gradient format of an
 * MXFP8 recipe: largest value 57344 = 1.75 * 2^15, the scale rule with 57344
 * in place of 448); 0 = e4m3fn.
 * col_blocked = 1 writes the transposed copy in the K-tiled layout that the
 * MXFP8 weight-gradient GroupGemm (moe_group_gemm_wgrad_mx) reads, the copy
 * the pages keep "for back prop": a row of col_s has S = 4 (ceil(R/128) + E)
 * slots and the matching row of col_q 32 S bytes, slot s holding one 32-row
 * block (its scale byte at col_s[c][s], its 32 codes at col_q[c][32 s ..]);
 * group e's blocks take slots so_e, so_e + 1, ... with so_e = 4 sum_{j<e}
 * ceil(m_j/128), so every group starts on a 128-code boundary, and the slots
 * up to so_e + 4 ceil(m_e/128) that no row reaches (and the codes of a partial
 * block past the group's last row) hold zero codes with scale byte 127.
 * col_blocked = 0 is the dense layout above.  (host struct) */
typedef struct {
  uint8_t* row_q;
  uint8_t* row_s;
  uint8_t* col_q;
  uint8_t* col_s;
  int32_t e5m2;
  int32_t col_blocked;
} moe_mx_out_t;

/* Expert groups.  The counts are the ONLY copy of the group sizes and stay in
 * device memory ([BLOG] "Eliminando la sincronización host-device": tokens
 * per group are tracked in GPU memory, so no host sync is needed and a whole
 * iteration can be captured in a graph).  (host struct) */
typedef struct {
  const int32_t* counts;    /* device [E] */
  int32_t E;                /* 1 <= E <= 1024 */
  int32_t M_cap;            /* static row capacity of every grouped operand */
  int32_t* offsets_out;     /* nullable device [E+1]: exclusive scan of the clamped counts */
  int32_t* status_out;      /* nullable device word, OR-ed: bit0 a count < 0, bit1 sum > M_cap */
} moe_groups_t;

/* Operand descriptor of moe_group_gemm_quant. */
typedef enum {
  MOE_DT_BF16 = 0,
  MOE_DT_MXFP8 = 1,         /* e4m3fn bytes + E8M0 scales, 32-blocks along K */
  MOE_DT_MXFP8_E5M2 = 2     /* e5m2 bytes + E8M0 scales (a gradient, e.g. dgu for dX); the A operand
                               of moe_group_gemm_quant, either operand of moe_group_gemm_wgrad_mx */
} moe_dtype_t;

typedef enum {
  MOE_B_KN = 0,             /* B_e is [K][N] row-major (N contiguous), e.g. W2 [E][I][H] for FC2 */
  MOE_B_NK = 1,             /* B_e is stored [N][K] (K contiguous), i.e. used transposed:
                               out = A . B_e^T, e.g. W2 [E][I][H] in the dgrad dY2 . W2^T */
  MOE_B_PACKED = 2          /* B_e in the tile-blocked layout of moe_pack_weight (see there) */
} moe_b_layout_t;

typedef struct {
  int32_t dtype;            /* moe_dtype_t */
  int32_t layout;           /* A: ignored (always [M_cap][K] row-major); B: moe_b_layout_t */
  const void* data;         /* bf16 or e4m3 elements */
  const uint8_t* scales;    /* MXFP8 only: A [M_cap][K/32] E8M0 (block b of row r covers K
                               values 32b..32b+31); B from moe_pack_weight_mx */
} moe_operand_t;

/* Reads the device's compute-unit count once; call before graph capture.
 * Every other call initialises lazily on first use.  The persistent grid of
 * every GroupGemm is sized from that count ([BLOG] "Eliminando la
 * sincronización host-device": a fixed launch whose work split is decided on
 * the device, so the launch itself needs no host-side information that
 * changes between steps). */
moe_status_t moe_init(int device);

const char* moe_status_string(moe_status_t s);

/* Tile-blocked weight layout ("packed"), shared by moe_repack_gate_up and
 * moe_pack_weight.  A weight used as the B operand of out = A . B_e^T is
 * viewed per expert as [N][K] (K contiguous).  It is stored as blocks of 256
 * rows (n) by 64 columns (k) = 32 KiB each; block (nb, kb) starts at element
 * (nb * K/64 + kb) * 16384 of the expert, and experts are ceil(N/256) * 256 * K
 * elements apart.  Inside a block, the 16-byte chunk c (0..7, k = 64 kb + 8c
 * .. +7) of row r (n = 256 nb + r) sits at byte r * 128 + 16 * (c XOR s(r)),
 * s(r) = (r mod 8) XOR (2 ((r / 8) mod 2) + (r / 16) mod 2): the order in
 * which the kernels stage it in LDS, so each block streams from memory
 * contiguously.  Rows n >= N are zero.  Requires K % 64 == 0. */
size_t moe_packed_weight_bytes(int E, int N, int K);

/* Packs per-expert weights into the tile-blocked layout above: the same
 * offline weight preparation as the gate/up repack ([BLOG] "Optimizando GLU
 * vía epílogos GEMM fusionados", Figure 2: the weights are rearranged once, off
 * the training step, into the order the kernel consumes), here without the
 * gate/up interleave, for the other GroupGemm operands.
 * src_layout MOE_B_NK: src is [E][N][K]; MOE_B_KN: src is [E][K][N] (transposed
 * while packing).  Uses: FC2's W2 [E][I][H] as MOE_B_KN with N = H, K = I;
 * dgrad's W2 [E][I][H] as MOE_B_NK with N = I, K = H; dX's plain W1 [E][H][2I]
 * as MOE_B_NK with N = H, K = 2I.  Bit-exact (a permutation plus zero padding). */
moe_status_t moe_pack_weight(const void* src, int E, int N, int K, int src_layout, void* dst,
                             void* stream);

/* MXFP8 weight for the block-scaled GroupGemm ([BLOG] "Fusionando
 * cuantización MXFP8…": MXFP8 blocks of 32 values with one E8M0 scale; here a
 * weight quantised once, offline, along the reduction dimension K).
 * Element bytes: per expert ceil(N/256) * 256 * K (e4m3fn codes), as blocks
 * of 256 rows (n) by 128 K values = 32 KiB; block (nb, kb) starts at byte
 * (nb * K/128 + kb) * 32768 of the expert; the 16-byte chunk c (0..7, k =
 * 128 kb + 16 c .. +15) of row r sits at byte r * 128 + 16 * (c XOR s(r)),
 * s(r) as above.  Scale bytes: per expert ceil(N/256) * 256 * K/32; the
 * dword at byte ((nb * K/128 + kb) * 256 + r) * 4 holds the E8M0 scales of
 * row r's four 32-blocks of block (nb, kb), block b in byte b.  Rows n >= N
 * are zero with scale byte 0.  Requires K % 128 == 0. */
size_t moe_packed_mx_weight_bytes(int E, int N, int K);
size_t moe_packed_mx_scale_bytes(int E, int N, int K);

/* Quantises a bf16 weight to that MXFP8 layout: for each output column n and
 * each run of 32 consecutive k, amax gives the E8M0 exponent X (the smallest
 * power of two with amax / 2^X <= 448; 0xFF if a value is NaN) and every
 * value becomes e4m3fn(v / 2^X), rounded to nearest even.  src_layout as for
 * moe_pack_weight (FC2's W2 [E][I][H]: MOE_B_KN with N = H, K = I).
 * Requires N % 64 == 0, K % 128 == 0; dst_q, dst_s 16-byte aligned. */
moe_status_t moe_pack_weight_mx(const void* src, int E, int N, int K, int src_layout,
                                void* dst_q, void* dst_s, void* stream);

/* The gate/up-repacked W1 as MXFP8 (the FC1 weight of the MXFP8 recipe):
 * W1 [E][H][2I] bf16 (plain: gate | up) quantised along H (the reduction
 * dimension) and stored in the MXFP8 layout above with N = 2I in the packed
 * gate/up order of moe_repack_gate_up and K = H.  Sizes:
 * moe_packed_mx_weight_bytes(E, 2I, H), moe_packed_mx_scale_bytes(E, 2I, H).
 * Requires H % 128 == 0, I % 64 == 0. */
moe_status_t moe_repack_gate_up_mx(const void* w1, int E, int H, int I, void* dst_q, void* dst_s,
                                   void* stream);

/* Bytes of the packed W1 for E experts, hidden H, intermediate I:
 * moe_packed_weight_bytes(E, 2I, H). */
size_t moe_packed_w1_bytes(int E, int H, int I);

/* Offline gate/up repack ([BLOG] "Optimizando GLU…" and its Figure 2: W1's
 * columns are repacked into interleaved gate and input (up) blocks so that one
 * GEMM tile holds half a tile width of each; done once at checkpoint load).
 * w1:        bf16 [E][H][2I], plain: columns [0,I) gate, [I,2I) up.
 * w1_packed: the tile-blocked layout above with N = 2I (packed order), K = H,
 *            where packed row 128p + s is gate column 64p + s for s < 64 and up
 *            column I + 64p + (s-64) for s >= 64.  Each 256-row block therefore
 *            holds two (64 gate | 64 up) pairs.  Requires I % 64 == 0,
 *            H % 64 == 0.  Bit-exact. */
moe_status_t moe_repack_gate_up(const void* w1, int E, int H, int I, void* w1_packed,
                                void* stream);

/* Inverse of moe_repack_gate_up (checkpoint save, tests).  Bit-exact. */
moe_status_t moe_unpack_gate_up(const void* w1_packed, int E, int H, int I, void* w1,
                                void* stream);

/* Device routing and grouping ([MEGA] §2.1: each token's k experts are the
 * k largest router logits; §4.3: rows of one expert laid out contiguously).
 * Exactly one of logits (fp32 [T][E]) / topk_ids (int32 [T][k]) is non-NULL.
 * Ties go to the lower expert id.  Outputs (all device, all required except
 * xg): topk_ids_out [T][k]; counts [E]; offsets [E+1]; dst [T][k], the grouped
 * row of pair (t, j); src [T*k], the token of each grouped row.  Within an
 * expert the pairs keep ascending (t, j) order, so the result is unique and
 * deterministic.  If x (bf16 [T][H]) and xg (bf16 [T*k][H]) are given, xg
 * receives the gathered rows xg[r] = x[src[r]].  Given topk_ids outside
 * [0, E) are not grouped: their dst entries and the rows of xg from
 * offsets[E] on are left as they were, and src entries from offsets[E] on are
 * set to -1.  Requires k <= E <= 1024, k <= 16,
 * T*k < 2^31, H % 8 == 0. */
moe_status_t moe_route_group(const float* logits, const int32_t* topk_ids, int T, int E, int k,
                             int32_t* topk_ids_out, int32_t* counts, int32_t* offsets,
                             int32_t* dst, int32_t* src, const void* x, int H, void* xg,
                             void* stream);

/* GroupGemm + Activation (+ Quantize/Transpose), the fused FC1 ([BLOG] kernel
 * family, second kernel).  For each expert e, with A_e = xg rows of group e:
 *     z = A_e . W1_e (+ bias_e)          fp32 accumulate, W1 from moe_repack_gate_up
 *     preact = bf16(z)                   optional, [M_cap][2I] in PLAIN order
 *     y = bf16(GLU epilogue of z)        optional, [M_cap][I]
 *     mx = MXFP8 copies of y             optional (row-wise and/or transposed)
 * xg: bf16 [M_cap][H]; w1_packed from moe_repack_gate_up.
 * Non-gated form (ep->gated == 0): W1 [E][H][I] packed by moe_pack_weight
 * (MOE_B_KN source, N = I, K = H), z and preact are [M_cap][I], y = bf16(a(z)
 * * row_scale); bias [E][I].
 * Requires H % 64 == 0, I % 64 == 0.
 * One persistent launch; tiles are scheduled from the device counts.
 * cu_margin: compute units left free for concurrent kernels (0 = use all). */
moe_status_t moe_group_gemm_glu_fwd(const void* xg, const moe_groups_t* groups,
                                    const void* w1_packed, int H, int I,
                                    const moe_epilogue_t* ep, void* y, void* preact,
                                    const moe_mx_out_t* mx, int cu_margin, void* stream);

/* moe_group_gemm_glu_fwd with MXFP8 inputs ([BLOG] "Fusionando cuantización
 * MXFP8…": the MXFP8 training recipe's FC1): xg = e4m3 [M_cap][H] with E8M0
 * row-block scales [M_cap][H/32] (e.g. moe_mxfp8_quantize of the bf16 rows),
 * w1 = MOE_B_PACKED from moe_repack_gate_up_mx.  z is accumulated in fp32 by
 * the block-scaled MFMA from the dequantised operands; the epilogue and the
 * outputs are those of moe_group_gemm_glu_fwd.  Requires H % 128 == 0,
 * I % 64 == 0. */
moe_status_t moe_group_gemm_glu_fwd_mx(const moe_operand_t* xg, const moe_groups_t* groups,
                                       const moe_operand_t* w1, int H, int I,
                                       const moe_epilogue_t* ep, void* y, void* preact,
                                       const moe_mx_out_t* mx, int cu_margin, void* stream);

/* GroupGemm + dActivation (+ Quantize/Transpose), the fused backward of FC1's
 * activation ([BLOG] "Optimizando GLU…": in back prop the epilogue reads the
 * GEMM output, computes the dGLU and writes it out).  Per expert:
 *     G = dy2_e . W2_e^T                 fp32 accumulate; dy2 bf16 [M_cap][H];
 *                                        w2: FC2's weight [E][I][H] bf16 as
 *                                        MOE_B_NK, or moe_pack_weight of it
 *                                        (MOE_B_NK source, N = I, K = H) as
 *                                        MOE_B_PACKED
 *     with g, u from preact (bf16 [M_cap][2I] plain, post-bias, pre-clamp),
 *     gc = clamp(g), uc = clamp(u) + up_offset, rs = row_scale or 1:
 *     du = G * a(gc) * rs * [up_lo <= u <= up_hi]
 *     dg = G * uc * rs * a'(gc) * [gate_lo <= g <= gate_hi]
 *     dgu = bf16([dg | du])              [M_cap][2I] plain order
 *     mx = MXFP8 copies of dgu           optional
 * Non-gated form (ep->gated == 0): preact and dgu are [M_cap][I] and
 * dgu = bf16(G * rs * a'(z)); the parameter gradients are not available
 * (MOE_ERR_UNSUPPORTED), the rotated amax is.
 * ep->bias is ignored (already inside preact).  Requires H % 64 == 0,
 * I % 64 == 0. */
moe_status_t moe_group_gemm_dglu_bwd(const void* dy2, const moe_operand_t* w2, int H, int I,
                                     const moe_groups_t* groups, const void* preact,
                                     const moe_epilogue_t* ep, void* dgu,
                                     const moe_mx_out_t* mx, int cu_margin, void* stream);

/* GroupGemm + Quantize ([BLOG] kernel family, first kernel): out_e = A_e . B_e
 * with bf16 and/or MXFP8 output.  A: [M_cap][K] grouped rows; B per the
 * layout in b->layout (MOE_B_PACKED is the fast path).  c_bf16: nullable bf16
 * [M_cap][N].  bf16 x bf16 on every B layout, or MXFP8 x MXFP8 ([BLOG]
 * "GroupGemm + Quantize" with MXFP8 inputs): A = e4m3fn [M_cap][K] with E8M0
 * row-block scales [M_cap][K/32] (e.g. the row-wise MX output of
 * moe_group_gemm_glu_fwd), B = MOE_B_PACKED from moe_pack_weight_mx, and
 *     out_e = sum_k (q_a * 2^(s_a - 127)) (q_b * 2^(s_b - 127))
 * accumulated in fp32 by the block-scaled MFMA.  Mixed bf16 / MXFP8 inputs
 * are MOE_ERR_UNSUPPORTED.  Requires K % 64 == 0 (K % 128 == 0 for MXFP8),
 * N % 64 == 0. */
moe_status_t moe_group_gemm_quant(const moe_operand_t* a, const moe_operand_t* b, int N, int K,
                                  const moe_groups_t* groups, void* c_bf16,
                                  const moe_mx_out_t* mx, int cu_margin, void* stream);

/* Weight gradients as K-grouped GroupGemms ([BLOG] "Fusionando cuantización
 * MXFP8…": the transposed copies exist for back prop, i.e. for these
 * products).  For each expert e with rows [o_e, o_e + m_e):
 *     c_e = a_e^T . b_e          fp32 accumulate, fp32 output [E][P][Q]
 * a: bf16 [M_cap][P] grouped rows, b: bf16 [M_cap][Q] grouped rows; the
 * reduction runs over the group's rows (counts in device memory only).
 * dW1 = wgrad(xg [M_cap][H], dgu [M_cap][2I]) -> [E][H][2I] (plain W1 order);
 * dW2 = wgrad(y [M_cap][I], dy2 [M_cap][H]) -> [E][I][H].
 * accumulate = 0 overwrites c (an empty group writes zeros); 1 adds to it.
 * Requires P % 64 == 0, Q % 64 == 0; a, b, c 16-byte aligned. */
moe_status_t moe_group_gemm_wgrad(const void* a, const void* b, int P, int Q,
                                  const moe_groups_t* groups, float* c, int accumulate,
                                  int cu_margin, void* stream);

/* MXFP8 weight gradients ([BLOG] "Fusionando cuantización MXFP8 y NVFP4": the
 * epilogues also write a transposed MXFP8 copy "for back prop"; these are
 * the products that read it): the same K-grouped GroupGemm as
 * moe_group_gemm_wgrad, C_e = A_e^T B_e in fp32 [E][P][Q], on the
 * block-scaled MFMA, each operand a transposed MXFP8 copy in the K-tiled
 * layout of moe_mx_out_t (col_blocked = 1) over the same groups:
 *   a->data  [P][32 S] codes, a->scales [P][S] E8M0 (the col_q/col_s of an
 *            [M_cap][P] tensor), S = 4 (ceil(M_cap/128) + E);
 *   b->data  [Q][32 S], b->scales [Q][S] likewise;
 *   dtype    MOE_DT_MXFP8 (e4m3 codes) or MOE_DT_MXFP8_E5M2, per operand;
 *            layout ignored.
 * The result is the exact product of the dequantised copies up to fp32
 * accumulation: dW1 from the copies of xg and dgu, dW2 from those of y and
 * dy2.  accumulate = 0 overwrites c (an empty group writes zeros); 1 adds.
 * Requires P % 64 == 0, Q % 64 == 0; codes and c 16-byte aligned, scales
 * 4-byte aligned. */
moe_status_t moe_group_gemm_wgrad_mx(const moe_operand_t* a, const moe_operand_t* b, int P, int Q,
                                     const moe_groups_t* groups, float* c, int accumulate,
                                     int cu_margin, void* stream);

/* Unfused GLU pass ([BLOG] "¿Dónde se va el cómputo en un bloque MoE?": the
 * activation as its own memory-bound pass between the GEMMs, the baseline the
 * fused epilogue replaces): y = GLU epilogue of z, where z is
 * the plain-order bf16 [M_cap][2I] FC1 output WITHOUT bias (bias, if any, is
 * added here).  Same arithmetic as the fused epilogue, as its own kernel. */
moe_status_t moe_glu_unfused(const void* z, const moe_groups_t* groups, int I,
                             const moe_epilogue_t* ep, void* y, void* stream);

/* Unfused dGLU pass (the baseline of the fused backward epilogue, [BLOG]
 * "Optimizando GLU vía epílogos GEMM fusionados": the activation gradient as a
 * memory-bound pass after the GEMM).  g: dL/dy bf16 [M_cap][I] as the plain
 * dgrad GroupGemm wrote it (moe_group_gemm_quant of dY2 with W2); z: the saved
 * pre-activation bf16 [M_cap][2I] (plain order, post-bias); dgu: bf16
 * [M_cap][2I] output, d(gate) in columns [0, I), d(up) in [I, 2I).  Same
 * arithmetic as moe_group_gemm_dglu_bwd's epilogue (row scale, clamp
 * gradients, activation derivative) on the bf16-rounded g.  Routed rows only
 * (offsets from the device counts); gated forms only (ep->gated = 1, else
 * MOE_ERR_UNSUPPORTED).  Requires I % 64 == 0; g, z, dgu 16-byte aligned. */
moe_status_t moe_dglu_unfused(const void* g, const void* z, const moe_groups_t* groups, int I,
                              const moe_epilogue_t* ep, void* dgu, void* stream);

/* Standalone MXFP8 quantize/transpose ([BLOG] "Fusionando cuantización MXFP8 y
 * NVFP4": the separate pass that reads the bf16 activation output and writes
 * the MXFP8 copy and its transposed version, which the fused epilogues
 * replace; also the offline weight prep) of
 * a bf16 [R][C] matrix.  Row-wise blocks run along C.  Column-wise blocks run
 * down 32 rows; with groups (counts over the first rows, M_cap = R) they
 * restart at each group's first row exactly as in the fused epilogues and
 * col_s is [C][ceil(R/32)+E]; without groups the whole matrix is one group
 * and col_s is [C][ceil(R/32)].  So quantising one expert's W2_e [I][H]
 * column-wise yields exactly the [H][I] e4m3 + [H][I/32] scale operand that
 * MOE_B_NK expects.  Requires C % 32 == 0. */
moe_status_t moe_mxfp8_quantize(const void* v, int R, int C, const moe_groups_t* groups,
                                const moe_mx_out_t* mx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GLU_H */
