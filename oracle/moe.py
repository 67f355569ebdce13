"""Plain CPU oracle of the sync-free MoE expert MLP (GroupGEMM + GLU family).

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference that the HIP library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the GPU path: no kernels, headers, tables
or helpers.  It loops expert by expert, computes in float64 (a float32 mode
exists only for timing) and rounds with its own encoders in ``formats.py``.

Sources ("pages"):
  [BLOG]  "Boosting MoE Training Throughput with Advanced Fusion Kernels"
          (Spanish translation), sections "Optimizando GLU vía epílogos GEMM
          fusionados", "Eliminando la sincronización host-device",
          "Fusionando cuantización MXFP8 y NVFP4", Figure 2.
  [WIKI]  "MoE Fusion Kernels" (aisparkup wiki), kernel-pattern table.
  [MEGA]  DeepSeek MegaMoE / DeepGEMM walkthrough (hnwysp.cn), §2.1 routing,
          §4.3 grouped GEMM over contiguous per-expert rows, §5.3 tail tiles.

Readings where the pages are silent (each listed in the design notes):
  * gate = FC1 columns [0, I) (activated), up = columns [I, 2I) (linear);
  * the repack pairs 64 gate columns with the same 64 up columns per 128;
  * epilogue order: bias -> clamp -> activation -> product -> row scale -> bf16;
    the saved pre-activation is post-bias, pre-clamp, rounded to bf16;
  * clamp gradients pass on the closed interval [lo, hi];
  * MX scale: smallest power of two X with amax/X <= 448 (formats.py);
  * MX column blocks are 32 rows that restart at each group's first row;
    group e's scale columns start at sum_{j<e} ceil(m_j/32).

Parity pins for every function here live in tests/test_oracle_*.py.  The
exact bf16 bits of float-valued GEMMs are only bounded (accumulation order),
and the GELU form (erf default, tanh optional) and the one-sided GPT-OSS clamp
variant are pinned only by their closed forms: parity unpinned by the pages
for those choices.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .formats import (bf16_bits_to_f64, f64_to_bf16_bits, mx_quantize_block)

GATE_UP_HALF = 64   # columns of gate (and of up) per packed 128-column pair


# ============================================================================ routing
def route_topk(logits: np.ndarray, k: int):
    """Top-k routing and contiguous per-expert grouping ([MEGA] §2.1, §4.3).

    Each token t picks the k experts with the largest logit, ties to the lower
    expert id (softmax is monotone, so this equals top-k on the probabilities;
    the probabilities themselves are not needed by the grouped GEMM).  Rows
    routed to the same expert are then laid out contiguously ([MEGA] §4.3):
    expert e owns grouped rows [offsets[e], offsets[e+1]); within an expert the
    (token, slot) pairs keep ascending (t, j) order.

    Returns ids [T][k] int32, counts [E], offsets [E+1], dst [T][k] (grouped
    row of pair (t, j)) and src [T*k] (token of each grouped row).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    expert_idx = np.arange(E)
    for t in range(T):
        # sort by (-logit, expert id): lexsort sorts by the last key first
        order = np.lexsort((expert_idx, -logits[t].astype(np.float64)))
        ids[t] = order[:k]
    counts, offsets, dst, src = group_pairs(ids, E)
    return ids, counts, offsets, dst, src


def group_pairs(ids: np.ndarray, E: int):
    """Contiguous per-expert grouping of the (token, slot) pairs of ids [T][k]
    ([MEGA] §4.3): expert e owns grouped rows [offsets[e], offsets[e+1]), its
    pairs in ascending (t, j) order.  Pairs whose id lies outside [0, E) are
    not grouped: their dst is -1 and they own no row.

    Returns counts [E], offsets [E+1], dst [T][k] and src [offsets[E]] (the
    token of each grouped row).
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    # grouped row r holds pair pair_order[r]: the valid pairs sorted stably by expert
    vidx = np.flatnonzero(valid)
    pair_order = vidx[np.argsort(flat[valid], kind="stable")]
    dst = np.full(T * k, -1, dtype=np.int32)
    dst[pair_order] = np.arange(len(pair_order), dtype=np.int32)
    src = (pair_order // k).astype(np.int32)
    return counts, offsets, dst.reshape(T, k), src


def exclusive_offsets(counts) -> np.ndarray:
    counts = np.asarray(counts, dtype=np.int64)
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    return off


def gather_rows(x_bits: np.ndarray, src: np.ndarray) -> np.ndarray:
    """Grouped activations: row r of the result is token src[r] ([MEGA] §4.3)."""
    return np.asarray(x_bits)[np.asarray(src, dtype=np.int64)]


# ============================================================================ repack
def packed_column_of(j: np.ndarray, I: int) -> np.ndarray:
    """Packed position of plain FC1 column j (gate j < I, up j >= I).

    [BLOG] "Optimizando GLU…" and Figure 2: the weights are repacked into
    gate and input (up) columns so that one tile holds half a tile width of
    each.  Pair p = 128 packed columns = gate columns 64p..64p+63 followed by
    up columns I+64p..I+64p+63.
    """
    j = np.asarray(j, dtype=np.int64)
    is_up = j >= I
    c = np.where(is_up, j - I, j)
    return (c // GATE_UP_HALF) * (2 * GATE_UP_HALF) + np.where(is_up, GATE_UP_HALF, 0) + c % GATE_UP_HALF


def repack_gate_up(w1_bits: np.ndarray, b1_bits: Optional[np.ndarray] = None):
    """Offline repack of W1 [E][H][2I] (plain: gate | up) to the packed layout.

    Result W1p [E][2I][H]: packed column n holds plain column j with
    packed_column_of(j) == n, stored K-contiguous (transposed).  The bias
    [E][2I] is permuted the same way.  Pure permutation + transpose.
    """
    E, H, N2 = w1_bits.shape
    I = N2 // 2
    pos = packed_column_of(np.arange(N2), I)
    w1p = np.empty((E, N2, H), dtype=w1_bits.dtype)
    w1p[:, pos, :] = np.transpose(w1_bits, (0, 2, 1))
    b1p = None
    if b1_bits is not None:
        b1p = np.empty_like(b1_bits)
        b1p[:, pos] = b1_bits
    return w1p, b1p


def unpack_gate_up(w1p_bits: np.ndarray, b1p_bits: Optional[np.ndarray] = None):
    E, N2, H = w1p_bits.shape
    I = N2 // 2
    pos = packed_column_of(np.arange(N2), I)
    w1 = np.transpose(w1p_bits[:, pos, :], (0, 2, 1)).copy()
    b1 = None if b1p_bits is None else b1p_bits[:, pos].copy()
    return w1, b1


# ============================================================================ activations
@dataclass
class Epilogue:
    """GLU epilogue parameters ([BLOG] "Optimizando GLU…": SwiGLU, GeGLU and
    sReLU, with feature scaling, clamping and bias addition)."""
    act: str = "swiglu"          # swiglu | geglu | geglu_tanh | srelu
    gated: bool = True
    alpha: float = 1.0           # SwiGLU: silu_a(g) = g * sigmoid(alpha * g)
    gate_lo: float = -math.inf
    gate_hi: float = math.inf
    up_lo: float = -math.inf
    up_hi: float = math.inf
    up_offset: float = 0.0
    bias: Optional[np.ndarray] = None        # bf16 bits [E][2I] plain order
    row_scale: Optional[np.ndarray] = None   # float32 [M_cap]


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def _phi(x):     # standard normal pdf
    return np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _Phi(x):     # standard normal cdf via erf
    from scipy.special import erf
    return 0.5 * (1.0 + erf(x / math.sqrt(2.0)))


_GELU_TANH_C = math.sqrt(2.0 / math.pi)


def activation(g, act: str, alpha: float = 1.0):
    """a(g) for the supported activations (float64)."""
    g = np.asarray(g, dtype=np.float64)
    if act == "swiglu":
        return g * _sigmoid(alpha * g)
    if act == "geglu":
        return g * _Phi(g)
    if act == "geglu_tanh":
        return 0.5 * g * (1.0 + np.tanh(_GELU_TANH_C * (g + 0.044715 * g ** 3)))
    if act == "srelu":
        r = np.maximum(g, 0.0)
        return r * r
    raise ValueError(act)


def activation_grad(g, act: str, alpha: float = 1.0):
    """a'(g) (float64), the closed-form derivatives of ``activation``."""
    g = np.asarray(g, dtype=np.float64)
    if act == "swiglu":
        s = _sigmoid(alpha * g)
        return s * (1.0 + alpha * g * (1.0 - s))
    if act == "geglu":
        return _Phi(g) + g * _phi(g)
    if act == "geglu_tanh":
        u = _GELU_TANH_C * (g + 0.044715 * g ** 3)
        t = np.tanh(u)
        du = _GELU_TANH_C * (1.0 + 3 * 0.044715 * g * g)
        return 0.5 * (1.0 + t) + 0.5 * g * (1.0 - t * t) * du
    if act == "srelu":
        return 2.0 * np.maximum(g, 0.0)
    raise ValueError(act)


def glu_from_preact(z: np.ndarray, ep: Epilogue, row_scale: Optional[np.ndarray] = None):
    """GLU output (float64, before rounding) from pre-activations z [R][2I] or [R][N].

    Gated: g = z[:, :I], u = z[:, I:]; y = a(clip(g)) * (clip(u) + up_offset).
    Non-gated: y = a(z).  Then y *= row_scale[row] when given.
    """
    z = np.asarray(z, dtype=np.float64)
    if ep.gated:
        I = z.shape[1] // 2
        g = np.clip(z[:, :I], ep.gate_lo, ep.gate_hi)
        u = np.clip(z[:, I:], ep.up_lo, ep.up_hi) + ep.up_offset
        y = activation(g, ep.act, ep.alpha) * u
    else:
        y = activation(z, ep.act, ep.alpha)
    if row_scale is not None:
        y = y * np.asarray(row_scale, dtype=np.float64)[:, None]
    return y


# ============================================================================ GEMMs
def _as_f(bits, dtype):
    return bf16_bits_to_f64(bits).astype(dtype, copy=False)


def fc1_glu(xg_bits, counts, w1_bits, ep: Epilogue, dtype=np.float64):
    """Fused FC1 + GLU, written as its plain definition, expert by expert.

    [BLOG] "Optimizando GLU…": FC1's output is split into the gate and the
    input (up) halves and combined by the GLU; the fusion changes memory
    traffic, not the maths.  For each expert e with m_e > 0:
        Z_e = Xg[o_e:o_e+m_e] @ W1_e (+ b1_e)       (plain, un-repacked W1)
        preact = bf16(Z), y = bf16(GLU(Z))
    Zero-row experts produce nothing.  Returns (preact bits [M][2I], y bits
    [M][I]) covering rows [0, M); rows beyond M are never produced.
    """
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    M = int(off[-1])
    E, H, N = w1_bits.shape
    NO = N // 2 if ep.gated else N
    preact = np.zeros((M, N), dtype=np.uint16)
    y = np.zeros((M, NO), dtype=np.uint16)
    rs_all = None if ep.row_scale is None else np.asarray(ep.row_scale, dtype=np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        z = _as_f(xg_bits[a:b], dtype) @ _as_f(w1_bits[e], dtype)
        z = z.astype(np.float64)
        if ep.bias is not None:
            z = z + bf16_bits_to_f64(ep.bias[e])[None, :]
        preact[a:b] = f64_to_bf16_bits(z)
        rs = None if rs_all is None else rs_all[a:b]
        y[a:b] = f64_to_bf16_bits(glu_from_preact(z, ep, rs))
    return preact, y


def group_gemm(a_bits, counts, b_bits, dtype=np.float64):
    """GroupGemm ([BLOG] kernel family, "GroupGemm + Quantize"): out_e = A_e @ B_e.

    a_bits [M][K] grouped rows, b_bits [E][K][N]; returns bf16 bits [M][N].
    """
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    M = int(off[-1])
    E, K, N = b_bits.shape
    out = np.zeros((M, N), dtype=np.uint16)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        c = _as_f(a_bits[a:b], dtype) @ _as_f(b_bits[e], dtype)
        out[a:b] = f64_to_bf16_bits(c.astype(np.float64))
    return out


def dglu(G, z, ep: Epilogue, row_scale: Optional[np.ndarray] = None):
    """dGLU epilogue ([BLOG] "Optimizando GLU…": in back prop the epilogue reads
    the GEMM output, computes dSwiGLU and writes it out).

    G [R][I] is dL/dy (float64); z [R][2I] the saved (post-bias, pre-clamp)
    pre-activations as float64.  With g_c = clip(g), u_c = clip(u)+off:
        du = G * a(g_c) * rs * [ul <= u <= uh]
        dg = G * u_c * rs * a'(g_c) * [gl <= g <= gh]
    Returns float64 [R][2I] = [dg | du] (un-rounded).
    """
    z = np.asarray(z, dtype=np.float64)
    I = z.shape[1] // 2
    g, u = z[:, :I], z[:, I:]
    gc = np.clip(g, ep.gate_lo, ep.gate_hi)
    uc = np.clip(u, ep.up_lo, ep.up_hi) + ep.up_offset
    Gs = np.asarray(G, dtype=np.float64)
    if row_scale is not None:
        Gs = Gs * np.asarray(row_scale, dtype=np.float64)[:, None]
    gmask = ((g >= ep.gate_lo) & (g <= ep.gate_hi)).astype(np.float64)
    umask = ((u >= ep.up_lo) & (u <= ep.up_hi)).astype(np.float64)
    du = Gs * activation(gc, ep.act, ep.alpha) * umask
    dg = Gs * uc * activation_grad(gc, ep.act, ep.alpha) * gmask
    return np.concatenate([dg, du], axis=1)


def dgrad_dglu(dy2_bits, counts, w2_bits, preact_bits, ep: Epilogue, dtype=np.float64):
    """Backward GroupGemm + dGLU: G_e = dY2_e @ W2_e^T, then ``dglu``.

    dy2 [M][H], w2 [E][I][H], preact [M][2I]; returns dgu bf16 bits [M][2I]
    in plain (gate | up) order.
    """
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    M = int(off[-1])
    E, I, H = w2_bits.shape
    out = np.zeros((M, 2 * I), dtype=np.uint16)
    rs_all = None if ep.row_scale is None else np.asarray(ep.row_scale, dtype=np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        G = _as_f(dy2_bits[a:b], dtype) @ _as_f(w2_bits[e], dtype).T
        rs = None if rs_all is None else rs_all[a:b]
        z = bf16_bits_to_f64(preact_bits[a:b])
        out[a:b] = f64_to_bf16_bits(dglu(G.astype(np.float64), z, ep, rs))
    return out


def dgrad_dact(dy2_bits, counts, w2_bits, preact_bits, ep: Epilogue, dtype=np.float64):
    """Backward of the non-gated form y = a(z) * rs (reading: sReLU, listed by
    [BLOG] beside the GLUs, taken without a gate; the same for any
    activation): dz = G * rs * a'(z) with G = dY2_e W2_e^T and z the saved bf16
    pre-activation [M][I].  Returns dz bf16 bits [M][I]."""
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    M = int(off[-1])
    E, I, H = w2_bits.shape
    out = np.zeros((M, I), dtype=np.uint16)
    rs_all = None if ep.row_scale is None else np.asarray(ep.row_scale, dtype=np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        G = (_as_f(dy2_bits[a:b], dtype) @ _as_f(w2_bits[e], dtype).T).astype(np.float64)
        if rs_all is not None:
            G = G * rs_all[a:b, None]
        z = bf16_bits_to_f64(preact_bits[a:b])
        out[a:b] = f64_to_bf16_bits(G * activation_grad(z, ep.act, ep.alpha))
    return out


def dx(dgu_bits, counts, w1_bits, dtype=np.float64):
    """dX_e = dgu_e @ W1_e^T with the plain (un-repacked) W1 [E][H][2I]."""
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    M = int(off[-1])
    E, H, N2 = w1_bits.shape
    out = np.zeros((M, H), dtype=np.uint16)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        c = _as_f(dgu_bits[a:b], dtype) @ _as_f(w1_bits[e], dtype).T
        out[a:b] = f64_to_bf16_bits(c.astype(np.float64))
    return out


def fc1_glu_mx(aq, as_, counts, w1q_t, w1s_t, ep: "Epilogue"):
    """FC1 + GLU with MXFP8 inputs ([BLOG] "Fusionando cuantización MXFP8…"):
    the exact dequantise-then-multiply pre-activation z_e = deq(A_e) deq(W_e)
    (+ bias), then the same epilogue as ``fc1_glu``.  aq [M][H] e4m3 codes
    with as_ [M][H/32] row scales; w1q_t [E][2I][H] the codes of W1_e^T in
    PLAIN (gate | up) order with w1s_t [E][2I][H/32].  Returns (preact, y)
    bf16 bits, as ``fc1_glu``."""
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    M = int(off[-1])
    E, N2, H = w1q_t.shape
    I = N2 // 2
    preact = np.zeros((M, 2 * I), dtype=np.uint16)
    y = np.zeros((M, I), dtype=np.uint16)
    rs_all = None if ep.row_scale is None else np.asarray(ep.row_scale, dtype=np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        z = mx_dequantize_rows(aq[a:b], as_[a:b]) @ mx_dequantize_rows(w1q_t[e], w1s_t[e]).T
        if ep.bias is not None:
            z = z + bf16_bits_to_f64(np.asarray(ep.bias)[e])[None, :]
        preact[a:b] = f64_to_bf16_bits(z)
        rs = None if rs_all is None else rs_all[a:b]
        y[a:b] = f64_to_bf16_bits(glu_from_preact(z, ep, rs))
    return preact, y


def tensor_amax(y_bits, counts) -> float:
    """Per-tensor amax of the FC1 output ([BLOG] "Fusionando cuantización
    MXFP8 y NVFP4": for NVFP4 the forward kernel emits the bf16 output and
    its per-tensor amax): max |y| over the routed rows [0, sum m_e) of the
    bf16 values as stored.  NaN entries are skipped (reading: an amax feeds a
    scale, and the GPU's maximum ignores NaN); no routed rows gives 0."""
    M = int(np.sum(np.asarray(counts, dtype=np.int64)))
    v = np.abs(bf16_bits_to_f64(np.asarray(y_bits)[:M]))
    v = v[~np.isnan(v)]
    return float(v.max()) if v.size else 0.0


def sylvester_hadamard(n: int) -> np.ndarray:
    """The Sylvester Hadamard matrix of order n (a power of two): H_1 = [1],
    H_2k = [[H_k, H_k], [H_k, -H_k]]."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rht16_amax(dgu_bits, counts, signs: int = 0) -> float:
    """Amax of the Hadamard rotation of the transposed backward output ([BLOG]
    "Fusionando cuantización MXFP8 y NVFP4": in back prop the kernel computes
    the amax of the Hadamard-rotated transpose of its output).  Readings: the
    rotation acts along the token dimension (the one the weight-gradient GEMM
    reduces over), in runs of 16 rows that restart at each group's first row
    (a run never mixes experts), a group's last run padded with zero rows; it
    is the orthonormal R = H16 S / 4 with S = diag(s_i), s_i = -1 where bit i
    of ``signs`` is set.  Returns max |R X| over all runs X (16 x 2I) of the
    bf16 values; NaN skipped; 0 without routed rows."""
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    s = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
    R = sylvester_hadamard(16) * s[None, :] / 4.0
    v = bf16_bits_to_f64(np.asarray(dgu_bits))
    amax = 0.0
    for e in range(len(counts)):
        for r0 in range(int(off[e]), int(off[e + 1]), 16):
            r1 = min(r0 + 16, int(off[e + 1]))
            X = np.zeros((16, v.shape[1]))
            X[: r1 - r0] = v[r0:r1]
            rot = np.abs(R @ X)
            rot = rot[~np.isnan(rot)]
            if rot.size:
                amax = max(amax, float(rot.max()))
    return amax


def bias_grad(dgu_bits, counts) -> np.ndarray:
    """Gradient of the FC1 bias: z = x W1 + b1 gives dL/db1_e = the sum over
    expert e's rows of dL/dz = dgu ("Boosting MoE Training Throughput with
    Advanced Fusion Kernels": the backward epilogue produces dgu; its column
    sums complete the backward step).  Reading: the sum of the bf16 values as
    stored.  Returns float64 [E][2I] in plain (gate | up) order; an empty
    expert gives zeros."""
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    v = bf16_bits_to_f64(np.asarray(dgu_bits))
    out = np.zeros((len(counts), v.shape[1]))
    for e in range(len(counts)):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            out[e] = v[a:b].sum(axis=0)
    return out


def row_scale_grad(dy2_bits, counts, w2_bits, preact_bits, ep: Epilogue) -> np.ndarray:
    """Gradient of the per-row scale: y_r = a(g_c) u_c rs_r gives dL/drs_r =
    sum_j G[r][j] a(g_c)[r][j] u_c[r][j] with G = dY2_e W2_e^T = dL/dy (the
    same GEMM as ``dgrad_dglu``) and g, u from the saved bf16
    pre-activation.  Returns float64 [M] over the routed rows."""
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    M = int(off[-1])
    out = np.zeros(M)
    ep_u = dataclasses.replace(ep, bias=None, row_scale=None)     # the unscaled y
    for e in range(len(counts)):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        G = bf16_bits_to_f64(dy2_bits[a:b]) @ bf16_bits_to_f64(w2_bits[e]).T
        yu = glu_from_preact(bf16_bits_to_f64(preact_bits[a:b]), ep_u)
        out[a:b] = np.sum(G * yu, axis=1)
    return out


def wgrad(a_bits, counts, b_bits, dtype=np.float64):
    """Weight gradient as a K-grouped GroupGemm: for each expert e with rows
    [o_e, o_e + m_e), C_e = A_e^T @ B_e, the reduction running over the
    group's rows ("Boosting MoE Training Throughput with Advanced Fusion
    Kernels": the column-wise copies exist "for back prop", i.e. for these
    products).  dW1 = wgrad(Xg, dgu) [E][H][2I] (plain W1 order) and
    dW2 = wgrad(y, dY2) [E][I][H].  An empty group gives zeros.  Returns
    float64 [E][P][Q]; the GPU keeps fp32.
    """
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    P, Q = a_bits.shape[1], b_bits.shape[1]
    out = np.zeros((len(counts), P, Q), dtype=np.float64)
    for e in range(len(counts)):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        out[e] = (_as_f(a_bits[a:b], dtype).T @ _as_f(b_bits[a:b], dtype)).astype(np.float64)
    return out


def wgrad_abs(a_bits, counts, b_bits):
    """sum_k |a_k| |b_k| for every element of ``wgrad`` (the scale of its
    rounding error under fp32 accumulation)."""
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    P, Q = a_bits.shape[1], b_bits.shape[1]
    out = np.zeros((len(counts), P, Q), dtype=np.float64)
    for e in range(len(counts)):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            out[e] = np.abs(bf16_bits_to_f64(a_bits[a:b])).T @ np.abs(bf16_bits_to_f64(b_bits[a:b]))
    return out


# ============================================================================ MXFP8
MX_BLOCK = 32


def mx_quantize_rows(v_bits, fmt: str = "e4m3"):
    """Row-wise MXFP8 ([BLOG] "Fusionando cuantización MXFP8…"): each run of 32
    consecutive columns of a row is one block with its own E8M0 scale; the
    elements are e4m3 codes, or e5m2 codes with ``fmt="e5m2"`` (gradients).

    v_bits [R][C] bf16 (C % 32 == 0).  Returns (q [R][C] uint8, s [R][C/32] uint8).
    """
    v = bf16_bits_to_f64(v_bits)
    R, C = v.shape
    q = np.zeros((R, C), dtype=np.uint8)
    s = np.zeros((R, C // MX_BLOCK), dtype=np.uint8)
    for r in range(R):
        for cb in range(C // MX_BLOCK):
            codes, byte = mx_quantize_block(v[r, cb * MX_BLOCK:(cb + 1) * MX_BLOCK], fmt)
            q[r, cb * MX_BLOCK:(cb + 1) * MX_BLOCK] = codes
            s[r, cb] = byte
    return q, s


def mx_scale_col_offsets(counts, blocked: bool = False) -> np.ndarray:
    """Scale-column (slot) offset of each group: so_e = sum_{j<e} ceil(m_j / 32),
    or in the K-tiled layout 4 sum_{j<e} ceil(m_j / 128)."""
    c = np.asarray(counts, dtype=np.int64)
    blocks = 4 * ((c + 127) // 128) if blocked else (c + MX_BLOCK - 1) // MX_BLOCK
    so = np.zeros(len(c) + 1, dtype=np.int64)
    so[1:] = np.cumsum(blocks)
    return so


def mx_col_slots(m_cap: int, E: int, blocked: bool = False) -> int:
    """Scale columns per row of a transposed copy: ceil(M_cap/32) + E, or
    4 (ceil(M_cap/128) + E) in the K-tiled layout."""
    return 4 * ((m_cap + 127) // 128 + E) if blocked else (m_cap + MX_BLOCK - 1) // MX_BLOCK + E


def mx_quantize_cols(v_bits, counts, m_cap: Optional[int] = None, fmt: str = "e4m3",
                     blocked: bool = False):
    """Column-wise (transposed) MXFP8 copy ([BLOG] "Fusionando cuantización
    MXFP8…": MXFP8 output plus a transposed version for back prop).

    Blocks are 32 consecutive rows of one column that restart at each group's
    first row; a group's last block may be partial and takes its amax over its
    valid rows only.  Returns (col_q, col_s).  Dense layout: col_q [C][M_cap]
    (block codes at the block's rows), col_s [C][ceil(M_cap/32)+E]; positions no
    group writes stay 0 here (the GPU leaves them untouched).  K-tiled layout
    (``blocked``; the operand layout of the MXFP8 weight gradient): col_s
    [C][S], S = 4 (ceil(M_cap/128) + E), col_q [C][32 S] with slot s = one
    block (codes at bytes 32 s .. 32 s + 31); group e's blocks take slots
    so_e + b, so_e = 4 sum_{j<e} ceil(m_j/128); the codes of rows past the
    group in its last block are 0, and its slots up to so_e + 4 ceil(m_e/128)
    that hold no row have zero codes and scale byte 127.
    """
    v = bf16_bits_to_f64(v_bits)
    R, C = v.shape
    counts = np.asarray(counts, dtype=np.int64)
    E = len(counts)
    off = exclusive_offsets(counts)
    if m_cap is None:
        m_cap = R
    so = mx_scale_col_offsets(counts, blocked)
    ncols = mx_col_slots(m_cap, E, blocked)
    col_q = np.zeros((C, 32 * ncols if blocked else m_cap), dtype=np.uint8)
    col_s = np.zeros((C, ncols), dtype=np.uint8)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        for blk, r0 in enumerate(range(a, b, MX_BLOCK)):
            r1 = min(r0 + MX_BLOCK, b)
            for c in range(C):
                codes, byte = mx_quantize_block(v[r0:r1, c], fmt)
                if blocked:
                    slot = int(so[e]) + blk
                    col_q[c, 32 * slot:32 * slot + (r1 - r0)] = codes
                else:
                    col_q[c, r0:r1] = codes
                col_s[c, so[e] + blk] = byte
        if blocked:
            for blk in range((b - a + MX_BLOCK - 1) // MX_BLOCK, int(so[e + 1] - so[e])):
                col_s[:, so[e] + blk] = 127
    return col_q, col_s


def mx_dequantize_cols(col_q, col_s, counts, m_cap: int, fmt: str = "e4m3",
                       blocked: bool = False) -> np.ndarray:
    """Values of a transposed MXFP8 copy (``mx_quantize_cols`` layouts), as
    float64 [M][C] over the routed rows: row r of group e, column c is
    decode(code) * 2^(scale - 127) of the block holding it."""
    from .formats import e8m0_value, fp8_decode
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    so = mx_scale_col_offsets(counts, blocked)
    C = col_q.shape[0]
    M = int(off[-1])
    out = np.zeros((M, C))
    for e in range(len(counts)):
        a, b = int(off[e]), int(off[e + 1])
        for blk, r0 in enumerate(range(a, b, MX_BLOCK)):
            r1 = min(r0 + MX_BLOCK, b)
            slot = int(so[e]) + blk
            codes = (col_q[:, 32 * slot:32 * slot + (r1 - r0)] if blocked else col_q[:, r0:r1])
            out[r0:r1] = (fp8_decode(codes, fmt) * e8m0_value(col_s[:, slot])[:, None]).T
    return out


def wgrad_mx(aq, as_, bq, bs, counts, m_cap: int, a_fmt: str = "e4m3", b_fmt: str = "e4m3",
             blocked: bool = True) -> np.ndarray:
    """MXFP8 weight gradient: the K-grouped GroupGemm of ``wgrad`` on
    transposed MXFP8 copies ("Boosting MoE Training Throughput with Advanced
    Fusion Kernels", section "Fusionando cuantización MXFP8 y NVFP4": the
    transposed copy exists for back prop), as the exact
    dequantise-then-multiply definition: C_e = deq(A)_e^T deq(B)_e in float64
    over the group's rows.  aq/as_ the copy of an [M_cap][P] tensor (codes,
    scales), bq/bs of an [M_cap][Q] one.  Returns float64 [E][P][Q]."""
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    A = mx_dequantize_cols(aq, as_, counts, m_cap, a_fmt, blocked)
    B = mx_dequantize_cols(bq, bs, counts, m_cap, b_fmt, blocked)
    out = np.zeros((len(counts), A.shape[1], B.shape[1]))
    for e in range(len(counts)):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            out[e] = A[a:b].T @ B[a:b]
    return out


def mx_dequantize_rows(q, s, fmt: str = "e4m3"):
    from .formats import e8m0_value, fp8_decode
    R, C = q.shape
    vals = fp8_decode(q, fmt)
    sc = np.repeat(e8m0_value(s), MX_BLOCK, axis=1)[:, :C]
    return vals * sc


def group_gemm_mx(aq, as_, counts, bq, bs, dtype=np.float64, a_fmt: str = "e4m3"):
    """MXFP8 x MXFP8 GroupGemm, as the exact dequantize-then-multiply definition.

    aq [M][K] e4m3 codes (e5m2 with ``a_fmt="e5m2"``, e.g. a gradient) with
    as_ [M][K/32] row scales; bq [E][N][K] e4m3 codes (the weight stored
    K-contiguous per output column) with bs [E][N][K/32].
    out_e = bf16( (deq A_e) @ (deq B_e)^T ).
    """
    counts = np.asarray(counts, dtype=np.int64)
    off = exclusive_offsets(counts)
    M = int(off[-1])
    E, N, K = bq.shape
    out = np.zeros((M, N), dtype=np.uint16)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        A = mx_dequantize_rows(aq[a:b], as_[a:b], a_fmt).astype(dtype)
        B = mx_dequantize_rows(bq[e], bs[e]).astype(dtype)
        out[a:b] = f64_to_bf16_bits((A @ B.T).astype(np.float64))
    return out
