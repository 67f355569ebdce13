"""GPU parity of the MXFP8 x MXFP8 GroupGemm (block-scaled MFMA) and of the
offline MXFP8 weight pack, through the C ABI, against the CPU oracle.

MXFP8 here follows "Boosting MoE Training Throughput with Advanced Fusion
Kernels", section "Fusionando cuantización MXFP8…": blocks of 32 values along
the reduction dimension, one E8M0 scale each, e4m3 elements.  Quantised codes
and scales are compared bit-exactly; the GEMM's bf16 output within
    |gpu - ref| <= 2e-2 (1 + |ref|) + 2.2e-4 sum_k |a_k b_k| (+ D)
of the exact dequantise-then-multiply result.  The second term covers the
block-scaled MFMA's internal accumulation, which is not strict fp32 (its
deviation beyond the output rounding reached 2^-13.18 sum |a b| over the MXFP8
tests; every test prints the largest deviation it saw).  D appears only where the GPU
product reads codes the GPU quantised itself (a chained forward): the sum of
|a'_k - a_k| |b_k| over the code differences, which the MXFP8 copy checks
bound separately.  A wrong scale or a misplaced K block gives errors of the
order of sum |a b| itself.
Every expected value comes from the oracle on oracle-side inputs.
"""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O
from tests.gpu_util import (BF16_NAN_SENTINEL, MX_ACC_REL, assert_bf16_close, assert_mx_gemm_close,
                            dev_bits, dev_bytes, dev_i32, empty_bits, empty_bytes, host_bits,
                            mx_acc_excess, mx_gemm_terms, packed_mx_layout)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_glu_amd as G
    G.moe_init(0)
    return G


def _sync():
    import torch
    torch.cuda.synchronize()


def _weight_nk(seed, E, N, K, std=0.05):
    """bf16 [E][N][K] with per-row magnitudes spread over 2^-20 .. 2^20 and an
    all-zero 32-block, so scales cover a wide exponent range."""
    g = np.random.default_rng(seed)
    w = g.standard_normal((E, N, K)).astype(np.float32) * np.float32(std)
    w *= (2.0 ** g.integers(-20, 21, size=(E, N, 1))).astype(np.float32)
    w[0, 0, :32] = 0.0
    return W.to_bf16_bits(w)


def _oracle_weight_mx(w_nk):
    E, N, K = w_nk.shape
    bq = np.zeros((E, N, K), np.uint8)
    bs = np.zeros((E, N, K // 32), np.uint8)
    for e in range(E):
        bq[e], bs[e] = O.mx_quantize_rows(w_nk[e])
    return bq, bs


def _pack_mx_gpu(G, w_nk, layout):
    E, N, K = w_nk.shape
    src = w_nk if layout == "NK" else np.ascontiguousarray(np.transpose(w_nk, (0, 2, 1)))
    d_q = empty_bytes((G.moe_packed_mx_weight_bytes(E, N, K),))
    d_s = empty_bytes((G.moe_packed_mx_scale_bytes(E, N, K),))
    G.moe_pack_weight_mx(dev_bits(src), E, N, K, G.B_NK if layout == "NK" else G.B_KN, d_q, d_s)
    return d_q, d_s


@pytest.mark.parametrize("layout,E,N,K", [("KN", 2, 192, 256), ("NK", 1, 256, 128),
                                          ("KN", 3, 320, 384)])
def test_pack_weight_mx_bit_exact(G, layout, E, N, K):
    w_nk = _weight_nk(N + K + E, E, N, K)
    d_q, d_s = _pack_mx_gpu(G, w_nk, layout)
    _sync()
    q_ref, s_ref = packed_mx_layout(*_oracle_weight_mx(w_nk))
    assert np.array_equal(d_q.cpu().numpy(), q_ref)
    assert np.array_equal(d_s.cpu().numpy(), s_ref)


def _group_gemm_mx_gpu(G, aq, as_, counts, d_q, d_s, N, K, m_cap):
    c = empty_bits((m_cap, N))
    a_op = G.operand(dev_bytes(aq), dtype=G.DT_MXFP8, scales=dev_bytes(as_))
    b_op = G.operand(d_q, dtype=G.DT_MXFP8, layout=G.B_PACKED, scales=d_s)
    G.moe_group_gemm_quant(a_op, b_op, N, K, G.groups(dev_i32(counts), m_cap), c)
    _sync()
    return host_bits(c)


@pytest.mark.parametrize("counts,K,N", [([300, 0, 213], 384, 320),   # odd K-tile count
                                        ([700, 129], 256, 256),      # several m-tiles
                                        ([5], 128, 64),              # one partial tile
                                        ([0, 0, 40, 0], 512, 192)])  # mostly empty experts
def test_group_gemm_mx(G, counts, K, N):
    counts = np.array(counts)
    E, M = len(counts), int(counts.sum())
    m_cap = M + 7
    g = np.random.default_rng(K + N + M)
    a = W.to_bf16_bits(g.standard_normal((m_cap, K)).astype(np.float32))
    aq, as_ = O.mx_quantize_rows(a)
    w_nk = W.to_bf16_bits((g.standard_normal((E, N, K)) * 0.05).astype(np.float32))
    d_q, d_s = _pack_mx_gpu(G, w_nk, "KN")
    out = _group_gemm_mx_gpu(G, aq, as_, counts, d_q, d_s, N, K, m_cap)
    bq, bs = _oracle_weight_mx(w_nk)
    ref = O.group_gemm_mx(aq[:M], as_[:M], counts, bq, bs)
    assert_mx_gemm_close(out[:M], ref, aq[:M], as_[:M], counts, bq, bs, f"group_gemm_mx {counts.tolist()}",
                         normwise=1e-2)
    assert np.all(out[M:] == BF16_NAN_SENTINEL)


def test_group_gemm_mx_heavy_tails(G):
    """Student-t activations (config-5 style) with per-row magnitude spread."""
    counts = np.array([260, 77])
    E, M, K, N = 2, 337, 256, 128
    a = W.student_t_rows_bf16(5, M, K)
    aq, as_ = O.mx_quantize_rows(a)
    w_nk = _weight_nk(9, E, N, K, std=0.02)
    d_q, d_s = _pack_mx_gpu(G, w_nk, "NK")
    out = _group_gemm_mx_gpu(G, aq, as_, counts, d_q, d_s, N, K, M)
    bq, bs = _oracle_weight_mx(w_nk)
    ref = O.group_gemm_mx(aq, as_, counts, bq, bs)
    assert_mx_gemm_close(out, ref, aq, as_, counts, bq, bs, "group_gemm_mx student-t", normwise=1e-2)


def test_fc1_mx_rows_feed_fc2_mx(G):
    """FC1 + SwiGLU with the fused row-wise MXFP8 output, consumed directly by
    the block-scaled FC2; the expected value is the oracle's own chain (FC1,
    SwiGLU, MXFP8 rows, dequantise-then-multiply FC2)."""
    import torch
    counts = [200, 0, 57, 300]
    E, H, I = 4, 128, 256
    d = W.small_grouped(31, counts, H, I, m_cap=600)
    m_cap, M = d["M_cap"], d["M"]
    w1p = empty_bits((G.moe_packed_w1_bytes(E, H, I) // 2,))
    G.moe_repack_gate_up(dev_bits(d["w1"]), E, H, I, w1p)
    y = empty_bits((m_cap, I))
    row_q, row_s = empty_bytes((m_cap, I)), empty_bytes((m_cap, I // 32))
    grp = G.groups(dev_i32(d["counts"]), m_cap)
    G.moe_group_gemm_glu_fwd(dev_bits(d["x"]), grp, w1p, H, I, G.epilogue("swiglu"), y, None,
                             G.mx_out(row_q=row_q, row_s=row_s))
    w2_nk = np.ascontiguousarray(np.transpose(d["w2"], (0, 2, 1)))      # [E][H][I]
    d_q, d_s = _pack_mx_gpu(G, w2_nk, "NK")
    out2 = empty_bits((m_cap, H))
    G.moe_group_gemm_quant(G.operand(row_q, dtype=G.DT_MXFP8, scales=row_s),
                           G.operand(d_q, dtype=G.DT_MXFP8, layout=G.B_PACKED, scales=d_s),
                           H, I, grp, out2)
    _sync()
    _, ry = O.fc1_glu(d["x"][:M], d["counts"], d["w1"], O.Epilogue())
    yq, ys = O.mx_quantize_rows(ry)
    bq, bs = _oracle_weight_mx(w2_nk)
    ref = O.group_gemm_mx(yq, ys, d["counts"], bq, bs)
    assert_mx_gemm_close(host_bits(out2)[:M], ref, yq, ys, d["counts"], bq, bs, "fc1 mx -> fc2 mx",
                         gpu_aq=row_q.cpu().numpy()[:M], gpu_as=row_s.cpu().numpy()[:M],
                         normwise=2e-2)


# ---------------------------------------------------------------- MXFP8 FC1 (inputs)
def _oracle_w1_mx(w1):
    """MXFP8 codes/scales of W1_e^T [2I][H] in plain order, and in the packed
    gate/up row order (the layout moe_repack_gate_up_mx writes)."""
    E, H, N2 = w1.shape
    w1t = np.ascontiguousarray(np.transpose(w1, (0, 2, 1)))
    q, s = _oracle_weight_mx(w1t)
    perm = O.packed_column_of(np.arange(N2), N2 // 2)      # plain column -> packed row
    qp, sp = np.zeros_like(q), np.zeros_like(s)
    qp[:, perm], sp[:, perm] = q, s
    return q, s, qp, sp


@pytest.mark.parametrize("E,H,I", [(2, 128, 64), (3, 256, 192), (1, 384, 320)])
def test_repack_gate_up_mx_bit_exact(G, E, H, I):
    w1 = W.to_bf16_bits((np.random.default_rng(H + I).standard_normal((E, H, 2 * I)) * 0.05)
                        .astype(np.float32))
    d_q = empty_bytes((G.moe_packed_mx_weight_bytes(E, 2 * I, H),))
    d_s = empty_bytes((G.moe_packed_mx_scale_bytes(E, 2 * I, H),))
    G.moe_repack_gate_up_mx(dev_bits(w1), E, H, I, d_q, d_s)
    _sync()
    _, _, qp, sp = _oracle_w1_mx(w1)
    q_ref, s_ref = packed_mx_layout(qp, sp)
    assert np.array_equal(d_q.cpu().numpy(), q_ref)
    assert np.array_equal(d_s.cpu().numpy(), s_ref)


def _fc1_mx_gpu(G, aq, as_, counts, w1, H, I, m_cap, ep, mx=False):
    E = w1.shape[0]
    d_q = empty_bytes((G.moe_packed_mx_weight_bytes(E, 2 * I, H),))
    d_s = empty_bytes((G.moe_packed_mx_scale_bytes(E, 2 * I, H),))
    G.moe_repack_gate_up_mx(dev_bits(w1), E, H, I, d_q, d_s)
    y, pre = empty_bits((m_cap, I)), empty_bits((m_cap, 2 * I))
    bufs = None
    if mx:
        bufs = dict(row_q=empty_bytes((m_cap, I)), row_s=empty_bytes((m_cap, I // 32)))
    G.moe_group_gemm_glu_fwd_mx(G.operand(dev_bytes(aq), dtype=G.DT_MXFP8, scales=dev_bytes(as_)),
                                G.groups(dev_i32(counts), m_cap),
                                G.operand(d_q, dtype=G.DT_MXFP8, layout=G.B_PACKED, scales=d_s),
                                H, I, ep, y, pre, None if bufs is None else G.mx_out(**bufs))
    _sync()
    out = dict(y=host_bits(y), pre=host_bits(pre))
    if bufs:
        out.update({k: v.cpu().numpy() for k, v in bufs.items()})
    return out


@pytest.mark.parametrize("bias", [False, True])
def test_fc1_glu_fwd_mx(G, bias):
    counts = np.array([300, 0, 57, 260])
    E, H, I = 4, 256, 320                 # I = 320: a half n-tile
    M = int(counts.sum())
    m_cap = M + 9
    d = W.small_grouped(34, counts, H, I, bias=bias, m_cap=m_cap)
    x = W.student_t_rows_bf16(34, m_cap, H)
    aq, as_ = O.mx_quantize_rows(x)
    kw = dict(alpha=1.702, gate_lo=-7.0, gate_hi=7.0, up_lo=-7.0, up_hi=7.0) if bias else {}
    ep = G.epilogue(bias=dev_bits(d["b1"]) if bias else None, **kw)
    out = _fc1_mx_gpu(G, aq, as_, counts, d["w1"], H, I, m_cap, ep)
    q, s, _, _ = _oracle_w1_mx(d["w1"])
    ep_o = O.Epilogue(bias=d["b1"] if bias else None, **kw)
    rp, ry = O.fc1_glu_mx(aq[:M], as_[:M], counts, q, s, ep_o)
    S, _, X = mx_gemm_terms(aq[:M], as_[:M], counts, q, s)
    if bias:
        off = np.concatenate([[0], np.cumsum(counts)])
        for e in range(E):
            X[off[e]:off[e + 1]] += F.bf16_bits_to_f64(d["b1"][e])
    mx_acc_excess(out["pre"][:M], S, np.zeros_like(S), X, f"fc1 mx preact bias={bias}")
    zb = MX_ACC_REL * S                                     # accumulation bound on z
    assert_bf16_close(out["pre"][:M], rp, what="fc1 mx preact", extra=zb)
    # y = a(g) u: an error dz of z moves y by at most |a'(g)| |u| dz_g + |a(g)| dz_u,
    # with |a'| <= 1.1 and |a(g)| <= |g| for SwiGLU (alpha >= 1)
    zr = np.abs(F.bf16_bits_to_f64(rp))
    ey = 1.2 * zr[:, I:] * zb[:, :I] + (zr[:, :I] + 1.0) * zb[:, I:]
    assert_bf16_close(out["y"][:M], ry, what="fc1 mx y", normwise=2e-2, extra=ey)
    assert np.all(out["y"][M:] == BF16_NAN_SENTINEL) and np.all(out["pre"][M:] == BF16_NAN_SENTINEL)


def test_mxfp8_forward_chain(G):
    """The MXFP8 forward: rows quantised on the GPU, FC1 + SwiGLU on the
    block-scaled MFMA writing the MXFP8 rows of y, FC2 on the block-scaled
    MFMA; the oracle runs the same chain from the same bf16 inputs."""
    counts = np.array([200, 0, 57, 300])
    E, H, I = 4, 256, 256
    M = int(counts.sum())
    d = W.small_grouped(35, counts, H, I, m_cap=M)
    x = W.student_t_rows_bf16(35, M, H)
    xq, xs = empty_bytes((M, H)), empty_bytes((M, H // 32))
    G.moe_mxfp8_quantize(dev_bits(x), M, H, None, G.mx_out(row_q=xq, row_s=xs))
    _sync()
    aq, as_ = O.mx_quantize_rows(x)
    assert np.array_equal(xq.cpu().numpy(), aq) and np.array_equal(xs.cpu().numpy(), as_)
    out = _fc1_mx_gpu(G, aq, as_, counts, d["w1"], H, I, M, G.epilogue(), mx=True)
    w2_nk = np.ascontiguousarray(np.transpose(d["w2"], (0, 2, 1)))
    d_q, d_s = _pack_mx_gpu(G, w2_nk, "NK")
    out2 = empty_bits((M, H))
    G.moe_group_gemm_quant(G.operand(dev_bytes(out["row_q"]), dtype=G.DT_MXFP8,
                                     scales=dev_bytes(out["row_s"])),
                           G.operand(d_q, dtype=G.DT_MXFP8, layout=G.B_PACKED, scales=d_s),
                           H, I, G.groups(dev_i32(counts), M), out2)
    _sync()
    q1, s1, _, _ = _oracle_w1_mx(d["w1"])
    _, ry = O.fc1_glu_mx(aq, as_, counts, q1, s1, O.Epilogue())
    yq, ys = O.mx_quantize_rows(ry)
    bq, bs = _oracle_weight_mx(w2_nk)
    ref = O.group_gemm_mx(yq, ys, counts, bq, bs)
    assert_mx_gemm_close(host_bits(out2), ref, yq, ys, counts, bq, bs, "mx forward chain",
                         gpu_aq=out["row_q"], gpu_as=out["row_s"], normwise=3e-2)
