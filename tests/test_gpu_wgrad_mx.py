"""GPU parity of the MXFP8 weight gradients and of the K-tiled transposed
MXFP8 copies they read ("Boosting MoE Training Throughput with Advanced Fusion
Kernels", section "Fusionando cuantización MXFP8 y NVFP4": the epilogues
write a transposed copy for back prop), through the C ABI.

* K-tiled copies from the standalone quantiser, the FC1 + GLU epilogue and
  the dgrad + dGLU epilogue against the oracle's quantisation of the oracle's
  values (scales by the E8M0 rule, codes byte for byte where the source
  values agree, padding slots exact).
* moe_group_gemm_wgrad_mx on copies the oracle quantised: bit for bit on
  small-integer inputs (every product and partial sum exact), and within
  |gpu - ref| <= MX_ACC_REL sum|a b| + m_e 2^-24 sum|a b| on Gaussian inputs
  (the block-scaled MFMA's accumulation and fp32 summation).
* The chain FC1 (K-tiled copy of y) and the quantised dY2 feeding the MXFP8
  dW2, against the oracle's chain; the allowance adds sum |a' - a| |b| over
  the GPU's own y codes (bounded separately by the copy check).
Every expected value comes from the oracle on oracle-side inputs.
"""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O
from tests.gpu_util import (MX_ACC_REL, assert_mx_cols, dev_bits, dev_bytes, dev_i32, empty_bits,
                            empty_bytes, host_bits)

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


def _cols_buffers(G, C, m_cap, E):
    S = G.mx_col_slots(m_cap, E, blocked=True)
    return empty_bytes((C, 32 * S)), empty_bytes((C, S)), S


def _gpu_quantize_cols(G, v, counts, m_cap, e5=False):
    C = v.shape[1]
    q, s, _ = _cols_buffers(G, C, m_cap, len(counts))
    G.moe_mxfp8_quantize(dev_bits(v), m_cap, C, G.groups(dev_i32(counts), m_cap),
                         G.mx_out(col_q=q, col_s=s, e5m2=e5, col_blocked=True))
    _sync()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_k_tiled_columns_bit_exact(G, fmt):
    counts = np.array([40, 0, 129, 5, 128, 300])
    M = int(counts.sum())
    m_cap = M + 9
    rng = np.random.default_rng(71)
    v = W.to_bf16_bits((rng.standard_normal((m_cap, 96)) * 2.0 ** rng.integers(-6, 6, (m_cap, 1)))
                       .astype(np.float32))
    q, s = _gpu_quantize_cols(G, v, counts, m_cap, e5=fmt == "e5m2")
    rq, rs = O.mx_quantize_cols(v[:M], counts, m_cap=m_cap, fmt=fmt, blocked=True)
    used = int(O.mx_scale_col_offsets(counts, blocked=True)[-1])
    assert np.array_equal(s[:, :used], rs[:, :used])
    assert np.array_equal(q[:, :32 * used], rq[:, :32 * used])
    assert np.all(s[:, used:] == 0xA5) and np.all(q[:, 32 * used:] == 0xA5)   # untouched


def test_fc1_and_dglu_epilogues_write_k_tiled_copies(G):
    counts = np.array([300, 0, 57, 260, 1])
    E, H, I = len(counts), 128, 192
    M = int(counts.sum())
    m_cap = M + 7
    d = W.small_grouped(72, counts, H, I, m_cap=m_cap)
    w1p = empty_bits((G.moe_packed_w1_bytes(E, H, I) // 2,))
    G.moe_repack_gate_up(dev_bits(d["w1"]), E, H, I, w1p)
    y, pre = empty_bits((m_cap, I)), empty_bits((m_cap, 2 * I))
    yq, ys, _ = _cols_buffers(G, I, m_cap, E)
    grp = G.groups(dev_i32(counts), m_cap)
    G.moe_group_gemm_glu_fwd(dev_bits(d["x"]), grp, w1p, H, I, G.epilogue("swiglu"), y, pre,
                             G.mx_out(col_q=yq, col_s=ys, col_blocked=True))
    _sync()
    rp, ry = O.fc1_glu(d["x"][:M], counts, d["w1"], O.Epilogue())
    assert_mx_cols(yq.cpu().numpy(), ys.cpu().numpy(), host_bits(y)[:M], ry, counts, m_cap,
                   "fc1 y k-tiled cols", blocked=True)
    # dgrad + dGLU from the oracle's pre-activation, e5m2 copy of dgu
    rng = np.random.default_rng(73)
    dy2 = W.to_bf16_bits((rng.standard_normal((m_cap, H)) * 0.1).astype(np.float32))
    pre_in = np.zeros((m_cap, 2 * I), np.uint16)
    pre_in[:M] = rp
    w2p = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))
    G.moe_pack_weight(dev_bits(d["w2"]), E, I, H, G.B_NK, w2p)
    dgu = empty_bits((m_cap, 2 * I))
    gq, gs, _ = _cols_buffers(G, 2 * I, m_cap, E)
    G.moe_group_gemm_dglu_bwd(dev_bits(dy2), G.operand(w2p, layout=G.B_PACKED), H, I, grp,
                              dev_bits(pre_in), G.epilogue("swiglu"), dgu,
                              G.mx_out(col_q=gq, col_s=gs, e5m2=True, col_blocked=True))
    _sync()
    rdgu = O.dgrad_dglu(dy2[:M], counts, d["w2"], rp, O.Epilogue())
    assert_mx_cols(gq.cpu().numpy(), gs.cpu().numpy(), host_bits(dgu)[:M], rdgu, counts, m_cap,
                   "dgu k-tiled cols", fmt="e5m2", blocked=True)


def _wgrad_mx_gpu(G, aq, as_, bq, bs, counts, m_cap, P, Q, a_e5=False, b_e5=False, init=None,
                  accumulate=False):
    import torch
    E = len(counts)
    if init is None:
        c = torch.full((E, P, Q), float("nan"), dtype=torch.float32, device="cuda")
    else:
        c = torch.from_numpy(init.astype(np.float32)).cuda()
    a_op = G.operand(dev_bytes(aq), dtype=G.DT_MXFP8_E5M2 if a_e5 else G.DT_MXFP8, scales=dev_bytes(as_))
    b_op = G.operand(dev_bytes(bq), dtype=G.DT_MXFP8_E5M2 if b_e5 else G.DT_MXFP8, scales=dev_bytes(bs))
    G.moe_group_gemm_wgrad_mx(a_op, b_op, P, Q, G.groups(dev_i32(counts), m_cap), c, accumulate)
    _sync()
    return c.cpu().numpy().astype(np.float64)


def _abs_terms(aq, as_, bq, bs, counts, m_cap, fa, fb):
    A = np.abs(O.mx_dequantize_cols(aq, as_, counts, m_cap, fa, blocked=True))
    B = np.abs(O.mx_dequantize_cols(bq, bs, counts, m_cap, fb, blocked=True))
    off = np.concatenate([[0], np.cumsum(counts)])
    out = np.zeros((len(counts), A.shape[1], B.shape[1]))
    for e in range(len(counts)):
        if off[e + 1] > off[e]:
            out[e] = A[off[e]:off[e + 1]].T @ B[off[e]:off[e + 1]]
    return out


@pytest.mark.parametrize("counts,P,Q,fa,fb", [([130, 0, 31, 64, 1, 300], 192, 320, "e4m3", "e4m3"),
                                              ([513], 256, 64, "e4m3", "e5m2"),
                                              ([0, 97, 0], 64, 256, "e5m2", "e5m2")])
def test_wgrad_mx_integer_exact(G, counts, P, Q, fa, fb):
    """Small integers are exact in both formats and their products and sums
    stay exact integers in fp32: the result is the oracle's bit for bit."""
    counts = np.array(counts)
    M = int(counts.sum())
    m_cap = M + 5
    rng = np.random.default_rng(74 + P)
    a = W.to_bf16_bits(rng.integers(-7, 8, (m_cap, P)).astype(np.float32))
    b = W.to_bf16_bits(rng.integers(-7, 8, (m_cap, Q)).astype(np.float32))
    aq, as_ = O.mx_quantize_cols(a[:M], counts, m_cap=m_cap, fmt=fa, blocked=True)
    bq, bs = O.mx_quantize_cols(b[:M], counts, m_cap=m_cap, fmt=fb, blocked=True)
    got = _wgrad_mx_gpu(G, aq, as_, bq, bs, counts, m_cap, P, Q, fa == "e5m2", fb == "e5m2")
    ref = O.wgrad_mx(aq, as_, bq, bs, counts, m_cap, fa, fb)
    assert np.array_equal(got, ref)
    assert np.array_equal(ref, O.wgrad(a[:M], counts, b[:M]))   # the copies are exact here


@pytest.mark.parametrize("counts,fa,fb", [([200, 0, 77, 129], "e4m3", "e5m2"),
                                          ([1000, 3], "e4m3", "e4m3")])
def test_wgrad_mx_gaussian(G, counts, fa, fb):
    counts = np.array(counts)
    M = int(counts.sum())
    P, Q = 128, 192
    rng = np.random.default_rng(75)
    a = W.to_bf16_bits(rng.standard_normal((M, P)).astype(np.float32))
    b = W.to_bf16_bits((rng.standard_normal((M, Q)) * 1e-2).astype(np.float32))
    aq, as_ = O.mx_quantize_cols(a, counts, m_cap=M, fmt=fa, blocked=True)
    bq, bs = O.mx_quantize_cols(b, counts, m_cap=M, fmt=fb, blocked=True)
    got = _wgrad_mx_gpu(G, aq, as_, bq, bs, counts, M, P, Q, fa == "e5m2", fb == "e5m2")
    ref = O.wgrad_mx(aq, as_, bq, bs, counts, M, fa, fb)
    S = _abs_terms(aq, as_, bq, bs, counts, M, fa, fb)
    bound = (MX_ACC_REL + max(int(counts.max()), 1) * 2.0 ** -24) * S
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        dev = np.where(S > 0, err / S, 0.0)
    print(f"[mx-acc] wgrad_mx {counts.tolist()} {fa}/{fb}: max |err| / sum|ab| = "
          f"2^{np.log2(max(dev.max(), 1e-300)):.2f}")
    assert np.all(err <= bound + 1e-30), f"{np.sum(err > bound)} elements out of bound"
    nr = np.linalg.norm(ref)
    assert np.linalg.norm(got - ref) / nr <= 1e-4


def test_wgrad_mx_accumulate_and_empty_groups(G):
    counts = np.array([0, 64, 0])
    M, P, Q = 64, 64, 128
    rng = np.random.default_rng(76)
    a = W.to_bf16_bits(rng.integers(-3, 4, (M, P)).astype(np.float32))
    b = W.to_bf16_bits(rng.integers(-3, 4, (M, Q)).astype(np.float32))
    aq, as_ = O.mx_quantize_cols(a, counts, m_cap=M, blocked=True)
    bq, bs = O.mx_quantize_cols(b, counts, m_cap=M, blocked=True)
    init = rng.integers(-5, 6, (3, P, Q)).astype(np.float64)
    got = _wgrad_mx_gpu(G, aq, as_, bq, bs, counts, M, P, Q, init=init, accumulate=True)
    assert np.array_equal(got, init + O.wgrad_mx(aq, as_, bq, bs, counts, M))
    got0 = _wgrad_mx_gpu(G, aq, as_, bq, bs, counts, M, P, Q)
    assert np.all(got0[0] == 0) and np.all(got0[2] == 0)


def test_fc1_copy_and_quantised_dy2_feed_mxfp8_dw2(G):
    """dW2 = y^T dY2 from the K-tiled copies: y's written by the FC1 + SwiGLU
    epilogue, dY2's by the standalone quantiser (e5m2), against the oracle's
    chain.  The GPU's y may differ from the oracle's by a bf16 rounding, so
    the allowance adds sum_k |y'_k - y_k| |dy_k| over the two copies."""
    counts = np.array([300, 0, 57, 129])
    E, H, I = len(counts), 128, 128
    M = int(counts.sum())
    d = W.small_grouped(77, counts, H, I, m_cap=M)
    rng = np.random.default_rng(77)
    dy2 = W.to_bf16_bits((rng.standard_normal((M, H)) * 0.1).astype(np.float32))
    w1p = empty_bits((G.moe_packed_w1_bytes(E, H, I) // 2,))
    G.moe_repack_gate_up(dev_bits(d["w1"]), E, H, I, w1p)
    y = empty_bits((M, I))
    yq, ys, _ = _cols_buffers(G, I, M, E)
    grp = G.groups(dev_i32(counts), M)
    G.moe_group_gemm_glu_fwd(dev_bits(d["x"]), grp, w1p, H, I, G.epilogue("swiglu"), y, None,
                             G.mx_out(col_q=yq, col_s=ys, col_blocked=True))
    dq, ds_ = _gpu_quantize_cols(G, dy2, counts, M, e5=True)
    import torch
    c = torch.full((E, I, H), float("nan"), dtype=torch.float32, device="cuda")
    G.moe_group_gemm_wgrad_mx(G.operand(yq, dtype=G.DT_MXFP8, scales=ys),
                              G.operand(dev_bytes(dq), dtype=G.DT_MXFP8_E5M2, scales=dev_bytes(ds_)),
                              I, H, grp, c)
    _sync()
    got = c.cpu().numpy().astype(np.float64)
    _, ry = O.fc1_glu(d["x"], counts, d["w1"], O.Epilogue())
    rq, rs = O.mx_quantize_cols(ry, counts, m_cap=M, blocked=True)
    bq, bs = O.mx_quantize_cols(dy2, counts, m_cap=M, fmt="e5m2", blocked=True)
    used = int(O.mx_scale_col_offsets(counts, blocked=True)[-1])
    assert np.array_equal(dq[:, :32 * used], bq[:, :32 * used]) and np.array_equal(ds_[:, :used], bs[:, :used])
    ref = O.wgrad_mx(rq, rs, bq, bs, counts, M, "e4m3", "e5m2")
    S = _abs_terms(rq, rs, bq, bs, counts, M, "e4m3", "e5m2")
    Ag = O.mx_dequantize_cols(yq.cpu().numpy(), ys.cpu().numpy(), counts, M, blocked=True)
    Ar = O.mx_dequantize_cols(rq, rs, counts, M, blocked=True)
    B = np.abs(O.mx_dequantize_cols(bq, bs, counts, M, "e5m2", blocked=True))
    off = np.concatenate([[0], np.cumsum(counts)])
    D = np.zeros_like(S)
    for e in range(E):
        D[e] = np.abs(Ag - Ar)[off[e]:off[e + 1]].T @ B[off[e]:off[e + 1]]
    bound = (MX_ACC_REL + int(counts.max()) * 2.0 ** -24) * S + D
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)) and np.all(err <= bound + 1e-30), f"{np.sum(err > bound)} out of bound"
