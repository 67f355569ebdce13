"""Gradients of the epilogue's own parameters from the backward dGLU kernel:
d(bias) = per-expert column sums of dgu, d(row_scale) = sum_j G a(g_c) u_c,
both added atomically into caller-zeroed fp32 buffers.

Checks: on sReLU with ternary data every dgu value, product and sum is a small
integer, exact in fp32 whatever the order, so both gradients must equal the
oracle's bit for bit.  On SwiGLU with row scales, d(bias) must equal the
column sums of the GPU's own dgu up to fp32 summation (n 2^-24 sum|v|) and the
oracle's within the summed bf16 tolerance of dgu; d(row_scale) must agree with
the oracle's within fp32 accumulation error (1e-4 of sum |G a u|).  Asking for
them leaves dgu unchanged, and rows past the routed ones stay untouched.
"""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O
from tests.gpu_util import assert_bf16_close, dev_bits, dev_i32, empty_bits, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_glu_amd as G
    G.moe_init(0)
    return G


def _dglu_grads(G, dy2, w2, pre, counts, m_cap, ep_kw, rs=None, grads=True, layout="PACKED"):
    import torch
    E, I, H = w2.shape
    if layout == "PACKED":
        d_w2 = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))
        G.moe_pack_weight(dev_bits(w2), E, I, H, G.B_NK, d_w2)
        op = G.operand(d_w2, layout=G.B_PACKED)
    else:
        op = G.operand(dev_bits(w2), layout=G.B_NK)
    dgu = empty_bits((m_cap, 2 * I))
    db = torch.zeros((E, 2 * I), dtype=torch.float32, device="cuda") if grads else None
    drs = torch.full((m_cap,), 0.0, dtype=torch.float32, device="cuda") if grads else None
    if grads:
        drs[int(np.sum(counts)):] = 12345.0          # sentinel: rows past the routed ones
    d_rs = torch.from_numpy(rs).cuda() if rs is not None else None
    ep = G.epilogue(row_scale=d_rs, dbias_out=db, drow_scale_out=drs, **ep_kw)
    G.moe_group_gemm_dglu_bwd(dev_bits(dy2), op, H, I, G.groups(dev_i32(counts), m_cap),
                              dev_bits(pre), ep, dgu, None)
    torch.cuda.synchronize()
    out = dict(dgu=host_bits(dgu))
    if grads:
        out["db"] = db.cpu().numpy().astype(np.float64)
        out["drs"] = drs.cpu().numpy().astype(np.float64)
    return out


@pytest.mark.parametrize("layout", ["PACKED", "NK"])
def test_param_grads_integer_exact(G, layout):
    counts = np.array([40, 0, 300, 17, 100, 130])   # 100: a half tile past 64 rows; 130: a full tile past 128
    E, H, I = len(counts), 64, 192
    M = int(counts.sum())
    m_cap = M + 11
    dy2 = W.ternary_bf16(81, (m_cap, H))
    w2 = W.ternary_bf16(82, (E, I, H))
    pre = W.ternary_bf16(83, (m_cap, 2 * I))
    out = _dglu_grads(G, dy2, w2, pre, counts, m_cap, dict(act="srelu"), layout=layout)
    ep = O.Epilogue(act="srelu")
    ref = O.dgrad_dglu(dy2[:M], counts, w2, pre[:M], ep)
    assert np.array_equal(out["dgu"][:M], ref)
    assert np.array_equal(out["db"], O.bias_grad(ref, counts))
    want = O.row_scale_grad(dy2[:M], counts, w2, pre[:M], ep)
    assert np.array_equal(out["drs"][:M], want)
    assert np.all(out["drs"][M:] == 12345.0)


def test_param_grads_swiglu_with_row_scale(G):
    counts = np.array([64, 0, 300, 1, 270])
    E, H, I = len(counts), 256, 320
    M = int(counts.sum())
    m_cap = M + 9
    rng = np.random.default_rng(84)
    dy2 = W.to_bf16_bits((rng.standard_normal((m_cap, H)) * 0.1).astype(np.float32))
    w2 = W.to_bf16_bits((rng.standard_normal((E, I, H)) * 0.05).astype(np.float32))
    pre = W.to_bf16_bits((rng.standard_normal((m_cap, 2 * I)) * 2).astype(np.float32))
    rs = rng.uniform(0.5, 1.5, m_cap).astype(np.float32)
    kw = dict(act="swiglu", alpha=1.702, gate_lo=-3.0, gate_hi=3.0, up_lo=-3.0, up_hi=3.0)
    plain = _dglu_grads(G, dy2, w2, pre, counts, m_cap, kw, rs=rs, grads=False)
    out = _dglu_grads(G, dy2, w2, pre, counts, m_cap, kw, rs=rs)
    assert np.array_equal(out["dgu"], plain["dgu"])
    ep = O.Epilogue(row_scale=rs, **kw)
    ref = O.dgrad_dglu(dy2[:M], counts, w2, pre[:M], ep)
    assert_bf16_close(out["dgu"][:M], ref, what="dgu")
    # d(bias): the GPU's own dgu summed (fp32 order only), then the oracle's
    own = F.bf16_bits_to_f64(out["dgu"][:M])
    off = np.concatenate([[0], np.cumsum(counts)])
    for e in range(E):
        blk = own[off[e]:off[e + 1]]
        s_abs = np.abs(blk).sum(axis=0)
        assert np.all(np.abs(out["db"][e] - blk.sum(axis=0)) <= len(blk) * 2.0 ** -24 * s_abs + 1e-30)
    tol = np.zeros_like(out["db"])
    refv = F.bf16_bits_to_f64(ref)
    for e in range(E):
        tol[e] = np.sum(2e-2 * (1.0 + np.abs(refv[off[e]:off[e + 1]])), axis=0)
    assert np.all(np.abs(out["db"] - O.bias_grad(ref, counts)) <= tol)
    # d(row_scale) against the oracle
    want = O.row_scale_grad(dy2[:M], counts, w2, pre[:M], ep)
    Gm = np.concatenate([F.bf16_bits_to_f64(dy2[off[e]:off[e + 1]]) @ F.bf16_bits_to_f64(w2[e]).T
                         for e in range(E)])
    yu = O.glu_from_preact(F.bf16_bits_to_f64(pre[:M]), O.Epilogue(**kw))
    bound = 1e-4 * np.sum(np.abs(Gm * yu), axis=1) + 1e-6
    err = np.abs(out["drs"][:M] - want)
    assert np.all(err <= bound), (np.argmax(err - bound), err.max())
    assert np.all(out["drs"][M:] == 12345.0)
