"""The non-gated form (gated = 0): FC1 writes y = a(x W1 + b) * rs over I
columns from W1 [E][H][I] packed by moe_pack_weight, optionally with the
pre-activation, the MXFP8 copies of y and max|y|; the backward writes
dz = G * rs * a'(z) from the saved z.  Against the oracle within the bf16
tolerance; bit for bit on ternary sReLU data (every value a small integer)."""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O
from tests.gpu_util import (BF16_NAN_SENTINEL, assert_bf16_close, assert_mx_cols, assert_mx_rows,
                            dev_bits, dev_i32, empty_bits, empty_bytes, host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_glu_amd as G
    G.moe_init(0)
    return G


def _fwd(G, x, counts, w1, m_cap, act, bias=None, rs=None, mx=False):
    import torch
    E, H, I = w1.shape
    d_w1 = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))
    G.moe_pack_weight(dev_bits(w1), E, I, H, G.B_KN, d_w1)
    y, pre = empty_bits((m_cap, I)), empty_bits((m_cap, I))
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    d_rs = torch.from_numpy(rs).cuda() if rs is not None else None
    ep = G.epilogue(act, gated=False, bias=dev_bits(bias) if bias is not None else None,
                    row_scale=d_rs, amax_out=amax)
    bufs = None
    if mx:
        bufs = dict(row_q=empty_bytes((m_cap, I)), row_s=empty_bytes((m_cap, I // 32)),
                    col_q=empty_bytes((I, m_cap)), col_s=empty_bytes((I, (m_cap + 31) // 32 + E)))
    G.moe_group_gemm_glu_fwd(dev_bits(x), G.groups(dev_i32(counts), m_cap), d_w1, H, I, ep, y, pre,
                             G.mx_out(**bufs) if mx else None)
    torch.cuda.synchronize()
    out = dict(y=host_bits(y), pre=host_bits(pre), amax=float(amax.item()))
    if mx:
        out.update({k: v.cpu().numpy() for k, v in bufs.items()})
    return out


def _bwd(G, dy2, w2, pre, counts, m_cap, act, rs=None, signs=None):
    import torch
    E, I, H = w2.shape
    d_w2 = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))
    G.moe_pack_weight(dev_bits(w2), E, I, H, G.B_NK, d_w2)
    dz = empty_bits((m_cap, I))
    amax = torch.zeros(1, dtype=torch.float32, device="cuda") if signs is not None else None
    d_rs = torch.from_numpy(rs).cuda() if rs is not None else None
    ep = G.epilogue(act, gated=False, row_scale=d_rs, amax_out=amax, rht_signs=signs or 0)
    G.moe_group_gemm_dglu_bwd(dev_bits(dy2), G.operand(d_w2, layout=G.B_PACKED), H, I,
                              G.groups(dev_i32(counts), m_cap), dev_bits(pre), ep, dz, None)
    torch.cuda.synchronize()
    return host_bits(dz), (None if amax is None else float(amax.item()))


@pytest.mark.parametrize("act", ["srelu", "swiglu"])
def test_non_gated_fc1(G, act):
    counts = np.array([300, 0, 1, 257, 64])
    E, H, I = len(counts), 128, 320
    M = int(counts.sum())
    m_cap = M + 13
    rng = np.random.default_rng(91)
    x = W.to_bf16_bits(rng.standard_normal((m_cap, H)).astype(np.float32))
    w1 = W.to_bf16_bits((rng.standard_normal((E, H, I)) * 0.1).astype(np.float32))
    b1 = W.to_bf16_bits((rng.standard_normal((E, I)) * 0.2).astype(np.float32))
    rs = rng.uniform(0.5, 1.5, m_cap).astype(np.float32)
    out = _fwd(G, x, counts, w1, m_cap, act, bias=b1, rs=rs, mx=True)
    rp, ry = O.fc1_glu(x[:M], counts, w1, O.Epilogue(act=act, gated=False, bias=b1, row_scale=rs))
    assert_bf16_close(out["pre"][:M], rp, what="pre")
    assert_bf16_close(out["y"][:M], ry, what="y")
    assert np.all(out["y"][M:] == BF16_NAN_SENTINEL) and np.all(out["pre"][M:] == BF16_NAN_SENTINEL)
    assert out["amax"] == np.float32(np.max(np.abs(F.bf16_bits_to_f64(out["y"][:M]))))
    assert_mx_rows(out["row_q"][:M], out["row_s"][:M], out["y"][:M], ry, "y mx rows")
    assert_mx_cols(out["col_q"], out["col_s"], out["y"][:M], ry, counts, m_cap, "y mx cols")


def test_non_gated_srelu_integer_exact(G):
    counts = np.array([40, 0, 300, 17])
    E, H, I = len(counts), 64, 192
    M = int(counts.sum())
    m_cap = M + 5
    x = W.ternary_bf16(92, (m_cap, H))
    w1 = W.ternary_bf16(93, (E, H, I), density=0.25)
    out = _fwd(G, x, counts, w1, m_cap, "srelu")
    rp, ry = O.fc1_glu(x[:M], counts, w1, O.Epilogue(act="srelu", gated=False))
    assert np.array_equal(out["pre"][:M], rp) and np.array_equal(out["y"][:M], ry)
    dy2 = W.ternary_bf16(94, (m_cap, H))
    w2 = W.ternary_bf16(95, (E, I, H))
    pre = W.ternary_bf16(96, (m_cap, I))
    dz, _ = _bwd(G, dy2, w2, pre, counts, m_cap, "srelu")
    assert np.array_equal(dz[:M], O.dgrad_dact(dy2[:M], counts, w2, pre[:M], O.Epilogue(act="srelu")))
    assert np.all(dz[M:] == BF16_NAN_SENTINEL)


@pytest.mark.parametrize("act", ["srelu", "geglu"])
def test_non_gated_backward(G, act):
    counts = np.array([64, 0, 300, 1, 270])
    E, H, I = len(counts), 256, 320
    M = int(counts.sum())
    m_cap = M + 9
    rng = np.random.default_rng(97)
    dy2 = W.to_bf16_bits((rng.standard_normal((m_cap, H)) * 0.1).astype(np.float32))
    w2 = W.to_bf16_bits((rng.standard_normal((E, I, H)) * 0.05).astype(np.float32))
    pre = W.to_bf16_bits((rng.standard_normal((m_cap, I)) * 2).astype(np.float32))
    rs = rng.uniform(0.5, 1.5, m_cap).astype(np.float32)
    dz, amax = _bwd(G, dy2, w2, pre, counts, m_cap, act, rs=rs, signs=0x1234)
    ref = O.dgrad_dact(dy2[:M], counts, w2, pre[:M], O.Epilogue(act=act, row_scale=rs))
    assert_bf16_close(dz[:M], ref, what="dz", normwise=2e-2)
    want = O.rht16_amax(ref, counts, 0x1234)
    tol = 4 * 2e-2 * (1.0 + float(np.max(np.abs(F.bf16_bits_to_f64(ref)))))
    assert abs(amax - want) <= tol, (amax, want)
