"""The e5m2 option of the MXFP8 copies (the gradient format of an MXFP8
recipe) and the MXFP8 GroupGemm taking e5m2 activations (dgu x W1 for dX).

* Every finite bf16 value of magnitude <= vmax goes through the standalone
  quantiser in blocks whose amax is vmax (scale 2^0), for e5m2 (57344) and
  e4m3 (448): the codes must equal the oracle's byte for byte (this covers
  the hardware conversion of every representable input, subnormals and ties
  included).
* Random Student-t rows: row and column copies equal the oracle's bytes.
* MXFP8 GroupGemm with e5m2 A and e4m3 packed W: within the MXFP8 tolerance
  of the oracle's dequantise-then-multiply (A quantised by the oracle).
* dgrad + dGLU writing e5m2 copies of dgu: checked like the e4m3 ones.
"""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O
from tests.gpu_util import (BF16_NAN_SENTINEL, assert_bf16_close, assert_mx_cols, assert_mx_gemm_close,
                            assert_mx_rows, dev_bits, dev_bytes, dev_i32, empty_bits, empty_bytes,
                            host_bits)
from tests.test_gpu_mxfp8 import _oracle_weight_mx, _pack_mx_gpu, _weight_nk

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


def _all_bf16_upto(vmax):
    b = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)     # every finite positive bf16
    v = F.bf16_bits_to_f64(b)
    b = b[v <= vmax]
    return np.concatenate([b, b | np.uint16(0x8000)])


@pytest.mark.parametrize("fmt,vmax", [("e5m2", 57344.0), ("e4m3", 448.0)])
def test_quantize_every_bf16_value(G, fmt, vmax):
    vals = _all_bf16_upto(vmax)
    n = len(vals)
    R = (n + 30) // 31
    blk = np.zeros((R, 32), dtype=np.uint16)
    blk[:, 0] = F.f64_to_bf16_bits(np.array([vmax]))[0]
    flat = np.zeros(R * 31, dtype=np.uint16)
    flat[:n] = vals
    blk[:, 1:] = flat.reshape(R, 31)
    bufs = dict(row_q=empty_bytes((R, 32)), row_s=empty_bytes((R, 1)))
    G.moe_mxfp8_quantize(dev_bits(blk), R, 32, None, G.mx_out(**bufs, e5m2=(fmt == "e5m2")))
    _sync()
    q, s = O.mx_quantize_rows(blk, fmt)
    assert np.all(s == 127)
    gq = bufs["row_q"].cpu().numpy()
    bad = np.argwhere(gq != q)
    assert bad.size == 0, [(int(blk[r, c]), int(gq[r, c]), int(q[r, c])) for r, c in bad[:5]]
    assert np.array_equal(bufs["row_s"].cpu().numpy(), s)


def test_quantize_e5m2_rows_and_cols(G):
    rng = np.random.default_rng(61)
    R, C = 77, 96
    v = W.to_bf16_bits((rng.standard_t(3, size=(R, C)) * np.exp2(rng.integers(-30, 30, (R, 1))))
                       .astype(np.float32))
    bufs = dict(row_q=empty_bytes((R, C)), row_s=empty_bytes((R, C // 32)),
                col_q=empty_bytes((C, R)), col_s=empty_bytes((C, (R + 31) // 32)))
    G.moe_mxfp8_quantize(dev_bits(v), R, C, None, G.mx_out(**bufs, e5m2=True))
    _sync()
    q, s = O.mx_quantize_rows(v, "e5m2")
    assert np.array_equal(bufs["row_q"].cpu().numpy(), q)
    assert np.array_equal(bufs["row_s"].cpu().numpy(), s)
    cq, cs = O.mx_quantize_cols(v, [R], m_cap=R, fmt="e5m2")
    assert np.array_equal(bufs["col_q"].cpu().numpy(), cq)
    assert np.array_equal(bufs["col_s"].cpu().numpy(), cs[:, :(R + 31) // 32])


@pytest.mark.parametrize("counts,K,N", [([300, 0, 213], 384, 320), ([5], 128, 64)])
def test_group_gemm_mx_e5m2_activations(G, counts, K, N):
    counts = np.array(counts)
    E, M = len(counts), int(counts.sum())
    m_cap = M + 7
    g = np.random.default_rng(K + N + 3)
    a = W.to_bf16_bits((g.standard_normal((m_cap, K)) * 1e-3).astype(np.float32))   # gradient-sized
    aq, as_ = O.mx_quantize_rows(a, "e5m2")
    w_nk = _weight_nk(K + N, E, N, K)
    d_q, d_s = _pack_mx_gpu(G, w_nk, "KN")
    c = empty_bits((m_cap, N))
    G.moe_group_gemm_quant(G.operand(dev_bytes(aq), dtype=G.DT_MXFP8_E5M2, scales=dev_bytes(as_)),
                           G.operand(d_q, dtype=G.DT_MXFP8, layout=G.B_PACKED, scales=d_s), N, K,
                           G.groups(dev_i32(counts), m_cap), c)
    _sync()
    out = host_bits(c)
    bq, bs = _oracle_weight_mx(w_nk)
    ref = O.group_gemm_mx(aq[:M], as_[:M], counts, bq, bs, a_fmt="e5m2")
    assert_mx_gemm_close(out[:M], ref, aq[:M], as_[:M], counts, bq, bs, "group_gemm_mx e5m2",
                         a_fmt="e5m2", normwise=1e-2)
    assert np.all(out[M:] == BF16_NAN_SENTINEL)
    # the e4m3 reading of the same bytes is a different matrix: the format flag matters
    assert not np.array_equal(O.group_gemm_mx(aq[:M], as_[:M], counts, bq, bs), ref)


def test_dglu_e5m2_copies(G):
    counts = np.array([64, 0, 300, 1, 270])
    E, H, I = len(counts), 256, 320
    M = int(counts.sum())
    m_cap = M + 9
    rng = np.random.default_rng(62)
    dy2 = W.to_bf16_bits((rng.standard_normal((m_cap, H)) * 0.1).astype(np.float32))
    w2 = W.to_bf16_bits((rng.standard_normal((E, I, H)) * 0.05).astype(np.float32))
    pre = W.to_bf16_bits((rng.standard_normal((m_cap, 2 * I)) * 2).astype(np.float32))
    d_w2p = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))
    G.moe_pack_weight(dev_bits(w2), E, I, H, G.B_NK, d_w2p)
    dgu = empty_bits((m_cap, 2 * I))
    bufs = dict(row_q=empty_bytes((m_cap, 2 * I)), row_s=empty_bytes((m_cap, 2 * I // 32)),
                col_q=empty_bytes((2 * I, m_cap)), col_s=empty_bytes((2 * I, (m_cap + 31) // 32 + E)))
    G.moe_group_gemm_dglu_bwd(dev_bits(dy2), G.operand(d_w2p, layout=G.B_PACKED), H, I,
                              G.groups(dev_i32(counts), m_cap), dev_bits(pre), G.epilogue("swiglu"),
                              dgu, G.mx_out(**bufs, e5m2=True))
    _sync()
    got = host_bits(dgu)
    ref = O.dgrad_dglu(dy2[:M], counts, w2, pre[:M], O.Epilogue())
    assert_bf16_close(got[:M], ref, what="dgu", normwise=2e-2)
    assert_mx_rows(bufs["row_q"].cpu().numpy()[:M], bufs["row_s"].cpu().numpy()[:M], got[:M], ref,
                   "dgu e5m2 rows", fmt="e5m2")
    assert_mx_cols(bufs["col_q"].cpu().numpy(), bufs["col_s"].cpu().numpy(), got[:M], ref, counts,
                   m_cap, "dgu e5m2 cols", fmt="e5m2")
