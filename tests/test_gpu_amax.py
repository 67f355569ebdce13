"""Per-tensor amax of the FC1 output, emitted by the GLU epilogue ([BLOG]
"Fusionando cuantización MXFP8 y NVFP4": the NVFP4 forward writes the bf16
output and its per-tensor amax).  The GPU value must equal the maximum |y|
of the bf16 values the same call stored (bit for bit: both are maxima of the
same bf16 numbers) and agree with the oracle's amax of its own y within the
bf16 output tolerance.  Rows past the routed ones (which a bias would make
non-zero if they were counted) must not contribute.
"""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O
from tests.gpu_util import assert_bf16_close, dev_bits, dev_i32, empty_bits, host_bits
from tests.test_gpu_parity import _check_fc1, _fc1_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_glu_amd as G
    G.moe_init(0)
    return G


def _own_amax(y_bits, M):
    v = np.abs(F.bf16_bits_to_f64(y_bits[:M]))
    return float(v.max()) if v.size else 0.0


def _check_amax(got, y_gpu, ry, counts, what):
    M = int(np.sum(counts))
    assert got == np.float32(_own_amax(y_gpu, M)), f"{what}: amax {got} != max|y| {_own_amax(y_gpu, M)}"
    ref = O.tensor_amax(ry, counts)
    assert abs(got - ref) <= 2e-2 * (1.0 + ref), f"{what}: amax {got} vs oracle {ref}"


@pytest.mark.parametrize("mx", [False, True])
def test_fc1_amax_ragged_with_bias_and_padding(G, mx):
    counts = np.array([300, 0, 1, 257, 64])
    E, H, I = len(counts), 128, 320
    M = int(counts.sum())
    m_cap = M + 41
    d = W.small_grouped(61, counts, H, I, bias=True, m_cap=m_cap)
    rs = np.random.default_rng(4).uniform(0.5, 1.5, m_cap).astype(np.float32)
    kw = dict(alpha=1.702, gate_lo=-7.0, gate_hi=7.0, up_lo=-7.0, up_hi=7.0)
    out = _fc1_gpu(G, d["x"], counts, d["w1"], I, kw, m_cap=m_cap, bias=d["b1"], row_scale=rs,
                   mx=mx, amax_init=0.0)
    _, ry = _check_fc1(out, d["x"], counts, d["w1"], O.Epilogue(bias=d["b1"], row_scale=rs, **kw),
                       m_cap, "amax")
    _check_amax(out["amax"], out["y"], ry, counts, f"fc1 mx={mx}")


def test_fc1_amax_is_a_running_maximum(G):
    """The epilogue raises the value it finds: a larger prior value stays."""
    counts = np.array([200, 90])
    H, I = 128, 128
    d = W.small_grouped(62, counts, H, I)
    out = _fc1_gpu(G, d["x"], counts, d["w1"], I, {}, amax_init=1.0e6)
    assert out["amax"] == 1.0e6
    out = _fc1_gpu(G, d["x"], counts, d["w1"], I, {}, preact=False, amax_init=0.0)
    assert out["amax"] == np.float32(_own_amax(out["y"], 290)) and out["amax"] > 0.0


def test_fc1_amax_without_routed_rows(G):
    counts = np.zeros(3, dtype=np.int64)
    d = W.small_grouped(63, [1, 1, 1], 64, 64, bias=True, m_cap=40)
    out = _fc1_gpu(G, d["x"], counts, d["w1"], 64, {}, m_cap=40, bias=d["b1"], amax_init=0.0)
    assert out["amax"] == 0.0


def test_fc1_mx_inputs_amax(G):
    """moe_group_gemm_glu_fwd_mx (MXFP8 operands) emits the same amax of its y."""
    import torch
    from tests.test_gpu_mxfp8 import _fc1_mx_gpu
    counts = np.array([300, 0, 57, 260])
    E, H, I = 4, 256, 320
    M = int(counts.sum())
    m_cap = M + 9
    d = W.small_grouped(64, counts, H, I, m_cap=m_cap)
    aq, as_ = O.mx_quantize_rows(W.student_t_rows_bf16(64, m_cap, H))
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = _fc1_mx_gpu(G, aq, as_, counts, d["w1"], H, I, m_cap, G.epilogue(amax_out=amax))
    got = float(amax.item())
    assert got == np.float32(_own_amax(out["y"], M)) and got > 0.0


# ------------------------------------------------------------------ backward
def _dglu_gpu(G, dy2, w2, pre, counts, m_cap, ep_kw, amax_init=None, signs=0, rs=None):
    import torch
    E, I, H = w2.shape
    d_w2p = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))
    G.moe_pack_weight(dev_bits(w2), E, I, H, G.B_NK, d_w2p)
    dgu = empty_bits((m_cap, 2 * I))
    d_amax = None
    if amax_init is not None:
        d_amax = torch.full((1,), float(amax_init), dtype=torch.float32, device="cuda")
    d_rs = torch.from_numpy(rs).cuda() if rs is not None else None
    ep = G.epilogue(row_scale=d_rs, amax_out=d_amax, rht_signs=signs, **ep_kw)
    G.moe_group_gemm_dglu_bwd(dev_bits(dy2), G.operand(d_w2p, layout=G.B_PACKED), H, I,
                              G.groups(dev_i32(counts), m_cap), dev_bits(pre), ep, dgu, None)
    torch.cuda.synchronize()
    return host_bits(dgu), (None if d_amax is None else float(d_amax.item()))


@pytest.mark.parametrize("signs", [0, 0xA5C3])
def test_dglu_rht_amax_integer_exact(G, signs):
    """sReLU on ternary data: dgu is a small integer (exact in bf16) and every
    rotated value a multiple of 1/4, so the GPU amax must equal the oracle's
    bit for bit.  Ragged groups (partial runs), an empty group, and I = 192
    (a 64-column chunk of the tile past I)."""
    counts = np.array([40, 0, 300, 17])
    E, H, I = len(counts), 64, 192
    M = int(counts.sum())
    m_cap = M + 23
    dy2 = W.ternary_bf16(71, (m_cap, H))
    w2 = W.ternary_bf16(72, (E, I, H))
    pre = W.ternary_bf16(73, (m_cap, 2 * I))
    got, amax = _dglu_gpu(G, dy2, w2, pre, counts, m_cap, dict(act="srelu"), amax_init=0.0,
                          signs=signs)
    ref = O.dgrad_dglu(dy2[:M], counts, w2, pre[:M], O.Epilogue(act="srelu"))
    assert np.array_equal(got[:M], ref)
    want = O.rht16_amax(ref, counts, signs)
    assert want > 0 and amax == want, (amax, want)


def test_dglu_rht_amax_swiglu(G):
    """SwiGLU with row scales and random row signs: the amax agrees with the
    oracle's within the propagated bf16 tolerance (a rotated value moves by
    at most the sum of 16 element errors over 4), and asking for it leaves
    dgu unchanged."""
    counts = np.array([64, 0, 300, 1, 270])
    E, H, I = len(counts), 256, 320
    M = int(counts.sum())
    m_cap = M + 9
    rng = np.random.default_rng(74)
    dy2 = W.to_bf16_bits((rng.standard_normal((m_cap, H)) * 0.1).astype(np.float32))
    w2 = W.to_bf16_bits((rng.standard_normal((E, I, H)) * 0.05).astype(np.float32))
    pre = W.to_bf16_bits((rng.standard_normal((m_cap, 2 * I)) * 2).astype(np.float32))
    rs = rng.uniform(0.5, 1.5, m_cap).astype(np.float32)
    kw = dict(act="swiglu", alpha=1.702)
    plain, _ = _dglu_gpu(G, dy2, w2, pre, counts, m_cap, kw, rs=rs)
    got, amax = _dglu_gpu(G, dy2, w2, pre, counts, m_cap, kw, amax_init=0.0, signs=0x3C96, rs=rs)
    assert np.array_equal(got, plain)
    ref = O.dgrad_dglu(dy2[:M], counts, w2, pre[:M], O.Epilogue(row_scale=rs, **kw))
    assert_bf16_close(got[:M], ref, what="dgu")
    want = O.rht16_amax(ref, counts, 0x3C96)
    tol = 4 * 2e-2 * (1.0 + float(np.max(np.abs(F.bf16_bits_to_f64(ref)))))
    assert abs(amax - want) <= tol, (amax, want, tol)
