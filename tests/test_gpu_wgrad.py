"""GPU parity of the weight-gradient K-grouped GroupGemm (dW1 = Xg^T dgu,
dW2 = y^T dY2) against the oracle, through the C ABI.

Tolerance: the products of bf16 values are exact in fp32, so the only error
is fp32 summation over a group's m_e rows, bounded by m_e * 2^-24 *
sum_k |a_k b_k| (recursive summation); a normwise relative error <= 1e-5 is
asserted as well.  On ternary inputs every partial sum is a small integer and
the result is compared bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from oracle import moe as O
from tests.gpu_util import dev_bits, dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_glu_amd as G
    G.moe_init(0)
    return G


def _wgrad_gpu(G, a, b, counts, m_cap, init=None, accumulate=False):
    import torch
    E, P, Q = len(counts), a.shape[1], b.shape[1]
    if init is None:
        c = torch.full((E, P, Q), float("nan"), dtype=torch.float32, device="cuda")
    else:
        c = torch.from_numpy(init.astype(np.float32)).cuda()
    G.moe_group_gemm_wgrad(dev_bits(a), dev_bits(b), P, Q, G.groups(dev_i32(counts), m_cap), c,
                           accumulate)
    torch.cuda.synchronize()
    return c.cpu().numpy().astype(np.float64)


def _assert_wgrad_close(got, a, b, counts, what):
    ref = O.wgrad(a, counts, b)
    bound = max(int(np.max(counts)), 1) * 2.0 ** -24 * O.wgrad_abs(a, counts, b)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    bad = err > bound + 1e-30
    assert not np.any(bad), f"{what}: {bad.sum()} elements out of bound, e.g. {np.argwhere(bad)[:3]}"
    nr = np.linalg.norm(ref)
    if nr > 0:
        assert np.linalg.norm(got - ref) / nr <= 1e-5, what


@pytest.mark.parametrize("counts,P,Q", [([129, 0, 400, 3, 256], 192, 320),
                                        ([700], 256, 256),
                                        ([0, 65, 0, 64, 63], 64, 448)])
def test_wgrad_ragged(G, counts, P, Q):
    counts = np.array(counts)
    M = int(counts.sum())
    m_cap = M + 5
    rng = np.random.default_rng(P + Q + M)
    a = W.to_bf16_bits(rng.standard_normal((m_cap, P)).astype(np.float32))
    b = W.to_bf16_bits((rng.standard_normal((m_cap, Q)) * 0.1).astype(np.float32))
    got = _wgrad_gpu(G, a, b, counts, m_cap)
    _assert_wgrad_close(got, a[:M], b[:M], counts, "wgrad")
    for e in np.nonzero(counts == 0)[0]:
        assert np.all(got[e] == 0.0)


def test_wgrad_integer_exact(G):
    counts = np.array([300, 17, 0, 260])
    M, P, Q = int(counts.sum()), 128, 192
    a = W.ternary_bf16(5, (M, P))
    b = W.ternary_bf16(6, (M, Q))
    got = _wgrad_gpu(G, a, b, counts, M)
    assert np.array_equal(got, O.wgrad(a, counts, b))


def test_wgrad_accumulate(G):
    counts = np.array([90, 0, 170])
    M, P, Q = int(counts.sum()), 128, 128
    rng = np.random.default_rng(7)
    a = W.ternary_bf16(8, (M, P))
    b = W.ternary_bf16(9, (M, Q))
    init = rng.integers(-50, 50, size=(3, P, Q)).astype(np.float64)
    got = _wgrad_gpu(G, a, b, counts, M, init=init, accumulate=True)
    assert np.array_equal(got, init + O.wgrad(a, counts, b))


def test_wgrads_of_the_expert_mlp(G):
    """dW1 and dW2 of a routed step from the oracle's own forward and dGLU."""
    counts = np.array([200, 0, 57, 300])
    E, H, I = 4, 128, 256
    d = W.small_grouped(33, counts, H, I)
    M = d["M"]
    pre, y = O.fc1_glu(d["x"], counts, d["w1"], O.Epilogue())
    dy2 = W.to_bf16_bits((np.random.default_rng(3).standard_normal((M, H)) * 0.05).astype(np.float32))
    dgu = O.dgrad_dglu(dy2, counts, d["w2"], pre, O.Epilogue())
    dW1 = _wgrad_gpu(G, d["x"], dgu, counts, M)
    _assert_wgrad_close(dW1, d["x"], dgu, counts, "dW1")
    assert dW1.shape == d["w1"].shape
    dW2 = _wgrad_gpu(G, y, dy2, counts, M)
    _assert_wgrad_close(dW2, y, dy2, counts, "dW2")
    assert dW2.shape == d["w2"].shape
