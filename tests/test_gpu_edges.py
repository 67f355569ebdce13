"""Edge cases of the grouped kernels against the oracle, through the C ABI:
every expert empty, one expert holding every row (the dense-MLP case), the
smallest supported sizes (a single K-tile, a single gate/up pair, a half
n-tile), many experts (up to the ABI's 1024) with mostly empty groups, and a
row capacity far above the routed rows.  Rows past the routed ones must stay
untouched (sentinels).
"""
import numpy as np
import pytest

import workloads as W
from oracle import moe as O
from tests.gpu_util import (BF16_NAN_SENTINEL, assert_bf16_close, dev_bits, dev_i32, empty_bits,
                            host_bits)
from tests.test_gpu_parity import _check_fc1, _fc1_gpu, _quant_gpu

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


def test_all_experts_empty(G):
    counts = np.zeros(5, dtype=np.int64)
    E, H, I, m_cap = 5, 128, 128, 300
    d = W.small_grouped(41, [1] * E, H, I, m_cap=m_cap)
    out = _fc1_gpu(G, d["x"], counts, d["w1"], I, {}, m_cap=m_cap, preact=True)
    assert out["off"].tolist() == [0] * (E + 1) and out["status"] == 0
    assert np.all(out["y"] == BF16_NAN_SENTINEL) and np.all(out["preact"] == BF16_NAN_SENTINEL)
    b = W.to_bf16_bits((np.random.default_rng(1).standard_normal((E, I, H)) * 0.05).astype(np.float32))
    q = _quant_gpu(G, d["x"][:, :I], counts, dev_bits(b), G.B_KN, H, I, m_cap)
    assert np.all(q["c"] == BF16_NAN_SENTINEL)


def test_single_expert_dense(G):
    """E = 1: the dense MLP as a one-group GroupGemm (FC1 + SwiGLU, then FC2)."""
    counts = np.array([700])
    H, I = 256, 384
    d = W.small_grouped(42, counts, H, I)
    out = _fc1_gpu(G, d["x"], counts, d["w1"], I, {}, preact=True)
    _, ry = _check_fc1(out, d["x"], counts, d["w1"], O.Epilogue(), 700, "dense")
    w2p = empty_bits((G.moe_packed_weight_bytes(1, H, I) // 2,))
    G.moe_pack_weight(dev_bits(d["w2"]), 1, H, I, G.B_KN, w2p)
    q = _quant_gpu(G, ry, counts, w2p, G.B_PACKED, H, I, 700)
    assert_bf16_close(q["c"], O.group_gemm(ry, counts, d["w2"]), what="dense fc2")


@pytest.mark.parametrize("H,I", [(64, 64), (64, 192), (128, 320)])
def test_fc1_smallest_sizes(G, H, I):
    """One K-tile (H = 64), one gate/up pair (I = 64: half of a 256-wide
    n-tile), and an odd pair count (I = 320) with bias and clamps."""
    counts = np.array([33, 0, 257])
    d = W.small_grouped(43, counts, H, I, bias=True, m_cap=300)
    kw = dict(alpha=1.702, gate_lo=-7.0, gate_hi=7.0, up_lo=-7.0, up_hi=7.0)
    out = _fc1_gpu(G, d["x"], counts, d["w1"], I, kw, bias=d["b1"], m_cap=300, preact=True)
    _check_fc1(out, d["x"], counts, d["w1"], O.Epilogue(bias=d["b1"], **kw), 300, f"H{H} I{I}")


@pytest.mark.parametrize("E", [256, 1024])
def test_many_experts_mostly_empty(G, E):
    """Many groups: most empty, a few ragged ones, the tile scan over all E."""
    rng = np.random.default_rng(E)
    counts = np.zeros(E, dtype=np.int64)
    hot = rng.choice(E, size=7, replace=False)
    counts[hot] = rng.integers(1, 300, size=7)
    counts[E - 1] = 5                               # the last expert is never skipped
    H, I = 64, 64
    M = int(counts.sum())
    d = W.small_grouped(44, [1] * E, H, I, m_cap=M + 11)
    out = _fc1_gpu(G, d["x"], counts, d["w1"], I, {}, m_cap=M + 11, preact=True)
    _check_fc1(out, d["x"], counts, d["w1"], O.Epilogue(), M + 11, f"E{E}")


def test_capacity_far_above_rows(G):
    """M_cap = 4096 with 200 routed rows: the grid and scan are sized by the
    capacity, the work by the device counts."""
    counts = np.array([120, 80])
    H, I, m_cap = 128, 128, 4096
    d = W.small_grouped(45, counts, H, I, m_cap=m_cap)
    out = _fc1_gpu(G, d["x"], counts, d["w1"], I, {}, m_cap=m_cap, preact=True)
    _check_fc1(out, d["x"], counts, d["w1"], O.Epilogue(), m_cap, "capacity")


def test_quant_minimum_and_half_tile(G):
    """N = 64 (a quarter n-tile) and N = 320 (1.25 n-tiles) with K = 64."""
    counts = np.array([70, 0, 190])
    for N in (64, 320):
        K = 64
        M = int(counts.sum())
        rng = np.random.default_rng(N)
        a = W.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        b = W.to_bf16_bits((rng.standard_normal((3, K, N)) * 0.05).astype(np.float32))
        bp = empty_bits((G.moe_packed_weight_bytes(3, N, K) // 2,))
        G.moe_pack_weight(dev_bits(b), 3, N, K, G.B_KN, bp)
        q = _quant_gpu(G, a, counts, bp, G.B_PACKED, N, K, M)
        assert_bf16_close(q["c"], O.group_gemm(a, counts, b), what=f"quant N{N}")


@pytest.mark.parametrize("margin", [100, 250])
def test_cu_margin_leaves_results_unchanged(G, margin):
    """Fewer persistent workgroups (CUs left to concurrent kernels; with 100
    the grid is no longer a multiple of the 8 XCDs) compute the same bits."""
    counts = np.array([300, 0, 77, 512])
    H, I = 64, 2560        # 20 n-tiles: enough tiles for a grid of 156 (margin 100) or 6
    d = W.small_grouped(46, counts, H, I)
    ref = _fc1_gpu(G, d["x"], counts, d["w1"], I, {}, preact=True)
    got = _fc1_gpu(G, d["x"], counts, d["w1"], I, {}, preact=True, cu_margin=margin)
    assert np.array_equal(got["y"], ref["y"]) and np.array_equal(got["preact"], ref["preact"])


@pytest.mark.parametrize("E,I", [(1024, 64), (48, 320)])
def test_dglu_many_short_groups(G, E, I):
    """dgrad + dSwiGLU with many groups whose last m-tile holds at most 128
    rows (run as 128 x 128 quarter tiles, one per 128 columns of I: with
    I = 64 one quarter per group, with I = 320 three, the last one a column
    half past I), against the oracle; then with fewer workgroups (a grid that
    is not a multiple of the 8 XCDs), which must give the same bits."""
    rng = np.random.default_rng(E + I)
    counts = np.zeros(E, dtype=np.int64)
    hot = rng.choice(E, size=min(E, 40), replace=False)
    counts[hot] = rng.integers(1, 420, size=len(hot))
    counts[E - 1] = 128                             # exactly a short tile's rows
    H = 128
    M = int(counts.sum())
    m_cap = M + 5
    dy2 = W.to_bf16_bits((rng.standard_normal((m_cap, H)) * 0.1).astype(np.float32))
    w2 = W.to_bf16_bits((rng.standard_normal((E, I, H)) * 0.05).astype(np.float32))
    pre = W.to_bf16_bits((rng.standard_normal((m_cap, 2 * I)) * 2).astype(np.float32))
    w2p = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))
    G.moe_pack_weight(dev_bits(w2), E, I, H, G.B_NK, w2p)
    op = G.operand(w2p, layout=G.B_PACKED)
    grp = G.groups(dev_i32(counts), m_cap)
    outs = []
    for margin in (0, 100):
        dgu = empty_bits((m_cap, 2 * I))
        G.moe_group_gemm_dglu_bwd(dev_bits(dy2), op, H, I, grp, dev_bits(pre),
                                  G.epilogue("swiglu", alpha=1.702), dgu, cu_margin=margin)
        _sync()
        outs.append(host_bits(dgu))
    ref = O.dgrad_dglu(dy2[:M], counts, w2, pre[:M], O.Epilogue(act="swiglu", alpha=1.702))
    assert_bf16_close(outs[0][:M], ref, what=f"dgu E{E} I{I}", normwise=2e-2)
    assert np.all(outs[0][M:] == BF16_NAN_SENTINEL)
    assert np.array_equal(outs[0], outs[1])
