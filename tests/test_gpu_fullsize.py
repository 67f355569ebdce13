"""Parity at the full workload sizes, in the launch configuration bench.py
times, on sampled rows the oracle computes one by one (every output row of a
grouped GEMM depends only on its own input row and its expert's weights).

Workloads: DeepSeek-V3-like expert share (FC1+SwiGLU, FC2, dgrad+dSwiGLU, dX),
GPT-OSS-like FC1 (routing, alpha 1.702, clamp 7, bias, empty and hot experts).
"""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O
from tests.gpu_util import (assert_bf16_close, dev_bits, dev_i32, empty_bits, expert_of_rows,
                            host_bits, sample_rows)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


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


@pytest.fixture(scope="module")
def dsv3_run(G):
    """One full step of the DeepSeek-V3-like share on the GPU, as bench.py runs it."""
    import torch
    d = W.dsv3(with_w2=True)
    dy2_h = W.dsv3_dy2()
    E, M, H, I = d["E"], d["M"], d["H"], d["I"]
    counts = d["counts"]
    x, w1, w2, dy2 = dev_bits(d["x"]), dev_bits(d["w1"]), dev_bits(d["w2"]), dev_bits(dy2_h)
    cnt = dev_i32(counts)
    off = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
    w1p = empty_bits((G.moe_packed_w1_bytes(E, H, I) // 2,))
    G.moe_repack_gate_up(w1, E, H, I, w1p)
    w1x = empty_bits((G.moe_packed_weight_bytes(E, H, 2 * I) // 2,))   # dX: N = H, K = 2I
    G.moe_pack_weight(w1, E, H, 2 * I, G.B_NK, w1x)
    w2f = empty_bits((G.moe_packed_weight_bytes(E, H, I) // 2,))       # FC2: N = H, K = I
    G.moe_pack_weight(w2, E, H, I, G.B_KN, w2f)
    w2d = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))       # dgrad: N = I, K = H
    G.moe_pack_weight(w2, E, I, H, G.B_NK, w2d)
    y, pre = empty_bits((M, I)), empty_bits((M, 2 * I))
    out2, dgu, dx = empty_bits((M, H)), empty_bits((M, 2 * I)), empty_bits((M, H))
    grp = G.groups(cnt, M, off)
    ep = G.epilogue("swiglu")
    G.moe_group_gemm_glu_fwd(x, grp, w1p, H, I, ep, y, pre)
    G.moe_group_gemm_quant(G.operand(y), G.operand(w2f, layout=G.B_PACKED), H, I, grp, out2)
    G.moe_group_gemm_dglu_bwd(dy2, G.operand(w2d, layout=G.B_PACKED), H, I, grp, pre, ep, dgu)
    G.moe_group_gemm_quant(G.operand(dgu), G.operand(w1x, layout=G.B_PACKED), H, 2 * I, grp, dx)
    _sync()
    res = dict(d=d, dy2=dy2_h, off=off.cpu().numpy(), y=host_bits(y), pre=host_bits(pre),
               out2=host_bits(out2), dgu=host_bits(dgu), dx=host_bits(dx))
    del x, w1, w2, dy2, w1p, w1x, w2f, w2d
    return res


def test_dsv3_offsets_bit_exact(dsv3_run):
    c = dsv3_run["d"]["counts"]
    assert np.array_equal(dsv3_run["off"], O.exclusive_offsets(c).astype(np.int32))


def test_dsv3_fc1_glu_sampled_rows(dsv3_run):
    d = dsv3_run["d"]
    counts, I = d["counts"], d["I"]
    rows = sample_rows(counts, per_group=2, seed=1)
    experts = expert_of_rows(counts, rows)
    ep = O.Epilogue()
    for e in np.unique(experts):
        rr = rows[experts == e]
        pre, y = O.fc1_glu(d["x"][rr], [len(rr)], d["w1"][e:e + 1], ep)
        assert_bf16_close(dsv3_run["y"][rr], y, what=f"dsv3 y expert {e}")
        assert_bf16_close(dsv3_run["pre"][rr], pre, what=f"dsv3 preact expert {e}")


def test_dsv3_fc2_sampled_rows(dsv3_run):
    d = dsv3_run["d"]
    counts = d["counts"]
    rows = sample_rows(counts, per_group=1, seed=2)
    experts = expert_of_rows(counts, rows)
    for e in np.unique(experts):
        rr = rows[experts == e]
        _, y_r = O.fc1_glu(d["x"][rr], [len(rr)], d["w1"][e:e + 1], O.Epilogue())
        ref = O.group_gemm(y_r, [len(rr)], d["w2"][e:e + 1])
        assert_bf16_close(dsv3_run["out2"][rr], ref, what=f"dsv3 fc2 expert {e}")


def test_dsv3_dgrad_dglu_sampled_rows(dsv3_run):
    d = dsv3_run["d"]
    counts = d["counts"]
    rows = sample_rows(counts, per_group=1, seed=3)
    experts = expert_of_rows(counts, rows)
    for e in np.unique(experts):
        rr = rows[experts == e]
        pre_r, _ = O.fc1_glu(d["x"][rr], [len(rr)], d["w1"][e:e + 1], O.Epilogue())
        ref = O.dgrad_dglu(dsv3_run["dy2"][rr], [len(rr)], d["w2"][e:e + 1], pre_r, O.Epilogue())
        assert_bf16_close(dsv3_run["dgu"][rr], ref, what=f"dsv3 dgu expert {e}", normwise=2e-2)


def test_dsv3_dx_sampled_rows(dsv3_run):
    d = dsv3_run["d"]
    counts = d["counts"]
    rows = sample_rows(counts, per_group=1, seed=4)
    experts = expert_of_rows(counts, rows)
    for e in np.unique(experts):
        rr = rows[experts == e]
        pre_r, _ = O.fc1_glu(d["x"][rr], [len(rr)], d["w1"][e:e + 1], O.Epilogue())
        dgu_r = O.dgrad_dglu(dsv3_run["dy2"][rr], [len(rr)], d["w2"][e:e + 1], pre_r, O.Epilogue())
        ref = O.dx(dgu_r, [len(rr)], d["w1"][e:e + 1])
        assert_bf16_close(dsv3_run["dx"][rr], ref, what=f"dsv3 dx expert {e}", normwise=2e-2)


def test_gptoss_route_and_fc1_sampled_rows(G):
    import torch
    d = W.gptoss(with_weights=True)
    T, E, k, H, I = d["T"], d["E"], d["k"], d["H"], d["I"]
    lim, alpha = d["limit"], d["alpha"]
    TK = T * k
    logits = torch.from_numpy(d["logits"]).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    dst = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src = torch.empty(TK, dtype=torch.int32, device="cuda")
    x = dev_bits(d["x"])
    xg = empty_bits((TK, H))
    G.moe_route_group(logits, None, T, E, k, ids, cnt, off, dst, src, x, H, xg)
    w1p = empty_bits((G.moe_packed_w1_bytes(E, H, I) // 2,))
    G.moe_repack_gate_up(dev_bits(d["w1"]), E, H, I, w1p)
    b1 = dev_bits(d["b1"])
    y, pre = empty_bits((TK, I)), empty_bits((TK, 2 * I))
    ep = G.epilogue("swiglu", alpha=alpha, gate_lo=-lim, gate_hi=lim, up_lo=-lim, up_hi=lim,
                    bias=b1)
    G.moe_group_gemm_glu_fwd(xg, G.groups(cnt, TK), w1p, H, I, ep, y, pre)
    _sync()
    _, rc, roff, rdst, rsrc = O.route_topk(d["logits"], k)
    assert np.array_equal(cnt.cpu().numpy(), rc) and np.array_equal(src.cpu().numpy(), rsrc)
    assert rc[0] == 0 and rc.max() > 2 * TK / E
    gy, gpre = host_bits(y), host_bits(pre)
    rows = sample_rows(rc, per_group=2, seed=5)
    experts = expert_of_rows(rc, rows)
    ep_o = O.Epilogue(alpha=alpha, gate_lo=-lim, gate_hi=lim, up_lo=-lim, up_hi=lim)
    for e in np.unique(experts):
        rr = rows[experts == e]
        ep_o.bias = d["b1"][e:e + 1]
        pre_r, y_r = O.fc1_glu(d["x"][rsrc[rr]], [len(rr)], d["w1"][e:e + 1], ep_o)
        assert_bf16_close(gy[rr], y_r, what=f"gptoss y expert {e}")
        assert_bf16_close(gpre[rr], pre_r, what=f"gptoss preact expert {e}")
