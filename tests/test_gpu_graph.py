"""Sync-free property: the whole step (routing, FC1 + GLU, FC2, dgrad + dGLU,
dX) is captured once as a hipGraph and replayed with NEW routings written into
the same device buffers, without re-capture and without any host readback
("Boosting MoE Training Throughput with Advanced Fusion Kernels", section
"Eliminando la sincronización host-device").  Every replay is checked against
the oracle for the routing it ran with.
"""
import numpy as np
import pytest

import workloads as W
from oracle import moe as O
from tests.gpu_util import assert_bf16_close, dev_bits, empty_bits, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_glu_amd as G
    G.moe_init(0)
    return G


def test_full_step_graph_replay_with_new_routing(G):
    import torch
    T, E, k, H, I = 300, 6, 2, 192, 128
    TK = T * k
    rng = np.random.default_rng(77)
    x_h = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w1_h = W.to_bf16_bits((rng.standard_normal((E, H, 2 * I)) * 0.05).astype(np.float32))
    w2_h = W.to_bf16_bits((rng.standard_normal((E, I, H)) * 0.05).astype(np.float32))
    dy2_h = W.to_bf16_bits((rng.standard_normal((TK, H)) * 0.05).astype(np.float32))

    logits = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    x, w1, w2, dy2 = dev_bits(x_h), dev_bits(w1_h), dev_bits(w2_h), dev_bits(dy2_h)
    w1p = empty_bits((G.moe_packed_w1_bytes(E, H, I) // 2,))
    G.moe_repack_gate_up(w1, E, H, I, w1p)
    w1x = empty_bits((G.moe_packed_weight_bytes(E, H, 2 * I) // 2,))
    G.moe_pack_weight(w1, E, H, 2 * I, G.B_NK, w1x)
    w2f = empty_bits((G.moe_packed_weight_bytes(E, H, I) // 2,))
    G.moe_pack_weight(w2, E, H, I, G.B_KN, w2f)
    w2d = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))
    G.moe_pack_weight(w2, E, I, H, G.B_NK, w2d)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    dst = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src = torch.empty(TK, dtype=torch.int32, device="cuda")
    xg = empty_bits((TK, H))
    y, pre = empty_bits((TK, I)), empty_bits((TK, 2 * I))
    out2, dgu, dx = empty_bits((TK, H)), empty_bits((TK, 2 * I)), empty_bits((TK, H))
    grp = G.groups(cnt, TK)
    ep = G.epilogue("swiglu")
    op_y, op_w2 = G.operand(y), G.operand(w2f, layout=G.B_PACKED)
    op_dgu, op_w1x = G.operand(dgu), G.operand(w1x, layout=G.B_PACKED)
    op_w2d = G.operand(w2d, layout=G.B_PACKED)

    def step():
        G.moe_route_group(logits, None, T, E, k, ids, cnt, off, dst, src, x, H, xg)
        G.moe_group_gemm_glu_fwd(xg, grp, w1p, H, I, ep, y, pre)
        G.moe_group_gemm_quant(op_y, op_w2, H, I, grp, out2)
        G.moe_group_gemm_dglu_bwd(dy2, op_w2d, H, I, grp, pre, ep, dgu)
        G.moe_group_gemm_quant(op_dgu, op_w1x, H, 2 * I, grp, dx)

    # warm up on a side stream, then capture (the library makes no allocation,
    # synchronisation or host query while capturing)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    for replay, seed in enumerate([101, 102, 103]):
        lg = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
        if replay == 1:
            lg[:, 2] = -np.inf          # an empty expert in one of the routings
        logits.copy_(torch.from_numpy(lg))
        # eager work between replays
        scratch = torch.ones(1 << 20, device="cuda") * 2.0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(scratch.sum()) == 2.0 * (1 << 20)

        _, rc, roff, _, rsrc = O.route_topk(lg, k)
        assert np.array_equal(cnt.cpu().numpy(), rc), replay
        assert np.array_equal(off.cpu().numpy(), roff), replay
        assert np.array_equal(src.cpu().numpy(), rsrc), replay
        xg_r = O.gather_rows(x_h, rsrc)
        assert np.array_equal(host_bits(xg), xg_r)
        rp, ry = O.fc1_glu(xg_r, rc, w1_h, O.Epilogue())
        assert_bf16_close(host_bits(y), ry, what=f"replay {replay} y")
        assert_bf16_close(host_bits(pre), rp, what=f"replay {replay} preact")
        # the rest of the chain from the oracle's own intermediates
        rdgu = O.dgrad_dglu(dy2_h, rc, w2_h, rp, O.Epilogue())
        assert_bf16_close(host_bits(out2), O.group_gemm(ry, rc, w2_h), what=f"replay {replay} fc2")
        assert_bf16_close(host_bits(dgu), rdgu, what=f"replay {replay} dgu", normwise=2e-2)
        assert_bf16_close(host_bits(dx), O.dx(rdgu, rc, w1_h), what=f"replay {replay} dx",
                          normwise=2e-2)


def test_graph_replays_on_one_routing_are_bit_identical(G):
    """Determinism: the captured step replayed several times on the same
    routing (with eager work and synchronisations between the replays) and
    the same step run eagerly give bit-identical outputs, every index array
    and every bf16 element.  The step kernels use no atomics and a fixed
    accumulation order per output element, so nothing may vary."""
    import torch
    T, E, k, H, I = 700, 5, 2, 256, 192          # I = 192: a half n-tile in FC1/dgrad
    TK = T * k
    rng = np.random.default_rng(78)
    x_h = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w1_h = W.to_bf16_bits((rng.standard_normal((E, H, 2 * I)) * 0.05).astype(np.float32))
    w2_h = W.to_bf16_bits((rng.standard_normal((E, I, H)) * 0.05).astype(np.float32))
    dy2_h = W.to_bf16_bits((rng.standard_normal((TK, H)) * 0.05).astype(np.float32))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    logits = torch.from_numpy(lg).cuda()
    x, w1, w2, dy2 = dev_bits(x_h), dev_bits(w1_h), dev_bits(w2_h), dev_bits(dy2_h)
    w1p = empty_bits((G.moe_packed_w1_bytes(E, H, I) // 2,))
    G.moe_repack_gate_up(w1, E, H, I, w1p)
    w1x = empty_bits((G.moe_packed_weight_bytes(E, H, 2 * I) // 2,))
    G.moe_pack_weight(w1, E, H, 2 * I, G.B_NK, w1x)
    w2f = empty_bits((G.moe_packed_weight_bytes(E, H, I) // 2,))
    G.moe_pack_weight(w2, E, H, I, G.B_KN, w2f)
    w2d = empty_bits((G.moe_packed_weight_bytes(E, I, H) // 2,))
    G.moe_pack_weight(w2, E, I, H, G.B_NK, w2d)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    dst = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src = torch.empty(TK, dtype=torch.int32, device="cuda")
    xg = empty_bits((TK, H))
    y, pre = empty_bits((TK, I)), empty_bits((TK, 2 * I))
    out2, dgu, dx = empty_bits((TK, H)), empty_bits((TK, 2 * I)), empty_bits((TK, H))
    grp = G.groups(cnt, TK)
    ep = G.epilogue("swiglu")
    op_y, op_w2 = G.operand(y), G.operand(w2f, layout=G.B_PACKED)
    op_dgu, op_w1x = G.operand(dgu), G.operand(w1x, layout=G.B_PACKED)
    op_w2d = G.operand(w2d, layout=G.B_PACKED)
    outs = dict(ids=ids, cnt=cnt, off=off, dst=dst, src=src, xg=xg, y=y, pre=pre, out2=out2,
                dgu=dgu, dx=dx)

    def step():
        G.moe_route_group(logits, None, T, E, k, ids, cnt, off, dst, src, x, H, xg)
        G.moe_group_gemm_glu_fwd(xg, grp, w1p, H, I, ep, y, pre)
        G.moe_group_gemm_quant(op_y, op_w2, H, I, grp, out2)
        G.moe_group_gemm_dglu_bwd(dy2, op_w2d, H, I, grp, pre, ep, dgu)
        G.moe_group_gemm_quant(op_dgu, op_w1x, H, 2 * I, grp, dx)

    def snapshot():
        torch.cuda.synchronize()
        return {n: t.cpu().numpy().copy() for n, t in outs.items()}

    def clobber():                       # make stale results visible
        for t in outs.values():
            t.fill_(-3)
        torch.cuda.synchronize()

    step()
    eager = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for replay in range(3):
        clobber()
        scratch = torch.ones(1 << 20, device="cuda") * 3.0      # eager work between replays
        g.replay()
        got = snapshot()
        assert float(scratch.sum()) == 3.0 * (1 << 20)
        for n in outs:
            assert np.array_equal(got[n], eager[n]), f"replay {replay}: {n} differs from the eager step"
    clobber()
    step()
    again = snapshot()
    for n in outs:
        assert np.array_equal(again[n], eager[n]), f"second eager step: {n} differs"
    # and the outputs are the oracle's (routing bit-exact, y within tolerance)
    _, rc, roff, _, rsrc = O.route_topk(lg, k)
    assert np.array_equal(eager["cnt"], rc) and np.array_equal(eager["src"], rsrc)
    _, ry = O.fc1_glu(O.gather_rows(x_h, rsrc), rc, w1_h, O.Epilogue())
    assert_bf16_close(eager["y"].view(np.uint16), ry, what="determinism y")
