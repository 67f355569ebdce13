"""Weight gradients at the DeepSeek-V3-like expert share's full size (32
experts, Zipf(1.1) counts summing to 16384 rows), in the launch configuration
bench.py times, on sampled output elements the oracle computes one by one:
dW1 = Xg^T dgu [32][7168][4096] and dW2 = y^T dY2 [32][2048][7168] in bf16
(moe_group_gemm_wgrad), and dW1 from K-tiled MXFP8 copies
(moe_group_gemm_wgrad_mx).

The gradient operands are seeded synthetic tensors of the chain's shapes and
scales (dgu ~ N(0, 1e-2), y ~ N(0, 0.1), dY2 ~ N(0, 5.906e-3)), drawn on the
host: every expected value is the oracle's on oracle-side inputs.  Each
sampled element is a sum over one expert's rows; the bound is the one of the
small-size tests (fp32 summation, plus the block-scaled MFMA's allowance).
"""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O
from tests.gpu_util import MX_ACC_REL, dev_bits, dev_bytes, dev_i32, empty_bytes

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def G():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_glu_amd as G
    G.moe_init(0)
    return G


@pytest.fixture(scope="module")
def data():
    d = W.dsv3(with_w2=False)
    M, H, I = d["M"], d["H"], d["I"]
    g = np.random.default_rng(91)
    dgu = W.to_bf16_bits((g.standard_normal((M, 2 * I)) * 1e-2).astype(np.float32))
    y = W.to_bf16_bits((g.standard_normal((M, I)) * 0.1).astype(np.float32))
    return dict(d=d, dgu=dgu, y=y, dy2=W.dsv3_dy2())


def _samples(counts, P, Q, seed, n_exp=6, n_el=24):
    """(expert, p, q) triples: the largest and smallest experts and random
    others, each with first/last indices and random ones."""
    g = np.random.default_rng(seed)
    order = np.argsort(counts)
    experts = sorted({int(order[-1]), int(order[0])} |
                     set(g.choice(len(counts), n_exp - 2, replace=False).tolist()))
    out = []
    for e in experts:
        ps = np.concatenate([[0, P - 1], g.integers(0, P, n_el - 2)])
        qs = np.concatenate([[Q - 1, 0], g.integers(0, Q, n_el - 2)])
        out += [(e, int(p), int(q)) for p, q in zip(ps, qs)]
    return out


def _check(got, a, b, counts, samples, what, mx_terms=None):
    off = np.concatenate([[0], np.cumsum(counts)])
    if mx_terms is None:
        A, B = F.bf16_bits_to_f64(a), F.bf16_bits_to_f64(b)
    worst = 0.0
    for e, p, q in samples:
        r0, r1 = int(off[e]), int(off[e + 1])
        if mx_terms is None:
            ap, bq = A[r0:r1, p], B[r0:r1, q]
            extra = 0.0
        else:
            ap, bq = mx_terms[0][e][p], mx_terms[1][e][q]
            extra = MX_ACC_REL
        ref = float(np.dot(ap, bq))
        s = float(np.dot(np.abs(ap), np.abs(bq)))
        bound = (extra + max(r1 - r0, 1) * 2.0 ** -24) * s
        err = abs(float(got[e, p, q]) - ref)
        worst = max(worst, err / s if s > 0 else 0.0)
        assert err <= bound + 1e-30, f"{what}: element {(e, p, q)} gpu={got[e, p, q]} ref={ref} bound={bound}"
    print(f"[wgrad] {what}: {len(samples)} sampled elements, max |err| / sum|ab| = {worst:.3g}")


def test_dsv3_dw1_dw2_bf16_sampled(G, data):
    import torch
    d = data["d"]
    counts, M, H, I = d["counts"], d["M"], d["H"], d["I"]
    grp = G.groups(dev_i32(counts), M)
    dw1 = torch.full((len(counts), H, 2 * I), float("nan"), dtype=torch.float32, device="cuda")
    G.moe_group_gemm_wgrad(dev_bits(d["x"]), dev_bits(data["dgu"]), H, 2 * I, grp, dw1)
    torch.cuda.synchronize()
    s1 = _samples(counts, H, 2 * I, 1)
    g1 = dw1.cpu().numpy()
    del dw1
    _check(g1, d["x"], data["dgu"], counts, s1, "dW1 bf16")
    del g1
    dw2 = torch.full((len(counts), I, H), float("nan"), dtype=torch.float32, device="cuda")
    G.moe_group_gemm_wgrad(dev_bits(data["y"]), dev_bits(data["dy2"]), I, H, grp, dw2)
    torch.cuda.synchronize()
    g2 = dw2.cpu().numpy()
    del dw2
    _check(g2, data["y"], data["dy2"], counts, _samples(counts, I, H, 2), "dW2 bf16")


def test_dsv3_dw1_mxfp8_sampled(G, data):
    """dW1 from K-tiled copies that the GPU quantiser writes (e4m3 for Xg,
    e5m2 for dgu); the oracle quantises the sampled columns of its own
    inputs, which must give the GPU's copies byte for byte."""
    import torch
    d = data["d"]
    counts, M, H, I = d["counts"], d["M"], d["H"], d["I"]
    E = len(counts)
    grp = G.groups(dev_i32(counts), M)
    S = G.mx_col_slots(M, E, blocked=True)
    xq, xs = empty_bytes((H, 32 * S)), empty_bytes((H, S))
    gq, gs = empty_bytes((2 * I, 32 * S)), empty_bytes((2 * I, S))
    G.moe_mxfp8_quantize(dev_bits(d["x"]), M, H, grp, G.mx_out(col_q=xq, col_s=xs, col_blocked=True))
    G.moe_mxfp8_quantize(dev_bits(data["dgu"]), M, 2 * I, grp,
                         G.mx_out(col_q=gq, col_s=gs, e5m2=True, col_blocked=True))
    dw1 = torch.full((E, H, 2 * I), float("nan"), dtype=torch.float32, device="cuda")
    G.moe_group_gemm_wgrad_mx(G.operand(xq, dtype=G.DT_MXFP8, scales=xs),
                              G.operand(gq, dtype=G.DT_MXFP8_E5M2, scales=gs), H, 2 * I, grp, dw1)
    torch.cuda.synchronize()
    samples = _samples(counts, H, 2 * I, 3)
    ps = sorted({p for _, p, _ in samples})
    qs = sorted({q for _, _, q in samples})
    # the oracle's K-tiled copies of the sampled columns, checked against the GPU's
    xcq, xcs = O.mx_quantize_cols(d["x"][:, ps], counts, m_cap=M, blocked=True)
    gcq, gcs = O.mx_quantize_cols(data["dgu"][:, qs], counts, m_cap=M, fmt="e5m2", blocked=True)
    used = int(O.mx_scale_col_offsets(counts, blocked=True)[-1])
    assert np.array_equal(xq.cpu().numpy()[ps][:, :32 * used], xcq[:, :32 * used])
    assert np.array_equal(xs.cpu().numpy()[ps][:, :used], xcs[:, :used])
    assert np.array_equal(gq.cpu().numpy()[qs][:, :32 * used], gcq[:, :32 * used])
    assert np.array_equal(gs.cpu().numpy()[qs][:, :used], gcs[:, :used])
    A = O.mx_dequantize_cols(xcq, xcs, counts, M, blocked=True)              # [M][len(ps)]
    B = O.mx_dequantize_cols(gcq, gcs, counts, M, "e5m2", blocked=True)      # [M][len(qs)]
    off = np.concatenate([[0], np.cumsum(counts)])
    ta = {e: {p: A[off[e]:off[e + 1], i] for i, p in enumerate(ps)} for e in range(E)}
    tb = {e: {q: B[off[e]:off[e + 1], i] for i, q in enumerate(qs)} for e in range(E)}
    got = dw1.cpu().numpy()
    _check(got, None, None, counts, samples, "dW1 mxfp8", mx_terms=(ta, tb))
