"""Pins of the oracle's MoE functions against brute force, closed forms,
invariants and finite differences.

Each test is chosen so that a plausible mistake in the oracle (a dropped bias,
swapped gate/up halves, a transposed operand, a wrong sign in a derivative,
an off-by-one in the grouping) fails it.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O


# ------------------------------------------------------------------ routing / grouping
def _route_bruteforce(logits, k):
    T, E = logits.shape
    ids = []
    for t in range(T):
        pairs = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        ids.append(pairs[:k])
    counts = [0] * E
    for t in range(T):
        for j in range(k):
            counts[ids[t][j]] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    fill = list(offsets[:-1])
    dst = [[0] * k for _ in range(T)]
    src = [0] * (T * k)
    for t in range(T):                       # (t, j) ascending = stable
        for j in range(k):
            e = ids[t][j]
            dst[t][j] = fill[e]
            src[fill[e]] = t
            fill[e] += 1
    return ids, counts, offsets, dst, src


@pytest.mark.parametrize("T,E,k,seed", [(7, 4, 2, 0), (33, 8, 3, 1), (64, 5, 1, 2), (20, 6, 6, 3)])
def test_route_matches_bruteforce(T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.integers(-3, 4, size=(T, E)).astype(np.float32)   # many exact ties
    ids, counts, off, dst, src = O.route_topk(logits, k)
    bids, bcounts, boff, bdst, bsrc = _route_bruteforce(logits, k)
    assert ids.tolist() == bids
    assert counts.tolist() == bcounts and off.tolist() == boff
    assert dst.tolist() == bdst and src.tolist() == bsrc


@pytest.mark.parametrize("T,E,k,seed", [(9, 5, 3, 0), (40, 7, 2, 1), (1, 3, 1, 2)])
def test_group_pairs_with_invalid_ids_bruteforce(T, E, k, seed):
    # ids outside [0, E) (negative, E, far above) are left out of the grouping
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)
    ids[0, 0] = 1000
    counts, off, dst, src = O.group_pairs(ids, E)
    rows = []                                  # (expert, t, j) in grouped order
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    rows.append((e, t, j))
    assert counts.tolist() == [sum(1 for r in rows if r[0] == e) for e in range(E)]
    assert off.tolist() == [sum(1 for r in rows if r[0] < e) for e in range(E + 1)]
    assert src.tolist() == [t for _, t, _ in rows]
    bdst = [[-1] * k for _ in range(T)]
    for r, (_, t, j) in enumerate(rows):
        bdst[t][j] = r
    assert dst.tolist() == bdst


@pytest.mark.parametrize("T,E,k,seed", [(7, 4, 2, 0), (33, 8, 3, 1), (1, 3, 1, 2)])
def test_gather_rows_against_loop_and_dst(T, E, k, seed):
    """gather_rows (the expected value of every grouped-row check): grouped row
    r is token src[r], element by element in a Python loop; and read through
    dst, pair (t, j) lands on row dst[t][j] holding token t's row."""
    rng = np.random.default_rng(300 + seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    H = 5
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    ids, counts, offsets, dst, src = _route_bruteforce(logits, k)
    xg = O.gather_rows(x, np.array(src, dtype=np.int32))
    assert xg.shape == (T * k, H) and xg.dtype == np.uint16
    for r in range(T * k):
        for c in range(H):
            assert int(xg[r, c]) == int(x[src[r], c])
    for t in range(T):
        for j in range(k):
            assert np.array_equal(xg[dst[t][j]], x[t])
    # a token permutation moves rows with their tokens: gathering x[perm] with
    # src' = inv(perm)[src] gives the same grouped rows
    perm = rng.permutation(T)
    inv = np.argsort(perm)
    assert np.array_equal(O.gather_rows(x[perm], inv[np.array(src)]), xg)
    # no routed pair: an empty result with H columns
    assert O.gather_rows(x, np.zeros(0, dtype=np.int32)).shape == (0, H)


def test_route_invariants_gptoss():
    d = W.gptoss(with_weights=False)
    ids, counts, off, dst, src = O.route_topk(d["logits"], d["k"])
    T, k, E = d["T"], d["k"], d["E"]
    assert counts.sum() == T * k and off[-1] == T * k
    assert np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(dst.reshape(-1)), np.arange(T * k))
    for t in (0, 17, T - 1):
        assert len(set(ids[t].tolist())) == k
        for j in range(k):
            r = dst[t, j]
            assert src[r] == t and off[ids[t, j]] <= r < off[ids[t, j] + 1]
    mean = T * k / E
    assert counts[0] == 0 and counts.max() > 2 * mean      # the workload's stated properties


def test_route_tiny_empty_expert():
    d = W.tiny(empty_expert=True)
    _, counts, off, _, _ = O.route_topk(d["logits"], d["k"])
    assert counts[3] == 0 and off[3] == off[4]


def test_dsv3_counts_zipf():
    c = W.dsv3_counts()
    assert c.sum() == 16384 and len(c) == 32
    s = np.sort(c)[::-1]
    assert s.tolist()[:4] == [4649, 2169, 1388, 1012] and s[-1] == 103
    # proportional to r^-1.1 within apportionment error
    w = np.arange(1, 33) ** -1.1
    assert np.all(np.abs(s - 16384 * w / w.sum()) < 1.0)


# ------------------------------------------------------------------ repack
def test_repack_roundtrip_and_permutation():
    rng = np.random.default_rng(3)
    E, H, I = 3, 16, 192
    w = rng.integers(0, 2 ** 16, size=(E, H, 2 * I)).astype(np.uint16)
    b = rng.integers(0, 2 ** 16, size=(E, 2 * I)).astype(np.uint16)
    wp, bp = O.repack_gate_up(w, b)
    assert wp.shape == (E, 2 * I, H)
    w2, b2 = O.unpack_gate_up(wp, bp)
    assert np.array_equal(w2, w) and np.array_equal(b2, b)
    assert np.array_equal(np.sort(wp.reshape(-1)), np.sort(w.reshape(-1)))
    # each 128-column packed block holds gate j..j+63 then the same up columns
    for p in range(I // 64):
        for s in range(64):
            assert np.array_equal(wp[:, 128 * p + s, :], w[:, :, 64 * p + s])
            assert np.array_equal(wp[:, 128 * p + 64 + s, :], w[:, :, I + 64 * p + s])


# ------------------------------------------------------------------ FC1 + GLU
def _act_scalar(g, act, alpha):
    if act == "swiglu":
        return g / (1.0 + math.exp(-alpha * g)) if g > -700 else 0.0
    if act == "geglu":
        return 0.5 * g * (1.0 + math.erf(g / math.sqrt(2.0)))
    if act == "geglu_tanh":
        return 0.5 * g * (1.0 + math.tanh(math.sqrt(2 / math.pi) * (g + 0.044715 * g ** 3)))
    if act == "srelu":
        return max(g, 0.0) ** 2
    raise ValueError


def _fc1_glu_loops(x, counts, w1, ep, bias=None):
    """Brute force in pure Python loops: the GLU identity
    y = act(x.Wg + bg) * (x.Wu + bu) on the plain (un-repacked) W1."""
    E, H, N2 = w1.shape
    I = N2 // 2
    off = np.concatenate([[0], np.cumsum(counts)])
    M = int(off[-1])
    y = np.zeros((M, I))
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for i in range(I):
                g = sum(x[r, h] * w1[e, h, i] for h in range(H))
                u = sum(x[r, h] * w1[e, h, I + i] for h in range(H))
                if bias is not None:
                    g += bias[e, i]
                    u += bias[e, I + i]
                g = min(max(g, ep.gate_lo), ep.gate_hi)
                u = min(max(u, ep.up_lo), ep.up_hi) + ep.up_offset
                y[r, i] = _act_scalar(g, ep.act, ep.alpha) * u
    return y


@pytest.mark.parametrize("act", ["swiglu", "geglu", "geglu_tanh", "srelu"])
def test_fc1_glu_matches_bruteforce_loops(act):
    rng = np.random.default_rng(4)
    counts = np.array([3, 0, 5, 1])
    E, H, I = 4, 6, 64
    x = W.to_bf16_bits(rng.standard_normal((9, H)).astype(np.float32))
    w1 = W.to_bf16_bits(rng.standard_normal((E, H, 2 * I)).astype(np.float32) * 0.5)
    b1 = W.to_bf16_bits(rng.standard_normal((E, 2 * I)).astype(np.float32) * 0.1)
    ep = O.Epilogue(act=act, alpha=1.702 if act == "swiglu" else 1.0, gate_lo=-1.0, gate_hi=1.5,
                    up_lo=-2.0, up_hi=1.0, up_offset=0.25, bias=b1)
    preact, y = O.fc1_glu(x, counts, w1, ep)
    ref = _fc1_glu_loops(F.bf16_bits_to_f64(x), counts, F.bf16_bits_to_f64(w1), ep,
                         F.bf16_bits_to_f64(b1))
    assert np.array_equal(y, F.f64_to_bf16_bits(ref))
    assert y.shape == (9, I) and preact.shape == (9, 2 * I)


def test_fc1_glu_through_packed_weights():
    """The packed layout carries the pairing: a GEMM on the packed weights whose
    every 128-column block is split 64 | 64 gives the same GLU as gate | up."""
    rng = np.random.default_rng(5)
    E, H, I = 2, 32, 128
    counts = np.array([7, 4])
    x = W.to_bf16_bits(rng.standard_normal((11, H)).astype(np.float32))
    w1 = W.to_bf16_bits(rng.standard_normal((E, H, 2 * I)).astype(np.float32) * 0.3)
    wp, _ = O.repack_gate_up(w1)
    ep = O.Epilogue()
    _, y = O.fc1_glu(x, counts, w1, ep)
    xf = F.bf16_bits_to_f64(x)
    off = [0, 7, 11]
    ypk = np.zeros((11, I))
    for e in range(E):
        zp = xf[off[e]:off[e + 1]] @ F.bf16_bits_to_f64(wp[e]).T       # packed order
        for p in range(I // 64):
            g = zp[:, 128 * p:128 * p + 64]
            u = zp[:, 128 * p + 64:128 * p + 128]
            ypk[off[e]:off[e + 1], 64 * p:64 * p + 64] = g / (1 + np.exp(-g)) * u
    assert np.array_equal(y, F.f64_to_bf16_bits(ypk))


def test_fc1_zero_token_experts_produce_nothing():
    rng = np.random.default_rng(6)
    E, H, I = 3, 8, 64
    w1 = W.to_bf16_bits(rng.standard_normal((E, H, 2 * I)).astype(np.float32))
    x = W.to_bf16_bits(rng.standard_normal((5, H)).astype(np.float32))
    p1, y1 = O.fc1_glu(x, [0, 5, 0], w1, O.Epilogue())
    # same rows, expert 0/2 weights replaced by NaN: nothing changes
    w1n = w1.copy()
    w1n[0] = 0x7FC0
    w1n[2] = 0x7FC0
    p2, y2 = O.fc1_glu(x, [0, 5, 0], w1n, O.Epilogue())
    assert np.array_equal(y1, y2) and np.array_equal(p1, p2)
    assert y1.shape[0] == 5


def test_fc1_row_permutation_within_group():
    rng = np.random.default_rng(7)
    E, H, I = 2, 16, 64
    counts = np.array([6, 5])
    w1 = W.to_bf16_bits(rng.standard_normal((E, H, 2 * I)).astype(np.float32) * 0.2)
    x = W.to_bf16_bits(rng.standard_normal((11, H)).astype(np.float32))
    perm = np.concatenate([rng.permutation(6), 6 + rng.permutation(5)])
    p1, y1 = O.fc1_glu(x, counts, w1, O.Epilogue())
    p2, y2 = O.fc1_glu(x[perm], counts, w1, O.Epilogue())
    assert np.array_equal(y1[perm], y2) and np.array_equal(p1[perm], p2)
    q1, s1 = O.mx_quantize_rows(y1)
    q2, s2 = O.mx_quantize_rows(y2)
    assert np.array_equal(q1[perm], q2) and np.array_equal(s1[perm], s2)


# ------------------------------------------------------------------ activations
def test_activation_special_values():
    z = np.array([0.0])
    assert O.activation(z, "swiglu")[0] == 0.0
    assert O.activation_grad(z, "swiglu")[0] == 0.5
    assert O.activation(z, "geglu")[0] == 0.0
    assert O.activation_grad(z, "geglu")[0] == 0.5
    assert O.activation_grad(z, "geglu_tanh")[0] == 0.5
    assert O.activation_grad(z, "srelu")[0] == 0.0
    big = np.array([-1e4, -800.0])
    for a in ("swiglu", "geglu", "geglu_tanh", "srelu"):
        v = O.activation(big, a)
        d = O.activation_grad(big, a)
        assert np.all(np.isfinite(v)) and np.all(np.abs(v) < 1e-30)
        assert np.all(np.isfinite(d)) and np.all(np.abs(d) < 1e-30)
    assert O.activation(np.array([3.0]), "srelu")[0] == 9.0
    # silu(x) -> x for large x; gelu(x) -> x
    assert abs(O.activation(np.array([40.0]), "swiglu")[0] - 40.0) < 1e-12
    assert abs(O.activation(np.array([40.0]), "geglu")[0] - 40.0) < 1e-12


@pytest.mark.parametrize("act,alpha", [("swiglu", 1.0), ("swiglu", 1.702), ("geglu", 1.0),
                                       ("geglu_tanh", 1.0), ("srelu", 1.0)])
def test_activation_grad_finite_difference(act, alpha):
    g = np.linspace(-6, 6, 241) + 0.013
    h = 1e-6
    fd = (O.activation(g + h, act, alpha) - O.activation(g - h, act, alpha)) / (2 * h)
    an = O.activation_grad(g, act, alpha)
    assert np.max(np.abs(fd - an) / np.maximum(1, np.abs(an))) < 1e-7


# ------------------------------------------------------------------ backward: finite differences
def _tiny_chain(seed, act, ep_kw):
    rng = np.random.default_rng(seed)
    T, H, I, E = 4, 8, 8, 2
    counts = np.array([3, 1])
    x = F.bf16_round(rng.standard_normal((T, H)))
    w1 = F.bf16_round(rng.standard_normal((E, H, 2 * I)) * 0.5)
    b1 = F.bf16_round(rng.standard_normal((E, 2 * I)) * 0.1)
    w2 = F.bf16_round(rng.standard_normal((E, I, H)) * 0.5)
    dy2 = F.bf16_round(rng.standard_normal((T, H)))
    ep = O.Epilogue(act=act, **ep_kw)
    return counts, x, w1, b1, w2, dy2, ep


def _loss(x, counts, w1, b1, w2, dy2, ep):
    """L = <dY2, FC2(GLU(FC1(X)))> in exact float64 (no rounding)."""
    off = np.concatenate([[0], np.cumsum(counts)])
    L = 0.0
    for e in range(len(counts)):
        a, b = off[e], off[e + 1]
        z = x[a:b] @ w1[e] + b1[e]
        y = O.glu_from_preact(z, ep)
        L += float(np.sum(dy2[a:b] * (y @ w2[e])))
    return L


@pytest.mark.parametrize("act,ep_kw", [
    ("swiglu", {}), ("swiglu", dict(alpha=1.702, gate_lo=-0.7, gate_hi=0.7, up_lo=-0.7, up_hi=0.7)),
    ("geglu", {}), ("geglu_tanh", dict(up_offset=1.0)), ("srelu", {}),
])
def test_dglu_and_dx_against_finite_differences(act, ep_kw):
    counts, x, w1, b1, w2, dy2, ep = _tiny_chain(21, act, ep_kw)
    off = np.concatenate([[0], np.cumsum(counts)])
    # analytic: G = dY2 W2^T, dz = dglu(G, z), dX = dz W1^T
    dz_all, dx_all, z_all = [], [], []
    for e in range(2):
        a, b = off[e], off[e + 1]
        z = x[a:b] @ w1[e] + b1[e]
        G = dy2[a:b] @ w2[e].T
        dz = O.dglu(G, z, ep)
        dz_all.append(dz)
        dx_all.append(dz @ w1[e].T)
        z_all.append(z)
    dX = np.concatenate(dx_all)

    # finite differences on X
    checked = 0
    for t in range(x.shape[0]):
        for hh in range(x.shape[1]):
            h = 1e-6 * max(1.0, abs(x[t, hh]))
            xp, xm = x.copy(), x.copy()
            xp[t, hh] += h
            xm[t, hh] -= h
            # skip points whose perturbation crosses a clamp bound or the srelu kink
            e = int(np.searchsorted(off, t, side="right") - 1)
            z = x[t] @ w1[e] + b1[e]
            dzmax = 2 * h * np.max(np.abs(w1[e][hh]))
            I = z.shape[0] // 2
            bounds = [ep.gate_lo, ep.gate_hi]
            near = np.any([np.any(np.abs(z[:I] - bd) <= 2 * dzmax) for bd in bounds if np.isfinite(bd)])
            near |= np.any([np.any(np.abs(z[I:] - bd) <= 2 * dzmax) for bd in (ep.up_lo, ep.up_hi) if np.isfinite(bd)])
            if act == "srelu":
                near |= np.any(np.abs(z[:I]) <= 2 * dzmax)
            if near:
                continue
            fd = (_loss(xp, counts, w1, b1, w2, dy2, ep) - _loss(xm, counts, w1, b1, w2, dy2, ep)) / (2 * h)
            assert abs(fd - dX[t, hh]) <= 1e-6 * max(1.0, abs(fd)), (t, hh, fd, dX[t, hh])
            checked += 1
    assert checked >= 16


def test_dgrad_dglu_and_dx_bf16_functions_match_f64_chain():
    """The bf16-rounding oracle functions equal the float64 chain above up to
    the final bf16 rounding of each output."""
    rng = np.random.default_rng(22)
    E, H, I = 3, 32, 64
    counts = np.array([5, 0, 9])
    M = 14
    dy2 = W.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    w2 = W.to_bf16_bits(rng.standard_normal((E, I, H)).astype(np.float32) * 0.2)
    w1 = W.to_bf16_bits(rng.standard_normal((E, H, 2 * I)).astype(np.float32) * 0.2)
    pre = W.to_bf16_bits(rng.standard_normal((M, 2 * I)).astype(np.float32))
    ep = O.Epilogue(alpha=1.702, gate_lo=-7, gate_hi=7, up_lo=-7, up_hi=7)
    dgu = O.dgrad_dglu(dy2, counts, w2, pre, ep)
    off = [0, 5, 5, 14]
    for e in (0, 2):
        a, b = off[e], off[e + 1]
        G = F.bf16_bits_to_f64(dy2[a:b]) @ F.bf16_bits_to_f64(w2[e]).T
        want = O.dglu(G, F.bf16_bits_to_f64(pre[a:b]), ep)
        assert np.array_equal(dgu[a:b], F.f64_to_bf16_bits(want))
    dX = O.dx(dgu, counts, w1)
    for e in (0, 2):
        a, b = off[e], off[e + 1]
        want = F.bf16_bits_to_f64(dgu[a:b]) @ F.bf16_bits_to_f64(w1[e]).T
        assert np.array_equal(dX[a:b], F.f64_to_bf16_bits(want))


# ------------------------------------------------------------------ GEMM, integer-exact
def test_group_gemm_integer_exact_against_loops():
    E, K, N = 3, 40, 24
    counts = np.array([4, 0, 6])
    a = W.ternary_bf16(1, (10, K))
    b = np.stack([W.ternary_bf16(2 + e, (K, N)) for e in range(E)])
    out = O.group_gemm(a, counts, b)
    af, bf = F.bf16_bits_to_f64(a), F.bf16_bits_to_f64(b)
    off = [0, 4, 4, 10]
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for n in range(N):
                s = 0.0
                for k in range(K):
                    s += af[r, k] * bf[e, k, n]
                assert F.bf16_bits_to_f64(out[r:r + 1, n:n + 1])[0, 0] == s


# ------------------------------------------------------------------ MXFP8 rows / cols
def test_mx_rows_scale_rule_and_bound():
    rng = np.random.default_rng(30)
    v = W.to_bf16_bits((rng.standard_t(3, size=(7, 96)) * 0.5).astype(np.float32))
    q, s = O.mx_quantize_rows(v)
    vf = F.bf16_bits_to_f64(v)
    deq = O.mx_dequantize_rows(q, s)
    for r in range(7):
        for cb in range(3):
            blk = vf[r, 32 * cb:32 * cb + 32]
            X = 2.0 ** (int(s[r, cb]) - 127)
            amax = np.max(np.abs(blk))
            assert amax / X <= 448 and (amax == 0 or amax / (X / 2) > 448)
            assert np.all(np.abs(deq[r, 32 * cb:32 * cb + 32] - blk) <= 0.5 * F.e4m3_ulp(blk / X) * X)


def test_mx_cols_restart_per_group_and_match_rows_of_transpose():
    rng = np.random.default_rng(31)
    counts = np.array([64, 0, 37, 5])
    M = int(counts.sum())
    m_cap = M + 11
    C = 64
    v = W.to_bf16_bits(rng.standard_normal((m_cap, C)).astype(np.float32))
    col_q, col_s = O.mx_quantize_cols(v[:M], counts, m_cap=m_cap)
    assert col_q.shape == (C, m_cap) and col_s.shape == (C, (m_cap + 31) // 32 + 4)
    so = O.mx_scale_col_offsets(counts)
    assert so.tolist() == [0, 2, 2, 4, 5]
    # group 0 has two full blocks: equals the row-wise quantisation of its transpose
    q0, s0 = O.mx_quantize_rows(np.ascontiguousarray(v[0:64].T))
    assert np.array_equal(col_q[:, 0:64], q0) and np.array_equal(col_s[:, 0:2], s0)
    # group 2 (rows 64..100): a full block then a partial 5-row block; group 3 partial
    vf = F.bf16_bits_to_f64(v)
    for (r0, r1, sc) in [(64, 96, 2), (96, 101, 3), (101, 106, 4)]:
        for c in range(C):
            blk = vf[r0:r1, c]
            X = 2.0 ** (int(col_s[c, sc]) - 127)
            assert np.max(np.abs(blk)) / X <= 448
            assert np.max(np.abs(blk)) == 0 or np.max(np.abs(blk)) / (X / 2) > 448
            deq = F.e4m3_decode(col_q[c, r0:r1]) * X
            assert np.all(np.abs(deq - blk) <= 0.5 * F.e4m3_ulp(blk / X) * X)
    # rows beyond M are never written
    assert np.all(col_q[:, M:] == 0)


def test_group_gemm_mx_against_loops():
    rng = np.random.default_rng(32)
    E, K, N = 2, 64, 8
    counts = np.array([3, 2])
    a = W.to_bf16_bits(rng.standard_normal((5, K)).astype(np.float32))
    aq, as_ = O.mx_quantize_rows(a)
    bw = W.to_bf16_bits(rng.standard_normal((E, N, K)).astype(np.float32))
    bq = np.zeros((E, N, K), np.uint8)
    bs = np.zeros((E, N, K // 32), np.uint8)
    for e in range(E):
        bq[e], bs[e] = O.mx_quantize_rows(bw[e])
    out = O.group_gemm_mx(aq, as_, counts, bq, bs)
    off = [0, 3, 5]
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for n in range(N):
                s = 0.0
                for k in range(K):
                    xa = F.e4m3_decode(aq[r, k]) * 2.0 ** (int(as_[r, k // 32]) - 127)
                    xb = F.e4m3_decode(bq[e, n, k]) * 2.0 ** (int(bs[e, n, k // 32]) - 127)
                    s += xa * xb
                assert out[r, n] == F.f64_to_bf16_bits(np.array([s]))[0]



def test_wgrad_abs_against_loops():
    """wgrad_abs (the error scale of every weight-gradient GPU bound) is
    sum over each group's rows of |a[r][i]| |b[r][j]|, written out as a loop;
    signs never cancel (it bounds |wgrad| from above) and an empty group
    gives zeros."""
    rng = np.random.default_rng(52)
    counts = np.array([4, 0, 3, 1])
    M, P, Q = 8, 3, 5
    a = W.to_bf16_bits(rng.standard_normal((M + 2, P)).astype(np.float32))
    b = W.to_bf16_bits(rng.standard_normal((M + 2, Q)).astype(np.float32))
    got = O.wgrad_abs(a, counts, b)
    assert got.shape == (4, P, Q) and np.all(got[1] == 0.0)
    A, B = F.bf16_bits_to_f64(a), F.bf16_bits_to_f64(b)
    off = [0, 4, 4, 7, 8]
    for e in range(4):
        for i in range(P):
            for j in range(Q):
                s = 0.0
                for r in range(off[e], off[e + 1]):
                    s += abs(A[r, i]) * abs(B[r, j])
                assert got[e, i, j] == pytest.approx(s, rel=1e-15, abs=1e-300)
    assert np.all(np.abs(O.wgrad(a, counts, b)) <= got * (1 + 1e-12))
    # all-positive operands: no cancellation, so it equals wgrad itself
    ap, bp = a & np.uint16(0x7FFF), b & np.uint16(0x7FFF)
    assert np.allclose(O.wgrad_abs(ap, counts, bp), O.wgrad(ap, counts, bp), rtol=1e-15, atol=0)
    # flipping the sign of operand rows changes wgrad but not wgrad_abs
    assert np.array_equal(O.wgrad_abs(a ^ np.uint16(0x8000), counts, b), got)


# ------------------------------------------------------------------ weight gradients
def test_wgrad_against_loops_and_empty_groups():
    rng = np.random.default_rng(51)
    counts = np.array([3, 0, 2])
    M, P, Q = 5, 4, 6
    a = W.to_bf16_bits(rng.standard_normal((M + 2, P)).astype(np.float32))
    b = W.to_bf16_bits(rng.standard_normal((M + 2, Q)).astype(np.float32))
    out = O.wgrad(a, counts, b)
    assert out.shape == (3, P, Q)
    assert np.all(out[1] == 0.0)
    off = [0, 3, 3, 5]
    A, B = F.bf16_bits_to_f64(a), F.bf16_bits_to_f64(b)
    for e in range(3):
        for i in range(P):
            for j in range(Q):
                s = 0.0
                for r in range(off[e], off[e + 1]):
                    s += A[r, i] * B[r, j]
                assert out[e, i, j] == pytest.approx(s, rel=1e-15, abs=1e-300)
    # rows past the routed ones never enter
    b2 = b.copy()
    b2[M:] = 0x7FC0
    assert np.array_equal(O.wgrad(a, counts, b2), out)


@pytest.mark.parametrize("act,ep_kw", [("swiglu", {}),
                                       ("swiglu", dict(alpha=1.702, gate_lo=-0.7, gate_hi=0.7,
                                                       up_lo=-0.7, up_hi=0.7)),
                                       ("geglu", {})])
def test_wgrads_against_finite_differences(act, ep_kw):
    """dW1 = wgrad(X, dgu) and dW2 = wgrad(y, dY2) are the gradients of
    L = <dY2, FC2(GLU(FC1(X)))> with respect to W1 and W2."""
    counts, x, w1, b1, w2, dy2, ep = _tiny_chain(23, act, ep_kw)
    off = np.concatenate([[0], np.cumsum(counts)])
    dz_all, y_all = [], []
    for e in range(2):
        a, b = off[e], off[e + 1]
        z = x[a:b] @ w1[e] + b1[e]
        dz_all.append(O.dglu(dy2[a:b] @ w2[e].T, z, ep))
        y_all.append(O.glu_from_preact(z, ep))
    dz, y = np.concatenate(dz_all), np.concatenate(y_all)
    # the oracle takes bf16 bit patterns: dz and y are rounded to bf16 first,
    # so compare within that rounding (2^-8 of sum |a||b|); a transposed or
    # swapped operand, or rows of the wrong group, would miss by O(1)
    dzb, yb = F.f64_to_bf16_bits(dz), F.f64_to_bf16_bits(y)
    xb, dyb = F.f64_to_bf16_bits(x), F.f64_to_bf16_bits(dy2)
    dW1, dW2 = O.wgrad(xb, counts, dzb), O.wgrad(yb, counts, dyb)
    tol1 = 2.0 ** -8 * O.wgrad_abs(xb, counts, dzb) + 1e-9
    tol2 = 2.0 ** -8 * O.wgrad_abs(yb, counts, dyb) + 1e-9
    checked = 0
    for e in range(2):
        for (wname, wt, grad, tol) in (("w1", w1, dW1, tol1), ("w2", w2, dW2, tol2)):
            for idx in [(0, 0), (1, 3), (wt.shape[1] - 1, wt.shape[2] - 1), (2, 5)]:
                h = 1e-6 * max(1.0, abs(wt[e][idx]))
                wp, wm = wt.copy(), wt.copy()
                wp[e][idx] += h
                wm[e][idx] -= h
                args_p = (x, counts, wp, b1, w2, dy2, ep) if wname == "w1" else (x, counts, w1, b1, wp, dy2, ep)
                args_m = (x, counts, wm, b1, w2, dy2, ep) if wname == "w1" else (x, counts, w1, b1, wm, dy2, ep)
                fd = (_loss(*args_p) - _loss(*args_m)) / (2 * h)
                if wname == "w1" and ep_kw:
                    # skip perturbations that move a pre-activation across a clamp bound
                    a, b = off[e], off[e + 1]
                    z = x[a:b] @ w1[e] + b1[e]
                    dzmax = 2 * h * np.max(np.abs(x[a:b, idx[0]]))
                    bounds = [ep.gate_lo, ep.gate_hi, ep.up_lo, ep.up_hi]
                    if np.any([np.any(np.abs(z - bd) <= 2 * dzmax) for bd in bounds]):
                        continue
                assert abs(fd - grad[e][idx]) <= tol[e][idx] + 1e-6 * abs(fd), (wname, e, idx, fd, grad[e][idx])
                checked += 1
    assert checked >= 12


def _mx_exact_values(rng, shape):
    """bf16 bits of values that MXFP8 quantisation reproduces exactly: each
    32-block is e4m3 values times 2^E with its first value at 448 * 2^E (so
    the block's scale rule gives E back)."""
    R, C = shape
    codes = rng.integers(0, 0x7F, size=(R, C)).astype(np.uint8)      # finite e4m3 codes
    codes[:, ::32] = 0x7E                                            # 448
    sign = rng.integers(0, 2, size=(R, C)).astype(np.uint8) << 7
    E = rng.integers(-12, 3, size=(R, C // 32))
    v = F.e4m3_decode(codes | sign) * np.repeat(2.0 ** E, 32, axis=1)
    return F.f64_to_bf16_bits(v)


@pytest.mark.parametrize("bias", [False, True])
def test_fc1_glu_mx_equals_fc1_glu_on_exactly_quantised_inputs(bias):
    rng = np.random.default_rng(61)
    counts = np.array([5, 0, 3])
    E, H, I = 3, 64, 32
    x = _mx_exact_values(rng, (8, H))
    w1t = np.stack([_mx_exact_values(rng, (2 * I, H)) for _ in range(E)])   # W1_e^T [2I][H]
    w1 = np.ascontiguousarray(np.transpose(w1t, (0, 2, 1)))
    b1 = W.to_bf16_bits((rng.standard_normal((E, 2 * I)) * 0.1).astype(np.float32)) if bias else None
    ep = O.Epilogue(alpha=1.702, gate_lo=-7, gate_hi=7, up_lo=-7, up_hi=7, bias=b1)
    aq, as_ = O.mx_quantize_rows(x)
    assert np.array_equal(F.f64_to_bf16_bits(O.mx_dequantize_rows(aq, as_)), x)   # exact round trip
    wq = np.zeros((E, 2 * I, H), np.uint8)
    ws = np.zeros((E, 2 * I, H // 32), np.uint8)
    for e in range(E):
        wq[e], ws[e] = O.mx_quantize_rows(w1t[e])
    pre_mx, y_mx = O.fc1_glu_mx(aq, as_, counts, wq, ws, ep)
    pre, y = O.fc1_glu(x, counts, w1, ep)
    assert np.array_equal(pre_mx, pre) and np.array_equal(y_mx, y)


def test_tensor_amax_planted_values():
    """Planted extremes: the largest magnitude is negative, a larger one sits in
    a row past the routed ones, NaN is skipped, and no routed rows gives 0."""
    y = np.zeros((6, 4), dtype=np.uint16)
    y[0, 1] = 0x4040                     # 3.0
    y[3, 2] = 0xC060                     # -3.5
    y[4, 0] = 0x7FC0                     # NaN (routed)
    y[5, 3] = 0x4300                     # 128.0 in an unrouted row
    counts = np.array([2, 0, 3])         # M = 5
    assert O.tensor_amax(y, counts) == 3.5
    assert O.tensor_amax(y, np.array([6])) == 128.0
    assert O.tensor_amax(y, np.array([0, 0])) == 0.0
    y[1, 0] = 0xFF80                     # -inf
    assert O.tensor_amax(y, counts) == math.inf


def test_tensor_amax_of_fc1_bounds_the_glu_closed_form():
    """amax of y from fc1_glu against the closed form of one routed row:
    with W1 one-hot, z = x's entries, so y_j = silu(x_g) x_u in bf16 and the
    amax is the largest of those products."""
    H, I = 8, 4
    x = W.to_bf16_bits(np.array([[1.0, -2.0, 0.5, 3.0, 2.0, -1.0, 0.25, 4.0]], dtype=np.float32))
    w1 = np.zeros((1, H, 2 * I), dtype=np.float32)
    for j in range(2 * I):
        w1[0, j, j] = 1.0                # z_j = x_j
    _, y = O.fc1_glu(x, np.array([1]), W.to_bf16_bits(w1), O.Epilogue())
    g, u = np.array([1.0, -2.0, 0.5, 3.0]), np.array([2.0, -1.0, 0.25, 4.0])
    silu = g / (1.0 + np.exp(-g))
    want = np.max(np.abs(F.bf16_bits_to_f64(F.f64_to_bf16_bits(silu * u))))
    assert O.tensor_amax(y, np.array([1])) == want
    assert abs(want - 3.0 / (1.0 + math.exp(-3.0)) * 4.0) < 0.05


def test_sylvester_hadamard_against_library_and_orthogonality():
    import scipy.linalg
    for n in (1, 2, 4, 16):
        assert np.array_equal(O.sylvester_hadamard(n), scipy.linalg.hadamard(n))
    h = O.sylvester_hadamard(16)
    assert np.array_equal(h @ h.T, 16 * np.eye(16))


def _bf(vals):
    return W.to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_rht16_amax_closed_forms():
    """Closed forms of the 16-row rotation R = H16 S / 4 on one column."""
    c = 3.0
    # a lone entry x: every output is +-x/4
    col = np.zeros((16, 1)); col[5, 0] = -6.0
    assert O.rht16_amax(_bf(col), [16]) == 1.5
    # a constant run: all of it lands in output 0 (4c), whatever the uniform sign
    col = np.full((16, 1), c)
    assert O.rht16_amax(_bf(col), [16]) == 4 * c
    assert O.rht16_amax(_bf(col), [16], signs=0xFFFF) == 4 * c
    # one flipped row: output 0 is 14c/4, every other output +-2c/4
    assert O.rht16_amax(_bf(col), [16], signs=0x0001) == 3.5 * c
    # a partial run of 4 rows is padded with zeros: outputs 0, 4, 8, 12 are c
    assert O.rht16_amax(_bf(np.full((4, 1), c)), [4]) == c
    # runs restart at each group's first row: rows 5..20 form one run of
    # group 1 (not 11 + 5 rows of two runs aligned at row 0)
    col = np.zeros((21, 1)); col[5:] = c
    assert O.rht16_amax(_bf(col), [5, 16]) == 4 * c
    assert O.rht16_amax(_bf(col), [21]) == 11 * c / 4
    # rows past the routed ones do not count; no routed rows gives 0
    assert O.rht16_amax(_bf(col), [5, 0]) == 0.0


def test_rht16_amax_against_library_hadamard():
    """Random ragged groups with random signs against an explicit product
    with scipy's Hadamard matrix, run by run."""
    import scipy.linalg
    rng = np.random.default_rng(11)
    counts = np.array([37, 0, 16, 1, 50])
    x = _bf(rng.standard_normal((int(counts.sum()) + 3, 24)))
    signs = int(rng.integers(0, 1 << 16))
    v = F.bf16_bits_to_f64(x)
    S = np.diag([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
    best, r = 0.0, 0
    for m in counts:
        for k in range(0, int(m), 16):
            blk = np.zeros((16, 24))
            n = min(16, int(m) - k)
            blk[:n] = v[r + k: r + k + n]
            best = max(best, float(np.abs(scipy.linalg.hadamard(16) @ S @ blk).max()) / 4)
        r += int(m)
    assert O.rht16_amax(x, counts, signs) == best
    # Parseval on the full runs: the rotation keeps every run's norm
    blk = v[:16]
    R = O.sylvester_hadamard(16) @ S / 4
    assert np.isclose(np.linalg.norm(R @ blk), np.linalg.norm(blk))


def _dyadic_chain(seed, act, ep_kw):
    """A tiny chain whose pre-activations are exact in bf16 (x in {-1,0,1},
    W1 in {-0.5,0,0.5}, b1 in {-0.25,0,0.25}: z is a multiple of 0.25 below
    4.25 in magnitude), so the oracle's bf16 pre-activation equals the exact z."""
    rng = np.random.default_rng(seed)
    T, H, I, E = 5, 8, 8, 2
    counts = np.array([3, 2])
    x = rng.integers(-1, 2, (T, H)).astype(np.float64)
    w1 = rng.integers(-1, 2, (E, H, 2 * I)) * 0.5
    b1 = rng.integers(-1, 2, (E, 2 * I)) * 0.25
    w2 = F.bf16_round(rng.standard_normal((E, I, H)) * 0.5)
    dy2 = F.bf16_round(rng.standard_normal((T, H)))
    rs = F.bf16_round(rng.uniform(0.5, 1.5, T))
    ep = O.Epilogue(act=act, **ep_kw)
    return counts, x, w1, b1, w2, dy2, rs, ep


def _loss_rs(x, counts, w1, b1, w2, dy2, rs, ep):
    off = np.concatenate([[0], np.cumsum(counts)])
    L = 0.0
    for e in range(len(counts)):
        a, b = off[e], off[e + 1]
        z = x[a:b] @ w1[e] + b1[e]
        y = O.glu_from_preact(z, ep) * rs[a:b, None]
        L += float(np.sum(dy2[a:b] * (y @ w2[e])))
    return L


@pytest.mark.parametrize("act,ep_kw", [("swiglu", dict(alpha=1.702)), ("geglu", {}),
                                       ("srelu", dict(gate_lo=-1.0, gate_hi=1.0, up_offset=0.5))])
def test_bias_and_row_scale_grads_against_finite_differences(act, ep_kw):
    """dL/db1 and dL/drs of L = <dY2, FC2(GLU(X W1 + b1) * rs)> by central
    differences in float64, against bias_grad (on the float64 dgu rounded to
    bf16: bound = that rounding) and row_scale_grad."""
    counts, x, w1, b1, w2, dy2, rs, ep = _dyadic_chain(5, act, ep_kw)
    off = np.concatenate([[0], np.cumsum(counts)])
    z = np.concatenate([x[off[e]:off[e + 1]] @ w1[e] + b1[e] for e in range(2)])
    assert np.array_equal(F.bf16_round(z), z)
    G = np.concatenate([dy2[off[e]:off[e + 1]] @ w2[e].T for e in range(2)])
    dz = O.dglu(G, z, ep, rs)
    bits = F.f64_to_bf16_bits
    db = O.bias_grad(bits(dz), counts)
    drs = O.row_scale_grad(bits(dy2), counts, bits(w2), bits(z), ep)
    checked = 0
    for e in range(2):
        for c in range(z.shape[1]):
            h = 1e-6
            bp, bm = b1.copy(), b1.copy()
            bp[e, c] += h
            bm[e, c] -= h
            zr = z[off[e]:off[e + 1], c]
            lo, hi = (ep.gate_lo, ep.gate_hi) if c < 8 else (ep.up_lo, ep.up_hi)
            if np.any(np.abs(zr - lo) < 4 * h) or np.any(np.abs(zr - hi) < 4 * h) or (
                    act == "srelu" and c < 8 and np.any(np.abs(zr) < 4 * h)):
                continue
            fd = (_loss_rs(x, counts, w1, bp, w2, dy2, rs, ep) -
                  _loss_rs(x, counts, w1, bm, w2, dy2, rs, ep)) / (2 * h)
            bound = 1e-6 * max(1.0, abs(fd)) + 2.0 ** -8 * np.sum(np.abs(dz[off[e]:off[e + 1], c]))
            assert abs(db[e, c] - fd) <= bound, (e, c, db[e, c], fd)
            checked += 1
    assert checked >= 16
    for r in range(x.shape[0]):
        h = 1e-6
        rp, rm = rs.copy(), rs.copy()
        rp[r] += h
        rm[r] -= h
        fd = (_loss_rs(x, counts, w1, b1, w2, dy2, rp, ep) -
              _loss_rs(x, counts, w1, b1, w2, dy2, rm, ep)) / (2 * h)
        assert abs(drs[r] - fd) <= 1e-6 * max(1.0, abs(fd)), (r, drs[r], fd)


def test_bias_grad_sums_rows_of_each_group():
    v = np.arange(24, dtype=np.float64).reshape(6, 4) - 7
    counts = np.array([2, 0, 3])          # rows 0-1, none, 2-4; row 5 unrouted
    db = O.bias_grad(F.f64_to_bf16_bits(v), counts)
    assert np.array_equal(db[0], v[0] + v[1])
    assert np.array_equal(db[1], np.zeros(4))
    assert np.array_equal(db[2], v[2] + v[3] + v[4])


@pytest.mark.parametrize("act", ["srelu", "swiglu", "geglu"])
def test_non_gated_forward_and_backward(act):
    """Non-gated y = a(z) * rs: the forward against a scalar loop, the
    backward dz against central differences of L = <dY2, FC2(y)> in z on a
    bf16-exact chain (z = x W1 + b1 exact in bf16)."""
    rng = np.random.default_rng(31)
    T, H, I = 5, 8, 8
    counts = np.array([3, 2])
    x = rng.integers(-1, 2, (T, H)).astype(np.float64)
    w1 = rng.integers(-1, 2, (2, H, I)) * 0.5
    b1 = rng.integers(-1, 2, (2, I)) * 0.25
    w2 = F.bf16_round(rng.standard_normal((2, I, H)) * 0.5)
    dy2 = F.bf16_round(rng.standard_normal((T, H)))
    rs = F.bf16_round(rng.uniform(0.5, 1.5, T))
    bits = F.f64_to_bf16_bits
    ep = O.Epilogue(act=act, gated=False, bias=bits(b1), row_scale=rs)
    pre, y = O.fc1_glu(bits(x), counts, bits(w1), ep)
    off = [0, 3, 5]
    for e in range(2):
        for r in range(off[e], off[e + 1]):
            for j in range(I):
                z = sum(x[r, k] * w1[e, k, j] for k in range(H)) + b1[e, j]
                assert F.bf16_bits_to_f64(pre[r, j]) == z
                want = O.activation(np.array([z]), act, 1.0)[0] * rs[r]
                assert F.bf16_bits_to_f64(y[r, j]) == F.bf16_round(np.array([want]))[0]
    dz = F.bf16_bits_to_f64(O.dgrad_dact(bits(dy2), counts, bits(w2), pre, O.Epilogue(act=act, row_scale=rs)))
    z_all = F.bf16_bits_to_f64(pre)

    def loss(z):
        L = 0.0
        for e in range(2):
            a, b = off[e], off[e + 1]
            yy = O.activation(z[a:b], act, 1.0) * rs[a:b, None]
            L += float(np.sum(dy2[a:b] * (yy @ w2[e])))
        return L

    checked = 0
    for r in range(T):
        for j in range(I):
            if act == "srelu" and abs(z_all[r, j]) < 1e-3:
                continue
            h = 1e-6
            zp, zm = z_all.copy(), z_all.copy()
            zp[r, j] += h
            zm[r, j] -= h
            fd = (loss(zp) - loss(zm)) / (2 * h)
            assert abs(dz[r, j] - fd) <= 2.0 ** -8 * abs(fd) + 1e-6, (r, j, dz[r, j], fd)
            checked += 1
    assert checked >= 20


# ------------------------------------------------------------------ K-tiled copies, MXFP8 wgrad
def test_mx_cols_blocked_layout_matches_dense_blocks():
    """The K-tiled transposed copy holds the dense copy's blocks, each group
    from slot 4 sum_{j<e} ceil(m_j/128), one 32-byte slot per block, the codes
    of rows past a group zero, and its unused slots up to the next multiple of
    4 with zero codes and scale byte 127."""
    rng = np.random.default_rng(61)
    counts = [40, 0, 129, 5, 128]
    m_cap = 310
    v = W.to_bf16_bits((rng.standard_normal((m_cap, 6)) * 3).astype(np.float32))
    qd, sd = O.mx_quantize_cols(v, counts, m_cap=m_cap)
    qb, sb = O.mx_quantize_cols(v, counts, m_cap=m_cap, blocked=True)
    S = O.mx_col_slots(m_cap, len(counts), blocked=True)
    assert S == 4 * ((m_cap + 127) // 128 + len(counts)) and qb.shape == (6, 32 * S) and sb.shape == (6, S)
    so_d, so_b = O.mx_scale_col_offsets(counts), O.mx_scale_col_offsets(counts, blocked=True)
    assert so_b.tolist() == [0, 4, 4, 12, 16, 20]
    off = np.concatenate([[0], np.cumsum(counts)])
    for e, m in enumerate(counts):
        nb = (m + 31) // 32
        for b in range(nb):
            n = min(32, m - 32 * b)
            sl = so_b[e] + b
            assert np.array_equal(sb[:, sl], sd[:, so_d[e] + b])
            assert np.array_equal(qb[:, 32 * sl:32 * sl + n], qd[:, off[e] + 32 * b:off[e] + 32 * b + n])
            assert np.all(qb[:, 32 * sl + n:32 * sl + 32] == 0)
        for b in range(nb, so_b[e + 1] - so_b[e]):
            sl = so_b[e] + b
            assert np.all(sb[:, sl] == 127) and np.all(qb[:, 32 * sl:32 * sl + 32] == 0)


@pytest.mark.parametrize("blocked", [False, True])
def test_mx_dequantize_cols_round_trip_bound(blocked):
    rng = np.random.default_rng(62)
    counts = [70, 33, 0, 1]
    M = sum(counts)
    v = W.to_bf16_bits((rng.standard_normal((M, 5)) * 2.0 ** rng.integers(-8, 8, (M, 1))).astype(np.float32))
    q, s = O.mx_quantize_cols(v, counts, m_cap=M, blocked=blocked)
    d = O.mx_dequantize_cols(q, s, counts, M, blocked=blocked)
    x = F.bf16_bits_to_f64(v)
    so = O.mx_scale_col_offsets(counts, blocked)
    off = np.concatenate([[0], np.cumsum(counts)])
    for e in range(len(counts)):
        for r in range(off[e], off[e + 1]):
            X = F.e8m0_value(s[:, so[e] + (r - off[e]) // 32])
            assert np.all(np.abs(d[r] - x[r]) <= 0.5 * F.e4m3_ulp(np.abs(x[r]) / X) * X)


def test_wgrad_mx_exact_on_exactly_quantisable_inputs():
    """Small integers (|v| <= 7) are exact in e4m3 and e5m2 whatever the block
    scale the rule picks, so the MXFP8 weight gradient on their copies equals
    wgrad of the bf16 values exactly, for both layouts and both formats."""
    rng = np.random.default_rng(63)
    counts = [130, 0, 31, 64, 1]
    M, P, Q = sum(counts), 6, 5
    a = W.to_bf16_bits(rng.integers(-7, 8, (M, P)).astype(np.float32))
    b = W.to_bf16_bits(rng.integers(-7, 8, (M, Q)).astype(np.float32))
    ref = O.wgrad(a, counts, b)
    for blocked in (False, True):
        for fa, fb in (("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")):
            aq, as_ = O.mx_quantize_cols(a, counts, m_cap=M, fmt=fa, blocked=blocked)
            bq, bs = O.mx_quantize_cols(b, counts, m_cap=M, fmt=fb, blocked=blocked)
            got = O.wgrad_mx(aq, as_, bq, bs, counts, M, fa, fb, blocked=blocked)
            assert np.array_equal(got, ref), (blocked, fa, fb)


def test_wgrad_mx_against_loop_over_codes():
    """Gaussian values: each product term decoded from its own code and scale
    byte in a Python loop (slot arithmetic written out for the K-tiled
    layout)."""
    rng = np.random.default_rng(64)
    counts = [37, 0, 70]
    M, P, Q = sum(counts), 3, 4
    a = W.to_bf16_bits(rng.standard_normal((M, P)).astype(np.float32))
    b = W.to_bf16_bits((rng.standard_normal((M, Q)) * 1e-3).astype(np.float32))
    aq, as_ = O.mx_quantize_cols(a, counts, m_cap=M, blocked=True)
    bq, bs = O.mx_quantize_cols(b, counts, m_cap=M, fmt="e5m2", blocked=True)
    got = O.wgrad_mx(aq, as_, bq, bs, counts, M, "e4m3", "e5m2")
    starts = [0, 37, 37]
    slot0 = [0, 4, 4]
    for e in range(3):
        for p in range(P):
            for q in range(Q):
                s = 0.0
                for k in range(counts[e]):
                    sl = slot0[e] + k // 32
                    xa = F.e4m3_decode(aq[p, 32 * sl + k % 32]) * 2.0 ** (int(as_[p, sl]) - 127)
                    xb = F.e5m2_decode(bq[q, 32 * sl + k % 32]) * 2.0 ** (int(bs[q, sl]) - 127)
                    s += xa * xb
                assert got[e, p, q] == pytest.approx(s, rel=1e-12, abs=1e-300)
    assert np.all(got[1] == 0)
