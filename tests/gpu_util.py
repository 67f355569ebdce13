"""Shared helpers of the GPU parity tests: host<->device copies of bf16 bit
patterns, sentinels, and the tolerance checks.

Tolerance for bf16 outputs of fp32-accumulated GEMMs: |gpu - ref| <=
2e-2 * (1 + |ref|) element-wise, with ref the fp64 oracle rounded to bf16.
A normwise relative error is also checked against a tighter bound where the
values are small (the element-wise bound is loose when |ref| << 1).
"""
from __future__ import annotations

import numpy as np

from oracle import formats as F

BF16_NAN_SENTINEL = 0x7FC1      # a NaN payload no kernel produces
BYTE_SENTINEL = 0xA5


def torch():
    import torch as _t
    return _t


def dev_bits(a: np.ndarray):
    """uint16 numpy -> int16 cuda tensor (same bits)."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def dev_i32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def empty_bits(shape, sentinel=BF16_NAN_SENTINEL):
    t = torch()
    return t.full(shape, np.int16(np.uint16(sentinel).view(np.int16)), dtype=t.int16, device="cuda")


def empty_bytes(shape, sentinel=BYTE_SENTINEL):
    t = torch()
    return t.full(shape, sentinel, dtype=t.uint8, device="cuda")


def normwise_rel(gpu_bits, ref_bits) -> float:
    """||gpu - ref||_2 / ||ref||_2 over bf16 bit patterns (0 when ref is 0)."""
    g = F.bf16_bits_to_f64(gpu_bits)
    r = F.bf16_bits_to_f64(ref_bits)
    nr = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / nr) if nr > 0 else 0.0


def assert_bf16_close(gpu_bits, ref_bits, rtol=2e-2, what="", normwise=None, extra=None,
                      report=False):
    """``extra``: an additional element-wise absolute bound (e.g. for sums
    whose hardware accumulation is not strict fp32).  ``report`` prints the
    normwise relative error and the largest element error."""
    g = F.bf16_bits_to_f64(gpu_bits)
    r = F.bf16_bits_to_f64(ref_bits)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    err = np.abs(g - r)
    bound = rtol * (1.0 + np.abs(r))
    if extra is not None:
        bound = bound + extra
    bad = err > bound
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance, e.g. "
                             + ", ".join(f"{tuple(i)} gpu={g[tuple(i)]} ref={r[tuple(i)]}" for i in idx))
    rel = normwise_rel(gpu_bits, ref_bits)
    if report:
        print(f"[norm] {what}: normwise relative error {rel:.3e}, "
              f"max |err| {float(err.max()) if err.size else 0.0:.3e}")
    if normwise is not None:
        assert rel <= normwise, f"{what}: normwise relative error {rel:.3e} > {normwise}"
    return float(err.max()) if err.size else 0.0


# Element-wise allowance, as a multiple of sum_k |a_k b_k|, for the block-scaled
# MFMA's accumulation, which is not strict fp32: twice the largest deviation
# measured over every MXFP8-operand test beyond the output's own rounding
# (2^-13.18 sum|ab|: the MXFP8 weight gradient over a 1000-row group; FC1 with
# MXFP8 inputs reached 2^-13.72 at K = 256; each test prints its own).  A
# misplaced scale or K block errs by the order of sum|ab| itself.
MX_ACC_REL = 2.2e-4


def mx_gemm_terms(aq, as_, counts, bq, bs, a_fmt="e4m3", gpu_aq=None, gpu_as=None):
    """For an MXFP8 x MXFP8 GroupGemm out_e = deq(A_e) deq(B_e)^T computed by
    the oracle from its own codes (aq, as_; bq, bs with B [E][N][K]): per
    output element, S = sum_k |a_k b_k| and, when the GPU's product read other
    A codes (gpu_aq, gpu_as: a GPU-quantised input, checked on its own against
    the oracle's quantisation), D = sum_k |a'_k - a_k| |b_k|, the most those
    input differences can move the exact product.  Also returns the exact
    fp64 products from the oracle's codes.  Returns (S, D, exact)."""
    from oracle import moe as O
    counts = np.asarray(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M, N = int(off[-1]), bq.shape[1]
    S, D, X = np.zeros((M, N)), np.zeros((M, N)), np.zeros((M, N))
    for e in range(len(counts)):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        A = O.mx_dequantize_rows(aq[a:b], as_[a:b], a_fmt)
        B = O.mx_dequantize_rows(bq[e], bs[e])
        S[a:b] = np.abs(A) @ np.abs(B).T
        X[a:b] = A @ B.T
        if gpu_aq is not None:
            Ag = O.mx_dequantize_rows(gpu_aq[a:b], gpu_as[a:b], a_fmt)
            D[a:b] = np.abs(Ag - A) @ np.abs(B).T
    return S, D, X


def mx_acc_excess(gpu_bits, S, D, X, what=""):
    """The largest accumulation deviation of a block-scaled product, as a
    multiple of sum |a b|: (|gpu - exact| - half a bf16 ulp - D) / S, printed
    as a power of two."""
    g = F.bf16_bits_to_f64(gpu_bits)
    mag = np.maximum(np.abs(g), np.abs(X))
    half_ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 8), 0.0)
    ex = np.maximum(np.abs(g - X) - half_ulp - D, 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(S > 0, ex / S, 0.0)
    m = float(r.max()) if r.size else 0.0
    at = ""
    if m > 0:
        i = np.unravel_index(np.argmax(r), r.shape)
        at = f" (there sum|ab| / |exact| = {S[i] / max(abs(X[i]), 1e-300):.3g})"
    print(f"[mx-acc] {what}: max accumulation deviation "
          + (f"2^{np.log2(m):.2f}" if m > 0 else "0") + " of sum|ab|" + at)
    return m


def assert_mx_gemm_close(gpu_bits, ref_bits, aq, as_, counts, bq, bs, what, a_fmt="e4m3",
                         gpu_aq=None, gpu_as=None, normwise=None):
    """An MXFP8 x MXFP8 product against the oracle's: |gpu - ref| <= 2e-2 (1 +
    |ref|) + MX_ACC_REL S + D (mx_gemm_terms); prints the measured
    accumulation deviation."""
    S, D, X = mx_gemm_terms(aq, as_, counts, bq, bs, a_fmt, gpu_aq, gpu_as)
    mx_acc_excess(gpu_bits, S, D, X, what)
    return assert_bf16_close(gpu_bits, ref_bits, what=what, normwise=normwise,
                             extra=MX_ACC_REL * S + D)


def sample_rows(counts, per_group=2, seed=0, max_rows=64):
    """Grouped rows to check one by one: first, last and random rows of groups."""
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(counts)])
    rows = []
    for e in range(len(counts)):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        pick = {a, b - 1}
        pick.update(rng.integers(a, b, size=per_group).tolist())
        rows.extend(sorted(pick))
    rows = np.array(sorted(set(rows)))
    if len(rows) > max_rows:
        keep = np.concatenate([rows[:8], rows[-8:], rng.choice(rows[8:-8], max_rows - 16, replace=False)])
        rows = np.array(sorted(set(keep.tolist())))
    return rows


def expert_of_rows(counts, rows):
    off = np.concatenate([[0], np.cumsum(counts)])
    return np.searchsorted(off, rows, side="right") - 1


def packed_layout(w_nk: np.ndarray) -> np.ndarray:
    """The tile-blocked weight format documented in include/moe_glu.h, written
    out in numpy from its definition: per expert [N][K] -> blocks of 256 rows x
    64 columns, block (nb, kb) at (nb * K/64 + kb) * 16384, chunk c of row r at
    16 * (c ^ s(r)) bytes into the row, s(r) = (r % 8) ^ (2 ((r // 8) % 2) + (r // 16) % 2); rows
    past N are zero.  Returns uint16 [E * ceil(N/256)*256 * K]."""
    E, N, K = w_nk.shape
    NB, KB = (N + 255) // 256, K // 64
    pad = np.zeros((E, NB * 256, K), dtype=np.uint16)
    pad[:, :N] = w_nk
    out = np.zeros((E, NB, KB, 256, 8, 8), dtype=np.uint16)
    blocks = pad.reshape(E, NB, 256, KB, 8, 8).transpose(0, 1, 3, 2, 4, 5)  # e nb kb r c q
    r = np.arange(256)
    key = (r % 8) ^ (2 * ((r // 8) % 2) + (r // 16) % 2)
    for c in range(8):
        out[:, :, :, r, c ^ key, :] = blocks[:, :, :, r, c, :]
    return out.reshape(-1)



def dev_bytes(a: np.ndarray):
    """uint8 numpy -> uint8 cuda tensor."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def packed_mx_layout(q_nk: np.ndarray, s_nk: np.ndarray):
    """The MXFP8 weight format documented in include/moe_glu.h, written out in
    numpy from its definition: codes [E][N][K] -> blocks of 256 rows x 128
    bytes, block (nb, kb) at (nb * K/128 + kb) * 32768, chunk c of row r at
    16 * (c ^ s(r)); scales [E][N][K/32] -> one dword per (nb, kb, r) holding
    the row's four block scales of that K-tile.  Rows past N are zero."""
    E, N, K = q_nk.shape
    NB, KB = (N + 255) // 256, K // 128
    qp = np.zeros((E, NB * 256, K), dtype=np.uint8)
    qp[:, :N] = q_nk
    sp = np.zeros((E, NB * 256, K // 32), dtype=np.uint8)
    sp[:, :N] = s_nk
    blocks = qp.reshape(E, NB, 256, KB, 8, 16).transpose(0, 1, 3, 2, 4, 5)   # e nb kb r c b
    out = np.zeros((E, NB, KB, 256, 8, 16), dtype=np.uint8)
    r = np.arange(256)
    key = (r % 8) ^ (2 * ((r // 8) % 2) + (r // 16) % 2)
    for c in range(8):
        out[:, :, :, r, c ^ key, :] = blocks[:, :, :, r, c, :]
    sc = sp.reshape(E, NB, 256, KB, 4).transpose(0, 1, 3, 2, 4)                # e nb kb r b
    return out.reshape(-1), np.ascontiguousarray(sc).reshape(-1)


MX_ELEM_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def mx_boundary_exempt(amax, fmt="e4m3"):
    """True where a block amax lies within one bf16 ulp of a scale boundary
    MAX * 2^k (MAX = the element format's largest value: the scale rule moves
    to the next power of two there), the only place where the E8M0 scale of a
    block may differ from the oracle's."""
    a = np.asarray(amax, dtype=np.float64)
    out = np.zeros(a.shape, dtype=bool)
    pos = np.isfinite(a) & (a > 0)
    m = MX_ELEM_MAX[fmt]
    k = np.round(np.log2(a[pos] / m))
    b = m * np.exp2(k)
    ulp = np.exp2(np.floor(np.log2(b)) - 7)          # bf16: 8 significant bits
    out[pos] = np.abs(a[pos] - b) <= ulp
    return out


def _mx_block_check(gq, gs, gv, rq, rs, rv, what, fmt="e4m3"):
    """MXFP8 blocks laid out as [..., nblk, 32] (codes, bf16 source values) and
    [..., nblk] (scale bytes), GPU (g*) against the oracle's quantisation of
    the oracle's values (r*).

    * Scales: every block's E8M0 byte equals the oracle's, except where the
      oracle block's amax is within one bf16 ulp of a scale boundary
      (mx_boundary_exempt); there it may be one step off.
    * Codes: byte for byte on blocks whose 32 source values are bit-identical
      on both sides; elsewhere (a bf16 rounding flip upstream) the GPU's
      dequantised value is within one element step at the ORACLE's scale,
      plus the flip, of the oracle's value.

    Returns (blocks, byte-exact blocks, scale exemptions used)."""
    rvals = F.bf16_bits_to_f64(rv)
    gvals = F.bf16_bits_to_f64(gv)
    same = np.all(gv == rv, axis=-1)
    assert np.array_equal(gq[same], rq[same]), f"{what}: codes differ on identical blocks"
    gsi, rsi = gs.astype(np.int64), rs.astype(np.int64)
    diff = gsi != rsi
    if np.any(diff):
        amax = np.max(np.abs(rvals), axis=-1)
        ex = mx_boundary_exempt(amax, fmt)
        bad = diff & ~(ex & (np.abs(gsi - rsi) == 1))
        if np.any(bad):
            idx = np.argwhere(bad)[:5]
            raise AssertionError(
                f"{what}: {int(bad.sum())} E8M0 scales differ from the oracle away from a boundary, e.g. "
                + ", ".join(f"{tuple(i)} gpu={int(gsi[tuple(i)])} ref={int(rsi[tuple(i)])} "
                            f"amax={amax[tuple(i)]}" for i in idx))
    if np.any(~same):
        xr = F.e8m0_value(rs[~same])[..., None]
        deq = F.fp8_decode(gq[~same], fmt) * F.e8m0_value(gs[~same])[..., None]
        ref, gval = rvals[~same], gvals[~same]
        ulp = F.e4m3_ulp if fmt == "e4m3" else F.e5m2_ulp
        bound = ulp(np.abs(ref) / xr) * xr + np.abs(gval - ref)
        assert np.all(np.abs(deq - ref) <= bound), f"{what}: dequantised values out of bound"
    exact = int(np.sum(np.all(gq == rq, axis=-1) & ~diff))
    return int(same.size), exact, int(np.sum(diff))


def _report_mx(what, stats):
    n, exact, ex = stats
    print(f"[mx] {what}: {n} blocks, {exact / max(n, 1):.2%} byte-exact, "
          f"{ex} scale(s) one step off at a boundary")


def assert_mx_rows(gpu_q, gpu_s, gpu_vals, ref_vals, what="mx rows", fmt="e4m3"):
    """Row-wise MXFP8 copy of a GPU bf16 tensor against the oracle's
    quantisation of the ORACLE's values (ref_vals); the GPU values only pick
    which blocks must match byte for byte (_mx_block_check)."""
    from oracle import moe as O
    rq, rs = O.mx_quantize_rows(ref_vals, fmt)
    R, C = ref_vals.shape
    nb = C // 32
    st = _mx_block_check(gpu_q.reshape(R, nb, 32), gpu_s.reshape(R, nb), gpu_vals.reshape(R, nb, 32),
                         rq.reshape(R, nb, 32), rs.reshape(R, nb), ref_vals.reshape(R, nb, 32), what,
                         fmt)
    _report_mx(what, st)
    return st


def assert_mx_cols(gpu_q, gpu_s, gpu_vals, ref_vals, counts, m_cap, what="mx cols", fmt="e4m3",
                   blocked=False):
    """Transposed MXFP8 copy (32-row blocks restarting at each group) against
    the oracle's quantisation of the oracle's values, as in assert_mx_rows.
    ``blocked``: the K-tiled layout, whose zero codes past a group's rows and
    padding slots (zero codes, scale byte 127) must match exactly."""
    from oracle import moe as O
    rq, rs = O.mx_quantize_cols(ref_vals, counts, m_cap=m_cap, fmt=fmt, blocked=blocked)
    so = O.mx_scale_col_offsets(counts, blocked)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    C = ref_vals.shape[1]
    tot = np.zeros(3, dtype=np.int64)
    for e in range(len(counts)):
        a, b = int(off[e]), int(off[e + 1])
        m = b - a
        if m == 0:
            continue
        nb = (m + 31) // 32
        pad = nb * 32 - m

        def blocks(v):   # [m][C] -> [C][nb][32], the tail padded with equal zeros
            t = np.concatenate([v, np.zeros((pad, C), v.dtype)]) if pad else v
            return t.T.reshape(C, nb, 32)

        if blocked:
            s0 = int(so[e])
            gq = gpu_q[:, 32 * s0:32 * (s0 + nb)].reshape(C, nb, 32)
            rqe = rq[:, 32 * s0:32 * (s0 + nb)].reshape(C, nb, 32)
            assert np.all(gq[:, -1, 32 - pad:] == 0) if pad else True, f"{what} group {e}: codes past the rows"
            s1 = int(so[e + 1])
            assert np.array_equal(gpu_s[:, s0 + nb:s1], rs[:, s0 + nb:s1]), f"{what} group {e}: padding scales"
            assert np.all(gpu_q[:, 32 * (s0 + nb):32 * s1] == 0), f"{what} group {e}: padding codes"
        else:
            gq = np.concatenate([gpu_q[:, a:b], np.zeros((C, pad), np.uint8)], axis=1).reshape(C, nb, 32)
            rqe = np.concatenate([rq[:, a:b], np.zeros((C, pad), np.uint8)], axis=1).reshape(C, nb, 32)
        tot += _mx_block_check(gq, gpu_s[:, so[e]:so[e] + nb], blocks(gpu_vals[a:b]),
                               rqe, rs[:, so[e]:so[e] + nb], blocks(ref_vals[a:b]), f"{what} group {e}",
                               fmt)
    st = tuple(int(v) for v in tot)
    _report_mx(what, st)
    return st
