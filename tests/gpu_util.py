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


def assert_bf16_close(gpu_bits, ref_bits, rtol=2e-2, what="", normwise=None, extra=None):
    """``extra``: an additional element-wise absolute bound (e.g. for sums
    whose hardware accumulation is not strict fp32)."""
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
    if normwise is not None:
        nr = np.linalg.norm(r)
        if nr > 0:
            rel = np.linalg.norm(g - r) / nr
            assert rel <= normwise, f"{what}: normwise relative error {rel:.3e} > {normwise}"
    return float(err.max()) if err.size else 0.0


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
    16 * (c ^ s(r)) bytes into the row, s(r) = (r % 8) ^ ((r // 8) % 4); rows
    past N are zero.  Returns uint16 [E * ceil(N/256)*256 * K]."""
    E, N, K = w_nk.shape
    NB, KB = (N + 255) // 256, K // 64
    pad = np.zeros((E, NB * 256, K), dtype=np.uint16)
    pad[:, :N] = w_nk
    out = np.zeros((E, NB, KB, 256, 8, 8), dtype=np.uint16)
    blocks = pad.reshape(E, NB, 256, KB, 8, 8).transpose(0, 1, 3, 2, 4, 5)  # e nb kb r c q
    r = np.arange(256)
    key = (r % 8) ^ ((r // 8) % 4)
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
    key = (r % 8) ^ ((r // 8) % 4)
    for c in range(8):
        out[:, :, :, r, c ^ key, :] = blocks[:, :, :, r, c, :]
    sc = sp.reshape(E, NB, 256, KB, 4).transpose(0, 1, 3, 2, 4)                # e nb kb r b
    return out.reshape(-1), np.ascontiguousarray(sc).reshape(-1)


def _mx_block_check(gq, gs, gv, rq, rs, rv, what, max_flip=0.02, fmt="e4m3"):
    """Blocks laid out as [..., nblk, 32] (codes, values) and [..., nblk] (scales).
    Blocks whose 32 source values are bit-identical on both sides must give
    identical bytes; the others (a bf16 rounding flip upstream) must still
    dequantise to within one element step (e4m3 or e5m2) of the oracle value
    plus the flip."""
    same = np.all(gv == rv, axis=-1)
    assert np.array_equal(gq[same], rq[same]), f"{what}: codes differ on identical blocks"
    assert np.array_equal(gs[same], rs[same]), f"{what}: scales differ on identical blocks"
    frac = 1.0 - same.mean() if same.size else 0.0
    assert frac <= max_flip, f"{what}: {frac:.3%} of blocks have different source values"
    if np.any(~same):
        scale = F.e8m0_value(gs[~same])[..., None]
        deq = F.fp8_decode(gq[~same], fmt) * scale
        ref = F.bf16_bits_to_f64(rv[~same])
        gval = F.bf16_bits_to_f64(gv[~same])
        ulp = F.e4m3_ulp if fmt == "e4m3" else F.e5m2_ulp
        bound = ulp(np.abs(ref) / scale) * scale + np.abs(gval - ref)
        assert np.all(np.abs(deq - ref) <= bound), f"{what}: flipped blocks out of bound"


def assert_mx_rows(gpu_q, gpu_s, gpu_vals, ref_vals, what="mx rows", max_flip=0.02, fmt="e4m3"):
    """Row-wise MXFP8 copy of a GPU bf16 tensor against the oracle's
    quantisation of the ORACLE's values (ref_vals); the GPU values only pick
    which blocks must match byte for byte.  max_flip bounds the fraction of
    blocks whose source values differ (a GEMM output whose bf16 rounding flips
    often, like dGLU's products, needs a large one)."""
    from oracle import moe as O
    rq, rs = O.mx_quantize_rows(ref_vals, fmt)
    R, C = ref_vals.shape
    nb = C // 32
    _mx_block_check(gpu_q.reshape(R, nb, 32), gpu_s.reshape(R, nb), gpu_vals.reshape(R, nb, 32),
                    rq.reshape(R, nb, 32), rs.reshape(R, nb), ref_vals.reshape(R, nb, 32), what,
                    max_flip, fmt)


def assert_mx_cols(gpu_q, gpu_s, gpu_vals, ref_vals, counts, m_cap, what="mx cols",
                   max_flip=0.02, fmt="e4m3"):
    """Transposed MXFP8 copy (32-row blocks restarting at each group) against
    the oracle's quantisation of the oracle's values, as in assert_mx_rows."""
    from oracle import moe as O
    rq, rs = O.mx_quantize_cols(ref_vals, counts, m_cap=m_cap, fmt=fmt)
    so = O.mx_scale_col_offsets(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    C = ref_vals.shape[1]
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

        gq = np.concatenate([gpu_q[:, a:b], np.zeros((C, pad), np.uint8)], axis=1).reshape(C, nb, 32)
        rqe = np.concatenate([rq[:, a:b], np.zeros((C, pad), np.uint8)], axis=1).reshape(C, nb, 32)
        _mx_block_check(gq, gpu_s[:, so[e]:so[e] + nb], blocks(gpu_vals[a:b]),
                        rqe, rs[:, so[e]:so[e] + nb], blocks(ref_vals[a:b]), f"{what} group {e}",
                        max_flip, fmt)
