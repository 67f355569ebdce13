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
