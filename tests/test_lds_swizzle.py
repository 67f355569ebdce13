"""The 16-byte chunk key of the LDS operand tiles and of the packed weight
layout (include/moe_glu.h, s(r)) against gfx950's 16-byte LDS read passes
(CPU only).

A 16-byte read is served in four passes of 16 lanes over 64 banks of 4 bytes;
a pass takes the lanes that agree in lane bit 5 and in the parity of lane bits
2..4 (measured on the GPU with single-pair conflict probes).  The fragment
reads of both MFMA loops must then be conflict-free: the 16 x 16 x 32 loop
(lane: row bits 0..3 of a 16-row block, chunk bits 0..1) and the 32 x 32 loops
(lane: row bits 0..4 of a 32-row block, chunk bit 0; the block-scaled fp8 loop
reads chunk pairs (c, c + 2) the same way).  The first key, (r % 8) ^ ((r // 8)
% 4), fails the 16 x 16 check: that is the case the test guards.
"""
import numpy as np

from tests.gpu_util import packed_layout


def _passes():
    out = {}
    for l in range(64):
        out.setdefault(((l >> 5) & 1, bin((l >> 2) & 7).count("1") & 1), []).append(l)
    return list(out.values())


def _key_from_layout():
    """s(r) for r = 0..255, read back from the packed layout helper: row r's
    logical chunk 0 lands at physical chunk s(r)."""
    w = np.zeros((1, 256, 64), dtype=np.uint16)
    for c in range(8):
        w[0, :, 8 * c:8 * c + 8] = c + 1
    p = packed_layout(w).reshape(256, 8, 8)[:, :, 0]
    return np.array([int(np.nonzero(p[r] == 1)[0][0]) for r in range(256)])


def _extra_cycles(addr_of_lane):
    extra = 0
    for g in _passes():
        banks = {}
        for l in g:
            for d in range(4):
                w = addr_of_lane[l] // 4 + d
                banks.setdefault(w % 64, set()).add(w)
        extra += max(len(v) for v in banks.values()) - 1
    return extra


def _reads(key):
    off = lambda r, c: r * 128 + 16 * (c ^ int(key[r]))
    m16 = [[off(r0 + (l & 15), c0 + (l >> 4)) for l in range(64)] for r0 in range(0, 256, 16) for c0 in (0, 4)]
    m32 = [[off(r0 + (l & 31), c0 + (l >> 5)) for l in range(64)] for r0 in range(0, 256, 32) for c0 in range(0, 8, 2)]
    return m16, m32


def test_pass_model_reproduces_the_measured_ratios():
    """No swizzle: 0.75 (16 x 16) and 0.875 (32 x 32) conflict cycles per
    active cycle; the first key: 0.50 and 0.00 (the probe's figures)."""
    for key, want in ((np.zeros(256, dtype=int), (0.75, 0.875)),
                      (np.array([(r % 8) ^ ((r // 8) % 4) for r in range(256)]), (0.5, 0.0))):
        for reads, w in zip(_reads(key), want):
            extra = sum(_extra_cycles(a) for a in reads)
            ideal = 4 * len(reads)
            assert abs(extra / (extra + ideal) - w) < 1e-9


def test_layout_key_is_conflict_free_for_both_fragment_shapes():
    key = _key_from_layout()
    assert sorted(key[:8]) == list(range(8))
    m16, m32 = _reads(key)
    assert sum(_extra_cycles(a) for a in m16) == 0
    assert sum(_extra_cycles(a) for a in m32) == 0
