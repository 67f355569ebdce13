"""CPU tests of the GPU tests' own checkers (tests/gpu_util.py): they must
accept the oracle's own results and reject planted mistakes.  Mistakes are
planted in oracle outputs, on the CPU; nothing here touches a GPU.

The E8M0 rule checked is the acceptance rule for MXFP8 outputs: scales equal
the oracle's except where the block amax lies within one bf16 ulp of a
power-of-two boundary of the scale rule (amax = 448 * 2^k for e4m3, 57344 *
2^k for e5m2), where one step either way is allowed.
"""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import moe as O
from tests.gpu_util import (MX_ACC_REL, assert_bf16_close, assert_mx_cols, assert_mx_gemm_close,
                            assert_mx_rows, mx_boundary_exempt)


def _rows(seed, R=6, C=64, scale=3.0):
    g = np.random.default_rng(seed)
    return W.to_bf16_bits((g.standard_normal((R, C)) * scale).astype(np.float32))


def test_boundary_exemption_values():
    b = np.array([448.0, 446.0, 450.0, 444.0, 452.0, 896.0, 892.0, 900.0, 904.0, 224.0, 0.0, 6.5])
    ex = mx_boundary_exempt(b)
    assert ex.tolist() == [True, True, True, False, False, True, True, True, False, True, False, False]
    assert mx_boundary_exempt(np.array([57344.0, 57344.0 + 256.0, 57344.0 - 512.0]), "e5m2").tolist() \
        == [True, True, False]
    assert not mx_boundary_exempt(np.array([np.nan, np.inf])).any()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_oracle_against_itself_passes_all_exact(fmt):
    v = _rows(1)
    q, s = O.mx_quantize_rows(v, fmt)
    n, exact, ex = assert_mx_rows(q, s, v, v, "self", fmt=fmt)
    assert (n, exact, ex) == (v.size // 32, v.size // 32, 0)


def test_scale_one_step_off_away_from_boundary_fails():
    v = _rows(2)
    q, s = O.mx_quantize_rows(v)
    amax = np.max(np.abs(F.bf16_bits_to_f64(v).reshape(6, 2, 32)), axis=-1)
    assert not mx_boundary_exempt(amax[0, 0])
    s2 = s.copy()
    s2[0, 0] += 1
    with pytest.raises(AssertionError, match="E8M0 scales differ"):
        assert_mx_rows(q, s2, v, v, "planted scale")


def test_scale_off_on_flipped_block_fails_even_if_codes_fit():
    """A source flip elsewhere in the block does not license a scale change."""
    v = _rows(3)
    q, s = O.mx_quantize_rows(v)
    g = v.copy()
    g[1, 5] ^= np.uint16(1)                # a one-ulp flip of a non-maximal element
    gq, gs = O.mx_quantize_rows(g)
    gs = gs.copy()
    gs[1, 0] += 1
    with pytest.raises(AssertionError, match="E8M0 scales differ"):
        assert_mx_rows(gq, gs, g, v, "planted scale on flipped block")


def test_boundary_flip_is_exempt_and_counted():
    """Oracle amax exactly 448: the GPU's bf16 value one ulp above (450)
    moves its scale one step up; that is the only allowed scale change."""
    v = _rows(4, R=2, C=32, scale=0.5)
    v[0, 7] = F.f64_to_bf16_bits(np.array([448.0]))[0]
    g = v.copy()
    g[0, 7] = F.f64_to_bf16_bits(np.array([450.0]))[0]
    gq, gs = O.mx_quantize_rows(g)
    rq, rs = O.mx_quantize_rows(v)
    assert int(gs[0, 0]) == int(rs[0, 0]) + 1
    n, exact, ex = assert_mx_rows(gq, gs, g, v, "boundary")
    assert (n, ex) == (2, 1) and exact == 1
    # two steps off at the same block is still rejected
    gs2 = gs.copy()
    gs2[0, 0] += 1
    with pytest.raises(AssertionError):
        assert_mx_rows(gq, gs2, g, v, "boundary two steps")


def test_codes_off_by_two_steps_fail():
    v = _rows(5)
    q, s = O.mx_quantize_rows(v)
    g = v.copy()
    g[2, 40] ^= np.uint16(1)
    gq, gs = O.mx_quantize_rows(g)
    gq = gq.copy()
    gq[2, 41] = (int(gq[2, 41]) & 0x80) | min((int(gq[2, 41]) & 0x7F) + 2, 0x7E)
    with pytest.raises(AssertionError, match="out of bound"):
        assert_mx_rows(gq, gs, g, v, "planted codes")
    q2 = q.copy()
    q2[0, 0] ^= 1                           # identical sources: any code change fails
    with pytest.raises(AssertionError, match="identical blocks"):
        assert_mx_rows(q2, s, v, v, "planted code")


def test_column_copies_check_per_group():
    counts = [40, 0, 23]
    v = _rows(6, R=63, C=4)
    q, s = O.mx_quantize_cols(v, counts, m_cap=70)
    n, exact, ex = assert_mx_cols(q, s, v, v, counts, 70, "cols")
    assert (n, exact, ex) == (4 * (2 + 1), 12, 0)
    s2 = s.copy()
    s2[1, 1] += 1                           # group 0's second block, column 1
    with pytest.raises(AssertionError, match="E8M0 scales differ"):
        assert_mx_cols(q, s2, v, v, counts, 70, "planted col scale")


def test_mx_gemm_bound_rejects_accumulation_error_above_the_allowance():
    g = np.random.default_rng(7)
    counts = [5]
    a = W.to_bf16_bits(g.standard_normal((5, 64)).astype(np.float32))
    b = W.to_bf16_bits(g.standard_normal((1, 3, 64)).astype(np.float32))
    aq, as_ = O.mx_quantize_rows(a)
    bq, bs = O.mx_quantize_rows(b[0])
    bq, bs = bq[None], bs[None]
    ref = O.group_gemm_mx(aq, as_, counts, bq, bs)
    assert_mx_gemm_close(ref, ref, aq, as_, counts, bq, bs, "self")
    A = O.mx_dequantize_rows(aq, as_)
    B = O.mx_dequantize_rows(bq[0], bs[0])
    S = np.abs(A) @ np.abs(B).T
    # an error of 4 x the allowance beyond the element-wise bound is caught
    bad = F.bf16_bits_to_f64(ref).copy()
    bad[0, 0] += 2e-2 * (1 + abs(bad[0, 0])) + 4 * MX_ACC_REL * S[0, 0] + 1e-3 * S[0, 0]
    with pytest.raises(AssertionError, match="out of tolerance"):
        assert_mx_gemm_close(F.f64_to_bf16_bits(bad), ref, aq, as_, counts, bq, bs, "planted")


def test_normwise_bound_is_enforced():
    r = _rows(8, scale=1e-2)
    gvals = F.bf16_bits_to_f64(r) * (1 + 1e-2)
    with pytest.raises(AssertionError, match="normwise"):
        assert_bf16_close(F.f64_to_bf16_bits(gvals), r, normwise=4e-3)


def test_blocked_column_copies_check_and_padding():
    counts = [40, 0, 23]
    v = _rows(9, R=63, C=4)
    q, s = O.mx_quantize_cols(v, counts, m_cap=70, blocked=True)
    n, exact, ex = assert_mx_cols(q, s, v, v, counts, 70, "cols blocked", blocked=True)
    assert (n, exact, ex) == (4 * (2 + 1), 12, 0)
    q2 = q.copy()
    q2[0, 32 * 3 + 5] = 1                   # group 0's padding slot 3
    with pytest.raises(AssertionError, match="padding codes"):
        assert_mx_cols(q2, s, v, v, counts, 70, "planted padding", blocked=True)
    q3 = q.copy()
    q3[1, 32 * 1 + 8 + 3] = 2               # group 0 block 1 holds rows 32..39: byte 11 is past them
    with pytest.raises(AssertionError, match="past the rows"):
        assert_mx_cols(q3, s, v, v, counts, 70, "planted tail", blocked=True)
