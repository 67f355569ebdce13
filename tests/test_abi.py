"""The C-ABI library loads, exports every entry point include/moe_glu.h
declares, and rejects bad arguments before launching anything (these calls
return on the host; no GPU is touched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_glu.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status_t|size_t|const char\*)\s+(moe_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("moe_repack_gate_up", "moe_group_gemm_glu_fwd", "moe_group_gemm_dglu_bwd",
              "moe_group_gemm_quant"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import grouped_gemm_glu_amd as G
    lib = ctypes.CDLL(G.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared()) == set(G.EXPORTED)


def test_status_strings():
    import grouped_gemm_glu_amd as G
    for s in range(7):
        assert G.raw_call("moe_status_string", s)
    assert G.moe_packed_w1_bytes(32, 7168, 2048) == 32 * 4096 * 7168 * 2
    assert G.moe_packed_w1_bytes(0, 1, 1) == 0


def test_host_argument_errors_return_before_launch():
    import grouped_gemm_glu_amd as G
    NULL = None
    ep = G.epilogue()
    fake = 1 << 20                         # never dereferenced: checks fail first
    grp = G.GroupsT(fake, 4, 1024, None, None)
    # unfused dGLU: null, shape, alignment, the non-gated form
    assert G.raw_call("moe_dglu_unfused", NULL, fake, ctypes.byref(grp), 256, ctypes.byref(ep),
                      fake, NULL) == 1
    assert G.raw_call("moe_dglu_unfused", fake, fake, ctypes.byref(grp), 100, ctypes.byref(ep),
                      fake, NULL) == 2
    assert G.raw_call("moe_dglu_unfused", fake + 2, fake, ctypes.byref(grp), 256,
                      ctypes.byref(ep), fake, NULL) == 3
    ep_plain = G.epilogue("srelu", gated=False)
    assert G.raw_call("moe_dglu_unfused", fake, fake, ctypes.byref(grp), 256,
                      ctypes.byref(ep_plain), fake, NULL) == 4
    # null required pointers
    assert G.raw_call("moe_group_gemm_glu_fwd", NULL, ctypes.byref(grp), fake, 256, 512,
                      ctypes.byref(ep), NULL, NULL, NULL, 0, NULL) == 1
    bad_grp = G.GroupsT(None, 4, 1024, None, None)
    assert G.raw_call("moe_group_gemm_glu_fwd", fake, ctypes.byref(bad_grp), fake, 256, 512,
                      ctypes.byref(ep), NULL, NULL, NULL, 0, NULL) == 1
    # shapes: I not a multiple of 64, H not a multiple of 64, E out of range
    assert G.raw_call("moe_group_gemm_glu_fwd", fake, ctypes.byref(grp), fake, 256, 500,
                      ctypes.byref(ep), NULL, NULL, NULL, 0, NULL) == 2
    assert G.raw_call("moe_group_gemm_glu_fwd", fake, ctypes.byref(grp), fake, 200, 512,
                      ctypes.byref(ep), NULL, NULL, NULL, 0, NULL) == 2
    grp_e = G.GroupsT(fake, 2000, 1024, None, None)
    assert G.raw_call("moe_group_gemm_glu_fwd", fake, ctypes.byref(grp_e), fake, 256, 512,
                      ctypes.byref(ep), NULL, NULL, NULL, 0, NULL) == 2
    # misaligned operand
    assert G.raw_call("moe_group_gemm_glu_fwd", fake + 2, ctypes.byref(grp), fake, 256, 512,
                      ctypes.byref(ep), NULL, NULL, NULL, 0, NULL) == 3
    # gated must be 0 (non-gated form) or 1
    ep_bad = G.epilogue()
    ep_bad.gated = 2
    assert G.raw_call("moe_group_gemm_glu_fwd", fake, ctypes.byref(grp), fake, 256, 512,
                      ctypes.byref(ep_bad), NULL, NULL, NULL, 0, NULL) == 4
    # the non-gated backward has no parameter gradients
    ep_ng = G.epilogue(gated=False, dbias_out=fake)
    w2op = G.operand(fake, layout=G.B_PACKED)
    assert G.raw_call("moe_group_gemm_dglu_bwd", fake, ctypes.byref(w2op), 256, 512, ctypes.byref(grp),
                      fake, ctypes.byref(ep_ng), fake, NULL, 0, NULL) == 4
    # MX outputs must come in (q, s) pairs
    mx = G.mx_out(row_q=fake)
    assert G.raw_call("moe_group_gemm_glu_fwd", fake, ctypes.byref(grp), fake, 256, 512,
                      ctypes.byref(ep), NULL, NULL, ctypes.byref(mx), 0, NULL) == 1
    # repack shapes
    assert G.raw_call("moe_repack_gate_up", fake, 4, 256, 96, fake, NULL) == 2
    assert G.raw_call("moe_repack_gate_up", NULL, 4, 256, 128, fake, NULL) == 1
    # quant: N not a multiple of 64
    a = G.operand(fake)
    b = G.operand(fake, layout=G.B_KN)
    assert G.raw_call("moe_group_gemm_quant", ctypes.byref(a), ctypes.byref(b), 100, 256,
                      ctypes.byref(grp), NULL, NULL, 0, NULL) == 2
    # routing: both or neither of logits / ids
    assert G.raw_call("moe_route_group", NULL, NULL, 8, 4, 2, fake, fake, fake, fake, fake,
                      NULL, 0, NULL, NULL) == 1
    assert G.raw_call("moe_route_group", fake, NULL, 8, 4, 5, fake, fake, fake, fake, fake,
                      NULL, 0, NULL, NULL) == 2
    # dgrad needs the saved pre-activation
    w2op = G.operand(fake, layout=G.B_PACKED)
    assert G.raw_call("moe_group_gemm_dglu_bwd", fake, ctypes.byref(w2op), 256, 512,
                      ctypes.byref(grp), NULL, ctypes.byref(ep), fake, NULL, 0, NULL) == 1
    # dgrad's W2 may be plain [N][K] or packed, not [K][N]
    w2kn = G.operand(fake, layout=G.B_KN)
    assert G.raw_call("moe_group_gemm_dglu_bwd", fake, ctypes.byref(w2kn), 256, 512,
                      ctypes.byref(grp), fake, ctypes.byref(ep), fake, NULL, 0, NULL) == 4
    # weight packing: K and N multiples of 64, source layout plain
    assert G.raw_call("moe_pack_weight", fake, 2, 256, 96, G.B_NK, fake, NULL) == 2
    assert G.raw_call("moe_pack_weight", fake, 2, 100, 128, G.B_NK, fake, NULL) == 2
    assert G.raw_call("moe_pack_weight", fake, 2, 256, 128, G.B_PACKED, fake, NULL) == 4
    assert G.raw_call("moe_pack_weight", fake + 2, 2, 256, 128, G.B_KN, fake, NULL) == 3
    # MXFP8 weight pack: K a multiple of 128
    assert G.raw_call("moe_pack_weight_mx", fake, 2, 256, 192, G.B_KN, fake, fake, NULL) == 2
    assert G.raw_call("moe_pack_weight_mx", fake, 2, 256, 256, G.B_KN, fake, NULL, NULL) == 1
    assert G.moe_packed_mx_weight_bytes(2, 300, 256) == 2 * 512 * 256
    assert G.moe_packed_mx_scale_bytes(2, 300, 256) == 2 * 512 * 8
    # MXFP8 GroupGemm: both operands MXFP8, B packed, scales present, K % 128 == 0
    amx = G.operand(fake, dtype=G.DT_MXFP8, scales=fake)
    bmx = G.operand(fake, dtype=G.DT_MXFP8, layout=G.B_PACKED, scales=fake)
    bbf = G.operand(fake, layout=G.B_PACKED)
    bmx_kn = G.operand(fake, dtype=G.DT_MXFP8, layout=G.B_KN, scales=fake)
    bmx_ns = G.operand(fake, dtype=G.DT_MXFP8, layout=G.B_PACKED)
    args = (256, 256, ctypes.byref(grp), fake, NULL, 0, NULL)
    assert G.raw_call("moe_group_gemm_quant", ctypes.byref(amx), ctypes.byref(bbf), *args) == 4
    assert G.raw_call("moe_group_gemm_quant", ctypes.byref(amx), ctypes.byref(bmx_kn), *args) == 4
    assert G.raw_call("moe_group_gemm_quant", ctypes.byref(amx), ctypes.byref(bmx_ns), *args) == 1
    assert G.raw_call("moe_group_gemm_quant", ctypes.byref(amx), ctypes.byref(bmx), 256, 192,
                      ctypes.byref(grp), fake, NULL, 0, NULL) == 2
    # packed sizes: experts padded to 256 rows
    assert G.moe_packed_weight_bytes(3, 300, 128) == 3 * 512 * 128 * 2
    assert G.moe_packed_w1_bytes(2, 192, 64) == 2 * 256 * 192 * 2
    assert G.moe_packed_weight_bytes(0, 256, 64) == 0
    # MXFP8 quantize: C not a multiple of 32
    mx2 = G.mx_out(row_q=fake, row_s=fake)
    assert G.raw_call("moe_mxfp8_quantize", fake, 64, 48, NULL, ctypes.byref(mx2), NULL) == 2
