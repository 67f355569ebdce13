"""Python binding of libmoeglu, the MI355X (gfx950) MoE GroupGEMM + GLU library.

Argument marshalling only: every entry point forwards device pointers and
sizes to the C ABI declared in include/moe_glu.h, with the same names.  Tensors
are torch tensors used purely as device memory; the stream defaults to torch's
current stream.  There is no CPU or PyTorch fallback: if the HIP library is
missing, importing this package fails.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeglu.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python grouped_gemm_glu_amd/build.py` (needs hipcc)")

_lib = ctypes.CDLL(LIB_PATH)

# ----------------------------------------------------------------------------- ABI mirror
MOE_OK = 0
ACT = {"swiglu": 0, "geglu": 1, "geglu_tanh": 2, "srelu": 3}
DT_BF16, DT_MXFP8, DT_MXFP8_E5M2 = 0, 1, 2
B_KN, B_NK, B_PACKED = 0, 1, 2


class EpilogueT(ctypes.Structure):
    _fields_ = [("act", ctypes.c_int32), ("gated", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("gate_lo", ctypes.c_float), ("gate_hi", ctypes.c_float),
                ("up_lo", ctypes.c_float), ("up_hi", ctypes.c_float),
                ("up_offset", ctypes.c_float), ("bias", ctypes.c_void_p),
                ("row_scale", ctypes.c_void_p), ("amax_out", ctypes.c_void_p),
                ("rht_signs", ctypes.c_uint32), ("dbias_out", ctypes.c_void_p),
                ("drow_scale_out", ctypes.c_void_p)]


class MxOutT(ctypes.Structure):
    _fields_ = [("row_q", ctypes.c_void_p), ("row_s", ctypes.c_void_p),
                ("col_q", ctypes.c_void_p), ("col_s", ctypes.c_void_p), ("e5m2", ctypes.c_int32),
                ("col_blocked", ctypes.c_int32)]


class GroupsT(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("E", ctypes.c_int32), ("M_cap", ctypes.c_int32),
                ("offsets_out", ctypes.c_void_p), ("status_out", ctypes.c_void_p)]


class OperandT(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "moe_init": ([_I], _I),
    "moe_status_string": ([_I], ctypes.c_char_p),
    "moe_packed_w1_bytes": ([_I, _I, _I], ctypes.c_size_t),
    "moe_packed_weight_bytes": ([_I, _I, _I], ctypes.c_size_t),
    "moe_pack_weight": ([_P, _I, _I, _I, _I, _P, _P], _I),
    "moe_packed_mx_weight_bytes": ([_I, _I, _I], ctypes.c_size_t),
    "moe_packed_mx_scale_bytes": ([_I, _I, _I], ctypes.c_size_t),
    "moe_pack_weight_mx": ([_P, _I, _I, _I, _I, _P, _P, _P], _I),
    "moe_repack_gate_up_mx": ([_P, _I, _I, _I, _P, _P, _P], _I),
    "moe_group_gemm_glu_fwd_mx": ([ctypes.POINTER(OperandT), ctypes.POINTER(GroupsT),
                                   ctypes.POINTER(OperandT), _I, _I, ctypes.POINTER(EpilogueT), _P,
                                   _P, ctypes.POINTER(MxOutT), _I, _P], _I),
    "moe_repack_gate_up": ([_P, _I, _I, _I, _P, _P], _I),
    "moe_unpack_gate_up": ([_P, _I, _I, _I, _P, _P], _I),
    "moe_route_group": ([_P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P], _I),
    "moe_group_gemm_glu_fwd": ([_P, ctypes.POINTER(GroupsT), _P, _I, _I,
                                ctypes.POINTER(EpilogueT), _P, _P, ctypes.POINTER(MxOutT), _I, _P], _I),
    "moe_group_gemm_dglu_bwd": ([_P, ctypes.POINTER(OperandT), _I, _I, ctypes.POINTER(GroupsT), _P,
                                 ctypes.POINTER(EpilogueT), _P, ctypes.POINTER(MxOutT), _I, _P], _I),
    "moe_group_gemm_quant": ([ctypes.POINTER(OperandT), ctypes.POINTER(OperandT), _I, _I,
                              ctypes.POINTER(GroupsT), _P, ctypes.POINTER(MxOutT), _I, _P], _I),
    "moe_group_gemm_wgrad": ([_P, _P, _I, _I, ctypes.POINTER(GroupsT), _P, _I, _I, _P], _I),
    "moe_group_gemm_wgrad_mx": ([ctypes.POINTER(OperandT), ctypes.POINTER(OperandT), _I, _I,
                                 ctypes.POINTER(GroupsT), _P, _I, _I, _P], _I),
    "moe_glu_unfused": ([_P, ctypes.POINTER(GroupsT), _I, ctypes.POINTER(EpilogueT), _P, _P], _I),
    "moe_dglu_unfused": ([_P, _P, ctypes.POINTER(GroupsT), _I, ctypes.POINTER(EpilogueT), _P, _P], _I),
    "moe_mxfp8_quantize": ([_P, _I, _I, ctypes.POINTER(GroupsT), ctypes.POINTER(MxOutT), _P], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.moe_status_string(status).decode()
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


def _check(fn: str, st: int):
    if st != MOE_OK:
        raise MoeError(fn, st)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------------------- helpers
# The struct builders hold references to the tensors whose addresses they
# store, so a tensor cannot be freed (and its memory reused) while a struct
# that points at it is alive.
def _keep(struct, *objs):
    struct._keep = objs
    return struct


def epilogue(act: str = "swiglu", alpha: float = 1.0, gate_lo: float = -math.inf,
             gate_hi: float = math.inf, up_lo: float = -math.inf, up_hi: float = math.inf,
             up_offset: float = 0.0, bias=None, row_scale=None, gated: bool = True,
             amax_out=None, rht_signs: int = 0, dbias_out=None,
             drow_scale_out=None) -> EpilogueT:
    """Builds the moe_epilogue_t struct; ``bias`` is plain-order bf16 [E][2I];
    ``amax_out`` a one-element float32 device tensor raised to the output's
    amax (forward) or to the amax of its 16-row Hadamard rotation (dGLU
    backward, row signs from the low 16 bits of ``rht_signs``);
    ``dbias_out`` float32 [E][2I] and ``drow_scale_out`` float32 [M_cap]
    (dGLU backward) are added to."""
    return _keep(EpilogueT(ACT[act], 1 if gated else 0, alpha, gate_lo, gate_hi, up_lo, up_hi,
                           up_offset, _ptr(bias), _ptr(row_scale), _ptr(amax_out),
                           rht_signs & 0xFFFF, _ptr(dbias_out), _ptr(drow_scale_out)),
                 bias, row_scale, amax_out, dbias_out, drow_scale_out)


def groups(counts, M_cap: int, offsets_out=None, status_out=None) -> GroupsT:
    return _keep(GroupsT(_ptr(counts), int(counts.numel()), int(M_cap), _ptr(offsets_out),
                         _ptr(status_out)), counts, offsets_out, status_out)


def mx_out(row_q=None, row_s=None, col_q=None, col_s=None, e5m2: bool = False,
           col_blocked: bool = False) -> MxOutT:
    """MXFP8 output buffers; ``e5m2`` selects e5m2 element codes (gradients);
    ``col_blocked`` the K-tiled layout of the transposed copy."""
    return _keep(MxOutT(_ptr(row_q), _ptr(row_s), _ptr(col_q), _ptr(col_s), 1 if e5m2 else 0,
                        1 if col_blocked else 0), row_q, row_s, col_q, col_s)


def mx_col_slots(M_cap: int, E: int, blocked: bool = False) -> int:
    """Scale columns of a transposed MXFP8 copy (row length of col_s); the
    codes of the blocked layout take 32 bytes per slot."""
    return 4 * ((M_cap + 127) // 128 + E) if blocked else (M_cap + 31) // 32 + E


def operand(data, dtype: int = DT_BF16, layout: int = 0, scales=None) -> OperandT:
    return _keep(OperandT(dtype, layout, _ptr(data), _ptr(scales)), data, scales)


def _ref(x):
    return None if x is None else ctypes.byref(x)


# ----------------------------------------------------------------------------- entry points
def moe_init(device: int = 0):
    _check("moe_init", _lib.moe_init(device))


def moe_packed_w1_bytes(E: int, H: int, I: int) -> int:
    return _lib.moe_packed_w1_bytes(E, H, I)


def moe_packed_weight_bytes(E: int, N: int, K: int) -> int:
    return _lib.moe_packed_weight_bytes(E, N, K)


def moe_pack_weight(src, E, N, K, src_layout, dst, stream=None):
    _check("moe_pack_weight",
           _lib.moe_pack_weight(_ptr(src), E, N, K, src_layout, _ptr(dst), _stream(stream)))


def moe_packed_mx_weight_bytes(E: int, N: int, K: int) -> int:
    return _lib.moe_packed_mx_weight_bytes(E, N, K)


def moe_packed_mx_scale_bytes(E: int, N: int, K: int) -> int:
    return _lib.moe_packed_mx_scale_bytes(E, N, K)


def moe_pack_weight_mx(src, E, N, K, src_layout, dst_q, dst_s, stream=None):
    _check("moe_pack_weight_mx",
           _lib.moe_pack_weight_mx(_ptr(src), E, N, K, src_layout, _ptr(dst_q), _ptr(dst_s),
                                   _stream(stream)))


def moe_repack_gate_up_mx(w1, E, H, I, dst_q, dst_s, stream=None):
    _check("moe_repack_gate_up_mx",
           _lib.moe_repack_gate_up_mx(_ptr(w1), E, H, I, _ptr(dst_q), _ptr(dst_s), _stream(stream)))


def moe_group_gemm_glu_fwd_mx(xg: OperandT, grp: GroupsT, w1: OperandT, H, I, ep: EpilogueT, y=None,
                              preact=None, mx: Optional[MxOutT] = None, cu_margin: int = 0,
                              stream=None):
    _check("moe_group_gemm_glu_fwd_mx",
           _lib.moe_group_gemm_glu_fwd_mx(ctypes.byref(xg), ctypes.byref(grp), ctypes.byref(w1), H, I,
                                          ctypes.byref(ep), _ptr(y), _ptr(preact), _ref(mx),
                                          cu_margin, _stream(stream)))


def moe_repack_gate_up(w1, E, H, I, w1_packed, stream=None):
    _check("moe_repack_gate_up",
           _lib.moe_repack_gate_up(_ptr(w1), E, H, I, _ptr(w1_packed), _stream(stream)))


def moe_unpack_gate_up(w1_packed, E, H, I, w1, stream=None):
    _check("moe_unpack_gate_up",
           _lib.moe_unpack_gate_up(_ptr(w1_packed), E, H, I, _ptr(w1), _stream(stream)))


def moe_route_group(logits, topk_ids, T, E, k, topk_ids_out, counts, offsets, dst, src,
                    x=None, H=0, xg=None, stream=None):
    _check("moe_route_group",
           _lib.moe_route_group(_ptr(logits), _ptr(topk_ids), T, E, k, _ptr(topk_ids_out),
                                _ptr(counts), _ptr(offsets), _ptr(dst), _ptr(src), _ptr(x), H,
                                _ptr(xg), _stream(stream)))


def moe_group_gemm_glu_fwd(xg, grp: GroupsT, w1_packed, H, I, ep: EpilogueT, y=None, preact=None,
                           mx: Optional[MxOutT] = None, cu_margin: int = 0, stream=None):
    _check("moe_group_gemm_glu_fwd",
           _lib.moe_group_gemm_glu_fwd(_ptr(xg), ctypes.byref(grp), _ptr(w1_packed), H, I,
                                       ctypes.byref(ep), _ptr(y), _ptr(preact), _ref(mx),
                                       cu_margin, _stream(stream)))


def moe_group_gemm_dglu_bwd(dy2, w2: OperandT, H, I, grp: GroupsT, preact, ep: EpilogueT, dgu=None,
                            mx: Optional[MxOutT] = None, cu_margin: int = 0, stream=None):
    _check("moe_group_gemm_dglu_bwd",
           _lib.moe_group_gemm_dglu_bwd(_ptr(dy2), ctypes.byref(w2), H, I, ctypes.byref(grp),
                                        _ptr(preact), ctypes.byref(ep), _ptr(dgu), _ref(mx),
                                        cu_margin, _stream(stream)))


def moe_group_gemm_quant(a: OperandT, b: OperandT, N, K, grp: GroupsT, c_bf16=None,
                         mx: Optional[MxOutT] = None, cu_margin: int = 0, stream=None):
    _check("moe_group_gemm_quant",
           _lib.moe_group_gemm_quant(ctypes.byref(a), ctypes.byref(b), N, K, ctypes.byref(grp),
                                     _ptr(c_bf16), _ref(mx), cu_margin, _stream(stream)))


def moe_group_gemm_wgrad(a, b, P, Q, grp: GroupsT, c, accumulate: bool = False,
                         cu_margin: int = 0, stream=None):
    _check("moe_group_gemm_wgrad",
           _lib.moe_group_gemm_wgrad(_ptr(a), _ptr(b), P, Q, ctypes.byref(grp), _ptr(c),
                                     1 if accumulate else 0, cu_margin, _stream(stream)))


def moe_group_gemm_wgrad_mx(a: OperandT, b: OperandT, P, Q, grp: GroupsT, c,
                            accumulate: bool = False, cu_margin: int = 0, stream=None):
    _check("moe_group_gemm_wgrad_mx",
           _lib.moe_group_gemm_wgrad_mx(ctypes.byref(a), ctypes.byref(b), P, Q, ctypes.byref(grp),
                                        _ptr(c), 1 if accumulate else 0, cu_margin,
                                        _stream(stream)))


def moe_glu_unfused(z, grp: GroupsT, I, ep: EpilogueT, y, stream=None):
    _check("moe_glu_unfused",
           _lib.moe_glu_unfused(_ptr(z), ctypes.byref(grp), I, ctypes.byref(ep), _ptr(y),
                                _stream(stream)))


def moe_dglu_unfused(g, z, grp: GroupsT, I, ep: EpilogueT, dgu, stream=None):
    _check("moe_dglu_unfused",
           _lib.moe_dglu_unfused(_ptr(g), _ptr(z), ctypes.byref(grp), I, ctypes.byref(ep), _ptr(dgu),
                                 _stream(stream)))


def moe_mxfp8_quantize(v, R, C, grp: Optional[GroupsT], mx: MxOutT, stream=None):
    _check("moe_mxfp8_quantize",
           _lib.moe_mxfp8_quantize(_ptr(v), R, C, _ref(grp), ctypes.byref(mx), _stream(stream)))


def raw_call(name: str, *args) -> int:
    """Calls a C entry point with raw ctypes arguments and returns its status
    (used by the argument-validation tests)."""
    return getattr(_lib, name)(*args)
