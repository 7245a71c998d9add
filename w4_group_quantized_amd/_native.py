"""ctypes binding of libmoe_w4.so: argument marshalling only.

Every function here forwards to the C entry point of the same name in
include/moe_w4.h; all computation happens in the HIP kernels.  Tensors are
torch tensors on the GPU (only their data pointers cross the boundary); the
stream defaults to torch's current stream.  A non-zero status raises
MoeError.  If the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_w4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python w4_group_quantized_amd/build.py` "
        "(there is no fallback implementation)")

# torch bundles its own HIP runtime (same soname as /opt/rocm's).  Whichever
# copy is loaded first serves the whole process, so load torch's before this
# library pulls in the system one: torch allocates every buffer we are given.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

MOE_RMSNORM = 1
MOE_RENORM = 2

EXPORTS = ("moe_workspace_size", "moe_workspace_init", "moe_route", "moe_permute", "moe_route_permute",
           "moe_w4_grouped_ffn", "moe_unpermute_combine", "moe_layer_forward",
           "moe_decode_stack_forward", "moe_layer_forward_noalloc",
           "moe_w4_dequant", "moe_w4_quantize", "moe_w4_pack", "moe_w8_quantize", "moe_status_str",
           "moe_last_hip_error")


class MoeLayer(ctypes.Structure):
    """Mirror of `moe_layer` (a host struct of device pointers)."""
    _fields_ = [
        ("num_experts", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("ffn", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("shared_ffn", ctypes.c_int32),
        ("router_w", ctypes.c_void_p),
        ("router_b", ctypes.c_void_p),
        ("gate_q", ctypes.c_void_p),
        ("gate_s", ctypes.c_void_p),
        ("up_q", ctypes.c_void_p),
        ("up_s", ctypes.c_void_p),
        ("down_q", ctypes.c_void_p),
        ("down_s", ctypes.c_void_p),
        ("shared_gate", ctypes.c_void_p),
        ("shared_up", ctypes.c_void_p),
        ("shared_down", ctypes.c_void_p),
        ("shared_bits", ctypes.c_int32),
        ("shared_gate_q", ctypes.c_void_p),
        ("shared_gate_s", ctypes.c_void_p),
        ("shared_up_q", ctypes.c_void_p),
        ("shared_up_s", ctypes.c_void_p),
        ("shared_down_q", ctypes.c_void_p),
        ("shared_down_s", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_LP = ctypes.POINTER(MoeLayer)

_sigs = {
    "moe_workspace_size": (_SZ, [_LP, _I32]),
    "moe_workspace_init": (ctypes.c_int, [_P, _SZ, _P]),
    "moe_route": (ctypes.c_int, [_LP, _P, _I32, _P, _P, _P, _SZ, _P]),
    "moe_permute": (ctypes.c_int, [_LP, _P, _P, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_permute": (ctypes.c_int, [_LP, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_w4_grouped_ffn": (ctypes.c_int, [_LP, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "moe_unpermute_combine": (ctypes.c_int, [_LP, _P, _P, _P, _P, _I32, ctypes.c_uint32,
                                             ctypes.c_float, _P, _P]),
    "moe_layer_forward": (ctypes.c_int, [_LP, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_uint32, ctypes.c_float, _P, _P, _SZ, _P]),
    "moe_decode_stack_forward": (ctypes.c_int, [ctypes.POINTER(_LP), _I32, _P, _I32, _P, _P, _P,
                                                _P, _P, _P, _P, ctypes.c_uint32, ctypes.c_float,
                                                _P, _P, _SZ, _P]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [_LP, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                                 ctypes.c_uint32, ctypes.c_float, _P, _P]),
    "moe_w4_dequant": (ctypes.c_int, [_P, _P, _I64, _I64, _I32, _P, _P]),
    "moe_w4_quantize": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "moe_w8_quantize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "moe_w4_pack": (ctypes.c_int, [_P, _P, _I64, _I64, _I32, _P, _P, _P]),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_hip_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = f"{fn} failed: status {status} ({lib.moe_status_str(status).decode()})"
        if status == -4:
            msg += f": {lib.moe_last_hip_error().decode()}"
        super().__init__(msg)


def _ptr(t):
    """Data pointer of a tensor, or an int address, or None -> NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


def make_layer(num_experts, hidden, ffn, top_k, router_w, router_b, gate_q, gate_s, up_q, up_s,
               down_q, down_s, shared_ffn=0, shared_gate=None, shared_up=None, shared_down=None,
               group_size=128, shared_w8=None) -> MoeLayer:
    """shared_w8: None, or ((gate_q, gate_s), (up_q, up_s), (down_q, down_s)) of
    an 8-bit shared expert (then shared_gate/up/down are not used)."""
    w8 = shared_w8 if shared_w8 is not None else ((None, None),) * 3
    return MoeLayer(num_experts, hidden, ffn, top_k, group_size, shared_ffn,
                    _ptr(router_w), _ptr(router_b), _ptr(gate_q), _ptr(gate_s), _ptr(up_q),
                    _ptr(up_s), _ptr(down_q), _ptr(down_s), _ptr(shared_gate), _ptr(shared_up),
                    _ptr(shared_down), 8 if shared_w8 is not None else 16,
                    _ptr(w8[0][0]), _ptr(w8[0][1]), _ptr(w8[1][0]), _ptr(w8[1][1]),
                    _ptr(w8[2][0]), _ptr(w8[2][1]))


def moe_workspace_size(layer: MoeLayer, max_tokens: int) -> int:
    return lib.moe_workspace_size(ctypes.byref(layer), max_tokens)


def moe_workspace_init(ws, ws_bytes, stream=None):
    _check("moe_workspace_init", lib.moe_workspace_init(_ptr(ws), ws_bytes, _stream(stream)))


def moe_route(layer, x, T, topk_idx, topk_w, ws, ws_bytes, stream=None):
    _check("moe_route", lib.moe_route(ctypes.byref(layer), _ptr(x), T, _ptr(topk_idx),
                                      _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream)))


def moe_permute(layer, x, topk_idx, T, offsets, perm_src, inv_pos, x_perm, ws, ws_bytes,
                stream=None):
    _check("moe_permute", lib.moe_permute(ctypes.byref(layer), _ptr(x), _ptr(topk_idx), T,
                                          _ptr(offsets), _ptr(perm_src), _ptr(inv_pos),
                                          _ptr(x_perm), _ptr(ws), ws_bytes, _stream(stream)))


def moe_route_permute(layer, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm, ws,
                      ws_bytes, stream=None):
    _check("moe_route_permute",
           lib.moe_route_permute(ctypes.byref(layer), _ptr(x), T, _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(offsets), _ptr(perm_src), _ptr(inv_pos), _ptr(x_perm),
                                 _ptr(ws), ws_bytes, _stream(stream)))


def moe_w4_grouped_ffn(layer, x, x_perm, perm_src, offsets, T, y_perm, y_shared, ws, ws_bytes,
                       stream=None):
    _check("moe_w4_grouped_ffn",
           lib.moe_w4_grouped_ffn(ctypes.byref(layer), _ptr(x), _ptr(x_perm), _ptr(perm_src),
                                  _ptr(offsets), T, _ptr(y_perm), _ptr(y_shared), _ptr(ws),
                                  ws_bytes, _stream(stream)))


def moe_unpermute_combine(layer, y_perm, y_shared, inv_pos, topk_w, T, flags, eps, out,
                          stream=None):
    _check("moe_unpermute_combine",
           lib.moe_unpermute_combine(ctypes.byref(layer), _ptr(y_perm), _ptr(y_shared),
                                     _ptr(inv_pos), _ptr(topk_w), T, flags, eps, _ptr(out),
                                     _stream(stream)))


def moe_layer_forward(layer, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm, y_perm,
                      y_shared, flags, eps, out, ws, ws_bytes, stream=None):
    _check("moe_layer_forward",
           lib.moe_layer_forward(ctypes.byref(layer), _ptr(x), T, _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(offsets), _ptr(perm_src), _ptr(inv_pos), _ptr(x_perm),
                                 _ptr(y_perm), _ptr(y_shared), flags, eps, _ptr(out), _ptr(ws),
                                 ws_bytes, _stream(stream)))


def layer_array(layers):
    """A host array of pointers to the given MoeLayer descriptions (keep the
    returned object alive while a call uses it)."""
    arr = (_LP * len(layers))(*[ctypes.pointer(d) for d in layers])
    arr._keep = list(layers)
    return arr


def moe_decode_stack_forward(layers, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, y_perm,
                             y_shared, flags, eps, acts, ws, ws_bytes, stream=None, n_layers=None):
    """layers: a sequence of MoeLayer, or an array made by layer_array."""
    arr = layers if isinstance(layers, ctypes.Array) else layer_array(layers)
    n = len(arr) if n_layers is None else n_layers
    _check("moe_decode_stack_forward",
           lib.moe_decode_stack_forward(arr, n, _ptr(x), T, _ptr(topk_idx), _ptr(topk_w),
                                        _ptr(offsets), _ptr(perm_src), _ptr(inv_pos),
                                        _ptr(y_perm), _ptr(y_shared), flags, eps, _ptr(acts),
                                        _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer_forward_noalloc(layer, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm,
                              y_perm, y_shared, flags, eps, out, stream=None):
    _check("moe_layer_forward_noalloc",
           lib.moe_layer_forward_noalloc(ctypes.byref(layer), _ptr(x), T, _ptr(topk_idx),
                                         _ptr(topk_w), _ptr(offsets), _ptr(perm_src),
                                         _ptr(inv_pos), _ptr(x_perm), _ptr(y_perm),
                                         _ptr(y_shared), flags, eps, _ptr(out), _stream(stream)))


def moe_w4_dequant(q, s, rows, cols, group_size, out, stream=None):
    _check("moe_w4_dequant", lib.moe_w4_dequant(_ptr(q), _ptr(s), rows, cols, group_size,
                                                _ptr(out), _stream(stream)))


def moe_w4_pack(q_rowmajor, s_rowmajor, rows, cols, group_size, q, s, stream=None):
    _check("moe_w4_pack", lib.moe_w4_pack(_ptr(q_rowmajor), _ptr(s_rowmajor), rows, cols,
                                          group_size, _ptr(q), _ptr(s), _stream(stream)))


def moe_w8_quantize(w, rows, cols, q, s, stream=None):
    _check("moe_w8_quantize", lib.moe_w8_quantize(_ptr(w), rows, cols, _ptr(q), _ptr(s),
                                                  _stream(stream)))


def moe_w4_quantize(w, rows, cols, group_size, q, s, stream=None):
    _check("moe_w4_quantize", lib.moe_w4_quantize(_ptr(w), rows, cols, group_size, _ptr(q),
                                                  _ptr(s), _stream(stream)))


def moe_status_str(status: int) -> str:
    return lib.moe_status_str(status).decode()
