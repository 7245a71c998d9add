"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before launching
anything (so none of these calls touches a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4.h")

N = pytest.importorskip("w4_group_quantized_amd._native",
                        reason="libmoe_w4.so not built (python w4_group_quantized_amd/build.py)")

OK, EINVAL, EUNSUP, EWS = 0, -1, -2, -3
FAKE = 1 << 20          # a 16-byte aligned non-null address that is never dereferenced
MISALIGNED = FAKE + 4


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert set(names) == set(N.EXPORTS), names
    for n in names:
        assert hasattr(N.lib, n), n


def layer(**kw):
    d = dict(num_experts=8, hidden=256, ffn=512, top_k=2, router_w=FAKE, router_b=None,
             gate_q=FAKE, gate_s=FAKE, up_q=FAKE, up_s=FAKE, down_q=FAKE, down_s=FAKE)
    d.update(kw)
    return N.make_layer(**d)


def route(L, x=FAKE, T=4, idx=FAKE, w=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return N.lib.moe_route(ctypes.byref(L), x, T, idx, w, ws, ws_bytes, None)


def test_workspace_size_and_invalid_layers():
    L = layer()
    assert N.moe_workspace_size(L, 16) > 0
    assert N.moe_workspace_size(L, 0) >= 0
    assert N.moe_workspace_size(layer(hidden=200), 16) == 0
    assert N.moe_workspace_size(L, -1) == 0
    assert N.moe_workspace_size(L, 32) >= N.moe_workspace_size(L, 16)
    for gs in (64, 256):      # the other group sizes are valid layers
        assert N.moe_workspace_size(layer(group_size=gs), 16) == N.moe_workspace_size(L, 16)


@pytest.mark.parametrize("kw,status", [
    (dict(group_size=32), EUNSUP),
    (dict(group_size=512), EUNSUP),
    (dict(group_size=256, hidden=384), EUNSUP),   # hidden not a whole number of groups
    (dict(group_size=256, ffn=640), EUNSUP),      # ffn not a whole number of groups
    (dict(hidden=200), EUNSUP),
    (dict(ffn=100), EUNSUP),
    (dict(top_k=9), EUNSUP),
    (dict(top_k=0), EUNSUP),
    (dict(num_experts=2000), EUNSUP),
])
def test_route_rejects_unsupported_layers(kw, status):
    assert route(layer(**kw)) == status


def test_route_argument_errors():
    L = layer()
    assert route(L, T=-1) == EINVAL
    assert route(L, x=None) == EINVAL
    assert route(L, x=MISALIGNED) == EINVAL
    assert route(layer(router_w=None)) == EINVAL
    assert route(L, ws_bytes=16) == EWS
    assert route(L, T=0, x=None, idx=None, w=None, ws=None, ws_bytes=0) == OK   # no-op


def test_other_calls_argument_errors():
    L = layer()
    big = 1 << 30
    assert N.lib.moe_permute(ctypes.byref(L), FAKE, None, 4, FAKE, FAKE, FAKE, FAKE, FAKE, big,
                             None) == EINVAL
    assert N.lib.moe_permute(ctypes.byref(L), FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 8,
                             None) == EWS
    ffn = N.lib.moe_w4_grouped_ffn
    # (layer, x, x_perm, perm_src, offsets, T, y_perm, y_shared, ws, ws_bytes, stream)
    assert ffn(ctypes.byref(layer(down_q=None)), FAKE, FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, big,
               None) == EINVAL
    assert ffn(ctypes.byref(L), FAKE, None, None, FAKE, 4, FAKE, None, FAKE, big,
               None) == EINVAL                        # no x_perm and no perm_src
    assert ffn(ctypes.byref(L), None, None, FAKE, FAKE, 4, FAKE, None, FAKE, big,
               None) == EINVAL                        # no x_perm and no x
    T_far = (1 << 31) // (2 * L.hidden)   # gathering from x needs T*H*2 < 2^31
    assert ffn(ctypes.byref(L), FAKE, None, FAKE, FAKE, T_far, FAKE, None, FAKE, big,
               None) == EUNSUP
    Ls = layer(shared_ffn=256)       # shared expert declared but its weights missing
    assert ffn(ctypes.byref(Ls), FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, big,
               None) == EINVAL
    rp = N.lib.moe_route_permute
    # (layer, x, T, idx, w, offsets, perm_src, inv_pos, x_perm, ws, ws_bytes, stream)
    assert rp(ctypes.byref(L), FAKE, 4, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, big,
              None) == EINVAL
    assert rp(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE, big,
              None) == EINVAL
    assert rp(ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 64,
              None) == EWS
    assert rp(ctypes.byref(L), None, 0, None, None, None, None, None, None, None, 0, None) == OK
    assert N.lib.moe_unpermute_combine(ctypes.byref(L), FAKE, None, FAKE, FAKE, 4, 4, 1e-6, FAKE,
                                       None) == EINVAL                      # unknown flag
    assert N.lib.moe_unpermute_combine(ctypes.byref(L), FAKE, None, FAKE, FAKE, 4, 1, -1.0,
                                       FAKE, None) == EINVAL                # negative eps
    assert N.lib.moe_w4_dequant(FAKE, FAKE, 16, 100, 128, FAKE, None) == EUNSUP
    assert N.lib.moe_w4_dequant(FAKE, FAKE, 16, 256, 32, FAKE, None) == EUNSUP    # group 32
    assert N.lib.moe_w4_dequant(FAKE, FAKE, 16, 384, 256, FAKE, None) == EUNSUP   # 384 % 256
    assert N.lib.moe_w4_quantize(FAKE, 16, 256, 128, None, FAKE, None) == EINVAL
    assert N.lib.moe_w4_quantize(FAKE, -16, 256, 128, FAKE, FAKE, None) == EINVAL
    assert N.lib.moe_w4_quantize(FAKE, 8, 256, 128, FAKE, FAKE, None) == EUNSUP   # rows % 16
    assert N.lib.moe_w4_quantize(FAKE, 16, 256, 100, FAKE, FAKE, None) == EUNSUP  # group 100
    assert N.lib.moe_w4_quantize(FAKE, 16, 384, 256, FAKE, FAKE, None) == EUNSUP  # 384 % 256
    assert N.lib.moe_w4_quantize(None, 0, 256, 64, None, None, None) == OK  # empty: no-op


def test_layer_forward_argument_errors():
    """The whole-layer call checks every stage's arguments before launching."""
    L = layer()
    big = 1 << 30
    fwd = N.lib.moe_layer_forward
    # (layer, x, T, idx, w, offsets, perm_src, inv_pos, x_perm, y_perm, y_shared, flags, eps,
    #  out, ws, ws_bytes, stream)
    args = [ctypes.byref(L), FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 0, 1e-6,
            FAKE, FAKE, big, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return fwd(*a)

    assert call(a1=None) == EINVAL                      # no x
    assert call(a3=MISALIGNED) == EINVAL                # topk_idx misaligned
    assert call(a6=None) == EINVAL                      # no perm_src
    assert call(a8=MISALIGNED) == EINVAL                # x_perm misaligned
    assert call(a9=None) == EINVAL                      # no y_perm
    assert call(a11=4) == EINVAL                        # unknown flag
    assert call(a11=1, a12=-1.0) == EINVAL              # negative eps
    assert call(a13=None) == EINVAL                     # no out
    assert call(a15=64) == EWS
    assert call(a0=ctypes.byref(layer(top_k=9))) == EUNSUP
    assert call(a2=(1 << 31) // (2 * L.hidden)) == EUNSUP   # gather from x needs T*H*2 < 2^31
    Ls = layer(shared_ffn=256)
    assert call(a0=ctypes.byref(Ls), a10=FAKE) == EINVAL   # shared weights missing
    Ls2 = layer(shared_ffn=256, shared_gate=FAKE, shared_up=FAKE, shared_down=FAKE)
    assert call(a0=ctypes.byref(Ls2)) == EINVAL            # shared expert but no y_shared
    assert call(a2=0, a1=None, a3=None, a4=None, a5=None, a6=None, a7=None, a9=None,
                a13=None, a14=None, a15=0) == OK            # T = 0: no-op


def test_decode_stack_argument_errors():
    """The stacked decode step checks every layer and every buffer before
    launching: no layers, layers of different shapes, and each stage's
    argument errors."""
    L0, L1 = layer(), layer()
    big = 1 << 30
    fwd = N.lib.moe_decode_stack_forward
    arr = N.layer_array([L0, L1])
    # (layers, n, x, T, idx, w, offsets, perm_src, inv_pos, y_perm, y_shared, flags, eps, acts,
    #  ws, ws_bytes, stream)
    args = [arr, 2, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1e-6, FAKE, FAKE, big,
            None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return fwd(*a)

    assert call(a0=None) == EINVAL                      # no layer array
    assert call(a1=0) == EINVAL                         # no layers
    assert call(a2=None) == EINVAL                      # no x
    assert call(a4=MISALIGNED) == EINVAL                # topk_idx misaligned
    assert call(a7=None) == EINVAL                      # no perm_src
    assert call(a9=None) == EINVAL                      # no y_perm
    assert call(a11=4) == EINVAL                        # unknown flag
    assert call(a11=1, a12=-1.0) == EINVAL              # negative eps
    assert call(a13=None) == EINVAL                     # no acts
    assert call(a15=64) == EWS
    assert call(a3=(1 << 31) // (2 * L0.hidden)) == EUNSUP   # rows of x gathered with 32-bit offsets
    for kw in (dict(ffn=256), dict(hidden=512), dict(num_experts=16), dict(top_k=4),
               dict(shared_ffn=256, shared_gate=FAKE, shared_up=FAKE, shared_down=FAKE)):
        assert call(a0=N.layer_array([L0, layer(**kw)])) == EUNSUP, kw   # shapes differ
    # group sizes may differ: the call gets as far as the workspace check
    assert call(a0=N.layer_array([L0, layer(group_size=64)]), a15=64) == EWS
    assert call(a0=N.layer_array([L0, layer(top_k=9)])) == EUNSUP        # an invalid layer
    assert call(a0=N.layer_array([L0, layer(gate_q=None)])) == EINVAL    # a layer's weights
    assert call(a3=0, a2=None, a4=None, a5=None, a6=None, a7=None, a8=None, a9=None,
                a13=None, a14=None, a15=0) == OK            # T = 0: no-op


def test_8bit_shared_expert_arguments():
    big = 1 << 30
    ffn = N.lib.moe_w4_grouped_ffn
    L8 = layer(shared_ffn=256)
    L8.shared_bits = 8            # 8-bit shared expert declared, its arrays missing
    assert ffn(ctypes.byref(L8), FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, big, None) == EINVAL
    L8.shared_gate_q = L8.shared_up_q = L8.shared_down_q = FAKE
    L8.shared_gate_s = L8.shared_up_s = L8.shared_down_s = FAKE
    assert ffn(ctypes.byref(L8), FAKE, FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, big,
               None) == EINVAL                                              # no y_shared
    Lb = layer()
    Lb.shared_bits = 4
    assert N.moe_workspace_size(Lb, 4) == 0                                 # unsupported
    assert N.lib.moe_w8_quantize(FAKE, 16, 200, FAKE, FAKE, None) == EUNSUP
    assert N.lib.moe_w8_quantize(FAKE, 8, 256, FAKE, FAKE, None) == EUNSUP
    assert N.lib.moe_w8_quantize(FAKE, 16, 256, None, FAKE, None) == EINVAL
    assert N.lib.moe_w8_quantize(None, 0, 256, None, None, None) == OK


def test_layer_struct_matches_the_header():
    """The binding's mirror of moe_layer has the header's fields in order."""
    src = open(HEADER).read()
    body = src[src.index("typedef struct moe_layer {"):src.index("} moe_layer;")]
    names = re.findall(r"\b(\w+);", body)
    assert names == [f[0] for f in N.MoeLayer._fields_], names


def test_status_strings():
    for s in (OK, EINVAL, EUNSUP, EWS, -4):
        assert N.moe_status_str(s)
    assert "unknown" in N.moe_status_str(-99)


def test_pack_arguments():
    pack = N.lib.moe_w4_pack
    assert pack(FAKE, FAKE, 16, 200, 128, FAKE, FAKE, None) == EUNSUP      # cols % 128
    assert pack(FAKE, FAKE, 8, 256, 128, FAKE, FAKE, None) == EUNSUP       # rows % 16
    assert pack(FAKE, FAKE, 16, 384, 256, FAKE, FAKE, None) == EUNSUP      # cols % group
    assert pack(FAKE, FAKE, 16, 256, 32, FAKE, FAKE, None) == EUNSUP       # group size
    assert pack(FAKE, FAKE, -16, 256, 128, FAKE, FAKE, None) == EINVAL
    assert pack(None, FAKE, 16, 256, 128, FAKE, FAKE, None) == EINVAL
    assert pack(FAKE, MISALIGNED, 16, 256, 128, FAKE, FAKE, None) == EINVAL
    assert pack(FAKE, FAKE, 16, 256, 128, FAKE, None, None) == EINVAL
    assert pack(None, None, 0, 256, 128, None, None, None) == OK            # nothing to do


def test_workspace_init_arguments():
    init = N.lib.moe_workspace_init
    assert init(FAKE, 16383, None) == EWS
    assert init(None, 16384, None) == EINVAL
    assert init(MISALIGNED, 16384, None) == EINVAL
