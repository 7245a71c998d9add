"""Device-resident W4 MoE layer: weights, preallocated buffers, one forward.

PyTorch provides device memory and streams only; every step of the layer
runs in the HIP kernels behind the C entry points, called in order on one
stream with no host synchronization in between.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _native as N


@dataclass
class MoEBuffers:
    """Outputs and workspace of one layer forward for up to `max_tokens` tokens."""
    max_tokens: int
    topk_idx: torch.Tensor      # int32 [T, k]
    topk_w: torch.Tensor        # fp32 [T, k]
    offsets: torch.Tensor       # int32 [E+1]
    perm_src: torch.Tensor      # int32 [T*k]
    inv_pos: torch.Tensor       # int32 [T*k]
    x_perm: torch.Tensor        # fp16 [T*k, H]
    y_perm: torch.Tensor        # fp16 [T*k, H]
    y_shared: torch.Tensor      # fp16 [T, H] (empty when no shared expert)
    out: torch.Tensor           # fp16 [T, H]
    ws: torch.Tensor            # uint8 workspace


class W4MoELayer:
    """One MoE layer whose routed experts are int4 with fp16 group scales
    (group size gs = 128, or 64 / 256; read off the scale shapes unless
    given) and whose optional shared expert is fp16.  All tensors live on one
    GPU.

    router_w fp16 [E,H], router_b fp32 [E] or None,
    gate_q/up_q uint8 [E,F,H/2], gate_s/up_s fp16 [E,F,H/gs],
    down_q uint8 [E,H,F/2], down_s fp16 [E,H,F/gs],
    shared = None or (Wg fp16 [Fs,H], Wu fp16 [Fs,H], Wd fp16 [H,Fs]),
    or shared_w8 = ((gate_q uint8 [Fs,H], gate_s fp16 [Fs,H/128]), (up ...),
    (down_q [H,Fs], down_s [H,Fs/128])): an 8-bit shared expert (see
    quantize_w8).
    """

    def __init__(self, top_k, router_w, router_b, gate_q, gate_s, up_q, up_s, down_q, down_s,
                 shared=None, group_size=None, shared_w8=None):
        E, H = router_w.shape
        F = gate_q.shape[1]
        self.E, self.H, self.F, self.k = E, H, F, top_k
        if shared is not None and shared_w8 is not None:
            raise ValueError("give the shared expert either in fp16 or in 8 bits")
        self.Fs = (shared[0].shape[0] if shared is not None else
                   shared_w8[0][0].shape[0] if shared_w8 is not None else 0)
        if group_size is None:
            group_size = H // gate_s.shape[2]
            if gate_s.shape[2] * group_size != H or down_s.shape[2] * group_size != F:
                raise ValueError("scale shapes do not give one group size for both matrices")
        self.group_size = group_size
        self.tensors = (router_w, router_b, gate_q, gate_s, up_q, up_s, down_q, down_s, shared,
                        shared_w8)
        sg, su, sd = shared if shared is not None else (None, None, None)
        self.desc = N.make_layer(E, H, F, top_k, router_w, router_b, gate_q, gate_s, up_q, up_s,
                                 down_q, down_s, self.Fs, sg, su, sd, group_size=self.group_size,
                                 shared_w8=shared_w8)

    @property
    def device(self):
        return self.tensors[0].device

    def workspace_size(self, max_tokens: int) -> int:
        return N.moe_workspace_size(self.desc, max_tokens)

    def alloc(self, max_tokens: int) -> MoEBuffers:
        d, T, k, H, E = self.device, max_tokens, self.k, self.H, self.E
        i32, f16 = torch.int32, torch.float16
        ws = torch.empty((max(self.workspace_size(T), 16384),), dtype=torch.uint8, device=d)
        N.moe_workspace_init(ws, ws.numel())   # its counter block starts at zero
        return MoEBuffers(
            max_tokens=T,
            topk_idx=torch.empty((T, k), dtype=i32, device=d),
            topk_w=torch.empty((T, k), dtype=torch.float32, device=d),
            offsets=torch.empty((E + 1,), dtype=i32, device=d),
            perm_src=torch.empty((T * k,), dtype=i32, device=d),
            inv_pos=torch.empty((T * k,), dtype=i32, device=d),
            x_perm=torch.empty((T * k, H), dtype=f16, device=d),
            y_perm=torch.empty((T * k, H), dtype=f16, device=d),
            y_shared=torch.empty((T if self.Fs else 0, H), dtype=f16, device=d),
            out=torch.empty((T, H), dtype=f16, device=d),
            ws=ws,
        )

    # the stages, each one C call
    def route(self, x, buf, T, stream=None):
        N.moe_route(self.desc, x, T, buf.topk_idx, buf.topk_w, buf.ws, buf.ws.numel(), stream)

    def permute(self, x, buf, T, gather=True, stream=None):
        N.moe_permute(self.desc, x, buf.topk_idx, T, buf.offsets, buf.perm_src, buf.inv_pos,
                      buf.x_perm if gather else None, buf.ws, buf.ws.numel(), stream)

    def route_permute(self, x, buf, T, gather=False, stream=None):
        N.moe_route_permute(self.desc, x, T, buf.topk_idx, buf.topk_w, buf.offsets, buf.perm_src,
                            buf.inv_pos, buf.x_perm if gather else None, buf.ws, buf.ws.numel(),
                            stream)

    def ffn(self, x, buf, T, use_x_perm=False, stream=None):
        N.moe_w4_grouped_ffn(self.desc, x, buf.x_perm if use_x_perm else None, buf.perm_src,
                             buf.offsets, T, buf.y_perm, buf.y_shared if self.Fs else None,
                             buf.ws, buf.ws.numel(), stream)

    def combine(self, buf, T, rmsnorm=False, eps=1e-6, out=None, renorm=False, stream=None):
        flags = (N.MOE_RMSNORM if rmsnorm else 0) | (N.MOE_RENORM if renorm else 0)
        N.moe_unpermute_combine(self.desc, buf.y_perm, buf.y_shared if self.Fs else None,
                                buf.inv_pos, buf.topk_w, T, flags, eps,
                                buf.out if out is None else out, stream)

    def forward(self, x, buf, T=None, rmsnorm=False, eps=1e-6, out=None, gather=False,
                renorm=False, stream=None):
        """x fp16 [T, H] on the device -> buf.out (or `out`) fp16 [T, H].

        One C call (moe_layer_forward): route + permute (one launch for small
        batches), the grouped FFN reading token rows through perm_src (or from
        buf.x_perm, written by the permutation, with gather=True), and the
        combine (with renorm=True the k combine weights of a token are rescaled
        to sum to 1)."""
        T = x.shape[0] if T is None else T
        if T > buf.max_tokens:
            raise ValueError("more tokens than the buffers were allocated for")
        o = buf.out if out is None else out
        flags = (N.MOE_RMSNORM if rmsnorm else 0) | (N.MOE_RENORM if renorm else 0)
        N.moe_layer_forward(self.desc, x, T, buf.topk_idx, buf.topk_w, buf.offsets, buf.perm_src,
                            buf.inv_pos, buf.x_perm if gather else None, buf.y_perm,
                            buf.y_shared if self.Fs else None, flags, eps, o, buf.ws,
                            buf.ws.numel(), stream)
        return buf.out[:T] if out is None else out

    def forward_staged(self, x, buf, T=None, rmsnorm=False, eps=1e-6, out=None, gather=False,
                       renorm=False, stream=None):
        """The same layer as three C calls: moe_route_permute,
        moe_w4_grouped_ffn, moe_unpermute_combine."""
        T = x.shape[0] if T is None else T
        if T > buf.max_tokens:
            raise ValueError("more tokens than the buffers were allocated for")
        self.route_permute(x, buf, T, gather=gather, stream=stream)
        self.ffn(x, buf, T, use_x_perm=gather, stream=stream)
        self.combine(buf, T, rmsnorm, eps, out, renorm, stream)
        return buf.out[:T] if out is None else out


class W4MoEStack:
    """Stacked layers of one shape (the same experts, hidden, ffn, top-k and
    shared ffn) run as one decode step, the output of each layer being the
    input of the next: moe_decode_stack_forward."""

    def __init__(self, layers):
        self.layers = list(layers)
        if not self.layers:
            raise ValueError("a stack needs at least one layer")
        l0 = self.layers[0]
        for layer in self.layers:
            if (layer.E, layer.H, layer.F, layer.k, layer.Fs) != (l0.E, l0.H, l0.F, l0.k, l0.Fs):
                raise ValueError("stacked layers must share experts, hidden, ffn, top-k and "
                                 "shared ffn")
        self.arr = N.layer_array([layer.desc for layer in self.layers])

    def alloc(self, max_tokens: int) -> MoEBuffers:
        return self.layers[0].alloc(max_tokens)

    def forward(self, x, buf, acts=None, T=None, rmsnorm=True, eps=1e-6, renorm=False,
                n_layers=None, stream=None):
        """x fp16 [T, H] on the device -> acts fp16 [n_layers, T, H], every
        layer's output (the last one is the step's output).  The routing
        buffers of `buf` hold the last layer's routing afterwards."""
        T = x.shape[0] if T is None else T
        if T > buf.max_tokens:
            raise ValueError("more tokens than the buffers were allocated for")
        n = len(self.layers) if n_layers is None else n_layers
        if not 1 <= n <= len(self.layers):
            raise ValueError("n_layers out of range")
        H = self.layers[0].H
        if acts is None:
            acts = torch.empty((n, T, H), dtype=torch.float16, device=x.device)
        if acts.dtype != torch.float16 or not acts.is_contiguous() or \
                tuple(acts.shape[1:]) != (T, H) or acts.shape[0] < n:
            raise ValueError("acts must be contiguous fp16 [n_layers, T, H]")
        flags = (N.MOE_RMSNORM if rmsnorm else 0) | (N.MOE_RENORM if renorm else 0)
        N.moe_decode_stack_forward(self.arr, x, T, buf.topk_idx, buf.topk_w, buf.offsets,
                                   buf.perm_src, buf.inv_pos, buf.y_perm,
                                   buf.y_shared if self.layers[0].Fs else None, flags, eps, acts,
                                   buf.ws, buf.ws.numel(), stream, n_layers=n)
        return acts


def quantize_fp16(w: torch.Tensor, group_size: int = 128, stream=None):
    """Group-quantize an fp16 device matrix [rows, cols] with the HIP kernel.

    Returns (packed uint8 [rows, cols/2], scales fp16 [rows, cols/group_size])."""
    rows, cols = w.shape
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=w.device)
    s = torch.empty((rows, cols // group_size), dtype=torch.float16, device=w.device)
    N.moe_w4_quantize(w, rows, cols, group_size, q, s, stream)
    return q, s


def pack_plain(q_rowmajor: torch.Tensor, s_rowmajor: torch.Tensor, group_size: int = 128,
               stream=None):
    """Already-quantized codes stored plainly (uint8 [rows, cols/2], byte c/2
    = column c in bits 0-3 and c+1 in bits 4-7 as two's-complement nibbles;
    scales fp16 [rows, cols/group_size]) -> (packed uint8 [rows, cols/2],
    scales fp16 [rows, cols/group_size]) in the library's format."""
    rows, half = q_rowmajor.shape
    q = torch.empty_like(q_rowmajor)
    s = torch.empty_like(s_rowmajor)
    N.moe_w4_pack(q_rowmajor, s_rowmajor, rows, half * 2, group_size, q, s, stream)
    return q, s


def quantize_w8(w: torch.Tensor, stream=None):
    """8-bit g128 quantization of an fp16 device matrix [rows, cols] (the
    shared expert's format).  Returns (codes uint8 [rows, cols], scales fp16
    [rows, cols/128])."""
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
    s = torch.empty((rows, cols // 128), dtype=torch.float16, device=w.device)
    N.moe_w8_quantize(w, rows, cols, q, s, stream)
    return q, s


def dequantize(q: torch.Tensor, s: torch.Tensor, stream=None):
    """Exact fp32 dequantization of one packed matrix (the test hook); the
    group size is read off the shapes."""
    rows, half = q.shape
    out = torch.empty((rows, half * 2), dtype=torch.float32, device=q.device)
    N.moe_w4_dequant(q, s, rows, half * 2, (half * 2) // s.shape[1], out, stream)
    return out
