"""Python binding of the MI355X MoE layer library (libmoe.so, include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  Functions
with the C names take torch tensors for every buffer (outputs included);
``Layer`` allocates those buffers and chains the calls.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

from ._lib import (DTYPES, MOE_BF16, MOE_F32, MOE_MXFP8, OP_BACKWARD, OP_COMBINE, OP_DECODE,
                   OP_DISPATCH, OP_EXPERT_FFN, OP_FORWARD, OP_ROUTE, LIB_PATH, MoeError, MoeShape,
                   check, lib)

__all__ = ["make_shape", "check_shape", "workspace_bytes", "moe_route", "moe_dispatch", "moe_expert_ffn",
           "moe_expert_ffn_timed",
           "moe_combine", "moe_forward", "moe_decode", "moe_backward", "moe_backward_mx",
           "moe_quantize_mx", "quantize_mx_t_backward_weights", "Layer",
           "MoeError",
           "LIB_PATH"]


def make_shape(T: int, d: int, E: int, k: int, f: int, C: Optional[int] = None, fs: int = 0,
               dtype: str = "bf16") -> MoeShape:
    import math
    if C is None:
        C = int(math.ceil(1.25 * T * k))
    return MoeShape(tokens=T, capacity=C, hidden=d, experts=E, top_k=k, ffn=f, shared_ffn=fs,
                    dtype=DTYPES[dtype] if isinstance(dtype, str) else int(dtype))


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors only")
    return t.data_ptr()


def _s(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def check_shape(shape: MoeShape) -> None:
    """Raise MoeError if the library would reject `shape` (host-side validation only)."""
    check("moe_check_shape", lib().moe_check_shape(shape))


def workspace_bytes(shape: MoeShape, op: int) -> int:
    return int(lib().moe_workspace_bytes(shape, op))


def workspace(shape: MoeShape, op: int, device) -> torch.Tensor:
    """A zero-filled workspace buffer of the size `op` needs (at least 256 bytes)."""
    return torch.zeros(max(workspace_bytes(shape, op), 256), dtype=torch.uint8, device=device)


def moe_route(shape, x, w_router, b_router, topk_idx, topk_gate, expert_count, ws, stream=None):
    check("moe_route", lib().moe_route(shape, _p(x), _p(w_router), _p(b_router), _p(topk_idx),
                                       _p(topk_gate), _p(expert_count), _p(ws), ws.numel(),
                                       _s(stream)))


def moe_dispatch(shape, x, topk_idx, ring_head, ring_x, ring_x_scale, expert_offset, copy_slot,
                 slot_copy, ws, stream=None):
    check("moe_dispatch", lib().moe_dispatch(shape, _p(x), _p(topk_idx), int(ring_head), _p(ring_x),
                                             _p(ring_x_scale), _p(expert_offset), _p(copy_slot),
                                             _p(slot_copy), _p(ws), ws.numel(), _s(stream)))


def moe_expert_ffn(shape, ring_x, ring_x_scale, expert_offset, ring_head, w_gate, w_up, w_down,
                   w_gate_scale, w_up_scale, w_down_scale, ring_y, saved_au, ws, stream=None):
    check("moe_expert_ffn", lib().moe_expert_ffn(
        shape, _p(ring_x), _p(ring_x_scale), _p(expert_offset), int(ring_head), _p(w_gate),
        _p(w_up), _p(w_down), _p(w_gate_scale), _p(w_up_scale), _p(w_down_scale), _p(ring_y),
        _p(saved_au), _p(ws), ws.numel(), _s(stream)))


def moe_expert_ffn_timed(shape, ring_x, ring_x_scale, expert_offset, ring_head, w_gate, w_up,
                         w_down, w_gate_scale, w_up_scale, w_down_scale, ring_y, saved_au, ws,
                         events, stream=None):
    """moe_expert_ffn that records events[0..2] (torch.cuda.Event) around GEMM-1 and GEMM-2."""
    import ctypes
    for e in events:          # torch creates the HIP event on its first record()
        if e.cuda_event == 0:
            e.record()
    arr = (ctypes.c_void_p * 3)(*[e.cuda_event for e in events])
    check("moe_expert_ffn_timed", lib().moe_expert_ffn_timed(
        shape, _p(ring_x), _p(ring_x_scale), _p(expert_offset), int(ring_head), _p(w_gate),
        _p(w_up), _p(w_down), _p(w_gate_scale), _p(w_up_scale), _p(w_down_scale), _p(ring_y),
        _p(saved_au), _p(ws), ws.numel(), ctypes.cast(arr, ctypes.c_void_p), _s(stream)))


def moe_combine(shape, ring_y, copy_slot, topk_gate, y, stream=None):
    check("moe_combine", lib().moe_combine(shape, _p(ring_y), _p(copy_slot), _p(topk_gate), _p(y),
                                           _s(stream)))


def moe_forward(shape, x, w_router, b_router, w_gate, w_up, w_down, ring_head, topk_idx, topk_gate,
                expert_count, ring_x, expert_offset, copy_slot, slot_copy, ring_y, saved_au, y, ws,
                spin_limit=0, stream=None):
    """The whole forward in one cooperative launch (bf16)."""
    check("moe_forward", lib().moe_forward(
        shape, _p(x), _p(w_router), _p(b_router), _p(w_gate), _p(w_up), _p(w_down), int(ring_head),
        _p(topk_idx), _p(topk_gate), _p(expert_count), _p(ring_x), _p(expert_offset), _p(copy_slot),
        _p(slot_copy), _p(ring_y), _p(saved_au), _p(y), int(spin_limit), _p(ws), ws.numel(),
        _s(stream)))


def moe_decode(shape, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
               topk_idx, topk_gate, ws, stream=None):
    check("moe_decode", lib().moe_decode(shape, _p(x), _p(w_router), _p(b_router), _p(w_gate),
                                         _p(w_up), _p(w_down), _p(ws_gate), _p(ws_up),
                                         _p(ws_down), _p(y), _p(topk_idx), _p(topk_gate), _p(ws),
                                         ws.numel(), _s(stream)))


def moe_backward(shape, dy, x, w_router, topk_idx, topk_gate, ring_x, expert_offset, copy_slot,
                 slot_copy, ring_head, saved_au, w_gate, w_up, w_down, dx, dw_gate, dw_up,
                 dw_down, dw_router, ws, stream=None):
    check("moe_backward", lib().moe_backward(
        shape, _p(dy), _p(x), _p(w_router), _p(topk_idx), _p(topk_gate), _p(ring_x),
        _p(expert_offset), _p(copy_slot), _p(slot_copy), int(ring_head), _p(saved_au),
        _p(w_gate), _p(w_up), _p(w_down), _p(dx), _p(dw_gate), _p(dw_up), _p(dw_down),
        _p(dw_router), _p(ws), ws.numel(), _s(stream)))


def moe_backward_mx(shape, dy, x, w_router, topk_idx, topk_gate, expert_offset, copy_slot,
                    slot_copy, ring_head, saved_au, w_gu_t, w_gu_t_scale, w_down_t, w_down_t_scale,
                    dx, dw_gate, dw_up, dw_down, dw_router, ws, stream=None):
    check("moe_backward_mx", lib().moe_backward_mx(
        shape, _p(dy), _p(x), _p(w_router), _p(topk_idx), _p(topk_gate), _p(expert_offset),
        _p(copy_slot), _p(slot_copy), int(ring_head), _p(saved_au), _p(w_gu_t), _p(w_gu_t_scale),
        _p(w_down_t), _p(w_down_t_scale), _p(dx), _p(dw_gate), _p(dw_up), _p(dw_down),
        _p(dw_router), _p(ws), ws.numel(), _s(stream)))


def quantize_mx_t_backward_weights(w_gate, w_up, w_down, stream=None):
    """The MXFP8 backward's weights from the bf16 ones: (w_gu_t [E,d,2f], its scales,
    w_down_t [E,f,d], its scales), via moe_quantize_mx_t."""
    E, f, d = w_gate.shape
    dev = w_gate.device
    gu = torch.empty((E, d, 2 * f), dtype=torch.uint8, device=dev)
    gus = torch.empty((2 * f // 128, E * d, 4), dtype=torch.uint8, device=dev)
    dn = torch.empty((E, f, d), dtype=torch.uint8, device=dev)
    dns = torch.empty((d // 128, E * f, 4), dtype=torch.uint8, device=dev)
    L = lib()
    s = _s(stream)
    check("moe_quantize_mx_t", L.moe_quantize_mx_t(_p(w_gate), E, f, d, _p(gu), 2 * f, 0, _p(gus), s))
    check("moe_quantize_mx_t", L.moe_quantize_mx_t(_p(w_up), E, f, d, _p(gu), 2 * f, f, _p(gus), s))
    check("moe_quantize_mx_t", L.moe_quantize_mx_t(_p(w_down), E, d, f, _p(dn), d, 0, _p(dns), s))
    return gu, gus, dn, dns


def quantize_mx_training_weights(w_gate, w_up, w_down, stream=None):
    """Every MX weight an MXFP8 training step needs, from the bf16 ones, reading each once
    (moe_quantize_mx_both): ((W_gate, W_up, W_down) codes, (their scales), and the
    backward's w_gu_t, w_gu_t scales, w_down_t, w_down_t scales) -- the outputs of
    quantize_mx on each weight and of quantize_mx_t_backward_weights, bit for bit."""
    E, f, d = w_gate.shape
    dev = w_gate.device
    codes = tuple(torch.empty(w.shape, dtype=torch.uint8, device=dev) for w in (w_gate, w_up, w_down))
    scales = (torch.empty((d // 128, E * f, 4), dtype=torch.uint8, device=dev),
              torch.empty((d // 128, E * f, 4), dtype=torch.uint8, device=dev),
              torch.empty((f // 128, E * d, 4), dtype=torch.uint8, device=dev))
    gu = torch.empty((E, d, 2 * f), dtype=torch.uint8, device=dev)
    gus = torch.empty((2 * f // 128, E * d, 4), dtype=torch.uint8, device=dev)
    dn = torch.empty((E, f, d), dtype=torch.uint8, device=dev)
    dns = torch.empty((d // 128, E * f, 4), dtype=torch.uint8, device=dev)
    L = lib()
    s = _s(stream)
    for w, c, sc, ct, ld, col0, sct, R, Cc in ((w_gate, codes[0], scales[0], gu, 2 * f, 0, gus, f, d),
                                               (w_up, codes[1], scales[1], gu, 2 * f, f, gus, f, d),
                                               (w_down, codes[2], scales[2], dn, d, 0, dns, d, f)):
        check("moe_quantize_mx_both", L.moe_quantize_mx_both(_p(w), E, R, Cc, _p(c), _p(sc), _p(ct),
                                                             ld, col0, _p(sct), s))
    return codes, scales, (gu, gus, dn, dns)


def moe_quantize_mx(src, codes, scales, stream=None):
    rows = src.numel() // src.shape[-1]
    check("moe_quantize_mx", lib().moe_quantize_mx(_p(src), rows, src.shape[-1], _p(codes),
                                                   _p(scales), _s(stream)))


def quantize_mx(src: torch.Tensor, stream=None):
    """(codes uint8, scales uint8) of a bf16 tensor, MX along its last dimension; the
    scales in the library's layout [cols/128][rows][4] (rows = all leading dimensions)."""
    codes = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
    rows = src.numel() // src.shape[-1]
    scales = torch.empty((src.shape[-1] // 128, rows, 4), dtype=torch.uint8, device=src.device)
    moe_quantize_mx(src, codes, scales, stream)
    return codes, scales


@dataclass
class Layer:
    """Buffers of one layer shape, and the forward / backward / decode as chained C calls.

    Expert weights are passed per call; for MXFP8 pass their MX codes and scales."""
    shape: MoeShape
    device: torch.device
    bufs: Dict[str, torch.Tensor] = field(default_factory=dict)

    @classmethod
    def create(cls, T, d, E, k, f, C=None, fs=0, dtype="bf16", device="cuda"):
        return cls(make_shape(T, d, E, k, f, C, fs, dtype), torch.device(device))

    @property
    def act_dtype(self):
        return torch.float32 if self.shape.dtype == MOE_F32 else torch.bfloat16

    def _buf(self, name, shape, dtype):
        b = self.bufs.get(name)
        if b is None or tuple(b.shape) != tuple(shape) or b.dtype != dtype:
            b = torch.zeros(shape, dtype=dtype, device=self.device)
            self.bufs[name] = b
        return b

    def _ws(self, op):
        n = max(workspace_bytes(self.shape, op), 256)
        return self._buf(f"ws{op}", (n,), torch.uint8)

    def route(self, x, w_router, b_router=None):
        s = self.shape
        T, k, E = s.tokens, s.top_k, s.experts
        idx = self._buf("topk_idx", (T, k), torch.int32)
        gate = self._buf("topk_gate", (T, k), torch.float32)
        cnt = self._buf("expert_count", (E,), torch.int32)
        moe_route(s, x, w_router, b_router, idx, gate, cnt, self._ws(OP_ROUTE))
        return idx, gate, cnt

    def dispatch(self, x, topk_idx, head=0):
        s = self.shape
        mx = s.dtype == MOE_MXFP8
        ring = self._buf("ring_x", (s.capacity, s.hidden), torch.uint8 if mx else self.act_dtype)
        rsc = self._buf("ring_x_scale", (s.hidden // 128, s.capacity, 4), torch.uint8) if mx else None
        off = self._buf("expert_offset", (s.experts + 1,), torch.int32)
        cs = self._buf("copy_slot", (s.tokens, s.top_k), torch.int32)
        sc = self._buf("slot_copy", (s.capacity,), torch.int32)
        moe_dispatch(s, x, topk_idx, head, ring, rsc, off, cs, sc, self._ws(OP_DISPATCH))
        return ring, rsc, off, cs, sc

    def expert_ffn(self, ring_x, ring_x_scale, expert_offset, head, w_gate, w_up, w_down,
                   scales=(None, None, None), save_au=False, events=None):
        s = self.shape
        ydt = torch.float32 if s.dtype == MOE_F32 else torch.bfloat16
        ring_y = self._buf("ring_y", (s.capacity, s.hidden), ydt)
        au = self._buf("saved_au", (s.capacity, 2 * s.ffn), torch.bfloat16) if save_au else None
        if events is None:
            moe_expert_ffn(s, ring_x, ring_x_scale, expert_offset, head, w_gate, w_up, w_down,
                           scales[0], scales[1], scales[2], ring_y, au, self._ws(OP_EXPERT_FFN))
        else:
            moe_expert_ffn_timed(s, ring_x, ring_x_scale, expert_offset, head, w_gate, w_up, w_down,
                                 scales[0], scales[1], scales[2], ring_y, au,
                                 self._ws(OP_EXPERT_FFN), events)
        return ring_y, au

    def combine(self, ring_y, copy_slot, topk_gate):
        s = self.shape
        y = self._buf("y", (s.tokens, s.hidden), torch.float32 if s.dtype == MOE_F32 else torch.bfloat16)
        moe_combine(s, ring_y, copy_slot, topk_gate, y)
        return y

    def forward(self, x, w_router, b_router, w_gate, w_up, w_down, scales=(None, None, None),
                head=0, save_au=False, events=None):
        idx, gate, cnt = self.route(x, w_router, b_router)
        ring, rsc, off, cs, sc = self.dispatch(x, idx, head)
        ring_y, au = self.expert_ffn(ring, rsc, off, head, w_gate, w_up, w_down, scales, save_au,
                                     events)
        y = self.combine(ring_y, cs, gate)
        return y

    def forward_fused(self, x, w_router, b_router, w_gate, w_up, w_down, head=0, save_au=False,
                      spin_limit=0):
        """The forward as one kernel launch (moe_forward), into the same buffers as forward()."""
        s = self.shape
        T, k, E, C = s.tokens, s.top_k, s.experts, s.capacity
        b = {"topk_idx": ((T, k), torch.int32), "topk_gate": ((T, k), torch.float32),
             "expert_count": ((E,), torch.int32), "ring_x": ((C, s.hidden), torch.bfloat16),
             "expert_offset": ((E + 1,), torch.int32), "copy_slot": ((T, k), torch.int32),
             "slot_copy": ((C,), torch.int32), "ring_y": ((C, s.hidden), torch.bfloat16),
             "y": ((T, s.hidden), torch.bfloat16)}
        t = {n: self._buf(n, shp, dt) for n, (shp, dt) in b.items()}
        au = self._buf("saved_au", (C, 2 * s.ffn), torch.bfloat16) if save_au else None
        moe_forward(s, x, w_router, b_router, w_gate, w_up, w_down, head, t["topk_idx"],
                    t["topk_gate"], t["expert_count"], t["ring_x"], t["expert_offset"],
                    t["copy_slot"], t["slot_copy"], t["ring_y"], au, t["y"], self._ws(OP_FORWARD),
                    spin_limit)
        return t["y"]

    def forward_status(self) -> int:
        """The fused forward's status word (bit 0: a grid barrier gave up); a host read."""
        ws = self.bufs.get(f"ws{OP_FORWARD}")
        return 0 if ws is None else int(ws[8:12].view(torch.int32).item())

    def decode(self, x, w_router, b_router, w_gate, w_up, w_down, ws_gate=None, ws_up=None,
               ws_down=None):
        s = self.shape
        y = self._buf("y", (s.tokens, s.hidden), torch.bfloat16)
        idx = self._buf("topk_idx", (s.tokens, s.top_k), torch.int32)
        gate = self._buf("topk_gate", (s.tokens, s.top_k), torch.float32)
        moe_decode(s, x, w_router, b_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y, idx,
                   gate, self._ws(OP_DECODE))
        return y, idx, gate

    def backward_mx(self, dy, x, w_router, w_gu_t, w_gu_t_scale, w_down_t, w_down_t_scale, head=0):
        """The MXFP8 layer's gradients after forward(..., save_au=True) with the same buffers."""
        s = self.shape
        b = self.bufs
        dx = self._buf("dx", (s.tokens, s.hidden), torch.bfloat16)
        dwg = self._buf("dw_gate", (s.experts, s.ffn, s.hidden), torch.bfloat16)
        dwu = self._buf("dw_up", (s.experts, s.ffn, s.hidden), torch.bfloat16)
        dwd = self._buf("dw_down", (s.experts, s.hidden, s.ffn), torch.bfloat16)
        dwr = self._buf("dw_router", (s.experts, s.hidden), torch.float32)
        moe_backward_mx(s, dy, x, w_router, b["topk_idx"], b["topk_gate"], b["expert_offset"],
                        b["copy_slot"], b["slot_copy"], head, b["saved_au"], w_gu_t, w_gu_t_scale,
                        w_down_t, w_down_t_scale, dx, dwg, dwu, dwd, dwr, self._ws(OP_BACKWARD))
        return dx, dwg, dwu, dwd, dwr

    def backward(self, dy, x, w_router, w_gate, w_up, w_down, head=0):
        """Gradients after a forward(..., save_au=True) with the same buffers."""
        s = self.shape
        b = self.bufs
        dx = self._buf("dx", (s.tokens, s.hidden), torch.bfloat16)
        dwg = self._buf("dw_gate", (s.experts, s.ffn, s.hidden), torch.bfloat16)
        dwu = self._buf("dw_up", (s.experts, s.ffn, s.hidden), torch.bfloat16)
        dwd = self._buf("dw_down", (s.experts, s.hidden, s.ffn), torch.bfloat16)
        dwr = self._buf("dw_router", (s.experts, s.hidden), torch.float32)
        moe_backward(s, dy, x, w_router, b["topk_idx"], b["topk_gate"], b["ring_x"],
                     b["expert_offset"], b["copy_slot"], b["slot_copy"], head, b["saved_au"],
                     w_gate, w_up, w_down, dx, dwg, dwu, dwd, dwr, self._ws(OP_BACKWARD))
        return dx, dwg, dwu, dwd, dwr


class RingStack:
    """L MoE layers of one shape sharing one token ring (dzen.guru page, ring-buffer
    paragraph of "Три решения…": a fixed ring whose head advances layer by layer,
    walked in reverse by the backward).

    Layer l dispatches its n = T*k copies at head_l = (head_0 + l*n) mod C, so the
    ring keeps every layer's dispatched rows and saved [A|U] until the backward,
    which consumes the layers last first (the newest segment first) and, inside a
    layer, experts E-1 -> 0 and rows last slot first: nothing is recomputed.  The
    layers are chained directly (x_{l+1} = y_l).  C >= L*n, so no segment is
    overwritten while it is live; segments may wrap past the end of the ring.
    Every step is one of the library's calls; this class only keeps the buffers."""

    def __init__(self, L, T, d, E, k, f, C=None, device="cuda"):
        n = T * k
        C = C if C is not None else L * int(math.ceil(1.25 * n))
        if C < L * n:
            raise ValueError(f"ring of {C} rows cannot hold {L} layers of {n} copies")
        self.L, self.n = L, n
        self.shape = make_shape(T, d, E, k, f, C)
        check_shape(self.shape)   # e.g. a ring of 4 GiB or more per array is rejected
        self.device = torch.device(device)
        dev = self.device
        z = lambda *s, dtype=torch.int32: torch.zeros(s, dtype=dtype, device=dev)
        self.ring_x = z(C, d, dtype=torch.bfloat16)
        self.saved_au = z(C, 2 * f, dtype=torch.bfloat16)
        self.ring_y = z(C, d, dtype=torch.bfloat16)
        self.slot_copy = z(C)
        self.per = [dict(idx=z(T, k), gate=z(T, k, dtype=torch.float32), cnt=z(E),
                         off=z(E + 1), cs=z(T, k), x=z(T, d, dtype=torch.bfloat16),
                         y=z(T, d, dtype=torch.bfloat16)) for _ in range(L)]
        self.ws = {op: z(max(workspace_bytes(self.shape, op), 256), dtype=torch.uint8)
                   for op in (OP_ROUTE, OP_DISPATCH, OP_EXPERT_FFN, OP_BACKWARD)}
        self.heads = [0] * L

    def forward(self, x, weights, head0=0):
        """weights[l] = (w_router, b_router, w_gate, w_up, w_down).  Returns y_{L-1}."""
        s, C = self.shape, self.shape.capacity
        self.heads = [(head0 + l * self.n) % C for l in range(self.L)]
        cur = x
        for l, (w_r, b_r, w_g, w_u, w_d) in enumerate(weights):
            p, h = self.per[l], self.heads[l]
            p["x"].copy_(cur)
            moe_route(s, p["x"], w_r, b_r, p["idx"], p["gate"], p["cnt"], self.ws[OP_ROUTE])
            moe_dispatch(s, p["x"], p["idx"], h, self.ring_x, None, p["off"], p["cs"],
                         self.slot_copy, self.ws[OP_DISPATCH])
            moe_expert_ffn(s, self.ring_x, None, p["off"], h, w_g, w_u, w_d, None, None, None,
                           self.ring_y, self.saved_au, self.ws[OP_EXPERT_FFN])
            moe_combine(s, self.ring_y, p["cs"], p["gate"], p["y"])
            cur = p["y"]
        return cur

    def backward(self, dy, weights, dw=None):
        """Layers L-1 -> 0 (each layer's input gradient is kept as per[l]["dx"]).  Returns
        dx_0 and, per layer, (dw_gate, dw_up, dw_down, dw_router);
        with `dw` given (one set of gradient buffers) every layer writes into it and the
        list holds that set L times (the caller consumes each layer's before the next)."""
        s = self.shape
        T, d, E, f = s.tokens, s.hidden, s.experts, s.ffn
        dev = self.device
        grads = [None] * self.L
        cur = dy
        for l in reversed(range(self.L)):
            w_r, _, w_g, w_u, w_d = weights[l]
            p = self.per[l]
            g = dw if dw is not None else (
                torch.empty(E, f, d, dtype=torch.bfloat16, device=dev),
                torch.empty(E, f, d, dtype=torch.bfloat16, device=dev),
                torch.empty(E, d, f, dtype=torch.bfloat16, device=dev),
                torch.empty(E, d, dtype=torch.float32, device=dev))
            dx = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
            moe_backward(s, cur, p["x"], w_r, p["idx"], p["gate"], self.ring_x, p["off"],
                         p["cs"], self.slot_copy, self.heads[l], self.saved_au, w_g, w_u, w_d,
                         dx, g[0], g[1], g[2], g[3], self.ws[OP_BACKWARD])
            grads[l] = g
            p["dx"] = dx
            cur = dx
        return cur, grads
