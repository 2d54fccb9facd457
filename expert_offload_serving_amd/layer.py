"""Device-side convenience wrappers over the C ABI (allocation of outputs and
workspaces with torch, struct packing, error checks).  No computation happens
here: every step runs in libmoe_nvfp4.so's kernels.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import _lib
from ._lib import check


def to_device_u8(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) -> a torch.bfloat16 device tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to(device).view(torch.bfloat16)


@dataclasses.dataclass
class DeviceLayer:
    """One layer's expert storage in HBM: a bank of equally sized slots, the
    expert -> slot map, the shared expert's slot (index into the bank, -1 for
    none) and the shared gate vector (bf16 [H])."""
    H: int
    I: int
    E: int
    k: int
    bank: torch.Tensor            # u8 [num_slots, slot_bytes]
    slot_of_expert: torch.Tensor  # i32 [E]
    shared_slot: int
    wg: torch.Tensor              # bf16 [H]

    fmt: str = "nvfp4"            # slot format: "nvfp4" or "mxfp4"

    def __post_init__(self):
        sb = (_lib.moe_nvfp4_slot_bytes if self.fmt == "nvfp4" else _lib.moe_mxfp4_slot_bytes)(self.H, self.I)
        if sb == 0 or self.bank.dim() != 2 or self.bank.shape[1] != sb:
            raise ValueError(f"bank must be [slots, {sb}] bytes for H={self.H}, I={self.I} ({self.fmt})")

    @property
    def slot_bytes(self) -> int:
        return self.bank.shape[1]

    def struct(self, slot_of_expert: torch.Tensor | None = None, shared: bool = True) -> _lib.LayerStruct:
        s = _lib.LayerStruct()
        s.H, s.I, s.E, s.k = self.H, self.I, self.E, self.k
        s.bank_base = self.bank.data_ptr()
        s.slot_bytes = self.slot_bytes
        s.num_slots = self.bank.shape[0]
        s.slot_of_expert = (self.slot_of_expert if slot_of_expert is None else slot_of_expert).data_ptr()
        if shared and self.shared_slot >= 0:
            s.shared_slot = self.bank[self.shared_slot].data_ptr()
            s.shared_gate_w = self.wg.data_ptr()
        else:
            s.shared_slot = None
            s.shared_gate_w = None
        return s


@dataclasses.dataclass
class Routing:
    ids: torch.Tensor            # i32 [T, k]
    w: torch.Tensor              # f32 [T, k]
    offsets: torch.Tensor        # i32 [E+1]
    sorted_assign: torch.Tensor  # i32 [T*k]
    assign_pos: torch.Tensor     # i32 [T*k]

    @staticmethod
    def empty(T: int, E: int, k: int, device="cuda") -> "Routing":
        i32 = dict(dtype=torch.int32, device=device)
        return Routing(torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=device),
                       torch.empty(E + 1, **i32), torch.empty(T * k, **i32), torch.empty(T * k, **i32))


def route(logits: torch.Tensor, k: int, out: Routing | None = None, stream=None) -> Routing:
    T, E = logits.shape
    r = Routing.empty(T, E, k, logits.device) if out is None else out
    nb = _lib.moe_route_workspace_bytes(T, E, k)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=logits.device) if nb else None
    check(_lib.moe_route_topk(logits, T, E, k, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, ws, nb, stream))
    return r


def router_logits(x: torch.Tensor, w_router: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """logits [T, E] f32 = x [T, H] bf16 . w_router [E, H] bf16^T on the matrix cores."""
    T, H = x.shape
    E = w_router.shape[0]
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if out is None else out
    check(_lib.moe_router_logits(x, w_router, T, H, E, logits, stream))
    return logits


def router_route(x: torch.Tensor, w_router: torch.Tensor, k: int, out: Routing | None = None,
                 logits: torch.Tensor | None = None, stream=None):
    """Router projection and top-k routing in one call; returns (logits, routing)."""
    T, H = x.shape
    E = w_router.shape[0]
    r = Routing.empty(T, E, k, x.device) if out is None else out
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    nb = _lib.moe_route_workspace_bytes(T, E, k)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=x.device) if nb else None
    check(_lib.moe_router_topk(x, w_router, T, H, E, k, logits, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos,
                               ws, nb, stream))
    return logits, r


def workspace(T: int, layer: DeviceLayer) -> torch.Tensor:
    f = _lib.moe_nvfp4_forward_workspace_bytes if layer.fmt == "nvfp4" else _lib.moe_mxfp4_forward_workspace_bytes
    nb = f(T, layer.H, layer.I, layer.E, layer.k)
    return torch.empty(max(nb, 1), dtype=torch.uint8, device=layer.bank.device)


def forward(layer: DeviceLayer, x: torch.Tensor, r: Routing, y: torch.Tensor | None = None, accumulate: bool = False,
            ws: torch.Tensor | None = None, slot_of_expert: torch.Tensor | None = None, shared: bool = True,
            stream=None) -> torch.Tensor:
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, layer.H), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(T, layer)
    st = layer.struct(slot_of_expert, shared)
    f = _lib.moe_nvfp4_forward if layer.fmt == "nvfp4" else _lib.moe_mxfp4_forward
    check(f(st, x, T, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, y, int(accumulate), ws, ws.numel(),
            stream))
    return y


def route_forward(layer: DeviceLayer, logits: torch.Tensor, x: torch.Tensor, y: torch.Tensor | None = None,
                  accumulate: bool = False, out: Routing | None = None, ws: torch.Tensor | None = None,
                  slot_of_expert: torch.Tensor | None = None, shared: bool = True, stream=None):
    """Routing and forward in one call; returns (y, routing)."""
    T, E = logits.shape
    r = Routing.empty(T, E, layer.k, x.device) if out is None else out
    if y is None:
        y = torch.empty((T, layer.H), dtype=torch.float32, device=x.device)
    mx = layer.fmt == "mxfp4"
    if ws is None:
        f = _lib.moe_mxfp4_route_forward_workspace_bytes if mx else _lib.moe_nvfp4_route_forward_workspace_bytes
        nb = f(T, layer.H, layer.I, layer.E, layer.k)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=x.device)
    st = layer.struct(slot_of_expert, shared)
    f = _lib.moe_mxfp4_route_forward if mx else _lib.moe_nvfp4_route_forward
    check(f(st, logits, x, T, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, y, int(accumulate), ws,
            ws.numel(), stream))
    return y, r


def dequant(codes: torch.Tensor, scales: torch.Tensor, globals_: torch.Tensor, stream=None) -> torch.Tensor:
    """fp32 [rows, K] of a row-major NVFP4 matrix: codes u8 [rows, K/2], scales u8 [rows, K/16], globals f32 [rows]."""
    rows, K = codes.shape[0], 2 * codes.shape[1]
    out = torch.empty((rows, K), dtype=torch.float32, device=codes.device)
    check(_lib.moe_nvfp4_dequant(codes, scales, globals_, rows, K, out, stream))
    return out


def dequant_slot(slot: torch.Tensor, H: int, I: int, matrix: int, stream=None) -> torch.Tensor:
    """fp32 gate_up (matrix 0, [2I, H]) or down (matrix 1, [H, I]) of one device slot."""
    shape = (2 * I, H) if matrix == 0 else (H, I)
    out = torch.empty(shape, dtype=torch.float32, device=slot.device)
    check(_lib.moe_nvfp4_dequant_slot(slot, H, I, matrix, out, stream))
    return out


def slice_bank(bank: torch.Tensor, H: int, I: int, r: int, n: int, stream=None) -> torch.Tensor:
    sb = _lib.moe_nvfp4_slot_bytes(H, I // n)
    out = torch.empty((bank.shape[0], sb), dtype=torch.uint8, device=bank.device)
    check(_lib.moe_nvfp4_slice_bank(bank, bank.shape[0], H, I, r, n, out, stream))
    return out


def mx_dequant(blocks_t: torch.Tensor, scales_t: torch.Tensor, stream=None) -> torch.Tensor:
    """fp32 [N, K] of an MXFP4 matrix in the checkpoints' transposed layout (blocks_t u8 [K/2, N], scales_t [K/32, N])."""
    K, N = 2 * blocks_t.shape[0], blocks_t.shape[1]
    out = torch.empty((N, K), dtype=torch.float32, device=blocks_t.device)
    check(_lib.moe_mxfp4_dequant(blocks_t, scales_t, N, K, out, stream))
    return out


def mx_dequant_slot(slot: torch.Tensor, H: int, I: int, matrix: int, stream=None) -> torch.Tensor:
    shape = (2 * I, H) if matrix == 0 else (H, I)
    out = torch.empty(shape, dtype=torch.float32, device=slot.device)
    check(_lib.moe_mxfp4_dequant_slot(slot, H, I, matrix, out, stream))
    return out


def mx_slice_bank(bank: torch.Tensor, H: int, I: int, r: int, n: int, stream=None) -> torch.Tensor:
    sb = _lib.moe_mxfp4_slot_bytes(H, I // n)
    out = torch.empty((bank.shape[0], sb), dtype=torch.uint8, device=bank.device)
    check(_lib.moe_mxfp4_slice_bank(bank, bank.shape[0], H, I, r, n, out, stream))
    return out
