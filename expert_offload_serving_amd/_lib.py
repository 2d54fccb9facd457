"""ctypes binding of libmoe_nvfp4.so: the C ABI declared in include/moe_nvfp4.h.

Argument marshalling only.  Device buffers are passed as torch tensors (their
data pointers), streams as torch.cuda streams; every computation runs in the
library's HIP kernels.  Importing works without a GPU; loading the library
raises if it has not been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_nvfp4.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED_SHAPE = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_NOT_PINNED = 4
MOE_ERR_HIP = 5

EXPORTED = [
    "moe_last_error", "moe_nvfp4_slot_bytes", "moe_route_workspace_bytes", "moe_route_topk",
    "moe_nvfp4_forward_workspace_bytes", "moe_nvfp4_forward", "expert_cache_fill", "moe_cache_create",
    "moe_cache_destroy", "moe_cache_plan", "moe_nvfp4_slice_bank", "moe_nvfp4_dequant", "moe_nvfp4_dequant_slot",
    "moe_nvfp4_route_forward_workspace_bytes", "moe_nvfp4_route_forward", "moe_router_logits", "moe_router_topk",
    "moe_release_streams", "moe_nvfp4_noalloc_scratch_bytes", "moe_nvfp4_route_forward_noalloc",
    "moe_mxfp4_slot_bytes", "moe_mxfp4_forward_workspace_bytes", "moe_mxfp4_forward",
    "moe_mxfp4_route_forward_workspace_bytes", "moe_mxfp4_route_forward", "moe_mxfp4_dequant",
    "moe_mxfp4_dequant_slot", "moe_mxfp4_slice_bank", "moe_offload_device_bytes", "moe_offload_create",
    "moe_offload_destroy", "moe_offload_layer",
]


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class LayerStruct(ctypes.Structure):
    """moe_nvfp4_layer_t."""
    _fields_ = [
        ("H", ctypes.c_int), ("I", ctypes.c_int), ("E", ctypes.c_int), ("k", ctypes.c_int),
        ("bank_base", ctypes.c_void_p), ("slot_bytes", ctypes.c_size_t), ("num_slots", ctypes.c_int),
        ("slot_of_expert", ctypes.c_void_p), ("shared_slot", ctypes.c_void_p), ("shared_gate_w", ctypes.c_void_p),
    ]


_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m expert_offload_serving_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_nvfp4_slot_bytes.restype = _sz
        L.moe_nvfp4_slot_bytes.argtypes = [_i, _i]
        L.moe_route_workspace_bytes.restype = _sz
        L.moe_route_workspace_bytes.argtypes = [_i, _i, _i]
        L.moe_route_topk.restype = _i
        L.moe_route_topk.argtypes = [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_router_logits.restype = _i
        L.moe_router_logits.argtypes = [_vp, _vp, _i, _i, _i, _vp, _vp]
        L.moe_router_topk.restype = _i
        L.moe_router_topk.argtypes = [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_nvfp4_forward_workspace_bytes.restype = _sz
        L.moe_nvfp4_forward_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
        L.moe_nvfp4_forward.restype = _i
        L.moe_nvfp4_forward.argtypes = [ctypes.POINTER(LayerStruct), _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                        _vp, _sz, _vp]
        L.moe_nvfp4_route_forward_workspace_bytes.restype = _sz
        L.moe_nvfp4_route_forward_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
        L.moe_nvfp4_route_forward.restype = _i
        L.moe_nvfp4_route_forward.argtypes = [ctypes.POINTER(LayerStruct), _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _i, _vp, _sz, _vp]
        L.expert_cache_fill.restype = _i
        L.expert_cache_fill.argtypes = [_vp, _sz, _i, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(_vp), _i, _vp,
                                        _vp]
        L.moe_cache_create.restype = _vp
        L.moe_cache_create.argtypes = [_i, _i, _i]
        L.moe_cache_destroy.restype = None
        L.moe_cache_destroy.argtypes = [_vp]
        L.moe_cache_plan.restype = _i
        L.moe_cache_plan.argtypes = [_vp, _i, ctypes.POINTER(ctypes.c_int32), _i, ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(_i), ctypes.POINTER(_i)]
        L.moe_nvfp4_slice_bank.restype = _i
        L.moe_nvfp4_slice_bank.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _vp]
        L.moe_nvfp4_dequant.restype = _i
        L.moe_nvfp4_dequant.argtypes = [_vp, _vp, _vp, _i, _i, _vp, _vp]
        L.moe_nvfp4_dequant_slot.restype = _i
        L.moe_nvfp4_dequant_slot.argtypes = [_vp, _i, _i, _i, _vp, _vp]
        L.moe_release_streams.restype = _i
        L.moe_release_streams.argtypes = []
        L.moe_mxfp4_slot_bytes.restype = _sz
        L.moe_mxfp4_slot_bytes.argtypes = [_i, _i]
        L.moe_mxfp4_forward_workspace_bytes.restype = _sz
        L.moe_mxfp4_forward_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
        L.moe_mxfp4_forward.restype = _i
        L.moe_mxfp4_forward.argtypes = [ctypes.POINTER(LayerStruct), _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                        _vp, _sz, _vp]
        L.moe_mxfp4_route_forward_workspace_bytes.restype = _sz
        L.moe_mxfp4_route_forward_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
        L.moe_mxfp4_route_forward.restype = _i
        L.moe_mxfp4_route_forward.argtypes = [ctypes.POINTER(LayerStruct), _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp,
                                              _vp, _i, _vp, _sz, _vp]
        L.moe_mxfp4_dequant.restype = _i
        L.moe_mxfp4_dequant.argtypes = [_vp, _vp, _i, _i, _vp, _vp]
        L.moe_mxfp4_dequant_slot.restype = _i
        L.moe_mxfp4_dequant_slot.argtypes = [_vp, _i, _i, _i, _vp, _vp]
        L.moe_mxfp4_slice_bank.restype = _i
        L.moe_mxfp4_slice_bank.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _vp]
        L.moe_offload_device_bytes.restype = _sz
        L.moe_offload_device_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
        L.moe_offload_create.restype = _vp
        L.moe_offload_create.argtypes = [_i, _i, _i, _i, _i, _i, _vp, _i, ctypes.POINTER(_vp), _vp, _sz, _vp]
        L.moe_offload_destroy.restype = None
        L.moe_offload_destroy.argtypes = [_vp]
        L.moe_offload_layer.restype = _i
        L.moe_offload_layer.argtypes = [_vp, _i, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_i),
                                        ctypes.POINTER(_i)]
        L.moe_nvfp4_noalloc_scratch_bytes.restype = _sz
        L.moe_nvfp4_noalloc_scratch_bytes.argtypes = []
        L.moe_nvfp4_route_forward_noalloc.restype = _i
        L.moe_nvfp4_route_forward_noalloc.argtypes = [ctypes.POINTER(LayerStruct), _vp, _vp, _i, _vp, _vp, _vp, _vp,
                                                      _vp, _vp, _i, _vp]
        _lib = L
    return _lib


def check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def last_error() -> str:
    return lib().moe_last_error().decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- raw entry points (same names as the C ABI)

def moe_nvfp4_slot_bytes(H: int, I: int) -> int:
    return int(lib().moe_nvfp4_slot_bytes(H, I))


def moe_route_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(lib().moe_route_workspace_bytes(T, E, k))


def moe_route_topk(logits, T, E, k, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, ws=None,
                   ws_bytes=0, stream=None) -> int:
    return lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets),
                                _ptr(sorted_assign), _ptr(assign_pos), _ptr(ws), ws_bytes, _stream(stream))


def moe_router_logits(x, w_router, T, H, E, logits, stream=None) -> int:
    return lib().moe_router_logits(_ptr(x), _ptr(w_router), T, H, E, _ptr(logits), _stream(stream))


def moe_router_topk(x, w_router, T, H, E, k, logits, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos,
                    ws=None, ws_bytes=0, stream=None) -> int:
    return lib().moe_router_topk(_ptr(x), _ptr(w_router), T, H, E, k, _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                 _ptr(expert_offsets), _ptr(sorted_assign), _ptr(assign_pos), _ptr(ws), ws_bytes,
                                 _stream(stream))


def moe_nvfp4_forward_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib().moe_nvfp4_forward_workspace_bytes(T, H, I, E, k))


def moe_nvfp4_forward(layer: LayerStruct, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, y,
                      accumulate, ws, ws_bytes, stream=None) -> int:
    return lib().moe_nvfp4_forward(ctypes.byref(layer), _ptr(x), T, _ptr(topk_ids), _ptr(topk_w),
                                   _ptr(expert_offsets), _ptr(sorted_assign), _ptr(assign_pos), _ptr(y),
                                   int(accumulate), _ptr(ws), ws_bytes, _stream(stream))


def moe_nvfp4_route_forward_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib().moe_nvfp4_route_forward_workspace_bytes(T, H, I, E, k))


def moe_nvfp4_route_forward(layer: LayerStruct, logits, x, T, topk_ids, topk_w, expert_offsets, sorted_assign,
                            assign_pos, y, accumulate, ws, ws_bytes, stream=None) -> int:
    return lib().moe_nvfp4_route_forward(ctypes.byref(layer), _ptr(logits), _ptr(x), T, _ptr(topk_ids),
                                         _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_assign), _ptr(assign_pos),
                                         _ptr(y), int(accumulate), _ptr(ws), ws_bytes, _stream(stream))


def moe_nvfp4_noalloc_scratch_bytes() -> int:
    return int(lib().moe_nvfp4_noalloc_scratch_bytes())


def moe_nvfp4_route_forward_noalloc(layer: LayerStruct, logits, x, T, topk_ids, topk_w, expert_offsets,
                                    sorted_assign, assign_pos, y, accumulate, stream=None) -> int:
    return lib().moe_nvfp4_route_forward_noalloc(ctypes.byref(layer), _ptr(logits), _ptr(x), T, _ptr(topk_ids),
                                                 _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_assign),
                                                 _ptr(assign_pos), _ptr(y), int(accumulate), _stream(stream))


def moe_mxfp4_slot_bytes(H: int, I: int) -> int:
    return int(lib().moe_mxfp4_slot_bytes(H, I))


def moe_mxfp4_forward_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib().moe_mxfp4_forward_workspace_bytes(T, H, I, E, k))


def moe_mxfp4_forward(layer: LayerStruct, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, y,
                      accumulate, ws, ws_bytes, stream=None) -> int:
    return lib().moe_mxfp4_forward(ctypes.byref(layer), _ptr(x), T, _ptr(topk_ids), _ptr(topk_w),
                                   _ptr(expert_offsets), _ptr(sorted_assign), _ptr(assign_pos), _ptr(y),
                                   int(accumulate), _ptr(ws), ws_bytes, _stream(stream))


def moe_mxfp4_route_forward_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib().moe_mxfp4_route_forward_workspace_bytes(T, H, I, E, k))


def moe_mxfp4_route_forward(layer: LayerStruct, logits, x, T, topk_ids, topk_w, expert_offsets, sorted_assign,
                            assign_pos, y, accumulate, ws, ws_bytes, stream=None) -> int:
    return lib().moe_mxfp4_route_forward(ctypes.byref(layer), _ptr(logits), _ptr(x), T, _ptr(topk_ids),
                                         _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_assign), _ptr(assign_pos),
                                         _ptr(y), int(accumulate), _ptr(ws), ws_bytes, _stream(stream))


def moe_mxfp4_dequant(blocks_t, scales_t, N, K, out, stream=None) -> int:
    return lib().moe_mxfp4_dequant(_ptr(blocks_t), _ptr(scales_t), N, K, _ptr(out), _stream(stream))


def moe_mxfp4_dequant_slot(slot, H, I, matrix, out, stream=None) -> int:
    return lib().moe_mxfp4_dequant_slot(_ptr(slot), H, I, matrix, _ptr(out), _stream(stream))


def moe_mxfp4_slice_bank(src_bank, num_slots, H, I, r, n, dst_bank, stream=None) -> int:
    return lib().moe_mxfp4_slice_bank(_ptr(src_bank), num_slots, H, I, r, n, _ptr(dst_bank), _stream(stream))


def expert_cache_fill(cache_base, slot_bytes, num_slots, dst_slots, srcs, copy_stream=None, done_event=None) -> int:
    n = len(dst_slots)
    d = (ctypes.c_int32 * max(1, n))(*[int(v) for v in dst_slots])
    s = (ctypes.c_void_p * max(1, n))(*[int(v) for v in srcs])
    ev = None
    if done_event is not None:
        if isinstance(done_event, int):
            ev = done_event
        else:
            # torch creates the HIP event of a torch.cuda.Event on its first record; until then its handle is 0
            # and a stream's wait_event on it is a no-op.  Recording it once here creates it, and the library's
            # record after the copies is then the one that waits see.
            if not done_event.cuda_event:
                done_event.record(copy_stream if copy_stream is not None and not isinstance(copy_stream, int)
                                  else None)
            ev = done_event.cuda_event
            if not ev:
                raise MoeError(MOE_ERR_INVALID_ARGUMENT, "done_event has no HIP event")
    return lib().expert_cache_fill(_ptr(cache_base), slot_bytes, num_slots, d, s, n, _stream(copy_stream), ev)


def moe_nvfp4_slice_bank(src_bank, num_slots, H, I, r, n, dst_bank, stream=None) -> int:
    return lib().moe_nvfp4_slice_bank(_ptr(src_bank), num_slots, H, I, r, n, _ptr(dst_bank), _stream(stream))


def moe_nvfp4_dequant(codes, scales, globals_, rows, K, out, stream=None) -> int:
    return lib().moe_nvfp4_dequant(_ptr(codes), _ptr(scales), _ptr(globals_), rows, K, _ptr(out), _stream(stream))


def moe_nvfp4_dequant_slot(slot, H, I, matrix, out, stream=None) -> int:
    return lib().moe_nvfp4_dequant_slot(_ptr(slot), H, I, matrix, _ptr(out), _stream(stream))


def moe_release_streams() -> int:
    return lib().moe_release_streams()


def moe_offload_device_bytes(num_layers: int, num_experts: int, k: int, T_max: int, H: int, I: int) -> int:
    return int(lib().moe_offload_device_bytes(num_layers, num_experts, k, T_max, H, I))


class OffloadEngine:
    """moe_offload_create / moe_offload_layer / moe_offload_destroy: the layer-step engine over the expert cache.
    cache: device u8 [num_slots, slot_bytes]; host_ptrs: layer-major list of pinned slot addresses; dev_ws: a
    device u8 tensor of at least moe_offload_device_bytes(...) (kept alive by the engine object)."""

    def __init__(self, num_layers, num_experts, k, H, I, T_max, cache, host_ptrs, dev_ws, stream=None):
        n = num_layers * num_experts
        assert len(host_ptrs) == n
        self._ptrs = (ctypes.c_void_p * n)(*[int(p) for p in host_ptrs])
        self._keep = (cache, dev_ws)
        self._h = lib().moe_offload_create(num_layers, num_experts, k, H, I, T_max, _ptr(cache), cache.shape[0],
                                           self._ptrs, _ptr(dev_ws), dev_ws.numel(), _stream(stream))
        if not self._h:
            raise MoeError(MOE_ERR_INVALID_ARGUMENT, last_error())

    def layer(self, layer, logits, x, T, shared_slot, shared_gate_w, y, stream=None, copy_stream=None):
        """Runs one layer-step; returns (n_hit, n_miss)."""
        nh, nm = ctypes.c_int(), ctypes.c_int()
        check(lib().moe_offload_layer(self._h, layer, _ptr(logits), _ptr(x), T, _ptr(shared_slot),
                                      _ptr(shared_gate_w), _ptr(y), _stream(stream), _stream(copy_stream),
                                      ctypes.byref(nh), ctypes.byref(nm)))
        return nh.value, nm.value

    def close(self):
        if self._h:
            lib().moe_offload_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ExpertCache:
    """moe_cache_create / moe_cache_plan / moe_cache_destroy: the host-side slot manager."""

    def __init__(self, num_layers: int, num_experts: int, num_slots: int):
        self._h = lib().moe_cache_create(num_layers, num_experts, num_slots)
        if not self._h:
            raise MoeError(MOE_ERR_INVALID_ARGUMENT, last_error())
        self.E = num_experts

    def plan(self, layer: int, ids):
        """ids: iterable of routed expert ids.  Returns (slot_of_expert[E], miss_experts, miss_slots, n_hit)."""
        ids = [int(v) for v in ids]
        n = len(ids)
        a = (ctypes.c_int32 * max(1, n))(*ids)
        som = (ctypes.c_int32 * self.E)()
        me = (ctypes.c_int32 * max(1, n))()
        ms = (ctypes.c_int32 * max(1, n))()
        nm, nh = ctypes.c_int(), ctypes.c_int()
        check(lib().moe_cache_plan(self._h, layer, a, n, som, me, ms, ctypes.byref(nm), ctypes.byref(nh)))
        return list(som), list(me[:nm.value]), list(ms[:nm.value]), nh.value

    def close(self):
        if self._h:
            lib().moe_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
