"""CPU oracle for the NVFP4 routed-MoE layer (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke
check and the CPU-baseline leg of the benchmark.  The HIP library and its
Python binding never import this package.  Every function follows the plain
definition written out in oracle.c (fp32 dequant, double accumulation).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall"]


def build() -> str:
    """Compile oracle.c with gcc into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None

_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_e2m1.restype = ctypes.c_double
        L.oracle_e2m1.argtypes = [ctypes.c_int]
        L.oracle_e4m3.restype = ctypes.c_double
        L.oracle_e4m3.argtypes = [ctypes.c_int]
        L.oracle_dequant.restype = None
        L.oracle_dequant.argtypes = [_u8p, _u8p, _f32p, ctypes.c_int, ctypes.c_int, _f32p]
        L.oracle_shape_ok.restype = ctypes.c_int
        L.oracle_shape_ok.argtypes = [ctypes.c_int, ctypes.c_int]
        L.oracle_dequant_slot.restype = ctypes.c_int
        L.oracle_dequant_slot.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f32p]
        L.oracle_unpack_slot.restype = ctypes.c_int
        L.oracle_unpack_slot.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, _u8p, _f32p]
        L.oracle_route.restype = ctypes.c_int
        L.oracle_route.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _f32p]
        L.oracle_router_logits.restype = None
        L.oracle_router_logits.argtypes = [_u16p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f32p]
        L.oracle_permute.restype = None
        L.oracle_permute.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _i32p, _i32p]
        L.oracle_shared_gate.restype = None
        L.oracle_shared_gate.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _u16p, _f64p]
        L.oracle_slot_bytes.restype = ctypes.c_size_t
        L.oracle_slot_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        L.oracle_forward.restype = ctypes.c_int
        L.oracle_forward.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, ctypes.c_size_t,
                                     _i32p, ctypes.c_long, _u16p, _u16p, ctypes.c_int, _i32p, _f32p,
                                     ctypes.c_void_p, ctypes.c_int, _f32p, ctypes.c_int]
        L.oracle_slice_slot.restype = ctypes.c_int
        L.oracle_slice_slot.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p]
        L.oracle_e8m0.restype = ctypes.c_double
        L.oracle_e8m0.argtypes = [ctypes.c_int]
        L.oracle_mx_dequant_t.restype = None
        L.oracle_mx_dequant_t.argtypes = [_u8p, _u8p, ctypes.c_int, ctypes.c_int, _f32p]
        L.oracle_mx_slot_bytes.restype = ctypes.c_size_t
        L.oracle_mx_slot_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        L.oracle_mx_dequant_slot.restype = ctypes.c_int
        L.oracle_mx_dequant_slot.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f32p]
        L.oracle_mx_unpack_slot.restype = ctypes.c_int
        L.oracle_mx_unpack_slot.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, _u8p]
        L.oracle_mx_slice_slot.restype = ctypes.c_int
        L.oracle_mx_slice_slot.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p]
        L.oracle_mx_forward.restype = ctypes.c_int
        L.oracle_mx_forward.argtypes = L.oracle_forward.argtypes
        L.oracle_lru_run.restype = ctypes.c_int
        L.oracle_lru_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, _i32p, _i32p, _i32p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(int(code))


def e4m3(byte: int) -> float:
    return lib().oracle_e4m3(int(byte))


def slot_bytes(H: int, I: int) -> int:
    return int(lib().oracle_slot_bytes(H, I))


def dequant(codes, scales, globals_) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    g = np.ascontiguousarray(globals_, dtype=np.float32)
    rows, K = codes.shape[0], codes.shape[1] * 2
    assert scales.shape == (rows, K // 16) and g.shape == (rows,)
    out = np.empty((rows, K), dtype=np.float32)
    lib().oracle_dequant(codes, scales, g, rows, K, out)
    return out


def _matrix_shape(H: int, I: int, matrix: int):
    if not lib().oracle_shape_ok(H, I) or matrix not in (0, 1):
        raise ValueError(f"bad slot shape H={H} I={I} matrix={matrix}")
    return (2 * I, H) if matrix == 0 else (H, I)


def dequant_slot(slot, H: int, I: int, matrix: int) -> np.ndarray:
    """fp32 [N, K] of gate_up (matrix 0, [2I, H]) or down (matrix 1, [H, I]) of one slot."""
    N, K = _matrix_shape(H, I, matrix)
    slot = np.ascontiguousarray(slot, dtype=np.uint8).reshape(-1)
    out = np.empty((N, K), dtype=np.float32)
    lib().oracle_dequant_slot(slot, H, I, matrix, out)
    return out


def unpack_slot(slot, H: int, I: int, matrix: int):
    """Row-major (codes [N, K/2], scales [N, K/16], globals [N]) of one matrix of a slot."""
    N, K = _matrix_shape(H, I, matrix)
    slot = np.ascontiguousarray(slot, dtype=np.uint8).reshape(-1)
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 16), dtype=np.uint8)
    g = np.empty(N, dtype=np.float32)
    lib().oracle_unpack_slot(slot, H, I, matrix, codes, scales, g)
    return codes, scales, g


def route(logits, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    if lib().oracle_route(logits, T, E, k, ids, w) != 0:
        raise ValueError("NaN router logit")
    return ids, w


def router_logits(x, w_router) -> np.ndarray:
    """logits [T, E] = x [T, H] . w_router [E, H]^T (bf16 bit patterns in), double accumulation, f32 out."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w_router = np.ascontiguousarray(w_router, dtype=np.uint16)
    T, H = x.shape
    E = w_router.shape[0]
    assert w_router.shape[1] == H
    out = np.empty((T, E), dtype=np.float32)
    lib().oracle_router_logits(x, w_router, T, H, E, out)
    return out


def permute(ids, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_assign = np.empty(T * k, dtype=np.int32)
    assign_pos = np.empty(T * k, dtype=np.int32)
    lib().oracle_permute(ids, T, E, k, offsets, sorted_assign, assign_pos)
    return offsets, sorted_assign, assign_pos


def shared_gate(x, wg) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T, H = x.shape
    s = np.empty(T, dtype=np.float64)
    lib().oracle_shared_gate(x, T, H, np.ascontiguousarray(wg, dtype=np.uint16), s)
    return s


def forward(H, I, E, k, bank, slot_of_expert, shared_slot, wg, x, ids, w, tokens=None, nthreads: int = 0,
            fmt: str = "nvfp4"):
    """Layer output y (f32) for all tokens, or for the listed tokens in list order.  fmt: "nvfp4" or "mxfp4"
    (the bank's slot format)."""
    bank = np.ascontiguousarray(bank, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T = x.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    if tokens is None:
        tok_ptr, n = None, T
        keep = None
    else:
        keep = np.ascontiguousarray(tokens, dtype=np.int32)
        tok_ptr, n = keep.ctypes.data, keep.size
    y = np.empty((n, H), dtype=np.float32)
    fn = {"nvfp4": lib().oracle_forward, "mxfp4": lib().oracle_mx_forward}[fmt]
    sb = bank.shape[-1] if bank.ndim == 2 else (slot_bytes(H, I) if fmt == "nvfp4" else mx_slot_bytes(H, I))
    rc = fn(H, I, E, k, bank.reshape(-1), sb,
                              np.ascontiguousarray(slot_of_expert, dtype=np.int32), int(shared_slot),
                              np.ascontiguousarray(wg, dtype=np.uint16), x, T, ids, w, tok_ptr, n, y, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_forward: bad arguments")
    del keep
    return y


def slice_slot(slot, H: int, I: int, r: int, n: int) -> np.ndarray:
    slot = np.ascontiguousarray(slot, dtype=np.uint8).reshape(-1)
    out = np.empty(slot_bytes(H, I // n), dtype=np.uint8)
    if lib().oracle_slice_slot(slot, H, I, r, n, out) != 0:
        raise ValueError("slice is not a valid slot shape (I/n must be a multiple of 32)")
    return out


def lru_run(ids, E: int, C: int, want_maps: bool = True):
    """ids: int32 [steps, L, T*k].  Returns hits [steps, L], misses [steps, L], slot_map, miss_slots."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    steps, L, n = ids.shape
    hits = np.empty((steps, L), dtype=np.int32)
    misses = np.empty((steps, L), dtype=np.int32)
    smap = np.empty((steps, L, E), dtype=np.int32) if want_maps else None
    mslots = np.empty((steps, L, n), dtype=np.int32) if want_maps else None
    rc = lib().oracle_lru_run(L, E, C, steps, n, 1, ids, hits, misses,
                              smap.ctypes.data if want_maps else None, mslots.ctypes.data if want_maps else None)
    if rc != 0:
        raise ValueError("cache smaller than one layer-step's distinct experts")
    return hits, misses, smap, mslots


# ---------------------------------------------------------------- MXFP4

def e8m0(byte: int) -> float:
    return lib().oracle_e8m0(int(byte))


def mx_slot_bytes(H: int, I: int) -> int:
    return int(lib().oracle_mx_slot_bytes(H, I))


def mx_dequant_t(blocks_t, scales_t) -> np.ndarray:
    """fp32 W [N, K] of an MXFP4 matrix stored transposed: blocks_t u8 [K/2, N], scales_t u8 [K/32, N]."""
    blocks_t = np.ascontiguousarray(blocks_t, dtype=np.uint8)
    scales_t = np.ascontiguousarray(scales_t, dtype=np.uint8)
    K, N = blocks_t.shape[0] * 2, blocks_t.shape[1]
    assert scales_t.shape == (K // 32, N)
    out = np.empty((N, K), dtype=np.float32)
    lib().oracle_mx_dequant_t(blocks_t, scales_t, N, K, out)
    return out


def mx_dequant_slot(slot, H: int, I: int, matrix: int) -> np.ndarray:
    N, K = _matrix_shape(H, I, matrix)
    slot = np.ascontiguousarray(slot, dtype=np.uint8).reshape(-1)
    out = np.empty((N, K), dtype=np.float32)
    lib().oracle_mx_dequant_slot(slot, H, I, matrix, out)
    return out


def mx_unpack_slot(slot, H: int, I: int, matrix: int):
    """The transposed checkpoint tensors (blocks_t [K/2, N], scales_t [K/32, N]) of one matrix of an MXFP4 slot."""
    N, K = _matrix_shape(H, I, matrix)
    slot = np.ascontiguousarray(slot, dtype=np.uint8).reshape(-1)
    blocks_t = np.empty((K // 2, N), dtype=np.uint8)
    scales_t = np.empty((K // 32, N), dtype=np.uint8)
    lib().oracle_mx_unpack_slot(slot, H, I, matrix, blocks_t, scales_t)
    return blocks_t, scales_t


def mx_slice_slot(slot, H: int, I: int, r: int, n: int) -> np.ndarray:
    slot = np.ascontiguousarray(slot, dtype=np.uint8).reshape(-1)
    out = np.empty(mx_slot_bytes(H, I // n), dtype=np.uint8)
    if lib().oracle_mx_slice_slot(slot, H, I, r, n, out) != 0:
        raise ValueError("slice is not a valid slot shape (I/n must be a multiple of 32)")
    return out
