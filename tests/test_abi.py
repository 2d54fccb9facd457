"""The C ABI library on the CPU: it loads, exports every function declared in
include/moe_nvfp4.h, validates arguments before touching the GPU, and its
host-side cache slot manager reproduces the oracle's LRU model exactly."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from expert_offload_serving_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "moe_nvfp4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text))
    return sorted(n for n in names if n.startswith(("moe_", "expert_")))


def test_library_exports_every_declared_function():
    L = _lib.lib()
    decl = _declared_functions()
    assert len(decl) >= 12
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(_lib.EXPORTED) == decl


def test_slot_bytes():
    assert _lib.moe_nvfp4_slot_bytes(2560, 640) == 2_780_160
    assert _lib.moe_nvfp4_slot_bytes(2560, 320) == 1_395_200
    assert _lib.moe_nvfp4_slot_bytes(256, 64) == 29_184
    for H, I in [(2560, 641), (2576, 640), (0, 64), (-32, 64), (256, 16), (96, 32), (320, 64)]:
        assert _lib.moe_nvfp4_slot_bytes(H, I) == 0
    for H, I in [(128, 32), (2560, 640), (7168, 2048)]:
        assert _lib.moe_nvfp4_slot_bytes(H, I) == oracle.slot_bytes(H, I)


def test_route_validation_without_gpu():
    dummy = 0x1000
    c = _lib.moe_route_topk
    assert c(dummy, 4, 8, 9, dummy, dummy, dummy, dummy, dummy, None, 0, 0) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert c(dummy, -1, 8, 2, dummy, dummy, dummy, dummy, dummy, None, 0, 0) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert c(dummy, 4, 2048, 2, dummy, dummy, dummy, dummy, dummy, None, 0, 0) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert c(dummy, 4, 8, 0, dummy, dummy, dummy, dummy, dummy, None, 0, 0) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert c(None, 4, 8, 2, dummy, dummy, dummy, dummy, dummy, None, 0, 0) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert "null" in _lib.last_error()
    assert c(None, 0, 8, 2, None, None, None, None, None, None, 0, 0) == _lib.MOE_OK  # T == 0 is a no-op


def _layer(H=2560, I=640, E=256, k=8, slot_bytes=None, bank=0x100000, shared=None, wg=None, num_slots=257):
    s = _lib.LayerStruct()
    s.H, s.I, s.E, s.k = H, I, E, k
    s.bank_base = bank
    s.slot_bytes = _lib.moe_nvfp4_slot_bytes(H, I) if slot_bytes is None else slot_bytes
    s.num_slots = num_slots
    s.slot_of_expert = 0x2000
    s.shared_slot = shared
    s.shared_gate_w = wg
    return s


def test_forward_validation_without_gpu():
    d = 0x3000
    f = lambda L, T=1, ws=0x200000, nb=1 << 30, acc=0: _lib.moe_nvfp4_forward(L, d, T, d, d, d, d, d, d, acc, ws, nb, 0)
    assert f(_layer(I=650)) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert f(_layer(slot_bytes=123)) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert "slot_bytes" in _lib.last_error()
    assert f(_layer(k=300)) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(), T=-2) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(), acc=2) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(bank=0x100010)) == _lib.MOE_ERR_INVALID_ARGUMENT          # misaligned bank
    assert f(_layer(shared=0x400000, wg=None)) == _lib.MOE_ERR_INVALID_ARGUMENT  # shared without gate
    need = _lib.moe_nvfp4_forward_workspace_bytes(16, 2560, 640, 256, 8)
    assert need > 16 * 9 * (2560 + 640) * 4
    assert f(_layer(), T=16, nb=need - 1) == _lib.MOE_ERR_WORKSPACE_TOO_SMALL
    assert f(_layer(), T=16, ws=0x200010, nb=need) == _lib.MOE_ERR_INVALID_ARGUMENT  # misaligned workspace
    assert f(_layer(), T=0) == _lib.MOE_OK


def test_route_forward_validation_without_gpu():
    d = 0x3000
    f = lambda L, lg=d, T=1, ws=0x200000, nb=1 << 30: _lib.moe_nvfp4_route_forward(L, lg, d, T, d, d, d, d, d, d, 0,
                                                                                  ws, nb, 0)
    assert f(_layer(I=650)) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert f(_layer(), lg=None) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert "logits" in _lib.last_error()
    assert f(_layer(k=300)) == _lib.MOE_ERR_INVALID_ARGUMENT
    need = _lib.moe_nvfp4_route_forward_workspace_bytes(16, 2560, 640, 256, 8)
    assert need >= _lib.moe_nvfp4_forward_workspace_bytes(16, 2560, 640, 256, 8)
    assert f(_layer(), T=16, nb=need - 1) == _lib.MOE_ERR_WORKSPACE_TOO_SMALL
    big = _lib.moe_nvfp4_route_forward_workspace_bytes(4096, 2560, 640, 256, 8)
    assert big >= _lib.moe_nvfp4_forward_workspace_bytes(4096, 2560, 640, 256, 8) + \
        _lib.moe_route_workspace_bytes(4096, 256, 8)
    assert f(_layer(), T=0) == _lib.MOE_OK


def test_mx_route_forward_validation_without_gpu():
    d = 0x3000
    mx = _lib.moe_mxfp4_slot_bytes(2560, 640)
    f = lambda L, lg=d, T=1, ws=0x200000, nb=1 << 30: _lib.moe_mxfp4_route_forward(L, lg, d, T, d, d, d, d, d, d, 0,
                                                                                  ws, nb, 0)
    assert f(_layer(slot_bytes=mx), lg=None) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert "logits" in _lib.last_error()
    assert f(_layer()) == _lib.MOE_ERR_INVALID_ARGUMENT  # an NVFP4 slot size
    # T = 17 runs the prefill path: its workspace is larger than the one given
    assert f(_layer(slot_bytes=mx), T=17, nb=1 << 10) == _lib.MOE_ERR_WORKSPACE_TOO_SMALL
    need = _lib.moe_mxfp4_route_forward_workspace_bytes(16, 2560, 640, 256, 8)
    assert need >= _lib.moe_mxfp4_forward_workspace_bytes(16, 2560, 640, 256, 8) + \
        _lib.moe_route_workspace_bytes(16, 256, 8)
    assert f(_layer(slot_bytes=mx), T=16, nb=need - 1) == _lib.MOE_ERR_WORKSPACE_TOO_SMALL
    assert _lib.moe_mxfp4_route_forward_workspace_bytes(17, 2560, 640, 256, 8) >= \
        _lib.moe_mxfp4_forward_workspace_bytes(17, 2560, 640, 256, 8) > 1 << 10
    assert f(_layer(slot_bytes=mx), T=0) == _lib.MOE_OK


def test_forward_refuses_buffers_of_2gib():
    """Every buffer the kernels address through 32-bit offsets must stay below 2 GiB: shapes whose workspace or
    output would reach it are refused before anything is enqueued (no GPU needed)."""
    d = 0x3000
    f = lambda L, T: _lib.moe_nvfp4_forward(L, d, T, d, d, d, d, d, d, 0, 0x200000, 1 << 62, 0)
    # the prefill workspace first reaches 2 GiB at T = 33,939 for these shapes
    assert _lib.moe_nvfp4_forward_workspace_bytes(33_938, 2560, 640, 256, 8) < 1 << 31
    assert _lib.moe_nvfp4_forward_workspace_bytes(33_939, 2560, 640, 256, 8) >= 1 << 31
    assert f(_layer(), 33_939) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert "2 GiB" in _lib.last_error()
    assert f(_layer(), 200_000) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert f(_layer(), 0) == _lib.MOE_OK  # T = 0 stays a valid no-op


def test_other_entry_points_validate():
    ds = _lib.moe_nvfp4_dequant_slot
    assert ds(0x100, 96, 32, 0, 0x100, 0) == _lib.MOE_ERR_UNSUPPORTED_SHAPE   # H % 128
    assert ds(0x100, 128, 48, 0, 0x100, 0) == _lib.MOE_ERR_UNSUPPORTED_SHAPE  # I % 32
    assert ds(0x100, 128, 32, 2, 0x100, 0) == _lib.MOE_ERR_INVALID_ARGUMENT   # matrix
    assert ds(0x101, 128, 32, 0, 0x100, 0) == _lib.MOE_ERR_INVALID_ARGUMENT   # misaligned
    assert ds(None, 128, 32, 0, 0x100, 0) == _lib.MOE_ERR_INVALID_ARGUMENT
    dq = _lib.moe_nvfp4_dequant
    assert dq(0x100, 0x100, 0x100, 4, 40, 0x100, 0) == _lib.MOE_ERR_UNSUPPORTED_SHAPE   # K % 16
    assert dq(0x100, 0x100, 0x100, -1, 32, 0x100, 0) == _lib.MOE_ERR_UNSUPPORTED_SHAPE  # rows < 0
    assert dq(0x102, 0x100, 0x100, 4, 32, 0x100, 0) == _lib.MOE_ERR_INVALID_ARGUMENT    # codes misaligned
    assert dq(0x100, 0x100, 0x100, 4, 32, 0x108, 0) == _lib.MOE_ERR_INVALID_ARGUMENT    # out misaligned
    assert dq(0x100, None, 0x100, 4, 32, 0x100, 0) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert dq(None, None, None, 0, 32, None, 0) == _lib.MOE_OK                          # rows == 0: no-op
    assert _lib.moe_release_streams() == _lib.MOE_OK                                    # nothing created yet
    assert _lib.moe_nvfp4_slice_bank(1, 4, 2560, 640, 0, 8, 1, 0) == _lib.MOE_ERR_UNSUPPORTED_SHAPE  # 80 % 32 != 0
    assert _lib.moe_nvfp4_slice_bank(1, 4, 2560, 640, 2, 2, 1, 0) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert _lib.moe_nvfp4_slice_bank(1, 0, 2560, 640, 0, 2, 1, 0) == _lib.MOE_OK
    assert _lib.expert_cache_fill(1, 64, 4, [4], [1], 0, None) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert _lib.expert_cache_fill(1, 64, 4, [-1], [1], 0, None) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert _lib.expert_cache_fill(1, 64, 4, [0], [0], 0, None) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert _lib.expert_cache_fill(None, 64, 4, [], [], 0, None) == _lib.MOE_OK


def test_cache_manager_matches_oracle_lru():
    rng = np.random.default_rng(12)
    steps, L, E, n, C = 30, 4, 32, 10, 25
    ids = rng.integers(0, E, (steps, L, n), dtype=np.int32)
    hits, misses, smap, mslots = oracle.lru_run(ids, E, C)
    mgr = _lib.ExpertCache(L, E, C)
    for st in range(steps):
        for l in range(L):
            som, me, ms, nh = mgr.plan(l, ids[st, l])
            assert nh == hits[st, l] and len(me) == misses[st, l]
            assert list(ms) == list(mslots[st, l][:misses[st, l]])
            assert som == list(smap[st, l])
            assert me == sorted(me) and set(me) <= set(ids[st, l].tolist())


def test_cache_manager_errors():
    with pytest.raises(_lib.MoeError):
        _lib.ExpertCache(0, 4, 4)
    mgr = _lib.ExpertCache(1, 8, 2)
    with pytest.raises(_lib.MoeError):
        mgr.plan(0, [0, 1, 2])      # three distinct experts, two slots
    with pytest.raises(_lib.MoeError):
        mgr.plan(0, [9])            # id out of range
    with pytest.raises(_lib.MoeError):
        mgr.plan(1, [0])            # layer out of range
