"""moe_nvfp4_route_forward_noalloc (the allocation-free variant of
moe_nvfp4_route_forward, whose workspace is a fixed array inside the library)
against moe_nvfp4_route_forward with a caller workspace, through the C ABI
(marker: gpu).  The two run the same kernels on the same inputs, so routing
outputs and layer outputs must be identical bit for bit; the outputs are also
checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from expert_offload_serving_amd import _lib
from expert_offload_serving_amd import layer as dl
from expert_offload_serving_amd import synth
from tests.gpu_common import assert_close, device_layer, need_gpu

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def layer():
    need_gpu()
    _lib.lib()
    L = synth.permute_slots(synth.make_layer("decode_bs16", T=16, n_distinct=8, seed=61), np.random.default_rng(62),
                            spare=8)
    return L, device_layer(L)


def _outputs(T, E, k):
    r = dl.Routing.empty(T, E, k)
    for t in (r.ids, r.offsets, r.sorted_assign, r.assign_pos):
        t.fill_(-5)
    r.w.fill_(-5.0)
    return r, torch.full((T, 2560), 9.0, dtype=torch.float32, device="cuda")


def _noalloc(st, lg, x, T, r, y, stream=None):
    return _lib.moe_nvfp4_route_forward_noalloc(st, lg, x, T, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos,
                                                y, 0, stream)


def _regular(st, lg, x, T, r, y):
    nb = _lib.moe_nvfp4_route_forward_workspace_bytes(T, st.H, st.I, st.E, st.k)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    rc = _lib.moe_nvfp4_route_forward(st, lg, x, T, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, y, 0, ws,
                                      nb)
    return rc, ws


def _same(a, b, what):
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32)), what


def test_noalloc_matches_route_forward_two_calls(layer):
    """Two calls in a row, the second with fewer tokens (T = 16, then T = 3), each equal to the regular entry
    point with a caller workspace, and to the oracle."""
    L, dev = layer
    st = dev.struct()
    assert _lib.moe_nvfp4_noalloc_scratch_bytes() >= _lib.moe_nvfp4_route_forward_workspace_bytes(16, 2560, 640,
                                                                                                   256, 8)
    for T, seed in ((16, 71), (3, 72)):
        _announce(f"noalloc vs route_forward T={T}")
        xb, lgn = synth.fresh_tokens(seed, T, L.H, L.E, "uniform")
        x, lg = dl.to_device_bf16(xb), torch.from_numpy(lgn).cuda()
        r1, y1 = _outputs(T, L.E, L.k)
        _lib.check(_noalloc(st, lg, x, T, r1, y1))
        r2, y2 = _outputs(T, L.E, L.k)
        rc, _ = _regular(st, lg, x, T, r2, y2)
        _lib.check(rc)
        torch.cuda.synchronize()
        for name in ("ids", "w", "offsets", "sorted_assign", "assign_pos"):
            _same(getattr(r1, name), getattr(r2, name), f"T={T} {name}")
        _same(y1, y2, f"T={T} y")
        ids, w = oracle.route(lgn, L.k)
        assert np.array_equal(r1.ids.cpu().numpy(), ids)
        ref = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, xb, ids, w)
        assert_close(y1.cpu().numpy(), ref, f"noalloc T={T} vs oracle")


def test_noalloc_graph_replays(layer):
    """Captured in a HIP graph (a caller that cannot allocate): replays, with eager work between them, equal the
    eager call."""
    L, dev = layer
    st = dev.struct()
    T = 8
    _announce(f"noalloc graph replays T={T}")
    xb, lgn = synth.fresh_tokens(81, T, L.H, L.E, "uniform")
    x, lg = dl.to_device_bf16(xb), torch.from_numpy(lgn).cuda()
    r, y = _outputs(T, L.E, L.k)
    _lib.check(_noalloc(st, lg, x, T, r, y))
    torch.cuda.synchronize()
    want = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _lib.check(_noalloc(st, lg, x, T, r, y, stream=s))
    torch.cuda.synchronize()
    for rep in range(3):
        y.zero_()
        r2, y2 = _outputs(3, L.E, L.k)  # eager work on the same scratch between replays
        _lib.check(_noalloc(st, lg[:3].contiguous(), x[:3].contiguous(), 3, r2, y2))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(y, want, f"replay {rep}")


def test_noalloc_refusals_enqueue_nothing(layer):
    """Shapes outside the allocation-free variant's reach are refused with nothing written: the prefill path
    (T = 17), and a decode shape whose workspace exceeds the fixed array (I = 1280 at T = 16)."""
    L, dev = layer
    st = dev.struct()
    T = 17
    xb, lgn = synth.fresh_tokens(91, T, L.H, L.E, "uniform")
    x, lg = dl.to_device_bf16(xb), torch.from_numpy(lgn).cuda()
    r, y = _outputs(T, L.E, L.k)
    assert _noalloc(st, lg, x, T, r, y) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert "decode path" in _lib.last_error()
    big = dev.struct()
    big.I = 1280
    big.slot_bytes = _lib.moe_nvfp4_slot_bytes(2560, 1280)
    assert _lib.moe_nvfp4_route_forward_workspace_bytes(16, 2560, 1280, 256, 8) > \
        _lib.moe_nvfp4_noalloc_scratch_bytes()
    r2, y2 = _outputs(16, L.E, L.k)
    assert _noalloc(big, lg[:16].contiguous(), x[:16].contiguous(), 16, r2, y2) == _lib.MOE_ERR_WORKSPACE_TOO_SMALL
    assert _noalloc(st, lg, x, 0, r, y) == _lib.MOE_OK  # T = 0: a no-op
    torch.cuda.synchronize()
    for rr, yy in ((r, y), (r2, y2)):
        assert bool((rr.ids == -5).all()) and bool((rr.offsets == -5).all())
        assert bool((yy == 9.0).all())
