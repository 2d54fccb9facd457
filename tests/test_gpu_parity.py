"""GPU parity of the HIP library against the CPU oracle (marker: gpu).

Integer work (top-k ids, the permutation, dequantised bits, sliced bytes)
must match bit for bit; layer outputs must be within relative L2 2e-3 and
max |err| <= 1e-2 * max |ref|.  Inputs are the seeded synthetic workloads of
expert_offload_serving_amd.synth.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from expert_offload_serving_amd import _lib
from expert_offload_serving_amd import layer as dl
from expert_offload_serving_amd import synth
from tests.gpu_common import assert_close, device_layer, device_logits, device_x, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    _lib.lib()  # loud failure if the library is missing on a GPU machine


def _announce(msg):
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------- dequant

def test_dequant_bitexact_all_code_scale_pairs():
    """Every (code, scale byte) pair under several globals, in both matrices of a slot, bit for bit against the
    oracle's dequant of the same row-major values."""
    _announce("dequant 16 codes x 256 scales x 5 globals (H=256, I=640)")
    H, I = 256, 640
    gl = np.array([1.0, 0.5, 3.7e-5, -2.25, 1.0e30], dtype=np.float32)
    def all_pairs(N, K, shift):
        codes_row = np.array([((2 * j + shift) % 16) | (((2 * j + 1 + shift) % 16) << 4) for j in range(K // 2)],
                             dtype=np.uint8)
        codes = np.tile(codes_row, (N, 1))
        blocks = np.arange(N * (K // 16)).reshape(N, K // 16)
        scales = ((blocks + shift) % 256).astype(np.uint8)
        globals_ = gl[(np.arange(N) * 7 + shift) % len(gl)]
        return codes, scales, globals_
    gu, dn = all_pairs(2 * I, H, 0), all_pairs(H, I, 3)
    slot = synth.pack_slot(gu, dn, H, I)
    dslot = torch.from_numpy(slot).cuda()
    for m, parts in enumerate((gu, dn)):
        want = oracle.dequant(*parts)
        assert np.array_equal(np.isnan(want), np.isnan(oracle.dequant_slot(slot, H, I, m)))
        got = dl.dequant_slot(dslot, H, I, m).cpu().numpy()
        nan_w, nan_g = np.isnan(want), np.isnan(got)
        assert np.array_equal(nan_w, nan_g)
        assert np.array_equal(want[~nan_w].view(np.uint32), got[~nan_g].view(np.uint32))


def test_dequant_bitexact_real_bank():
    _announce("dequant real expert slot (H=2560, I=640)")
    H, I = 2560, 640
    slot = synth.random_expert_slot(np.random.default_rng(7), H, I)
    dslot = torch.from_numpy(slot).cuda()
    for m in (0, 1):
        want = oracle.dequant_slot(slot, H, I, m)
        got = dl.dequant_slot(dslot, H, I, m)
        assert np.array_equal(want.view(np.uint32), got.cpu().numpy().view(np.uint32))


def _bits_equal(got: np.ndarray, want: np.ndarray):
    """Equal bit patterns, with every NaN position matching (NaN payloads are not compared)."""
    nan_w, nan_g = np.isnan(want), np.isnan(got)
    assert np.array_equal(nan_w, nan_g)
    assert np.array_equal(want[~nan_w].view(np.uint32), got[~nan_g].view(np.uint32))


def test_dequant_rowmajor_bitexact_all_code_scale_pairs():
    """The row-major decode entry (no slot layout involved): every (code, scale byte) pair under several globals,
    ragged row counts and K from one scale block up, bit for bit against the oracle's dequant."""
    gl = np.array([1.0, 0.5, 3.7e-5, -2.25, 1.0e30, 2.0 ** -126, 0.0], dtype=np.float32)
    # rows x K = 16 codes in every position of a 16-block, 256 scale bytes, each (code, scale) pair present
    codes_row = np.array([(2 * j % 16) | (((2 * j + 1) % 16) << 4) for j in range(8)], dtype=np.uint8)
    for rows, K, what in [(256 * 7, 16, "all pairs x globals"), (37, 48, "ragged"), (1, 4096, "one long row"),
                          (1000, 32, "many rows")]:
        _announce(f"dequant row-major rows={rows} K={K} ({what})")
        codes = np.tile(codes_row, (rows, K // 16))
        r_ = np.arange(rows)[:, None]
        blocks = np.arange(K // 16)[None, :]
        scales = ((r_ + 37 * blocks) % 256).astype(np.uint8)
        if what.startswith("all pairs"):
            scales = (np.arange(rows)[:, None] % 256).astype(np.uint8).repeat(K // 16, axis=1)
        globals_ = gl[(np.arange(rows) // 256 + np.arange(rows)) % len(gl)]
        want = oracle.dequant(codes, scales, globals_)
        got = dl.dequant(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                         torch.from_numpy(globals_).cuda()).cpu().numpy()
        _bits_equal(got, want)


# ---------------------------------------------------------------- routing

def _route_both(logits: np.ndarray, k: int):
    T, E = logits.shape
    r = dl.route(torch.from_numpy(np.ascontiguousarray(logits)).cuda(), k)
    torch.cuda.synchronize()
    ids, w = oracle.route(logits, k)
    off, srt, pos = oracle.permute(ids, E)
    return r, (ids, w, off, srt, pos)


def _check_route(logits, k, what):
    _announce(f"route {what} T={logits.shape[0]} E={logits.shape[1]} k={k}")
    r, (ids, w, off, srt, pos) = _route_both(logits, k)
    assert np.array_equal(r.ids.cpu().numpy(), ids), what
    assert np.array_equal(r.offsets.cpu().numpy(), off), what
    assert np.array_equal(r.sorted_assign.cpu().numpy(), srt), what
    assert np.array_equal(r.assign_pos.cpu().numpy(), pos), what
    gw = r.w.cpu().numpy()
    ulps = np.abs(gw.view(np.int32).astype(np.int64) - w.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, f"{what}: weights differ by {ulps.max()} ulp"


@pytest.mark.parametrize("name", ["tiny", "decode_bs1", "decode_bs16", "prefill_2048"])
def test_route_bitexact_configs(name):
    H, I, E, k, T, seed, kind = synth.CONFIGS[name]
    rng = np.random.default_rng(seed)
    logits = synth.make_logits(rng, T, E, kind)
    _check_route(logits, k, name)


def test_route_ties_zero_counts_and_extremes():
    rng = np.random.default_rng(1)
    # heavy ties: logits from a tiny set of values
    logits = rng.integers(0, 3, (37, 64)).astype(np.float32)
    logits[:, 5] = -0.0
    logits[:, 6] = 0.0
    _check_route(logits, 8, "ties")
    # zero-count experts: 16 experts forced to lose (prefill case with skew)
    lg = synth.make_logits(np.random.default_rng(2), 300, 256, "zipf")
    lg[:, :16] = -1e30
    _check_route(lg, 8, "zero-count experts")
    _check_route(rng.standard_normal((5, 32)).astype(np.float32), 1, "k=1")
    _check_route(rng.standard_normal((3, 16)).astype(np.float32), 16, "k=E")
    _check_route(rng.standard_normal((20, 1024)).astype(np.float32), 8, "E=1024 two-kernel path")
    _check_route(rng.standard_normal((16, 1024)).astype(np.float32), 300, "k=300 fused path")


# ---------------------------------------------------------------- router projection

def _router_inputs(T, H, E, seed):
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = synth.f32_to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    return x, w


def _check_router_logits(got, x, w, what):
    """fp32 accumulation of H exact bf16 products: |err| <= H * 2^-24 * sum_h |x_h w_h| (plus the final rounding)."""
    ref = oracle.router_logits(x, w).astype(np.float64)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    bound = (x.shape[1] + 1) * 2.0 ** -24 * (np.abs(xf) @ np.abs(wf).T)
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= bound).all(), f"{what}: max err/bound {(err / np.maximum(bound, 1e-300)).max():.3g}"
    return ref


@pytest.mark.parametrize("T,H,E", [(1, 2560, 256), (3, 2560, 256), (16, 2560, 256), (17, 2560, 256),
                                   (300, 2560, 256), (5, 256, 8), (20, 512, 1000), (33, 768, 40), (2, 256, 1),
                                   (16, 4096, 1024)])
def test_router_logits_vs_oracle(T, H, E):
    _announce(f"router logits T={T} H={H} E={E}")
    x, w = _router_inputs(T, H, E, 100 + T)
    got = dl.router_logits(torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    _check_router_logits(got.cpu().numpy(), x, w, f"T={T} H={H} E={E}")


def test_router_logits_prefill_2048_sampled_rows_and_repeatable():
    T, H, E = 2048, 2560, 256
    _announce(f"router logits T={T} H={H} E={E} (sampled rows, repeat)")
    x, w = _router_inputs(T, H, E, 7)
    xd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    a = dl.router_logits(xd, wd)
    b = dl.router_logits(xd, wd)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "router logits not bit-identical between calls"
    rows = np.array([0, 1, 31, 32, 33, 1000, 2015, 2047])
    _check_router_logits(a.cpu().numpy()[rows], x[rows], w, "T=2048 sampled")


def test_router_topk_selects_on_its_logits():
    # the top-k decision is taken on the kernel's fp32 logits: the oracle's routing of those same logits must match
    for T, H, E, k in [(1, 2560, 256, 8), (16, 2560, 256, 8), (300, 2560, 256, 8), (4, 256, 8, 2)]:
        _announce(f"router topk T={T} H={H} E={E} k={k}")
        x, w = _router_inputs(T, H, E, 11 + T)
        logits, r = dl.router_route(torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), k)
        torch.cuda.synchronize()
        lg = logits.cpu().numpy()
        _check_router_logits(lg, x, w, f"topk T={T}")
        ids, wt = oracle.route(lg, k)
        off, srt, pos = oracle.permute(ids, E)
        assert np.array_equal(r.ids.cpu().numpy(), ids)
        assert np.array_equal(r.offsets.cpu().numpy(), off)
        assert np.array_equal(r.sorted_assign.cpu().numpy(), srt)
        assert np.array_equal(r.assign_pos.cpu().numpy(), pos)
        ulps = np.abs(r.w.cpu().numpy().view(np.int32).astype(np.int64) - wt.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1


def test_router_topk_graph_replays():
    """moe_router_topk captured in a HIP graph: every replay (with eager work in between) equals the eager call."""
    for T in (1, 16, 300):
        _announce(f"router_topk graph replays T={T}")
        H, E, k = 2560, 256, 8
        x, w = _router_inputs(T, H, E, 40 + T)
        xd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
        r = dl.Routing.empty(T, E, k)
        logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        dl.router_route(xd, wd, k, out=r, logits=logits)
        torch.cuda.synchronize()
        want = [t.clone() for t in (logits, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos)]
        nb = _lib.moe_route_workspace_bytes(T, E, k)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                _lib.check(_lib.moe_router_topk(xd, wd, T, H, E, k, logits, r.ids, r.w, r.offsets, r.sorted_assign,
                                                r.assign_pos, ws, nb, None))
        torch.cuda.synchronize()
        for rep in range(3):
            for t in (logits, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos):
                t.zero_()
            dl.router_route(xd, wd, k)  # eager work between replays
            g.replay()
            torch.cuda.synchronize()
            got = (logits, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos)
            for a_, b_ in zip(got, want):
                assert torch.equal(a_, b_), (T, rep)


def test_router_rejects_bad_shapes_and_empty_is_noop():
    x, w = _router_inputs(4, 2560, 16, 3)
    xd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    out = torch.full((4, 16), 7.0, device="cuda")
    assert _lib.moe_router_logits(xd, wd, 4, 2000, 16, out, None) == _lib.MOE_ERR_UNSUPPORTED_SHAPE  # H % 256
    assert _lib.moe_router_logits(xd, wd, 4, 2560, 2000, out, None) == _lib.MOE_ERR_UNSUPPORTED_SHAPE  # E > 1024
    assert _lib.moe_router_logits(xd, wd, -1, 2560, 16, out, None) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert _lib.moe_router_logits(None, wd, 4, 2560, 16, out, None) == _lib.MOE_ERR_INVALID_ARGUMENT
    assert _lib.moe_router_logits(xd, wd, 0, 2560, 16, out, None) == _lib.MOE_OK
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused or empty call wrote its output"


# ---------------------------------------------------------------- forward

def _gpu_forward(L, T=None, slot_map=None, shared=True, y=None, accumulate=False):
    dev = device_layer(L)
    x = device_x(L)
    r = dl.route(device_logits(L), L.k)
    sm = None if slot_map is None else torch.from_numpy(np.ascontiguousarray(slot_map, dtype=np.int32)).cuda()
    out = dl.forward(dev, x, r, y=y, accumulate=accumulate, slot_of_expert=sm, shared=shared)
    torch.cuda.synchronize()
    return out, r


def _oracle_forward(L, tokens=None, slot_map=None, shared=True):
    ids, w = oracle.route(L.logits, L.k)
    sm = L.slot_of_expert if slot_map is None else slot_map
    return oracle.forward(L.H, L.I, L.E, L.k, L.bank, sm, L.shared_slot if shared else -1, L.wg, L.x, ids, w,
                          tokens=tokens)


def test_forward_tiny():
    _announce("forward tiny H=256 I=64 E=8 k=2 T=4")
    L = synth.make_layer("tiny")
    y, _ = _gpu_forward(L)
    rel = assert_close(y.cpu().numpy(), _oracle_forward(L), "tiny")
    print(f"tiny rel L2 {rel:.2e}")


@pytest.mark.parametrize("T", [1, 2, 3, 8, 16])
def test_forward_decode_shapes(T):
    _announce(f"forward decode H=2560 I=640 E=256 k=8 T={T}")
    L = synth.make_layer("decode_bs16", T=T, n_distinct=12, seed=100 + T)
    y, _ = _gpu_forward(L)
    ref = _oracle_forward(L)
    rel = assert_close(y.cpu().numpy(), ref, f"decode T={T}")
    print(f"decode T={T} rel L2 {rel:.2e}")


def test_forward_decode_bs1_config():
    _announce("forward decode_bs1 config (seed 1)")
    L = synth.make_layer("decode_bs1", n_distinct=16)
    y, _ = _gpu_forward(L)
    assert_close(y.cpu().numpy(), _oracle_forward(L), "decode_bs1")


def test_forward_small_shapes_and_ragged():
    """Small and odd sizes: H=128 (one 128-column step, fewer steps than waves), I=32 (one slice), I=96 (a partial
    128-column step of down), E=5/7, T across both paths."""
    for (H, I, E, k, T) in [(128, 32, 5, 2, 3), (128, 32, 5, 2, 17), (384, 96, 7, 3, 40), (384, 96, 7, 3, 11),
                            (256, 64, 8, 8, 16), (384, 320, 256, 8, 16), (128, 640, 64, 8, 16),
                            (384, 640, 256, 8, 16), (128, 640, 256, 8, 16)]:
        # the last four have enough (expert, slice) items for the wave-item decode kernel (32-row items for
        # the first two, 64-row items for the last two), with padded gate_up steps (H/128 = 3 and 1) and
        # padded down record groups (H/64 = 6 and 2)
        _announce(f"forward H={H} I={I} E={E} k={k} T={T}")
        rng = np.random.default_rng(H + I + T)
        bank = synth.make_bank(rng, H, I, E + 1, 9)  # every slot distinct
        L = synth.LayerInputs(H, I, E, k, T, bank, np.arange(E, dtype=np.int32), E,
                              synth.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32) * 0.02),
                              synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)),
                              rng.standard_normal((T, E)).astype(np.float32))
        y, _ = _gpu_forward(L)
        assert_close(y.cpu().numpy(), _oracle_forward(L), f"H={H} I={I} T={T}")


def _route_forward_vs_separate(L, what, slot_map=None, shared=True):
    """moe_nvfp4_route_forward against moe_route_topk + moe_nvfp4_forward on the same inputs: routing outputs bit
    for bit, y bit for bit (the same kernels after the prologue), and y against the oracle."""
    dev = device_layer(L)
    x = device_x(L)
    lg = device_logits(L)
    sm = None if slot_map is None else torch.from_numpy(np.ascontiguousarray(slot_map, dtype=np.int32)).cuda()
    r_sep = dl.route(lg, L.k)
    y_sep = dl.forward(dev, x, r_sep, slot_of_expert=sm, shared=shared)
    y_one, r_one = dl.route_forward(dev, lg, x, slot_of_expert=sm, shared=shared)
    torch.cuda.synchronize()
    for name in ("ids", "w", "offsets", "sorted_assign", "assign_pos"):
        a, b = getattr(r_sep, name).cpu().numpy(), getattr(r_one, name).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{what}: routing output {name} differs"
    assert np.array_equal(y_sep.cpu().numpy().view(np.uint32), y_one.cpu().numpy().view(np.uint32)), what
    assert_close(y_one.cpu().numpy(), _oracle_forward(L, slot_map=slot_map, shared=shared), what)


def test_route_tied_blocks_and_group_shapes():
    """Selection order under structured ties: 64 keys tied at the top spread over every (16-lane row, slot) group,
    65 of them, one key above the tie, k = 16 with E = 256, and E = 16 (fewer logits than lanes), each bit-exact
    against the oracle through the routing launch and through the decode kernel's own routing (one token)."""
    rng = np.random.default_rng(77)
    E = 256
    def grouped(n_tied, above=False):
        lg = (rng.standard_normal(E) * 0.1 - 5.0).astype(np.float32)
        # group (row r, slot i) holds experts 64 i + 16 r + [0, 16); 4 tied keys in each of the 16 groups
        tied = [64 * i + 16 * r + j for i in range(4) for r in range(4) for j in range(4)]
        extra = [64 * i + 16 * r + 4 for i in range(4) for r in range(4)]
        for e in (tied + extra)[:n_tied]:
            lg[e] = 1.0
        if above:
            lg[0] = 1.5  # replaces a tied key: still 64 candidates
        return lg[None, :]
    cases = [(grouped(64), 8, "64 tied candidates"), (grouped(65), 8, "65 candidates (rounds)"),
             (grouped(64, above=True), 8, "one key above 64 tied"),
             (rng.standard_normal((1, E)).astype(np.float32), 16, "k = 16 groups of 16"),
             (rng.standard_normal((1, 16)).astype(np.float32), 8, "E = 16: fewer groups than k")]
    for lg, k, what in cases:
        _check_route(lg, k, what)
        _check_route(np.repeat(lg, 3, axis=0), k, what + " x3 tokens")
    # the decode kernel's own routing (one token, E = 256, k = 8) on the tied cases
    for lg, k, what in cases[:3]:
        _announce(f"route_forward one token: {what}")
        L = _small_layer(rng, 256, 64, E, k, 1, n_distinct=12)
        L.logits = lg
        _route_forward_vs_separate(L, f"route_forward {what}")


@pytest.mark.parametrize("T", [1, 3, 8, 16])
def test_route_forward_decode(T):
    """Routing inside the decode kernels (E <= 256, T <= 8: one wave per token); T = 16 routes in its own launch."""
    _announce(f"route_forward decode T={T}")
    L = synth.make_layer("decode_bs16", T=T, n_distinct=8, seed=300 + T)
    _route_forward_vs_separate(L, f"route_forward T={T}")


def test_route_forward_ties_skips_and_fallbacks():
    rng = np.random.default_rng(9)
    # heavy ties and -0/+0 at decode size, with skipped experts and no shared expert
    L = synth.make_layer("decode_bs16", T=5, n_distinct=6, seed=9)
    L.logits = rng.integers(0, 3, L.logits.shape).astype(np.float32)
    L.logits[:, 5] = -0.0
    L.logits[:, 6] = 0.0
    ids, w = oracle.route(L.logits, L.k)
    sm = L.slot_of_expert.copy()
    sm[np.unique(ids)[::3]] = -1
    _announce("route_forward ties, skipped experts, no shared expert")
    _route_forward_vs_separate(L, "route_forward ties", slot_map=sm, shared=False)
    lg = device_logits(L)
    _, r = dl.route_forward(device_layer(L), lg, device_x(L))
    torch.cuda.synchronize()
    off, srt, pos = oracle.permute(ids, L.E)
    assert np.array_equal(r.ids.cpu().numpy(), ids) and np.array_equal(r.offsets.cpu().numpy(), off)
    assert np.array_equal(r.sorted_assign.cpu().numpy(), srt) and np.array_equal(r.assign_pos.cpu().numpy(), pos)
    # the separate-routing fallbacks: prefill size, and more experts than the kernels route themselves
    _announce("route_forward prefill T=40 (separate routing launch)")
    _route_forward_vs_separate(synth.make_layer("prefill_2048", T=40, n_distinct=6), "route_forward T=40")
    _announce("route_forward E=300 decode (separate routing launch)")
    H, I, E, k, T = 256, 64, 300, 4, 3
    bank = synth.make_bank(rng, H, I, E + 1, 5)
    L2 = synth.LayerInputs(H, I, E, k, T, bank, np.arange(E, dtype=np.int32), E,
                           synth.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32) * 0.02),
                           synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)),
                           rng.standard_normal((T, E)).astype(np.float32))
    _route_forward_vs_separate(L2, "route_forward E=300")


def _small_layer(rng, H, I, E, k, T, n_distinct=9):
    bank = synth.make_bank(rng, H, I, E + 1, n_distinct)  # every slot distinct
    return synth.LayerInputs(H, I, E, k, T, bank, np.arange(E, dtype=np.int32), E,
                             synth.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32) * 0.02),
                             synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)),
                             rng.standard_normal((T, E)).astype(np.float32))


def test_route_forward_bad_layer_enqueues_nothing():
    """A layer argument the forward refuses is caught before the routing is enqueued (nothing written)."""
    for name, T in [("decode_bs16", 12), ("prefill_2048", 64)]:
        _announce(f"route_forward refusal {name} T={T}")
        L = synth.make_layer(name, T=T, n_distinct=4)
        dev = device_layer(L)
        x, lg = device_x(L), device_logits(L)
        r = dl.Routing.empty(T, L.E, L.k)
        for t in (r.ids, r.offsets, r.sorted_assign, r.assign_pos):
            t.fill_(-7)
        nb = _lib.moe_nvfp4_route_forward_workspace_bytes(T, L.H, L.I, L.E, L.k)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        y = torch.full((T, L.H), 3.0, dtype=torch.float32, device="cuda")
        st = dev.struct()
        st.slot_bytes = st.slot_bytes + 256  # does not match H and I
        rc = _lib.moe_nvfp4_route_forward(st, lg, x, T, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, y, 0,
                                          ws, nb, None)
        torch.cuda.synchronize()
        assert rc == _lib.MOE_ERR_INVALID_ARGUMENT
        for t in (r.ids, r.offsets, r.sorted_assign, r.assign_pos):
            assert bool((t == -7).all()), "routing was enqueued before the refusal"
        assert bool((y == 3.0).all())


def test_forward_limits():
    """The decode path at its limits: 1024 experts with top-64 (T*k = 1024 assignments, the most it takes; 64-row
    items), one token with top-64, and the smallest prefill batch (T = 17)."""
    rng = np.random.default_rng(17)
    for (H, I, E, k, T) in [(256, 64, 1024, 64, 16), (256, 64, 1024, 64, 1), (256, 64, 64, 8, 17)]:
        _announce(f"forward limits H={H} I={I} E={E} k={k} T={T}")
        L = _small_layer(rng, H, I, E, k, T)
        y, _ = _gpu_forward(L)
        assert_close(y.cpu().numpy(), _oracle_forward(L), f"limits E={E} k={k} T={T}")
        _route_forward_vs_separate(L, f"route_forward limits E={E} k={k} T={T}")


def test_one_token_calls_sharing_a_workspace():
    """One token, up to 16 output rows in the combine: calls that share one workspace (route_forward and forward
    alternating, accumulate on and off, with and without the shared expert) match the oracle each time; the
    workspace starts as garbage, since no region of it has to start at any value."""
    rng = np.random.default_rng(41)
    for (H, I, E, k) in [(256, 64, 8, 2), (512, 96, 16, 15), (2560, 640, 256, 8)]:
        _announce(f"one-token calls sharing a workspace H={H} I={I} E={E} k={k}")
        L = _small_layer(rng, H, I, E, k, 1, n_distinct=min(E + 1, 12))
        dev = device_layer(L)
        nb = _lib.moe_nvfp4_route_forward_workspace_bytes(1, H, I, E, k)
        ws = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")
        for it in range(4):
            L.x = synth.f32_to_bf16_bits(rng.standard_normal((1, H)).astype(np.float32))
            L.logits = rng.standard_normal((1, E)).astype(np.float32)
            x, lg = device_x(L), device_logits(L)
            shared = it != 2
            acc = it == 3
            y0 = torch.from_numpy(rng.standard_normal((1, H)).astype(np.float32)).cuda()
            y = y0.clone()
            if it % 2 == 0:
                y, _ = dl.route_forward(dev, lg, x, y=y, accumulate=acc, ws=ws, shared=shared)
            else:
                y = dl.forward(dev, x, dl.route(lg, k), y=y, accumulate=acc, ws=ws, shared=shared)
            torch.cuda.synchronize()
            want = _oracle_forward(L, shared=shared) + (y0.cpu().numpy() if acc else 0.0)
            assert_close(y.cpu().numpy(), want, f"one token H={H} k={k} call {it}")


def test_route_forward_graph_replays():
    """route_forward captured in a HIP graph: every replay (with eager work in between) equals the eager call."""
    for name, T in [("decode_bs1", 1), ("decode_bs16", 16), ("prefill_2048", 96)]:
        _announce(f"route_forward graph replays {name} T={T}")
        L = synth.make_layer(name, T=T, n_distinct=6)
        dev = device_layer(L)
        x, lg = device_x(L), device_logits(L)
        r = dl.Routing.empty(T, L.E, L.k)
        nb = _lib.moe_nvfp4_route_forward_workspace_bytes(T, L.H, L.I, L.E, L.k)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        y = torch.empty((T, L.H), dtype=torch.float32, device="cuda")
        y_eager, _ = dl.route_forward(dev, lg, x, y=y, out=r, ws=ws)
        want = y_eager.clone()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                dl.route_forward(dev, lg, x, y=y, out=r, ws=ws)
        torch.cuda.synchronize()
        for rep in range(3):
            y.zero_()
            dl.route_forward(dev, lg, x, y=torch.empty_like(y), out=dl.Routing.empty(T, L.E, L.k))  # eager work
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().view(np.uint32), want.cpu().numpy().view(np.uint32)), (name, rep)


def test_forward_no_shared_and_skipped_experts():
    _announce("forward without shared expert; slot map with skipped experts")
    L = synth.make_layer("tiny", T=6)
    y, _ = _gpu_forward(L, shared=False)
    assert_close(y.cpu().numpy(), _oracle_forward(L, shared=False), "no shared")
    sm = L.slot_of_expert.copy()
    sm[[1, 4, 6]] = -1
    y2, _ = _gpu_forward(L, slot_map=sm)
    assert_close(y2.cpu().numpy(), _oracle_forward(L, slot_map=sm), "skipped experts")
    # every expert skipped and no shared expert: y = 0, or y unchanged with accumulate
    none = np.full(L.E, -1, dtype=np.int32)
    y3, _ = _gpu_forward(L, slot_map=none, shared=False)
    assert np.all(y3.cpu().numpy() == 0)
    base = torch.full((L.T, L.H), 1.5, dtype=torch.float32, device="cuda")
    y4, _ = _gpu_forward(L, slot_map=none, shared=False, y=base, accumulate=True)
    assert np.all(y4.cpu().numpy() == 1.5)


def test_forward_accumulate_split_equals_whole():
    """Offload pattern: hits-only call, then misses-only call with accumulate, equals the single call."""
    for name, T in [("decode_bs16", 16), ("prefill_2048", 64)]:
        _announce(f"split hits/misses {name} T={T}")
        L = synth.make_layer(name, T=T, n_distinct=8)
        whole, _ = _gpu_forward(L)
        rng = np.random.default_rng(3)
        miss = rng.random(L.E) < 0.4
        hits_map = np.where(miss, -1, L.slot_of_expert).astype(np.int32)
        miss_map = np.where(miss, L.slot_of_expert, -1).astype(np.int32)
        y, _ = _gpu_forward(L, slot_map=hits_map)
        y2, _ = _gpu_forward(L, slot_map=miss_map, shared=False, y=y, accumulate=True)
        w = whole.cpu().numpy()
        assert_close(y2.cpu().numpy(), w, f"split {name}")
        assert_close(y2.cpu().numpy(), _oracle_forward(L), f"split vs oracle {name}")


def test_forward_run_to_run_bitidentical():
    for name, T in [("decode_bs16", 16), ("decode_bs1", 1), ("prefill_2048", 200)]:
        _announce(f"bit-identical reruns {name} T={T}")
        L = synth.make_layer(name, T=T, n_distinct=8)
        dev = device_layer(L)
        x = device_x(L)
        r = dl.route(device_logits(L), L.k)
        ws = dl.workspace(T, dev)
        outs = [dl.forward(dev, x, r, ws=ws).cpu().numpy() for _ in range(3)]
        assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])


# ---------------------------------------------------------------- prefill

def test_forward_prefill_small_vs_oracle():
    _announce("prefill T=300 H=2560 I=640 E=256 k=8, all tokens")
    L = synth.make_layer("prefill_2048", T=300, n_distinct=8)
    y, _ = _gpu_forward(L)
    rel = assert_close(y.cpu().numpy(), _oracle_forward(L), "prefill T=300")
    print(f"prefill T=300 rel L2 {rel:.2e}")


def test_forward_prefill_2048_sampled():
    """The 2048-token config in the launch configuration the benchmark times; 48 sampled tokens vs the oracle."""
    _announce("prefill 2048 sampled tokens")
    L = synth.make_layer("prefill_2048", n_distinct=16)
    y, r = _gpu_forward(L)
    counts = np.diff(r.offsets.cpu().numpy())
    print(f"per-expert counts: min {counts.min()} median {int(np.median(counts))} max {counts.max()}")
    toks = np.random.default_rng(0).choice(L.T, 48, replace=False).astype(np.int32)
    ref = _oracle_forward(L, tokens=toks)
    assert_close(y.cpu().numpy()[toks], ref, "prefill 2048 sampled")


def test_forward_prefill_zero_count_experts():
    _announce("prefill with 16 zero-count experts")
    L = synth.make_layer("prefill_2048", T=160, n_distinct=8)
    L.logits[:, :16] = -1e30
    y, r = _gpu_forward(L)
    assert np.all(np.diff(r.offsets.cpu().numpy())[:16] == 0)
    assert_close(y.cpu().numpy(), _oracle_forward(L), "prefill zero-count")


# ---------------------------------------------------------------- I-slice

@pytest.mark.parametrize("T", [16, 64])
def test_slice_partials_sum_to_full(T):
    """Intermediate-axis slices I_local = 320 run one after the other on one GPU; their sum equals the full-I result."""
    _announce(f"I-slice check T={T}")
    L = synth.make_layer("decode_bs16", T=T, n_distinct=6)
    dev = device_layer(L)
    x = device_x(L)
    r = dl.route(device_logits(L), L.k)
    full = dl.forward(dev, x, r)
    acc = torch.zeros_like(full)
    for rr in range(2):
        sb = dl.slice_bank(dev.bank, L.H, L.I, rr, 2)
        want_bytes = np.stack([oracle.slice_slot(s, L.H, L.I, rr, 2) for s in L.bank])
        assert np.array_equal(sb.cpu().numpy(), want_bytes), "sliced bytes differ from the oracle's slicer"
        part = dl.DeviceLayer(L.H, L.I // 2, L.E, L.k, sb, dev.slot_of_expert, L.shared_slot, dev.wg)
        dl.forward(part, x, r, y=acc, accumulate=rr > 0)
    torch.cuda.synchronize()
    assert_close(acc.cpu().numpy(), full.cpu().numpy(), "slice sum vs full (GPU)")
    assert_close(acc.cpu().numpy(), _oracle_forward(L), "slice sum vs oracle")


# ---------------------------------------------------------------- expert cache

def test_cache_fill_bytes_and_pinned_check():
    _announce("expert_cache_fill")
    H, I = 256, 64
    sb = synth.slot_nbytes(H, I)
    rng = np.random.default_rng(4)
    host = torch.from_numpy(rng.integers(0, 256, (6, sb), dtype=np.uint8)).pin_memory()
    cache = torch.zeros((4, sb), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    done = torch.cuda.Event()
    srcs = [host[i].data_ptr() for i in (5, 0, 3)]
    _lib.check(_lib.expert_cache_fill(cache, sb, 4, [2, 0, 3], srcs, side, done))
    torch.cuda.current_stream().wait_event(done)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    assert np.array_equal(got[2], host[5].numpy()) and np.array_equal(got[0], host[0].numpy())
    assert np.array_equal(got[3], host[3].numpy()) and np.all(got[1] == 0)
    unpinned = np.zeros(sb, dtype=np.uint8)
    rc = _lib.expert_cache_fill(cache, sb, 4, [1], [unpinned.ctypes.data], side, None)
    assert rc == _lib.MOE_ERR_NOT_PINNED
    rc = _lib.expert_cache_fill(cache, sb, 4, [4], srcs[:1], side, None)
    assert rc == _lib.MOE_ERR_INVALID_ARGUMENT


def test_offload_layer_steps_match_resident():
    """A few offloaded layer-steps (cache smaller than the experts, host LRU, fills on a side stream,
    hits then misses) give the resident result; hit/miss counts match the oracle's LRU model."""
    _announce("offload steps vs resident")
    H, I, E, k, T, L_layers, steps, C = 256, 64, 16, 2, 3, 3, 5, 10
    rng = np.random.default_rng(48)
    sb = synth.slot_nbytes(H, I)
    base = np.stack([synth.random_expert_slot(rng, H, I) for _ in range(E + 1)])
    host = torch.empty((L_layers, E, sb), dtype=torch.uint8).pin_memory()
    for l in range(L_layers):
        for e in range(E):
            host[l, e] = torch.from_numpy(base[(e + 5 * l) % E])
    wg = synth.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32) * 0.02)
    cache = torch.zeros((C, sb), dtype=torch.uint8, device="cuda")
    shared = dl.to_device_u8(base[E][None, :])
    mgr = _lib.ExpertCache(L_layers, E, C)
    side = torch.cuda.Stream()
    all_ids = []
    for st in range(steps):
        for l in range(L_layers):
            x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
            logits = rng.standard_normal((T, E)).astype(np.float32)
            r = dl.route(torch.from_numpy(logits).cuda(), k)
            ids = r.ids.cpu().numpy()
            all_ids.append(ids.reshape(-1).copy())
            som, miss_e, miss_s, n_hit = mgr.plan(l, ids.reshape(-1))
            som = np.array(som, dtype=np.int32)
            hits_map = som.copy()
            hits_map[miss_e] = -1
            miss_map = np.full(E, -1, dtype=np.int32)
            miss_map[miss_e] = som[miss_e]
            done = torch.cuda.Event()
            _lib.check(_lib.expert_cache_fill(cache, sb, C, miss_s, [host[l, e].data_ptr() for e in miss_e], side,
                                              done))
            assert done.cuda_event != 0          # the wait below must see a real event
            dev = dl.DeviceLayer(H, I, E, k, cache, torch.from_numpy(som).cuda(), -1, dl.to_device_bf16(wg))
            xd = dl.to_device_bf16(x)
            # hits first (the copies may still be in flight), then wait and add the misses
            sh_layer = dl.DeviceLayer(H, I, E, k, cache, torch.from_numpy(hits_map).cuda(), -1, dev.wg)
            st_h = sh_layer.struct()
            st_h.shared_slot = shared.data_ptr()
            st_h.shared_gate_w = dev.wg.data_ptr()
            y = torch.empty((T, H), dtype=torch.float32, device="cuda")
            ws = dl.workspace(T, dev)
            _lib.check(_lib.moe_nvfp4_forward(st_h, xd, T, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, y,
                                              0, ws, ws.numel()))
            torch.cuda.current_stream().wait_event(done)
            hm = torch.from_numpy(miss_map).cuda()
            dl.forward(dev, xd, r, y=y, accumulate=True, ws=ws, slot_of_expert=hm, shared=False)
            torch.cuda.synchronize()
            # resident reference from the host bank of this layer
            bank = np.concatenate([host[l].numpy(), base[E][None, :]])
            ids_o, w_o = oracle.route(logits, k)
            ref = oracle.forward(H, I, E, k, bank, np.arange(E, dtype=np.int32), E, wg, x, ids_o, w_o)
            assert_close(y.cpu().numpy(), ref, f"offload step {st} layer {l}")
    hits, misses, _, _ = oracle.lru_run(np.array(all_ids, dtype=np.int32).reshape(steps, L_layers, -1), E, C)
    mgr2 = _lib.ExpertCache(L_layers, E, C)
    ids_arr = np.array(all_ids).reshape(steps, L_layers, -1)
    for st in range(steps):
        for l in range(L_layers):
            _, me, _, nh = mgr2.plan(l, ids_arr[st, l])
            assert nh == hits[st, l] and len(me) == misses[st, l]
