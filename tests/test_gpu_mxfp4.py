"""GPU parity of the MXFP4 bank format against the oracle (marker: gpu).

The decode of MXFP4 weights (E2M1 with E8M0 scales per 32) must be bit-exact
in fp32 through both of the forward's decode routes (the scaled matrix cores
for gate_up, the fp4 -> bf16 converter for down); the slicer byte-exact;
layer outputs within relative L2 2e-3 and max |err| <= 1e-2 * max |ref| at
every decode batch size's launch configuration, with every slot distinct and
the experts at random positions of a larger bank.
"""
import hashlib
import os

import numpy as np
import pytest
import torch

import oracle
from expert_offload_serving_amd import _lib
from expert_offload_serving_amd import layer as dl
from expert_offload_serving_amd import synth
from tests.gpu_common import assert_close, device_layer, device_logits, device_x, need_gpu

pytestmark = pytest.mark.gpu
NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    _lib.lib()


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _bits_equal(got, want, what):
    nan_w, nan_g = np.isnan(want), np.isnan(got)
    assert np.array_equal(nan_w, nan_g), f"{what}: NaN positions differ ({nan_w.sum()} vs {nan_g.sum()})"
    bad = want[~nan_w].view(np.uint32) != got[~nan_g].view(np.uint32)
    assert not bad.any(), f"{what}: {bad.sum()} values differ, e.g. want {want[~nan_w][bad][:4]} got {got[~nan_g][bad][:4]}"


def test_mx_dequant_transposed_every_code_and_scale_byte():
    """moe_mxfp4_dequant on the checkpoints' transposed layout: every (code, E8M0 byte) pair, bit for bit."""
    N, K = 256, 512
    _announce(f"mxfp4 dequant transposed N={N} K={K}, all codes x all scale bytes")
    codes_row = np.array([(2 * j % 16) | (((2 * j + 1) % 16) << 4) for j in range(K // 2)], dtype=np.uint8)
    blocks_t = np.ascontiguousarray(np.tile(codes_row[:, None], (1, N)))
    scales_t = np.tile(np.arange(N, dtype=np.uint8)[None, :], (K // 32, 1))
    scales_t[1::2] = ((scales_t[1::2].astype(np.int64) + 101) % 256).astype(np.uint8)
    want = oracle.mx_dequant_t(blocks_t, scales_t)
    got = dl.mx_dequant(torch.from_numpy(blocks_t).cuda(), torch.from_numpy(np.ascontiguousarray(scales_t)).cuda())
    _bits_equal(got.cpu().numpy(), want, "mx dequant transposed")


@pytest.mark.parametrize("scales", ["realistic", "every_byte"])
def test_mx_dequant_slot_through_forward_decode(scales):
    """One MXFP4 slot's gate_up through the scaled matrix cores (one-hot activations) and its down through the
    bf16 converter: bit for bit against the oracle's slot dequant."""
    H, I = 2560, 640
    rng = np.random.default_rng(5)
    slot = synth.random_expert_slot(rng, H, I, fmt="mxfp4")
    if scales == "every_byte":  # every E8M0 byte except NaN, in both matrices
        regs = synth.mx_slot_regions(H, I)
        for r_ in (1, 3):
            off, size = regs[r_]
            slot[off:off + size] = (np.arange(size) % 255).astype(np.uint8)
    _announce(f"mxfp4 dequant slot H={H} I={I} ({scales} scales)")
    dslot = torch.from_numpy(slot).cuda()
    for m in (0, 1):
        got, want = dl.mx_dequant_slot(dslot, H, I, m).cpu().numpy(), oracle.mx_dequant_slot(slot, H, I, m)
        if m == 0:
            # through the matrix cores a -0 weight plus the one-hot's zero products sums to +0 (IEEE -0 + +0);
            # the sign of zero is the only thing that route does not carry, every other bit must match
            assert np.all(got[want == 0] == 0)
            want = np.where(want == 0, np.float32(0.0), want)
        _bits_equal(got, want, f"mx slot matrix {m}")


def test_mx_slice_bank_bytes_and_sum():
    """The slicer against the oracle's byte for byte; the two I/2 slices' layer outputs add up to the full one."""
    T = 16
    L = synth.make_layer("decode_bs16", T=T, n_distinct=6, seed=55, fmt="mxfp4")
    _announce(f"mxfp4 slice I=640 -> 2 x 320, T={T}")
    dev = device_layer(L, "mxfp4")
    x = device_x(L)
    r = dl.route(device_logits(L), L.k)
    full = dl.forward(dev, x, r)
    acc = torch.zeros_like(full)
    for rr in range(2):
        sb = dl.mx_slice_bank(dev.bank, L.H, L.I, rr, 2)
        want = np.stack([oracle.mx_slice_slot(s, L.H, L.I, rr, 2) for s in L.bank[:L.E + 1]])
        assert np.array_equal(sb.cpu().numpy()[:L.E + 1], want), "sliced bytes differ from the oracle's slicer"
        part = dl.DeviceLayer(L.H, L.I // 2, L.E, L.k, sb, dev.slot_of_expert, L.shared_slot, dev.wg, "mxfp4")
        dl.forward(part, x, r, y=acc, accumulate=rr > 0)
    torch.cuda.synchronize()
    ids, w = oracle.route(L.logits, L.k)
    ref = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, ids, w,
                         nthreads=NTHREADS, fmt="mxfp4")
    assert_close(acc.cpu().numpy(), full.cpu().numpy(), "mx slice sum vs full")
    assert_close(acc.cpu().numpy(), ref, "mx slice sum vs oracle")


def test_mx_forward_tiny():
    H, I, E, k, T = 256, 64, 8, 2, 4
    rng = np.random.default_rng(0)
    bank = synth.make_bank(rng, H, I, E + 1, None, fmt="mxfp4")
    L = synth.LayerInputs(H, I, E, k, T, bank, np.arange(E, dtype=np.int32), E,
                          synth.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32) * 0.02),
                          synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)),
                          rng.standard_normal((T, E)).astype(np.float32))
    _announce("mxfp4 forward tiny H=256 I=64 E=8 k=2 T=4")
    y = dl.forward(device_layer(L, "mxfp4"), device_x(L), dl.route(device_logits(L), k))
    torch.cuda.synchronize()
    ids, w = oracle.route(L.logits, k)
    ref = oracle.forward(H, I, E, k, bank, L.slot_of_expert, E, L.wg, L.x, ids, w, fmt="mxfp4")
    rel = assert_close(y.cpu().numpy(), ref, "mx tiny")
    print(f"mx tiny rel L2 {rel:.2e}")


@pytest.fixture(scope="module")
def mx_layer():
    L = synth.permute_slots(synth.make_layer("decode_bs16", T=16, n_distinct=16, seed=116, fmt="mxfp4"),
                            np.random.default_rng(117), spare=40)
    used = [int(s) for s in L.slot_of_expert] + [L.shared_slot]
    assert len({hashlib.sha1(L.bank[j].tobytes()).digest() for j in used}) == len(used)
    return L


@pytest.mark.parametrize("T", [1, 3, 8, 16])
def test_mx_forward_full_shape_distinct_permuted(mx_layer, T):
    """MXFP4 layer at H=2560, I=640, 256 experts top-8, every slot distinct, experts at random slots."""
    xb, lg = synth.fresh_tokens(1200 + T, T, mx_layer.H, mx_layer.E, "uniform")
    L = synth.LayerInputs(mx_layer.H, mx_layer.I, mx_layer.E, mx_layer.k, T, mx_layer.bank, mx_layer.slot_of_expert,
                          mx_layer.shared_slot, mx_layer.wg, xb, lg)
    _announce(f"mxfp4 forward full shape T={T}")
    dev = device_layer(L, "mxfp4")
    r = dl.route(device_logits(L), L.k)
    y = dl.forward(dev, device_x(L), r)
    y2 = dl.forward(dev, device_x(L), r)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32)), "not bit-reproducible"
    ids, w = oracle.route(L.logits, L.k)
    ref = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, ids, w,
                         nthreads=NTHREADS, fmt="mxfp4")
    rel = assert_close(y.cpu().numpy(), ref, f"mx forward T={T}")
    print(f"mx T={T} rel L2 {rel:.2e}")


@pytest.mark.parametrize("T", [1, 3, 8, 12])
def test_mx_route_forward_matches_route_then_forward(mx_layer, T):
    """moe_mxfp4_route_forward against moe_route_topk + moe_mxfp4_forward on the same inputs: routing outputs bit
    for bit and y bit for bit (T <= 8 routes inside the forward's kernel, T = 12 in its own launch), y against the
    oracle; then run again with the shared expert left out and accumulating into y."""
    xb, lg = synth.fresh_tokens(1500 + T, T, mx_layer.H, mx_layer.E, "uniform")
    L = synth.LayerInputs(mx_layer.H, mx_layer.I, mx_layer.E, mx_layer.k, T, mx_layer.bank, mx_layer.slot_of_expert,
                          mx_layer.shared_slot, mx_layer.wg, xb, lg)
    _announce(f"mxfp4 route_forward T={T}")
    dev = device_layer(L, "mxfp4")
    x, lgd = device_x(L), device_logits(L)
    r_sep = dl.route(lgd, L.k)
    y_sep = dl.forward(dev, x, r_sep)
    y_one, r_one = dl.route_forward(dev, lgd, x)
    torch.cuda.synchronize()
    for name in ("ids", "w", "offsets", "sorted_assign", "assign_pos"):
        a, b = getattr(r_sep, name).cpu().numpy(), getattr(r_one, name).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"T={T}: routing output {name} differs"
    assert np.array_equal(y_sep.cpu().numpy().view(np.uint32), y_one.cpu().numpy().view(np.uint32)), f"T={T}"
    ids, w = oracle.route(L.logits, L.k)
    ref = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, ids, w,
                         nthreads=NTHREADS, fmt="mxfp4")
    assert_close(y_one.cpu().numpy(), ref, f"mx route_forward T={T}")
    y0 = torch.from_numpy(np.random.default_rng(T).standard_normal((T, L.H)).astype(np.float32)).cuda()
    y_acc, _ = dl.route_forward(dev, lgd, x, y=y0.clone(), accumulate=True, shared=False)
    torch.cuda.synchronize()
    ref_ns = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, -1, L.wg, L.x, ids, w,
                            nthreads=NTHREADS, fmt="mxfp4")
    assert_close(y_acc.cpu().numpy(), ref_ns + y0.cpu().numpy(), f"mx route_forward accumulate T={T}")


@pytest.mark.parametrize("T", [14, 16])
def test_mx_decode_distinct_experts_per_token(mx_layer, T):
    """Every token routed to 8 experts of its own: 8T active experts plus the shared one.  As 32-row items (20 per
    expert) they would be 2,260 at T=14 and 2,580 at T=16, more than one per wave (2,048), so the kernel runs
    64-row items: 1,130 and 1,290, one per wave."""
    xb, lg = synth.fresh_tokens(1700 + T, T, mx_layer.H, mx_layer.E, "uniform")
    lg = lg.copy()
    for t in range(T):
        lg[t, 8 * t:8 * t + 8] = 2.0 + np.arange(8, dtype=np.float32) * 0.125
    L = synth.LayerInputs(mx_layer.H, mx_layer.I, mx_layer.E, mx_layer.k, T, mx_layer.bank, mx_layer.slot_of_expert,
                          mx_layer.shared_slot, mx_layer.wg, xb, lg)
    _announce(f"mxfp4 decode, T={T}, {8 * T} distinct experts + shared")
    ids, w = oracle.route(L.logits, L.k)
    assert len(np.unique(ids)) == 8 * T
    dev = device_layer(L, "mxfp4")
    r = dl.route(device_logits(L), L.k)
    y = dl.forward(dev, device_x(L), r)
    y2 = dl.forward(dev, device_x(L), r)
    torch.cuda.synchronize()
    assert np.array_equal(r.ids.cpu().numpy(), ids)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32)), "not bit-reproducible"
    ref = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, ids, w,
                         nthreads=NTHREADS, fmt="mxfp4")
    rel = assert_close(y.cpu().numpy(), ref, f"mx distinct experts T={T}")
    print(f"mx distinct experts T={T} rel L2 {rel:.2e}")


@pytest.mark.parametrize("I", [1280, 672])
def test_mx_decode_second_items_per_wave(I):
    """16 tokens on 8 experts each of their own (128 + the shared expert) at H=1024: I=1280 gives 2,580 items of 64
    rows and I=672 (not a multiple of 64) 2,709 items of 32 rows, both more than the 2,048 waves, so waves run a
    second item after their first (the persistent wave kernel's multi-item path, for both item heights)."""
    H, E, k, T = 1024, 128, 8, 16
    r_w, r_x, r_l, r_g = np.random.default_rng(4000 + I).spawn(4)
    bank = synth.make_bank(r_w, H, I, E + 1, n_distinct=8, fmt="mxfp4")
    x = synth.f32_to_bf16_bits(r_x.standard_normal((T, H), dtype=np.float32))
    lg = r_l.random((T, E), dtype=np.float32)
    for t in range(T):
        lg[t, 8 * t:8 * t + 8] = 2.0 + np.arange(8, dtype=np.float32) * 0.125
    wg = synth.f32_to_bf16_bits(r_g.standard_normal(H, dtype=np.float32) * np.float32(0.02))
    L = synth.LayerInputs(H, I, E, k, T, bank, np.arange(E, dtype=np.int32), E, wg, x, lg)
    _announce(f"mxfp4 decode second items, H={H} I={I} T={T}")
    ids, w = oracle.route(L.logits, L.k)
    assert len(np.unique(ids)) == 8 * T
    dev = device_layer(L, "mxfp4")
    r = dl.route(device_logits(L), L.k)
    y = dl.forward(dev, device_x(L), r)
    y2 = dl.forward(dev, device_x(L), r)
    torch.cuda.synchronize()
    assert np.array_equal(r.ids.cpu().numpy(), ids)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32)), "not bit-reproducible"
    ref = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, ids, w,
                         nthreads=NTHREADS, fmt="mxfp4")
    rel = assert_close(y.cpu().numpy(), ref, f"mx second items I={I}")
    print(f"mx second items I={I} rel L2 {rel:.2e}")


def test_mx_forward_refuses_wrong_slot_size_and_small_workspace(mx_layer):
    L = mx_layer
    dev = device_layer(L, "mxfp4")
    x = torch.zeros((17, L.H), dtype=torch.bfloat16, device="cuda")
    r = dl.Routing.empty(17, L.E, L.k)
    y = torch.full((17, L.H), 3.0, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    st = dev.struct()
    need = _lib.moe_mxfp4_forward_workspace_bytes(17, L.H, L.I, L.E, L.k)
    assert need > ws.numel()
    rc = _lib.moe_mxfp4_forward(st, x, 17, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, y, 0, ws, ws.numel())
    assert rc == _lib.MOE_ERR_WORKSPACE_TOO_SMALL
    st.slot_bytes = _lib.moe_nvfp4_slot_bytes(L.H, L.I)  # an NVFP4 slot size
    rc = _lib.moe_mxfp4_forward(st, x, 4, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, y, 0, ws, ws.numel())
    assert rc == _lib.MOE_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())


# ---------------------------------------------------------------- prefill (T > 16): the grouped GEMMs over MXFP4

def _mx_with_tokens(base, T, seed, kind="uniform"):
    xb, lg = synth.fresh_tokens(seed, T, base.H, base.E, kind)
    return synth.LayerInputs(base.H, base.I, base.E, base.k, T, base.bank, base.slot_of_expert, base.shared_slot,
                             base.wg, xb, lg)


@pytest.mark.parametrize("T", [17, 40, 300])
def test_mx_prefill_vs_oracle(mx_layer, T):
    """MXFP4 prefill (128/64/32-row tiles of the grouped GEMMs) at H=2560, I=640, 256 experts top-8, every slot
    distinct, experts at random slots; every token against the oracle; bit-reproducible."""
    L = _mx_with_tokens(mx_layer, T, 1700 + T)
    _announce(f"mxfp4 prefill T={T}")
    dev = device_layer(L, "mxfp4")
    x = device_x(L)
    r = dl.route(device_logits(L), L.k)
    y = dl.forward(dev, x, r)
    y2 = dl.forward(dev, x, r)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "not bit-reproducible"
    ids, w = oracle.route(L.logits, L.k)
    ref = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, ids, w,
                         nthreads=NTHREADS, fmt="mxfp4")
    rel = assert_close(y.cpu().numpy(), ref, f"mx prefill T={T}")
    print(f"mx prefill T={T} rel L2 {rel:.2e}")


def test_mx_prefill_2048_all_tokens_distinct_permuted():
    """The 2048-token prefill (Zipf routing) over an MXFP4 bank in the benchmark's launch configuration, every
    token against the oracle, with all 257 experts distinct and stored at random slots of a larger bank."""
    L = synth.permute_slots(synth.make_layer("prefill_2048", n_distinct=16, fmt="mxfp4"), np.random.default_rng(2049),
                            spare=40)
    used = [int(s) for s in L.slot_of_expert] + [L.shared_slot]
    assert len({hashlib.sha1(L.bank[j].tobytes()).digest() for j in used}) == len(used), "two experts share weights"
    assert not np.array_equal(L.slot_of_expert, np.arange(L.E))
    _announce(f"mxfp4 prefill 2048 all tokens, distinct permuted bank ({L.bank.shape[0]} slots)")
    dev = device_layer(L, "mxfp4")
    r = dl.route(device_logits(L), L.k)
    y = dl.forward(dev, device_x(L), r)
    torch.cuda.synchronize()
    counts = np.diff(r.offsets.cpu().numpy())
    print(f"per-expert counts: min {counts.min()} median {int(np.median(counts))} max {counts.max()}", flush=True)
    ids, w = oracle.route(L.logits, L.k)
    assert np.array_equal(r.ids.cpu().numpy(), ids), "top-k ids differ from the oracle"
    ref = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, ids, w,
                         nthreads=NTHREADS, fmt="mxfp4")
    rel = assert_close(y.cpu().numpy(), ref, "mx prefill 2048 all tokens")
    print(f"mx prefill 2048 rel L2 {rel:.2e}")


def test_mx_prefill_odd_shapes():
    """Small and odd sizes on the prefill path: one 128-column step (H=128), one 32-row slice (I=32), a partial
    128-column tile of I (I=96) and a partial 256-column exponent chunk (H=384)."""
    for (H, I, E, k, T) in [(128, 32, 5, 2, 17), (384, 96, 7, 3, 40), (384, 640, 64, 8, 40)]:
        rng = np.random.default_rng(H + I + T)
        bank = synth.make_bank(rng, H, I, E + 1, None, fmt="mxfp4")
        L = synth.LayerInputs(H, I, E, k, T, bank, np.arange(E, dtype=np.int32), E,
                              synth.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32) * 0.02),
                              synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)),
                              rng.standard_normal((T, E)).astype(np.float32))
        _announce(f"mxfp4 prefill H={H} I={I} E={E} k={k} T={T}")
        y = dl.forward(device_layer(L, "mxfp4"), device_x(L), dl.route(device_logits(L), k))
        torch.cuda.synchronize()
        ids, w = oracle.route(L.logits, k)
        ref = oracle.forward(H, I, E, k, bank, L.slot_of_expert, E, L.wg, L.x, ids, w, fmt="mxfp4")
        assert_close(y.cpu().numpy(), ref, f"mx prefill H={H} I={I} T={T}")


def test_mx_prefill_route_forward_and_left_out_slots(mx_layer):
    """route_forward at T=40 (routing launch + prefill) equals route + forward bit for bit; a slot map with experts
    past the bank or -1 leaves them out, with and without the shared expert, accumulating into y."""
    T = 40
    L = _mx_with_tokens(mx_layer, T, 1900)
    _announce("mxfp4 prefill route_forward and left-out slots T=40")
    dev = device_layer(L, "mxfp4")
    x, lgd = device_x(L), device_logits(L)
    r_sep = dl.route(lgd, L.k)
    y_sep = dl.forward(dev, x, r_sep)
    y_one, r_one = dl.route_forward(dev, lgd, x)
    ids, w = oracle.route(L.logits, L.k)
    routed = np.unique(ids)
    bad = L.slot_of_expert.copy()
    n = L.bank.shape[0]
    bad[routed[0::3]] = n
    bad[routed[1::5]] = -1
    want_map = np.where(bad >= n, -1, bad).astype(np.int32)
    y0 = torch.from_numpy(np.random.default_rng(5).standard_normal((T, L.H)).astype(np.float32)).cuda()
    y_acc = dl.forward(dev, x, r_sep, y=y0.clone(), accumulate=True, shared=False,
                       slot_of_expert=torch.from_numpy(bad).cuda())
    torch.cuda.synchronize()
    for name in ("ids", "w", "offsets", "sorted_assign", "assign_pos"):
        a, b = getattr(r_sep, name).cpu().numpy(), getattr(r_one, name).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"routing output {name} differs"
    assert torch.equal(y_sep, y_one)
    ref = oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, ids, w,
                         nthreads=NTHREADS, fmt="mxfp4")
    assert_close(y_one.cpu().numpy(), ref, "mx prefill route_forward")
    ref_left = oracle.forward(L.H, L.I, L.E, L.k, L.bank, want_map, -1, L.wg, L.x, ids, w, nthreads=NTHREADS,
                              fmt="mxfp4")
    assert_close(y_acc.cpu().numpy(), ref_left + y0.cpu().numpy(), "mx prefill left-out slots, accumulate")
