"""GPU parity at the full layer shape (H=2560, I=640, 256 experts, top-8) with
every expert slot distinct and the experts stored at random positions of a
larger bank (marker: gpu).

The banks here are laid out so that an indexing mistake cannot hide: every
routed expert and the shared expert hold different weights, the slot map is a
random permutation into a bank with spare slots, and the spare slots hold
random bytes whose scale bytes include the E4M3 NaN code.  Each case runs in
the launch configuration of its batch size (single-item and multi-item fused
kernel, 32- and 64-row wave kernels, the prefill grouped GEMMs) and is
compared with the oracle on every token: ids and permutation bit for bit,
outputs within relative L2 2e-3 and max |err| <= 1e-2 * max |ref|.
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


def _assert_slots_distinct(L: synth.LayerInputs):
    used = [int(s) for s in L.slot_of_expert] + ([L.shared_slot] if L.shared_slot >= 0 else [])
    digests = {hashlib.sha1(L.bank[j].tobytes()).digest() for j in used}
    assert len(digests) == len(used), "two experts share their weights"
    assert L.shared_slot not in set(int(s) for s in L.slot_of_expert)


def _permuted_layer(name: str, T: int, seed: int, spare: int = 40) -> synth.LayerInputs:
    L = synth.permute_slots(synth.make_layer(name, T=T, n_distinct=16, seed=seed), np.random.default_rng(seed + 7),
                            spare=spare)
    _assert_slots_distinct(L)
    assert not np.array_equal(L.slot_of_expert, np.arange(L.E))
    return L


@pytest.fixture(scope="module")
def decode_layer():
    """One permuted, all-distinct bank at the decode shape; tests draw their own tokens and logits."""
    return _permuted_layer("decode_bs16", 16, seed=16)


def _with_tokens(L: synth.LayerInputs, T: int, seed: int, kind: str = "uniform") -> synth.LayerInputs:
    x, lg = synth.fresh_tokens(seed, T, L.H, L.E, kind)
    return synth.LayerInputs(L.H, L.I, L.E, L.k, T, L.bank, L.slot_of_expert, L.shared_slot, L.wg, x, lg)


def _oracle(L: synth.LayerInputs, slot_map=None, shared=True):
    ids, w = oracle.route(L.logits, L.k)
    sm = L.slot_of_expert if slot_map is None else slot_map
    y = oracle.forward(L.H, L.I, L.E, L.k, L.bank, sm, L.shared_slot if shared else -1, L.wg, L.x, ids, w,
                       nthreads=NTHREADS)
    return ids, w, y


def _check_routing(r: dl.Routing, ids, w, E, what):
    off, srt, pos = oracle.permute(ids, E)
    assert np.array_equal(r.ids.cpu().numpy(), ids), what
    assert np.array_equal(r.offsets.cpu().numpy(), off), what
    assert np.array_equal(r.sorted_assign.cpu().numpy(), srt), what
    assert np.array_equal(r.assign_pos.cpu().numpy(), pos), what
    ulps = np.abs(r.w.cpu().numpy().view(np.int32).astype(np.int64) - w.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, what


@pytest.mark.parametrize("T", [1, 3, 8, 16])
def test_decode_full_shape_distinct_permuted(decode_layer, T):
    """T=1: single-item fused kernel; T=3: multi-item fused kernel; T=8: 32-row wave kernel; T=16: 64-row wave
    kernel.  Both the separate routing + forward calls and route_forward (which routes inside the forward's first
    kernel for T <= 8)."""
    L = _with_tokens(decode_layer, T, 1000 + T)
    _announce(f"decode full shape, distinct permuted bank ({L.bank.shape[0]} slots), T={T}")
    ids, w, ref = _oracle(L)
    dev = device_layer(L)
    x, lg = device_x(L), device_logits(L)
    r = dl.route(lg, L.k)
    y = dl.forward(dev, x, r)
    y2, r2 = dl.route_forward(dev, lg, x)
    torch.cuda.synchronize()
    _check_routing(r, ids, w, L.E, f"route T={T}")
    _check_routing(r2, ids, w, L.E, f"route_forward routing T={T}")
    rel = assert_close(y.cpu().numpy(), ref, f"forward T={T}")
    assert_close(y2.cpu().numpy(), ref, f"route_forward T={T}")
    print(f"T={T} rel L2 {rel:.2e}")


@pytest.mark.parametrize("T", [14, 16])
def test_decode_leftover_items_run_together(decode_layer, T):
    """Every token routed to 8 experts of its own: T*8 active experts plus the shared one, 64-row items (10 per
    expert): 1,130 items at T=14, 1,290 at T=16, against one item per SIMD (1,024).  The items past that run
    cooperatively on the four item waves of a workgroup, in one round (T=14) or two (T=16)."""
    L = _with_tokens(decode_layer, T, 2000 + T)
    lg = np.random.default_rng(3000 + T).random((T, L.E), dtype=np.float32)
    for t in range(T):
        lg[t, 8 * t:8 * t + 8] = 2.0 + np.arange(8, dtype=np.float32) * 0.125
    L = synth.LayerInputs(L.H, L.I, L.E, L.k, T, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, lg)
    _announce(f"decode leftover items, T={T}, {T * 8} distinct experts + shared")
    ids, w, ref = _oracle(L)
    assert len(np.unique(ids)) == 8 * T
    dev = device_layer(L)
    x, dlg = device_x(L), device_logits(L)
    r = dl.route(dlg, L.k)
    y = dl.forward(dev, x, r)
    y_again = dl.forward(dev, x, r)
    torch.cuda.synchronize()
    _check_routing(r, ids, w, L.E, f"route T={T}")
    assert torch.equal(y, y_again), "forward not bit-identical between calls"
    rel = assert_close(y.cpu().numpy(), ref, f"forward T={T}")
    print(f"T={T} rel L2 {rel:.2e}")


def test_prefill_2048_all_tokens_distinct_permuted():
    """The 2048-token prefill config (Zipf routing, seed 2048) in the benchmark's launch configuration, every
    token against the oracle, with all 257 experts distinct and stored at random slots."""
    L = _permuted_layer("prefill_2048", 2048, seed=2048)
    _announce(f"prefill 2048 all tokens, distinct permuted bank ({L.bank.shape[0]} slots)")
    dev = device_layer(L)
    r = dl.route(device_logits(L), L.k)
    y = dl.forward(dev, device_x(L), r)
    torch.cuda.synchronize()
    counts = np.diff(r.offsets.cpu().numpy())
    print(f"per-expert counts: min {counts.min()} median {int(np.median(counts))} max {counts.max()}", flush=True)
    ids, w, ref = _oracle(L)
    _check_routing(r, ids, w, L.E, "prefill 2048")
    rel = assert_close(y.cpu().numpy(), ref, "prefill 2048 all tokens")
    print(f"prefill 2048 rel L2 {rel:.2e}")


@pytest.mark.parametrize("T", [4, 40])
def test_out_of_range_slots_are_left_out(decode_layer, T):
    """Slot indices at or past num_slots behave exactly like -1 (the expert is left out) on both paths."""
    L = _with_tokens(decode_layer, T, 2000 + T)
    ids, _ = oracle.route(L.logits, L.k)
    routed = np.unique(ids)
    bad = L.slot_of_expert.copy()
    n = L.bank.shape[0]
    bad[routed[0::3]] = n                 # one past the end
    bad[routed[1::3]] = n + 1000          # far past the end
    bad[routed[2::7]] = -1
    want_map = np.where(bad >= n, -1, bad).astype(np.int32)
    _announce(f"out-of-range slot map T={T} ({int((bad >= n).sum())} experts past the bank)")
    dev = device_layer(L)
    r = dl.route(device_logits(L), L.k)
    y = dl.forward(dev, device_x(L), r, slot_of_expert=torch.from_numpy(bad).cuda())
    y2, _ = dl.route_forward(dev, device_logits(L), device_x(L), slot_of_expert=torch.from_numpy(bad).cuda())
    torch.cuda.synchronize()
    _, _, ref = _oracle(L, slot_map=want_map)
    assert_close(y.cpu().numpy(), ref, f"out-of-range map T={T}")
    assert_close(y2.cpu().numpy(), ref, f"out-of-range map route_forward T={T}")


def _scale_gate_up_globals(L: synth.LayerInputs, row_exp) -> synth.LayerInputs:
    """The same layer with each expert's gate_up row globals multiplied by 2^row_exp[row] (exact)."""
    off, size = synth.slot_regions(L.H, L.I)[2]
    bank = L.bank.copy()
    g = bank[:, off:off + size].view(np.float32).reshape(bank.shape[0], 2 * L.I)
    used = list(L.slot_of_expert) + ([L.shared_slot] if L.shared_slot >= 0 else [])
    g[used] *= np.exp2(np.asarray(row_exp, dtype=np.float64)).astype(np.float32)[None, :]  # spare slots hold noise
    return synth.LayerInputs(L.H, L.I, L.E, L.k, L.T, bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, L.logits)


@pytest.mark.parametrize("T", [16, 17])
@pytest.mark.parametrize("mode", ["large", "small", "mixed"])
def test_hidden_state_beyond_fp16_range(decode_layer, T, mode):
    """Hidden values far outside the fp16 normal range: gate_up globals times 2^9 make |h| reach ~1e6 (above the
    fp16 maximum 65504), times 2^-9 make every |h| fall below 2^-14 (fp16 subnormals); 'mixed' alternates the two
    by 128-row block of I, so one token row holds tiles 2^36 apart.  T=16 runs the decode path, T=17 the prefill
    path; both must match the oracle."""
    I = decode_layer.I
    rows = np.arange(2 * I) % I
    e = {"large": np.full(2 * I, 9), "small": np.full(2 * I, -9),
         "mixed": np.where((rows // 128) % 2 == 0, 9, -9)}[mode]
    L = _scale_gate_up_globals(_with_tokens(decode_layer, T, 3000 + T), e)
    _announce(f"hidden state range {mode} T={T}")
    dev = device_layer(L)
    r = dl.route(device_logits(L), L.k)
    y = dl.forward(dev, device_x(L), r)
    torch.cuda.synchronize()
    _, _, ref = _oracle(L)
    rel = assert_close(y.cpu().numpy(), ref, f"hidden range {mode} T={T}")
    print(f"{mode} T={T} max|y| {np.abs(ref).max():.3e} rel L2 {rel:.2e}")


def test_offload_full_shape_steps_match_oracle():
    """The offload engine at the full shape: 2 layers x 256 experts in pinned host memory (every expert of every
    layer distinct), an HBM cache of 72 slots with the host LRU, bs 8 with Zipf(1.2) routing per layer, 3 steps.
    Each layer-step fills its misses on a side stream while the hits-only forward runs, then the misses-only
    forward accumulates; every layer-step matches the oracle, and the hit/miss counts match its LRU model."""
    H, I, E, k, T, NL, steps, C = 2560, 640, 256, 8, 8, 2, 3, 72
    _announce(f"offload full shape: {NL} layers x {E} experts pinned, cache {C} slots, {steps} steps at bs {T}")
    rng = np.random.default_rng(4848)
    sb = synth.slot_nbytes(H, I)
    base = synth.make_bank(rng, H, I, 16, 16)
    flips = np.random.default_rng(4849)
    host = torch.empty((NL, E, sb), dtype=torch.uint8).pin_memory()
    hv = host.numpy()
    for l in range(NL):
        for e in range(E):
            hv[l, e] = synth.flip_code_signs(base[(e + 5 * l) % 16], H, I, flips)
    shared_np = np.stack([synth.flip_code_signs(base[l], H, I, flips) for l in range(NL)])
    shared = torch.from_numpy(shared_np).cuda()
    wg = synth.f32_to_bf16_bits(rng.standard_normal((NL, H)).astype(np.float32) * np.float32(0.02))
    wgd = [dl.to_device_bf16(wg[l]) for l in range(NL)]
    ranks = [rng.permutation(E) + 1 for _ in range(NL)]
    cache = torch.zeros((C, sb), dtype=torch.uint8, device="cuda")
    mgr = _lib.ExpertCache(NL, E, C)
    side = torch.cuda.Stream()
    all_ids = []
    for st in range(steps):
        for l in range(NL):
            x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
            logits = synth.zipf_gumbel_logits(rng, T, E, 1.2, ranks[l])
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
            xd = dl.to_device_bf16(x)
            hit_layer = dl.DeviceLayer(H, I, E, k, cache, torch.from_numpy(hits_map).cuda(), -1, wgd[l])
            st_h = hit_layer.struct()
            st_h.shared_slot = shared[l].data_ptr()
            st_h.shared_gate_w = wgd[l].data_ptr()
            y = torch.empty((T, H), dtype=torch.float32, device="cuda")
            ws = dl.workspace(T, hit_layer)
            _lib.check(_lib.moe_nvfp4_forward(st_h, xd, T, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, y,
                                              0, ws, ws.numel()))
            torch.cuda.current_stream().wait_event(done)
            dl.forward(hit_layer, xd, r, y=y, accumulate=True, ws=ws,
                       slot_of_expert=torch.from_numpy(miss_map).cuda(), shared=False)
            torch.cuda.synchronize()
            # the oracle on a compact bank of this layer's routed experts and its shared expert
            routed = np.unique(ids)
            bank = np.concatenate([hv[l, routed], shared_np[l][None]])
            sm = np.full(E, -1, dtype=np.int32)
            sm[routed] = np.arange(routed.size, dtype=np.int32)
            ids_o, w_o = oracle.route(logits, k)
            assert np.array_equal(ids_o, ids)
            ref = oracle.forward(H, I, E, k, bank, sm, routed.size, wg[l], x, ids_o, w_o, nthreads=NTHREADS)
            assert_close(y.cpu().numpy(), ref, f"offload step {st} layer {l} ({len(miss_e)} misses, {n_hit} hits)")
    hits, misses, _, _ = oracle.lru_run(np.array(all_ids, dtype=np.int32).reshape(steps, NL, -1), E, C)
    mgr2 = _lib.ExpertCache(NL, E, C)
    ids_arr = np.array(all_ids).reshape(steps, NL, -1)
    for st in range(steps):
        for l in range(NL):
            _, me, _, nh = mgr2.plan(l, ids_arr[st, l])
            assert nh == hits[st, l] and len(me) == misses[st, l]
    assert hits.sum() > 0 and misses[1:].sum() > 0, "the steps should see both hits and evictions"
