"""The offload engine (moe_offload_layer: device-side cache lookup, hits
forward before the host plans, LRU fills on a side stream, misses forward)
against the oracle at the full layer shape (marker: gpu).

Every layer-step's output is compared with the oracle's layer on the same
routing (every token), and the engine's hit and miss counts with the
oracle's LRU model over the same routed ids.  Cache sizes cover heavy
eviction, the residencies the benchmark sweeps (a quarter, a half, all of the
expert-layers), and a 512-token prefill chunk whose cache hits are read in
place from HBM.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from expert_offload_serving_amd import _lib
from expert_offload_serving_amd import layer as dl
from expert_offload_serving_amd import synth
from tests.gpu_common import assert_close, need_gpu

pytestmark = pytest.mark.gpu
NTHREADS = min(16, os.cpu_count() or 1)
H, I, E, K = 2560, 640, 256, 8


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    _lib.lib()


@pytest.fixture(scope="module")
def banks():
    """4 layers x 256 experts in pinned host memory, every (layer, expert) distinct; one shared expert per layer."""
    NL = 4
    rng = np.random.default_rng(4242)
    sb = synth.slot_nbytes(H, I)
    base = synth.make_bank(rng, H, I, 16, 16)
    flips = np.random.default_rng(4243)
    host = torch.empty((NL, E, sb), dtype=torch.uint8, pin_memory=True)
    hv = host.numpy()
    for l in range(NL):
        for e in range(E):
            hv[l, e] = synth.flip_code_signs(base[(e + 3 * l) % 16], H, I, flips)
    shared_np = np.stack([synth.flip_code_signs(base[l], H, I, flips) for l in range(NL)])
    wg = synth.f32_to_bf16_bits(rng.standard_normal((NL, H)).astype(np.float32) * np.float32(0.02))
    ranks = [rng.permutation(E) + 1 for _ in range(NL)]
    return dict(NL=NL, host=host, hv=hv, shared_np=shared_np, wg=wg, ranks=ranks, sb=sb)


def _run(banks, C, T, steps, seed, layers=None):
    NL = banks["NL"] if layers is None else layers
    sb = banks["sb"]
    rng = np.random.default_rng(seed)
    cache = torch.empty((C, sb), dtype=torch.uint8, device="cuda")
    dws = torch.empty(_lib.moe_offload_device_bytes(NL, E, K, T, H, I), dtype=torch.uint8, device="cuda")
    ptrs = [banks["host"][l, e].data_ptr() for l in range(NL) for e in range(E)]
    eng = _lib.OffloadEngine(NL, E, K, H, I, T, cache, ptrs, dws)
    shared = torch.from_numpy(banks["shared_np"][:NL]).cuda()
    wgd = [dl.to_device_bf16(banks["wg"][l]) for l in range(NL)]
    copy = torch.cuda.Stream()
    ids_log, counts = [], []
    for st in range(steps):
        for l in range(NL):
            x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
            logits = synth.zipf_gumbel_logits(rng, T, E, 1.2, banks["ranks"][l])
            y = torch.empty((T, H), dtype=torch.float32, device="cuda")
            nh, nm = eng.layer(l, torch.from_numpy(logits).cuda(), dl.to_device_bf16(x), T, shared[l], wgd[l], y,
                               copy_stream=copy)
            torch.cuda.synchronize()
            ids, w = oracle.route(logits, K)
            ids_log.append(ids.reshape(-1).copy())
            counts.append((nh, nm))
            routed = np.unique(ids)
            bank = np.concatenate([banks["hv"][l, routed], banks["shared_np"][l][None]])
            sm = np.full(E, -1, dtype=np.int32)
            sm[routed] = np.arange(routed.size, dtype=np.int32)
            ref = oracle.forward(H, I, E, K, bank, sm, routed.size, banks["wg"][l], x, ids, w, nthreads=NTHREADS)
            assert_close(y.cpu().numpy(), ref, f"engine C={C} T={T} step {st} layer {l} ({nh} hits, {nm} misses)")
    hits, misses, _, _ = oracle.lru_run(np.array(ids_log, dtype=np.int32).reshape(steps, NL, -1), E, C,
                                        want_maps=False)
    got = np.array(counts).reshape(steps, NL, 2)
    assert np.array_equal(got[..., 0], hits) and np.array_equal(got[..., 1], misses)
    eng.close()
    return got, np.array(ids_log, dtype=np.int32).reshape(steps, NL, -1)


@pytest.mark.parametrize("frac", [0.07, 0.25, 0.5, 1.0])
def test_engine_decode_bs8_residency_sweep(banks, frac):
    """bs 8 decode steps at cache sizes of 7% (heavy eviction), 25%, 50% and 100% of the 4 x 256 expert-layers."""
    C = max(72, int(frac * banks["NL"] * E))
    print(f"[case] offload engine decode bs 8, cache {C} slots ({frac:.0%})", flush=True)
    got, ids = _run(banks, C, 8, 3, seed=int(frac * 1000) + 1)
    if frac == 1.0:  # nothing is ever evicted: a miss is exactly an expert the layer has not routed before
        for l in range(banks["NL"]):
            seen = set()
            for st in range(ids.shape[0]):
                cur = set(ids[st, l].tolist())
                assert got[st, l, 1] == len(cur - seen)
                seen |= cur
    print(f"hits {got[..., 0].sum()} misses {got[..., 1].sum()}")


def test_engine_prefill_chunk_hits_in_place(banks):
    """A 512-token prefill chunk per layer-step (about 230 distinct experts each) through the engine: the hits are
    read where they sit in HBM, only the misses cross PCIe; a cache of 300 slots forces evictions across layers."""
    print("[case] offload engine prefill T=512, cache 300 slots, 2 layers x 2 steps", flush=True)
    got, _ = _run(banks, 300, 512, 2, seed=77, layers=2)
    assert got[..., 0].sum() > 0 and got[..., 1].sum() > 0
