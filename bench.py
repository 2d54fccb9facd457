#!/usr/bin/env python3
"""Benchmark of the NVFP4 routed-MoE layer (route + forward) on one MI355X.

A step is one pass of the layer over one batch of synthetic tokens: top-k
routing and permutation, then the NVFP4 expert forward with the shared
expert and the combine.  Inputs (activations, logits, weights) are resident
in HBM before timing; every step uses fresh routing and, to keep the 256 MB
Infinity Cache from serving repeated experts, one of several copies of the
expert bank in turn.  The steps are captured in a HIP graph and replayed.

Default run: every workload, printed as ONE JSON line whose top level is the
decode shape the metric is quoted on (H=2560, I=640, 256 experts top-8 with
uniform-random logits, one shared expert, batch 1) and whose "configs" entry
holds the full result of decode batch 16, the 2048-token prefill chunk, the
offloaded 48-layer run and the MXFP4 bank format at decode batch 1 and 16 and
the 2048-token prefill, each with its own roofline and CPU baseline.
`--config NAME` prints that workload's line alone.

The arithmetic (dtype field): NVFP4 weights decoded exactly to fp16, bf16
activations entered as fp16 times a per-token power of two, fp16 matrix-core
products accumulated in fp32.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME|all]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

import numpy as np

METRIC = "MoE-layer tokens/s + expert-weight HBM GB/s (% peak), H2560 I640 NVFP4"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PCIE_PEAK_GBS = 64.0      # PCIe Gen5 x16, one direction
DTYPE = "nvfp4w-fp16mfma-fp32acc"
METRIC_MX = "MoE-layer tokens/s + expert-weight HBM GB/s (% peak), H2560 I640 MXFP4"
DTYPE_MX = "mxfp4w-fp8x2scaledmfma-bf16x2mfma-fp32acc"
DTYPE_MX_PREFILL = "mxfp4w-bf16mfma-bf16x2h-fp32acc"  # MXFP4 prefill: weights decoded exactly to bf16


# HBM bytes per call of the roofline unit from two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE, summed over the call's
# kernels and scaled by what the same counters read for a plain copy of known size), with a digest of the kernel
# sources they were taken on.  Reported as roofline.traffic only while those sources are unchanged.
COUNTED_TRAFFIC = {
    "decode_bs1": (29_530_115, "a4931601b49db091"),
    "decode_bs16": (319_185_524, "a4931601b49db091"),
    "prefill_2048": (1_180_886_918, "6284de10fb5c8ffc"),
    "mxfp4_decode_bs1": (27_784_280, "ba5cf7dc0aa7c44f"),
    "mxfp4_decode_bs16": (301_502_598, "ba5cf7dc0aa7c44f"),
    "mxfp4_prefill_2048": (1_177_178_029, "6284de10fb5c8ffc"),
}
KERNEL_SOURCES = {"decode": ["decode.hip", "decode_common.hpp", "route_device.hpp", "nvfp4_device.hpp"],
                  "mxfp4": ["mxfp4.hip", "decode_common.hpp", "route_device.hpp", "nvfp4_device.hpp"],
                  "prefill": ["prefill.hip", "nvfp4_device.hpp"]}


def kernel_digest(kind: str) -> str:
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "expert_offload_serving_amd", "csrc")
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(base, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counted_traffic(name: str, kind: str):
    ent = COUNTED_TRAFFIC.get(name)
    if ent is None or kernel_digest(kind) != ent[1]:
        return None
    return ent[0]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- inputs

def split_name(name: str):
    """Workload name -> (base config, slot format): "mxfp4_decode_bs1" is decode_bs1 over MXFP4 slots."""
    return (name[len("mxfp4_"):], "mxfp4") if name.startswith("mxfp4_") else (name, "nvfp4")


def build_inputs(name: str, steps: int, replicas: int, distinct: int):
    """Host inputs: the expert bank (E routed + 1 shared slot), per-step activations and logits."""
    from expert_offload_serving_amd import synth
    base, fmt = split_name(name)
    H, I, E, k, T, seed, kind = synth.CONFIGS[base]
    r_w, r_x, r_l, r_g = np.random.default_rng(seed).spawn(4)
    t0 = time.time()
    bank = synth.make_bank(r_w, H, I, E + 1, distinct, fmt)
    log(f"{name}: quantized {min(distinct, E + 1)} distinct experts into {E + 1} slots in {time.time() - t0:.1f}s")
    wg = synth.f32_to_bf16_bits(r_g.standard_normal(H, dtype=np.float32) * np.float32(0.02))
    xs = synth.f32_to_bf16_bits(r_x.standard_normal((steps, T, H), dtype=np.float32))
    logits = np.stack([synth.make_logits(r_l, T, E, kind) for _ in range(steps)])
    return dict(H=H, I=I, E=E, k=k, T=T, bank=bank, wg=wg, xs=xs, logits=logits, replicas=replicas, fmt=fmt)


# ---------------------------------------------------------------- GPU run

def run_gpu(inp, steps: int, warmup: int, slice_check: bool = True):
    import torch
    from expert_offload_serving_amd import _lib
    from expert_offload_serving_amd import layer as dl

    H, I, E, k, T, R = inp["H"], inp["I"], inp["E"], inp["k"], inp["T"], inp["replicas"]
    dev = torch.device("cuda:0")
    nslot = E + 1
    base = dl.to_device_u8(inp["bank"], dev)
    bank = torch.empty((R * nslot, base.shape[1]), dtype=torch.uint8, device=dev)
    for r in range(R):
        bank[r * nslot:(r + 1) * nslot].copy_(base)
    del base
    wg = dl.to_device_bf16(inp["wg"], dev)
    maps = torch.arange(E, dtype=torch.int32, device=dev)[None, :] + nslot * torch.arange(
        R, dtype=torch.int32, device=dev)[:, None]
    fmt = inp["fmt"]
    layers = [dl.DeviceLayer(H, I, E, k, bank, maps[r].contiguous(), r * nslot + E, wg, fmt) for r in range(R)]
    structs = [l.struct() for l in layers]
    total = steps + warmup
    xs = dl.to_device_bf16(inp["xs"][:total].reshape(total * T, H), dev).view(total, T, H)
    logits = torch.from_numpy(np.ascontiguousarray(inp["logits"][:total])).to(dev)
    routes = [dl.Routing.empty(T, E, k, dev) for _ in range(total)]
    ws = dl.workspace(T, layers[0])
    rf_bytes = (_lib.moe_mxfp4_route_forward_workspace_bytes if fmt == "mxfp4"
                else _lib.moe_nvfp4_route_forward_workspace_bytes)(T, H, I, E, k)
    ws_rf = torch.empty(rf_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty((total, T, H), dtype=torch.float32, device=dev)
    rws = _lib.moe_route_workspace_bytes(T, E, k)
    rws_t = torch.empty(max(1, rws), dtype=torch.uint8, device=dev)

    def step(s: int, do_route: bool = True, do_forward: bool = True):
        """A step is one moe_nvfp4_route_forward call (MXFP4: moe_mxfp4_route_forward); do_route / do_forward
        select the separate calls (moe_route_topk, moe_nvfp4_forward / moe_mxfp4_forward)."""
        r = routes[s]
        mx = fmt == "mxfp4"
        if do_route and do_forward:
            f = _lib.moe_mxfp4_route_forward if mx else _lib.moe_nvfp4_route_forward
            _lib.check(f(structs[s % R], logits[s], xs[s], T, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos,
                         y[s], 0, ws_rf, rf_bytes, None))
        elif do_route:
            _lib.check(_lib.moe_route_topk(logits[s], T, E, k, r.ids, r.w, r.offsets, r.sorted_assign,
                                           r.assign_pos, rws_t, rws, None))
        else:
            f = _lib.moe_mxfp4_forward if mx else _lib.moe_nvfp4_forward
            _lib.check(f(structs[s % R], xs[s], T, r.ids, r.w, r.offsets, r.sorted_assign, r.assign_pos, y[s], 0,
                         ws, ws.numel(), None))

    # eager warm-up, then an eager reference of the last timed step
    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    step(total - 1)
    torch.cuda.synchronize()
    y_eager = y[total - 1].clone()

    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    g_step, g_fwd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g_step, stream=s):
            for i in range(warmup, total):
                step(i)
        with torch.cuda.graph(g_fwd, stream=s):
            for i in range(warmup, total):
                step(i, do_route=False)
    torch.cuda.synchronize()
    # graphs replayed once untimed (first replay uploads the graph)
    g_step.replay()
    g_fwd.replay()
    torch.cuda.synchronize()

    # timed region: whole steps (route + forward)
    cur = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_step.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    replay_ok = torch.equal(y[total - 1], y_eager)

    # the step's calls, HIP events on the stream they run on
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(cur)
    g_step.replay()
    ev1.record(cur)
    torch.cuda.synchronize()
    call_ms = ev0.elapsed_time(ev1) / steps
    # forward kernels only (routing given), HIP events
    ev0.record(cur)
    g_fwd.replay()
    ev1.record(cur)
    torch.cuda.synchronize()
    fwd_ms = ev0.elapsed_time(ev1) / steps
    # route kernel only
    g_route = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g_route, stream=s):
            for i in range(warmup, total):
                step(i, do_forward=False)
    g_route.replay()
    torch.cuda.synchronize()
    ev0.record(cur)
    g_route.replay()
    ev1.record(cur)
    torch.cuda.synchronize()
    route_ms = ev0.elapsed_time(ev1) / steps

    # intermediate-axis slice check (decode): the last step's routing through the two I/2 slices of the bank,
    # run one after the other on this GPU, the second accumulating into the first; the sum against the full-I
    # output of the same step (bank copy 0 holds the same bytes as every other copy)
    sc_out = None
    if slice_check and T <= 16 and I % 64 == 0:
        slicer = dl.mx_slice_bank if fmt == "mxfp4" else dl.slice_bank
        r_last = routes[total - 1]
        acc = torch.empty((T, H), dtype=torch.float32, device=dev)
        for rr in range(2):
            part = dl.DeviceLayer(H, I // 2, E, k, slicer(bank[:nslot], H, I, rr, 2), maps[0].contiguous(), E, wg, fmt)
            dl.forward(part, xs[total - 1], r_last, y=acc, accumulate=rr > 0)
        torch.cuda.synchronize()
        full = y[total - 1].double()
        diff = acc.double() - full
        sc_out = {"I_local": I // 2, "slices": 2,
                       "rel_l2_vs_full": float(diff.norm() / full.norm()),
                       "max_abs_err_over_max_abs": float(diff.abs().max() / full.abs().max())}

    distinct = []
    for i in range(warmup, total):
        off = routes[i].offsets.cpu().numpy()
        distinct.append(int(np.count_nonzero(np.diff(off))))
    counts = np.diff(routes[total - 1].offsets.cpu().numpy())
    return dict(wall=wall, fwd_ms=fwd_ms, call_ms=call_ms, route_ms=route_ms, distinct=distinct, replay_ok=replay_ok,
                y_last=y[total - 1].cpu().numpy(), ids_last=routes[total - 1].ids.cpu().numpy(),
                counts_max=int(counts.max()), counts_min=int(counts.min()), slice_check=sc_out)


# ---------------------------------------------------------------- CPU baseline (the oracle)

def oracle_threads():
    """Threads for the oracle: the host's physical cores (lscpu), capped by the CPUs this process may run on and
    by its cgroup CPU quota (an oversubscribed OpenMP pool would measure spin-waiting, not the oracle)."""
    phys = None
    try:
        out = subprocess.run(["lscpu", "-p=core,socket"], capture_output=True, text=True, timeout=20).stdout
        phys = len({ln for ln in out.splitlines() if ln and not ln.startswith("#")}) or None
    except (OSError, subprocess.SubprocessError):
        pass
    avail = len(os.sched_getaffinity(0))
    quota = None
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()
        if q != "max":
            quota = max(1, int(int(q) // int(per)))
    except (OSError, ValueError):
        pass
    n = min(v for v in (phys, avail, quota) if v)
    return n, {"lscpu_physical_cores": phys, "affinity_cpus": avail, "cgroup_cpu_quota": quota}


# Per-repetition sample of each workload for the oracle (one oracle call per step, as the GPU runs them).
CPU_SAMPLES = {"decode_bs1": 4, "decode_bs16": 1, "prefill_2048": 128, "offload": 2, "mxfp4_decode_bs1": 4,
               "mxfp4_decode_bs16": 1, "mxfp4_prefill_2048": 128}


def cpu_leg(name: str, reps: int = 5) -> dict:
    """Runs in a child process (OMP_NUM_THREADS / OMP_PROC_BIND set before the OpenMP runtime starts): the oracle
    (routing + the whole layer forward, fp64 accumulation) timed on a sample of the workload, one warm-up then the
    median of `reps` repetitions."""
    import oracle
    from expert_offload_serving_amd import synth
    threads = int(os.environ["OMP_NUM_THREADS"])
    n = CPU_SAMPLES[name]
    fmt = "nvfp4"
    if name == "offload":
        H, I, E, k, T, seed = 2560, 640, 256, 8, 8, 48
        r_w, r_x, r_l, r_g = np.random.default_rng(seed).spawn(4)
        bank = synth.make_bank(r_w, H, I, E + 1, 32)
        ranks = r_l.permutation(E) + 1
        steps = [(synth.f32_to_bf16_bits(r_x.standard_normal((T, H), dtype=np.float32)),
                  synth.zipf_gumbel_logits(r_l, T, E, 1.2, ranks)) for _ in range(n)]
        what = f"{n} layer-steps of bs {T} (Zipf(1.2) routing), one oracle call each"
        per_rep_tokens = n * T
    else:
        base, fmt = split_name(name)
        H, I, E, k, T, seed, kind = synth.CONFIGS[base]
        r_w, r_x, r_l, r_g = np.random.default_rng(seed).spawn(4)
        bank = synth.make_bank(r_w, H, I, E + 1, 32, fmt)
        if T > 16:  # the prefill chunk: its first n tokens, routed and computed as one call
            x = synth.f32_to_bf16_bits(r_x.standard_normal((T, H), dtype=np.float32))
            lg = synth.make_logits(r_l, T, E, kind)
            steps = [(x[:n], lg[:n])]
            what = f"the first {n} tokens of the {T}-token chunk in one oracle call"
            per_rep_tokens = n
        else:
            steps = [(synth.f32_to_bf16_bits(r_x.standard_normal((T, H), dtype=np.float32)),
                      synth.make_logits(r_l, T, E, kind)) for _ in range(n)]
            what = f"{n} step(s) of {T} token(s), one oracle call each"
            per_rep_tokens = n * T
    wg = synth.f32_to_bf16_bits(r_g.standard_normal(H, dtype=np.float32) * np.float32(0.02))
    som = np.arange(E, dtype=np.int32)

    def once():
        t0 = time.perf_counter()
        for x, lg in steps:
            ids, w = oracle.route(lg, k)
            oracle.forward(H, I, E, k, bank, som, E, wg, x, ids, w, nthreads=threads, fmt=fmt)
        return time.perf_counter() - t0

    once()
    times = [once() for _ in range(reps)]
    med = statistics.median(times)
    return {"value": round(per_rep_tokens / med, 3), "seconds_per_rep": [round(t, 3) for t in times],
            "sample": f"{what}: routing and the whole layer forward (all expert FFNs, shared expert, combine) "
                      f"through the oracle, fp64 accumulation; 1 warm-up then the median of {reps} repetitions of "
                      f"{per_rep_tokens} tokens"}


def cpu_baseline(name: str, unit: str) -> dict:
    """The oracle timed on the host's cores in a child process, so that OMP_NUM_THREADS and OMP_PROC_BIND=close
    are in force when its OpenMP runtime starts."""
    threads, how = oracle_threads()
    env = dict(os.environ, OMP_NUM_THREADS=str(threads), OMP_PROC_BIND="close", OMP_PLACES="cores")
    t0 = time.perf_counter()
    res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-leg", name], capture_output=True,
                         text=True, env=env, timeout=900)
    if res.returncode != 0:
        return {"error": res.stderr[-500:], "kind": "oracle"}
    leg = json.loads(res.stdout.strip().splitlines()[-1])
    return {"value": leg["value"], "unit": unit, "cores": threads, "kind": "oracle", "sample": leg["sample"],
            "threads_from": how, "omp": "OMP_PROC_BIND=close OMP_PLACES=cores",
            "seconds_per_rep": leg["seconds_per_rep"], "wall_s": round(time.perf_counter() - t0, 1)}


def parity_sample(inp, res, tokens):
    """Relative L2 error of the last timed step's output against the oracle (a few tokens)."""
    import oracle
    H, I, E, k, T = inp["H"], inp["I"], inp["E"], inp["k"], inp["T"]
    last = res["last_index"]
    x = inp["xs"][last]
    lg = inp["logits"][last]
    ids, w = oracle.route(lg, k)
    if not np.array_equal(ids, res["ids_last"]):
        return {"ids_bitexact": False}
    toks = np.arange(min(tokens, T), dtype=np.int32)
    ref = oracle.forward(H, I, E, k, inp["bank"], np.arange(E, dtype=np.int32), E, inp["wg"], x, ids, w,
                         tokens=toks, fmt=inp["fmt"])
    got = res["y_last"][toks].astype(np.float64)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    return {"ids_bitexact": True, "rel_l2": rel, "tokens_checked": int(toks.size)}


# ---------------------------------------------------------------- offload

def bench_offload(steps: int, warmup: int, distinct: int, want_cpu: bool = True,
                  residency: float = 0.37, distinct_banks: bool = True, T: int = 8):
    """48 MoE layers whose 256 experts live in pinned host memory behind one HBM cache holding `residency`
    (default 37%) of the 12,288 expert-layer slots (global LRU, cold start).  Per layer-step, one
    moe_offload_layer call: route on the GPU, look the routed experts up in the engine's device-side directory,
    start the hits-only forward, plan on the host meanwhile (one wait for the small lookup result), copy the misses
    on two side streams, then the misses-only forward accumulates.  With want_cpu, the CPU leg checks the host LRU and the last layer-step
    against the oracle.  With distinct_banks (the default) every one of the 48 x 256 experts has its own pinned
    host slot (34.16 GB); otherwise the experts alias 256 pinned base slots.  T: tokens per layer-step (8: decode
    at batch 8; 2048: a prefill chunk, whose cache hits are read in place from HBM).  Returns the JSON dict."""
    import torch
    from expert_offload_serving_amd import _lib, synth
    from expert_offload_serving_amd import layer as dl

    H, I, E, k, L = 2560, 640, 256, 8, 48
    seed = 48
    r_w, r_x, r_l, r_g = np.random.default_rng(seed).spawn(4)
    sb = synth.slot_nbytes(H, I)
    n_slots = max(1, min(L * E, int(residency * L * E)))
    t0 = time.time()
    base_np = synth.make_bank(r_w, H, I, E, distinct)          # 256 base experts (distinct of them quantized)
    log(f"offload: quantized {min(distinct, E)} distinct experts into {E} base slots in {time.time() - t0:.1f}s")
    # expert (l, e) is base expert (e + 37 l) mod 256 with its code signs flipped by layer l's own mask, so every
    # (layer, expert) has distinct weights and its own pinned slot
    def base_of(l, e):
        return (e + 37 * l) % E
    banks_note = None
    host = None
    if distinct_banks:
        t0 = time.time()
        try:
            host = torch.empty((L, E, sb), dtype=torch.uint8, pin_memory=True)
        except RuntimeError as err:  # page-locking 34 GB refused: fall back to the aliased banks, and say so
            banks_note = f"distinct pinned banks refused ({err}); aliased base slots used"
            log(f"offload: {banks_note}")
            host = None
        if host is not None:
            base_t = torch.from_numpy(base_np)
            mrng = np.random.default_rng(4800)
            regions = synth.slot_regions(H, I)
            for l in range(L):
                mask = np.zeros(sb, dtype=np.uint8)
                for r_ in (0, 3):  # code regions: sign bits only
                    off, size = regions[r_]
                    mask[off:off + size] = mrng.integers(0, 256, size, dtype=np.uint8) & np.uint8(0x88)
                idx = torch.tensor([base_of(l, e) for e in range(E)])
                torch.bitwise_xor(base_t[idx], torch.from_numpy(mask), out=host[l])
            host_ptr = [[host[l, e].data_ptr() for e in range(E)] for l in range(L)]
            log(f"offload: {L} x {E} distinct expert slots pinned ({L * E * sb / 1e9:.2f} GB) in "
                f"{time.time() - t0:.1f}s")
    if host is None:
        # the 48 x 256 banks alias 256 pinned base slots, each serving 48 (layer, expert) pairs
        host_base = torch.from_numpy(base_np).pin_memory()
        host_ptr = [[host_base[base_of(l, e)].data_ptr() for e in range(E)] for l in range(L)]

    def host_slot_np(l, e):
        return host[l, e].numpy() if host is not None else base_np[base_of(l, e)]
    dev = torch.device("cuda:0")
    cache = torch.empty((n_slots, sb), dtype=torch.uint8, device=dev)
    shared_np = np.stack([base_np[(200 + l) % E] for l in range(L)])
    shared = torch.from_numpy(shared_np).to(dev)
    wg_np = synth.f32_to_bf16_bits(r_g.standard_normal((L, H), dtype=np.float32) * np.float32(0.02))
    wg = dl.to_device_bf16(wg_np, dev).view(L, H)
    total = steps + warmup
    ranks = [r_l.permutation(E) + 1 for _ in range(L)]
    logits_np = np.empty((total, L, T, E), dtype=np.float32)
    for l in range(L):
        for s_ in range(total):
            logits_np[s_, l] = synth.zipf_gumbel_logits(r_l, T, E, 1.2, ranks[l])
    logits = torch.from_numpy(logits_np).to(dev)
    NX = 16
    xs_np = synth.f32_to_bf16_bits(r_x.standard_normal((NX, T, H), dtype=np.float32))
    xs = dl.to_device_bf16(xs_np.reshape(NX * T, H), dev).view(NX, T, H)

    dws = torch.empty(_lib.moe_offload_device_bytes(L, E, k, T, H, I), dtype=torch.uint8, device=dev)
    eng = _lib.OffloadEngine(L, E, k, H, I, T, cache, [host_ptr[l][e_] for l in range(L) for e_ in range(E)], dws)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    copy = torch.cuda.Stream(device=dev)
    stats = {"hits": np.zeros((total, L), np.int64), "misses": np.zeros((total, L), np.int64)}

    def layer_step(s_, l):
        """One moe_offload_layer call: route, device-side lookup, hits forward, host LRU plan overlapping it,
        misses copied on two copy streams, misses forward."""
        stats["hits"][s_, l], stats["misses"][s_, l] = eng.layer(l, logits[s_, l], xs[(s_ * L + l) % NX], T,
                                                                  shared[l], wg[l], y, copy_stream=copy)

    log(f"offload: {L} layers x {E} experts, cache {n_slots} slots ({n_slots * sb / 1e9:.1f} GB), "
        f"{warmup} warm-up + {steps} timed steps at bs {T}")
    t_cold = time.perf_counter()
    for s_ in range(warmup):
        for l in range(L):
            layer_step(s_, l)
    torch.cuda.synchronize()
    t_cold = time.perf_counter() - t_cold
    log(f"offload: warm-up done in {t_cold:.1f}s, hit rate {stats['hits'][:warmup].sum() / max(1, stats['hits'][:warmup].sum() + stats['misses'][:warmup].sum()):.3f}")
    t0 = time.perf_counter()
    for s_ in range(warmup, total):
        for l in range(L):
            layer_step(s_, l)
        if (s_ - warmup) % 16 == 15:
            log(f"offload: step {s_ - warmup + 1}/{steps}")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # a cache that holds every expert-layer never evicts: replaying the last timed steps' routing then hits on
    # every expert, which times the engine's all-hit layer-step (one forward, no copies)
    all_hits = None
    if n_slots >= L * E:
        replay = list(range(max(warmup, total - 8), total))
        saved = {key: v.copy() for key, v in stats.items()}
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for s_ in replay:
            for l in range(L):
                layer_step(s_, l)
        torch.cuda.synchronize()
        ta = time.perf_counter() - ta
        assert stats["misses"][replay].sum() == 0
        all_hits = round(ta * 1e3 / (len(replay) * L), 4)
        stats.update(saved)

    # pinned host -> HBM copy rate alone (64 slots over two copy streams, host clock)
    n_probe = 64
    copies = [copy, torch.cuda.Stream(device=dev)]
    for c_ in range(2):  # a stream's first use sets up its queue: not part of the measurement
        _lib.check(_lib.expert_cache_fill(cache, sb, n_slots, [c_], [host_ptr[0][c_]], copies[c_], None))
    torch.cuda.synchronize()
    tp = time.perf_counter()
    for c_ in range(2):
        part = list(range(c_, n_probe, 2))
        _lib.check(_lib.expert_cache_fill(cache, sb, n_slots, part, [host_ptr[j // E % L][j % E] for j in part],
                                          copies[c_], None))
    torch.cuda.synchronize()
    h2d_gbs = n_probe * sb / (time.perf_counter() - tp) / 1e9

    cpu_checks = None
    if want_cpu:
        # the CPU leg: the host LRU against the oracle's model on the same ids; the last layer-step against the
        # oracle
        import oracle
        ids_log = np.stack([np.stack([oracle.route(logits_np[s_, l], k)[0].reshape(-1) for l in range(L)])
                            for s_ in range(total)])
        h_ref, m_ref, _, _ = oracle.lru_run(ids_log, E, n_slots, want_maps=False)
        lru_ok = bool(np.array_equal(h_ref, stats["hits"]) and np.array_equal(m_ref, stats["misses"]))
        s_last, l_last = total - 1, L - 1
        ids_o, w_o = oracle.route(logits_np[s_last, l_last], k)
        toks = np.arange(2, dtype=np.int32)
        routed = np.unique(ids_o[toks])
        bank_o = np.stack([host_slot_np(l_last, int(e_)) for e_ in routed] + [shared_np[l_last]])
        som_o = np.full(E, -1, dtype=np.int32)
        som_o[routed] = np.arange(routed.size, dtype=np.int32)
        ref = oracle.forward(H, I, E, k, bank_o, som_o, routed.size, wg_np[l_last],
                             xs_np[(s_last * L + l_last) % NX], ids_o, w_o, tokens=toks)
        got = y.cpu().numpy()[toks].astype(np.float64)
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        cpu_checks = {"lru_matches_oracle_model": lru_ok, "rel_l2_last_layer_step": rel,
                      "tokens_checked": int(toks.size)}
        log("offload: timing the oracle (child process)")
        cpu_checks["cpu_baseline"] = cpu_baseline("offload" if T <= 16 else "prefill_2048", "layer-tokens/s")

    hits, misses = stats["hits"][warmup:].sum(), stats["misses"][warmup:].sum()
    miss_bytes = misses * sb
    layer_tok_s = T * steps * L / wall
    pcie = miss_bytes / wall / 1e9
    return {
        "metric": "MoE-layer tokens/s with the expert cache (offload), H2560 I640 NVFP4",
        "value": round(layer_tok_s, 2), "unit": "layer-tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(wall * 1e3 / steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": f"offload{'' if T <= 16 else '_prefill' + str(T)}_48x256_cache"
                               f"{round(100 * n_slots / (L * E))}", "H": H, "I": I, "E": E, "k": k, "T": T, "layers": L,
                   "cache_slots": n_slots, "residency": round(n_slots / (L * E), 4), "routing": "Zipf(1.2) per layer",
                   "host_banks": (f"{L} x {E} distinct pinned expert slots ({L * E * sb / 1e9:.2f} GB)" if host is not None
                                  else f"{E} pinned base slots ({E * sb / 1e9:.2f} GB); expert (l, e) = base "
                                       f"(e + 37 l) mod {E}" + (f" [{banks_note}]" if banks_note else "")),
                   "distinct_quantized_experts": min(distinct, E), "parallelism": "single GPU"},
        "roofline": {"bound": "pcie", "achieved": round(pcie, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(pcie / PCIE_PEAK_GBS, 4), "traffic": None,
                     "kernel": "moe_offload_layer (device-side cache lookup, hits forward while the host plans, "
                               "misses copied on two side streams, misses forward)",
                     "per_launch": f"{misses / max(1, steps * L):.2f} missed slots x {sb} B per layer-step"},
        "offload": {"hit_rate_steady": round(hits / max(1, hits + misses), 4),
                    "hit_rate_warmup": round(stats["hits"][:warmup].sum() /
                                             max(1, stats["hits"][:warmup].sum() + stats["misses"][:warmup].sum()), 4),
                    "model_tokens_per_s": round(T * steps / wall, 2), "ms_per_layer_step": round(wall * 1e3 / (steps * L), 4),
                    "miss_GB_per_step": round(miss_bytes / steps / 1e9, 3), "h2d_copy_GBps_alone": round(h2d_gbs, 2),
                    **({"ms_per_layer_step_all_hits": all_hits} if all_hits is not None else {}),
                    "warmup_s": round(t_cold, 2)},
        **({"cpu_baseline": cpu_checks.pop("cpu_baseline"), "parity": cpu_checks} if cpu_checks is not None else {}),
    }


# ---------------------------------------------------------------- main

def bench_config(name: str, steps: int, warmup: int, replicas: int, distinct: int, want_cpu: bool,
                 slice_check: bool = True):
    from expert_offload_serving_amd import synth
    inp = build_inputs(name, steps + warmup, replicas, distinct)
    H, I, E, k, T = inp["H"], inp["I"], inp["E"], inp["k"], inp["T"]
    log(f"{name}: running {warmup} warmup + {steps} timed steps, {replicas} bank copies")
    res = run_gpu(inp, steps, warmup, slice_check)
    res["last_index"] = steps + warmup - 1
    mx = inp["fmt"] == "mxfp4"
    sb = synth.mx_slot_nbytes(H, I) if mx else synth.slot_nbytes(H, I)
    ms_step = res["wall"] * 1e3 / steps
    tokens_s = T * steps / res["wall"]
    mean_d = float(np.mean(res["distinct"]))
    bytes_fwd = (mean_d + 1) * sb                       # touched expert slots incl. the shared expert
    prefill = T > 16
    # roofline unit: a decode step is one route_forward call (up to 8 tokens its first kernel routes in its
    # prologue), so that call is the unit; prefill routes in kernels of its own, so its unit is the forward call
    fwd_s = (res["fwd_ms"] if prefill else res["call_ms"]) * 1e-3
    gbs = bytes_fwd / fwd_s / 1e9
    flops = synth.prefill_flops(T, H, I, k)
    if prefill:
        tf = flops / fwd_s / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": counted_traffic(name, "prefill"),
                "kernel": ("moe_mxfp4_forward prefill (prep_plan_kernel, tile_gemm_kernel<..., MX> over 128/64/32-row "
                           "tiles for gate_up and down on v_mfma_f32_16x16x32_bf16, combine_kernel), timed together "
                           "with HIP events") if mx else
                          ("moe_nvfp4_forward prefill (prep_plan_kernel, tile_gemm_kernel over 128/64/32-row tiles for "
                           "gate_up and down, combine_kernel), timed together with HIP events"),
                "per_launch": f"{flops / 1e9:.2f} GFLOP per forward (2*3*I*H*(T*k+T))"}
    elif mx:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": counted_traffic(name, "mxfp4"),
                "kernel": "moe_mxfp4_route_forward decode call (mx_fused_kernel or mx_wave_kernel, routing in "
                          "the prologue up to 8 tokens and in route_small_kernel above: gate_up on "
                          "v_mfma_scale_f32_16x16x128_f8f6f4, down on v_mfma_f32_16x16x32_bf16; then "
                          "dcombine_kernel), timed together with HIP events",
                "per_launch": f"{bytes_fwd / 1e6:.2f} MB expert weights per forward ((D+1) x {sb} B, "
                              f"mean D = {mean_d:.2f})"}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": counted_traffic(name, "decode"),
                "kernel": "moe_nvfp4_route_forward decode call (up to 8 tokens fused_kernel routes in its "
                          "prologue; above, route_small_kernel then wave_kernel; then dcombine_kernel), "
                          "timed together with HIP events",
                "per_launch": f"{bytes_fwd / 1e6:.2f} MB expert weights per forward ((D+1) x {sb} B, "
                              f"mean D = {mean_d:.2f})"}
    out = {
        "metric": METRIC_MX if mx else METRIC, "value": round(tokens_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": (DTYPE_MX_PREFILL if prefill else DTYPE_MX) if mx else DTYPE, "data": "synthetic",
        "config": {"workload": name, "H": H, "I": I, "E": E, "k": k, "T": T, "shared_expert": True,
                   "bank_copies": replicas, "distinct_quantized_experts": min(distinct, E + 1),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"route_us": round(res["route_ms"] * 1e3, 2), "forward_us": round(res["fwd_ms"] * 1e3, 2),
                  "route_forward_us": round(res["call_ms"] * 1e3, 2),
                  "step_us": round(ms_step * 1e3, 2), "expert_weight_GBps_forward": round(gbs, 1),
                  "expert_weight_GBps_step": round(bytes_fwd / (ms_step * 1e-3) / 1e9, 1),
                  "graph_replay_matches_eager": bool(res["replay_ok"])},
    }
    if res["slice_check"] is not None:
        out["slice_check"] = res["slice_check"]
    if prefill:
        out["layer"]["forward_TFLOPs"] = round(flops / fwd_s / 1e12, 2)
        out["layer"]["expert_count_range"] = [res["counts_min"], res["counts_max"]]
    if want_cpu:
        # the CPU-baseline leg (the only part of the benchmark that runs the oracle): the oracle timed on a
        # sample of this workload, and the last timed step's output checked against it
        log(f"{name}: timing the oracle (child process)")
        out["cpu_baseline"] = cpu_baseline(name, "tokens/s")
        try:
            out["parity"] = parity_sample(inp, res, 4)
        except Exception as e:  # the parity sample is a report, not the measurement
            out["parity"] = {"error": str(e)}
    return out


ROUTER_CONFIGS = {"router_bs1": 1, "router_bs16": 16, "router_2048": 2048}


def bench_router(name: str, steps: int, warmup: int, replicas: int) -> dict:
    """Router projection (moe_router_logits) and router + top-k (moe_router_topk) at H=2560, E=256, k=8.

    The weights rotate over `replicas` copies (R x 1.31 MB, more than the Infinity Cache holds) so every step
    reads them from HBM, as a decode step does after the other layers have streamed through."""
    import torch
    from expert_offload_serving_amd import _lib, synth
    from expert_offload_serving_amd import layer as dl
    T, H, E, k = ROUTER_CONFIGS[name], 2560, 256, 8
    rng = np.random.default_rng(77 + T)
    x = torch.from_numpy(synth.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))).cuda()
    base = synth.f32_to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    wr = torch.from_numpy(base).cuda().unsqueeze(0).repeat(replicas, 1, 1).contiguous()
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    r = dl.Routing.empty(T, E, k)
    nb = _lib.moe_route_workspace_bytes(T, E, k)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

    def call(i: int, topk: bool):
        w = wr[i % replicas]
        if topk:
            _lib.check(_lib.moe_router_topk(x, w, T, H, E, k, logits, r.ids, r.w, r.offsets, r.sorted_assign,
                                            r.assign_pos, ws, nb, None))
        else:
            _lib.check(_lib.moe_router_logits(x, w, T, H, E, logits, None))

    def timed(topk: bool) -> float:
        for i in range(warmup):
            call(i, topk)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                call(i, topk)
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3  # us per call

    us_logits = timed(False)
    us_topk = timed(True)
    wbytes = E * H * 2
    decode = T <= 16
    flops = 2.0 * T * E * H
    if decode:
        gbs = (wbytes + T * H * 2 + T * E * 4) / (us_logits * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": f"router_gemv_kernel<2, {1 if T == 1 else (2 if T == 2 else 4)}> (moe_router_logits), HIP events around a graph of calls",
                "per_launch": f"{(wbytes + T * H * 2 + T * E * 4) / 1e6:.3f} MB (router weights, x, logits)"}
    else:
        tf = flops / (us_logits * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "router_logits_kernel<2, 4> (moe_router_logits), HIP events around a graph of calls",
                "per_launch": f"{flops / 1e9:.3f} GFLOP (2*T*E*H)"}
    return {"metric": "router projection + top-k tokens/s, bf16 W_r [E, H]", "value": round(T / (us_topk * 1e-6), 2),
            "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(us_topk / 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": name, "H": H, "E": E, "k": k, "T": T, "weight_copies": replicas,
                       "parallelism": "single GPU"},
            "roofline": roof,
            "router": {"logits_us": round(us_logits, 2), "router_topk_us": round(us_topk, 2)}}


def copy_calibration(nbytes: int, reps: int) -> None:
    """A plain device copy of known size (torch's elementwise negation of an fp32 buffer: reads and writes
    nbytes each), launched reps times; its FETCH_SIZE / WRITE_SIZE per dispatch calibrate the counters."""
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch.neg fp32 (vectorized_elementwise_kernel)",
                                           "read_bytes": n * 4, "write_bytes": n * 4, "dispatches": reps}}),
          flush=True)


REPLICAS = {"decode_bs1": 16, "decode_bs16": 8, "prefill_2048": 4,  # bank copies rotated over steps
            "mxfp4_decode_bs1": 16, "mxfp4_decode_bs16": 8, "mxfp4_prefill_2048": 4}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="all",
                    choices=["decode_bs1", "decode_bs16", "prefill_2048", "offload", "offload_prefill", "mxfp4_decode_bs1",
                             "mxfp4_decode_bs16", "mxfp4_prefill_2048", "all", *ROUTER_CONFIGS])
    ap.add_argument("--replicas", type=int, default=0,
                    help="copies of the expert bank rotated over steps (default 16 at bs 1, 8 at bs 16, 4 prefill)")
    ap.add_argument("--distinct", type=int, default=32, help="experts quantized; the other slots are sign-flipped "
                                                              "copies of them (every slot distinct)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-slice-check", action="store_true",
                    help="decode: skip the I/2 slice check after the timed region (profiling runs: its kernels "
                         "would join the counted ones)")
    ap.add_argument("--residency", type=float, default=0.37,
                    help="offload: fraction of the 48 x 256 expert-layers the HBM cache holds")
    ap.add_argument("--aliased-banks", action="store_true",
                    help="offload: 256 pinned base slots aliased by the 48 layers instead of 48 x 256 distinct ones")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (for calibrating HBM byte counters) and exit")
    ap.add_argument("--cpu-leg", default=None, help=argparse.SUPPRESS)  # internal: the oracle timing child process
    args = ap.parse_args()
    if args.cpu_leg:
        print(json.dumps(cpu_leg(args.cpu_leg)), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the layer runs on a single MI355X here (--gpus {args.gpus}, "
              f"WORLD_SIZE {world} requested); see the design notes for how it would shard.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 4)
        return
    from expert_offload_serving_amd import _lib
    _lib.lib()
    want_cpu = not args.no_cpu_baseline

    def run(name):
        if name in ROUTER_CONFIGS:
            return bench_router(name, args.steps, args.warmup, 256)
        if name == "offload":
            steps, warmup = (64, 16) if args.steps == 200 and args.warmup == 10 else (args.steps, args.warmup)
            return bench_offload(steps, warmup, args.distinct, want_cpu, args.residency,
                                 not args.aliased_banks)
        if name == "offload_prefill":  # 2048-token chunks through all 48 layers: a few steps
            return bench_offload(3, 1, args.distinct, want_cpu, args.residency, not args.aliased_banks, T=2048)
        steps, warmup = args.steps, args.warmup
        if name.endswith("prefill_2048"):
            steps, warmup = max(1, min(steps, 20)), max(1, min(warmup, 3))
        reps = args.replicas or REPLICAS[name]
        return bench_config(name, steps, warmup, reps, args.distinct, want_cpu, not args.no_slice_check)

    if args.config != "all":
        print(json.dumps(run(args.config)), flush=True)
        return
    # every workload, one line: the headline decode batch 1 at the top level, the others under "configs"
    head = run("decode_bs1")
    head["configs"] = {}
    for name in ("decode_bs16", "prefill_2048", "offload", "offload_prefill", "mxfp4_decode_bs1",
                 "mxfp4_decode_bs16", "mxfp4_prefill_2048"):
        head["configs"][name] = run(name)
        torch.cuda.empty_cache()
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()
