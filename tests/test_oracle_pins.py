"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks an oracle function against something other than its own
formula: format tables from the OCP specifications (golden files), a
library decoder (torch's float8_e4m3fn), library sorting/softmax/matmul,
closed forms, hand-worked traces and algebraic invariants.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from expert_offload_serving_amd import synth


def _read_table(path):
    rows = []
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append(line.split())
    return rows


# ---------------------------------------------------------------- formats

def test_e2m1_matches_ocp_table(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "e2m1_values.txt"))
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1(int(code))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e4m3_spot_values(golden_dir):
    for byte, val in _read_table(os.path.join(golden_dir, "e4m3_spot.txt")):
        got = oracle.e4m3(int(byte, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (byte, got)


def test_e4m3_all_bytes_match_torch_decoder():
    lib_vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        got = oracle.e4m3(b)
        if math.isnan(lib_vals[b]):
            assert math.isnan(got), b
        else:
            assert got == lib_vals[b] and math.copysign(1, got) == math.copysign(1, lib_vals[b]), b


def test_e2m1_times_e4m3_is_exact_in_f32_and_bf16():
    """Every code x scale product has <= 6 significant bits: exact in f32 and bf16."""
    for c in range(16):
        for b in range(256):
            s = oracle.e4m3(b)
            if math.isnan(s):
                continue
            p = oracle.e2m1(c) * s
            p32 = float(np.float32(p))
            assert p32 == p
            pb = float(torch.tensor(p, dtype=torch.float64).to(torch.bfloat16).to(torch.float64))
            assert pb == p


# ---------------------------------------------------------------- dequant

def _independent_dequant(codes, scales, g):
    """Dequant via a literal E2M1 table and torch's E4M3 decoder, numpy float32 ops."""
    table = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
                     dtype=np.float32)
    rows, half = codes.shape
    nib = np.empty((rows, half * 2), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    sv = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    q = table[nib] * np.repeat(sv, 16, axis=1)          # exact
    return (q * g[:, None]).astype(np.float32)           # one rounding


def test_dequant_matches_independent_decode_bitexact():
    rng = np.random.default_rng(5)
    rows, K = 37, 96
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (rows, K // 16), dtype=np.uint8)
    scales[(scales & 0x7F) == 0x7F] = 0x38                # avoid NaN scales (not produced by the encoder)
    g = (rng.standard_normal(rows) * 1e-3).astype(np.float32)
    got = oracle.dequant(codes, scales, g)
    want = _independent_dequant(codes, scales, g)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_dequant_nibble_order_and_scale_blocks():
    """Byte 0x21 holds element 0 = code 1 (0.5) in its low nibble and element 1 = code 2 (1.0) in its high nibble;
    scale byte j covers elements [16j, 16j+16) of the row."""
    K = 32
    codes = np.zeros((1, K // 2), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 8] = 0xF7                                    # elements 16, 17: code 7 (6.0), code 15 (-6.0)
    scales = np.array([[0x38, 0x40]], dtype=np.uint8)     # 1.0 for block 0, 2.0 for block 1
    out = oracle.dequant(codes, scales, np.array([0.5], dtype=np.float32))
    assert out[0, 0] == 0.25 and out[0, 1] == 0.5
    assert out[0, 16] == 6.0 and out[0, 17] == -6.0
    assert np.all(out[0, 2:16] == 0) and np.all(out[0, 18:] == 0)


# ---------------------------------------------------------------- routing

def test_route_matches_bruteforce_sort_and_softmax():
    rng = np.random.default_rng(11)
    for T, E, k in [(5, 8, 2), (3, 64, 8), (4, 16, 16), (2, 9, 1)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        ids, w = oracle.route(logits, k)
        for t in range(T):
            want = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert list(ids[t]) == want
            sw = scipy.special.softmax(logits[t, want].astype(np.float64)).astype(np.float32)
            np.testing.assert_allclose(w[t], sw, rtol=2e-7, atol=0)
            assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) <= k * 2.0 ** -23


def test_route_ties_go_to_lower_index_and_k1_weight_is_one():
    logits = np.array([[-1.0, 3.0, 3.0, -0.0, 0.0, 3.0]], dtype=np.float32)
    ids, w = oracle.route(logits, 4)
    assert list(ids[0]) == [1, 2, 5, 3]                   # -0 == +0: index 3 before 4
    np.testing.assert_allclose(w[0, :3], w[0, 0])
    ids1, w1 = oracle.route(logits, 1)
    assert ids1[0, 0] == 1 and w1[0, 0] == 1.0


def test_route_rejects_nan():
    with pytest.raises(ValueError):
        oracle.route(np.array([[0.0, np.nan]], dtype=np.float32), 1)


# ---------------------------------------------------------------- router projection

def _bf16(v):
    return synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_router_logits_hand_worked_values():
    # x = [1, 2, -0.5], rows of w: [1, 1, 1] -> 2.5; [3, -1, 4] -> 3 - 2 - 2 = -1; [0.25, 0.125, 8] -> 0.5 - 4 = -3.5
    x = _bf16([[1.0, 2.0, -0.5]])
    w = _bf16([[1.0, 1.0, 1.0], [3.0, -1.0, 4.0], [0.25, 0.125, 8.0]])
    assert oracle.router_logits(x, w).tolist() == [[2.5, -1.0, -3.5]]


def test_router_logits_one_hot_picks_a_weight_column():
    rng = np.random.default_rng(5)
    w = _bf16(rng.standard_normal((7, 24)) * 0.02)
    for h in (0, 11, 23):
        x = np.zeros((1, 24), dtype=np.uint16)
        x[0, h] = 0x3F80  # bf16 1.0
        got = oracle.router_logits(x, w)[0]
        assert np.array_equal(got, synth.bf16_bits_to_f32(w[:, h]))


def test_router_logits_round_once_after_exact_accumulation():
    # 1 + 2^-24 + 2^-24 = 1 + 2^-23 exactly (a float32); accumulating in float32 would lose both small terms
    # (1 + 2^-24 is a tie that rounds to even, i.e. back to 1).
    x = _bf16([[1.0, 1.0, 1.0]])
    w = _bf16([[1.0, 2.0 ** -24, 2.0 ** -24], [1.0, 2.0 ** -24, 0.0], [1.0, 1.5 * 2.0 ** -24, 0.0]])
    got = oracle.router_logits(x, w)[0]
    assert got[0] == np.float32(1.0 + 2.0 ** -23)
    assert got[1] == np.float32(1.0)                       # exact tie -> even
    assert got[2] == np.float32(1.0 + 2.0 ** -23)          # above the tie -> up


def test_router_logits_match_exact_rational_sum():
    from fractions import Fraction
    rng = np.random.default_rng(9)
    x = _bf16(rng.standard_normal((3, 40)))
    w = _bf16(rng.standard_normal((5, 40)) * 0.02)
    got = oracle.router_logits(x, w)
    xf, wf = synth.bf16_bits_to_f32(x), synth.bf16_bits_to_f32(w)
    for t in range(3):
        for e in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[t], wf[e]))
            # the double accumulation can round; it stays within 40 double roundings of the exact sum
            assert abs(Fraction(float(got[t, e])) - exact) <= abs(exact) * Fraction(1, 2 ** 23) + Fraction(1, 2 ** 60)


def test_permute_matches_stable_argsort():
    rng = np.random.default_rng(3)
    for T, E, k in [(1, 256, 8), (16, 256, 8), (300, 32, 4), (7, 5, 5)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        off, srt, pos = oracle.permute(ids, E)
        flat = ids.reshape(-1)
        want = np.argsort(flat, kind="stable")
        assert np.array_equal(srt, want)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        assert np.array_equal(pos[srt], np.arange(T * k))


# ---------------------------------------------------------------- layer

def _byte_offsets(N, K, down):
    """Code and scale byte offsets of every (row, column) / (row, block) of a slot matrix, computed directly from
    the format's formulas (numpy broadcasting; no reshapes shared with the packer or the oracle)."""
    r = np.arange(N)[:, None]
    c = np.arange(K)[None, :]
    b = np.arange(K // 16)[None, :]
    i, g, e = r % 16, (c // 8) % 4, c % 8
    if not down:
        T, t = N // 16, r // 16
        code = 16 * (64 * ((c // 128) * T + t) + 16 * g + i) + 4 * ((c // 32) % 4) + e // 2
        scale = 4 * (16 * (2 * ((b // 8) * T + t) + b % 2) + i) + (b // 2) % 4
    else:
        P, p, j = N // 64, r // 64, (r // 16) % 4
        code = 16 * (64 * ((c // 32) * P + p) + 16 * g + i) + 4 * j + e // 2
        scale = 4 * (16 * (2 * ((b // 2) * P + p) + b % 2) + i) + j
    return code, scale


def _formula_unpack(slot, H, I, matrix):
    """(nibbles [N, K], scale bytes [N, K/16], globals [N]) of one slot matrix via _byte_offsets."""
    reg = synth.slot_regions(H, I)
    N, K = (2 * I, H) if matrix == 0 else (H, I)
    base = 3 * matrix
    def region(idx):
        off, size = reg[base + idx]
        return slot[off:off + size]
    code_off, scale_off = _byte_offsets(N, K, matrix == 1)
    nib = (region(0)[code_off] >> (4 * (np.arange(K)[None, :] & 1))) & 0xF
    return nib.astype(np.uint8), region(1)[scale_off], region(2).view(np.float32)


def _pack_nibbles(nib):
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def _dense_dequant_slot(slot, H, I):
    mats = []
    for m in (0, 1):
        nib, sc, g = _formula_unpack(slot, H, I, m)
        mats.append(_independent_dequant(_pack_nibbles(nib), sc, g).astype(np.float64))
    return mats[0], mats[1]


def test_slot_operand_order_matches_formulas():
    """The packer writes, and the oracle reads, every code nibble, scale byte and global where the format's byte
    formulas put them (plain Python loops over every element of a small slot)."""
    H, I = 256, 32
    rng = np.random.default_rng(21)
    parts = []
    for N, K in ((2 * I, H), (H, I)):
        parts.append((rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
                      rng.integers(0, 256, (N, K // 16), dtype=np.uint8),
                      rng.standard_normal(N).astype(np.float32)))
        parts[-1][1][(parts[-1][1] & 0x7F) == 0x7F] = 0x38    # no NaN scales (the encoder never makes them)
    slot = synth.pack_slot(parts[0], parts[1], H, I)
    reg = synth.slot_regions(H, I)
    for m, (N, K) in enumerate(((2 * I, H), (H, I))):
        codes, scales, g = parts[m]
        c_reg = slot[reg[3 * m][0]:][:reg[3 * m][1]]
        s_reg = slot[reg[3 * m + 1][0]:][:reg[3 * m + 1][1]]
        for r in range(N):
            for c in range(K):
                if m == 0:
                    off = 16 * (64 * ((c // 128) * (N // 16) + r // 16) + 16 * ((c // 8) % 4) + r % 16) \
                        + 4 * ((c // 32) % 4) + (c % 8) // 2
                else:
                    off = 16 * (64 * ((c // 32) * (N // 64) + r // 64) + 16 * ((c // 8) % 4) + r % 16) \
                        + 4 * ((r // 16) % 4) + (c % 8) // 2
                assert (c_reg[off] >> (4 * (c % 2))) & 0xF == (codes[r, c // 2] >> (4 * (c % 2))) & 0xF, (m, r, c)
            for bk in range(K // 16):
                if m == 0:
                    off = 4 * (16 * (2 * ((bk // 8) * (N // 16) + r // 16) + bk % 2) + r % 16) + (bk // 2) % 4
                else:
                    off = 4 * (16 * (2 * ((bk // 2) * (N // 64) + r // 64) + bk % 2) + r % 16) + (r // 16) % 4
                assert s_reg[off] == scales[r, bk], (m, r, bk)
        uc, us, ug = oracle.unpack_slot(slot, H, I, m)
        assert np.array_equal(uc, codes) and np.array_equal(us, scales)
        assert np.array_equal(ug.view(np.uint32), g.view(np.uint32))
        want = _independent_dequant(codes, scales, g)
        assert np.array_equal(oracle.dequant_slot(slot, H, I, m).view(np.uint32), want.view(np.uint32))


def test_slot_shape_guard():
    assert oracle.slot_bytes(128, 32) > 0
    for H, I in ((96, 32), (320, 64), (128, 48)):
        with pytest.raises(ValueError):
            oracle.dequant_slot(np.zeros(oracle.slot_bytes(H, I), np.uint8), H, I, 0)


def _bruteforce_layer(L, ids, w, shared=True):
    """Dense float64 reference: torch matmul, torch.nn.functional.silu, torch.sigmoid."""
    X = torch.from_numpy(synth.bf16_bits_to_f32(L.x).astype(np.float64))
    Y = torch.zeros((L.T, L.H), dtype=torch.float64)
    dense = {}
    def ffn(slot_idx, xrows):
        if slot_idx not in dense:
            dense[slot_idx] = [torch.from_numpy(m) for m in _dense_dequant_slot(L.bank[slot_idx], L.H, L.I)]
        Wgu, Wdn = dense[slot_idx]
        A = xrows @ Wgu.T
        Hh = torch.nn.functional.silu(A[:, :L.I]) * A[:, L.I:]
        return Hh @ Wdn.T
    for t in range(L.T):
        for j in range(L.k):
            s = int(L.slot_of_expert[ids[t, j]])
            if s >= 0:
                Y[t] += float(w[t, j]) * ffn(s, X[t:t + 1])[0]
        if shared and L.shared_slot >= 0:
            gate = torch.sigmoid(X[t] @ torch.from_numpy(synth.bf16_bits_to_f32(L.wg).astype(np.float64)))
            Y[t] += gate * ffn(L.shared_slot, X[t:t + 1])[0]
    return Y.numpy()


def _run_oracle(L, ids, w, **kw):
    return oracle.forward(L.H, L.I, L.E, L.k, L.bank, L.slot_of_expert, L.shared_slot, L.wg, L.x, ids, w, **kw)


def test_forward_tiny_matches_dense_bruteforce():
    L = synth.make_layer("tiny")
    ids, w = oracle.route(L.logits, L.k)
    y = _run_oracle(L, ids, w)
    ref = _bruteforce_layer(L, ids, w)
    assert np.max(np.abs(y - ref)) <= 1e-6 * np.max(np.abs(ref))
    assert np.abs(ref).max() > 0


def test_forward_token_subset_and_skipped_experts():
    L = synth.make_layer("tiny", T=6)
    ids, w = oracle.route(L.logits, L.k)
    full = _run_oracle(L, ids, w)
    sub = _run_oracle(L, ids, w, tokens=[4, 1])
    assert np.array_equal(sub, full[[4, 1]])
    # leaving every routed expert out leaves exactly the gated shared expert
    L2 = synth.make_layer("tiny", T=6)
    L2.slot_of_expert = np.full(L2.E, -1, dtype=np.int32)
    only_shared = _run_oracle(L2, ids, w)
    ref = _bruteforce_layer(L2, ids, w)
    assert np.max(np.abs(only_shared - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_forward_special_cases():
    L = synth.make_layer("tiny")
    ids, w = oracle.route(L.logits, L.k)
    # all-zero bank -> y = 0
    Z = synth.make_layer("tiny")
    Z.bank = np.zeros_like(Z.bank)
    assert np.all(_run_oracle(Z, ids, w) == 0)
    # w_g = 0 -> sigmoid(0) = 1/2: y = routed + shared/2
    G = synth.make_layer("tiny")
    G.wg = np.zeros_like(G.wg)
    y = _run_oracle(G, ids, w)
    G2 = synth.make_layer("tiny"); G2.wg = np.zeros_like(G2.wg); G2.shared_slot = -1
    routed = _run_oracle(G2, ids, w)
    G3 = synth.make_layer("tiny"); G3.wg = np.zeros_like(G3.wg); G3.slot_of_expert[:] = -1
    shared = _run_oracle(G3, ids, w)
    np.testing.assert_allclose(y, routed + shared, rtol=1e-6, atol=1e-7)
    s = oracle.shared_gate(G.x, G.wg)
    assert np.all(s == 0.5)


def test_forward_closed_form_all_ones_expert():
    """One expert whose every weight is 1 (codes 2 = 1.0, scale 0x38 = 1.0, globals 1): with x = 0.5 everywhere,
    a_r = H/2 for every row, h_i = silu(H/2) * H/2, o_r = I * h; k=1 gives w=1 and y = o."""
    H, I, E = 128, 32, 1
    sb = synth.slot_nbytes(H, I)
    slot = np.zeros(sb, dtype=np.uint8)
    reg = synth.slot_regions(H, I)
    for i in (0, 3):
        off, size = reg[i]; slot[off:off + size] = 0x22
    for i in (1, 4):
        off, size = reg[i]; slot[off:off + size] = 0x38
    for i in (2, 5):
        off, size = reg[i]; slot[off:off + size] = np.ones(size // 4, dtype=np.float32).view(np.uint8)
    bank = slot[None, :]
    x = synth.f32_to_bf16_bits(np.full((1, H), 0.5, dtype=np.float32))
    a = H / 2.0
    want = I * (a / (1.0 + math.exp(-a))) * a
    y = oracle.forward(H, I, E, 1, bank, np.array([0], np.int32), -1, np.zeros(H, np.uint16), x,
                       np.array([[0]], np.int32), np.array([[1.0]], np.float32))
    assert np.all(y == np.float32(want))


# ---------------------------------------------------------------- slicing and geometry

def test_slot_geometry_matches_pages():
    assert oracle.slot_bytes(2560, 640) == 2_780_160
    assert oracle.slot_bytes(256, 64) == 29_184
    half = oracle.slot_bytes(2560, 320)
    assert half == 1_395_200
    # PR #385 / issue #62 R9700 comment: 655 half-slots of "~1.33 MiB" are about 0.848 GiB
    assert round(half / 2 ** 20, 2) == 1.33
    assert abs(655 * half / 2 ** 30 - 0.848) < 0.005


def test_slice_dequant_equals_dequant_slice():
    H, I = 128, 128
    slot = synth.random_expert_slot(np.random.default_rng(2), H, I)
    Wgu, Wdn = _dense_dequant_slot(slot, H, I)
    for n in (2, 4):
        Il = I // n
        for r in range(n):
            sl = oracle.slice_slot(slot, H, I, r, n)
            Sgu, Sdn = _dense_dequant_slot(sl, H, Il)
            rows = np.r_[r * Il:(r + 1) * Il, I + r * Il:I + (r + 1) * Il]
            assert np.array_equal(Sgu, Wgu[rows])
            assert np.array_equal(Sdn, Wdn[:, r * Il:(r + 1) * Il])


def test_slice_partials_sum_to_full():
    L = synth.make_layer("tiny", T=5)
    ids, w = oracle.route(L.logits, L.k)
    full = _run_oracle(L, ids, w).astype(np.float64)
    tot = np.zeros_like(full)
    for r in range(2):
        S = synth.make_layer("tiny", T=5)
        S.bank = np.stack([oracle.slice_slot(b, L.H, L.I, r, 2) for b in L.bank])
        S.I = L.I // 2
        tot += _run_oracle(S, ids, w)
    assert np.max(np.abs(tot - full)) <= 1e-6 * np.max(np.abs(full))


def test_slice_rejects_partial_blocks():
    with pytest.raises(ValueError):
        oracle.slice_slot(np.zeros(synth.slot_nbytes(128, 64), np.uint8), 128, 64, 0, 4)


# ---------------------------------------------------------------- LRU model

def test_lru_hand_trace(golden_dir):
    rows = []
    for line in open(os.path.join(golden_dir, "lru_trace.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            a, b, c = line.split("|")
            rows.append(([int(v) for v in a.split()], [int(v) for v in b.split()], [int(v) for v in c.split()]))
    steps, L = 3, 2
    ids = np.zeros((steps, L, 2), dtype=np.int32)
    for (st, l, i0, i1), _, _ in rows:
        ids[st, l] = (i0, i1)
    hits, misses, smap, mslots = oracle.lru_run(ids, E=4, C=3)
    for (st, l, _, _), (h, m), ms in rows:
        assert hits[st, l] == h and misses[st, l] == m
        assert list(mslots[st, l][:m]) == ms
    assert list(smap[2, 1]) == [0, -1, 1, -1]


def test_lru_invariants():
    rng = np.random.default_rng(9)
    steps, L, E, n = 20, 3, 16, 6
    ids = rng.integers(0, E, (steps, L, n), dtype=np.int32)
    hits, misses, smap, mslots = oracle.lru_run(ids, E=E, C=12)
    for st in range(steps):
        for l in range(L):
            d = len(set(ids[st, l].tolist()))
            assert hits[st, l] + misses[st, l] == d
            routed = sorted(set(ids[st, l].tolist()))
            slots = smap[st, l][routed]
            assert np.all(slots >= 0) and len(set(slots.tolist())) == d
    # a pool holding everything misses only on first touch
    h2, m2, _, _ = oracle.lru_run(ids, E=E, C=L * E)
    first = sum(len(set(ids[:, l].reshape(-1).tolist())) for l in range(L))
    assert int(m2.sum()) == first


# ---------------------------------------------------------------- MXFP4 (the second fp4 bank format)

def test_e8m0_all_bytes_match_torch_decoder_and_closed_form():
    """E8M0 (OCP MX shared scale): 2^(byte - 127), 0xFF is NaN; every byte against torch's float8_e8m0fnu
    decoder and spot values of the closed form."""
    lib_vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for b in range(256):
        got = oracle.e8m0(b)
        if b == 255:
            assert math.isnan(got) and math.isnan(lib_vals[b])
        else:
            assert got == lib_vals[b] == 2.0 ** (b - 127), b
    assert oracle.e8m0(127) == 1.0 and oracle.e8m0(0) == 2.0 ** -127 and oracle.e8m0(254) == 2.0 ** 127


def _independent_mx_dequant_t(blocks_t, scales_t):
    """numpy decode of the transposed layout: W[n, c] from nibble c%2 of blocks_t[c//2, n] and scales_t[c//32, n],
    element values from the OCP E2M1 table, scales from torch's E8M0 decoder."""
    e2m1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    e8m0 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    K2, N = blocks_t.shape
    codes = np.empty((N, 2 * K2), dtype=np.int64)
    codes[:, 0::2] = (blocks_t.T & 15)
    codes[:, 1::2] = (blocks_t.T >> 4)
    scale = np.repeat(e8m0[scales_t.T.astype(np.int64)], 32, axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        return (e2m1[codes] * scale).astype(np.float32)


def _bits_equal(a, b):
    nan_a, nan_b = np.isnan(a), np.isnan(b)
    assert np.array_equal(nan_a, nan_b)
    assert np.array_equal(a[~nan_a].view(np.uint32), b[~nan_b].view(np.uint32))


def test_mx_dequant_every_code_and_scale_byte_bitexact():
    """Every (code, E8M0 byte) pair, including 0 (2^-127: f32 subnormal products), 254 (6 * 2^127 overflows f32
    to inf) and 255 (NaN), against the independent decode."""
    N, K = 256, 512
    codes_row = np.array([(2 * j % 16) | (((2 * j + 1) % 16) << 4) for j in range(K // 2)], dtype=np.uint8)
    blocks_t = np.tile(codes_row[:, None], (1, N))                 # [K/2, N], every code in every block
    scales_t = np.tile(np.arange(N, dtype=np.uint8)[None, :], (K // 32, 1))  # column n uses scale byte n
    scales_t[1::2] = ((scales_t[1::2].astype(np.int64) + 101) % 256).astype(np.uint8)  # other bytes, odd blocks
    _bits_equal(oracle.mx_dequant_t(blocks_t, scales_t), _independent_mx_dequant_t(blocks_t, scales_t))


def test_mx_dequant_transposed_layout_hand_case():
    """One hand-worked element per layout rule: blocks_t[j, n] holds W[n, 2j] low and W[n, 2j+1] high;
    scales_t[b, n] scales W[n, 32b .. 32b+31]."""
    N, K = 3, 64
    blocks_t = np.zeros((K // 2, N), dtype=np.uint8)
    scales_t = np.full((K // 32, N), 127, dtype=np.uint8)
    blocks_t[5, 2] = 0x7A          # W[2, 10] = e2m1(0xA) = -1.0, W[2, 11] = e2m1(0x7) = 6.0
    scales_t[0, 2] = 129           # block 0 of row 2 scaled by 4
    blocks_t[20, 1] = 0x03         # W[1, 40] = 1.5 in block 1
    scales_t[1, 1] = 120           # times 2^-7
    W = oracle.mx_dequant_t(blocks_t, scales_t)
    want = np.zeros((N, K), dtype=np.float32)
    want[2, 10], want[2, 11], want[1, 40] = -4.0, 24.0, 1.5 * 2.0 ** -7
    assert np.array_equal(W, want)


def _mx_formula_offsets(N, K, down):
    """The MXFP4 slot's byte formulas re-derived in plain loops: code byte and scale byte of every element."""
    code = np.empty((N, K), dtype=np.int64)
    scale = np.empty((N, K // 32), dtype=np.int64)
    for r in range(N):
        i = r % 16
        for c in range(K):
            if not down:   # 16-row x 128-column tile per KiB; lane 16a + i holds columns [32a, 32a + 32)
                q, a, e, t = c // 128, (c // 32) % 4, c % 32, r // 16
                code[r, c] = 16 * (64 * (q * (N // 16) + t) + 16 * a + i) + e // 2
            else:          # 64-row x 32-column tile per KiB, as the NVFP4 down matrix
                kc, g, e, p, j = c // 32, (c // 8) % 4, c % 8, r // 64, (r // 16) % 4
                code[r, c] = 16 * (64 * (kc * (N // 64) + p) + 16 * g + i) + 4 * j + e // 2
        for b in range(K // 32):
            if not down:
                q, a, t = b // 4, b % 4, r // 16
                scale[r, b] = 64 * (q * (N // 16) + t) + 16 * a + i
            else:
                p, j = r // 64, (r // 16) % 4
                scale[r, b] = 64 * (b * (N // 64) + p) + 4 * i + j
    return code, scale


def test_mx_slot_operand_order_matches_formulas():
    """The packer writes, and the oracle reads back, exactly the byte formulas: the formulas re-derived in
    plain loops place every element, the oracle's unpacking returns the checkpoint tensors, and the slot
    dequant equals the transposed-layout dequant bit for bit."""
    H, I = 256, 64
    rng = np.random.default_rng(21)
    gu = (rng.integers(0, 256, (H // 2, 2 * I), dtype=np.uint8), rng.integers(100, 150, (H // 32, 2 * I), dtype=np.uint8))
    dn = (rng.integers(0, 256, (I // 2, H), dtype=np.uint8), rng.integers(100, 150, (I // 32, H), dtype=np.uint8))
    slot = synth.pack_mx_slot(gu, dn, H, I)
    regions = synth.mx_slot_regions(H, I)
    for m, ((bt, st), (creg, sreg)) in enumerate(zip((gu, dn), ((0, 1), (2, 3)))):
        N, K = bt.shape[1], bt.shape[0] * 2
        code_off, scale_off = _mx_formula_offsets(N, K, m == 1)
        cbase, sbase = regions[creg][0], regions[sreg][0]
        nib = np.empty((N, K), dtype=np.int64)
        nib[:, 0::2], nib[:, 1::2] = bt.T & 15, bt.T >> 4
        got_nib = (slot[cbase + code_off] >> (4 * (np.arange(K)[None, :] % 2))) & 15
        assert np.array_equal(got_nib, nib)
        assert np.array_equal(slot[sbase + scale_off], st.T)
        b2, s2 = oracle.mx_unpack_slot(slot, H, I, m)
        assert np.array_equal(b2, bt) and np.array_equal(s2, st)
        _bits_equal(oracle.mx_dequant_slot(slot, H, I, m), _independent_mx_dequant_t(bt, st))
    assert slot.size == oracle.mx_slot_bytes(H, I) == 3 * I * H // 2 + 3 * I * H // 32


def test_mx_slice_along_n_and_k_equals_slice_of_dequant():
    """Slicing I (issue #62: mxfp4's slice runs along N of the transposed gate_up and along K of down): the
    dequant of each slice is the matching slice of the full dequant, and the checkpoint tensors of the slice are
    column / row slices of the full ones."""
    H, I, n = 256, 128, 2
    slot = synth.random_expert_slot(np.random.default_rng(8), H, I, fmt="mxfp4")
    Wgu, Wdn = oracle.mx_dequant_slot(slot, H, I, 0), oracle.mx_dequant_slot(slot, H, I, 1)
    (gb, gs), (db, ds) = oracle.mx_unpack_slot(slot, H, I, 0), oracle.mx_unpack_slot(slot, H, I, 1)
    Il = I // n
    for r in range(n):
        sl = oracle.mx_slice_slot(slot, H, I, r, n)
        rows = np.r_[r * Il:(r + 1) * Il, I + r * Il:I + (r + 1) * Il]
        _bits_equal(oracle.mx_dequant_slot(sl, H, Il, 0), Wgu[rows])
        _bits_equal(oracle.mx_dequant_slot(sl, H, Il, 1), Wdn[:, r * Il:(r + 1) * Il])
        sgb, sgs = oracle.mx_unpack_slot(sl, H, Il, 0)
        sdb, sds = oracle.mx_unpack_slot(sl, H, Il, 1)
        assert np.array_equal(sgb, gb[:, rows]) and np.array_equal(sgs, gs[:, rows])          # along N
        assert np.array_equal(sdb, db[r * Il // 2:(r + 1) * Il // 2])                         # along K/2
        assert np.array_equal(sds, ds[r * Il // 32:(r + 1) * Il // 32])
    with pytest.raises(ValueError):
        oracle.mx_slice_slot(slot, H, I, 0, 8)  # I/n = 16: not a whole scale block


def test_mx_forward_matches_dense_bruteforce():
    """The MXFP4 layer (tiny shape) against a float64 numpy brute force over the independently decoded weights."""
    H, I, E, k, T = 256, 64, 8, 2, 5
    rng = np.random.default_rng(31)
    bank = synth.make_bank(rng, H, I, E + 1, None, fmt="mxfp4")
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wg = synth.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32) * 0.02)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route(logits, k)
    got = oracle.forward(H, I, E, k, bank, np.arange(E, dtype=np.int32), E, wg, x, ids, w, fmt="mxfp4")
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    gf = synth.bf16_bits_to_f32(wg).astype(np.float64)
    def ffn(slot, xv):
        (gb, gs), (db, ds) = oracle.mx_unpack_slot(slot, H, I, 0), oracle.mx_unpack_slot(slot, H, I, 1)
        Wgu = _independent_mx_dequant_t(gb, gs).astype(np.float64)
        Wdn = _independent_mx_dequant_t(db, ds).astype(np.float64)
        a = Wgu @ xv
        h = a[:I] / (1.0 + np.exp(-a[:I])) * a[I:]
        return Wdn @ h
    want = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            want[t] += float(w[t, j]) * ffn(bank[ids[t, j]], xf[t])
        want[t] += 1.0 / (1.0 + np.exp(-(xf[t] @ gf))) * ffn(bank[E], xf[t])
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6 * np.abs(want).max())
