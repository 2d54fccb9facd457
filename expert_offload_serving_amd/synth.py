"""Seeded synthetic inputs for the NVFP4 routed-MoE layer.

This module only *makes* inputs: random weights and their NVFP4 encoding,
activations, router logits, the shared-expert gate vector, and the byte
layout of an expert slot.  It holds none of the layer's arithmetic (no
decode of codes or scales, no routing, no expert FFN): both the HIP library
and the CPU oracle read the bytes written here and decode them with their
own code.

Workloads follow the offloaded-MoE serving pages (FreeToken PR #385 "What
this adds" and issue #62 "What it touches"): gate_up is [2I, H] with the
gate rows first and the up rows after them, down is [H, I]; each row carries
packed 4-bit codes, one FP8 scale per 16 consecutive elements of the row,
and one fp32 global.  Sizes are the decode/prefill shapes of that model
family (H = 2560, I = 640) with 256 experts and top-8.

Encoding recipe (our reading; the pages do not state one): per row,
g = amax/(6*448) (1 when the row is all zero); per 16-block,
s = E4M3(amax_blk/(6*g)) rounded to nearest even and saturated at 448;
each element becomes the E2M1 code nearest to w/(s*g), ties to the even
mantissa, saturated at 6; a block whose scale rounds to 0 gets all-zero
codes.  Element 2j of a row sits in the low nibble of byte j of the
row-major code array; pack_slot then stores codes and scales in the slot's
matrix-core operand order (the byte formulas of the library header).
"""
from __future__ import annotations

import dataclasses

import numpy as np

# ----------------------------------------------------------------------------
# Slot regions: [gu_codes | gu_scales | gu_globals | dn_codes | dn_scales | dn_globals]
# ----------------------------------------------------------------------------


def slot_regions(H: int, I: int):
    """Byte (offset, size) of the six regions of one expert slot, in order."""
    sizes = [
        2 * I * H // 2,   # gate_up codes   (operand order)
        2 * I * H // 16,  # gate_up scales  (operand order)
        2 * I * 4,        # gate_up globals f32 [2I]
        H * I // 2,       # down codes      (operand order)
        H * I // 16,      # down scales     (operand order)
        H * 4,            # down globals    f32 [H]
    ]
    out, off = [], 0
    for s in sizes:
        out.append((off, s))
        off += s
    return out


def slot_nbytes(H: int, I: int) -> int:
    off, size = slot_regions(H, I)[-1]
    return off + size


# ----------------------------------------------------------------------------
# Encoders (float -> code bytes).  Generation only.
# ----------------------------------------------------------------------------


def encode_e4m3_nonneg(v: np.ndarray):
    """Round non-negative values to OCP E4M3FN, nearest-even, saturating at 448.

    Returns (byte codes u8, the rounded values as float32)."""
    v = np.minimum(np.asarray(v, dtype=np.float64), 448.0)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))      # >= -6
    q = np.exp2(e - 3.0)                                  # spacing of the binade
    m = np.rint(v / q)                                    # half-to-even
    val = m * q
    mant, ex = np.frexp(val)                              # val = mant * 2^ex, mant in [0.5, 1)
    normal = val >= 2.0 ** -6
    E = np.where(normal, ex + 6, 0)
    M = np.where(normal, np.rint((mant * 2.0 - 1.0) * 8.0), np.rint(val / 2.0 ** -9))
    byte = (E.astype(np.int64) << 3) | M.astype(np.int64)
    byte = np.where(val == 0.0, 0, byte)
    return byte.astype(np.uint8), val.astype(np.float32)


def encode_e2m1(r: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (ties to even mantissa, saturating at 6) of float32 r."""
    a = np.abs(r)
    mag = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
           + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    sign = (np.signbit(r)).astype(np.uint8) << 3
    return (mag.astype(np.uint8) | sign).astype(np.uint8)


def quantize_nvfp4(W: np.ndarray):
    """Quantize float32 W [rows, K] (K % 16 == 0) to (codes [rows,K/2], scales [rows,K/16], globals [rows])."""
    W = np.asarray(W, dtype=np.float32)
    rows, K = W.shape
    assert K % 16 == 0
    absW = np.abs(W)
    amax = absW.max(axis=1)
    g = np.where(amax > 0, amax / np.float32(6.0 * 448.0), np.float32(1.0)).astype(np.float32)
    blk = absW.reshape(rows, K // 16, 16).max(axis=2)
    target = (blk / (np.float32(6.0) * g[:, None])).astype(np.float32)
    s_byte, s_val = encode_e4m3_nonneg(target)
    denom = (s_val * g[:, None]).astype(np.float32)
    safe = np.where(denom > 0, denom, np.float32(1.0))
    r = (W.reshape(rows, K // 16, 16) / safe[..., None]).astype(np.float32)
    codes = encode_e2m1(r)
    codes = np.where((s_val > 0)[..., None], codes, np.uint8(0)).reshape(rows, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_byte.reshape(rows, K // 16), g


def _frag_gate_up(codes, scales, N: int, K: int):
    """Row-major gate_up parts -> the slot's column-grouped operand order.

    codes [N, K/2] byte b = 64q + 16m + 4g + e/2 of row r = 16t + i goes to lane
    record (q, t, 16g + i), dword m; scales [N, K/16] block 8q + 2m + h goes to
    (q, t, h, i), byte m."""
    NT, KQ = N // 16, K // 128
    c = codes.reshape(NT, 16, KQ, 4, 4, 4).transpose(2, 0, 4, 1, 3, 5)
    s = scales.reshape(NT, 16, KQ, 4, 2).transpose(2, 0, 4, 1, 3)
    return np.ascontiguousarray(c).reshape(-1), np.ascontiguousarray(s).reshape(-1)


def _frag_down(codes, scales, N: int, K: int):
    """Row-major down parts -> the slot's row-grouped operand order.

    Row r = 64p + 16j + i, codes byte b = 16k + 4g + e/2 goes to lane record
    (k, p, 16g + i), dword j; scale block 2k + h goes to (k, p, h, i), byte j."""
    NG, KC = N // 64, K // 32
    c = codes.reshape(NG, 4, 16, KC, 4, 4).transpose(3, 0, 4, 2, 1, 5)
    s = scales.reshape(NG, 4, 16, KC, 2).transpose(3, 0, 4, 2, 1)
    return np.ascontiguousarray(c).reshape(-1), np.ascontiguousarray(s).reshape(-1)


def pack_slot(gu, dn, H: int, I: int) -> np.ndarray:
    """One slot from the quantized row-major parts (codes, scales, globals) of gate_up and down."""
    assert H % 128 == 0 and I % 32 == 0, (H, I)
    gc, gs = _frag_gate_up(np.asarray(gu[0], np.uint8), np.asarray(gu[1], np.uint8), 2 * I, H)
    dc, ds = _frag_down(np.asarray(dn[0], np.uint8), np.asarray(dn[1], np.uint8), H, I)
    out = np.empty(slot_nbytes(H, I), dtype=np.uint8)
    parts = [gc, gs, np.asarray(gu[2], np.float32), dc, ds, np.asarray(dn[2], np.float32)]
    for (off, size), p in zip(slot_regions(H, I), parts):
        b = np.ascontiguousarray(p).view(np.uint8).reshape(-1)
        assert b.size == size, (b.size, size)
        out[off:off + size] = b
    return out


def random_expert_slot(rng: np.random.Generator, H: int, I: int, std: float = 0.02, fmt: str = "nvfp4") -> np.ndarray:
    """One expert: W_gu ~ N(0, std) [2I, H] and W_dn ~ N(0, std) [H, I], quantized and packed."""
    Wgu = rng.standard_normal((2 * I, H), dtype=np.float32) * np.float32(std)
    Wdn = rng.standard_normal((H, I), dtype=np.float32) * np.float32(std)
    if fmt == "mxfp4":
        return pack_mx_slot(mx_transposed(*quantize_mxfp4(Wgu)), mx_transposed(*quantize_mxfp4(Wdn)), H, I)
    return pack_slot(quantize_nvfp4(Wgu), quantize_nvfp4(Wdn), H, I)


# ----------------------------------------------------------------------------
# MXFP4 (OCP MX FP4: E2M1 elements, one E8M0 scale per 32 along the contraction axis, no global).
# Checkpoints store each matrix transposed: blocks_t [K/2, N] and scales_t [K/32, N].
# ----------------------------------------------------------------------------


def mx_slot_regions(H: int, I: int):
    """Byte (offset, size) of the four regions of one MXFP4 slot: gate_up codes, gate_up scales, down codes,
    down scales (no globals)."""
    sizes = [2 * I * H // 2, 2 * I * H // 32, H * I // 2, H * I // 32]
    out, off = [], 0
    for sz in sizes:
        out.append((off, sz))
        off += sz
    return out


def mx_slot_nbytes(H: int, I: int) -> int:
    off, size = mx_slot_regions(H, I)[-1]
    return off + size


def quantize_mxfp4(W: np.ndarray):
    """OCP MX recipe: per 32-block, shared exponent floor(log2(amax)) - 2 (E2M1's largest exponent), stored as
    E8M0 (bias 127, clamped to [0, 254]); elements the nearest E2M1 code of w / 2^e, ties to the even mantissa,
    saturating at 6; an all-zero block gets scale byte 127.  Returns row-major codes [N, K/2] (even column in the
    low nibble) and scales [N, K/32]."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % 32 == 0
    blk = np.abs(W).reshape(N, K // 32, 32).max(axis=2).astype(np.float64)
    e = np.where(blk > 0, np.floor(np.log2(np.where(blk > 0, blk, 1.0))) - 2, 0).astype(np.int64)
    sbyte = np.clip(e + 127, 0, 254)
    scale = np.exp2((sbyte - 127).astype(np.float64))
    r = (W.reshape(N, K // 32, 32).astype(np.float64) / scale[..., None]).astype(np.float32)
    codes = encode_e2m1(r).reshape(N, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sbyte.astype(np.uint8)


def mx_transposed(codes: np.ndarray, scales: np.ndarray):
    """Row-major (codes [N, K/2], scales [N, K/32]) -> the checkpoints' (blocks_t [K/2, N], scales_t [K/32, N])."""
    return np.ascontiguousarray(codes.T), np.ascontiguousarray(scales.T)


def pack_mx_slot(gu_t, dn_t, H: int, I: int) -> np.ndarray:
    """One MXFP4 slot from the transposed checkpoint tensors of gate_up (blocks_t [H/2, 2I], scales_t [H/32, 2I])
    and down (blocks_t [I/2, H], scales_t [I/32, H]), in the slot's matrix-core operand order (the byte formulas
    of the library header)."""
    assert H % 128 == 0 and I % 32 == 0, (H, I)
    N, K = 2 * I, H
    gc = np.ascontiguousarray(gu_t[0]).T.reshape(N // 16, 16, K // 128, 4, 16).transpose(2, 0, 3, 1, 4)
    gs = np.ascontiguousarray(gu_t[1]).T.reshape(N // 16, 16, K // 128, 4).transpose(2, 0, 3, 1)
    N, K = H, I
    dc = np.ascontiguousarray(dn_t[0]).T.reshape(N // 64, 4, 16, K // 32, 4, 4).transpose(3, 0, 4, 2, 1, 5)
    ds = np.ascontiguousarray(dn_t[1]).T.reshape(N // 64, 4, 16, K // 32).transpose(3, 0, 2, 1)
    out = np.empty(mx_slot_nbytes(H, I), dtype=np.uint8)
    for (off, size), part in zip(mx_slot_regions(H, I), (gc, gs, dc, ds)):
        b = np.ascontiguousarray(part).reshape(-1)
        assert b.size == size, (b.size, size)
        out[off:off + size] = b
    return out


# ----------------------------------------------------------------------------
# Activations and router logits
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def zipf_gumbel_logits(rng: np.random.Generator, T: int, E: int, s: float, ranks: np.ndarray) -> np.ndarray:
    """Logits whose top-k is sampling without replacement with p_e proportional to rank_e^-s.

    ln p_e + Gumbel(0,1) noise per (token, expert); ranks is a permutation of 1..E."""
    logp = -s * np.log(ranks.astype(np.float64))
    logp -= np.log(np.exp(logp).sum())
    u = rng.random((T, E))
    gumbel = -np.log(-np.log(np.clip(u, 1e-300, 1.0 - 1e-16)))
    return (logp[None, :] + gumbel).astype(np.float32)


# ----------------------------------------------------------------------------
# Layer workloads
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class LayerInputs:
    H: int
    I: int
    E: int
    k: int
    T: int
    bank: np.ndarray            # u8 [n_slots, slot_bytes]; slot E holds the shared expert
    slot_of_expert: np.ndarray  # i32 [E]
    shared_slot: int            # index into bank, or -1 for no shared expert
    wg: np.ndarray              # u16 bf16 bits [H], shared-expert gate projection
    x: np.ndarray               # u16 bf16 bits [T, H]
    logits: np.ndarray          # f32 [T, E]

    @property
    def slot_bytes(self) -> int:
        return self.bank.shape[1]


CONFIGS = {
    # name: (H, I, E, k, T, seed, logit kind)
    "tiny": (256, 64, 8, 2, 4, 0, "normal"),
    "decode_bs1": (2560, 640, 256, 8, 1, 1, "uniform"),
    "decode_bs16": (2560, 640, 256, 8, 16, 16, "uniform"),
    "prefill_2048": (2560, 640, 256, 8, 2048, 2048, "zipf"),
}


def flip_code_signs(slot: np.ndarray, H: int, I: int, rng: np.random.Generator, fmt: str = "nvfp4") -> np.ndarray:
    """A copy of `slot` whose E2M1 codes have their sign bits flipped by a random mask.

    The quantizer is sign-symmetric (scales and globals come from magnitudes), so the result is exactly the
    quantization of the base weights with those signs flipped: another properly quantized expert whose
    weights, for the symmetric N(0, std) draw, have the same distribution."""
    out = slot.copy()
    regions = slot_regions(H, I) if fmt == "nvfp4" else mx_slot_regions(H, I)
    for r in ((0, 3) if fmt == "nvfp4" else (0, 2)):  # gate_up codes, down codes
        off, size = regions[r]
        out[off:off + size] ^= rng.integers(0, 256, size, dtype=np.uint8) & np.uint8(0x88)
    return out


def make_bank(rng: np.random.Generator, H: int, I: int, n_slots: int, n_distinct: int | None = None,
              fmt: str = "nvfp4") -> np.ndarray:
    """n_slots quantized expert slots, every one distinct.  With n_distinct < n_slots only n_distinct experts
    are quantized; slot j >= n_distinct is base expert j % n_distinct with the signs of its codes flipped by a
    mask of its own (flip_code_signs), which keeps generation fast while no two slots hold the same weights."""
    nd = n_slots if n_distinct is None else max(1, min(n_distinct, n_slots))
    sb = slot_nbytes(H, I) if fmt == "nvfp4" else mx_slot_nbytes(H, I)
    bank = np.empty((n_slots, sb), dtype=np.uint8)
    for j in range(nd):
        bank[j] = random_expert_slot(rng, H, I, fmt=fmt)
    flips = rng.spawn(1)[0] if n_slots > nd else None
    for j in range(nd, n_slots):
        bank[j] = flip_code_signs(bank[j % nd], H, I, flips, fmt)
    return bank


def permute_slots(L: "LayerInputs", rng: np.random.Generator, spare: int = 40) -> "LayerInputs":
    """The same layer stored in a larger bank at random positions: E + 1 + spare slots, expert e at a random
    slot, the shared expert at another, and the spare slots filled with random bytes (whose scale bytes include
    the E4M3 NaN codes, so reading one shows up in the output).  The layer's values are unchanged."""
    n = L.E + 1 + spare
    order = rng.permutation(n)
    bank = rng.integers(0, 256, (n, L.slot_bytes), dtype=np.uint8)
    for e in range(L.E):
        bank[order[e]] = L.bank[L.slot_of_expert[e]]
    shared = -1
    if L.shared_slot >= 0:
        shared = int(order[L.E])
        bank[shared] = L.bank[L.shared_slot]
    som = order[:L.E].astype(np.int32)
    return LayerInputs(L.H, L.I, L.E, L.k, L.T, bank, som, shared, L.wg, L.x, L.logits)


def make_logits(rng: np.random.Generator, T: int, E: int, kind: str) -> np.ndarray:
    if kind == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if kind == "uniform":
        return rng.random((T, E), dtype=np.float32)
    if kind == "zipf":
        ranks = rng.permutation(E) + 1
        return zipf_gumbel_logits(rng, T, E, 1.2, ranks)
    raise ValueError(kind)


def make_layer(name: str, T: int | None = None, n_distinct: int | None = None, seed: int | None = None,
               shared: bool = True, fmt: str = "nvfp4") -> LayerInputs:
    """Build one configuration's inputs from its seed: streams (weights, x, logits, w_g).  fmt: the bank's slot
    format, "nvfp4" or "mxfp4"."""
    H, I, E, k, T0, seed0, kind = CONFIGS[name]
    T = T0 if T is None else T
    seed = seed0 if seed is None else seed
    r_w, r_x, r_l, r_g = np.random.default_rng(seed).spawn(4)
    n_slots = E + 1
    bank = make_bank(r_w, H, I, n_slots, n_distinct, fmt)
    x = f32_to_bf16_bits(r_x.standard_normal((T, H), dtype=np.float32))
    logits = make_logits(r_l, T, E, kind)
    wg = f32_to_bf16_bits(r_g.standard_normal(H, dtype=np.float32) * np.float32(0.02))
    return LayerInputs(H, I, E, k, T, bank, np.arange(E, dtype=np.int32), E if shared else -1, wg, x, logits)


def fresh_tokens(seed: int, T: int, H: int, E: int, kind: str):
    """New activations and logits for another step of the same layer (bench rotation)."""
    r_x, r_l = np.random.default_rng(seed).spawn(2)
    return f32_to_bf16_bits(r_x.standard_normal((T, H), dtype=np.float32)), make_logits(r_l, T, E, kind)


def expected_distinct(T: int, E: int, k: int) -> float:
    """E[#distinct experts] for T tokens each picking k of E uniformly without replacement."""
    return E * (1.0 - (1.0 - k / E) ** T)


def prefill_flops(T: int, H: int, I: int, k: int, shared: bool = True) -> float:
    """Algorithmic FLOPs of one prefill chunk: 2*3*I*H per (token, expert) pair."""
    return 2.0 * 3.0 * I * H * (T * k + (T if shared else 0))


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)

