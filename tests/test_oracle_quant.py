"""Pins for the oracle's bf16 helpers, quantiser and packed layout (CPU only).

Each check ties the oracle to something other than itself: torch's own
float32->bf16 conversion, exact rational arithmetic (fractions.Fraction),
brute-force search over every code, closed-form invariants, and hand-derived
packed bytes stored under tests/golden/.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def all_bf16_bits():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def finite_bf16_values():
    v = bf16.to_f64(all_bf16_bits())
    return v[np.isfinite(v)]


# ---------------------------------------------------------------- bf16 helpers

def test_bf16_decode_known_patterns():
    assert bf16.to_f64([0x3F80])[0] == 1.0
    assert bf16.to_f64([0xC000])[0] == -2.0
    assert bf16.to_f64([0x0001])[0] == 2.0 ** -133          # smallest subnormal
    assert bf16.to_f64([0x0080])[0] == 2.0 ** -126          # smallest normal
    assert bf16.to_f64([0x7F7F])[0] == (2 - 2 ** -7) * 2.0 ** 127
    assert np.isinf(bf16.to_f64([0x7F80])[0])


def test_round_to_bf16_matches_torch_conversion():
    # torch's float32 -> bfloat16 cast is round-to-nearest-even; float32 inputs
    # are exact in float64, so both must agree everywhere (normals, subnormals, ties).
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties: low half = 0x8000 with even and odd kept parts
    ties = (rng.integers(0, 1 << 16, size=20_000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    f = np.concatenate([bits, ties]).view(np.float32)
    f = f[np.isfinite(f)]
    f = f[np.abs(f) < 3.38e38]
    ours = bf16.round_to_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_round_to_bf16_fixed_points():
    v = finite_bf16_values()
    assert np.array_equal(bf16.round_to_bf16(v), v)
    assert np.array_equal(bf16.to_f64(bf16.to_bits(v)), v)


# ---------------------------------------------------------------- scale rule

def nearest_bf16_exact(x: Fraction, candidates):
    """Brute force: the bf16 candidate closest to x, ties to even significand."""
    best = None
    for c in candidates:
        dist = abs(Fraction(c) - x)
        key = (dist, int(bf16.to_bits([c])[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_scale_is_exactly_nearest_bf16_of_amax_over_7():
    # every bf16 amax in [1, 2) and a spread of binades, checked with exact rationals
    vals = finite_bf16_values()
    vals = vals[vals > 0]
    amax = np.concatenate([vals[(vals >= 1) & (vals < 2)] * 2.0 ** e for e in (-120, -20, -3, 0, 5, 90)])
    s = quant.scale_for(amax)
    pos = vals
    for a, got in zip(amax, s):
        x = Fraction(a) / 7
        lo = pos[pos <= float(x) * 1.01]
        cand = [lo.max()] + list(pos[(pos >= float(x) * 0.99) & (pos <= float(x) * 1.02)])
        assert got == nearest_bf16_exact(x, cand)


def test_scale_of_subnormal_amax_and_zero():
    assert quant.scale_for(0.0) == 0.0
    tiny = 2.0 ** -133                     # smallest bf16 subnormal: /7 rounds to 0
    assert quant.scale_for(tiny) == 0.0
    q, s = quant.quantize_values(np.full((1, 128), tiny))
    assert s[0, 0] == 0.0 and np.all(q == 0)


# ---------------------------------------------------------------- code rule

def brute_force_codes(w, s):
    """argmin over q in [-8, 7] of |w - q*s| (exact in float64), ties to even q."""
    qs = np.arange(-8, 8, dtype=np.float64)
    err = np.abs(w[:, None] - qs[None, :] * s)          # q*s and the difference are exact here
    best = err.min(axis=1, keepdims=True)
    cand = err == best
    even = cand & (qs[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1)[:, None], even, cand)
    return qs[np.argmax(pick, axis=1)].astype(np.int8)


def test_codes_brute_force_all_bf16_scales_in_1_2():
    vals = finite_bf16_values()
    for s in vals[(vals >= 1) & (vals < 2)]:
        w = vals[np.abs(vals) <= 8.5 * s]
        assert np.array_equal(quant.codes_for_scale(w, s), brute_force_codes(w, s)), s


def test_codes_scale_invariance_by_powers_of_two():
    # q depends only on w/s, so scaling both by 2^j (staying normal) changes nothing
    vals = finite_bf16_values()
    s = vals[(vals >= 1) & (vals < 2)][::7]
    w = vals[(np.abs(vals) <= 12) & (np.abs(vals) > 2 ** -20)]
    base = np.stack([quant.codes_for_scale(w, si) for si in s])
    for j in (-100, -30, 17, 100):
        moved = np.stack([quant.codes_for_scale(w * 2.0 ** j, si * 2.0 ** j) for si in s])
        assert np.array_equal(base, moved)


def random_bf16_weights(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(shape, generator=g) * std).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_quantize_invariants():
    wb = random_bf16_weights((64, 1024), 0.02, 7)
    w = bf16.to_f64(wb)
    q, s = quant.quantize_g128(wb)
    g = w.reshape(64, 8, 128)
    qg = q.reshape(64, 8, 128).astype(np.float64)
    # error bound of round-to-nearest
    assert np.all(np.abs(g - qg * s[..., None]) <= s[..., None] / 2)
    # the amax element of every non-zero group maps to +-7, codes stay in -7..7
    amax_idx = np.argmax(np.abs(g), axis=-1)
    qa = np.take_along_axis(qg, amax_idx[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(qa) == 7)
    assert q.min() >= -7 and q.max() <= 7
    # symmetric: quantize(-W) = -quantize(W) with the same scales
    qn, sn = quant.quantize_values(-w)
    assert np.array_equal(sn, s) and np.array_equal(qn, -q)
    # scales are bf16 values
    assert np.array_equal(bf16.round_to_bf16(s), s)


def test_quantize_idempotent_on_dequantised_weights():
    wb = random_bf16_weights((32, 512), 0.05, 11)
    q, s = quant.quantize_g128(wb)
    q2, s2 = quant.quantize_values(quant.dequantize(q, s))
    assert np.array_equal(s2, s) and np.array_equal(q2, q)


def test_zero_group():
    w = np.zeros((16, 256))
    w[3, 200] = 0.5
    q, s = quant.quantize_values(w)
    assert s[0, 0] == 0 and np.all(q[:, :128] == 0)
    assert s[3, 1] == quant.scale_for(0.5) and q[3, 200] == 7


# ---------------------------------------------------------------- packed layout

def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(3)
    for N, K, inter in ((16, 128, False), (64, 384, False), (64, 256, True), (96, 128, True)):
        q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        s = bf16.round_to_bf16(rng.uniform(0.001, 0.1, size=(N, K // 128)))
        codes, scales = quant.pack_v1(q, s, gateup_interleave=inter)
        assert codes.size == N * K // 2 and scales.size == N * K // 128
        q2, s2 = quant.unpack_v1(codes, scales, N, K, gateup_interleave=inter)
        assert np.array_equal(q, q2) and np.array_equal(s, s2)


def load_golden_pack():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "pack_v1_tiles.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tag, *rest = line.split()
            if tag == "case":
                cur = {"N": int(rest[0]), "K": int(rest[1]), "inter": rest[2] == "interleave",
                       "set": [], "fill": None, "expect": []}
                cases.append(cur)
            elif tag == "w":
                cur["set"].append((int(rest[0]), int(rest[1]), float(rest[2])))
            elif tag == "fill":
                cur["fill"] = rest[0]
            elif tag == "bytes":
                cur["expect"].append((int(rest[0]), bytes.fromhex("".join(rest[1:]))))
            elif tag == "scale":
                cur.setdefault("scales", []).append((int(rest[0]), int(rest[1], 16)))
    return cases


def test_pack_matches_hand_derived_golden_bytes():
    cases = load_golden_pack()
    assert cases
    for c in cases:
        w = np.zeros((c["N"], c["K"]))
        for r, k, v in c["set"]:
            w[r, k] = v
        q, s = quant.quantize_values(w)
        codes, scales = quant.pack_v1(q, s, gateup_interleave=c["inter"])
        # every byte not listed is 0x44 (all codes 8, i.e. q = 0, after the rotation)
        expect = np.full(codes.size, 0x44, dtype=np.uint8)
        for off, b in c["expect"]:
            expect[off:off + len(b)] = np.frombuffer(b, dtype=np.uint8)
        assert np.array_equal(codes, expect), c
        want_sc = np.zeros(scales.size, dtype=np.uint16)
        for idx, bits in c.get("scales", []):
            want_sc[idx] = bits
        assert np.array_equal(scales, want_sc), c


def test_blob_layout_olmoe():
    offs, total = quant.blob_layout(2048, 1024)
    assert offs == (0, 2097152, 2097152 + 65536, 2097152 + 65536 + 1048576)
    assert total == 3244032
    offs, total = quant.blob_layout(4096, 14336)
    assert total == 90832896
