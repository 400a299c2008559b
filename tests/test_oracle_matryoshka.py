"""Pins for the nested two/four-bit oracle (oracle.matryoshka; CPU only).

Independent references: hand-derived plane bytes (tests/golden/pack_m1_planes.txt),
the plane round trip, the arithmetic identities of the floor-and-compensation
weight (error exactly (1.5 - l) * s, zero mean over the sixteen codes), the
four-bit oracle layer (tau = 0 must equal it exactly), a dense-masked two-bit
formulation (tau > 1), and a brute-force per-expert precision decision.
"""
import os

import numpy as np

from oracle import bf16, ffn, matryoshka as mat, quant, route

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_bits(shape, std, seed):
    rng = np.random.default_rng(seed)
    return bf16.to_bits(bf16.round_to_bf16(rng.normal(0, std, size=shape)))


def load_golden():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "pack_m1_planes.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "case":
            cur = {"N": int(f[1]), "K": int(f[2]), "inter": f[3] == "interleave", "w": [], "hi": {}, "lo": {},
                   "scale": {}}
            cases.append(cur)
        elif f[0] == "w":
            cur["w"].append((int(f[1]), int(f[2]), float(f[3])))
        elif f[0] in ("hi", "lo"):
            cur[f[0]][int(f[1])] = bytes.fromhex(f[2])
        elif f[0] == "scale":
            cur["scale"][int(f[1])] = int(f[2], 16)
    return cases


def test_planes_match_hand_derived_golden_bytes():
    for case in load_golden():
        N, K = case["N"], case["K"]
        w = np.zeros((N, K))
        for r, c, v in case["w"]:
            w[r, c] = v
        q, s = quant.quantize_values(w)
        hi, lo, sc = mat.pack_m1(q, s, gateup_interleave=case["inter"])
        exp_hi = np.full(N * K // 4, 0x55, dtype=np.uint8)
        exp_lo = np.zeros(N * K // 4, dtype=np.uint8)
        for off, b in case["hi"].items():
            exp_hi[off:off + len(b)] = np.frombuffer(b, dtype=np.uint8)
        for off, b in case["lo"].items():
            exp_lo[off:off + len(b)] = np.frombuffer(b, dtype=np.uint8)
        assert np.array_equal(hi, exp_hi)
        assert np.array_equal(lo, exp_lo)
        exp_sc = np.zeros(N * K // 128, dtype=np.uint16)
        for i, v in case["scale"].items():
            exp_sc[i] = v
        assert np.array_equal(sc, exp_sc)


def test_plane_round_trip_and_nesting():
    rng = np.random.default_rng(3)
    for N, K, inter in ((32, 512, False), (64, 256, True)):
        q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        s = np.ones((N, K // 128))
        hi, lo, _ = mat.pack_m1(q, s, gateup_interleave=inter)
        h = mat.unpack_plane(hi, N, K, inter)
        l = mat.unpack_plane(lo, N, K, inter)
        assert np.array_equal(4 * h.astype(int) + l - 8, q)          # nested: c = 4h + l
        assert np.array_equal(h, (q.astype(int) + 8) // 4)            # h is the floor of c / 4


def test_floor_compensation_identities():
    rng = np.random.default_rng(4)
    w = bf16.to_f64(rand_bits((16, 256), 0.05, 5))
    q, s = quant.quantize_values(w)
    _, l = mat.split_planes(q)
    full, flo = mat.dequant_full(q, s), mat.dequant_floor(q, s)
    assert np.array_equal(full, quant.dequantize(q, s))               # four bits: the W4A16 weight
    assert np.array_equal(flo - full, quant.dequantize(1.5 - l.astype(float), s))
    codes = np.arange(16)
    err = (4 * (codes >> 2) + 1.5 - 8) - (codes - 8)                  # over the sixteen codes
    assert err.sum() == 0 and np.abs(err).max() == 1.5               # unbiased, at most 1.5 steps
    assert rng is not None


def test_blob_layout_m1_has_the_v1_sizes():
    for d, I in ((2048, 1024), (256, 512), (4096, 14336)):
        offs, total = mat.blob_layout_m1(d, I)
        v1offs, v1total = quant.blob_layout(d, I)
        assert total == v1total                # the two planes together are the nibble codes
        hi13, lo13, sc13, hi2, lo2, sc2 = offs
        # two-bit part first (w13 hi, w13 scales, w2 hi, w2 scales), then the low planes
        assert hi13 == 0 and sc13 == hi13 + 2 * I * d // 4 and hi2 >= sc13 + 2 * I * (d // 128) * 2
        assert sc2 == hi2 + d * I // 4 and lo13 >= sc2 + d * (I // 128) * 2 and lo2 == lo13 + 2 * I * d // 4
        assert mat.two_bit_prefix_m1(d, I) == lo13
        assert total - lo13 == 3 * I * d // 4    # the low planes: half of the code bytes


def layer_inputs(T, d, E, k, I, seed):
    w13 = [rand_bits((2 * I, d), 0.05, seed + 2 * e) for e in range(E)]
    w2 = [rand_bits((d, I), 0.05, seed + 2 * e + 1) for e in range(E)]
    return rand_bits((T, d), 1.0, seed + 99), rand_bits((E, d), 0.02, seed + 98), w13, w2


def test_layer_tau0_is_the_four_bit_layer_and_tau_above_one_is_all_two_bit():
    T, d, E, k, I = 12, 256, 8, 2, 256
    xb, wr, w13, w2 = layer_inputs(T, d, E, k, I, 40)
    bank = mat.MatBank(lambda e: w13[e], lambda e: w2[e])
    ref4 = ffn.moe_layer(xb, wr, ffn.DequantBank(lambda e: w13[e], lambda e: w2[e]), k)
    got4 = mat.moe_layer(xb, wr, bank, k, tau=0.0)
    assert all(got4["precision"].values())
    assert np.array_equal(got4["out"], ref4["out"])
    got2 = mat.moe_layer(xb, wr, bank, k, tau=2.0)
    assert not any(got2["precision"].values())
    # dense-masked two-bit formulation: out[t] = sum_j w_tj FFN_floor(x_t), no permutation
    _, ids, wts = route.route(xb, wr, k)
    x = bf16.to_f64(xb)
    for t in range(T):
        acc = np.zeros(d)
        for j in range(k):
            e = int(ids[t, j])
            q13, s13 = quant.quantize_g128(w13[e])
            q2, s2 = quant.quantize_g128(w2[e])
            acc = acc + wts[t, j] * ffn.expert_ffn(mat.dequant_floor(q13, s13), mat.dequant_floor(q2, s2), x[t:t + 1])[0]
        assert np.allclose(got2["out"][t], acc, rtol=1e-12, atol=1e-14)
    assert not np.allclose(got2["out"], got4["out"], rtol=1e-3, atol=0)


def test_precision_decision_brute_force():
    rng = np.random.default_rng(8)
    ids = rng.integers(0, 6, size=(20, 3))
    w = rng.random((20, 3))
    for tau in (0.0, 0.3, 0.7, 1.5):
        prec = mat.expert_precision(ids, w, tau)
        for e in set(ids.ravel().tolist()):
            best = max(w[t, j] for t in range(20) for j in range(3) if ids[t, j] == e)
            assert prec[e] == (best >= tau)
