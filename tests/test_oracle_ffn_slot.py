"""Pins for the oracle's expert FFN, combine, whole layer and slot-cache policy (CPU only).

Independent references: a textbook triple-loop SwiGLU MLP in pure Python
(E = 1, k = 1 reduces the layer to one dense MLP), a dense-masked formulation
out[t] = sum_e [e in top-k(t)] w_te FFN_e(x_t) that never permutes, zero
weights, and a hand-traced LRU sequence.
"""
import math

import numpy as np

from oracle import bf16, ffn, quant, route
from oracle.slot_cache import POLICY_COST, LRUSlotCache, SlotCacheSim


def rand_bits(shape, std, seed):
    rng = np.random.default_rng(seed)
    return bf16.to_bits(bf16.round_to_bf16(rng.normal(0, std, size=shape)))


def make_bank(E, d, I, seed):
    w13 = [rand_bits((2 * I, d), 0.05, seed + 2 * e) for e in range(E)]
    w2 = [rand_bits((d, I), 0.05, seed + 2 * e + 1) for e in range(E)]
    return w13, w2, ffn.DequantBank(lambda e: w13[e], lambda e: w2[e])


def test_single_expert_is_textbook_swiglu_mlp():
    d, I = 128, 128
    w13, w2, bank = make_bank(1, d, I, 10)
    xb = rand_bits((2, d), 1.0, 11)
    wr = rand_bits((1, d), 0.02, 12)
    res = ffn.moe_layer(xb, wr, bank, k=1)
    q13, s13 = quant.quantize_g128(w13[0])
    q2, s2 = quant.quantize_g128(w2[0])
    x = bf16.to_f64(xb)
    for t in range(2):
        h = []
        for i in range(I):
            g = sum(float(q13[i, c]) * float(s13[i, c // 128]) * x[t, c] for c in range(d))
            u = sum(float(q13[I + i, c]) * float(s13[I + i, c // 128]) * x[t, c] for c in range(d))
            h.append(g / (1.0 + math.exp(-g)) * u)
        y = [sum(float(q2[n, i]) * float(s2[n, i // 128]) * h[i] for i in range(I)) for n in range(d)]
        assert res["weights"][t, 0] == 1.0
        assert np.allclose(res["out"][t], y, rtol=1e-12, atol=1e-14)


def test_bf16_bank_single_expert_is_textbook_swiglu_mlp():
    # unquantised experts: the weights are the bf16 values themselves
    d, I = 128, 128
    w13 = rand_bits((2 * I, d), 0.05, 30)
    w2 = rand_bits((d, I), 0.05, 31)
    bank = ffn.Bf16Bank(lambda e: w13, lambda e: w2)
    xb = rand_bits((2, d), 1.0, 32)
    res = ffn.moe_layer(xb, rand_bits((1, d), 0.02, 33), bank, k=1)
    W13, W2, x = bf16.to_f64(w13), bf16.to_f64(w2), bf16.to_f64(xb)
    for t in range(2):
        h = []
        for i in range(I):
            g = sum(float(W13[i, c]) * x[t, c] for c in range(d))
            u = sum(float(W13[I + i, c]) * x[t, c] for c in range(d))
            h.append(g / (1.0 + math.exp(-g)) * u)
        y = [sum(float(W2[n, i]) * h[i] for i in range(I)) for n in range(d)]
        assert np.allclose(res["out"][t], y, rtol=1e-12, atol=1e-14)
    # and it differs from the four-bit layer on the same weights (quantisation is not a no-op)
    q = ffn.moe_layer(xb, rand_bits((1, d), 0.02, 33), ffn.DequantBank(lambda e: w13, lambda e: w2), k=1)
    assert not np.allclose(q["out"], res["out"], rtol=1e-3, atol=0)


def test_layer_equals_dense_masked_formulation():
    T, d, E, k, I = 16, 256, 8, 2, 512          # the tiny workload's shape
    w13, w2, bank = make_bank(E, d, I, 20)
    xb = rand_bits((T, d), 1.0, 21)
    wr = rand_bits((E, d), 0.02, 22)
    res = ffn.moe_layer(xb, wr, bank, k=k)
    x = bf16.to_f64(xb)
    l = route.logits_f32(xb, wr).astype(np.float64)
    out = np.zeros((T, d))
    for t in range(T):
        top = sorted(range(E), key=lambda e: (-l[t, e], e))[:k]
        z = sum(math.exp(l[t, e] - l[t, top[0]]) for e in top)
        for e in range(E):
            if e not in top:
                continue
            we = math.exp(l[t, e] - l[t, top[0]]) / z
            W13 = quant.dequantize(*quant.quantize_g128(w13[e]))
            W2 = quant.dequantize(*quant.quantize_g128(w2[e]))
            g, u = W13[:I] @ x[t], W13[I:] @ x[t]
            out[t] += we * (W2 @ (g / (1 + np.exp(-g)) * u))
    assert np.allclose(res["out"], out, rtol=1e-12, atol=1e-13)
    # every selected (token, expert) pair contributed: no expert dropped
    assert len(res["y"]) == T * k


def test_zero_weights_give_zero_output():
    d, I = 128, 256
    z13 = np.zeros((2 * I, d), dtype=np.uint16)
    z2 = np.zeros((d, I), dtype=np.uint16)
    bank = ffn.DequantBank(lambda e: z13, lambda e: z2)
    res = ffn.moe_layer(rand_bits((3, d), 1.0, 1), rand_bits((4, d), 0.02, 2), bank, k=2)
    assert np.all(res["out"] == 0)


def test_sampled_tokens_match_full_layer():
    T, d, E, k, I = 12, 128, 8, 3, 128
    _, _, bank = make_bank(E, d, I, 30)
    xb, wr = rand_bits((T, d), 1.0, 31), rand_bits((E, d), 0.02, 32)
    full = ffn.moe_layer(xb, wr, bank, k=k)
    part = ffn.moe_layer(xb, wr, bank, k=k, tokens=[0, 5, 11])
    # same values up to the matmul routine's summation order for different batch sizes
    assert np.allclose(part["out"], full["out"][[0, 5, 11]], rtol=1e-13, atol=1e-15)


def test_lru_hand_traced():
    c = LRUSlotCache(num_experts=8, num_slots=3)
    # step 1: needs {5, 1}: both miss, empty slots 0, 1 (lowest first), ascending ids
    r = c.step({5, 1})
    assert r == [([1, 5], [], [(1, 0), (5, 1)])]
    # step 2: needs {1, 2, 7}: hit 1; misses 2 -> empty slot 2; 7 -> LRU among non-hit
    #   slots {1 (expert 5, stamp 1), 2 (fresh... )} -- slot 2 is empty (stamp -1) so 2 takes it,
    #   then 7 takes slot 1 (expert 5, stamp 1)
    r = c.step({1, 2, 7})
    assert r == [([1, 2, 7], [1], [(2, 2), (7, 1)])]
    assert c.slot_expert == [1, 7, 2]
    # step 3: needs {0, 3, 4, 2, 6}: hit 2 (slot 2); round 1 misses 0, 3 go to slots 0, 1
    #   (both stamp 2, lower index first); round 2: 4, 6 -> LRU: slots 0,1,2 all stamp 3
    #   -> slots 0, 1
    r = c.step({0, 3, 4, 2, 6})
    assert r == [([0, 2, 3], [2], [(0, 0), (3, 1)]), ([4, 6], [], [(4, 0), (6, 1)])]
    assert c.slot_expert == [4, 6, 2]
    # step 4: needs {2}: pure hit, no copies
    assert c.step({2}) == [([2], [2], [])]


def test_prefetch_hand_traced():
    c = LRUSlotCache(num_experts=8, num_slots=3)
    c.step({5, 1})                                   # slots [1, 5, -], stamps [1, 1, -1]
    # predicted {1, 2, 7}: 1 resident (its slot kept); 2, 7 go to the empty slot 2,
    # then to slot 1 (expert 5, least recent among the rest)
    assert c.prefetch({1, 2, 7}, 3) == [(2, 2), (7, 1)]
    assert c.slot_expert == [1, 7, 2]
    assert c.step({1, 2, 7}) == [([1, 2, 7], [1, 2, 7], [])]   # all hits now
    d = LRUSlotCache(num_experts=8, num_slots=3)
    d.step({5, 1})
    assert d.prefetch({2, 7}, 1) == [(2, 2)]         # at most max_copies, ascending id
    assert d.prefetch({7}, 0) == []
    e = LRUSlotCache(num_experts=4, num_slots=2)
    e.step({0, 1})
    assert e.prefetch({0, 1, 2}, 5) == []            # every slot holds a predicted expert
    assert e.slot_expert == [0, 1]


def test_lru_never_evicts_a_hit_and_covers_all_needed():
    rng = np.random.default_rng(5)
    c = LRUSlotCache(num_experts=64, num_slots=16)
    for _ in range(200):
        need = set(rng.choice(64, size=rng.integers(1, 40), replace=False).tolist())
        pending, covered = set(need), set()
        while pending:
            before = c.resident()
            subset, hits, copies = c.load_round(pending)
            res = c.resident()
            assert len(subset) <= 16 and set(subset) <= pending
            assert all(e in res for e in subset)              # the whole round is resident
            assert all(res[e] == before[e] for e in hits)     # hits keep their slots
            assert set(hits) == {e for e in pending if e in before}
            assert not ({e for e, _ in copies} & set(hits))
            covered |= set(subset)
            pending -= set(subset)
        assert covered == need


def test_cost_aware_hand_traced():
    # decay 0.5: usage values are dyadic fractions, exact in float64
    c = SlotCacheSim(num_experts=8, num_slots=3, policy=POLICY_COST, decay=0.5)
    # step 1 {5, 1}: u1 = u5 = 0.5; misses by (u, id) -> [1, 5] into the empty slots 0, 1
    assert c.step({5, 1}) == [([1, 5], [], [(1, 0), (5, 1)])]
    # step 2 {1, 2, 7}: u1 = .75, u2 = u7 = .5, u5 = .25; hit 1; 2 -> empty slot 2, 7 -> slot 1 (expert 5)
    assert c.step({1, 2, 7}) == [([1, 2, 7], [1], [(2, 2), (7, 1)])]
    assert c.usage[1] == 0.75 and c.usage[5] == 0.25 and c.usage[7] == 0.5
    # step 3 {0, 2, 3, 4, 6}: u0 = u3 = u4 = u6 = .5, u1 = .375, u7 = .25, u2 = .75; round 1: hit 2,
    # misses 0, 3 (u ties, by id); victims by usage: slot 1 (expert 7, .25) before slot 0
    # (expert 1, .375) -- LRU would take slot 0 first (equal stamps, lower slot)
    # round 2: 4, 6 evict slots 0 (expert 3, .5, lower slot) and 1 (expert 0, .5); expert 2 (.75) stays
    assert c.step({0, 3, 4, 2, 6}) == [([0, 2, 3], [2], [(0, 1), (3, 0)]), ([4, 6], [], [(4, 0), (6, 1)])]
    assert c.slot_expert == [4, 6, 2]
    # step 4 {1, 2}: hit 2; 1 -> slot 0 (experts 4 and 6 tie on usage .25 and stamp: lower slot)
    assert c.step({1, 2}) == [([1, 2], [2], [(1, 0)])]
    assert c.slot_expert == [1, 6, 2]
    # a later round evicts the finished expert with the lower usage
    d = SlotCacheSim(num_experts=8, num_slots=2, policy=POLICY_COST, decay=0.5)
    d.step({0})                                      # u0 = .5
    r = d.step({0, 3, 5})                            # u0 = .75, u3 = u5 = .5: hit 0, then 3 (id order)
    assert r[0] == ([0, 3], [0], [(3, 1)])
    assert r[1] == ([5], [], [(5, 1)])               # 5 evicts expert 3 (u .5) rather than 0 (u .75)
    assert d.slot_expert == [0, 5]


def test_cost_aware_prefetch_hand_traced():
    c = SlotCacheSim(num_experts=8, num_slots=3, policy=POLICY_COST, decay=0.5)
    c.step({5, 1})
    c.step({1, 2, 7})                                # slots [1, 7, 2]; u1 .75, u2 = u7 .5, u5 .25
    # predicted {2, 5, 6}: 2 resident (kept); wanted 5 (u .25) before 6 (u 0); one copy into the
    # lowest-usage unpredicted slot: slot 1 (expert 7, .5) before slot 0 (expert 1, .75)
    assert c.prefetch({2, 5, 6}, 1) == [(5, 1)]
    assert c.slot_expert == [1, 5, 2]


def test_policies_cover_every_needed_expert_once_per_step():
    rng = np.random.default_rng(11)
    for policy in (0, POLICY_COST):
        c = SlotCacheSim(num_experts=64, num_slots=16, policy=policy, decay=0.9)
        for _ in range(150):
            need = set(rng.choice(64, size=rng.integers(1, 40), replace=False).tolist())
            rounds = c.step(need)
            got = [e for sub, _, _ in rounds for e in sub]
            assert sorted(got) == sorted(need)               # each needed expert in exactly one round
            copies = [e for _, _, cp in rounds for e, _ in cp]
            assert len(copies) == len(set(copies))           # never copied twice in a step
            assert all(len(sub) <= 16 for sub, _, _ in rounds)


def test_precision_aware_hand_traced():
    # blobs of 100 bytes whose first 40 are the two-bit part; LRU
    c = SlotCacheSim(num_experts=8, num_slots=3, prefix_bytes=40, blob_bytes=100)
    # step 1 {1, 5}, four bits for 5 only: 1 copies its prefix, 5 its whole blob
    r = c.step({1, 5}, full={5})
    assert r == [([1, 5], [], [(1, 0, "hi"), (5, 1, "all")])]
    assert c.slot_full == [False, True, False] and c.copy_bytes(r[0][2]) == 140
    # step 2 {1, 2}, four bits for 1: 1 stays in slot 0 and gets its low planes; 2 (two
    # bits) takes the empty slot 2
    r = c.step({1, 2}, full={1})
    assert r == [([1, 2], [1], [(1, 0, "lo"), (2, 2, "hi")])]
    assert c.slot_full == [True, True, False] and c.copy_bytes(r[0][2]) == 100
    # step 3 {2, 6, 7}, four bits for 6: 2 is a plain hit (two bits needed, two bits held);
    # 6 and 7 evict slots 1 (expert 5, older) and 0 (expert 1)
    r = c.step({2, 6, 7}, full={6})
    assert r == [([2, 6, 7], [2], [(6, 1, "all"), (7, 0, "hi")])]
    assert c.slot_expert == [7, 6, 2] and c.slot_full == [False, True, False]
    # a whole-blob request (full=None) completes a two-bit resident
    r = c.step({7})
    assert r == [([7], [7], [(7, 0, "lo")])] and c.slot_full[0]


def test_precision_aware_cost_weighs_reload_bytes():
    c = SlotCacheSim(num_experts=8, num_slots=2, policy=POLICY_COST, decay=0.5, prefix_bytes=40, blob_bytes=100)
    assert c.step({0, 1}, full={0}) == [([0, 1], [], [(0, 0, "all"), (1, 1, "hi")])]
    # step 2 {2} at four bits: u0 = u1 = .25; reload costs .25 * 100 (slot 0, whole blob) and
    # .25 * 40 (slot 1, prefix): the cheaper reload goes (LRU would evict slot 0)
    assert c.step({2}, full={2}) == [([2], [], [(2, 1, "all")])]
    assert c.slot_expert == [0, 2] and c.slot_full == [True, True]
