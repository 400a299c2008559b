"""Pins for the oracle's router, top-k, routing weights and permutation (CPU only).

Independent references: Python's sorted() over full orderings (brute force),
scipy's softmax, numpy's stable argsort, exact integer arithmetic, and the
closed-form special cases k = 1, k = E and constant logits.
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import align, bf16, route


def rand_bits(shape, std, seed):
    rng = np.random.default_rng(seed)
    return bf16.to_bits(bf16.round_to_bf16(rng.normal(0, std, size=shape)))


def test_logits_exact_on_integers():
    rng = np.random.default_rng(0)
    x = rng.integers(-4, 5, size=(5, 256)).astype(np.float64)
    w = rng.integers(-3, 4, size=(6, 256)).astype(np.float64)
    l = route.logits_f64(bf16.to_bits(x), bf16.to_bits(w))
    ref = np.array([[sum(int(a) * int(b) for a, b in zip(xr, wr)) for wr in w] for xr in x])
    assert np.array_equal(l, ref.astype(np.float64))


def test_topk_brute_force_full_sort():
    rng = np.random.default_rng(1)
    for E, k in ((8, 2), (8, 8), (5, 1), (64, 8)):
        # few distinct values -> many exact ties
        l = rng.integers(-3, 3, size=(50, E)).astype(np.float32)
        ids = route.topk_select(l, k)
        for t in range(50):
            ref = sorted(range(E), key=lambda e: (-float(l[t, e]), e))[:k]
            assert list(ids[t]) == ref


def test_weights_special_cases():
    rng = np.random.default_rng(2)
    l = rng.normal(0, 1, size=(20, 8)).astype(np.float32)
    ids1 = route.topk_select(l, 1)
    assert np.all(route.topk_weights(l, ids1) == 1.0)
    idsE = route.topk_select(l, 8)
    w = route.topk_weights(l, idsE)
    ref = np.take_along_axis(softmax(l.astype(np.float64), axis=1), idsE.astype(np.int64), 1)
    assert np.allclose(w, ref, rtol=1e-14, atol=0)
    lc = np.zeros((4, 8), dtype=np.float32)
    idc = route.topk_select(lc, 3)
    assert np.array_equal(idc, np.tile(np.arange(3), (4, 1)))
    assert np.allclose(route.topk_weights(lc, idc), 1.0 / 3, rtol=0, atol=1e-15)


def test_weights_invariants_and_renormalize_off():
    xb, wb = rand_bits((64, 256), 1.0, 3), rand_bits((16, 256), 0.02, 4)
    l, ids, w = route.route(xb, wb, 4)
    assert np.all(np.abs(w.sum(1) - 1) <= 1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == 4 for r in ids)
    w0 = route.topk_weights(l, ids, renormalize=False)
    full = softmax(l.astype(np.float64), axis=1)
    assert np.allclose(w0, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-14, atol=0)


def test_logits_rounded_once_to_f32():
    xb, wb = rand_bits((8, 512), 1.0, 5), rand_bits((16, 512), 0.02, 6)
    l64 = route.logits_f64(xb, wb)
    l32 = route.logits_f32(xb, wb)
    assert l32.dtype == np.float32 and np.array_equal(l32, l64.astype(np.float32))


# ---------------------------------------------------------------- align

def check_align(ids, E, bm=0):
    a = align.align(ids, E, bm)
    flat = np.asarray(ids).reshape(-1)
    ref = np.argsort(flat, kind="stable")
    assert np.array_equal(a["sorted_pairs"], ref)
    assert np.array_equal(a["counts"], np.bincount(flat, minlength=E))
    assert a["offsets"][0] == 0 and a["offsets"][-1] == flat.size
    assert np.array_equal(np.diff(a["offsets"]), a["counts"])
    assert np.array_equal(a["pair_pos"][a["sorted_pairs"]], np.arange(flat.size))
    assert np.array_equal(a["active"], np.unique(flat))
    if bm:
        t = -(-a["counts"] // bm)
        assert np.array_equal(np.diff(a["tile_offsets"]), t)
    return a


def test_align_random_and_edges():
    rng = np.random.default_rng(7)
    for T, E, k in ((16, 8, 2), (1, 64, 8), (333, 64, 8), (50, 1024, 4)):
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        check_align(ids, E, bm=64)
    check_align(np.zeros((0, 4), dtype=np.int32), 8, bm=16)              # empty
    check_align(np.full((37, 1), 5, dtype=np.int32), 8, bm=16)           # all on one expert
    a = check_align(np.array([[3, 1], [1, 3], [0, 3]]), 4)
    assert list(a["sorted_pairs"]) == [4, 1, 2, 0, 3, 5]                 # hand-sorted
    assert list(a["offsets"]) == [0, 1, 3, 3, 6]
    assert list(a["active"]) == [0, 1, 3]
