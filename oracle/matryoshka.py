"""Nested two/four-bit expert weights, floor-and-compensation dequantisation and a
per-expert precision chosen from the routing weights (oracle; test infrastructure only).

The lower-precision variant follows page "MatMoE: Dynamic Mixed-Precision
Quantization for Efficient MoE Inference" (arXiv abstract, 2611.01704): experts
run at several precisions from one nested (Matryoshka) quantised representation,
the lower precision is the floor of the higher one plus a compensation term, so
it reads only part of the stored bits, and each expert's precision follows its
routing scores.  The abstract fixes none of the details; the readings taken:

* the four-bit representation is this repository's group-128 symmetric int4
  (oracle.quant): code c = q + 8 in 0..15 and a bf16 scale s per group;
* the nested two-bit representation is the high two bits h = c >> 2 (the floor
  of c / 4); the low two bits l = c & 3 complete it, c = 4h + l;
* floor-and-compensation dequantisation of the two-bit weight: the dropped low
  bits are replaced by their mean over the four values, 1.5, so
  w2 = (4h + 1.5 - 8) * s = (4h - 6.5) * s; the four-bit weight is (4h + l - 8) * s
  = q * s, exactly the W4A16 weight;
* precision per expert per step: an expert runs at four bits when the largest
  routing weight among the (token, slot) pairs routed to it reaches the threshold
  tau, else at two bits (tau = 0: every expert four-bit; tau > 1: every expert
  two-bit).

Storage (this repository's layout m1): the h and l bits are kept in two separate
planes, so a two-bit expert reads half of the code bytes.  A weight W[N, K] with
N % 16 == 0 and K % 256 == 0 is cut into plane tiles of 16 rows x 256 columns (two
quantisation groups), tile (nb, kb) at byte offset (nb * K/256 + kb) * 1024 of its
plane, rows in the gate/up interleaved order of layout v1 and the same bf16 scale
array; lane L = 0..63 owns the 16 bytes at offset 16 * L: little-endian 32-bit
words j = 0..3, word j holding K steps i = 2j and 2j + 1 of row L % 16, columns
32 i + 8 (L // 16) + m (m = 0..7) of the tile (steps 0-3 are the first group,
4-7 the second).  Inside word j, element (i, m) with t = i - 2j has pair index
p = 4t + m // 2 and its 2-bit field starts at bit (5 + 2p + 16 (m % 2)) mod 32,
running upward and wrapping from bit 31 to bit 0; equivalently
word = rotl32(u, 5), u = sum v << (2p + 16 (m % 2)).
"""
import numpy as np

from . import bf16, quant, route as route_mod, align as align_mod
from .ffn import expert_ffn, combine

COMPENSATION = 1.5  # mean of the dropped low two bits (0, 1, 2, 3)


def split_planes(q):
    """Four-bit codes q (int, -8..7) -> (h, l) with q + 8 = 4h + l, both 0..3."""
    c = np.asarray(q, dtype=np.int64) + 8
    return (c >> 2).astype(np.uint8), (c & 3).astype(np.uint8)


def dequant_full(q, s):
    """Four-bit weight (4h + l - 8) * s, equal to q * s."""
    return quant.dequantize(q, s)


def dequant_floor(q, s):
    """Two-bit floor-and-compensation weight (4h + 1.5 - 8) * s."""
    h, _ = split_planes(q)
    v = 4.0 * h.astype(np.float64) + COMPENSATION - 8.0
    return quant.dequantize(v, s)


# field start of element (t, m) inside a plane word, before the rotation by 5
_PFIELD = np.array([[2 * (4 * t + m // 2) + 16 * (m % 2) for m in range(8)] for t in range(2)], dtype=np.uint32)


PLANE_K = 256          # columns per plane tile (two groups)
PLANE_TILE_BYTES = 1024


def _plane_words(v):
    """One plane (values 0..3, [N, K] in packed row order) -> uint32 words [N/16, K/256, 64, 4]."""
    N, K = v.shape
    # K index = kb*256 + 32*(2j + t) + 8*c + m ; row = nb*16 + r ; lane = 16*c + r
    c7 = v.astype(np.uint32).reshape(N // 16, 16, K // PLANE_K, 4, 2, 4, 8)   # nb, r, kb, j, t, c, m
    c7 = c7.transpose(0, 2, 5, 1, 3, 4, 6)                                    # nb, kb, c, r, j, t, m
    c7 = c7.reshape(N // 16, K // PLANE_K, 64, 4, 2, 8)                       # nb, kb, lane, j, t, m
    u = np.bitwise_or.reduce(np.bitwise_or.reduce(c7 << _PFIELD, axis=-1), axis=-1).astype(np.uint32)
    return quant._rotl32(u, 5)


def pack_m1(q, s, gateup_interleave=False):
    """One matrix: q [N, K], s [N, K/128] -> (hi uint8 [N*K/4], lo uint8 [N*K/4], scales uint16)."""
    q = np.asarray(q)
    N, K = q.shape
    if N % 16 or K % PLANE_K:
        raise ValueError("N must be a multiple of 16 and K a multiple of 256")
    if gateup_interleave:
        order = quant.gateup_row_order(N)
        q, s = q[order], np.asarray(s)[order]
    h, l = split_planes(q)
    hi = _plane_words(h).astype("<u4").reshape(-1).view(np.uint8).copy()
    lo = _plane_words(l).astype("<u4").reshape(-1).view(np.uint8).copy()
    sc = np.asarray(s, dtype=np.float64).reshape(N // 16, 16, K // 128).transpose(0, 2, 1)
    return hi, lo, bf16.to_bits(sc.reshape(-1))


def unpack_plane(plane, N, K, gateup_interleave=False):
    """Inverse of one plane of pack_m1: bytes -> values 0..3 [N, K] in source row order."""
    words = np.asarray(plane, dtype=np.uint8).view("<u4").astype(np.uint32).reshape(N // 16, K // PLANE_K, 64, 4)
    u = quant._rotr32(words, 5)
    v = (u[..., None, None] >> _PFIELD) & np.uint32(3)                   # nb, kb, lane, j, t, m
    v = v.reshape(N // 16, K // PLANE_K, 4, 16, 4, 2, 8)                 # nb, kb, c, r, j, t, m
    v = v.transpose(0, 3, 1, 4, 5, 2, 6).reshape(N, K)                   # nb, r, kb, j, t, c, m
    if gateup_interleave:
        v = v[np.argsort(quant.gateup_row_order(N))]
    return v.astype(np.uint8)


def blob_layout_m1(d, I, align=256):
    """Byte offsets of one expert's sections in layout m1, returned in the order
    (w13 hi, w13 lo, w13 scales, w2 hi, w2 lo, w2 scales), and the blob size.  The
    sections are placed as w13 hi, w13 scales, w2 hi, w2 scales, w13 lo, w2 lo
    (each on an ``align``-byte boundary): everything a two-bit expert reads is one
    prefix of the blob, and the low planes follow it (page "MoE-APEX: An
    Efficient MoE Inference System with Adaptive Precision Expert Offloading",
    "This paper's idea": a less critical expert that misses the cache is loaded at
    low precision, so only that prefix moves)."""
    def up(v):
        return (v + align - 1) // align * align
    size = {"hi13": 2 * I * d // 4, "lo13": 2 * I * d // 4, "sc13": 2 * I * (d // 128) * 2,
            "hi2": d * I // 4, "lo2": d * I // 4, "sc2": d * (I // 128) * 2}
    at, o = {}, 0
    for key in ("hi13", "sc13", "hi2", "sc2", "lo13", "lo2"):
        at[key] = o
        o = up(o + size[key])
    return tuple(at[key] for key in ("hi13", "lo13", "sc13", "hi2", "lo2", "sc2")), o


def two_bit_prefix_m1(d, I, align=256):
    """Bytes of the two-bit part at the start of a layout-m1 blob (high planes and
    scales): where the low planes begin."""
    offs, _ = blob_layout_m1(d, I, align)
    return offs[1]


def pack_expert_blob_m1(w13_bits, w2_bits):
    """Quantise one expert (w13 [2I, d], w2 [d, I] bf16 bits) into a layout-m1 blob (uint8)."""
    twoI, d = w13_bits.shape
    I = twoI // 2
    offs, total = blob_layout_m1(d, I)
    blob = np.zeros(total, dtype=np.uint8)
    q13, s13 = quant.quantize_g128(w13_bits)
    q2, s2 = quant.quantize_g128(w2_bits)
    parts = pack_m1(q13, s13, gateup_interleave=True) + pack_m1(q2, s2)
    for off, arr in zip(offs, parts):
        arr = arr.view(np.uint8) if arr.dtype != np.uint8 else arr
        blob[off:off + arr.size] = arr
    return blob


class MatBank:
    """Both precisions of every expert, from bf16 master weights on first use."""

    def __init__(self, w13_bits, w2_bits):
        self._w13, self._w2 = w13_bits, w2_bits
        self._cache = {}

    def get(self, e, full=True):
        key = (e, bool(full))
        if key not in self._cache:
            deq = dequant_full if full else dequant_floor
            q13, s13 = quant.quantize_g128(self._w13(e))
            q2, s2 = quant.quantize_g128(self._w2(e))
            self._cache[key] = (deq(q13, s13), deq(q2, s2))
        return self._cache[key]


def expert_precision(ids, weights, tau):
    """{expert: True for four bits, False for two} for the experts of a step."""
    flat_ids, flat_w = np.asarray(ids).reshape(-1), np.asarray(weights).reshape(-1)
    return {int(e): bool(np.max(flat_w[flat_ids == e]) >= tau) for e in np.unique(flat_ids)}


def moe_layer(x_bits, wr_bits, bank, k, tau, renormalize=True, tokens=None):
    """Whole layer with per-expert precision: route, align, per-pair SwiGLU FFN on the
    expert's weights at its precision, combine.  ``out`` [len(tokens), d] float64."""
    x_bits = np.asarray(x_bits)
    T = x_bits.shape[0]
    E = np.asarray(wr_bits).shape[0]
    logits, ids, w = route_mod.route(x_bits, wr_bits, k, renormalize)
    al = align_mod.align(ids, E)
    prec = expert_precision(ids, w, tau)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    pairs = (tokens[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    x = bf16.to_f64(x_bits)
    flat = ids.reshape(-1)
    y = {}
    for e in np.unique(flat[pairs]):
        sel = pairs[flat[pairs] == e]
        w13, w2 = bank.get(int(e), prec[int(e)])
        for p, row in zip(sel, expert_ffn(w13, w2, x[sel // k])):
            y[int(p)] = row
    return {"ids": ids, "weights": w, "align": al, "precision": prec, "tokens": tokens,
            "out": combine(w, y, tokens, k)}
