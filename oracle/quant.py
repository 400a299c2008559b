"""Group-128 symmetric int4 quantisation and the packed layout (oracle; test infrastructure only).

ExactMoE (page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16
Inference", Abstract) quantises only the routed experts' weights, to four bits,
symmetrically, in groups of 128.  The page fixes neither the scale rule, the
rounding, the code range nor the storage layout; the readings taken here:

* groups run along K, the input-channel axis of a weight W[N, K] (y = W x);
* scale s = bf16_rne(amax / 7) where amax is the largest |w| of the group,
  rounded to the nearest bf16 with ties to even (the scale is stored as bf16);
* q = clamp(round_half_even(w / s), -8, 7), and q = 0 for the whole group when
  s == 0.  With s >= amax/7 * (1 - 2^-8) the quotient never exceeds 7.03, so
  the codes in practice span -7..7 (symmetric); -8 stays decodable;
* the dequantised weight is exactly q * s.

Exactness of the definitions as computed here: w and s are bf16 values, so
w/s = (m_w / m_s) * 2^j with 8-bit integers m_w, m_s; if it is not exactly a
half-integer it lies at least 2^-12 (relative) away from one, far beyond the
2^-53 error of the float64 quotient, so rint(w/s) in float64 is the exact
round-half-even of the real quotient.  Likewise amax/7 = (m/7) * 2^j is either
a bf16 value already (7 | m) or has a period-3 binary expansion that stays at
least 2^-12 (relative) away from every bf16 rounding midpoint, so rounding the
float64 quotient gives the exact nearest bf16.

Packed layout v1 (this implementation's own format; the pages name a
kernel-native layout for other hardware, which is not followed).  A weight
W[N, K] with N % 16 == 0 and K % 128 == 0 is cut into tiles of 16 rows x 128
columns (one quantisation group per row):

* tile (nb, kb) occupies 1024 bytes at byte offset (nb * K/128 + kb) * 1024;
* inside a tile, lane L = 0..63 owns the 16 bytes at offset 16 * L; with
  r = L % 16 and c = L // 16 they hold row nb*16 + r, columns
  kb*128 + 32*i + 8*c + m for i = 0..3 (the little-endian 32-bit word i) and
  m = 0..7;
* inside word i the 4-bit code (q + 8) of element m sits in the bit field that
  starts at bit (3 + 4*(m // 2) + 16*(m % 2)) mod 32 and runs upward, wrapping
  from bit 31 to bit 0; equivalently, word = rotl32(u, 3) where
  u = sum_m code_m << (4*(m//2) + 16*(m%2));
* scales are a separate bf16 array [N/16][K/128][16]: scale of (row, group)
  at ((row // 16) * K/128 + group) * 16 + row % 16;
* with gate/up interleaving (W13 = [gate; up] with 2I rows) packed row tile 2j
  holds gate rows 16j..16j+15 and packed row tile 2j+1 holds up rows
  16j..16j+15 (source rows I+16j..I+16j+15).
"""
import numpy as np

from . import bf16

GROUP = 128
TILE_ROWS = 16
TILE_BYTES = 1024


def scale_for(amax):
    """Group scale: amax / 7 rounded to the nearest bf16 (ties to even)."""
    return bf16.round_to_bf16(np.asarray(amax, dtype=np.float64) / 7.0)


def codes_for_scale(w, s):
    """q = clamp(round_half_even(w / s), -8, 7); q = 0 where s == 0 (s broadcasts over w)."""
    w = np.asarray(w, dtype=np.float64)
    s = np.broadcast_to(np.asarray(s, dtype=np.float64), w.shape)
    q = np.clip(np.rint(w / np.where(s > 0, s, 1.0)), -8, 7)
    return np.where(s > 0, q, 0.0).astype(np.int8)


def quantize_values(w):
    """Quantise float64 values [..., N, K] -> (q int8 [..., N, K], s float64 [..., N, K/128])."""
    w = np.asarray(w, dtype=np.float64)
    *lead, N, K = w.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = w.reshape(*lead, N, K // GROUP, GROUP)
    s = scale_for(np.max(np.abs(g), axis=-1))
    q = codes_for_scale(g, s[..., None])
    return q.reshape(*lead, N, K), s


def quantize_g128(w_bits):
    """Quantise bf16 weights [..., N, K] (bit patterns) -> (q int8, s float64 [..., N, K/128])."""
    return quantize_values(bf16.to_f64(w_bits))


def dequantize(q, s):
    """W~[..., n, k] = q[..., n, k] * s[..., n, k // 128] (exact in float64)."""
    q = np.asarray(q, dtype=np.float64)
    *lead, N, K = q.shape
    return (q.reshape(*lead, N, K // GROUP, GROUP) * np.asarray(s)[..., None]).reshape(*lead, N, K)


def gateup_row_order(N):
    """Source row of each packed row when gate/up rows are interleaved (N = 2I)."""
    I = N // 2
    rows = np.arange(N)
    t, r = rows // TILE_ROWS, rows % TILE_ROWS
    return np.where(t % 2 == 0, (t // 2) * TILE_ROWS + r, I + (t // 2) * TILE_ROWS + r)


_FIELD = np.array([4 * (m // 2) + 16 * (m % 2) for m in range(8)], dtype=np.uint32)


def _rotl32(u, n):
    u = u.astype(np.uint32)
    return ((u << np.uint32(n)) | (u >> np.uint32(32 - n))).astype(np.uint32)


def _rotr32(u, n):
    return _rotl32(u, 32 - n)


def pack_v1(q, s, gateup_interleave=False):
    """Pack one matrix: q int [N, K], s [N, K/128] -> (codes uint8 [N*K/2], scales uint16 [N*K/128])."""
    q = np.asarray(q)
    N, K = q.shape
    if N % TILE_ROWS or K % GROUP:
        raise ValueError("N must be a multiple of 16 and K a multiple of 128")
    if gateup_interleave:
        if N % (2 * TILE_ROWS):
            raise ValueError("gate/up interleave needs N a multiple of 32")
        order = gateup_row_order(N)
        q, s = q[order], np.asarray(s)[order]
    code = (q.astype(np.int64) + 8).astype(np.uint32)
    # K index = kb*128 + 32*i + 8*c + m ; row = nb*16 + r ; lane = 16*c + r
    c6 = code.reshape(N // 16, 16, K // 128, 4, 4, 8)          # nb, r, kb, i, c, m
    c6 = c6.transpose(0, 2, 4, 1, 3, 5)                        # nb, kb, c, r, i, m
    c6 = c6.reshape(N // 16, K // 128, 64, 4, 8)               # nb, kb, lane, word, m
    u = np.bitwise_or.reduce(c6 << _FIELD, axis=-1).astype(np.uint32)
    words = _rotl32(u, 3)
    codes = words.astype("<u4").reshape(-1).view(np.uint8).copy()
    sc = np.asarray(s, dtype=np.float64).reshape(N // 16, 16, K // 128).transpose(0, 2, 1)
    scales = bf16.to_bits(sc.reshape(-1))
    return codes, scales


def unpack_v1(codes, scales, N, K, gateup_interleave=False):
    """Inverse of pack_v1: (codes, scales) -> (q int8 [N, K], s float64 [N, K/128])."""
    words = np.asarray(codes, dtype=np.uint8).view("<u4").astype(np.uint32)
    u = _rotr32(words.reshape(N // 16, K // 128, 64, 4), 3)
    c6 = (u[..., None] >> _FIELD) & np.uint32(0xF)              # nb, kb, lane, word, m
    c6 = c6.reshape(N // 16, K // 128, 4, 16, 4, 8)            # nb, kb, c, r, i, m
    c6 = c6.transpose(0, 3, 1, 4, 2, 5).reshape(N, K)          # nb, r, kb, i, c, m
    q = (c6.astype(np.int64) - 8).astype(np.int8)
    s = bf16.to_f64(np.asarray(scales, dtype=np.uint16)).reshape(N // 16, K // 128, 16)
    s = s.transpose(0, 2, 1).reshape(N, K // 128)
    if gateup_interleave:
        inv = np.argsort(gateup_row_order(N))
        q, s = q[inv], s[inv]
    return q, s


def blob_layout(d, I, align=256):
    """Byte offsets of one expert's packed sections: w13 codes, w13 scales, w2 codes, w2 scales.

    w13 is [2I, d] (gate/up interleaved), w2 is [d, I].  Each section starts on
    an ``align``-byte boundary; returns (offsets tuple, blob bytes).
    """
    def up(v):
        return (v + align - 1) // align * align
    sizes = (2 * I * d // 2, 2 * I * (d // GROUP) * 2, d * I // 2, d * (I // GROUP) * 2)
    offs, o = [], 0
    for sz in sizes:
        offs.append(o)
        o = up(o + sz)
    return tuple(offs), o


def pack_expert_blob(w13_bits, w2_bits):
    """Quantise and pack one expert (w13 [2I, d], w2 [d, I] bf16 bits) into one blob (uint8)."""
    twoI, d = w13_bits.shape
    I = twoI // 2
    offs, total = blob_layout(d, I)
    blob = np.zeros(total, dtype=np.uint8)
    q13, s13 = quantize_g128(w13_bits)
    c13, sc13 = pack_v1(q13, s13, gateup_interleave=True)
    q2, s2 = quantize_g128(w2_bits)
    c2, sc2 = pack_v1(q2, s2)
    for off, arr in zip(offs, (c13, sc13.view(np.uint8), c2, sc2.view(np.uint8))):
        blob[off:off + arr.size] = arr
    return blob
