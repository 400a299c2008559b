"""Per-pair SwiGLU expert FFN, routing-weighted combine, whole layer (oracle; test infrastructure only).

ExactMoE (page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16
Inference", Abstract) executes every selected expert (none pruned, substituted
or moved to the CPU) on its four-bit group-128 weights with BF16 activations.
The page does not name the expert activation or the combine; the readings
taken:

* expert e is a SwiGLU MLP on the dequantised weights:
  g = Wg_e x, u = Wu_e x, h = silu(g) * u with silu(z) = z / (1 + exp(-z)),
  y = Wd_e h; W13_e = [Wg_e; Wu_e] is [2I, d] (gate rows first), Wd_e is [d, I];
* out[t] = sum_j w[t, j] * y[(t, j)], summed over j in slot order;
* everything is float64; nothing is rounded to bf16 on the way (the output is
  compared before any final rounding).
"""
import numpy as np

from . import bf16, quant, route as route_mod, align as align_mod


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


class DequantBank:
    """Dequantised expert weights, produced from bf16 master weights on first use.

    ``w13_bits(e)`` and ``w2_bits(e)`` return the bf16 bit patterns of expert e
    (uint16 [2I, d] and [d, I]).  Each expert is quantised with quant.quantize_g128
    and dequantised exactly; results are cached.
    """

    def __init__(self, w13_bits, w2_bits):
        self._w13, self._w2 = w13_bits, w2_bits
        self._cache = {}

    def get(self, e):
        if e not in self._cache:
            q13, s13 = quant.quantize_g128(self._w13(e))
            q2, s2 = quant.quantize_g128(self._w2(e))
            self._cache[e] = (quant.dequantize(q13, s13), quant.dequantize(q2, s2))
        return self._cache[e]


class Bf16Bank:
    """Unquantised experts: the bf16 master weights themselves, as float64 (the
    BF16 side of the page's four-bit versus BF16 comparison).  Same interface as
    DequantBank."""

    def __init__(self, w13_bits, w2_bits):
        self._w13, self._w2 = w13_bits, w2_bits
        self._cache = {}

    def get(self, e):
        if e not in self._cache:
            self._cache[e] = (bf16.to_f64(self._w13(e)), bf16.to_f64(self._w2(e)))
        return self._cache[e]


def expert_ffn(w13, w2, X):
    """SwiGLU expert on rows of X [n, d] with dequantised w13 [2I, d], w2 [d, I] -> [n, d]."""
    I = w13.shape[0] // 2
    X = np.asarray(X, dtype=np.float64)
    g = X @ w13[:I].T
    u = X @ w13[I:].T
    h = silu(g) * u
    return h @ w2.T


def pair_outputs(x_bits, ids, bank, pairs=None):
    """y[p] for pairs p (all pairs when None): expert ids[p]'s FFN applied to token p // k."""
    x = bf16.to_f64(x_bits)
    T, k = ids.shape
    flat = ids.reshape(-1)
    pairs = np.arange(T * k) if pairs is None else np.asarray(pairs)
    y = {}
    for e in np.unique(flat[pairs]):
        sel = pairs[flat[pairs] == e]
        w13, w2 = bank.get(int(e))
        ye = expert_ffn(w13, w2, x[sel // k])
        for p, row in zip(sel, ye):
            y[int(p)] = row
    return y


def combine(weights, y, tokens, k):
    """out[t] = sum_j weights[t, j] * y[t*k + j] in j order, for the listed tokens."""
    out = []
    for t in tokens:
        acc = np.zeros_like(y[int(t) * k])
        for j in range(k):
            acc = acc + weights[t, j] * y[int(t) * k + j]
        out.append(acc)
    return np.stack(out) if out else np.zeros((0,))


def moe_layer(x_bits, wr_bits, bank, k, renormalize=True, tokens=None):
    """Whole layer: route, align, per-pair FFN, combine.

    Returns a dict with logits (float32), ids, weights, the alignment, and
    ``out`` [len(tokens), d] float64 for the requested tokens (all when None).
    """
    x_bits = np.asarray(x_bits)
    T = x_bits.shape[0]
    E = np.asarray(wr_bits).shape[0]
    logits, ids, w = route_mod.route(x_bits, wr_bits, k, renormalize)
    al = align_mod.align(ids, E)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    pairs = (tokens[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    y = pair_outputs(x_bits, ids, bank, pairs)
    out = combine(w, y, tokens, k)
    return {"logits": logits, "ids": ids, "weights": w, "align": al, "y": y,
            "tokens": tokens, "out": out}
