"""GPU parity at full size: every output token of every workload against the oracle.

Each workload's expert bank is drawn once per module (on the GPU), packed by the
library and dequantised by the oracle; every entry point and every kernel variant
that can run the layer is then compared with the oracle on all tokens of the step:

* route + align + grouped FFN (automatic variant choice), and the other variant
  forced (the MFMA prefill kernels at decode sizes, the decode kernels at
  prefill sizes);
* moe_decode_layer (routing inside the gate/up launch, down + combine fused);
* the slot-table path (an expert -> slot table keeps the two-pass decode
  kernels and the separate combine: what slot-cache rounds and per-expert calls
  run), in one call, in two rounds over disjoint halves, and one call per expert;
* the decode gate/up variant for d > 4096 (activations read per group).

Bars: routing ids bit-exact; routing weights within 1e-6; layer outputs within
max|gpu - ref| / max|ref| <= 1e-2, and the same for every token on its own
(bf16 outputs against the float64 oracle on identical dequantised weights).
All tokens are compared, so every (expert, 128-token tile) of the prefill kernels
has its first and last rows checked.
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe
from oracle import ffn as offn

from gpu_helpers import bits, check_layer_out, oracle_bank, say, warm_bank

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    moe.lib()
    yield
    torch.cuda.synchronize()


def make_layer(wl, layer):
    s = wl.shape
    say(f"drawing {wl.name} layer {layer}: d={s.d} E={s.E} k={s.k} I={s.I}")
    w13, w2 = synth.expert_weights(wl, layer, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    ob = warm_bank(oracle_bank(w13, w2), range(s.E))
    torch.cuda.synchronize()
    del w13, w2
    torch.cuda.empty_cache()
    return SimpleNamespace(wl=wl, s=s, layer=layer, bank=bank, ob=ob,
                           wr=synth.router_weight(wl, layer))


@pytest.fixture(scope="module")
def olmoe_decode():
    return make_layer(synth.OLMOE_DECODE, 3)


@pytest.fixture(scope="module")
def olmoe_prefill():
    return make_layer(synth.OLMOE_PREFILL, 1)


@pytest.fixture(scope="module")
def large():
    return make_layer(synth.LARGE, 1)


def oracle_step(L, x, renormalize=True):
    return offn.moe_layer(bits(x), bits(L.wr), L.ob, L.s.k, renormalize=renormalize)


def route_align(L, xd, wrd):
    r = moe.moe_route(xd, wrd, L.s.k)
    a = moe.moe_align(r.ids, L.s.E)
    return r, a


def check_route(r, ref):
    assert np.array_equal(r.ids.cpu().numpy(), ref["ids"])
    assert np.max(np.abs(r.weights.cpu().numpy() - ref["weights"]), initial=0.0) <= 1e-6


def ffn(L, xd, r, a, mode=moe.MODE_AUTO, table=None):
    out = moe.moe_w4a16_grouped_ffn(xd, r, a, L.bank, L.s.I, mode=mode, slot_of_expert=table)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def slot_rounds(L, xd, r, a, mode):
    """Two rounds over disjoint halves of the experts (slot tables with -1 = not in
    this round), the second accumulating and combining: a slot-cache step's calls."""
    s = L.s
    ws = moe.alloc_workspace(xd.shape[0], s.d, s.I, s.E, s.k, mode)
    out = torch.empty((xd.shape[0], s.d), dtype=torch.bfloat16, device=DEV)
    even = torch.tensor([e if e % 2 == 0 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    odd = torch.tensor([e if e % 2 == 1 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    moe.moe_w4a16_grouped_ffn_into(xd, r, a, L.bank, s.I, out, ws, mode, False, even)
    moe.moe_w4a16_grouped_ffn_into(xd, r, a, L.bank, s.I, out, ws, mode, True, odd)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def per_expert_calls(L, xd, r, a):
    """The sequential ablation variant: one call per active expert, combine on the last."""
    s = L.s
    ws = moe.alloc_workspace(xd.shape[0], s.d, s.I, s.E, s.k)
    out = torch.empty((xd.shape[0], s.d), dtype=torch.bfloat16, device=DEV)
    experts = [w[0] for w in moe.active_experts(a)]
    for i, e in enumerate(experts):
        only = torch.full((s.E,), -1, dtype=torch.int32, device=DEV)
        only[e] = e
        moe.moe_w4a16_grouped_ffn_into(xd, r, a, L.bank, s.I, out, ws, combine=(i == len(experts) - 1),
                                       slot_of_expert=only)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


# ------------------------------------------------------------------ OLMoE decode

@pytest.mark.parametrize("T", [1, 4, 16])
def test_olmoe_decode_every_token(olmoe_decode, T):
    L = olmoe_decode
    s = L.s
    say(f"OLMoE decode T={T}: every token, every entry point")
    x = synth.activations(L.wl, T, L.layer)
    ref = oracle_step(L, x)
    xd, wrd = x.to(DEV), L.wr.to(DEV)
    r, a = route_align(L, xd, wrd)
    check_route(r, ref)
    check_layer_out("grouped ffn (decode, down + combine fused)", ffn(L, xd, r, a), ref["out"])
    out, route = moe.moe_decode_layer(xd, wrd, L.bank, s.I, s.k)
    torch.cuda.synchronize()
    check_route(route, ref)
    check_layer_out("moe_decode_layer", out.float().cpu().numpy(), ref["out"])
    ident = torch.arange(s.E, dtype=torch.int32, device=DEV)
    check_layer_out("slot-table decode path (two-pass + combine)",
                    ffn(L, xd, r, a, moe.MODE_DECODE, ident), ref["out"])
    check_layer_out("slot rounds over two halves", slot_rounds(L, xd, r, a, moe.MODE_DECODE), ref["out"])
    check_layer_out("one call per expert", per_expert_calls(L, xd, r, a), ref["out"])
    check_layer_out("prefill kernels forced", ffn(L, xd, r, a, moe.MODE_PREFILL), ref["out"])


def test_olmoe_decode_layer_counters_and_no_renormalize(olmoe_decode):
    L = olmoe_decode
    s = L.s
    say("OLMoE decode T=4 moe_decode_layer without renormalisation, three calls on one counter block")
    x = synth.activations(L.wl, 4, L.layer, step=1)
    ref = oracle_step(L, x, renormalize=False)
    xd, wrd = x.to(DEV), L.wr.to(DEV)
    route = moe.alloc_route(4, s.E, s.k, DEV)
    out = torch.empty((4, s.d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(moe.decode_layer_workspace_bytes(4, s.d, s.I, s.E, s.k), dtype=torch.uint8, device=DEV)
    ctr = moe.alloc_layer_counters(DEV)
    for c in range(3):
        out.fill_(float("nan"))
        moe.moe_decode_layer_into(xd, wrd, L.bank, s.I, s.k, route, out, ws, ctr, renormalize=False)
        torch.cuda.synchronize()
        assert int(ctr.abs().sum()) == 0, f"counters after call {c}"
        check_route(route, ref)
        check_layer_out(f"call {c}", out.float().cpu().numpy(), ref["out"])


# ------------------------------------------------------------------ OLMoE prefill

@pytest.mark.parametrize("T", [512, 4096])
def test_olmoe_prefill_every_token(olmoe_prefill, T):
    L = olmoe_prefill
    s = L.s
    say(f"OLMoE prefill T={T}: every token")
    x = synth.activations(L.wl, T, L.layer)
    ref = oracle_step(L, x)
    xd, wrd = x.to(DEV), L.wr.to(DEV)
    r, a = route_align(L, xd, wrd)
    check_route(r, ref)
    counts = np.diff(ref["align"]["offsets"])
    say(f"  pairs per expert: min {counts.min()} max {counts.max()}")
    check_layer_out("grouped ffn (prefill kernels)", ffn(L, xd, r, a), ref["out"])
    # padded alignment (segments rounded up to 128 rows) feeds the same kernels
    ap = moe.moe_align(r.ids, s.E, block_m=128)
    check_layer_out("grouped ffn on the padded alignment", ffn(L, xd, r, ap), ref["out"])
    if T == 512:
        check_layer_out("decode kernels forced", ffn(L, xd, r, a, moe.MODE_DECODE), ref["out"])
        check_layer_out("slot rounds over two halves (prefill)", slot_rounds(L, xd, r, a, moe.MODE_PREFILL),
                        ref["out"])


@pytest.mark.parametrize("T", [48, 160, 168])
def test_olmoe_around_mode_threshold(olmoe_prefill, T):
    """Both grouped variants on every token around the automatic choice (decode kernels
    up to 20 expected pairs per expert, T k / E; T = 48: one 16-token block per pass,
    T = 160: two, the last step that picks them; T = 168: the MFMA-tiled kernels), and
    the automatic output bit-identical to the variant the rule names (the kernels are
    deterministic)."""
    L = olmoe_prefill
    s = L.s
    per_expert = T * s.k / s.E
    say(f"OLMoE T={T} ({per_expert:.1f} pairs per expert): both variants, every token")
    x = synth.activations(L.wl, T, L.layer)
    ref = oracle_step(L, x)
    xd, wrd = x.to(DEV), L.wr.to(DEV)
    r, a = route_align(L, xd, wrd)
    check_route(r, ref)
    dec = ffn(L, xd, r, a, moe.MODE_DECODE)
    pre = ffn(L, xd, r, a, moe.MODE_PREFILL)
    auto = ffn(L, xd, r, a)
    check_layer_out("decode kernels", dec, ref["out"])
    check_layer_out("prefill kernels", pre, ref["out"])
    assert np.array_equal(auto, dec if per_expert <= 20 else pre)


# ------------------------------------------------------------------ large expert

@pytest.mark.parametrize("T", [1, 64, 1024])
def test_large_expert_every_token(large, T):
    L = large
    s = L.s
    say(f"large expert T={T}: every token")
    x = synth.activations(L.wl, T, L.layer)
    ref = oracle_step(L, x)
    xd, wrd = x.to(DEV), L.wr.to(DEV)
    r, a = route_align(L, xd, wrd)
    check_route(r, ref)
    check_layer_out("grouped ffn (automatic variant)", ffn(L, xd, r, a), ref["out"])
    if T <= 16:
        out, route = moe.moe_decode_layer(xd, wrd, L.bank, s.I, s.k)
        torch.cuda.synchronize()
        check_route(route, ref)
        check_layer_out("moe_decode_layer", out.float().cpu().numpy(), ref["out"])
        ident = torch.arange(s.E, dtype=torch.int32, device=DEV)
        check_layer_out("slot-table decode path", ffn(L, xd, r, a, moe.MODE_DECODE, ident), ref["out"])
    other = moe.MODE_PREFILL if T <= 64 else moe.MODE_DECODE
    check_layer_out(f"other variant forced (mode {other})", ffn(L, xd, r, a, other), ref["out"])


# ------------------------------------------------------------------ wide d_model decode

@pytest.mark.parametrize("T", [1, 16])
def test_decode_wide_model_dim(T):
    # d = 8192 > 4096: the decode gate/up cannot stage the step's activations in
    # LDS and reads them per group instead; moe_decode_layer refuses the shape
    d, I, E, k = 8192, 256, 4, 2
    say(f"decode d={d} I={I} E={E} k={k} T={T}")
    w13 = synth.normal_bf16((E, 2 * I, d), 0.02, seed=811, device=DEV)
    w2 = synth.normal_bf16((E, d, I), 0.02, seed=812, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    ob = warm_bank(oracle_bank(w13, w2), range(E))
    wr = synth.normal_bf16((E, d), 0.02, seed=813)
    x = synth.normal_bf16((T, d), 1.0, seed=814 + T)
    ref = offn.moe_layer(bits(x), bits(wr), ob, k)
    L = SimpleNamespace(bank=bank, s=SimpleNamespace(d=d, I=I, E=E, k=k))
    xd, wrd = x.to(DEV), wr.to(DEV)
    r = moe.moe_route(xd, wrd, k)
    a = moe.moe_align(r.ids, E)
    check_route(r, ref)
    check_layer_out("grouped ffn (decode, fused combine)", ffn(L, xd, r, a), ref["out"])
    ident = torch.arange(E, dtype=torch.int32, device=DEV)
    check_layer_out("slot-table decode path", ffn(L, xd, r, a, moe.MODE_DECODE, ident), ref["out"])
    with pytest.raises(moe.MoeError):
        moe.moe_decode_layer(xd, wrd, bank, I, k)
