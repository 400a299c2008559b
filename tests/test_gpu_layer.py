"""GPU parity of moe_decode_layer (routing + grouped gate/up in one launch, down +
combine in a second) on the same seeded inputs.

Bars: logits, topk ids and weights bit-identical to moe_route_align; the layer
output bit-identical to moe_route_align + moe_w4a16_grouped_ffn where that path
accumulates each gate/up item's K range in one wavefront (steps with many active
experts: OLMoE T = 8, 16), else within 1e-2 of it (that path splits K over two
wavefronts when few experts are active: another fp32 summation order); routing
bit-exact and the output within max|gpu - ref| / max|ref| <= 1e-2 of the oracle;
the counters back at zero after every call.
"""
import numpy as np
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe
from oracle import ffn as offn

from gpu_helpers import bits, oracle_bank, rel_err, say, tol_for_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    moe.lib()
    yield
    torch.cuda.synchronize()


def two_call_path(x, wr, bank, I, k, renormalize=True):
    T, d = x.shape
    E = wr.shape[0]
    r = moe.alloc_route(T, E, k, DEV)
    a = moe.alloc_align(T, k, E, DEV)
    ctr = moe.alloc_counter(DEV)
    moe.moe_route_align_into(x, wr, k, r, a, ctr, renormalize)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    ws = moe.alloc_workspace(T, d, I, E, k, moe.MODE_DECODE)
    moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, I, out, ws, moe.MODE_DECODE)
    return out, r


def layer_equal_case(x, wr, bank, I, k, renormalize=True, calls=3, bitwise=False):
    T, d = x.shape
    E = wr.shape[0]
    ref, rr = two_call_path(x, wr, bank, I, k, renormalize)
    route = moe.alloc_route(T, E, k, DEV)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(moe.decode_layer_workspace_bytes(T, d, I, E, k), dtype=torch.uint8, device=DEV)
    ctr = moe.alloc_layer_counters(DEV)
    for c in range(calls):                       # the counters are reused call after call
        out.fill_(float("nan"))
        moe.moe_decode_layer_into(x, wr, bank, I, k, route, out, ws, ctr, renormalize)
        torch.cuda.synchronize()
        nz = torch.nonzero(ctr).flatten().tolist()
        assert not nz, f"counters not reset after call {c}: {[(i, int(ctr[i])) for i in nz]}"
        assert torch.equal(route.logits, rr.logits)
        assert torch.equal(route.ids, rr.ids)
        assert torch.equal(route.weights, rr.weights)
        if bitwise:
            assert torch.equal(out, ref), f"call {c}"
        else:
            assert rel_err(out.float().cpu().numpy(), ref.float().cpu().numpy()) <= tol_for_layer(), f"call {c}"
    return out, route


@pytest.mark.parametrize("T", [1, 3, 8, 16])
def test_layer_equals_two_calls_olmoe(T):
    say(f"decode layer vs route_align + ffn, OLMoE T={T}")
    wl = synth.OLMOE_DECODE
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 1, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    del w13, w2
    wr = synth.router_weight(wl, 1).to(DEV)
    x = synth.activations(wl, T, 1).to(DEV)
    layer_equal_case(x, wr, bank, s.I, s.k, bitwise=T >= 8)


@pytest.mark.parametrize("T,renorm", [(16, True), (5, False), (1, True)])
def test_layer_tiny_against_oracle(T, renorm):
    say(f"decode layer tiny T={T} renormalize={renorm}")
    wl = synth.TINY
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 0)
    bank, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    wr = synth.router_weight(wl, 0)
    x = synth.activations(wl, T, 0)
    out, route = layer_equal_case(x.to(DEV), wr.to(DEV), bank, s.I, s.k, renorm)
    ref = offn.moe_layer(bits(x), bits(wr), oracle_bank(w13, w2), s.k, renormalize=renorm)
    assert np.array_equal(route.ids.cpu().numpy(), ref["ids"])
    err = rel_err(out.float().cpu().numpy(), ref["out"])
    say(f"  max rel err {err:.3e}")
    assert err <= tol_for_layer()


def test_layer_olmoe_t16_against_oracle_sampled():
    say("decode layer OLMoE T=16 vs oracle (sampled tokens)")
    wl = synth.OLMOE_DECODE
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 5, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    wr = synth.router_weight(wl, 5)
    x = synth.activations(wl, 16, 5)
    out, route = moe.moe_decode_layer(x.to(DEV), wr.to(DEV), bank, s.I, s.k)
    torch.cuda.synchronize()
    tokens = [0, 7, 15]
    ref = offn.moe_layer(bits(x), bits(wr), oracle_bank(w13, w2), s.k, tokens=tokens)
    assert np.array_equal(route.ids.cpu().numpy(), ref["ids"])
    err = rel_err(out.float().cpu().numpy()[tokens], ref["out"])
    say(f"  max rel err {err:.3e}")
    assert err <= tol_for_layer()


def test_layer_large_and_wide_router():
    say("decode layer: large expert T=1, 4; E=1024 k=16 T=7")
    wl = synth.LARGE
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 2, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    del w13, w2
    wr = synth.router_weight(wl, 2).to(DEV)
    for T in (1, 4):
        layer_equal_case(synth.activations(wl, T, 2).to(DEV), wr, bank, s.I, s.k, calls=2)
    del bank
    # many small experts: E = 1024, k = 16 (every block builds a 1024-expert list)
    d, I, E, k, T = 256, 128, 1024, 16, 7
    w13 = synth.normal_bf16((E, 2 * I, d), 0.02, seed=31, device=DEV)
    w2 = synth.normal_bf16((E, d, I), 0.02, seed=32, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    wr = synth.normal_bf16((E, d), 0.02, seed=33, device=DEV)
    x = synth.normal_bf16((T, d), 1.0, seed=34, device=DEV)
    layer_equal_case(x, wr, bank, I, k, calls=2)
    layer_equal_case(x, wr, bank, I, k, renormalize=False, calls=1)


def test_layer_limits():
    say("decode layer limits")
    wl = synth.TINY
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 0, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    wr = synth.router_weight(wl, 0).to(DEV)
    x0 = torch.empty((0, s.d), dtype=torch.bfloat16, device=DEV)
    out0, _ = moe.moe_decode_layer(x0, wr, bank, s.I, s.k)
    assert out0.shape == (0, s.d)
    x = synth.activations(wl, 17, 0).to(DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_decode_layer(x, wr, bank, s.I, s.k)
