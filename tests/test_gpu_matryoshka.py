"""GPU parity of the nested two/four-bit path (moe_mat_from_w4, moe_mat_grouped_ffn)
against oracle.matryoshka on the same seeded inputs.

Bars: layout-m1 blobs byte-identical to the oracle's packer; routing bit-exact;
layer outputs within max|gpu - ref| / max|ref| <= 1e-2 with every expert at four
bits (tau = 0), at two bits (tau > 1) and mixed, the per-expert precision being the
oracle's decision on the same routing weights.
"""
import numpy as np
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe
from oracle import matryoshka as omat

from gpu_helpers import bits, check_layer_out, rel_err, say, tol_for_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    moe.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("d,I,E", [(256, 512, 3), (2048, 1024, 2)])
def test_mat_blobs_bit_exact(d, I, E):
    say(f"mat blobs d={d} I={I} E={E}")
    g = torch.Generator().manual_seed(d + I)
    w13 = (torch.randn((E, 2 * I, d), generator=g) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((E, d, I), generator=g) * 0.02).to(torch.bfloat16)
    w4, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    bank = moe.mat_from_w4(w4, d, I)
    torch.cuda.synchronize()
    lay = moe.mat_layout(d, I)
    offs, total = omat.blob_layout_m1(d, I)
    assert lay["blob_bytes"] == total
    assert [lay[k] for k in ("w13_hi", "w13_lo", "w13_scales", "w2_hi", "w2_lo", "w2_scales")] == list(offs)
    assert lay["two_bit_bytes"] == omat.two_bit_prefix_m1(d, I)
    got = bank.cpu().numpy()
    for e in range(E):
        ref = omat.pack_expert_blob_m1(bits(w13[e]), bits(w2[e]))
        assert np.array_equal(got[e], ref), f"expert {e}"


def mat_case(wl, T, tau, layer=0, sample=None, expect=None):
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, layer, device=DEV)
    wr = synth.router_weight(wl, layer).to(DEV)
    x = synth.activations(wl, T, layer).to(DEV)
    w4, _ = moe.pack_experts(w13, w2)
    bank = moe.mat_from_w4(w4, s.d, s.I)
    del w4
    r = moe.moe_route(x, wr, s.k)
    a = moe.moe_align(r.ids, s.E)
    out = torch.empty((T, s.d), dtype=torch.bfloat16, device=DEV)
    ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k, moe.MODE_DECODE)
    moe.moe_mat_grouped_ffn_into(x, r, a, bank, s.I, out, ws, tau)
    torch.cuda.synchronize()
    tokens = np.arange(T) if sample is None else np.asarray(sample)
    obank = omat.MatBank(lambda e: bits(w13[e]), lambda e: bits(w2[e]))
    ref = omat.moe_layer(bits(x), bits(wr), obank, s.k, tau, tokens=tokens)
    assert np.array_equal(r.ids.cpu().numpy(), ref["ids"])
    n4 = sum(ref["precision"].values())
    if expect == "mixed":
        assert 0 < n4 < len(ref["precision"]), ref["precision"]
    err = rel_err(out.float().cpu().numpy()[tokens], ref["out"])
    say(f"  mat {wl.name} T={T} tau={tau}: {n4}/{len(ref['precision'])} experts at four bits, max rel err {err:.3e}")
    assert err <= tol_for_layer()
    return out


def test_mat_layer_tiny_all_precisions():
    say("mat layer tiny")
    mat_case(synth.TINY, 16, 0.0)
    mat_case(synth.TINY, 16, 2.0)
    mat_case(synth.TINY, 16, 0.55, expect="mixed")
    mat_case(synth.TINY, 3, 0.5)


@pytest.mark.parametrize("T,tau", [(1, 0.0), (1, 2.0), (16, 0.0), (16, 2.0), (16, 0.14)])
def test_mat_layer_olmoe(T, tau):
    say(f"mat layer olmoe T={T} tau={tau}")
    mat_case(synth.OLMOE_DECODE, T, tau, layer=4, sample=None if T == 1 else [0, 9, 15],
             expect="mixed" if 0 < tau < 1 and T > 1 else None)


def test_mat_layer_large_t1():
    say("mat layer large T=1")
    mat_case(synth.LARGE, 1, 0.0, layer=3)
    mat_case(synth.LARGE, 1, 2.0, layer=3)


def test_mat_rejects_large_steps():
    say("mat limits")
    wl = synth.TINY
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 0, device=DEV)
    w4, _ = moe.pack_experts(w13, w2)
    bank = moe.mat_from_w4(w4, s.d, s.I)
    wr = synth.router_weight(wl, 0).to(DEV)
    x = synth.activations(wl, 17, 0).to(DEV)
    r = moe.moe_route(x, wr, s.k)
    a = moe.moe_align(r.ids, s.E)
    out = torch.empty((17, s.d), dtype=torch.bfloat16, device=DEV)
    ws = moe.alloc_workspace(17, s.d, s.I, s.E, s.k, moe.MODE_DECODE)
    with pytest.raises(moe.MoeError):
        moe.moe_mat_grouped_ffn_into(x, r, a, bank, s.I, out, ws, 0.0)


def mat_layer_case(wl, T, tau, layer=0, sample=None, expect=None):
    """moe_mat_decode_layer (fused routing + gate/up, down + combine on layout-m1
    blobs) against the oracle at the same tau; routing bit-identical to moe_route;
    with tau <= 0, out bit-identical to moe_decode_layer on the layout-v1 blobs the
    nested ones were made from."""
    s = wl.shape
    say(f"mat decode layer {wl.name} T={T} tau={tau}")
    w13, w2 = synth.expert_weights(wl, layer, device=DEV)
    wr = synth.router_weight(wl, layer).to(DEV)
    x = synth.activations(wl, T, layer).to(DEV)
    w4, _ = moe.pack_experts(w13, w2)
    bank = moe.mat_from_w4(w4, s.d, s.I)
    route = moe.alloc_route(T, s.E, s.k, DEV)
    out = torch.empty((T, s.d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(moe.decode_layer_workspace_bytes(T, s.d, s.I, s.E, s.k), 256), dtype=torch.uint8,
                     device=DEV)
    ctr = moe.alloc_layer_counters(DEV)
    moe.moe_mat_decode_layer_into(x, wr, bank, s.I, s.k, route, out, ws, ctr, tau)
    torch.cuda.synchronize()
    assert int(ctr.abs().sum()) == 0, "counters not left at zero (or the routing wait timed out)"
    r = moe.moe_route(x, wr, s.k)
    torch.cuda.synchronize()
    assert torch.equal(route.ids, r.ids)
    assert torch.equal(route.weights.view(torch.int32), r.weights.view(torch.int32))
    assert torch.equal(route.logits.view(torch.int32), r.logits.view(torch.int32))
    if tau <= 0:
        out4, _ = moe.moe_decode_layer(x, wr, w4, s.I, s.k)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out4.view(torch.int16)), "four-bit nested layer != moe_decode_layer"
    del w4
    tokens = np.arange(T) if sample is None else np.asarray(sample)
    obank = omat.MatBank(lambda e: bits(w13[e]), lambda e: bits(w2[e]))
    ref = omat.moe_layer(bits(x), bits(wr), obank, s.k, tau, tokens=tokens)
    assert np.array_equal(route.ids.cpu().numpy(), ref["ids"])
    n4 = sum(ref["precision"].values())
    if expect == "mixed":
        assert 0 < n4 < len(ref["precision"]), ref["precision"]
    say(f"  {n4}/{len(ref['precision'])} experts at four bits")
    check_layer_out(f"mat decode layer {wl.name} T={T} tau={tau}", out.float().cpu().numpy()[tokens], ref["out"])
    return out


def test_mat_decode_layer_tiny():
    mat_layer_case(synth.TINY, 16, 0.0)
    mat_layer_case(synth.TINY, 16, 2.0)
    mat_layer_case(synth.TINY, 16, 0.55, expect="mixed")
    mat_layer_case(synth.TINY, 3, 0.5)   # fewer pairs than experts: items over the active experts
    mat_layer_case(synth.TINY, 3, 0.0)


@pytest.mark.parametrize("T,tau", [(1, 0.0), (1, 2.0), (1, 0.3), (4, 0.0), (4, 0.14), (16, 0.0), (16, 2.0),
                                   (16, 0.14), (16, 0.1)])
def test_mat_decode_layer_olmoe(T, tau):
    mat_layer_case(synth.OLMOE_DECODE, T, tau, layer=4, sample=None if T <= 4 else [0, 9, 15],
                   expect="mixed" if 0 < tau < 1 and T > 1 else None)


def test_mat_decode_layer_large_t1():
    mat_layer_case(synth.LARGE, 1, 0.0, layer=3)
    mat_layer_case(synth.LARGE, 1, 2.0, layer=3)


def test_mat_decode_layer_limits():
    say("mat decode layer limits")
    wl = synth.TINY
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 0, device=DEV)
    w4, _ = moe.pack_experts(w13, w2)
    bank = moe.mat_from_w4(w4, s.d, s.I)
    wr = synth.router_weight(wl, 0).to(DEV)
    ctr = moe.alloc_layer_counters(DEV)
    for T, tau in ((17, 0.0), (4, float("nan"))):
        x = synth.activations(wl, T, 0).to(DEV)
        route = moe.alloc_route(T, s.E, s.k, DEV)
        out = torch.empty((T, s.d), dtype=torch.bfloat16, device=DEV)
        ws = torch.empty(max(moe.decode_layer_workspace_bytes(T, s.d, s.I, s.E, s.k), 256), dtype=torch.uint8,
                         device=DEV)
        with pytest.raises(moe.MoeError):
            moe.moe_mat_decode_layer_into(x, wr, bank, s.I, s.k, route, out, ws, ctr, tau)
    # a v1-sized stride below the nested blob size is refused like any short stride
    x = synth.activations(wl, 4, 0).to(DEV)
    route = moe.alloc_route(4, s.E, s.k, DEV)
    out = torch.empty((4, s.d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(moe.decode_layer_workspace_bytes(4, s.d, s.I, s.E, s.k), 256), dtype=torch.uint8,
                     device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_mat_decode_layer_into(x, wr, bank, s.I, s.k, route, out, ws, ctr, 0.0, bank_stride=256)
    torch.cuda.synchronize()
    assert int(ctr.abs().sum()) == 0
