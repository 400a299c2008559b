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

from gpu_helpers import bits, rel_err, say, tol_for_layer

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
