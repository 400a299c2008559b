"""GPU parity of the grouped pass over unquantised BF16 experts (moe_bf16_grouped_ffn)
against the oracle on the bf16 weights themselves (oracle.ffn.Bf16Bank).

Bar: max|gpu - ref| / max|ref| <= 1e-2 per layer output (h and the output are
rounded to bf16, sums are fp32); routing is the same bit-exact route/align as the
four-bit pass.
"""
import numpy as np
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe
from oracle import ffn as offn

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


def oracle_bf16_bank(w13, w2):
    return offn.Bf16Bank(lambda e: bits(w13[e]), lambda e: bits(w2[e]))


def run_bf16(x, wr, bank, I, k, slot_of_expert=None):
    r = moe.moe_route(x, wr, k)
    a = moe.moe_align(r.ids, wr.shape[0])
    T, d = x.shape
    out = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    ws = moe.alloc_workspace(T, d, I, wr.shape[0], k, moe.MODE_DECODE)
    moe.moe_bf16_grouped_ffn_into(x, r, a, bank, I, out, ws, True, slot_of_expert)
    torch.cuda.synchronize()
    return out, r, a


def bf16_case(wl, T, layer=0, sample=None):
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, layer, device=DEV)
    wr = synth.router_weight(wl, layer).to(DEV)
    x = synth.activations(wl, T, layer).to(DEV)
    bank = moe.pack_bf16_experts(w13, w2)
    out, r, _ = run_bf16(x, wr, bank, s.I, s.k)
    tokens = np.arange(T) if sample is None else np.asarray(sample)
    ref = offn.moe_layer(bits(x), bits(wr), oracle_bf16_bank(w13, w2), s.k, tokens=tokens)
    assert np.array_equal(r.ids.cpu().numpy(), ref["ids"])
    err = rel_err(out.float().cpu().numpy()[tokens], ref["out"])
    say(f"  bf16 {wl.name} T={T}: max rel err {err:.3e}")
    assert err <= tol_for_layer()


def test_bf16_pack_layout():
    say("bf16 pack layout")
    g = torch.Generator().manual_seed(3)
    E, d, I = 3, 256, 128
    w13 = torch.randn((E, 2 * I, d), generator=g).to(torch.bfloat16).to(DEV)
    w2 = torch.randn((E, d, I), generator=g).to(torch.bfloat16).to(DEV)
    bank = moe.pack_bf16_experts(w13, w2)
    torch.cuda.synchronize()
    assert moe.bf16_expert_bytes(d, I) == 6 * d * I
    b = bank.cpu()
    for e in range(E):
        assert torch.equal(b[e, :4 * I * d].view(torch.bfloat16).view(2 * I, d), w13[e].cpu())
        assert torch.equal(b[e, 4 * I * d:6 * I * d].view(torch.bfloat16).view(d, I), w2[e].cpu())


def test_bf16_layer_tiny():
    say("bf16 layer tiny")
    bf16_case(synth.TINY, 16)
    bf16_case(synth.TINY, 3)
    bf16_case(synth.TINY, 200, sample=[0, 77, 199])   # 50 pairs per expert: 4-block columns, ragged tail


@pytest.mark.parametrize("T", [1, 16])
def test_bf16_layer_olmoe_decode(T):
    say(f"bf16 layer olmoe T={T}")
    bf16_case(synth.OLMOE_DECODE, T, layer=5, sample=None if T == 1 else [0, 7, 15])


def test_bf16_layer_large_t1():
    say("bf16 layer large expert T=1")
    bf16_case(synth.LARGE, 1, layer=2)


def test_bf16_skewed_routing_and_subsets():
    # every token to experts 3 and 6 (n_e = T: many column blocks), then the two
    # halves of the experts in separate calls must equal one call bit for bit
    say("bf16 skewed routing / slot-table subsets")
    wl = synth.TINY
    s = wl.shape
    T = 45
    w13, w2 = synth.expert_weights(wl, 0, device=DEV)
    wr = torch.zeros((s.E, s.d), dtype=torch.bfloat16)
    wr[3, :] = 0.05
    wr[6, :] = 0.03
    x = synth.activations(wl, T, 0).abs().to(torch.bfloat16)
    bank = moe.pack_bf16_experts(w13, w2)
    out, r, a = run_bf16(x.to(DEV), wr.to(DEV), bank, s.I, s.k)
    ref = offn.moe_layer(bits(x), bits(wr), oracle_bf16_bank(w13, w2), s.k)
    assert rel_err(out.float().cpu().numpy(), ref["out"]) <= tol_for_layer()
    ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k, moe.MODE_DECODE)
    out2 = torch.empty_like(out)
    even = torch.tensor([e if e % 2 == 0 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    odd = torch.tensor([e if e % 2 == 1 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    moe.moe_bf16_grouped_ffn_into(x.to(DEV), r, a, bank, s.I, out2, ws, False, even)
    moe.moe_bf16_grouped_ffn_into(x.to(DEV), r, a, bank, s.I, out2, ws, True, odd)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)


def test_bf16_t0_and_argument_errors():
    say("bf16 T=0 / errors")
    wl = synth.TINY
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 0, device=DEV)
    bank = moe.pack_bf16_experts(w13, w2)
    wr = synth.router_weight(wl, 0).to(DEV)
    x0 = torch.empty((0, s.d), dtype=torch.bfloat16, device=DEV)
    out, _, _ = run_bf16(x0, wr, bank, s.I, s.k)
    assert out.shape == (0, s.d)
    x = synth.activations(wl, 4, 0).to(DEV)
    r = moe.moe_route(x, wr, s.k)
    a = moe.moe_align(r.ids, s.E)
    out = torch.empty((4, s.d), dtype=torch.bfloat16, device=DEV)
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_bf16_grouped_ffn_into(x, r, a, bank, s.I, out, small)
