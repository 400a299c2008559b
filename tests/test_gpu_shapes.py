"""GPU parity over irregular layer shapes (seeded): the fused decode layer
(moe_decode_layer) and the grouped expert FFN in both variants, each against the
float64 oracle on every token; and the fused decode layer on nested two/four-bit
blobs (moe_mat_decode_layer) against the nested oracle at several precision
thresholds, bit-identical to moe_decode_layer when every expert runs at four bits;
and prefill-sized steps through the MFMA-tiled kernels (ragged token tiles, row
tiles that overhang the model dimension, many experts).

The shapes reach the corners of the entry points' limits: a single K group each
way (d or I = 128), k = 1 and k = E, expert counts that are not multiples of 16,
more experts than the LDS rank top-k handles (E > 128: the wave-wide argmax), the
largest top-k (16), steps that route fewer pairs than there are experts and the
widest model dimension of the fused layer (d = 4096).  Bars as elsewhere: routing
ids bit-exact, weights within 1e-6, outputs within 1e-2 of the largest output over
the layer and per token.
"""
import numpy as np
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe
from oracle import ffn as offn

from gpu_helpers import bits, check_layer_out, oracle_bank, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (T, d, I, E, k)
SHAPES = [
    (1, 128, 128, 3, 1),
    (5, 128, 256, 5, 5),
    (7, 384, 128, 20, 3),
    (16, 256, 384, 40, 6),
    (13, 512, 256, 130, 4),
    (2, 640, 128, 64, 8),
    (16, 128, 128, 16, 16),
    (9, 4096, 128, 6, 2),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    moe.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,d,I,E,k", SHAPES)
def test_shape_every_token(T, d, I, E, k):
    say(f"shape T={T} d={d} I={I} E={E} k={k}")
    seed = 1000 * E + 10 * k + T
    w13 = synth.normal_bf16((E, 2 * I, d), 0.05, seed)
    w2 = synth.normal_bf16((E, d, I), 0.05, seed + 1)
    wr = synth.normal_bf16((E, d), 0.05, seed + 2)
    x = synth.normal_bf16((T, d), 1.0, seed + 3)
    ref = offn.moe_layer(bits(x), bits(wr), oracle_bank(w13, w2), k)
    bank, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    xd, wrd = x.to(DEV), wr.to(DEV)

    out, route = moe.moe_decode_layer(xd, wrd, bank, I, k)
    torch.cuda.synchronize()
    assert np.array_equal(route.ids.cpu().numpy(), ref["ids"])
    assert np.max(np.abs(route.weights.cpu().numpy() - ref["weights"])) <= 1e-6
    check_layer_out("moe_decode_layer", out.float().cpu().numpy(), ref["out"])

    r = moe.moe_route(xd, wrd, k)
    a = moe.moe_align(r.ids, E)
    for mode, name in ((moe.MODE_DECODE, "grouped ffn, decode kernels"),
                       (moe.MODE_PREFILL, "grouped ffn, MFMA-tiled kernels")):
        got = moe.moe_w4a16_grouped_ffn(xd, r, a, bank, I, mode=mode)
        torch.cuda.synchronize()
        check_layer_out(name, got.float().cpu().numpy(), ref["out"])


# nested two/four-bit blobs (d and I multiples of 256: plane tiles of two groups);
# (T, d, I, E, k, tau): tau <= 0 every expert at four bits, tau >= 1 at two
MAT_SHAPES = [
    (1, 256, 256, 3, 1, 0.0),
    (5, 256, 512, 5, 5, 2.0),
    (7, 512, 256, 20, 3, 0.3),
    (16, 256, 256, 40, 6, 0.1),
    (13, 512, 256, 130, 4, 0.2),
    (9, 4096, 256, 6, 2, 0.4),
]


@pytest.mark.parametrize("T,d,I,E,k,tau", MAT_SHAPES)
def test_mat_shape_every_token(T, d, I, E, k, tau):
    from oracle import matryoshka as omat
    say(f"nested shape T={T} d={d} I={I} E={E} k={k} tau={tau}")
    seed = 2000 * E + 10 * k + T
    w13 = synth.normal_bf16((E, 2 * I, d), 0.05, seed)
    w2 = synth.normal_bf16((E, d, I), 0.05, seed + 1)
    wr = synth.normal_bf16((E, d), 0.05, seed + 2)
    x = synth.normal_bf16((T, d), 1.0, seed + 3)
    obank = omat.MatBank(lambda e: bits(w13[e]), lambda e: bits(w2[e]))
    ref = omat.moe_layer(bits(x), bits(wr), obank, k, tau)
    w4, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    bank = moe.mat_from_w4(w4, d, I)
    xd, wrd = x.to(DEV), wr.to(DEV)
    route = moe.alloc_route(T, E, k, DEV)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(moe.decode_layer_workspace_bytes(T, d, I, E, k), 256), dtype=torch.uint8, device=DEV)
    ctr = moe.alloc_layer_counters(DEV)
    moe.moe_mat_decode_layer_into(xd, wrd, bank, I, k, route, out, ws, ctr, tau)
    torch.cuda.synchronize()
    assert int(ctr.abs().sum()) == 0
    assert np.array_equal(route.ids.cpu().numpy(), ref["ids"])
    check_layer_out("moe_mat_decode_layer", out.float().cpu().numpy(), ref["out"])
    if tau <= 0:
        out4, _ = moe.moe_decode_layer(xd, wrd, w4, I, k)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out4.view(torch.int16))


# prefill-sized steps: several 128-token tiles per expert with ragged tails, row
# tiles that overhang N (d = 384, 640), many experts with light last tiles
PREFILL_SHAPES = [
    (600, 384, 384, 20, 4),
    (333, 640, 256, 130, 6),
    (1000, 256, 128, 7, 2),
]


@pytest.mark.parametrize("T,d,I,E,k", PREFILL_SHAPES)
def test_prefill_shape_every_token(T, d, I, E, k):
    say(f"prefill shape T={T} d={d} I={I} E={E} k={k}")
    seed = 3000 * E + 10 * k + T
    w13 = synth.normal_bf16((E, 2 * I, d), 0.05, seed)
    w2 = synth.normal_bf16((E, d, I), 0.05, seed + 1)
    wr = synth.normal_bf16((E, d), 0.05, seed + 2)
    x = synth.normal_bf16((T, d), 1.0, seed + 3)
    ref = offn.moe_layer(bits(x), bits(wr), oracle_bank(w13, w2), k)
    bank, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    xd, wrd = x.to(DEV), wr.to(DEV)
    r = moe.moe_route(xd, wrd, k)
    a = moe.moe_align(r.ids, E)
    torch.cuda.synchronize()
    assert np.array_equal(r.ids.cpu().numpy(), ref["ids"])
    for mode, name in ((moe.MODE_PREFILL, "grouped ffn, MFMA-tiled kernels"),
                       (moe.MODE_AUTO, "grouped ffn, automatic choice")):
        got = moe.moe_w4a16_grouped_ffn(xd, r, a, bank, I, mode=mode)
        torch.cuda.synchronize()
        check_layer_out(name, got.float().cpu().numpy(), ref["out"])
