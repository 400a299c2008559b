"""HIP-graph capture of whole layer steps: every replay must equal the eager result
bit for bit, with eager work and synchronisations between the replays."""
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe

from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("wl,T", [(synth.TINY, 16), (synth.OLMOE_DECODE, 16), (synth.OLMOE_DECODE, 1)])
def test_graph_replays_equal_eager(wl, T):
    say(f"graph replay {wl.name} T={T}")
    s = wl.shape
    layers = []
    for l in range(2):
        w13, w2 = synth.expert_weights(wl, l, device=DEV)
        bank, _ = moe.pack_experts(w13, w2)
        del w13, w2
        layers.append(moe.MoELayer(synth.router_weight(wl, l).to(DEV), bank, s.I, s.k, T))
    x = synth.activations(wl, T, 0).to(DEV)

    def step():
        h = layers[0].forward(x)
        return layers[1].forward(h)

    ref = step().clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    for i in range(3):
        layers[1].out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        other = step()                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, ref)


@pytest.mark.parametrize("wl,T", [(synth.OLMOE_DECODE, 16), (synth.OLMOE_DECODE, 3)])
def test_graph_replays_decode_layer(wl, T):
    """moe_decode_layer (waits on its own device-scope counters) captured for two
    chained layers: every replay equals the eager step and leaves the counters zero."""
    say(f"graph replay moe_decode_layer {wl.name} T={T}")
    s = wl.shape
    banks, wrs = [], []
    for l in range(2):
        w13, w2 = synth.expert_weights(wl, l, device=DEV)
        bank, _ = moe.pack_experts(w13, w2)
        del w13, w2
        banks.append(bank)
        wrs.append(synth.router_weight(wl, l).to(DEV))
    x = synth.activations(wl, T, 0).to(DEV)
    routes = [moe.alloc_route(T, s.E, s.k, DEV) for _ in range(2)]
    outs = [torch.empty((T, s.d), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    ws = torch.empty(moe.decode_layer_workspace_bytes(T, s.d, s.I, s.E, s.k), dtype=torch.uint8, device=DEV)
    ctr = moe.alloc_layer_counters(DEV)

    def step():
        moe.moe_decode_layer_into(x, wrs[0], banks[0], s.I, s.k, routes[0], outs[0], ws, ctr)
        moe.moe_decode_layer_into(outs[0], wrs[1], banks[1], s.I, s.k, routes[1], outs[1], ws, ctr)
        return outs[1]

    ref = step().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        outs[1].zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[1], ref), f"replay {i}"
        assert int(torch.count_nonzero(ctr)) == 0
        other = step().clone()          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, ref)
