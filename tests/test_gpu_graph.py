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
