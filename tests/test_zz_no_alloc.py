"""moe_w4a16_grouped_ffn_noalloc (workspace in the library's per-GPU scratch) against
moe_w4a16_grouped_ffn with a caller workspace: the same kernels on the same
workspace layout, so the outputs must be equal bit for bit; two calls in a row,
the second with a smaller input, in both kernel variants, and slot-table rounds
(combine = 0, then combine = 1) whose per-pair results stay in the scratch
between calls.  Steps whose workspace exceeds the scratch are refused."""
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe

from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def layer():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    wl = synth.OLMOE_DECODE
    w13, w2 = synth.expert_weights(wl, 6, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    del w13, w2
    return wl, bank, synth.router_weight(wl, 6).to(DEV)


def routed(wl, wr, T, step):
    x = synth.activations(wl, T, 6, step=step).to(DEV)
    r = moe.moe_route(x, wr, wl.shape.k)
    a = moe.moe_align(r.ids, wl.shape.E)
    return x, r, a


def both(wl, bank, x, r, a, mode):
    s = wl.shape
    T = x.shape[0]
    ref = moe.moe_w4a16_grouped_ffn(x, r, a, bank, s.I, mode=mode)
    got = torch.full((T, s.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    moe.moe_w4a16_grouped_ffn_noalloc_into(x, r, a, bank, s.I, got, mode=mode)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("mode,Ts", [(moe.MODE_DECODE, (16, 4)), (moe.MODE_PREFILL, (512, 100))])
def test_noalloc_equals_workspace_call_twice(layer, mode, Ts):
    wl, bank, wr = layer
    for i, T in enumerate(Ts):
        say(f"noalloc grouped ffn mode={mode} call {i}: T={T}")
        x, r, a = routed(wl, wr, T, step=i)
        got, ref = both(wl, bank, x, r, a, mode)
        assert torch.equal(got, ref), f"call {i} (T={T})"


def test_noalloc_slot_rounds(layer):
    # two rounds over disjoint halves of the experts: the first leaves its per-pair
    # results in the scratch, the second adds its own and combines
    wl, bank, wr = layer
    s = wl.shape
    say("noalloc slot-table rounds, T=16 then T=3")
    even = torch.tensor([e if e % 2 == 0 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    odd = torch.tensor([e if e % 2 == 1 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    for i, T in enumerate((16, 3)):
        x, r, a = routed(wl, wr, T, step=10 + i)
        ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k, moe.MODE_DECODE)
        ref = torch.empty((T, s.d), dtype=torch.bfloat16, device=DEV)
        moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, s.I, ref, ws, moe.MODE_DECODE, False, even)
        moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, s.I, ref, ws, moe.MODE_DECODE, True, odd)
        got = torch.full((T, s.d), float("nan"), dtype=torch.bfloat16, device=DEV)
        moe.moe_w4a16_grouped_ffn_noalloc_into(x, r, a, bank, s.I, got, moe.MODE_DECODE, False, even)
        moe.moe_w4a16_grouped_ffn_noalloc_into(x, r, a, bank, s.I, got, moe.MODE_DECODE, True, odd)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {i} (T={T})"


def test_noalloc_refuses_steps_beyond_the_scratch(layer):
    wl, bank, wr = layer
    s = wl.shape
    T = 4096
    need = moe.ffn_workspace_bytes(T, s.d, s.I, s.E, s.k, moe.MODE_PREFILL)
    assert need > moe.NOALLOC_SCRATCH_BYTES
    say(f"noalloc refuses T={T} ({need} bytes of workspace)")
    x, r, a = routed(wl, wr, T, step=20)
    out = torch.empty((T, s.d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_w4a16_grouped_ffn_noalloc_into(x, r, a, bank, s.I, out, moe.MODE_PREFILL)
    assert ei.value.status == 3  # MOE_ERR_WORKSPACE
