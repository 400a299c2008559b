"""GPU parity: every step of the HIP path against the CPU oracle on the same seeded inputs.

Bars: packing, routing indices and the permutation bit-exact; routing weights
within 1e-6 absolute; layer outputs within max|gpu - ref| / max|ref| <= 1e-2
(bf16 outputs vs the float64 oracle on identical dequantised weights).
"""
import numpy as np
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe
from oracle import align as oalign
from oracle import bf16 as obf16
from oracle import ffn as offn
from oracle import quant as oquant
from oracle import route as oroute

from gpu_helpers import bits, check_layer_out, oracle_bank, rel_err, say, tol_for_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    moe.lib()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ pack

def gpu_blob(w13, w2):
    bank, lay = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    torch.cuda.synchronize()
    return bank.cpu().numpy(), lay


@pytest.mark.parametrize("d,I,E,std", [(256, 512, 3, 0.02), (128, 128, 2, 1.0), (2048, 1024, 1, 0.02)])
def test_pack_bit_exact(d, I, E, std):
    say(f"pack d={d} I={I} E={E}")
    g = torch.Generator().manual_seed(d + I + E)
    w13 = (torch.randn((E, 2 * I, d), generator=g) * std).to(torch.bfloat16)
    w2 = (torch.randn((E, d, I), generator=g) * std).to(torch.bfloat16)
    got, lay = gpu_blob(w13, w2)
    for e in range(E):
        ref = oquant.pack_expert_blob(bits(w13[e]), bits(w2[e]))
        assert np.array_equal(got[e], ref), f"expert {e}"


def test_pack_edge_values():
    say("pack edge values")
    I, d = 128, 256
    w = torch.zeros((1, 2 * I, d), dtype=torch.float32)
    w[0, 1, :128] = 0.0                                  # all-zero group -> scale 0, code 8
    w[0, 2, :128] = torch.linspace(-1, 1, 128)           # ties appear after scaling
    w[0, 3, 0] = 7.0
    w[0, 3, 1:9] = torch.tensor([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5])  # exact half-integers
    w[0, 4, :128] = 1e-38                                # subnormal-range amax
    w[0, 5, :128] = 3e38                                 # near the top of the range
    w[0, 6, 128:] = torch.arange(128) * 2.0 ** -120
    w[0, 7] = torch.randn(d) * 1e4
    wb = w.to(torch.bfloat16)
    w2 = (torch.randn((1, d, I)) * 0.02).to(torch.bfloat16)
    got, _ = gpu_blob(wb, w2)
    assert np.array_equal(got[0], oquant.pack_expert_blob(bits(wb[0]), bits(w2[0])))


# ------------------------------------------------------------------ route

@pytest.mark.parametrize("T,d,E,k", [(16, 256, 8, 2), (1, 2048, 64, 8), (4, 2048, 64, 8), (16, 2048, 64, 8),
                                     (333, 2048, 64, 8), (4096, 2048, 64, 8), (64, 4096, 8, 2), (7, 512, 1024, 16),
                                     (5, 128, 1, 1), (300, 256, 128, 16), (300, 256, 256, 8),
                                     # the float64 matrix-core kernel (16-token blocks >= CUs): ragged token
                                     # tail, experts not a multiple of 16, d not a multiple of 32, E = 128
                                     (4100, 136, 100, 6), (5000, 512, 128, 8), (4096, 64, 1, 1)])
def test_route_parity(T, d, E, k):
    say(f"route T={T} d={d} E={E} k={k}")
    g = torch.Generator().manual_seed(T * 7 + d + E)
    x = torch.randn((T, d), generator=g).to(torch.bfloat16)
    wr = (torch.randn((E, d), generator=g) * 0.02).to(torch.bfloat16)
    r = moe.moe_route(x.to(DEV), wr.to(DEV), k)
    torch.cuda.synchronize()
    l_gpu = r.logits.cpu().numpy()
    ids_gpu = r.ids.cpu().numpy()
    w_gpu = r.weights.cpu().numpy()
    l_ref = oroute.logits_f32(bits(x), bits(wr))
    # logits: float64 sums rounded once to float32 on both sides
    ulps = np.abs(l_gpu.view(np.int32).astype(np.int64) - l_ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, f"logit ulp distance {ulps.max()}"
    # selection is a pure function of the float32 logits: bit-exact on the GPU's logits
    assert np.array_equal(ids_gpu, oroute.topk_select(l_gpu, k))
    # and on the oracle's own logits (they agree), end to end
    assert np.array_equal(ids_gpu, oroute.topk_select(l_ref, k))
    w_ref = oroute.topk_weights(l_ref, ids_gpu)
    assert np.max(np.abs(w_gpu - w_ref)) <= 1e-6
    assert np.all(np.abs(w_gpu.sum(1) - 1) <= 1e-6)


def test_route_ties_and_no_renormalize():
    say("route ties / renormalize=0")
    T, d, E, k = 8, 256, 16, 4
    g = torch.Generator().manual_seed(5)
    x = torch.randn((T, d), generator=g).to(torch.bfloat16)
    wr = (torch.randn((E, d), generator=g) * 0.02).to(torch.bfloat16)
    wr[5] = wr[2]            # experts 2 and 5 tie exactly; so do 9, 11, 14
    wr[11] = wr[9]
    wr[14] = wr[9]
    r = moe.moe_route(x.to(DEV), wr.to(DEV), k, renormalize=False)
    torch.cuda.synchronize()
    l_ref = oroute.logits_f32(bits(x), bits(wr))
    assert np.array_equal(r.ids.cpu().numpy(), oroute.topk_select(l_ref, k))
    w_ref = oroute.topk_weights(l_ref, r.ids.cpu().numpy(), renormalize=False)
    assert np.max(np.abs(r.weights.cpu().numpy() - w_ref)) <= 1e-6
    xc = torch.zeros((3, d), dtype=torch.bfloat16)            # all logits 0 -> ids 0..k-1, weights 1/k
    rc = moe.moe_route(xc.to(DEV), wr.to(DEV), k)
    torch.cuda.synchronize()
    assert np.array_equal(rc.ids.cpu().numpy(), np.tile(np.arange(k), (3, 1)))
    assert np.allclose(rc.weights.cpu().numpy(), 1.0 / k, atol=1e-7)


# ------------------------------------------------------------------ align

def check_align_gpu(ids_np, E, block_m=0):
    ids = torch.from_numpy(np.ascontiguousarray(ids_np.astype(np.int32))).to(DEV)
    a = moe.moe_align(ids, E, block_m)
    torch.cuda.synchronize()
    ref = oalign.align(ids_np, E, block_m)
    P = ids_np.size
    assert np.array_equal(a.offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(a.sorted_pairs.cpu().numpy()[:P], ref["sorted_pairs"])
    assert np.array_equal(a.pair_pos.cpu().numpy()[:P], ref["pair_pos"])
    work = moe.active_experts(a)
    counts = np.diff(ref["offsets"])
    assert [w[0] for w in work] == ref["active"].tolist()
    assert all(w[1] == ref["offsets"][w[0]] and w[2] == counts[w[0]] for w in work)
    if block_m:
        assert np.array_equal(a.tile_offsets.cpu().numpy(), ref["tile_offsets"])


@pytest.mark.parametrize("T,E,k", [(1, 64, 8), (16, 8, 2), (16, 64, 8), (333, 64, 8), (4096, 64, 8),
                                   (1024, 8, 2), (50, 1024, 16), (3, 1, 1)])
def test_align_bit_exact(T, E, k):
    say(f"align T={T} E={E} k={k}")
    ids = synth.random_topk_ids(T, E, k, seed=T + E + k).numpy()
    check_align_gpu(ids, E, block_m=128)
    check_align_gpu(ids, E, block_m=0)


@pytest.mark.parametrize("T,E,k", [(600, 64, 8), (300, 1024, 16), (2049, 8, 2), (20001, 64, 8)])
def test_align_chunked_bit_exact(T, E, k):
    # 4096 pairs and more take the chunked kernel (one workgroup per 2048 pairs, at
    # most 64 workgroups: 160008 pairs use chunks of 4096, two super-batches per
    # wavefront): ragged last chunk, wide ids, few experts
    say(f"align chunked T={T} E={E} k={k}")
    ids = synth.random_topk_ids(T, E, k, seed=7 * T + E + k).numpy()
    check_align_gpu(ids, E, block_m=128)
    check_align_gpu(ids, E, block_m=0)


def test_align_chunked_edges():
    say("align chunked edges")
    check_align_gpu(np.full((5000, 1), 5, dtype=np.int32), 8, 128)      # one expert takes everything
    rng = np.random.default_rng(1)
    skew = rng.choice(4, size=(3000, 2), p=[0.7, 0.2, 0.05, 0.05])      # ragged, repeated ids per token
    check_align_gpu(skew, 64, 64)
    # out-of-range ids (dropped, pair_pos -1) inside several chunks: the valid pairs
    # must sit where the oracle puts them when the dropped ones are left out
    ids = synth.random_topk_ids(700, 64, 8, seed=3).numpy().astype(np.int32)
    ids[::7, 3] = -1
    ids[5, 0] = 64
    flat = ids.reshape(-1)
    keep = np.nonzero((flat >= 0) & (flat < 64))[0]
    ref = oalign.align(flat[keep], 64)
    a = moe.moe_align(torch.from_numpy(ids).to(DEV), 64, 0)
    torch.cuda.synchronize()
    assert np.array_equal(a.offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(a.sorted_pairs.cpu().numpy()[:keep.size], keep[ref["sorted_pairs"]])
    pos = np.full(flat.size, -1, dtype=np.int64)
    pos[keep] = ref["pair_pos"]
    assert np.array_equal(a.pair_pos.cpu().numpy()[:flat.size], pos)


def test_align_edges():
    say("align edges")
    check_align_gpu(np.zeros((0, 4), dtype=np.int32), 8, 16)            # empty
    check_align_gpu(np.full((3000, 1), 5, dtype=np.int32), 8, 128)      # one expert takes everything
    rng = np.random.default_rng(0)
    skew = rng.choice(4, size=(2000, 2), p=[0.7, 0.2, 0.05, 0.05])      # ragged, repeated ids per token
    check_align_gpu(skew, 64, 64)


@pytest.mark.parametrize("T,E,k,renorm", [(1, 64, 8, True), (16, 64, 8, True), (16, 64, 8, False),
                                          (128, 64, 8, True), (16, 8, 2, True), (7, 1024, 16, True),
                                          (2, 1024, 16, False), (100, 64, 16, True), (129, 64, 8, True)])
def test_route_align_fused_equals_separate(T, E, k, renorm):
    """moe_route_align (one launch up to 128 tokens, the separate calls above) gives
    bit-identical routing and permutation; three calls in a row reuse the counters."""
    say(f"route_align T={T} E={E} k={k} renormalize={renorm}")
    d = 2048 if E <= 64 else 512
    x = synth.normal_bf16((T, d), 1.0, seed=77 + T).to(DEV)
    wr = synth.normal_bf16((E, d), 0.02, seed=78 + E).to(DEV)
    r0 = moe.moe_route(x, wr, k, renormalize=renorm)
    a0 = moe.moe_align(r0.ids, E, block_m=128)
    counter = moe.alloc_counter(DEV)
    for rep in range(3):
        r1 = moe.alloc_route(T, E, k, DEV)
        a1 = moe.alloc_align(T, k, E, DEV, block_m=128)
        moe.moe_route_align_into(x, wr, k, r1, a1, counter, renormalize=renorm)
        torch.cuda.synchronize()
        assert torch.equal(r1.logits, r0.logits)
        assert torch.equal(r1.ids, r0.ids)
        assert torch.equal(r1.weights, r0.weights)
        for name in ("offsets", "sorted_pairs", "pair_pos", "tile_offsets"):
            assert torch.equal(getattr(a1, name), getattr(a0, name)), name
        U = int(a0.active[0])
        assert torch.equal(a1.active[:4 + 4 * U], a0.active[:4 + 4 * U])
        assert int(counter.abs().sum()) == 0
    # and against the oracle's selection
    _, ids, _ = oroute.route(bits(x.cpu()), bits(wr.cpu()), k, renormalize=renorm)
    assert np.array_equal(r0.ids.cpu().numpy(), ids)


# ------------------------------------------------------------------ whole layer

def run_layer(x, wr, bank, I, k, mode=moe.MODE_AUTO):
    r = moe.moe_route(x, wr, k)
    a = moe.moe_align(r.ids, wr.shape[0])
    out = moe.moe_w4a16_grouped_ffn(x, r, a, bank, I, mode=mode)
    torch.cuda.synchronize()
    return out, r, a


def layer_case(wl, T, layer=0, sample=None, device_weights=False, mode=moe.MODE_AUTO):
    s = wl.shape
    wdev = DEV if device_weights else "cpu"
    w13, w2 = synth.expert_weights(wl, layer, device=wdev)
    wr = synth.router_weight(wl, layer)
    x = synth.activations(wl, T, layer)
    bank, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    out, r, _ = run_layer(x.to(DEV), wr.to(DEV), bank, s.I, s.k, mode)
    tokens = np.arange(T) if sample is None else np.asarray(sample)
    ref = offn.moe_layer(bits(x), bits(wr), oracle_bank(w13, w2), s.k, tokens=tokens)
    assert np.array_equal(r.ids.cpu().numpy(), ref["ids"])
    got = out.float().cpu().numpy()[tokens]
    err = rel_err(got, ref["out"])
    say(f"  {wl.name} T={T} mode={mode}: max rel err {err:.3e}")
    assert err <= tol_for_layer()
    return err


def test_layer_tiny():
    say("layer tiny")
    layer_case(synth.TINY, 16)
    layer_case(synth.TINY, 16, mode=moe.MODE_PREFILL)
    layer_case(synth.TINY, 3)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_layer_olmoe_decode(T):
    say(f"layer olmoe decode T={T}")
    sample = None if T <= 4 else [0, 5, 10, 15]
    layer_case(synth.OLMOE_DECODE, T, layer=3, sample=sample, device_weights=True)


@pytest.mark.parametrize("T", [512, 4096])
def test_layer_olmoe_prefill_sampled(T):
    say(f"layer olmoe prefill T={T}")
    layer_case(synth.OLMOE_PREFILL, T, layer=1, sample=[0, T // 2 + 1, T - 1], device_weights=True)


def test_layer_large_expert_t1():
    say("layer large expert T=1")
    layer_case(synth.LARGE, 1, layer=0, device_weights=True)


@pytest.mark.parametrize("T", [64, 1024])
def test_layer_large_expert_sampled(T):
    say(f"layer large expert T={T}")
    layer_case(synth.LARGE, T, layer=1, sample=[0, T - 1], device_weights=True)


def test_layer_skewed_routing_and_ragged_blocks():
    # all tokens routed to expert 3 via the router weights: n_e = T, far beyond one 16/32-token block
    say("layer skewed routing")
    wl = synth.TINY
    s = wl.shape
    T = 45
    w13, w2 = synth.expert_weights(wl, 0)
    wr = torch.zeros((s.E, s.d), dtype=torch.bfloat16)
    wr[3, :] = 0.05
    wr[6, :] = 0.03
    x = synth.activations(wl, T, 0).abs().to(torch.bfloat16)   # positive -> experts 3 then 6 always win
    bank, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    for mode in (moe.MODE_DECODE, moe.MODE_PREFILL):
        out, r, a = run_layer(x.to(DEV), wr.to(DEV), bank, s.I, s.k, mode)
        assert set(np.unique(r.ids.cpu().numpy())) == {3, 6}
        ref = offn.moe_layer(bits(x), bits(wr), oracle_bank(w13, w2), s.k)
        assert rel_err(out.float().cpu().numpy(), ref["out"]) <= tol_for_layer()


def test_layer_prefill_mixed_tile_loads():
    # a router bias along one activation channel spreads the per-expert loads: experts
    # whose last 128-token tile holds at most 64 tokens (ordered after all other tiles),
    # experts with a fuller last tile, experts with several tiles and one with exactly two;
    # every token against the oracle
    say("layer prefill mixed tile loads")
    g = torch.Generator().manual_seed(31)
    d, I, E, k, T = 512, 256, 16, 4, 700
    w13 = (torch.randn((E, 2 * I, d), generator=g) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((E, d, I), generator=g) * 0.02).to(torch.bfloat16)
    wr = torch.randn((E, d), generator=g) * 0.02
    wr[:, 0] = 0.3 * torch.arange(E, dtype=torch.float32) / E
    wr = wr.to(torch.bfloat16)
    x = torch.randn((T, d), generator=g)
    x[:, 0] = 4.0
    x = x.to(torch.bfloat16)
    bank, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    ref = offn.moe_layer(bits(x), bits(wr), oracle_bank(w13, w2), k)
    n_e = np.bincount(ref["ids"].reshape(-1), minlength=E)
    rem = n_e % 128
    assert np.any((rem > 0) & (rem <= 64)) and np.any(rem > 64) and np.any(n_e > 128), n_e
    for mode in (moe.MODE_PREFILL, moe.MODE_AUTO):
        out, r, _ = run_layer(x.to(DEV), wr.to(DEV), bank, I, k, mode)
        assert np.array_equal(r.ids.cpu().numpy(), ref["ids"])
        check_layer_out(f"mixed loads mode={mode}", out.float().cpu().numpy(), ref["out"])


def test_layer_single_expert_top1():
    say("layer E=1 k=1")
    g = torch.Generator().manual_seed(9)
    d, I, T = 256, 256, 20
    w13 = (torch.randn((1, 2 * I, d), generator=g) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn((1, d, I), generator=g) * 0.05).to(torch.bfloat16)
    wr = (torch.randn((1, d), generator=g) * 0.02).to(torch.bfloat16)
    x = torch.randn((T, d), generator=g).to(torch.bfloat16)
    bank, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    out, r, _ = run_layer(x.to(DEV), wr.to(DEV), bank, I, 1)
    assert np.all(r.weights.cpu().numpy() == 1.0)
    ref = offn.moe_layer(bits(x), bits(wr), oracle_bank(w13, w2), 1)
    assert rel_err(out.float().cpu().numpy(), ref["out"]) <= tol_for_layer()


def test_layer_deterministic_and_t0():
    say("layer determinism / T=0")
    wl = synth.TINY
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 0)
    bank, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    wr = synth.router_weight(wl, 0).to(DEV)
    x = synth.activations(wl, 16, 0).to(DEV)
    o1, _, _ = run_layer(x, wr, bank, s.I, s.k)
    o2, _, _ = run_layer(x, wr, bank, s.I, s.k)
    assert torch.equal(o1, o2)
    x0 = torch.empty((0, s.d), dtype=torch.bfloat16, device=DEV)
    o0, _, _ = run_layer(x0, wr, bank, s.I, s.k)
    assert o0.shape == (0, s.d)


def test_slot_table_subsets_equal_resident():
    # running the experts in two disjoint subsets (slot table with -1 = skip), then
    # combining, must equal the one-pass result bit for bit
    say("ffn subsets via slot table")
    wl = synth.TINY
    s = wl.shape
    T = 16
    w13, w2 = synth.expert_weights(wl, 0)
    bank, _ = moe.pack_experts(w13.to(DEV), w2.to(DEV))
    wr = synth.router_weight(wl, 0).to(DEV)
    x = synth.activations(wl, T, 0).to(DEV)
    fused, r, a = run_layer(x, wr, bank, s.I, s.k, moe.MODE_DECODE)
    # an all-experts slot table keeps the separate combine kernel (the path that
    # subset calls use); with no table, steps of <= 16 tokens combine inside the
    # down pass, in another summation order
    ident = torch.arange(s.E, dtype=torch.int32, device=DEV)
    ref = moe.moe_w4a16_grouped_ffn(x, r, a, bank, s.I, moe.MODE_DECODE, slot_of_expert=ident)
    assert rel_err(fused.float().cpu().numpy(), ref.float().cpu().numpy()) <= tol_for_layer()
    ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k, moe.MODE_DECODE)
    out = torch.empty_like(ref)
    half = torch.tensor([e if e % 2 == 0 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    other = torch.tensor([e if e % 2 == 1 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, s.I, out, ws, moe.MODE_DECODE, False, half)
    moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, s.I, out, ws, moe.MODE_DECODE, True, other)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_slot_table_subsets_equal_resident_prefill():
    # the same in the prefill kernels, at a size where every workgroup walks several
    # tiles and half the experts have no slot (tiles skipped between computed ones)
    say("ffn subsets via slot table, prefill OLMoE T=1024")
    wl = synth.OLMOE_PREFILL
    s = wl.shape
    T = 1024
    w13, w2 = synth.expert_weights(wl, 3, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    del w13, w2
    wr = synth.router_weight(wl, 3).to(DEV)
    x = synth.activations(wl, T, 3).to(DEV)
    _, r, a = run_layer(x, wr, bank, s.I, s.k, moe.MODE_PREFILL)
    ident = torch.arange(s.E, dtype=torch.int32, device=DEV)
    ref = moe.moe_w4a16_grouped_ffn(x, r, a, bank, s.I, moe.MODE_PREFILL, slot_of_expert=ident)
    ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k, moe.MODE_PREFILL)
    out = torch.empty_like(ref)
    half = torch.tensor([e if e % 2 == 0 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    other = torch.tensor([e if e % 2 == 1 else -1 for e in range(s.E)], dtype=torch.int32, device=DEV)
    moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, s.I, out, ws, moe.MODE_PREFILL, False, half)
    moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, s.I, out, ws, moe.MODE_PREFILL, True, other)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("T", [1, 16])
def test_per_expert_calls_equal_fused(T):
    # the ablation's sequential variant: one grouped-FFN call per active expert (slot
    # table keeping only that expert), combine on the last call; same kernels as one
    # call with an all-experts slot table, so equal to it bit for bit, and within the
    # layer tolerance of the call without a table (OLMoE shape, decode path)
    say(f"per-expert calls vs fused T={T}")
    wl = synth.OLMOE_DECODE
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 2, device=DEV)
    bank, _ = moe.pack_experts(w13, w2)
    del w13, w2
    wr = synth.router_weight(wl, 2).to(DEV)
    x = synth.activations(wl, T, 2).to(DEV)
    fused, r, a = run_layer(x, wr, bank, s.I, s.k)
    ident = torch.arange(s.E, dtype=torch.int32, device=DEV)
    ref = moe.moe_w4a16_grouped_ffn(x, r, a, bank, s.I, slot_of_expert=ident)
    assert rel_err(fused.float().cpu().numpy(), ref.float().cpu().numpy()) <= tol_for_layer()
    ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k)
    out = torch.empty_like(ref)
    act = a.active.cpu()
    experts = act[4::4][:int(act[0])].tolist()
    assert len(experts) == len(set(r.ids.cpu().numpy().ravel().tolist()))
    for i, e in enumerate(experts):
        only = torch.full((s.E,), -1, dtype=torch.int32, device=DEV)
        only[e] = e
        moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, s.I, out, ws, combine=(i == len(experts) - 1),
                                       slot_of_expert=only)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
