"""GPU slot cache: experts in pinned host memory, S device slots, rounds when more
experts are needed than slots.  Outputs must equal the all-resident path bit for
bit (same kernels, same per-pair arithmetic) and the oracle within the layer
tolerance (every token), and the hit / miss / prefetch / slot sequence must equal
the oracle's LRU simulator."""
import numpy as np
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe
from oracle import ffn as offn
from oracle.slot_cache import POLICY_COST, POLICY_LRU, SlotCacheSim

from gpu_helpers import bits, check_layer_out, oracle_bank, say, warm_bank

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_slot_steps(wl, S, steps, T, seed_layer=0, prefetch=None, check_oracle=True, policy=POLICY_LRU,
                   copy_streams=1, decay=0.9):
    """Decode steps through an S-slot cache.  prefetch: None, "prev" (at the start of
    a step, the previous step's experts) or "next" (after a step's last round, the
    next step's experts from its routing: a predictor that can differ from the
    resident set, so copies happen).  Returns (rounds per step, hits, misses,
    prefetch copies)."""
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, seed_layer, device=DEV)
    wr = synth.router_weight(wl, seed_layer).to(DEV)
    bank, lay = moe.pack_experts(w13, w2)
    ob = warm_bank(oracle_bank(w13, w2), range(s.E)) if check_oracle else None
    B = lay["blob_bytes"]
    store = torch.empty((s.E, B), dtype=torch.uint8, pin_memory=True)
    store.copy_(bank.cpu())
    slots = torch.zeros((S, B), dtype=torch.uint8, device=DEV)
    cache = moe.SlotCache(s.E, S, B, store, slots)
    cache.configure(policy, decay, copy_streams)
    sim = SlotCacheSim(s.E, S, policy, decay)
    table = torch.full((s.E,), -1, dtype=torch.int32, device=DEV)
    main = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    done = torch.cuda.Event()
    ffn_done = torch.cuda.Event()
    ffn_done.record(main)
    ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k, moe.MODE_DECODE)
    xs = synth.ar1_activation_sequence(wl, T, seed_layer, steps, device="cpu")
    routes = [None] * steps

    def route(st):
        if routes[st] is None:
            x = xs[st].to(DEV)
            r = moe.moe_route(x, wr, s.k)
            a = moe.moe_align(r.ids, s.E)
            routes[st] = (x, r, a, {w[0] for w in moe.active_experts(a)})
        return routes[st]

    n_rounds = []
    prev = set()
    n_pref = 0
    for st in range(steps):
        if prefetch == "prev" and prev:
            n = cache.prefetch(prev, S, copy, ffn_done)
            assert n == len(sim.prefetch(prev, S)), st
            n_pref += n
        x, r, a, need = route(st)
        prev = need
        cache.begin_step(need)
        expect = sim.step(need)
        pending = set(need)
        out = torch.empty((T, s.d), dtype=torch.bfloat16, device=DEV)
        rounds = 0
        while pending:
            got, nh, nm = cache.load(pending, table, copy, ffn_done, done)
            esub, ehits, ecopies = expect[rounds]
            assert sorted(got) == esub and nh == len(ehits) and nm == len(ecopies), (st, rounds)
            main.wait_event(done)
            pending -= got
            moe.moe_w4a16_grouped_ffn_into(x, r, a, slots, s.I, out, ws, moe.MODE_DECODE, not pending, table)
            ffn_done.record(main)
            rounds += 1
        assert rounds == len(expect)
        if prefetch == "next" and st + 1 < steps:
            # the copies wait for this step's last round (they may overwrite its slots)
            nxt = route(st + 1)[3]
            n = cache.prefetch(nxt, S, copy, ffn_done)
            assert n == len(sim.prefetch(nxt, S)), st
            n_pref += n
        slot_state, _, _ = cache.state()
        assert slot_state == sim.slot_expert
        # all experts resident, through an all-experts slot table: the same two-pass
        # kernels as the slot-cache calls, so the outputs agree bit for bit
        ident = torch.arange(s.E, dtype=torch.int32, device=DEV)
        ref_out = moe.moe_w4a16_grouped_ffn(x, r, a, bank, s.I, mode=moe.MODE_DECODE, slot_of_expert=ident)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"step {st}"
        if ob is not None:
            ref = offn.moe_layer(bits(x), bits(wr), ob, s.k)
            assert np.array_equal(r.ids.cpu().numpy(), ref["ids"])
            check_layer_out(f"step {st} ({rounds} rounds)", out.float().cpu().numpy(), ref["out"])
        n_rounds.append(rounds)
    hits, misses = cache.state()[1:]
    cache.close()
    return n_rounds, hits, misses, n_pref


def test_slot_cache_tiny_rounds():
    say("slot cache tiny E=8 S=3")
    n_rounds, hits, misses, _ = run_slot_steps(synth.TINY, 3, 6, 16)
    assert max(n_rounds) >= 2


def test_slot_cache_olmoe_zipf_16_slots():
    say("slot cache olmoe zipf S=16")
    n_rounds, hits, misses, _ = run_slot_steps(synth.OLMOE_SLOT, 16, 6, 16)
    say(f"  rounds {n_rounds} hits {hits} misses {misses}")
    assert hits > 0 and misses > 0


def test_slot_cache_prefetch_olmoe_zipf_16_slots():
    say("slot cache prefetch olmoe zipf S=16")
    n_rounds, hits, misses, n_pref = run_slot_steps(synth.OLMOE_SLOT, 16, 6, 16, prefetch="prev",
                                                    check_oracle=False)
    say(f"  rounds {n_rounds} hits {hits} misses {misses} prefetched {n_pref}")
    assert hits > 0


@pytest.mark.parametrize("wl,S,T", [(synth.TINY, 3, 2), (synth.OLMOE_SLOT, 16, 16)])
def test_slot_cache_prefetch_next_step_copies(wl, S, T):
    # the next step's experts copied after a step's last round: the prefetch path
    # really moves data (the LRU simulator makes 2 copies at the tiny shape and 11
    # at the OLMoE shape over these 6 steps), and the next step's rounds find
    # those experts resident
    say(f"slot cache next-step prefetch {wl.name} S={S} T={T}")
    n_rounds, hits, misses, n_pref = run_slot_steps(wl, S, 6, T, prefetch="next")
    say(f"  rounds {n_rounds} hits {hits} misses {misses} prefetched {n_pref}")
    assert n_pref > 0


def test_slot_cache_injected_copy_failure(monkeypatch):
    say("slot cache injected failure")
    monkeypatch.setenv("MOE_SLOT_CACHE_FAIL_AFTER", "2")
    wl = synth.TINY
    s = wl.shape
    lay = moe.expert_layout(s.d, s.I)
    B = lay["blob_bytes"]
    store = torch.zeros((s.E, B), dtype=torch.uint8, pin_memory=True)
    slots = torch.zeros((4, B), dtype=torch.uint8, device=DEV)
    cache = moe.SlotCache(s.E, 4, B, store, slots)
    table = torch.full((s.E,), -1, dtype=torch.int32, device=DEV)
    copy = torch.cuda.Stream()
    done = torch.cuda.Event()
    with pytest.raises(moe.MoeError):
        cache.load({0, 1, 2, 3}, table, copy, None, done)
    torch.cuda.synchronize()
    slot_state, hits, misses = cache.state()
    # the first two copies went through, the third failed: its slot is empty, never half-loaded
    assert slot_state[:2] == [0, 1] and slot_state[2] == -1
    cache.close()


@pytest.mark.parametrize("wl,S,T,pf", [(synth.TINY, 3, 16, None), (synth.OLMOE_SLOT, 16, 16, None),
                                       (synth.OLMOE_SLOT, 16, 16, "next")])
def test_slot_cache_cost_aware_two_copy_streams(wl, S, T, pf):
    # the cost-aware policy (usage averages, victims by expected reload cost) with
    # the copies spread over two streams: sequence equal to the simulator's,
    # outputs equal to the resident path and within the tolerance of the oracle
    say(f"slot cache cost-aware, 2 copy streams, {wl.name} S={S} T={T} prefetch={pf}")
    n_rounds, hits, misses, n_pref = run_slot_steps(wl, S, 6, T, prefetch=pf, policy=POLICY_COST,
                                                    copy_streams=2, decay=0.5)
    say(f"  rounds {n_rounds} hits {hits} misses {misses} prefetched {n_pref}")
    assert misses > 0


def run_precision_steps(wl, S, steps, T, tau, policy, copy_streams=2, decay=0.5, seed_layer=0):
    """Slot-cache steps over nested two/four-bit blobs: an expert whose largest routing
    weight in the step is below tau is loaded (and run) at two bits."""
    from oracle import matryoshka as omat
    s = wl.shape
    tau32 = float(np.float32(tau))
    w13, w2 = synth.expert_weights(wl, seed_layer, device=DEV)
    wr = synth.router_weight(wl, seed_layer).to(DEV)
    w4, _ = moe.pack_experts(w13, w2)
    bank = moe.mat_from_w4(w4, s.d, s.I)
    del w4
    lay = moe.mat_layout(s.d, s.I)
    B, P = lay["blob_bytes"], lay["two_bit_bytes"]
    ob = omat.MatBank(lambda e: bits(w13[e]), lambda e: bits(w2[e]))
    store = torch.empty((s.E, B), dtype=torch.uint8, pin_memory=True)
    store.copy_(bank.cpu())
    slots = torch.zeros((S, B), dtype=torch.uint8, device=DEV)
    cache = moe.SlotCache(s.E, S, B, store, slots)
    cache.configure(policy, decay, copy_streams)
    cache.set_prefix(P)
    sim = SlotCacheSim(s.E, S, policy, decay, prefix_bytes=P, blob_bytes=B)
    table = torch.full((s.E,), -1, dtype=torch.int32, device=DEV)
    main = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    done, ffn_done = torch.cuda.Event(), torch.cuda.Event()
    ffn_done.record(main)
    ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k, moe.MODE_DECODE)
    ident = torch.arange(s.E, dtype=torch.int32, device=DEV)
    xs = synth.ar1_activation_sequence(wl, T, seed_layer, steps, device="cpu")
    n_two = n_need = upgrades = 0
    for st in range(steps):
        x = xs[st].to(DEV)
        r = moe.moe_route(x, wr, s.k)
        a = moe.moe_align(r.ids, s.E)
        ids, w = r.ids.cpu().numpy(), r.weights.cpu().numpy()
        need = set(np.unique(ids).tolist())
        full = {e for e in need if np.max(w[ids == e]) >= np.float32(tau)}
        n_two += len(need - full)
        n_need += len(need)
        cache.begin_step(need)
        expect = sim.step(need, full)
        pending = set(need)
        out = torch.empty((T, s.d), dtype=torch.bfloat16, device=DEV)
        rounds = 0
        while pending:
            got, nh, nm, nb = cache.load_precision(pending, full, table, copy, ffn_done, done)
            esub, ehits, ecopies = expect[rounds]
            assert sorted(got) == esub and nh == len(ehits), (st, rounds)
            assert nm == sum(1 for c in ecopies if c[2] != "lo"), (st, rounds)
            assert nb == sim.copy_bytes(ecopies), (st, rounds)
            upgrades += sum(1 for c in ecopies if c[2] == "lo")
            main.wait_event(done)
            pending -= got
            moe.moe_mat_grouped_ffn_into(x, r, a, slots, s.I, out, ws, tau32, not pending, table)
            ffn_done.record(main)
            rounds += 1
        assert rounds == len(expect)
        slot_state, _, _ = cache.state()
        assert slot_state == sim.slot_expert
        assert [bool(v) for v in cache.planes()[0]] == sim.slot_full
        ref_out = torch.empty_like(out)
        moe.moe_mat_grouped_ffn_into(x, r, a, bank, s.I, ref_out, ws, tau32, True, ident)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"step {st}"
        ref = omat.moe_layer(bits(x), bits(wr), ob, s.k, tau32)
        assert np.array_equal(ids, ref["ids"])
        check_layer_out(f"step {st} ({rounds} rounds, {len(need - full)}/{len(need)} experts at two bits)",
                        out.float().cpu().numpy(), ref["out"])
    _, hits, misses = cache.state()
    cache.close()
    return n_two, n_need, upgrades, hits, misses


@pytest.mark.parametrize("wl,S,tau,policy", [(synth.TINY, 3, 0.55, POLICY_LRU), (synth.OLMOE_SLOT, 16, 0.14, POLICY_COST),
                                             (synth.OLMOE_SLOT, 16, 0.1, POLICY_LRU)])
def test_slot_cache_precision_on_miss(wl, S, tau, policy):
    # misses of experts below tau copy only the two-bit prefix of their nested blob and
    # run at two bits; a resident two-bit expert needed at four bits gets its low planes
    say(f"slot cache precision on miss {wl.name} S={S} tau={tau} policy={policy}")
    n_two, n_need, upgrades, hits, misses = run_precision_steps(wl, S, 6, 16, tau, policy)
    say(f"  {n_two}/{n_need} experts at two bits, {upgrades} low-plane completions, hits {hits} misses {misses}")
    assert 0 < n_two < n_need
