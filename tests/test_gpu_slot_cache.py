"""GPU slot cache: experts in pinned host memory, S device slots, rounds when more
experts are needed than slots.  Outputs must equal the all-resident path bit for
bit (same kernels, same per-pair arithmetic), and the hit / miss / slot sequence
must equal the oracle's LRU simulator."""
import numpy as np
import pytest
import torch

import synth
import w4a16_grouped_expert_amd as moe
from oracle.slot_cache import LRUSlotCache

from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_slot_steps(wl, S, steps, T, seed_layer=0, prefetch=False):
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, seed_layer, device=DEV)
    wr = synth.router_weight(wl, seed_layer).to(DEV)
    bank, lay = moe.pack_experts(w13, w2)
    B = lay["blob_bytes"]
    store = torch.empty((s.E, B), dtype=torch.uint8, pin_memory=True)
    store.copy_(bank.cpu())
    slots = torch.zeros((S, B), dtype=torch.uint8, device=DEV)
    cache = moe.SlotCache(s.E, S, B, store, slots)
    sim = LRUSlotCache(s.E, S)
    table = torch.full((s.E,), -1, dtype=torch.int32, device=DEV)
    main = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    done = torch.cuda.Event()
    ffn_done = torch.cuda.Event()
    ffn_done.record(main)
    ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k, moe.MODE_DECODE)
    xs = synth.ar1_activation_sequence(wl, T, seed_layer, steps, device="cpu")
    n_rounds = []
    prev = set()
    for st in range(steps):
        x = xs[st].to(DEV)
        if prefetch and prev:
            # the previous step's experts, copied ahead of this step's rounds
            n = cache.prefetch(prev, S, copy, ffn_done)
            assert n == len(sim.prefetch(prev, S)), st
        r = moe.moe_route(x, wr, s.k)
        a = moe.moe_align(r.ids, s.E)
        need = {w[0] for w in moe.active_experts(a)}
        prev = need
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
        slot_state, _, _ = cache.state()
        assert slot_state == sim.slot_expert
        # all experts resident, through an all-experts slot table: the same two-pass
        # kernels as the slot-cache calls, so the outputs agree bit for bit
        ident = torch.arange(s.E, dtype=torch.int32, device=DEV)
        ref_out = moe.moe_w4a16_grouped_ffn(x, r, a, bank, s.I, mode=moe.MODE_DECODE, slot_of_expert=ident)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"step {st}"
        n_rounds.append(rounds)
    hits, misses = cache.state()[1:]
    cache.close()
    return n_rounds, hits, misses


def test_slot_cache_tiny_rounds():
    say("slot cache tiny E=8 S=3")
    n_rounds, hits, misses = run_slot_steps(synth.TINY, 3, 6, 16)
    assert max(n_rounds) >= 2


def test_slot_cache_olmoe_zipf_16_slots():
    say("slot cache olmoe zipf S=16")
    n_rounds, hits, misses = run_slot_steps(synth.OLMOE_SLOT, 16, 6, 16)
    say(f"  rounds {n_rounds} hits {hits} misses {misses}")
    assert hits > 0 and misses > 0


def test_slot_cache_prefetch_olmoe_zipf_16_slots():
    say("slot cache prefetch olmoe zipf S=16")
    n_rounds, hits, misses = run_slot_steps(synth.OLMOE_SLOT, 16, 6, 16, prefetch=True)
    say(f"  rounds {n_rounds} hits {hits} misses {misses}")
    assert hits > 0


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
