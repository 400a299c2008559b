"""Benchmark: W4A16 grouped-expert MoE layers on one MI355X.

Workload: OLMoE-1B-7B-shaped decode, 16 MoE layers (d_model 2048, 64 experts,
top-8, expert intermediate 1024, SwiGLU), int4 symmetric group-128 experts with
bf16 scales, bf16 router and activations, all 64 experts of every layer
resident in HBM (16 x 207.6 MB).  One step = routing + grouped gate/up + SwiGLU
(one launch) -> grouped down + combine (one launch) for each of the 16 layers on
fresh activations, T tokens per step (headline T = 16).

Prints one JSON line: MoE-layer tokens/s (T * layers / step time, the median of 3
trials of K graph-replayed steps), the achieved algorithmic HBM GB/s, the roofline
of the dominant kernel (routing + grouped gate/up) timed with HIP events on its
own stream (its measured HBM traffic comes from the committed rocprofv3 counter
summary under profiles/ when that was taken on the current kernel sources), a
batched-prefill layer (T = 4096) with the MFMA roofline of its grouped gate/up
kernel, the other workloads, and the cpu_baseline leg: the CPU oracle timed on a
bounded sample of the decode workload on the host's cores, and a parity verdict
per configuration (layer 0 of each, every token, against the oracle).  A raised
routing-wait flag of moe_decode_layer stops the run; a failed parity verdict
makes it exit non-zero after printing the line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_T_START = time.time()


def progress(msg):
    """One line on stderr as each part of the run ends (stdout carries only the JSON line)."""
    print(f"[bench {time.time() - _T_START:6.1f} s] {msg}", file=sys.stderr, flush=True)


METRIC = "MoE-layer tokens/s + achieved HBM GB/s (W4A16, OLMoE shape, T=1..4096)"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# HBM counters of the roofline kernel (routing + grouped gate/up of moe_decode_layer)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "routing_gateup_decode_olmoe_t16_hbm_counters.txt")
COUNTED_SOURCES = ["w4a16_grouped_expert_amd/csrc/layer_gateup.hpp", "w4a16_grouped_expert_amd/csrc/ffn_layer.hip",
                   "w4a16_grouped_expert_amd/csrc/ffn_common.hpp", "w4a16_grouped_expert_amd/csrc/common.hpp",
                   "w4a16_grouped_expert_amd/csrc/align_block.hpp", "w4a16_grouped_expert_amd/csrc/route_rank.hpp",
                   "w4a16_grouped_expert_amd/csrc/mat_format.hpp", "w4a16_grouped_expert_amd/csrc/down_combine.hpp"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--tokens", type=int, default=16, help="tokens per decode step (headline 16)")
    p.add_argument("--sweep", default="1,4", help="extra decode T values reported beside the headline")
    p.add_argument("--x-sets", type=int, default=8, help="distinct activation sets cycled over steps")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU-oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--prefill-tokens", type=int, default=4096, help="tokens of the prefill measurement (0: skip)")
    p.add_argument("--prefill-sweep", default="512", help="extra prefill T values")
    p.add_argument("--no-large", action="store_true", help="skip the large-expert shape")
    p.add_argument("--no-slot-cache", action="store_true", help="skip the 16-slot cache workload")
    p.add_argument("--no-ablation", action="store_true", help="skip the fused vs per-expert ablation")
    p.add_argument("--no-bf16", action="store_true", help="skip the BF16-expert comparison")
    p.add_argument("--no-mat", action="store_true", help="skip the nested two/four-bit comparison")
    p.add_argument("--two-call", action="store_true",
                   help="decode steps through moe_route_align + moe_w4a16_grouped_ffn instead of moe_decode_layer")
    p.add_argument("--slot-steps", type=int, default=24, help="timed steps of the slot-cache workload")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of known size (for HBM counter calibration)")
    return p.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


def host_facts():
    """CPU model, physical cores and the logical CPUs this process may run on."""
    model, cores = "unknown", set()
    phys = core = None
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k == "model name" and model == "unknown":
                model = v
            elif k == "physical id":
                phys = v
            elif k == "core id":
                core = v
            elif not k and phys is not None and core is not None:
                cores.add((phys, core))
                phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    usable = min(avail, int(cap)) if cap.isdigit() and int(cap) > 0 else avail
    return {"cpu_model": model, "physical_cores": len(cores) or None, "logical_cpus_available": avail,
            "threads_allowed": usable}


class Decoder:
    """16 resident MoE layers with shared per-step buffers: four-bit experts, or
    (bf16=True) the same experts unquantised for the W4 versus BF16 comparison."""

    def __init__(self, wl, T_max, device, bf16=False, mat=False, fused=True):
        import torch
        import synth
        import w4a16_grouped_expert_amd as moe
        self.moe, self.torch = moe, torch
        s = wl.shape
        self.wl, self.s, self.bf16, self.mat, self.tau = wl, s, bf16, mat, 0.0
        # steps of at most 16 tokens on four-bit or nested experts: the whole layer
        # in two launches (moe_decode_layer, moe_mat_decode_layer); else
        # moe_route_align + the grouped FFN call
        self.fused = fused and not bf16
        self.layers = []
        for l in range(wl.layers):
            w13, w2 = synth.expert_weights(wl, l, device=device)
            if bf16:
                bank = moe.pack_bf16_experts(w13, w2)
            else:
                bank, lay = moe.pack_experts(w13, w2)
                if mat:
                    bank = moe.mat_from_w4(bank, s.d, s.I)
            del w13, w2
            wr = synth.router_weight(wl, l, device="cpu").to(device)
            self.layers.append((wr, bank))
        torch.cuda.synchronize()
        self.blob_bytes = moe.bf16_expert_bytes(s.d, s.I) if bf16 else lay["blob_bytes"]
        self.T_max = T_max
        self.route = moe.alloc_route(T_max, s.E, s.k, device)
        self.align = moe.alloc_align(T_max, s.k, s.E, device)
        self.counter = moe.alloc_counter(device)
        need = max(max(moe.ffn_workspace_bytes(t, s.d, s.I, s.E, s.k), moe.ffn_workspace_bytes(t, s.d, s.I, s.E, s.k, moe.MODE_DECODE))
                   for t in range(1, T_max + 1))
        self.ws = torch.empty(need, dtype=torch.uint8, device=device)
        self.out = [torch.empty((T_max, s.d), dtype=torch.bfloat16, device=device) for _ in range(wl.layers)]
        if self.fused:
            t_l = min(T_max, 16)
            self.lws = torch.empty(moe.decode_layer_workspace_bytes(t_l, s.d, s.I, s.E, s.k), dtype=torch.uint8,
                                   device=device)
            self.lctr = moe.alloc_layer_counters(device)

    def uses_layer(self, T):
        return self.fused and T <= 16

    def check_wait_flag(self, where):
        """moe_decode_layer raises its last counter when a workgroup gave up waiting
        for the routing (its outputs are then invalid): a step timed with that flag
        up is not a valid measurement, so the run stops."""
        if not self.fused:
            return 0
        self.torch.cuda.synchronize()
        flag = int(self.lctr[-1].item())
        if flag:
            raise SystemExit(f"bench.py: moe_decode_layer routing wait timed out during {where} "
                             f"(flag {flag}); results invalid")
        return flag

    def layer(self, l, x):
        moe, s = self.moe, self.s
        T = x.shape[0]
        wr, bank = self.layers[l]
        r = moe.RouteOut(self.route.logits[:T], self.route.ids[:T], self.route.weights[:T])
        if self.uses_layer(T):
            if self.mat:
                moe.moe_mat_decode_layer_into(x, wr, bank, s.I, s.k, r, self.out[l][:T], self.lws, self.lctr,
                                              self.tau)
            else:
                moe.moe_decode_layer_into(x, wr, bank, s.I, s.k, r, self.out[l][:T], self.lws, self.lctr)
            return None
        a = moe.AlignOut(self.align.offsets, self.align.sorted_pairs[:T * s.k], self.align.pair_pos[:T * s.k],
                         self.align.active, None, 0)
        moe.moe_route_align_into(x, wr, s.k, r, a, self.counter)
        if self.bf16:
            moe.moe_bf16_grouped_ffn_into(x, r, a, bank, s.I, self.out[l][:T], self.ws)
        elif self.mat:
            moe.moe_mat_grouped_ffn_into(x, r, a, bank, s.I, self.out[l][:T], self.ws, self.tau)
        else:
            moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, s.I, self.out[l][:T], self.ws)
        return a

    def step(self, xs):
        for l, x in enumerate(xs):
            self.layer(l, x)

    def distinct_experts(self, xs):
        """Active experts per layer for this step (untimed pre-pass)."""
        us = []
        for l, x in enumerate(xs):
            self.layer(l, x)
            us.append(int(self.torch.unique(self.route.ids[:x.shape[0]]).numel()))
        return us


def run_ablation(dec, T, steps, x_sets=4):
    """Fused grouped execution against the same kernels launched one expert at a
    time: per layer the step's active experts are read back to the host (the loop
    over experts needs them there) and each runs as its own grouped-FFN call with
    an expert->slot table that keeps only that expert; the last call also runs
    the combine.  Both variants eager, K steps each, HIP events around the steps."""
    import torch
    import synth
    moe, s, wl = dec.moe, dec.s, dec.wl
    xs = [[synth.activations(wl, T, l, step=st, device="cuda") for l in range(wl.layers)] for st in range(x_sets)]
    only = torch.full((s.E, s.E), -1, dtype=torch.int32, device="cuda")
    only[torch.arange(s.E), torch.arange(s.E)] = torch.arange(s.E, dtype=torch.int32, device="cuda")

    def seq_step(xl, known=None):
        """known: the active experts of every layer (graph capture, no read-back)"""
        used = []
        for l, x in enumerate(xl):
            wr, bank = dec.layers[l]
            r = moe.RouteOut(dec.route.logits[:T], dec.route.ids[:T], dec.route.weights[:T])
            a = moe.AlignOut(dec.align.offsets, dec.align.sorted_pairs[:T * s.k], dec.align.pair_pos[:T * s.k],
                             dec.align.active, None, 0)
            moe.moe_route_align_into(x, wr, s.k, r, a, dec.counter)
            if known is None:
                act = a.active[:4 + 4 * s.E].cpu()
                experts = act[4::4][:int(act[0])].tolist()
            else:
                experts = known[l]
            for i, e in enumerate(experts):
                moe.moe_w4a16_grouped_ffn_into(x, r, a, bank, s.I, dec.out[l][:T], dec.ws,
                                               combine=(i == len(experts) - 1), slot_of_expert=only[e])
            used.append(experts)
        return used

    def timed(fn):
        for i in range(2):
            fn(xs[i % x_sets])
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            fn(xs[i % x_sets])
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    fused = timed(dec.step)
    seq = timed(seq_step)
    known = [seq_step(xl) for xl in xs]
    calls = sum(len(e) for e in known[0]) / wl.layers
    # both again from HIP graphs (the per-expert variant captured with each step's
    # experts known in advance): kernel time and launch gaps only, no host loop
    fused_graphs = capture_graphs(dec, xs)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for xl, kn in zip(xs, known):
            seq_step(xl, kn)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    seq_graphs = []
    for xl, kn in zip(xs, known):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            seq_step(xl, kn)
        seq_graphs.append(g)
    torch.cuda.synchronize()

    def replay(graphs):
        return lambda xl: graphs[[id(v) for v in xs].index(id(xl))].replay()

    fused_g = timed(replay(fused_graphs))
    seq_g = timed(replay(seq_graphs))
    del fused_graphs, seq_graphs
    return {"T": T, "expert_calls_per_layer": round(calls, 1),
            "eager": {"fused_ms_per_step": round(fused, 4), "sequential_ms_per_step": round(seq, 4),
                      "speedup": round(seq / fused, 3)},
            "graph": {"fused_ms_per_step": round(fused_g, 4), "sequential_ms_per_step": round(seq_g, 4),
                      "speedup": round(seq_g / fused_g, 3)},
            "fused_tokens_per_s": round(T * wl.layers / (fused_g * 1e-3), 1),
            "sequential_tokens_per_s": round(T * wl.layers / (seq_g * 1e-3), 1)}


def run_bf16_compare(Ts, steps, warmup, x_sets, w4_tokens_per_s):
    """The same 16-layer decode with the experts unquantised (BF16 blobs, 3.88x the
    bytes of the four-bit ones): tokens/s and HBM rate from HIP-graph replays,
    and the four-bit speedup at each T."""
    import torch
    import synth
    wl = synth.OLMOE_DECODE
    dec = Decoder(wl, max(Ts), "cuda", bf16=True)
    res = {}
    for T in Ts:
        r = run_decode(dec, T, steps, warmup, x_sets, timed_kernels=("gateup_bf16", "down_bf16", "combine", "route"))
        s = dec.s
        layer_bytes = r["mean_distinct_experts"] * dec.blob_bytes + s.E * s.d * 2 + 2 * T * s.d * 2
        res[f"T={T}"] = {"tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 4),
                         "hbm_gbps": round(layer_bytes * wl.layers / (r["ms_per_step"] * 1e-3) / 1e9, 1),
                         "kernels_us": {k: round(v["avg_us"], 3) for k, v in r["kernels"].items()},
                         "w4_speedup": round(w4_tokens_per_s[T] / r["tokens_per_s"], 3)}
    del dec
    torch.cuda.empty_cache()
    return {"workload": "olmoe_decode with BF16 experts (12.58 MB each, row-major, same route/align/combine)",
            "pages_w4_over_bf16": round(31.923 / 21.662, 3), "bytes_ratio": 3.879, **res}


def run_mat_compare(Ts, taus, steps, warmup, x_sets, w4_tokens_per_s):
    """Nested two/four-bit experts (layout m1): the same 16-layer decode with each
    expert's precision from its routing weights (four bits when its largest weight
    reaches tau); per T and tau the tokens/s from HIP graphs, the share of experts
    at four bits and the weight bytes read, against the four-bit path."""
    import torch
    import synth
    wl = synth.OLMOE_DECODE
    s = wl.shape
    dec = Decoder(wl, max(Ts), "cuda", mat=True)
    res = {}
    for T in Ts:
        xs = [[synth.activations(wl, T, l, step=st, device="cuda") for l in range(wl.layers)] for st in range(x_sets)]
        for tau in taus:
            dec.tau = tau
            kern = ("gateup_decode", "down_decode") if dec.uses_layer(T) else ("gateup_mat", "down_mat", "combine",
                                                                                  "route")
            r = run_decode(dec, T, steps, warmup, x_sets, timed_kernels=kern)
            # share of the step's experts at four bits (same decision as the kernels, from the routing weights)
            n4 = n = 0
            for xl in xs[:2]:
                for l, x in enumerate(xl):
                    dec.layer(l, x)
                    ids = dec.route.ids[:T].reshape(-1).long()
                    act = torch.unique(ids)
                    wmax = torch.zeros(s.E, device="cuda").scatter_reduce(
                        0, ids, dec.route.weights[:T].reshape(-1), "amax")
                    n4 += int((wmax[act] >= tau).sum())
                    n += int(act.numel())
            frac4 = n4 / max(1, n)
            res[f"T={T} tau={tau}"] = {
                "tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 4),
                "experts_at_four_bits": round(frac4, 3),
                "kernels_us": {k: round(v["avg_us"], 3) for k, v in r["kernels"].items()},
                "vs_w4": round(r["tokens_per_s"] / w4_tokens_per_s[T], 3)}
    del dec
    torch.cuda.empty_cache()
    return {"workload": "olmoe_decode with nested two/four-bit experts (layout m1) through the fused two-launch "
                        "decode layer (moe_mat_decode_layer, as the four-bit path); four bits when an expert's "
                        "largest routing weight in the step reaches tau, else two bits (high plane only, floor "
                        "plus compensation)", **res}


def expert_section_bytes(d, I):
    codes13, scales13 = 2 * I * d // 2, 2 * I * (d // 128) * 2
    codes2, scales2 = d * I // 2, d * (I // 128) * 2
    return codes13 + scales13, codes2 + scales2


def capture_graphs(dec, xs_sets):
    """One HIP graph per activation set, each holding a whole 16-layer step."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for xs in xs_sets:
            dec.step(xs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for xs in xs_sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dec.step(xs)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def run_decode(dec, T, steps, warmup, x_sets, timed_kernels=("gateup_decode", "down_decode", "combine", "route",
                                                              "align"), trials=3):
    """Time K steps replayed from HIP graphs, in `trials` trials (value: the median
    trial), then K eager steps with the dominant kernels bracketed by HIP events on
    their stream (roofline).  After each leg the routing-wait flag of
    moe_decode_layer is read; a raised flag stops the run."""
    import torch
    import synth
    moe = dec.moe
    wl, s = dec.wl, dec.s
    xs = [[synth.activations(wl, T, l, step=st, device="cuda") for l in range(wl.layers)] for st in range(x_sets)]
    U = [dec.distinct_experts(x) for x in xs]
    dec.check_wait_flag(f"the T={T} pre-pass")
    graphs = capture_graphs(dec, xs)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(warmup):
        graphs[i % x_sets].replay()
    torch.cuda.synchronize()
    trial_ms = []
    for _ in range(max(1, trials)):
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            graphs[i % x_sets].replay()
        t1.record()
        torch.cuda.synchronize()
        trial_ms.append(t0.elapsed_time(t1) / steps)
    ms = sorted(trial_ms)[len(trial_ms) // 2]
    del graphs
    dec.check_wait_flag(f"the T={T} graph replays")

    for i in range(warmup):
        dec.step(xs[i % x_sets])
    torch.cuda.synchronize()
    moe.timing_reset()
    moe.timing_enable(True)
    t0.record()
    for i in range(steps):
        dec.step(xs[i % x_sets])
    t1.record()
    torch.cuda.synchronize()
    moe.timing_enable(False)
    ms_eager = t0.elapsed_time(t1) / steps
    dec.check_wait_flag(f"the T={T} eager steps")
    res = {"T": T, "ms_per_step": ms, "ms_per_step_eager": ms_eager, "trial_ms_per_step": trial_ms, "kernels": {}}
    for kname in timed_kernels:
        tot, n = moe.timing_read(kname)
        if n:
            res["kernels"][kname] = {"avg_us": 1e3 * tot / n, "launches": n}
    used = [U[i % x_sets] for i in range(steps)]
    u_mean = sum(sum(u) for u in used) / (steps * wl.layers)
    b13, b2 = expert_section_bytes(s.d, s.I)
    router = s.E * s.d * 2
    io = 2 * T * s.d * 2
    layer_bytes = u_mean * (b13 + b2) + router + io
    res["mean_distinct_experts"] = u_mean
    res["layer_bytes"] = layer_bytes
    res["tokens_per_s"] = T * wl.layers / (ms * 1e-3)
    res["hbm_gbps"] = layer_bytes * wl.layers / (ms * 1e-3) / 1e9
    # dominant kernel: grouped gate/up; algorithmic bytes per launch = distinct experts x
    # (W13 codes + scales) + activations read + h written (bf16)
    gu_bytes = u_mean * b13 + T * s.d * 2 + T * s.k * s.I * 2
    if dec.uses_layer(T):
        gu_bytes += router  # the same launch computes the routing
    res["gateup_bytes_per_launch"] = gu_bytes
    return res


def measured_traffic():
    """HBM bytes per launch of the decode roofline kernel from the committed rocprofv3
    counter summary, if it was taken on the kernel sources as they are now."""
    import hashlib
    try:
        kv = {}
        for line in open(COUNTERS_FILE):
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in COUNTED_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if kv.get("source_sha256") != h.hexdigest():
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def run_prefill(T, reps=20, warmup=3):
    """One OLMoE-shaped layer at T tokens (batched prefill, uniform router): eager
    forward passes with HIP events around each kernel; MFMA roofline of the grouped
    gate/up kernel from its algorithmic flops (2 * T * k * d * 2I per launch)."""
    import torch
    import synth
    import w4a16_grouped_expert_amd as moe
    wl = synth.OLMOE_PREFILL
    s = wl.shape
    w13, w2 = synth.expert_weights(wl, 0, device="cuda")
    bank, _ = moe.pack_experts(w13, w2)
    del w13, w2
    wr = synth.router_weight(wl, 0, device="cpu").cuda()
    x = synth.activations(wl, T, 0, device="cuda")
    layer = moe.MoELayer(wr, bank, s.I, s.k, T)
    for _ in range(warmup):
        layer.forward(x)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    moe.timing_reset()
    moe.timing_enable(True)
    t0.record()
    for _ in range(reps):
        layer.forward(x)
    t1.record()
    torch.cuda.synchronize()
    moe.timing_enable(False)
    ms = t0.elapsed_time(t1) / reps
    kern = {}
    for kname in ("route", "align", "gateup_prefill", "down_prefill", "combine"):
        tot, n = moe.timing_read(kname)
        if n:
            kern[kname] = round(1e3 * tot / n, 3)
    P = T * s.k
    fl_gu, fl_dn = 2.0 * P * s.d * 2 * s.I, 2.0 * P * s.I * s.d
    gu = fl_gu / (kern["gateup_prefill"] * 1e-6) / 1e12
    dn = fl_dn / (kern["down_prefill"] * 1e-6) / 1e12
    del layer, bank
    torch.cuda.empty_cache()
    return {"workload": f"olmoe_prefill: 1 MoE layer, d=2048, E=64, top-8, I=1024, W4 g128, T={T} tokens, "
                        "uniform router (about T*8/64 tokens per expert)",
            "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_layer": round(ms, 4), "kernels_us": kern,
            "down_tflops": round(dn, 1),
            "roofline": {"bound": "mfma", "kernel": "k_prefill (gate/up)", "achieved": round(gu, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(gu / MFMA_BF16_PEAK_TFLOPS, 4),
                         "flops_per_launch": fl_gu, "avg_us": kern["gateup_prefill"]}}


def run_large(Ts, reps=10, warmup=3):
    """Large-expert shape (d=4096, E=8, top-2, I=14336, 4 layers, all resident): per T
    the 4-layer step timed with HIP events (steps of at most 16 tokens through
    moe_decode_layer, as the OLMoE decode legs; more tokens through route, align,
    grouped FFN and combine); HBM fraction on algorithmic bytes (distinct experts x
    blob + router + activations) and MFMA fraction on flops."""
    import torch
    import synth
    import w4a16_grouped_expert_amd as moe
    wl = synth.LARGE
    s = wl.shape
    layers = []
    for l in range(wl.layers):
        w13, w2 = synth.expert_weights(wl, l, device="cuda")
        bank, lay = moe.pack_experts(w13, w2)
        del w13, w2
        wr = synth.router_weight(wl, l, device="cpu").cuda()
        layers.append(moe.MoELayer(wr, bank, s.I, s.k, max(Ts)))
    torch.cuda.empty_cache()
    blob = lay["blob_bytes"]
    t_l = min(16, max(Ts))
    lws = torch.empty(max(moe.decode_layer_workspace_bytes(t_l, s.d, s.I, s.E, s.k), 256), dtype=torch.uint8,
                      device="cuda")
    lctr = moe.alloc_layer_counters("cuda")
    res = {}
    for T in Ts:
        xs = [synth.activations(wl, T, l, device="cuda") for l in range(wl.layers)]

        def step():
            for L, x in zip(layers, xs):
                if T <= 16:
                    r, _ = L.views(T)
                    moe.moe_decode_layer_into(x, L.w_router, L.bank, s.I, s.k, r, L.out[:T], lws, lctr)
                else:
                    L.forward(x)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        if T <= 16:
            if int(lctr[-1].item()):
                raise SystemExit("bench.py: moe_decode_layer routing wait timed out (large expert); results invalid")
            U = []
            for L, x in zip(layers, xs):
                r, _ = L.views(T)
                moe.moe_decode_layer_into(x, L.w_router, L.bank, s.I, s.k, r, L.out[:T], lws, lctr)
                U.append(int(torch.unique(r.ids).numel()))
        else:
            U = [int(L.align.active[0].item()) for L in layers]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            step()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        by = sum(U) * blob + wl.layers * (s.E * s.d * 2 + 2 * T * s.d * 2)
        fl = wl.layers * T * (s.k * 6 * s.d * s.I + 2 * s.d * s.E)
        res[f"T={T}"] = {"tokens_per_s": round(T * wl.layers / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
                         "hbm_gbps": round(by / (ms * 1e-3) / 1e9, 1),
                         "hbm_frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "mean_distinct_experts": sum(U) / len(U)}
    del layers
    torch.cuda.empty_cache()
    return {"workload": "large_expert: 4 MoE layers, d=4096, E=8, top-2, I=14336, W4 g128 experts resident; "
                        "whole-step time per T (T <= 16: moe_decode_layer, two launches per layer; else route + "
                        "align + grouped FFN + combine)", **res}


def h2d_ceiling(store, slots, streams=2, reps=3):
    """Pinned host -> device copies of whole expert blobs, back to back, alternating
    over `streams` copy streams: the host-link rate the slot cache can reach."""
    import torch
    n = store.shape[0]
    ss = [torch.cuda.Stream() for _ in range(streams)]
    best = 1e9
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            with torch.cuda.stream(ss[i % streams]):
                slots[i % slots.shape[0]].copy_(store[i], non_blocking=True)
        torch.cuda.synchronize()
        best = min(best, time.perf_counter() - t0)
    return n * store.shape[1] / best / 1e9


SLOT_VARIANTS = (
    # name, slots, policy (0 LRU, 1 cost-aware), copy streams, next-layer prefetch copies per layer,
    # tau of the two-bit misses (None: four-bit experts only)
    ("S=16 lru 1-stream", 16, 0, 1, 0, None),
    ("S=16 lru 2-streams", 16, 0, 2, 0, None),
    ("S=16 cost-aware 2-streams", 16, 1, 2, 0, None),
    ("S=16 cost-aware 2-streams next-layer-prefetch", 16, 1, 2, 1, None),
    ("S=16 cost-aware 2-streams two-bit-misses tau=0.1", 16, 1, 2, 0, 0.1),
    ("S=16 cost-aware 2-streams two-bit-misses tau=0.14", 16, 1, 2, 0, 0.14),
    ("S=32 cost-aware 2-streams", 32, 1, 2, 0, None),
    ("S=32 cost-aware 2-streams next-layer-prefetch", 32, 1, 2, 4, None),
    ("S=64", 64, 0, 2, 0, None),
)


def run_slot_cache(steps, warmup=8, T=16, variants=SLOT_VARIANTS):
    """Expert slot cache (OLMoE shape, 16 layers, Zipf(1.2) popularity, AR(1) step
    locality and layer inputs correlated along the residual stream): experts in
    pinned host memory, S device slots per layer, misses copied by hipMemcpyAsync
    on one or two copy streams before each FFN round.  Variants: replacement policy
    (LRU / cost-aware), copy streams, and the next-layer prefetch: layer l+1's
    router applied to layer l's input predicts its experts (read back with layer
    l's routing in one sync) and up to N of them are copied into layer l+1's slots
    while layer l runs; and two-bit misses (page "MoE-APEX: An Efficient MoE
    Inference System with Adaptive Precision Expert Offloading", "This paper's
    idea"): the store holds nested two/four-bit blobs, an expert whose largest
    routing weight in the step is below tau is loaded as its two-bit prefix and run
    at two bits."""
    import numpy as np
    import torch
    import synth
    import w4a16_grouped_expert_amd as moe
    wl = synth.OLMOE_SLOT
    s = wl.shape
    need_mat = any(v[5] is not None for v in variants)
    stores, mat_stores = [], []
    for l in range(wl.layers):
        w13, w2 = synth.expert_weights(wl, l, device="cuda")
        bank, lay = moe.pack_experts(w13, w2)
        del w13, w2
        B = lay["blob_bytes"]
        store = torch.empty((s.E, B), dtype=torch.uint8, pin_memory=True)
        store.copy_(bank)
        if need_mat:
            mstore = torch.empty((s.E, B), dtype=torch.uint8, pin_memory=True)
            mstore.copy_(moe.mat_from_w4(bank, s.d, s.I))
            mat_stores.append(mstore)
        del bank
        stores.append((store, synth.router_weight(wl, l).cuda()))
    torch.cuda.empty_cache()
    prefix = moe.mat_layout(s.d, s.I)["two_bit_bytes"]
    probe_slots = torch.empty((16, B), dtype=torch.uint8, device="cuda")
    ceiling = {"one_stream_gbps": round(h2d_ceiling(stores[0][0], probe_slots, 1), 2),
               "two_streams_gbps": round(h2d_ceiling(stores[0][0], probe_slots, 2), 2)}
    del probe_slots
    route = moe.alloc_route(T, s.E, s.k, "cuda")
    pred = moe.alloc_route(T, s.E, s.k, "cuda")
    al = moe.alloc_align(T, s.k, s.E, "cuda")
    counter = moe.alloc_counter("cuda")
    ws = moe.alloc_workspace(T, s.d, s.I, s.E, s.k, moe.MODE_DECODE)
    out = torch.empty((T, s.d), dtype=torch.bfloat16, device="cuda")
    seqs = [[x.cuda() for x in row] for row in synth.residual_stream_sequence(wl, T, warmup + steps)]
    main = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    probe = []

    def one(S, policy, n_streams, n_pref, tau, capture_probe):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        mixed = tau is not None
        tau32 = float(np.float32(tau)) if mixed else 0.0
        layers = []
        copied = [0]
        deviation = []
        for li, (store, wr) in enumerate(stores):
            slots = torch.zeros((S, B), dtype=torch.uint8, device="cuda")
            cache = moe.SlotCache(s.E, S, B, mat_stores[li] if mixed else store, slots)
            cache.configure(policy, 0.9, n_streams)
            if mixed:
                cache.set_prefix(prefix)
            layers.append({"wr": wr, "slots": slots, "cache": cache,
                           "table": torch.full((s.E,), -1, dtype=torch.int32, device="cuda"),
                           "ffn_done": torch.cuda.Event()})
        done = torch.cuda.Event()
        for L in layers:
            L["ffn_done"].record(main)
        n_layers = len(layers)

        def step(st, capture=False):
            rounds = misses = pref = floor = 0
            for l, L in enumerate(layers):
                x = seqs[st][l]
                moe.moe_route_align_into(x, L["wr"], s.k, route, al, counter)
                full = None
                if n_pref and l + 1 < n_layers:
                    # the next layer's router on this layer's input: its predicted experts
                    moe.moe_route_into(x, layers[l + 1]["wr"], s.k, pred)
                    both = torch.cat([al.active, pred.ids.reshape(-1)]).cpu()  # the one D2H sync per layer
                    U = int(both[0])
                    need = {int(v) for v in both[4:4 + 4 * U:4]}
                    predicted = {int(v) for v in both[4 + 4 * s.E:]}
                elif mixed:
                    # routing ids and weights too: an expert runs at four bits when its
                    # largest routing weight reaches tau (the rule of the nested kernels)
                    both = torch.cat([al.active, route.ids[:T].reshape(-1),
                                      route.weights[:T].reshape(-1).view(torch.int32)]).cpu()
                    U = int(both[0])
                    need = {int(v) for v in both[4:4 + 4 * U:4]}
                    ids_h = both[4 + 4 * s.E:4 + 4 * s.E + T * s.k].numpy()
                    w_h = both[4 + 4 * s.E + T * s.k:].numpy().view(np.float32)
                    full = {e for e in need if np.max(w_h[ids_h == e]) >= np.float32(tau)}
                    predicted = None
                else:
                    need = {w[0] for w in moe.active_experts(al)}  # the one D2H sync per layer
                    predicted = None
                floor += max(0, len(need) - S)  # copies no policy avoids: the rounds cycle the needed set
                L["cache"].begin_step(need)
                pending = set(need)
                first = True
                while pending:
                    if mixed:
                        got, nh, nm, nb = L["cache"].load_precision(pending, full, L["table"], copy, L["ffn_done"],
                                                                    done)
                        copied[0] += nb
                    else:
                        got, nh, nm = L["cache"].load(pending, L["table"], copy, L["ffn_done"], done)
                        copied[0] += nm * B
                    if first and predicted is not None:
                        nxt = layers[l + 1]
                        n = nxt["cache"].prefetch(predicted, n_pref, copy, nxt["ffn_done"])
                        pref += n
                        copied[0] += n * B
                    first = False
                    main.wait_event(done)
                    pending -= got
                    if mixed:
                        moe.moe_mat_grouped_ffn_into(x, route, al, L["slots"], s.I, out, ws, tau32, not pending,
                                                     L["table"])
                    else:
                        moe.moe_w4a16_grouped_ffn_into(x, route, al, L["slots"], s.I, out, ws, moe.MODE_DECODE,
                                                       not pending, L["table"])
                    L["ffn_done"].record(main)
                    rounds += 1
                    misses += nm
                if capture and capture_probe and l == 0:
                    probe.append((x, out.clone(), route.ids[:T].clone()))
                if capture and mixed and l == 0:
                    # kept for the comparison with the four-bit layer after the timed steps
                    deviation.append((x, out.clone(), moe.RouteOut(route.logits[:T].clone(), route.ids[:T].clone(),
                                                                   route.weights[:T].clone()),
                                      moe.AlignOut(al.offsets.clone(), al.sorted_pairs.clone(),
                                                   al.pair_pos.clone(), al.active.clone(), None, 0)))
            return rounds, misses, pref, floor

        for st in range(warmup):
            step(st)
        torch.cuda.synchronize()
        h0 = [L["cache"].state()[1:] for L in layers]
        t0 = time.perf_counter()
        rounds = misses = pref = floor = 0
        for st in range(warmup, warmup + steps):
            if st == warmup:
                copied[0] = 0
            r, m, p, fl = step(st, capture=((capture_probe or mixed) and st == warmup + steps - 1))
            rounds += r
            misses += m
            pref += p
            floor += fl
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        h1 = [L["cache"].state()[1:] for L in layers]
        hits = sum(b[0] - a[0] for a, b in zip(h0, h1))
        miss = sum(b[1] - a[1] for a, b in zip(h0, h1))
        peak = torch.cuda.max_memory_allocated() - base
        up = sum(L["cache"].planes()[1] for L in layers) if mixed else 0
        for L in layers:
            L["cache"].close()
        del layers
        torch.cuda.empty_cache()
        gbps = copied[0] / sec / 1e9
        extra = {}
        if mixed:
            diff = None
            if deviation:
                # layer 0 of the last timed step at four bits (all-resident bank), untimed
                x0, o0, r0, a0 = deviation[0]
                w4 = torch.empty((s.E, B), dtype=torch.uint8, device="cuda")
                w4.copy_(stores[0][0])
                ref = moe.moe_w4a16_grouped_ffn(x0, r0, a0, w4, s.I, moe.MODE_DECODE).float()
                diff = float((o0.float() - ref).abs().max() / ref.abs().max())
                del w4
            extra = {"tau": tau, "low_plane_completions_total": int(up),
                     "layer0_last_step_rel_diff_vs_four_bit": round(diff, 5) if diff is not None else None}
        return {"tokens_per_s": round(steps * T * wl.layers / sec, 1), "ms_per_step": round(1e3 * sec / steps, 3),
                "hit_rate": round(hits / max(1, hits + miss), 4), "misses_per_step": round(miss / steps, 2),
                "miss_floor_per_step": round(floor / steps, 2),
                "prefetches_per_step": round(pref / steps, 2),
                "copies_per_step": round((miss + pref) / steps, 2),
                "rounds_per_layer": round(rounds / (steps * wl.layers), 3),
                "h2d_mb_per_step": round(copied[0] / steps / 1e6, 1),
                "h2d_gbps": round(gbps, 2), "h2d_frac_of_ceiling": round(gbps / ceiling["two_streams_gbps"], 3),
                "slot_bytes_per_layer": S * B, "slot_bytes_total": S * B * wl.layers,
                "peak_device_bytes_during_run": int(peak), **extra}

    res = {"workload": f"olmoe_slot: 16 MoE layers, d=2048, E=64, top-8, I=1024, W4 g128; 64 experts per layer in "
                       f"pinned host memory, S device slots per layer, Zipf(1.2) popularity, AR(1) step locality "
                       f"(0.9), layer inputs correlated along the residual stream (0.9), T={T}",
           "resident_bytes_all_experts": s.E * B * wl.layers,
           "h2d_ceiling": {**ceiling, "what": "back-to-back pinned copies of whole expert blobs (3.24 MB)"},
           "timing": "wall clock over the timed steps (host round trip per layer for the needed set included)"}
    for name, S, policy, n_streams, n_pref, tau in variants:
        res[name] = one(S, policy, n_streams, n_pref, tau, capture_probe=(name == variants[0][0]))
    del stores, mat_stores
    torch.cuda.empty_cache()
    # layer 0 of the last timed step of the first variant (input, output, routing) for the parity check
    probe = [(x.cpu(), o.cpu(), ids.cpu().numpy()) for x, o, ids in probe[:1]]
    return res, (probe[0] if probe else None)


def _bits(t):
    import numpy as np
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _oracle_bank(wl, layer, experts, threads):
    """Oracle dequantised bank of the listed experts of one layer (drawn on the GPU
    with the bench's seeds, dequantised on `threads` host threads, untimed)."""
    from concurrent.futures import ThreadPoolExecutor
    import synth
    from oracle import ffn as offn
    experts = sorted(experts)
    w13, w2 = synth.expert_weights(wl, layer, device="cuda", experts=experts)
    host13 = {e: _bits(w13[i]) for i, e in enumerate(experts)}
    host2 = {e: _bits(w2[i]) for i, e in enumerate(experts)}
    del w13, w2
    bank = offn.DequantBank(lambda e: host13[e], lambda e: host2[e])
    with ThreadPoolExecutor(max_workers=max(1, min(threads, len(experts)))) as ex:
        list(ex.map(bank.get, experts))
    return bank


def cpu_baseline(wl, T, budget_s, threads, bank=None):
    """The CPU oracle on a bounded sample of the same workload: one OLMoE-shaped
    layer at T tokens (route, align, per-pair SwiGLU FFN in float64, combine),
    repeated until the time budget is used, its matrix products on `threads` host
    threads.  The experts' quantise/dequantise is done up front and not timed, as
    the GPU path packs its weights offline."""
    import synth
    from oracle import ffn as offn
    from oracle import route as oroute
    from threadpoolctl import threadpool_limits
    layer = 0
    wr = _bits(synth.router_weight(wl, layer))
    x = _bits(synth.activations(wl, T, layer, step=0))
    used = sorted(set(oroute.route(x, wr, wl.shape.k)[1].reshape(-1).tolist()))
    if bank is None:
        bank = _oracle_bank(wl, layer, used, threads)
    calls, elapsed = 0, 0.0
    with threadpool_limits(limits=threads):
        while elapsed < budget_s or calls == 0:
            t0 = time.perf_counter()
            offn.moe_layer(x, wr, bank, wl.shape.k)
            elapsed += time.perf_counter() - t0
            calls += 1
    return {"value": round(calls * T / elapsed, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"1 OLMoE-shaped layer (d=2048, E=64, top-8, I=1024) at T={T}, {len(used)} distinct "
                      f"experts, run {calls} times in {elapsed:.1f} s (float64 numpy oracle, matrix products on "
                      f"{threads} threads; expert dequantisation done beforehand, untimed)"}


def _errs(got, ref):
    import numpy as np
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    whole = float(np.max(np.abs(got - ref)) / den) if den > 0 else float(np.max(np.abs(got)))
    rden = np.max(np.abs(ref), axis=1)
    rnum = np.max(np.abs(got - ref), axis=1)
    tok = float(np.max(np.where(rden > 0, rnum / np.where(rden > 0, rden, 1.0), rnum)))
    return whole, tok, bool(np.all(np.isfinite(got)))


def parity_verdicts(args, threads, slot_probe=None):
    """Part of the cpu_baseline leg: for each measured configuration, layer 0 of its
    bank run once more through the same entry points the timing used, every output
    token compared with the oracle on the same seeded inputs (routing ids bit-exact,
    max|gpu - ref| / max|ref| <= 1e-2 over the layer and for every token on its
    own).  Returns ({config: verdict}, oracle bank of the decode layer)."""
    import numpy as np
    import torch
    import synth
    import w4a16_grouped_expert_amd as moe
    from oracle import ffn as offn
    from oracle import route as oroute
    from threadpoolctl import threadpool_limits
    tol = 1e-2
    res = {}

    def verdict(name, wl, bank_o, x, wr, out, ids):
        with threadpool_limits(limits=threads):
            ref = offn.moe_layer(_bits(x), _bits(wr), bank_o, wl.shape.k)
        whole, tok, finite = _errs(out.float().cpu().numpy(), ref["out"])
        ids_eq = bool(np.array_equal(ids.cpu().numpy(), ref["ids"]))
        res[name] = {"tokens_compared": int(x.shape[0]), "ids_bit_exact": ids_eq, "max_rel_err": round(whole, 6),
                     "worst_token_rel_err": round(tok, 6),
                     "pass": bool(ids_eq and finite and whole <= tol and tok <= tol)}
        progress(f"parity {name}: {'pass' if res[name]['pass'] else 'FAIL'}")

    def used_experts(wl, xs):
        wr = _bits(synth.router_weight(wl, 0))
        u = set()
        for x in xs:
            u |= set(oroute.route(_bits(x), wr, wl.shape.k)[1].reshape(-1).tolist())
        return u

    def gpu_bank(wl):
        w13, w2 = synth.expert_weights(wl, 0, device="cuda")
        bank, _ = moe.pack_experts(w13, w2)
        del w13, w2
        return bank

    # decode (the headline and the sweep): moe_decode_layer, as timed
    wl = synth.OLMOE_DECODE
    s = wl.shape
    Ts = sorted({args.tokens} | {int(t) for t in args.sweep.split(",") if t})
    xs = {T: synth.activations(wl, T, 0, step=0) for T in Ts}
    dec_bank = _oracle_bank(wl, 0, used_experts(wl, xs.values()), threads)
    bank = gpu_bank(wl)
    wr = synth.router_weight(wl, 0)
    for T in Ts:
        xd = xs[T].cuda()
        if T <= 16 and not args.two_call:
            out, r = moe.moe_decode_layer(xd, wr.cuda(), bank, s.I, s.k)
        else:
            L = moe.MoELayer(wr.cuda(), bank, s.I, s.k, T)
            out = L.forward(xd)
            r = L.route
        torch.cuda.synchronize()
        verdict(f"olmoe_decode T={T}", wl, dec_bank, xs[T], wr, out, r.ids[:T])
    del bank
    # prefill: route + align + grouped FFN, as timed
    if args.prefill_tokens > 0:
        wl = synth.OLMOE_PREFILL
        s = wl.shape
        Ts = sorted({args.prefill_tokens} | {int(t) for t in args.prefill_sweep.split(",") if t})
        xs = {T: synth.activations(wl, T, 0) for T in Ts}
        bank_o = _oracle_bank(wl, 0, range(s.E), threads)
        bank = gpu_bank(wl)
        wr = synth.router_weight(wl, 0)
        for T in Ts:
            L = moe.MoELayer(wr.cuda(), bank, s.I, s.k, T)
            out = L.forward(xs[T].cuda())
            torch.cuda.synchronize()
            verdict(f"olmoe_prefill T={T}", wl, bank_o, xs[T], wr, out, L.route.ids[:T])
            del L
        del bank, bank_o
    # large expert
    if not args.no_large:
        wl = synth.LARGE
        s = wl.shape
        xs = {T: synth.activations(wl, T, 0) for T in wl.tokens}
        bank_o = _oracle_bank(wl, 0, used_experts(wl, xs.values()), threads)
        bank = gpu_bank(wl)
        wr = synth.router_weight(wl, 0)
        for T in wl.tokens:
            L = moe.MoELayer(wr.cuda(), bank, s.I, s.k, T)
            out = L.forward(xs[T].cuda())
            torch.cuda.synchronize()
            verdict(f"large_expert T={T}", wl, bank_o, xs[T], wr, out, L.route.ids[:T])
            del L
        del bank, bank_o
    # slot cache: layer 0's output of the last timed step of the S=16 run
    if slot_probe is not None:
        wl = synth.OLMOE_SLOT
        x, out, ids = slot_probe
        bank_o = _oracle_bank(wl, 0, set(ids.reshape(-1).tolist()), threads)
        verdict("olmoe_slot S=16 lru (last timed step, layer 0)", wl, bank_o, x, synth.router_weight(wl, 0), out,
                torch.from_numpy(ids))
    torch.cuda.empty_cache()
    return res, dec_bank


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(sharding the layer over several GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import synth
    wl = synth.OLMOE_DECODE
    s = wl.shape
    Ts = sorted({args.tokens} | {int(t) for t in args.sweep.split(",") if t})
    dec = Decoder(wl, max(Ts), "cuda", fused=not args.two_call)
    head = run_decode(dec, args.tokens, args.steps, args.warmup, args.x_sets)
    progress(f"decode T={args.tokens}: {head['tokens_per_s']:.0f} tok/s")
    sweep = {}
    for T in Ts:
        if T == args.tokens:
            continue
        r = run_decode(dec, T, args.steps, args.warmup, args.x_sets)
        progress(f"decode T={T}: {r['tokens_per_s']:.0f} tok/s")
        sweep[f"T={T}"] = {k: r[k] for k in ("tokens_per_s", "hbm_gbps", "ms_per_step", "ms_per_step_eager",
                                             "mean_distinct_experts")}
        if "gateup_decode" in r.get("kernels", {}):
            kt = r["kernels"]["gateup_decode"]["avg_us"]
            sweep[f"T={T}"]["gateup_gbps"] = r["gateup_bytes_per_launch"] / (kt * 1e-6) / 1e9
    kern = head["kernels"]["gateup_decode"]
    achieved = head["gateup_bytes_per_launch"] / (kern["avg_us"] * 1e-6) / 1e9
    kname = ("k_layer_gateup (routing + grouped gate/up)" if dec.uses_layer(args.tokens)
             else "k_gateup_dense (grouped gate/up)")
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(), "avg_us": round(kern["avg_us"], 3),
                "bytes_per_launch": int(head["gateup_bytes_per_launch"])}
    out = {
        "metric": METRIC,
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "ms_per_step_eager": round(head["ms_per_step_eager"], 4),
        "trials": len(head["trial_ms_per_step"]),
        "trial_ms_per_step": [round(t, 4) for t in head["trial_ms_per_step"]],
        "timing": "value: the median of 3 trials, each timing K steps replayed from HIP graphs (one per "
                  "activation set); roofline: K steps run eagerly with HIP events around each grouped "
                  "gate/up launch on its stream",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, random-init; no trained checkpoint)",
        "config": {"workload": f"olmoe_decode: 16 MoE layers, d=2048, E=64, top-8, I=1024, SwiGLU, "
                               f"W4 g128 experts all resident, T={args.tokens} tokens/step",
                   "tokens_per_step": args.tokens, "layers": wl.layers},
        "hbm_gbps": round(head["hbm_gbps"], 1),
        "hbm_frac": round(head["hbm_gbps"] / HBM_PEAK_GBPS, 4),
        "mean_distinct_experts": round(head["mean_distinct_experts"], 2),
        "roofline": roofline,
        "kernels_us": {k: round(v["avg_us"], 3) for k, v in head["kernels"].items()},
        "routing_wait_timeouts": 0,  # moe_decode_layer's flag, read after every leg (a raised flag stops the run)
        "decode_sweep": sweep,
    }
    if not args.no_ablation:
        out["ablation_fused_vs_sequential"] = {
            "what": "same W4 kernels, all selected experts in one grouped call vs one call per expert, "
                    "steps of 16 layers; eager: the per-expert loop reads each layer's experts back to "
                    "the host; graph: both replayed from HIP graphs (the pages report 1.97x for their "
                    "fused kernels)",
            **{f"T={T}": run_ablation(dec, T, max(4, args.steps // 5)) for T in (args.tokens, 1)}}
        progress("fused vs per-expert ablation")
    del dec
    torch.cuda.empty_cache()
    w4 = {args.tokens: head["tokens_per_s"]}
    w4.update({int(k[2:]): v["tokens_per_s"] for k, v in sweep.items()})
    if not args.no_bf16:
        out["bf16_experts"] = run_bf16_compare(sorted(w4), args.steps, args.warmup, args.x_sets, w4)
        progress("bf16 experts")
    if not args.no_mat:
        out["nested_2_4_bit"] = run_mat_compare([t for t in (args.tokens, 1) if t in w4], (0.0, 0.14, 2.0),
                                                args.steps, args.warmup, args.x_sets, w4)
        progress("nested two/four-bit experts")
    if args.prefill_tokens > 0:
        out["prefill"] = run_prefill(args.prefill_tokens)
        progress(f"prefill T={args.prefill_tokens}")
        extra = {}
        for T in [int(t) for t in args.prefill_sweep.split(",") if t]:
            r = run_prefill(T)
            progress(f"prefill T={T}")
            extra[f"T={T}"] = {k: r[k] for k in ("tokens_per_s", "ms_per_layer", "kernels_us")}
            extra[f"T={T}"]["gateup_mfma_frac"] = r["roofline"]["frac"]
        if extra:
            out["prefill_sweep"] = extra
    if not args.no_large:
        out["large_expert"] = run_large(synth.LARGE.tokens)
        progress("large expert")
    slot_probe = None
    if not args.no_slot_cache:
        out["slot_cache"], slot_probe = run_slot_cache(args.slot_steps)
        progress("slot cache")
    ok = True
    if not args.no_cpu_baseline:
        host = host_facts()
        threads = host["threads_allowed"]
        verdicts, dec_bank = parity_verdicts(args, threads, slot_probe)
        ok = all(v["pass"] for v in verdicts.values())
        out["parity"] = {"bar": "routing ids bit-exact; max|gpu - oracle| / max|oracle| <= 1e-2 over the layer "
                                "and for every token (bf16 outputs vs the float64 oracle on identical "
                                "dequantised weights); layer 0 of each configuration, every token",
                         "all_pass": ok, "configs": verdicts}
        out["cpu_baseline"] = cpu_baseline(wl, args.tokens, args.cpu_seconds, threads, bank=dec_bank)
        progress("cpu baseline")
        out["cpu_baseline"]["host"] = host
    print(json.dumps(out))
    if not ok:
        print("bench.py: parity against the oracle failed for " +
              ", ".join(k for k, v in out["parity"]["configs"].items() if not v["pass"]), file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
