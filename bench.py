"""Benchmark of the cross-layer KV-sharing hot path on one MI355X.

Headline step (the mid-context decode workload: B=8, T=4096, 32 query / 8 KV
heads, D=128, bf16, 16 cross-decoder layers on one shared cache): compose the
new token's K', V' row into the cache (n=1), then run the 16 cross layers'
decode attention (split pass + log-sum-exp merge) over that same cache.
``value`` is the algorithmic KV bytes the 16 decode calls must read (K' + V'
once per layer) per second of step time, the step captured once in a HIP
graph and replayed (as a serving loop issues it); the headline detail also
gives the same step with its 17 launches issued from the host one by one.

Further legs, reported in the same JSON line: the compose of the 32K-token
prefill workload's 15 composed self-decoder layers (GB/s) and the backward of
one such layer, the causal chunked prefill over that workload's global cache
(TFLOP/s over unmasked pairs), that prefill's cache path with and without the
early exit, the compose-on-read comparator, one self-decoder decode step over
16 layers (fused append against compose-then-decode), the two long-context
decodes (131K tokens x 4 sequences; 1M tokens), and the achievable-bandwidth
probes (plain streaming kernels of libyoco_ceiling.so with the decode's and
the compose's traffic patterns). Per-launch figures come from launches issued
back to back in a HIP graph (replay time / launches); HBM-served ones rotate
over enough distinct buffers that the 256 MB Infinity Cache holds none of a
launch's inputs.

cpu_baseline: the fp64 oracle (as it stands) timed on the host cores over a
bounded sample of the headline workload (a few of its decode layers).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "decode-attn KV GB/s (% HBM peak), prefill TFLOP/s (% bf16 MFMA), compose GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="all", help="all | headline | comma list of: compose,prefill,long,million,ceiling,cor,backward,self,early_exit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--cpu-units", action="store_true", help="also time the oracle on one unit of each other workload")
    ap.add_argument("--clock-seconds", type=float, default=1.5,
                    help="seconds of back-to-back prefill during which the engine clock is sampled (0: skip)")
    ap.add_argument("--reps", type=int, default=10, help="timed repetitions of each non-headline leg")
    ap.add_argument("--decode-splits", type=int, default=0, help="split count of the headline decodes (0: automatic)")
    ap.add_argument("--long-splits", type=int, default=0, help="split count of the long-context decodes (0: automatic)")
    return ap.parse_args()


def up(x, torch):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


class Flusher:
    """Evicts the next kernel's inputs from the 256 MB Infinity Cache (and the L2s)
    outside the timed region, by touching 1 GiB of scratch memory.

    mode "read" streams the scratch buffer with ordinary (cache-allocating) loads
    of the bandwidth probe: the caches end up holding clean lines of a buffer
    no kernel uses. mode "write" fills it (torch fill_): the caches end up full
    of dirty lines, which the next kernel's misses must first write back to
    HBM, so its "cold" time also pays for that write-back."""

    def __init__(self, torch, mode="read"):
        self.mode = mode
        self.buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        if mode == "read":
            from cross_layer_shared_amd import ceiling as C
            self.buf.fill_(1.0)
            self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")
            self.read = lambda: C.yoco_ceiling_read(self.buf, self.sink, workgroups=0, threads=512,
                                                    nontemporal=False)

    def __call__(self):
        if self.mode == "read":
            self.read()
        else:
            self.buf.fill_(1.0)


def timed(torch, fn, reps, flush=None):
    """Median and minimum duration (ms) of fn() over reps launches, HIP events on the current stream."""
    durs = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        durs.append(a.elapsed_time(b))
    return float(np.median(durs)), float(np.min(durs))


def graph_time(torch, calls, reps):
    """Per-call duration (ms) of a sequence of launches issued back to back:
    the calls are captured once in a HIP graph, the graph is replayed reps
    times with HIP events around each replay, and each replay's time is divided
    by the number of calls. Returns (median, minimum) over the replays. No
    per-launch event overhead is counted; the gaps between the graph's kernels
    are."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in calls:
            c()
    graph.replay()
    torch.cuda.synchronize()
    durs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        b.synchronize()
        durs.append(a.elapsed_time(b) / len(calls))
    del graph
    return float(np.median(durs)), float(np.min(durs))


# ----------------------------------------------------------------- headline

def headline(args, torch, Y, S):
    w = S.DECODE_MID
    B, T, Hq, Hkv, D, L = w.B, w.T, w.Hq, w.Hkv, w.D, w.layers
    k_bits, v_bits = S.cache_kv(w)
    kc, vc = up(k_bits, torch), up(v_bits, torch)
    qs = [up(S.queries(w, layer=l, std=w.notes["q_std"]), torch) for l in range(L)]
    src = {k: up(v, torch) for k, v in S.compose_sources(w, layer=L // 2, n=1).items()}   # new token, layer L/2
    alpha = S.alphas(w.seed, L // 2)
    nsplit = args.decode_splits or Y.yoco_decode_num_splits(B, T, Hq, Hkv, D)
    ws = Y.decode_workspace(B, T, Hq, Hkv, D, nsplit)
    out = torch.empty((L, B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((L, B, Hq), dtype=torch.float32, device="cuda")
    # events bracket the 16 back-to-back decode launches of every timed step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def decode(l):
        Y.yoco_cross_attn_decode(qs[l], kc, vc, out[l], lse[l], workspace=ws, num_splits=nsplit)

    # One step: the new token's K', V' row is composed into the shared cache at
    # row T - 1 and the 16 cross layers decode over rows [0, T). The compose is
    # fused into the first layer's decode launch (it composes and appends the
    # row, then attends over the cache including it), so the step is 16 launches.
    def step(marks):
        if marks is not None:
            marks[0].record()
        Y.yoco_self_attn_decode(qs[0], src["k1"][:, 0], src["ki"][:, 0], src["v1"][:, 0], src["vi"][:, 0], kc, vc, alpha,
                                out[0], lse[0], workspace=ws, num_splits=nsplit)
        for l in range(1, L):
            decode(l)
        if marks is not None:
            marks[1].record()

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record()
    for i in range(args.steps):
        step(ev[i])
    e_ev.record()
    torch.cuda.synchronize()
    ms_per_step = s_ev.elapsed_time(e_ev) / args.steps
    host_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev])) / L

    layer_bytes = 2 * B * T * Hkv * D * 2
    value = L * layer_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = layer_bytes / (launch_ms * 1e-3) / 1e9

    # the same step captured once in a HIP graph and replayed (no host launch gaps);
    # the fused merge resets its counters on the device, so replays need no memset node
    graph_ms, graph_note = None, None
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(None)
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph
    except RuntimeError as e:   # reported; the eagerly launched step then stands as the value
        graph_note = f"graph capture failed: {e}"

    # warm per launch: the 16 decodes alone, captured in a graph and replayed, so
    # that 16 x this launch time is within the step time above
    warm_ms, _ = graph_time(torch, [lambda l=l: decode(l) for l in range(L)], args.steps)

    # HBM-served ("cold"): the same 16 decodes rotating over 8 copies of the cache
    # (1 GiB, four times the 256 MB Infinity Cache), so each launch finds its
    # 128 MiB evicted by the 896 MiB the seven launches before it read
    copies = [(kc.clone(), vc.clone()) for _ in range(8)]

    def decode_copy(l):
        ck, cv = copies[l % 8]
        Y.yoco_cross_attn_decode(qs[l], ck, cv, out[l], lse[l], workspace=ws, num_splits=nsplit)

    cold_ms, cold_min = graph_time(torch, [lambda l=l: decode_copy(l) for l in range(L)], args.reps)
    # and single launches timed with HIP events after a 1 GiB flush kernel (read or
    # write), which also count the event and dispatch overhead of one launch
    flushed = {}
    for mode in ("read", "write"):
        flush = Flusher(torch, mode)
        ms, mn = timed(torch, lambda: decode(0), args.reps, flush)
        flushed[mode] = {"ms": ms, "gbs": layer_bytes / (ms * 1e-3) / 1e9,
                         "best_gbs": layer_bytes / (mn * 1e-3) / 1e9}
        del flush
    del copies
    eager = {"ms_per_step": ms_per_step, "gbs": value, "host_ms_per_step": host_ms,
             "decode_avg_launch_ms": launch_ms, "decode_gbs": achieved}
    launch = "eager"
    if graph_ms is not None:
        ms_per_step, value, launch = graph_ms, L * layer_bytes / (graph_ms * 1e-3) / 1e9, "hip_graph"
    return {
        "value": value, "ms_per_step": ms_per_step, "launch": launch, "eager": eager, "graph_note": graph_note,
        "num_splits": nsplit, "layer_bytes": layer_bytes,
        "decode_warm_launch_ms": warm_ms, "decode_warm_gbs": layer_bytes / (warm_ms * 1e-3) / 1e9,
        "decode_cold_ms": cold_ms, "decode_cold_gbs": layer_bytes / (cold_ms * 1e-3) / 1e9,
        "decode_cold_best_gbs": layer_bytes / (cold_min * 1e-3) / 1e9,
        "decode_single_launch_after_flush": flushed,
    }


# ----------------------------------------------------------------- legs

def leg_compose(args, torch, Y, S):
    """Compose of the 15 composed self-decoder layers (i = 2..16) of the 32K-token
    workload, 384 MiB each, launched back to back in a HIP graph. Every layer has
    its own copy of K_1, V_1 as well as its own K_i, V_i and caches, so the
    Infinity Cache serves none of a call's bytes (in the model the 15 calls
    re-read one K_1, V_1, which it partly would)."""
    w = S.PREFILL_CHUNKED
    B, T, Hkv, D = w.B, w.T, w.Hkv, w.D
    k1 = up(S.layer_source(w, "k", 1), torch)
    v1 = up(S.layer_source(w, "v", 1), torch)
    layers = list(range(2, w.self_layers + 1))
    bytes_per_call = 6 * B * T * Hkv * D * 2
    sets = []
    for i in layers:
        ki = up(S.layer_source(w, "k", i), torch)
        vi = up(S.layer_source(w, "v", i), torch)
        kc = torch.empty((B, Hkv, T, D), dtype=torch.bfloat16, device="cuda")
        sets.append((k1.clone(), ki, v1.clone(), vi, kc, torch.empty_like(kc), S.alphas(w.seed, i)))
    calls = [lambda st=st: Y.yoco_compose_kv(st[0], st[1], st[2], st[3], st[4], st[5], 0, st[6]) for st in sets]
    ms, best = graph_time(torch, calls, max(3, args.reps // 2))
    # one call after a 1 GiB flush kernel, HIP events around the single launch
    flush = Flusher(torch)
    single, _ = timed(torch, calls[0], max(2, args.reps // 2), flush)
    del flush, sets
    return {"workload": "prefill_chunked stage A (15 compose calls, [1,32768,8,128] bf16)",
            "bytes_per_call": bytes_per_call, "ms": ms, "gbs": bytes_per_call / ms / 1e6,
            "best_gbs": bytes_per_call / best / 1e6, "hbm_frac": bytes_per_call / ms / 1e6 / HBM_PEAK_GBS,
            "timing": "15 calls back to back in a HIP graph, replay time / 15, median of the replays",
            "single_call_after_flush_gbs": bytes_per_call / single / 1e6}


def leg_compose_backward(args, torch, Y, S):
    """Backward of one composed layer of the 32K-token workload ([1, 32768, 8, 128] bf16):
    reads gk, gv, K_1, K_i, V_1, V_i, accumulates the fp32 dK_1, dV_1 and writes dK_i, dV_i."""
    w = S.PREFILL_CHUNKED
    B, T, Hkv, D = w.B, w.T, w.Hkv, w.D
    src = {k: up(v, torch) for k, v in S.compose_sources(w, layer=3).items()}
    gk = up(S.layer_source(w, "k", 4), torch).transpose(1, 2).contiguous()   # any cache-shaped gradient
    gv = up(S.layer_source(w, "v", 4), torch).transpose(1, 2).contiguous()
    g32 = [torch.zeros((B, T, Hkv, D), dtype=torch.float32, device="cuda") for _ in range(4)]
    dalpha = torch.zeros(4, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(4, Y.yoco_compose_backward_workspace_size(B, T, Hkv, D, 1) // 4), dtype=torch.float32,
                     device="cuda")
    alpha = S.alphas(w.seed, 3)
    fn = lambda: Y.yoco_compose_kv_backward(gk, gv, 0, src["k1"], src["ki"], src["v1"], src["vi"], *g32, alpha,  # noqa
                                            dalpha, workspace=ws)
    fn()
    # 4 calls back to back in a HIP graph (1.2 GB each, far beyond the Infinity Cache)
    ms, best = graph_time(torch, [fn] * 4, max(3, args.reps // 2))
    nbytes = B * T * Hkv * D * (6 * 2 + 2 * 8 + 2 * 4)
    return {"workload": "prefill_chunked, one composed layer's backward", "bytes_per_call": nbytes, "ms": ms,
            "gbs": nbytes / ms / 1e6, "best_gbs": nbytes / best / 1e6, "hbm_frac": nbytes / ms / 1e6 / HBM_PEAK_GBS}


class ClockSampler:
    """Samples the engine (GFX) clock of each XCD and the socket power of the
    GPU that runs cuda:0 through the amdsmi library, every 20 ms, on a thread,
    from `settle` seconds after the start (the clock ramps up from idle first).
    The dense bf16 peak assumes 2.4 GHz; the clock a box holds under sustained
    matrix-core load is lower, and this records it."""

    def __init__(self, torch, settle: float = 0.25):
        import threading
        import amdsmi
        self.smi, self.samples, self.stop = amdsmi, [], threading.Event()
        self.settle, self.t0 = settle, 0.0
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        if not handles:
            raise RuntimeError("amdsmi sees no GPU")
        self.handle = handles[0]
        bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
        if bus is not None and len(handles) > 1:
            for h in handles:
                if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                    self.handle = h
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self.stop.is_set():
            m = self.smi.amdsmi_get_gpu_metrics_info(self.handle)
            clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
            power = m.get("current_socket_power")
            if clks and time.perf_counter() - self.t0 >= self.settle:   # past the ramp from idle
                self.samples.append((sum(clks) / len(clks), min(clks), max(clks),
                                     power if isinstance(power, (int, float)) else None))
            self.stop.wait(0.02)

    def __enter__(self):
        self.t0 = time.perf_counter()
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join()
        self.smi.amdsmi_shut_down()


def clocked_window(torch, fn, seconds: float) -> dict:
    """Run fn back to back for about `seconds` while sampling the engine clock;
    returns the clock and power medians and the time per call in the window."""
    import statistics
    calls = 0
    with ClockSampler(torch) as smp:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            fn()
            calls += 1
            torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / calls
    if not smp.samples:
        raise RuntimeError("no clock samples")
    mean_mhz = [x[0] for x in smp.samples]
    power = [x[3] for x in smp.samples if x[3] is not None]
    return {"calls": calls, "ms_per_call": ms, "samples": len(smp.samples),
            "gfxclk_mhz_median": statistics.median(mean_mhz),
            "gfxclk_mhz_min_xcd": min(x[1] for x in smp.samples), "gfxclk_mhz_max_xcd": max(x[2] for x in smp.samples),
            "socket_power_w_median": statistics.median(power) if power else None}


def leg_prefill(args, torch, Y, S):
    w = S.PREFILL_CHUNKED
    B, T, Hq, Hkv, D, C = w.B, w.T, w.Hq, w.Hkv, w.D, w.chunk
    k_bits, v_bits = S.cache_kv(w)
    kc, vc = up(k_bits, torch), up(v_bits, torch)
    q = up(S.queries(w, rows=T), torch)
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")

    def run():
        for c0 in range(0, T, C):
            Y.yoco_cross_attn_prefill(q[:, c0:c0 + C], kc, vc, c0, out[:, c0:c0 + C])

    run()
    torch.cuda.synchronize()
    ms, best = timed(torch, run, max(2, args.reps // 2))
    flop = 4.0 * B * Hq * D * T * (T + 1) / 2
    # the same 8 chunk launches captured once in a HIP graph (no host launch gaps)
    graph_tflops, graph_note, graph = None, None, None
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        graph.replay()
        torch.cuda.synchronize()
        gms, _ = timed(torch, graph.replay, max(2, args.reps // 2))
        graph_tflops = flop / gms / 1e9
    except RuntimeError as e:   # reported; the eager figure stands
        graph_note, graph = f"graph capture failed: {e}", None
    # the engine clock the box holds while the prefill runs back to back
    clock = None
    if args.clock_seconds > 0:
        try:
            clock = clocked_window(torch, graph.replay if graph is not None else run, args.clock_seconds)
            clock["tflops"] = flop / clock["ms_per_call"] / 1e9
            mhz = clock["gfxclk_mhz_median"]
            clock["peak_at_clock_tflops"] = BF16_MFMA_PEAK_TFLOPS * mhz / 2400.0
            clock["mfma_frac_at_clock"] = clock["tflops"] / clock["peak_at_clock_tflops"]
        except Exception as e:   # noqa: BLE001 - the clock is context, never a reason to fail the bench
            clock = {"note": f"clock not sampled: {type(e).__name__}: {e}"}
    del graph
    return {"workload": "prefill_chunked (T=32768, chunk 4096, 32/8 heads, D=128, bf16)", "flop": flop,
            "ms": ms, "tflops": flop / ms / 1e9, "best_tflops": flop / best / 1e9,
            "mfma_frac": flop / ms / 1e9 / BF16_MFMA_PEAK_TFLOPS, "graph_tflops": graph_tflops,
            "graph_note": graph_note, "clock": clock}


def leg_long_decode(args, torch, Y, S, w, planted=False):
    k_bits, v_bits = S.cache_kv(w)
    q_bits = S.queries(w)
    if planted:
        S.plant_query_row_bf16(k_bits, q_bits, S.planted_position(w), w.notes["plant_scale"])
    else:
        S.scale_key_rows_bf16(k_bits, S.scaled_rows(w), w.notes["scale"])
    kc, vc = up(k_bits, torch), up(v_bits, torch)
    del k_bits, v_bits
    q = up(q_bits, torch)
    B, T, Hq, Hkv, D = w.B, w.T, w.Hq, w.Hkv, w.D
    nsplit = args.long_splits or Y.yoco_decode_num_splits(B, T, Hq, Hkv, D)
    ws = Y.decode_workspace(B, T, Hq, Hkv, D, nsplit)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    full = lambda: Y.yoco_cross_attn_decode(q, kc, vc, out, workspace=ws, num_splits=nsplit)  # noqa: E731
    full()
    # 4 launches back to back in a HIP graph: each reads 2 GiB, eight times the Infinity Cache
    ms, best = graph_time(torch, [full] * 4, max(3, args.reps // 2))
    flush = Flusher(torch)
    single, _ = timed(torch, full, max(2, args.reps // 2), flush)
    del flush
    nbytes = 2 * B * T * Hkv * D * 2
    return {"workload": w.name, "B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "num_splits": nsplit, "bytes": nbytes,
            "ms": ms, "gbs": nbytes / ms / 1e6, "best_gbs": nbytes / best / 1e6,
            "hbm_frac": nbytes / ms / 1e6 / HBM_PEAK_GBS,
            "single_launch_after_flush_gbs": nbytes / single / 1e6}


def leg_compose_on_read(args, torch, Y, S):
    """The I/O claim of caching the composed pair: decode over the composed cache
    (one KV set per layer) vs composing layer 1 and layer L/2 on read (two sets),
    on the mid-context decode workload, 16 layers back to back and flushed."""
    w = S.DECODE_MID
    B, T, Hq, Hkv, D, L = w.B, w.T, w.Hq, w.Hkv, w.D, w.layers
    raw = {k: up(np.ascontiguousarray(v.transpose(0, 2, 1, 3)), torch)
           for k, v in S.compose_sources(w, layer=L // 2).items()}
    alpha = S.alphas(w.seed, L // 2)
    kc, vc = torch.empty_like(raw["ki"]), torch.empty_like(raw["vi"])
    Y.yoco_compose_kv(Y.head_major(raw["k1"]), Y.head_major(raw["ki"]), Y.head_major(raw["v1"]),
                      Y.head_major(raw["vi"]), kc, vc, 0, alpha, B=B, n=T, Hkv=Hkv, D=D, dtype=1)
    qs = [up(S.queries(w, layer=l, std=w.notes["q_std"]), torch) for l in range(L)]
    nsplit = Y.yoco_decode_num_splits(B, T, Hq, Hkv, D)
    ws = Y.decode_workspace(B, T, Hq, Hkv, D, nsplit)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")

    def stored(l=0):
        Y.yoco_cross_attn_decode(qs[l], kc, vc, out, workspace=ws, num_splits=nsplit)

    def on_read(l=0):
        Y.yoco_cross_attn_decode_compose_on_read(qs[l], raw["k1"], raw["ki"], raw["v1"], raw["vi"], alpha, out,
                                                 workspace=ws, num_splits=nsplit)

    layer_bytes = 2 * B * T * Hkv * D * 2
    res = {}
    for name, fn, nbytes in (("composed_cache", stored, layer_bytes), ("compose_on_read", on_read, 2 * layer_bytes)):
        fn()
        warm, _ = timed(torch, lambda: [fn(l) for l in range(L)], args.reps)
        flush = Flusher(torch)
        cold, _ = timed(torch, fn, args.reps, flush)
        del flush
        res[name] = {"kv_bytes_per_layer": nbytes, "warm_ms_per_layer": warm / L, "cold_ms_per_layer": cold,
                     "warm_gbs": nbytes / (warm / L) / 1e6, "cold_gbs": nbytes / cold / 1e6}
    res["time_ratio_warm"] = res["compose_on_read"]["warm_ms_per_layer"] / res["composed_cache"]["warm_ms_per_layer"]
    res["time_ratio_cold"] = res["compose_on_read"]["cold_ms_per_layer"] / res["composed_cache"]["cold_ms_per_layer"]
    return res


def leg_self_decoder(args, torch, Y, S):
    """One decode step of the self-decoder half on the mid-context decode workload:
    L/2 = 16 layers, each attending over its own composed cache (16 distinct
    128 MiB caches, so no layer finds the previous one's rows in the Infinity
    Cache). Fused: one launch per layer composes the new token's row, appends it
    and attends. Unfused: compose (n=1) then decode, two launches per layer."""
    w = S.DECODE_MID
    B, T, Hq, Hkv, D = w.B, w.T, w.Hq, w.Hkv, w.D
    half = w.layers          # the self-decoder half has as many layers as the cross-decoder half
    k_bits, v_bits = S.cache_kv(w)
    k0, v0 = up(k_bits, torch), up(v_bits, torch)
    caches = [(k0.clone(), v0.clone()) for _ in range(half)]
    del k0, v0
    qs = [up(S.queries(w, layer=l, std=w.notes["q_std"]), torch) for l in range(half)]
    srcs = []
    for l in range(1, half + 1):
        new = S.compose_sources(w, layer=l, n=1)
        srcs.append({k: up(v, torch) for k, v in new.items()})              # [B, 1, Hkv, D]
    alphas = [S.IDENTITY_ALPHA if l == 1 else S.alphas(w.seed, l) for l in range(1, half + 1)]
    nsplit = Y.yoco_decode_num_splits(B, T, Hq, Hkv, D)
    ws = Y.decode_workspace(B, T, Hq, Hkv, D, nsplit)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")

    def fused():
        for l in range(half):
            s, (kc, vc) = srcs[l], caches[l]
            Y.yoco_self_attn_decode(qs[l], s["k1"][:, 0], s["ki"][:, 0], s["v1"][:, 0], s["vi"][:, 0], kc, vc,
                                    alphas[l], out, workspace=ws, num_splits=nsplit)

    def unfused():
        for l in range(half):
            s, (kc, vc) = srcs[l], caches[l]
            Y.yoco_compose_kv(s["k1"], s["ki"], s["v1"], s["vi"], kc, vc, T - 1, alphas[l])
            Y.yoco_cross_attn_decode(qs[l], kc, vc, out, workspace=ws, num_splits=nsplit)

    layer_bytes = 2 * B * T * Hkv * D * 2
    res = {"layers": half, "kv_bytes_per_layer": layer_bytes}
    for name, fn in (("fused", fused), ("compose_then_decode", unfused)):
        fn()
        ms, best = timed(torch, fn, args.reps)
        res[name] = {"ms_per_step": ms, "gbs": half * layer_bytes / ms / 1e6,
                     "best_gbs": half * layer_bytes / best / 1e6}
    res["speedup_fused"] = res["compose_then_decode"]["ms_per_step"] / res["fused"]["ms_per_step"]
    del caches
    return res


def leg_early_exit(args, torch, Y, S):
    """The prefill of the 32K-token workload (1 x 32768 tokens, 32/8 heads, D=128)
    through the cache path, with and without YOCO's early exit. Both compose the
    15 composed self-decoder layers (i = 2..16) for all T rows. With the early
    exit the 16 cross-decoder layers then run only for the last token (one
    decode call each over the shared K'_16, V'_16); without it each cross layer
    runs the full causal chunked prefill (8 chunks of 4096). The decode of the
    last token and the last prefill row are reported side by side (they must agree)."""
    w = S.PREFILL_CHUNKED
    B, T, Hq, Hkv, D, C = w.B, w.T, w.Hq, w.Hkv, w.D, w.chunk
    cross = w.self_layers                       # as many cross-decoder layers as self-decoder layers
    k1 = up(S.layer_source(w, "k", 1), torch)
    v1 = up(S.layer_source(w, "v", 1), torch)
    ki0 = up(S.layer_source(w, "k", 2), torch)
    vi0 = up(S.layer_source(w, "v", 2), torch)
    layers = list(range(2, w.self_layers + 1))
    # one layer's sources drawn on the host, copied on the device for the others:
    # distinct memory, so no compose finds its inputs in the Infinity Cache
    srcs = [(ki0, vi0)] + [(ki0.clone(), vi0.clone()) for _ in layers[1:]]
    caches = [(torch.empty((B, Hkv, T, D), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, Hkv, T, D), dtype=torch.bfloat16, device="cuda")) for _ in layers]
    alphas = [S.alphas(w.seed, i) for i in layers]
    kc, vc = caches[-1]                          # K'_{L/2}, V'_{L/2}: what every cross layer reads
    q = up(S.queries(w, rows=T), torch)
    q_last = q[:, T - 1].contiguous()
    nsplit = Y.yoco_decode_num_splits(B, T, Hq, Hkv, D)
    ws = Y.decode_workspace(B, T, Hq, Hkv, D, nsplit)
    out_dec = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    out_pf = torch.empty((B, C, Hq, D), dtype=torch.float32, device="cuda")

    def compose_all():
        for (ki, vi), (kcl, vcl), a in zip(srcs, caches, alphas):
            Y.yoco_compose_kv(k1, ki, v1, vi, kcl, vcl, 0, a)

    def early_exit():
        compose_all()
        for _ in range(cross):
            Y.yoco_cross_attn_decode(q_last, kc, vc, out_dec, workspace=ws, num_splits=nsplit)

    def full():
        compose_all()
        for _ in range(cross):
            for c0 in range(0, T, C):
                Y.yoco_cross_attn_prefill(q[:, c0:c0 + C], kc, vc, c0, out_pf)

    early_exit()
    full()
    torch.cuda.synchronize()
    agree = float((out_pf[:, C - 1] - out_dec).abs().max())
    ee_ms, ee_best = timed(torch, early_exit, args.reps)
    full_ms, _ = timed(torch, full, 2)
    compose_ms, _ = timed(torch, compose_all, args.reps)
    return {"cross_layers": cross, "composed_layers": len(layers), "early_exit_ms": ee_ms,
            "early_exit_best_ms": ee_best, "without_early_exit_ms": full_ms, "compose_only_ms": compose_ms,
            "cross_part_early_exit_ms": ee_ms - compose_ms, "cross_part_full_ms": full_ms - compose_ms,
            "speedup": full_ms / ee_ms, "max_abs_last_row_decode_vs_prefill": agree}


def leg_ceiling(args, torch, S):
    """Achievable-bandwidth probes (libyoco_ceiling.so), timed like the kernels they
    bound (back-to-back launches in a HIP graph): a plain streaming read of 128 MiB
    (the mid-context decode's cache; rotating over 8 buffers so that the Infinity
    Cache serves none of it, and on one buffer, which it serves) and of 2 GiB (the
    long decodes' caches), and the compose's four-reads-two-writes traffic at its
    384 MiB per call (rotating over 3 buffer sets), each over several launch
    shapes (workgroups x threads x loads in flight per thread for the reads,
    threads striding over a workgroup's range or wavefronts taking blocks);
    the best median of each is the ceiling of the matching kernel. And
    the matrix cores' sustained bf16 MFMA rate on N(0,1) and on zero operands,
    the ceiling of the prefill."""
    from cross_layer_shared_amd import ceiling as C
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    res = {}

    def best(out, cond):
        k, row = max(out["shapes"].items(), key=lambda kv: kv[1][cond]["gbs"])
        return {"shape": k, **row[cond]}

    def rate(nbytes, ms, mn):
        return {"ms": ms, "gbs": nbytes / ms / 1e6, "best_gbs": nbytes / mn / 1e6}

    # 128 MiB reads
    nb = 1 << 27
    bufs = [torch.empty(nb // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0) for _ in range(8)]
    out = {"bytes": nb, "shapes": {}}
    for wg, th, u in [(256, 512, 4), (256, 512, 8), (256, 512, 16), (256, 1024, 8), (512, 512, 8), (1024, 256, 8),
                      (0, 512, 8)]:
        rd = lambda i, wg=wg, th=th, u=u: C.yoco_ceiling_read(bufs[i], sink, workgroups=wg, threads=th,  # noqa: E731
                                                              loads_per_thread=u)
        row = {"hbm": rate(nb, *graph_time(torch, [lambda i=i: rd(i % 8) for i in range(16)], args.reps)),
               "warm": rate(nb, *graph_time(torch, [lambda: rd(0)] * 16, args.reps))}
        out["shapes"][f"{wg or 'stride'}x{th}x{u}"] = row
    for wg, th, u in [(256, 512, 4), (256, 512, 8), (512, 512, 8), (1024, 256, 8)]:   # per-wavefront blocks
        rd = lambda i, wg=wg, th=th, u=u: C.yoco_ceiling_read_blocks(bufs[i], sink, workgroups=wg,  # noqa: E731
                                                                     threads=th, loads_per_thread=u)
        row = {"hbm": rate(nb, *graph_time(torch, [lambda i=i: rd(i % 8) for i in range(16)], args.reps)),
               "warm": rate(nb, *graph_time(torch, [lambda: rd(0)] * 16, args.reps))}
        out["shapes"][f"blocks{wg}x{th}x{u}"] = row
    out["hbm"], out["warm"] = best(out, "hbm"), best(out, "warm")
    res["read_128MiB"] = out
    del bufs
    # 2 GiB reads
    nb = 1 << 31
    bufs = [torch.empty(nb // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0) for _ in range(2)]
    out = {"bytes": nb, "shapes": {}}
    for wg, th, u in [(256, 512, 8), (512, 512, 4), (512, 512, 8), (512, 512, 16), (1024, 512, 8), (2048, 256, 8)]:
        rd = lambda i, wg=wg, th=th, u=u: C.yoco_ceiling_read(bufs[i], sink, workgroups=wg, threads=th,  # noqa: E731
                                                              loads_per_thread=u)
        out["shapes"][f"{wg}x{th}x{u}"] = {"hbm": rate(nb, *graph_time(torch, [lambda i=i: rd(i % 2) for i in range(4)],
                                                                       max(3, args.reps // 2)))}
    for wg, th, u in [(512, 512, 8), (1024, 512, 8), (2048, 256, 8)]:   # per-wavefront blocks
        rd = lambda i, wg=wg, th=th, u=u: C.yoco_ceiling_read_blocks(bufs[i], sink, workgroups=wg,  # noqa: E731
                                                                     threads=th, loads_per_thread=u)
        out["shapes"][f"blocks{wg}x{th}x{u}"] = {
            "hbm": rate(nb, *graph_time(torch, [lambda i=i: rd(i % 2) for i in range(4)], max(3, args.reps // 2)))}
    out["hbm"] = best(out, "hbm")
    res["read_2GiB"] = out
    del bufs
    # compose traffic: 6 streams of 64 MiB (a 32K-token layer's K_1, K_i, V_1, V_i in, K', V' out)
    n = 1 << 25
    sets = [[torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0) for _ in range(6)] for _ in range(3)]
    nb = 6 * 2 * n
    out = {"bytes": nb, "shapes": {}}
    for th, u in [(256, 1), (512, 1), (1024, 1), (256, 2), (512, 2), (256, 4)]:
        fn = lambda i, th=th, u=u: C.yoco_ceiling_read4_write2(*sets[i], threads=th,  # noqa: E731
                                                               positions_per_thread=u)
        out["shapes"][f"{th}x{u}"] = {"hbm": rate(nb, *graph_time(torch, [lambda i=i: fn(i % 3) for i in range(6)],
                                                                  args.reps))}
    out["hbm"] = best(out, "hbm")
    res["read4_write2_384MiB"] = out
    del sets
    # matrix cores: back-to-back bf16 MFMAs (the prefill's instruction) on N(0,1)
    # operands, the prefill workload's data, and on zeros; the rate the chip
    # sustains depends on the operand values, so both are timed, each over the
    # same clock-sampled window as the prefill
    pool = {"normal": up(S.normal_bf16(S.PREFILL_CHUNKED.seed, (0x4D46,), (1 << 20,)), torch),
            "zeros": torch.zeros(1 << 20, dtype=torch.bfloat16, device="cuda")}
    fsink = torch.zeros(4, dtype=torch.float32, device="cuda")
    wg, iters = 256, 16384
    flop = C.mfma_flop(wg, iters)
    out = {"instruction": "v_mfma_f32_32x32x16_bf16", "workgroups": wg, "waves_per_simd": 2, "iters": iters,
           "flop_per_call": flop}
    for name, buf in pool.items():
        fn = lambda buf=buf: C.yoco_ceiling_mfma_bf16(buf, fsink, wg, iters)  # noqa: E731
        fn()
        torch.cuda.synchronize()
        row = {}
        if args.clock_seconds > 0:
            try:
                row = clocked_window(torch, fn, args.clock_seconds)
            except Exception as e:   # noqa: BLE001 - the clock is context; time the calls without it
                row = {"clock_note": f"clock not sampled: {type(e).__name__}: {e}"}
        if "ms_per_call" not in row:
            row["ms_per_call"], _ = timed(torch, fn, args.reps)
        row["tflops"] = flop / row["ms_per_call"] / 1e9
        row["frac_of_peak"] = row["tflops"] / BF16_MFMA_PEAK_TFLOPS
        out[name] = row
    res["mfma_bf16"] = out
    del pool
    return res


# ----------------------------------------------------------------- counter traffic

def counter_traffic():
    """HBM-side bytes per decode launch from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings), or None if the
    kernel source has changed since those counters were taken."""
    import hashlib
    rec_path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(rec_path):
        return None
    rec = json.load(open(rec_path))
    for rel, digest in rec["sources"].items():
        src = os.path.join(ROOT, rel)
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != digest:
            return None
    return 1024.0 * (rec["fetch_kib_per_launch"] * rec["fetch_scale"] + rec["write_kib_per_launch"] * rec["write_scale"])


# ----------------------------------------------------------------- CPU baseline

def cpu_baseline(args, S):
    """The fp64 oracle on the host: decode layers of the headline workload until
    about --cpu-seconds of work; reported in the headline unit (GB/s of KV)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = None
    w = S.DECODE_MID
    k_bits, v_bits = S.cache_kv(w)
    layer_bytes = 2 * w.B * w.T * w.Hkv * w.D * 2
    qs = [S.queries(w, layer=l, std=w.notes["q_std"]) for l in range(w.layers)]
    layers, t_total = 0, 0.0
    while t_total < args.cpu_seconds:      # cycle through the 16 layers until the time target
        t0 = time.perf_counter()
        O.decode_attention(qs[layers % w.layers], k_bits, v_bits)
        t_total += time.perf_counter() - t0
        layers += 1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    return {"value": layers * layer_bytes / t_total / 1e9, "unit": "GB/s", "cores": threads or cores,
            "host_cores_available": cores, "kind": "oracle",
            "sample": f"{layers} decode-layer calls of decode_mid_context, cycling through its 16 layers "
                      f"(fp64 NumPy, {t_total:.1f} s)"}


def cpu_units(S):
    """The fp64 oracle on the host for one work unit of each other workload (off by
    default: a few minutes of host time): one 32K-token compose layer, one decode
    call of each long context, and the causal prefill on the last 32 query rows of
    the 32K-token prompt (reported as TFLOP/s of those rows' unmasked pairs)."""
    import oracle as O
    res = {}
    w = S.PREFILL_CHUNKED
    src = S.compose_sources(w, layer=3)
    alpha = S.alphas(w.seed, 3)
    t0 = time.perf_counter()
    O.compose_kv(src["k1"], src["ki"], src["v1"], src["vi"], alpha)
    dt = time.perf_counter() - t0
    res["compose_layer"] = {"seconds": dt, "gbs": 6 * w.B * w.T * w.Hkv * w.D * 2 / dt / 1e9}
    del src
    for wl in (S.DECODE_LONG, S.DECODE_MILLION):
        k, v = S.cache_kv(wl)
        q = S.queries(wl)
        t0 = time.perf_counter()
        O.decode_attention(q, k, v)
        dt = time.perf_counter() - t0
        res[wl.name] = {"seconds": dt, "gbs": 2 * wl.B * wl.T * wl.Hkv * wl.D * 2 / dt / 1e9}
        del k, v
    k, v = S.cache_kv(w)
    q = S.queries(w, rows=w.chunk)
    rows = list(range(w.chunk - 32, w.chunk))
    p0 = w.T - w.chunk
    t0 = time.perf_counter()
    O.causal_prefill(q, k, v, p0, rows=rows)
    dt = time.perf_counter() - t0
    flop = 4.0 * w.B * w.Hq * w.D * sum(p0 + r + 1 for r in rows)
    res["prefill_last_32_rows"] = {"seconds": dt, "tflops": flop / dt / 1e12,
                                   "full_pass_seconds_at_this_rate": 8.796361457664e12 / (flop / dt)}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": f"this benchmark runs on one GPU; --gpus {args.gpus} is not supported "
                                   "(the hot path has no multi-GPU mode)"}))
        sys.exit(2)
    import torch

    import cross_layer_shared_amd as Y
    from synthetic import inputs as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    Y.load_library()
    legs = {"compose", "prefill", "long", "million", "ceiling", "cor", "backward", "self", "early_exit"} if args.legs == "all" else \
        set() if args.legs == "headline" else set(args.legs.split(","))

    h = headline(args, torch, Y, S)
    extra = {}
    if "ceiling" in legs:
        extra["ceiling"] = leg_ceiling(args, torch, S)
    if "compose" in legs:
        extra["compose"] = leg_compose(args, torch, Y, S)
    if "backward" in legs:
        extra["compose_backward"] = leg_compose_backward(args, torch, Y, S)
    if "prefill" in legs:
        extra["prefill"] = leg_prefill(args, torch, Y, S)
    if "cor" in legs:
        extra["compose_on_read_comparator"] = leg_compose_on_read(args, torch, Y, S)
    if "self" in legs:
        extra["self_decoder_step"] = leg_self_decoder(args, torch, Y, S)
    if "early_exit" in legs:
        extra["early_exit_prefill"] = leg_early_exit(args, torch, Y, S)
    if "long" in legs:
        extra["decode_long_context"] = leg_long_decode(args, torch, Y, S, S.DECODE_LONG)
    if "million" in legs:
        extra["decode_million_token"] = leg_long_decode(args, torch, Y, S, S.DECODE_MILLION, planted=True)
    torch.cuda.synchronize()

    if "ceiling" in extra:   # each HBM-bound figure beside the probe with its traffic pattern
        c = extra["ceiling"]
        vs = {"decode_mid_context_hbm": h["decode_cold_gbs"] / c["read_128MiB"]["hbm"]["gbs"],
              "decode_mid_context_warm": h["decode_warm_gbs"] / c["read_128MiB"]["warm"]["gbs"]}
        if "compose" in extra:
            vs["compose_hbm"] = extra["compose"]["gbs"] / c["read4_write2_384MiB"]["hbm"]["gbs"]
        for k in ("decode_long_context", "decode_million_token"):
            if k in extra:
                vs[k] = extra[k]["gbs"] / c["read_2GiB"]["hbm"]["gbs"]
        if "prefill" in extra:   # both from back-to-back windows of the same length
            pf = extra["prefill"]
            pf_tflops = (pf.get("clock") or {}).get("tflops") or pf["tflops"]
            vs["prefill_vs_mfma_on_normal_operands"] = pf_tflops / c["mfma_bf16"]["normal"]["tflops"]
        c["fraction_of_ceiling"] = vs

    w = S.DECODE_MID
    traffic_bytes = counter_traffic()
    # The dominant kernel is the decode split kernel. Its HBM figure is the
    # flushed launch (the 128 MiB cache fits the 256 MB Infinity Cache, so the
    # 16 back-to-back layers of a step are served from there, reported apart).
    cold_ms = h["decode_cold_ms"]
    traffic = None if traffic_bytes is None else traffic_bytes / (cold_ms * 1e-3) / 1e9
    ceil = extra.get("ceiling", {}).get("read_128MiB", {}).get("hbm")
    roofline = {"kernel": "decode_mfma_kernel<D=128, G=4, 8 waves> (bf16 split pass on the matrix cores, fused merge)",
                "bound": "hbm",
                "achieved": h["decode_cold_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": h["decode_cold_gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                "traffic_bytes_per_launch": traffic_bytes,
                "algorithmic_bytes_per_launch": h["layer_bytes"], "avg_launch_ms": cold_ms,
                "timing": "16 launches back to back in a HIP graph, rotating over 8 copies of the cache (1 GiB, "
                          "so the Infinity Cache serves none of them); replay time / 16, median of the replays "
                          "(HIP events on the launch stream)",
                "achievable_ceiling": None if ceil is None else {
                    "what": "plain 128 MiB streaming read (probe kernel), timed the same way, best launch shape",
                    "gbs": ceil["gbs"], "shape": ceil["shape"], "frac_of_ceiling": h["decode_cold_gbs"] / ceil["gbs"]},
                "infinity_cache_served": {
                    "achieved": h["decode_warm_gbs"], "avg_launch_ms": h["decode_warm_launch_ms"],
                    "timing": "16 launches on the one cache back to back in a HIP graph",
                    "note": "the 16 layers of a step re-read one 128 MiB cache, held by the 256 MB Infinity Cache: "
                            "not an HBM figure"}}
    line = {
        "metric": METRIC, "value": h["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "cross_layers": w.layers, "step": "16 x decode (split-K, fused merge), the first also composing and appending the new row",
                   "launch": h["launch"],
                   "seeds": {x.name: x.seed for x in S.WORKLOADS.values()}},
        "roofline": roofline,
        "headline_detail": h,
        "legs": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, S)
        if args.cpu_units:
            line["cpu_baseline"]["units"] = cpu_units(S)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
