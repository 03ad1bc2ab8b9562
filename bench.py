"""Benchmark of the paged decode hot path on one MI355X.

One step = one decode step of the ragged continuous-batching workload:
64 sequences (context log-uniform in [16, 8192], block_size 16, 65536-block
bf16 pool per layer, Llama-3.2-1B attention shapes: 32 query heads, 8 KV
heads, head_dim 64): one paged_attention_decode_plan (the automatic split's
plan for this step's lengths and tables, shared by every layer), then for
each of the 16 layers one
    paged_attention_decode_append(..., PKV_PARTITION_PLANNED)
call: store one new token per sequence (kv_append) and attend to the whole
context (paged_attention_decode) with the automatic split, in one kernel
launch whose log-sum-exp merge runs inside the kernel.  `--form auto` times
the same calls without a plan, `--form two-calls` kv_append followed by
paged_attention_decode per layer.  The step is captured once in a HIP graph
and replayed.

Prints ONE JSON line.  `value` is the whole step's algorithmic HBM bytes
divided by the step time (inputs resident in HBM).  `roofline` is for the
dominant kernel -- the combined append + decode kernel (the decode kernel
with --form two-calls) -- timed with HIP events over graph replays of its 16
calls on the stream the graph runs on.  `stream_floor` is a plain streaming
read of the same K/V bytes through the same tables (pagedkv_stream_blocks),
timed the same way over the same 16 pool pairs: the floor the decode kernel
is measured against.  `cpu_baseline` is the CPU oracle on a bounded sample
of the same workload, on all the host cores the process may use (at most
16) and, beside it, on one core.  `llama1b_layer` is the Llama-3.2-1B
single-layer decode (batch 8, context uniform in [128, 2048], one token
appended and attended) over 8 rotating pool pairs.  `prefill` reports the causal paged
prefill workload (4 x 512 + 2 x 2048 prompts) on the bf16 MFMA roofline, and
`rope_append` the rotary embedding of q and k fused with the append
(kv_append_rope) for the step's 64 new tokens and for the prefill prompts'
6144, on the HBM roofline.  `long_context` times the long-context split
workload (4 sequences of 32768 tokens) with fixed 512-token partitions merged
by log-sum-exp, with the automatic split, and with the automatic split's plan
(made once, outside the timed calls), on the HBM roofline.  `mixed_batch`
times one prefill launch over decode rows and prompt chunks together,
`copy_blocks` kv_copy_blocks (copy on write), and `scheduler` the host
block allocator and continuous-batching scheduler per step.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--form planned|auto|two-calls]

Every timed region follows W eager warm-up steps and at least WARM_S seconds
of untimed graph replays, so the figures are sustained rates.  Every leg
uses distinct buffers in turn (pools per layer, or rotating copies of at
least 1 GiB in all) so that no call finds its inputs in the 256 MB
last-level cache.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
LAYERS = 16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-rope", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the mixed-batch, block-copy and scheduler legs")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for counter scaling)")
    ap.add_argument("--form", choices=("planned", "auto", "two-calls"), default="planned",
                    help="planned: one plan per step + combined calls; auto: combined calls "
                         "without a plan; two-calls: kv_append then paged_attention_decode")
    ap.add_argument("--partition", type=int, default=-1,
                    help="decode partition_size (-1 = automatic split)")
    ap.add_argument("--only", choices=("prefill", "long", "mixed", "llama1b"), default=None,
                    help="run this one leg alone and print its JSON object (for profiling "
                         "a single kernel); the contract line is not printed")
    return ap.parse_args()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_193_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse_dpm(text):
    """A DPM clock table as the amdgpu driver prints it ("S: 125Mhz *",
    "1: 2400Mhz", one level a line, '*' on the current one): (levels in MHz,
    current level or None)."""
    levels, cur = [], None
    for line in text.splitlines():
        parts = line.split()
        if len(parts) < 2 or not parts[1].lower().endswith("mhz"):
            continue
        mhz = int(parts[1][:-3])
        levels.append(mhz)
        if parts[-1] == "*":
            cur = mhz
    return levels, cur


def gpu_clocks(torch, busy, samples=8):
    """The GPU the legs ran on, and its shader (sclk) and memory (mclk)
    clocks as the driver reports them: the DPM levels from the device's sysfs
    tables, and the level marked current, sampled every 5 ms while `busy()`
    has untimed work queued.  Clock fields are null where the tables cannot
    be read."""
    p = torch.cuda.get_device_properties(0)
    rec = {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
           "source": "sysfs pp_dpm_sclk / pp_dpm_mclk of the device, sampled during "
                     "untimed step replays after the timed region"}
    path = (f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:"
            f"{p.pci_device_id:02x}.0")

    def read(name):
        with open(os.path.join(path, name)) as f:
            return parse_dpm(f.read())

    busy()
    try:
        seen = {"sclk": [], "mclk": []}
        for _ in range(samples):
            time.sleep(0.005)
            for k in seen:
                seen[k].append(read(f"pp_dpm_{k}")[1])
        for k in seen:
            rec[f"{k}_mhz"] = {"levels": read(f"pp_dpm_{k}")[0], "current_under_load": seen[k]}
    except (OSError, ValueError):
        rec["sclk_mhz"] = rec["mclk_mhz"] = None
    torch.cuda.synchronize()
    return rec


def decode_bytes(lens, B, Hq, Hkv, D, out_bytes, bs=16):
    """Algorithmic HBM bytes of one decode call: K+V of every context token
    (2 * Hkv * D * 2 = 2048 B per token at 8 KV heads), q, out, block ids, lens."""
    kv = sum(int(L) for L in lens) * 2 * Hkv * D * 2
    ids = sum((int(L) + bs - 1) // bs for L in lens) * 4
    return kv + B * Hq * D * 2 + B * Hq * D * out_bytes + ids + 4 * B


def append_bytes(T_new, Hkv, D):
    return T_new * Hkv * D * 2 * 2 * 2  # K and V rows, read + write


def traffic_from_profiles(kernel_hash, form):
    """HBM bytes per launch of the timed kernel (combined append + decode with
    or without a plan, or decode alone) from committed counter runs, if they
    were taken on this exact kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "decode_ragged_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_hash:
        return None
    key = {"planned": "bytes_per_planned_append_decode_call",
           "auto": "bytes_per_append_decode_call", "two-calls": "bytes_per_decode_call"}[form]
    return rec.get(key)


def host_cores():
    """Threads the CPU baseline may use: the cores this process may run on,
    at most 16 (the host share of one GPU on the boxes it runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(case, k_layers, v_layers, layers=4, single_s=4.0, multi_s=3.0):
    """The oracle (single-threaded C, fp64, never tuned) on whole layers of
    the workload: once on one core, cycling through layers for at least
    `single_s` seconds; once on all the host cores the process may use, its
    (layer, sequence) decode calls dealt out to that many threads (ctypes
    releases the GIL, so they run in parallel) for at least `multi_s` seconds
    of wall time.  Returns a dict of GB/s over the same algorithmic bytes."""
    import threading
    import oracle
    from paged_kv_cache_193_amd import workloads as wl
    layers = min(layers, len(k_layers))
    compact = []
    for layer in range(layers):
        kc, vc, tc = wl.compact_for_oracle(case, k_layers[layer], v_layers[layer])
        compact.append((wl.as_u16(kc), wl.as_u16(vc), tc.numpy()))
    q16, lens = wl.as_u16(case.q), case.context_lens.numpy()
    layer_b = decode_bytes(case.context_lens.tolist(), case.B, case.Hq, case.Hkv, case.D, 2)
    # one core
    total_s, passes = 0.0, 0
    while total_s < single_s and passes < 256:
        k16, v16, tables = compact[passes % layers]
        t0 = time.perf_counter()
        oracle.decode(q16, k16, v16, tables, lens, case.scale)
        total_s += time.perf_counter() - t0
        passes += 1
    one = {"value": round(layer_b * passes / total_s / 1e9, 3), "cores": 1,
           "seconds": round(total_s, 2), "layer_passes": passes}
    # all cores: every (layer, sequence) unit of `layers` layers, longest first
    n = host_cores()
    units = sorted(((int(lens[b]), layer, b) for layer in range(layers) for b in range(case.B)),
                   reverse=True)
    groups = [[] for _ in range(n)]
    load = [0] * n
    for cost, layer, b in units:
        i = load.index(min(load))
        groups[i].append((layer, b))
        load[i] += cost + 1

    def work(g):
        for layer, b in g:
            k16, v16, tables = compact[layer]
            oracle.decode(q16[b:b + 1], k16, v16, tables[b:b + 1], lens[b:b + 1], case.scale)

    wall, rounds = 0.0, 0
    while wall < multi_s and rounds < 256:
        threads = [threading.Thread(target=work, args=(g,)) for g in groups if g]
        t0 = time.perf_counter()
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        wall += time.perf_counter() - t0
        rounds += 1
    many = {"value": round(layer_b * layers * rounds / wall / 1e9, 3),
            "cores": len([g for g in groups if g]), "seconds": round(wall, 2),
            "layer_passes": layers * rounds}
    return one, many


WARM_S = 0.1  # seconds of graph replays before a leg is timed


def graph_us(torch, call, steps, warmup, per_graph=8):
    """Average time of `call` over graph replays (per_graph calls per graph,
    so the gap between replays is not counted as kernel time), HIP events on
    the stream the graph runs on.  `warmup` eager calls, then at least
    WARM_S seconds of replays before the timed ones: the prefill kernel
    runs about 20% slower during its first ~30 ms of sustained load, as the
    GPU's clocks settle, and the legs report sustained rates."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            call()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARM_S:
        for _ in range(10):
            graph.replay()
        torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / (steps * per_graph) * 1e3


def run_prefill(torch, pkv, wl, steps, warmup, copies=8):
    """Causal paged prefill of 4 x 512 + 2 x 2048 prompts; returns a dict.
    `copies` copies of the pools and queries (1.2 GB in all) are used in turn,
    so no call finds its inputs in the 256 MB last-level cache."""
    dev = "cuda"
    p = wl.prefill_case()
    t, l, cu = p.block_tables.to(dev), p.context_lens.to(dev), p.cu_q_lens.to(dev)
    sets = []
    for _ in range(copies):
        k, v = p.k_cache.to(dev), p.v_cache.to(dev)
        pkv.kv_append(k, v, p.k_new.to(dev), p.v_new.to(dev), t, l, cu)
        sets.append((k, v, p.q.to(dev)))
    out = torch.empty(tuple(p.q.shape), dtype=torch.bfloat16, device=dev)
    qlens = (p.cu_q_lens[1:] - p.cu_q_lens[:-1]).tolist()
    maxq = max(qlens)

    def calls():
        for k, v, q in sets:
            pkv.paged_attention_prefill_causal(out, q, k, v, t, l, cu, p.scale, maxq)
    us = graph_us(torch, calls, steps, warmup, per_graph=1) / copies
    # visible (query, key) pairs: QK^T and PV, 2 flops per MAC, D = 64
    flops = sum(p.Hq * 2 * 2 * p.D * L * (L + 1) // 2 for L in qlens)
    tflops = flops / (us * 1e-6) / 1e12
    return {"workload": "causal paged prefill, prompts 4x512 + 2x2048, 32q/8kv heads, "
                        "head_dim 64, block_size 16, bf16",
            "us_per_call": round(us, 2), "flops": flops,
            "rotation": f"{copies} copies of pools and q used in turn",
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}}


def run_mfma_probe(torch, pkv, iters=20000, launches=10):
    """pagedkv_mfma_probe: bf16 MFMA chains and nothing else on 2048
    wavefronts, `launches` launches of `iters` rounds timed with HIP events
    after a warm-up; the issue rate the prefill's flops are measured against,
    taken at the GPU's running clock (sampled during untimed launches)."""
    sink = torch.empty(pkv.STREAM_SINK_BYTES // 4, dtype=torch.float32, device="cuda")
    for _ in range(3):
        pkv.mfma_probe(iters, sink)
    torch.cuda.synchronize()
    if not torch.all(sink == 4.0 * iters):
        raise RuntimeError("mfma probe: the folded result is not 4 * iters")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(launches):
        pkv.mfma_probe(iters, sink)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / launches
    tflops = pkv.mfma_probe_flops(iters) / (us * 1e-6) / 1e12
    clocks = gpu_clocks(torch, lambda: [pkv.mfma_probe(iters, sink) for _ in range(20)])
    return {"kernel": "mfma_probe_kernel (pagedkv_mfma_probe): 2048 wavefronts x 4 chains of "
                      f"v_mfma_f32_32x32x16_bf16, {iters} rounds, operands in registers",
            "us_per_call": round(us, 2), "flops": pkv.mfma_probe_flops(iters),
            "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
            "sclk_mhz_under_load": (clocks.get("sclk_mhz") or {}).get("current_under_load")}


def run_floor(torch, pkv, case, k_layers, v_layers, steps, warmup):
    """pagedkv_stream_blocks over the blocks the batch's contexts use (every
    KV head of each), one call per pool pair in turn: a plain streaming read
    of the bytes a decode call reads.  Returns (us per call, bytes per call)."""
    ids = case.extra["used_blocks"].to(torch.int32).to("cuda")
    sink = torch.zeros(pkv.STREAM_SINK_BYTES, dtype=torch.uint8, device="cuda")

    def calls():
        for k, v in zip(k_layers, v_layers):
            pkv.stream_blocks(k, v, ids, sink)
    us = graph_us(torch, calls, steps, warmup, per_graph=1) / len(k_layers)
    return us, ids.numel() * case.Hkv * case.block_size * case.D * 2 * 2


def floor_record(us, nbytes, kernel_us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "stream_blocks_kernel (pagedkv_stream_blocks)", "us_per_call": round(us, 2),
            "bytes": nbytes, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "decode_time_over_floor": round(kernel_us / us, 3)}


def run_llama1b(torch, pkv, wl, steps, warmup, copies=16):
    """Llama-3.2-1B single-layer decode: batch 8, context uniform in
    [128, 2048], 4096-block pool, one new token per sequence appended then
    attended.  `copies` pool pairs (128 MiB each) are used in turn; a call
    touches 21 MB of them, so 16 copies (336 MB touched, 2 GiB allocated)
    keep the 256 MB last-level cache from holding a call's blocks for its
    next turn."""
    dev = "cuda"
    case = wl.device_decode_case("llama1b", dev, layers=copies)
    k_layers, v_layers = case.extra["k_layers"], case.extra["v_layers"]
    B, Hq, Hkv, D = case.B, case.Hq, case.Hkv, case.D
    t, l, q = case.block_tables.to(dev), case.context_lens.to(dev), case.q.to(dev)
    kn, vn = case.k_new.to(dev), case.v_new.to(dev)
    max_ctx = case.max_context_len
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = pkv.decode_workspace(B, Hq, D, max_ctx, pkv.PARTITION_AUTO, dev)

    def combined():
        for k, v in zip(k_layers, v_layers):
            pkv.paged_attention_decode_append(out, q, k, v, kn, vn, t, l, case.scale, max_ctx,
                                              pkv.PARTITION_AUTO, ws)

    def two_calls():
        for k, v in zip(k_layers, v_layers):
            pkv.kv_append(k, v, kn, vn, t, l)
            pkv.paged_attention_decode(out, q, k, v, t, l, case.scale, max_ctx,
                                       pkv.PARTITION_AUTO, ws)
    us = graph_us(torch, combined, steps, warmup, per_graph=1) / copies
    us2 = graph_us(torch, two_calls, steps, warmup, per_graph=1) / copies
    fl_us, fl_b = run_floor(torch, pkv, case, k_layers, v_layers, steps, warmup)
    nbytes = decode_bytes(case.context_lens.tolist(), B, Hq, Hkv, D, 2) + append_bytes(B, Hkv, D)
    gbs = nbytes / (us * 1e-6) / 1e9
    res = {"workload": "Llama-3.2-1B single-layer decode: batch 8, context uniform [128, 2048], "
                       "32q/8kv heads, head_dim 64, block_size 16, 4096-block pool, one new "
                       "token per sequence appended then attended",
           "context_tokens": int(case.context_lens.sum()), "algorithmic_bytes": nbytes,
           "rotation": f"{copies} pool pairs used in turn",
           "us_per_call": round(us, 2),
           "kernel": "decode_auto_kernel<true,false> (paged_attention_decode_append, automatic "
                     "split)",
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
           "two_calls_us": round(us2, 2),
           "stream_floor": floor_record(fl_us, fl_b, us)}
    del case, k_layers, v_layers
    torch.cuda.empty_cache()
    return res


def run_long_context(torch, pkv, wl, steps, warmup, copies=4):
    """Long-context split decode: 4 sequences of 32768 tokens, the query of each
    attending to its whole context, with fixed 512-token partitions merged by
    log-sum-exp (partition_size = 512), with the automatic split, and with the
    automatic split's plan (made once: the lengths and tables do not change).  `copies`
    pool pairs (256 MiB each per pool) are used in turn so that the 256 MB
    last-level cache does not hold the previous call's blocks; returns a dict."""
    dev = "cuda"
    case = wl.device_decode_case("long", dev, layers=copies)
    k_layers, v_layers = case.extra["k_layers"], case.extra["v_layers"]
    B, Hq, Hkv, D = case.B, case.Hq, case.Hkv, case.D
    t, l, q = case.block_tables.to(dev), case.context_lens.to(dev), case.q.to(dev)
    max_ctx = case.max_context_len
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    dec_b = decode_bytes(case.context_lens.tolist(), B, Hq, Hkv, D, 2)
    res = {"workload": "long-context split decode: batch 4, context 32768 each, 32q/8kv "
                       "heads, head_dim 64, block_size 16, 16384-block pool",
           "algorithmic_bytes": dec_b}
    for name, part in (("partition_512", 512), ("auto", pkv.PARTITION_AUTO),
                       ("planned", pkv.PARTITION_PLANNED)):
        ws = pkv.decode_workspace(B, Hq, D, max_ctx, part, dev)
        if part == pkv.PARTITION_PLANNED:  # lengths and tables stay fixed: plan once
            pkv.paged_attention_decode_plan(k_layers[0], t, l, Hq, max_ctx, ws)

        def calls():
            for c in range(copies):
                pkv.paged_attention_decode(out, q, k_layers[c], v_layers[c], t, l,
                                           case.scale, max_ctx, part, ws)
        us = graph_us(torch, calls, steps, warmup, per_graph=1) / copies
        gbs = dec_b / (us * 1e-6) / 1e9
        res[name] = {"us_per_call": round(us, 2),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    fl_us, fl_b = run_floor(torch, pkv, case, k_layers, v_layers, steps, warmup)
    res["stream_floor"] = floor_record(fl_us, fl_b, res["partition_512"]["us_per_call"])
    del case, k_layers, v_layers
    torch.cuda.empty_cache()
    return res


def run_mixed_batch(torch, pkv, wl, steps, warmup, copies=8):
    """One paged_attention_prefill_causal launch over a mixed continuous batch:
    60 sequences decoding one token each (context log-uniform in [16, 2048])
    and 4 prompt chunks of 256 tokens on 768 cached tokens (chunked prefill),
    32q/8kv heads, head_dim 64.  Reported on both rooflines: visible
    (query, key) pairs x 4 * D * Hq flops against bf16 MFMA peak, and K/V of
    every context token + q + out + block ids against HBM."""
    dev = "cuda"
    g = wl.generator(21)
    dec_lens = wl.draw_lens(g, 60, ("loguniform", 16, 2048)).tolist()
    prompts = [1] * 60 + [256] * 4
    history = [int(L) - 1 for L in dec_lens] + [768] * 4
    p = wl.prefill_case(seed=21, prompts=prompts, history=history, num_blocks=8192)
    t, l, cu = p.block_tables.to(dev), p.context_lens.to(dev), p.cu_q_lens.to(dev)
    # `copies` pool pairs (256 MiB each) used in turn: a call touches about 62 MB,
    # so 8 copies (500 MB touched) keep the last-level cache from holding a
    # call's blocks for its next turn
    pools = []
    for _ in range(copies):
        kc, vc = p.k_cache.to(dev), p.v_cache.to(dev)
        pkv.kv_append(kc, vc, p.k_new.to(dev), p.v_new.to(dev), t, l, cu)
        pools.append((kc, vc))
    k, v = pools[0]
    q = p.q.to(dev)
    out = torch.empty(tuple(p.q.shape), dtype=torch.bfloat16, device=dev)

    def one_launch():
        for kc, vc in pools:
            pkv.paged_attention_prefill_causal(out, q, kc, vc, t, l, cu, p.scale, max(prompts))
    us = graph_us(torch, one_launch, steps, warmup, per_graph=1) / copies
    # the same batch as two launches: the decode rows through
    # paged_attention_decode (automatic split), the chunks through the prefill
    nd = prompts.count(1)
    out2 = torch.empty_like(out)
    max_dec = max(h + 1 for h in history[:nd])
    ws = pkv.decode_workspace(nd, p.Hq, p.D, max_dec, pkv.PARTITION_AUTO, dev)
    cu_c = (cu[nd:] - cu[nd]).contiguous()

    def two_launches():
        for kc, vc in pools:
            pkv.paged_attention_decode(out2[:nd], q[:nd], kc, vc, t[:nd], l[:nd], p.scale,
                                       max_dec, pkv.PARTITION_AUTO, ws)
            pkv.paged_attention_prefill_causal(out2[nd:], q[nd:], kc, vc, t[nd:], l[nd:], cu_c,
                                               p.scale, max(prompts[nd:]))
    us2 = graph_us(torch, two_launches, steps, warmup, per_graph=1) / copies
    # the two launches on two streams (fork and join inside the graph): the
    # decode rows and the chunks write disjoint rows and only read the pools
    side = torch.cuda.Stream()

    def two_streams():
        main = torch.cuda.current_stream()
        for kc, vc in pools:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                pkv.paged_attention_decode(out2[:nd], q[:nd], kc, vc, t[:nd], l[:nd], p.scale,
                                           max_dec, pkv.PARTITION_AUTO, ws)
            pkv.paged_attention_prefill_causal(out2[nd:], q[nd:], kc, vc, t[nd:], l[nd:], cu_c,
                                               p.scale, max(prompts[nd:]))
            main.wait_stream(side)
    out2.zero_()
    us3 = graph_us(torch, two_streams, steps, warmup, per_graph=1) / copies
    if not torch.allclose(out.float(), out2.float(), atol=2e-2, rtol=0):
        raise RuntimeError("mixed batch: the two-stream form differs from the one-launch form")

    def dec_only():
        for kc, vc in pools:
            pkv.paged_attention_decode(out2[:nd], q[:nd], kc, vc, t[:nd], l[:nd], p.scale,
                                       max_dec, pkv.PARTITION_AUTO, ws)

    def pre_only():
        for kc, vc in pools:
            pkv.paged_attention_prefill_causal(out2[nd:], q[nd:], kc, vc, t[nd:], l[nd:], cu_c,
                                               p.scale, max(prompts[nd:]))
    us2_dec = graph_us(torch, dec_only, steps, warmup, per_graph=1) / copies
    us2_pre = graph_us(torch, pre_only, steps, warmup, per_graph=1) / copies
    if not torch.allclose(out.float(), out2.float(), atol=2e-2, rtol=0):
        raise RuntimeError("mixed batch: the two-launch form differs from the one-launch form")
    ctx = [h + n for h, n in zip(history, prompts)]
    pairs = sum(sum(h + i + 1 for i in range(n)) for h, n in zip(history, prompts))
    flops = pairs * p.Hq * 4 * p.D
    T = sum(prompts)
    nbytes = (sum(ctx) * p.Hkv * p.D * 2 * 2 + T * p.Hq * p.D * 2 * 2
              + sum((c + 15) // 16 for c in ctx) * 4)
    tflops = flops / (us * 1e-6) / 1e12
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "mixed batch in one prefill launch: 60 decode rows (context "
                        "log-uniform [16, 2048]) + 4 chunks of 256 tokens on 768 cached "
                        "tokens, 32q/8kv heads, head_dim 64, bf16",
            "us_per_call": round(us, 2), "flops": flops, "algorithmic_bytes": nbytes,
            "rotation": f"{copies} pool pairs used in turn",
            "roofline_mfma": {"bound": "mfma", "achieved": round(tflops, 1),
                              "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(tflops / BF16_PEAK_TFLOPS, 4)},
            "roofline_hbm": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "two_launches_us": round(us2, 2),
            "two_streams_us": round(us3, 2),
            "two_launches_parts_us": {"decode_rows": round(us2_dec, 2),
                                      "prefill_chunks": round(us2_pre, 2)},
            "two_launches": "decode rows through paged_attention_decode (automatic split), "
                            "then the chunks through paged_attention_prefill_causal; "
                            "two_streams: the same two launches on two streams"}


def run_copy_blocks(torch, pkv, wl, steps, warmup, copies=4):
    """kv_copy_blocks (copy on write of shared blocks): 64 and 2048 whole
    blocks (16 KiB of K and 16 KiB of V each, read and written) between
    disjoint random blocks of an 8192-block pool pair; `copies` pool pairs
    (256 MiB each, 1 GiB in all) are used in turn, so the copies run from
    and to HBM rather than the last-level cache."""
    dev = "cuda"
    N, Hkv, bs, D = 8192, wl.HKV, wl.BLOCK_SIZE, wl.HEAD_DIM
    pools = [(torch.zeros((N, Hkv, bs, D), dtype=torch.bfloat16, device=dev),
              torch.zeros((N, Hkv, bs, D), dtype=torch.bfloat16, device=dev))
             for _ in range(copies)]
    perm = torch.randperm(N, generator=wl.generator(41)).to(torch.int32)
    res = {"rotation": f"{copies} pool pairs used in turn"}
    for n in (64, 2048):
        src, dst = perm[:n].to(dev), perm[n:2 * n].to(dev)

        def calls():
            for k, v in pools:
                pkv.kv_copy_blocks(k, v, src, dst)
        us = graph_us(torch, calls, steps, warmup, per_graph=1) / copies
        nbytes = n * Hkv * bs * D * 2 * 2 * 2
        gbs = nbytes / (us * 1e-6) / 1e9
        res[f"blocks_{n}"] = {"us_per_call": round(us, 2), "algorithmic_bytes": nbytes,
                              "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    del pools
    torch.cuda.empty_cache()
    return res


def run_scheduler(pkv, wl, n_requests=512):
    """Host block allocator + continuous-batching scheduler (pkv_sched_*):
    512 requests (prompt log-uniform in [16, 2048] tokens, up to 16-512 new
    tokens), 65536-block pool, batch <= 64, <= 8192 tokens per step, driven
    to completion; host time per step (C++ plus the ctypes marshalling of
    the step's arrays) and the share of empty KV slots with paged blocks
    against static reservations."""
    g = wl.generator(31)
    prompt = wl.draw_lens(g, n_requests, ("loguniform", 16, 2048)).tolist()
    new = wl.draw_lens(g, n_requests, ("loguniform", 16, 512)).tolist()
    s = pkv.Scheduler(65536, wl.BLOCK_SIZE, 512, 64, 8192)
    for rid in range(n_requests):
        s.add_request(rid, int(prompt[rid]), int(new[rid]))
    n_steps = 0
    t0 = time.perf_counter()
    while n_steps < 100000:
        b = s.step()
        if len(b["seq_ids"]) == 0:
            break
        n_steps += 1
    secs = time.perf_counter() - t0
    st = s.stats()
    s.close()
    cached = st["cached_token_steps"]
    return {"workload": "512 requests, prompt log-uniform [16, 2048], new tokens log-uniform "
                        "[16, 512], 65536-block pool, batch <= 64, <= 8192 tokens per step",
            "steps": n_steps, "us_per_step": round(secs / max(n_steps, 1) * 1e6, 2),
            "finished": st["finished"], "preemptions": st["preemptions"],
            "empty_slot_share": {
                "paged": round(1 - cached / st["paged_slot_steps"], 4),
                "static_per_request_max": round(1 - cached / st["static_request_slot_steps"], 4),
                "static_max_length": round(1 - cached / st["static_max_slot_steps"], 4)}}


def rope_append_bytes(T, Hq, Hkv, D):
    """kv_append_rope: q rows read and written (when given), k_new and v_new rows read
    and stored, and the token's cos and sin rows (D/2 fp32 each)."""
    return T * ((Hq + 2 * Hkv) * D * 2 * 2 + 2 * (D // 2) * 4)


def run_rope_append(torch, pkv, wl, steps, warmup, decode_args, copies=8):
    """kv_append_rope (RoPE of q and k fused with the append) for the decode step's
    new tokens (one per sequence, decode_args = per-layer pools, tables, lens of the
    step) and for the prefill workload's prompts (6144 new tokens); `copies` sets of
    inputs and pools are used in turn (1.3 GB for the prompts), so no call finds its
    inputs in the last-level cache.  Returns a dict."""
    dev = "cuda"
    res = {"rotation": f"{copies} input sets and pool pairs used in turn"}
    k_layers, v_layers, tables, lens, B, Hq, Hkv, D = decode_args
    g = wl.generator(11)
    dec_sets = [(k_layers[i % len(k_layers)], v_layers[i % len(k_layers)],
                 wl.randn_bf16(g, (B, Hkv, D)).to(dev), wl.randn_bf16(g, (B, Hkv, D)).to(dev),
                 wl.randn_bf16(g, (B, Hq, D)).to(dev)) for i in range(copies)]
    cases = {"decode_step": (dec_sets, tables, lens, None, int(lens.max()) + 1)}
    p = wl.prefill_case()
    pre_sets = [(p.k_cache.to(dev), p.v_cache.to(dev), p.k_new.to(dev), p.v_new.to(dev),
                 p.q.to(dev)) for _ in range(copies)]
    cases["prefill"] = (pre_sets, p.block_tables.to(dev), p.context_lens.to(dev),
                        p.cu_new_lens.to(dev), int(p.context_lens.max()))
    for name, (sets, t, l, cu, max_pos) in cases.items():
        cos, sin = (x.to(dev) for x in wl.rope_tables(max_pos, D))

        def calls():
            for k, v, kn, vn, q in sets:
                pkv.kv_append_rope(k, v, kn, vn, t, l, cos, sin, q=q, cu_new_lens=cu)
        us = graph_us(torch, calls, steps, warmup, per_graph=1) / copies
        T = sets[0][2].shape[0]
        nbytes = rope_append_bytes(T, sets[0][4].shape[1], Hkv, D)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"new_tokens": T, "us_per_call": round(us, 2), "algorithmic_bytes": nbytes,
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    del pre_sets, dec_sets, cases
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_193_amd as pkv
    from paged_kv_cache_193_amd import workloads as wl

    pkv.load_library()
    dev = "cuda"
    if args.only is not None:
        steps = max(args.steps, 10)
        fn = {"prefill": run_prefill, "long": run_long_context, "mixed": run_mixed_batch,
              "llama1b": run_llama1b}[args.only]
        print(json.dumps({"only": args.only, args.only: fn(torch, pkv, wl, steps, args.warmup)}),
              flush=True)
        return
    case = wl.device_decode_case("ragged", dev, layers=LAYERS)
    k_layers, v_layers = case.extra["k_layers"], case.extra["v_layers"]
    B, Hq, Hkv, D = case.B, case.Hq, case.Hkv, case.D
    tables, lens, q = case.block_tables.to(dev), case.context_lens.to(dev), case.q.to(dev)
    k_new, v_new = case.k_new.to(dev), case.v_new.to(dev)
    max_ctx = case.max_context_len
    outs = [torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(LAYERS)]
    ws = pkv.decode_workspace(B, Hq, D, max_ctx, args.partition, dev)
    ws_plan = pkv.decode_workspace(B, Hq, D, max_ctx, pkv.PARTITION_PLANNED, dev)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def planned_calls():
        for layer in range(LAYERS):
            pkv.paged_attention_decode_append(outs[layer], q, k_layers[layer], v_layers[layer],
                                              k_new, v_new, tables, lens, case.scale, max_ctx,
                                              pkv.PARTITION_PLANNED, ws_plan)

    def planned_step():
        pkv.paged_attention_decode_plan(k_layers[0], tables, lens, Hq, max_ctx, ws_plan)
        planned_calls()

    def fused_step():
        for layer in range(LAYERS):
            pkv.paged_attention_decode_append(outs[layer], q, k_layers[layer], v_layers[layer],
                                              k_new, v_new, tables, lens, case.scale, max_ctx,
                                              args.partition, ws)

    def two_call_step():
        for layer in range(LAYERS):
            pkv.kv_append(k_layers[layer], v_layers[layer], k_new, v_new, tables, lens)
            pkv.paged_attention_decode(outs[layer], q, k_layers[layer], v_layers[layer], tables,
                                       lens, case.scale, max_ctx, args.partition, ws)

    def decode_only():
        for layer in range(LAYERS):
            pkv.paged_attention_decode(outs[layer], q, k_layers[layer], v_layers[layer], tables,
                                       lens, case.scale, max_ctx, args.partition, ws)

    forms = {"planned": planned_step, "auto": fused_step, "two-calls": two_call_step}
    step = forms[args.form]
    # Eager warm-up, then capture the step (and, for comparison, the other
    # forms of the step and the decode calls alone) in HIP graphs: host-side
    # submission of 16-32 launches would otherwise be slower than the GPU work.
    # Every step stores the same new rows again, so repeated steps see the
    # same pools.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graphs = {}
    others = [f for f in forms if f != args.form]
    for name, fn in ([("step", step)] + [(f, forms[f]) for f in others] +
                     [("decode", decode_only), ("planned calls", planned_calls)]):
        graphs[name] = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graphs[name]):
            fn()
    for name in ["step"] + others:
        graphs[name].replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(eager, outs)):
            raise RuntimeError(f"graph replay ({name}) differs from the eager step")

    # replays until the GPU's clocks have settled (WARM_S seconds), untimed
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARM_S:
        for _ in range(10):
            graphs["step"].replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graphs["step"].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    def event_us(graph, calls):
        """Average time per call of a graph's calls, HIP events on the stream
        the graph replays on."""
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        graph.replay()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            graph.replay()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / (args.steps * calls)

    decode_us = event_us(graphs["decode"], LAYERS)
    device = gpu_clocks(torch, lambda: [graphs["step"].replay() for _ in range(100)])
    other_ms = {f: round(event_us(graphs[f], 1) * 1e-3, 4) for f in others}
    lens_list = case.context_lens.tolist()
    dec_b = decode_bytes(lens_list, B, Hq, Hkv, D, 2)
    step_b = LAYERS * (dec_b + append_bytes(B, Hkv, D))
    value = step_b / (ms_per_step * 1e-3) / 1e9
    if args.form == "two-calls":
        kernel = "decode_auto_kernel<false,false> (paged_attention_decode, one launch per layer)"
        kernel_us, kernel_b = decode_us, dec_b
    elif args.form == "auto":
        kernel = ("decode_auto_kernel<true,false> (paged_attention_decode_append, one launch "
                  "per layer)")
        kernel_us, kernel_b = event_us(graphs["step"], LAYERS), dec_b + append_bytes(B, Hkv, D)
    else:
        kernel = ("decode_auto_kernel<true,true> (paged_attention_decode_append with the "
                  "step's plan, one launch per layer)")
        kernel_us = event_us(graphs["planned calls"], LAYERS)
        kernel_b = dec_b + append_bytes(B, Hkv, D)
    achieved = kernel_b / (kernel_us * 1e-6) / 1e9
    khash = source_hash("decode.hip")
    traffic = traffic_from_profiles(khash, args.form)

    result = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) and seq-tokens/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/q, log-uniform context lengths)",
        "config": {"workload": "ragged continuous-batching decode: batch 64, context "
                               "log-uniform [16, 8192], 32q/8kv heads, head_dim 64, "
                               "block_size 16, 65536-block pool per layer, 16 layers per step "
                               + {"planned": "(one plan per step, one combined append + decode "
                                             "call per layer)",
                                  "auto": "(one combined append + decode call per layer)",
                                  "two-calls": "(kv_append + decode per layer)"}[args.form],
                   "batch": B, "layers": LAYERS, "context_tokens": sum(lens_list),
                   "max_context": max_ctx,
                   "partition_size": (pkv.PARTITION_PLANNED if args.form == "planned"
                                      else args.partition)},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kernel,
                     "us_per_call": round(kernel_us, 2), "algorithmic_bytes": kernel_b,
                     "kernel_source_hash": khash},
        "other_step_forms_ms_per_step": other_ms,
        "decode_only_us_per_call": round(decode_us, 2),
        "device": device,
    }
    # the same K/V bytes through the same tables, read by a plain streaming kernel
    fl_us, fl_b = run_floor(torch, pkv, case, k_layers, v_layers, args.steps, 3)
    result["stream_floor"] = floor_record(fl_us, fl_b, kernel_us)

    if not args.no_next:
        try:
            result["llama1b_layer"] = run_llama1b(torch, pkv, wl, max(args.steps, 10),
                                                  args.warmup)
        except pkv.PagedKVError as e:
            result["llama1b_layer"] = {"error": str(e)}

    if not args.no_prefill:
        try:
            result["prefill"] = run_prefill(torch, pkv, wl, max(args.steps, 10), args.warmup)
            probe = run_mfma_probe(torch, pkv)
            probe["prefill_over_probe"] = round(
                result["prefill"]["roofline"]["achieved"] / probe["achieved"], 4)
            result["prefill"]["mfma_probe"] = probe
        except pkv.PagedKVError as e:
            result["prefill"] = {"error": str(e)}

    if not args.no_long:
        try:
            result["long_context"] = run_long_context(torch, pkv, wl, max(args.steps, 10),
                                                      args.warmup)
        except pkv.PagedKVError as e:
            result["long_context"] = {"error": str(e)}

    if not args.no_next:
        for key, fn in (("mixed_batch", lambda: run_mixed_batch(torch, pkv, wl, max(args.steps, 10),
                                                                args.warmup)),
                        ("copy_blocks", lambda: run_copy_blocks(torch, pkv, wl, max(args.steps, 10),
                                                                args.warmup)),
                        ("scheduler", lambda: run_scheduler(pkv, wl))):
            try:
                result[key] = fn()
            except pkv.PagedKVError as e:
                result[key] = {"error": str(e)}

    if not args.no_rope:
        try:
            result["rope_append"] = run_rope_append(
                torch, pkv, wl, max(args.steps, 10), args.warmup,
                (k_layers, v_layers, tables, lens, B, case.Hq, case.Hkv, case.D))
        except pkv.PagedKVError as e:
            result["rope_append"] = {"error": str(e)}

    if not args.no_cpu_baseline:
        one, many = cpu_baseline(case, k_layers, v_layers)
        result["cpu_baseline"] = {
            "value": many["value"], "unit": "GB/s", "cores": many["cores"], "kind": "oracle",
            "sample": f"{many['layer_passes']} single-layer decode passes of the same workload "
                      f"(all 64 sequences of 4 layers' pools per round), {many['seconds']} s of "
                      f"wall time on {many['cores']} host threads, each running the "
                      f"single-threaded C oracle (fp64) on whole (layer, sequence) units",
            "single_core": {"value": one["value"], "unit": "GB/s", "cores": 1,
                            "sample": f"{one['layer_passes']} single-layer passes, "
                                      f"{one['seconds']} s on one core"}}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
