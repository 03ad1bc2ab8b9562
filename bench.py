"""Benchmark of the paged decode hot path on one MI355X.

One step = one decode step of the ragged continuous-batching workload:
64 sequences (context log-uniform in [16, 8192], block_size 16, 65536-block
bf16 pool per layer, Llama-3.2-1B attention shapes: 32 query heads, 8 KV
heads, head_dim 64): one paged_attention_decode_plan (the balanced split's
plan for this step's lengths and tables, shared by every layer), then for
each of the 16 layers one
    paged_attention_decode_append(..., PKV_PARTITION_PLANNED)
call: store one new token per sequence (kv_append) and attend to the whole
context (paged_attention_decode) with the balanced split, in one kernel
launch whose log-sum-exp merge runs inside the kernel.  `--form auto` times
the same calls without a plan, `--form two-calls` kv_append followed by
paged_attention_decode per layer.  The step is captured once in a HIP graph
and replayed.

Prints ONE JSON line.  `value` is the whole step's algorithmic HBM bytes
divided by the step time (inputs resident in HBM).  `roofline` is for the
dominant kernel -- the combined append + decode kernel (the decode kernel
with --form two-calls) -- timed with HIP events over graph replays of its 16
calls on the stream the graph runs on.  `cpu_baseline` is the CPU oracle on
a bounded sample of the same workload.  `prefill` reports the causal paged
prefill workload (4 x 512 + 2 x 2048 prompts) on the bf16 MFMA roofline, and
`rope_append` the rotary embedding of q and k fused with the append
(kv_append_rope) for the step's 64 new tokens and for the prefill prompts'
6144, on the HBM roofline.  `long_context` times the long-context split
workload (4 sequences of 32768 tokens) with fixed 512-token partitions merged
by log-sum-exp, with the balanced split, and with the balanced split's plan
(made once, outside the timed calls), on the HBM roofline.  `mixed_batch`
times one prefill launch over decode rows and prompt chunks together,
`copy_blocks` kv_copy_blocks (copy on write), and `scheduler` the host
block allocator and continuous-batching scheduler per step.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--form planned|auto|two-calls]

Every timed region follows W eager warm-up steps and at least WARM_S seconds
of untimed graph replays, so the figures are sustained rates.
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
                    help="decode partition_size (-1 = automatic balanced split)")
    ap.add_argument("--only", choices=("prefill", "long", "mixed"), default=None,
                    help="run this one leg alone and print its JSON object (for profiling "
                         "a single kernel); the contract line is not printed")
    return ap.parse_args()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_193_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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


def cpu_baseline(case, k_layers, v_layers, min_seconds=10.0):
    """The oracle (single-threaded C, fp64) on whole layers of the workload,
    cycling through the layers until at least `min_seconds` of CPU work;
    returns (GB/s over the same algorithmic bytes, seconds, layer passes)."""
    import oracle
    from paged_kv_cache_193_amd import workloads as wl
    total_s, total_b, passes = 0.0, 0, 0
    compact = {}
    while total_s < min_seconds and passes < 256:
        layer = passes % len(k_layers)
        if layer not in compact:
            kc, vc, tc = wl.compact_for_oracle(case, k_layers[layer], v_layers[layer])
            compact[layer] = (wl.as_u16(kc), wl.as_u16(vc), tc.numpy())
        k16, v16, tables = compact[layer]
        t0 = time.perf_counter()
        oracle.decode(wl.as_u16(case.q), k16, v16, tables, case.context_lens.numpy(), case.scale)
        total_s += time.perf_counter() - t0
        total_b += decode_bytes(case.context_lens.tolist(), case.B, case.Hq, case.Hkv, case.D, 2)
        passes += 1
    return total_b / total_s / 1e9, total_s, passes


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


def run_prefill(torch, pkv, wl, steps, warmup):
    """Causal paged prefill of 4 x 512 + 2 x 2048 prompts; returns a dict."""
    dev = "cuda"
    p = wl.prefill_case()
    k, v = p.k_cache.to(dev), p.v_cache.to(dev)
    t, l, cu = p.block_tables.to(dev), p.context_lens.to(dev), p.cu_q_lens.to(dev)
    pkv.kv_append(k, v, p.k_new.to(dev), p.v_new.to(dev), t, l, cu)
    q = p.q.to(dev)
    out = torch.empty(tuple(p.q.shape), dtype=torch.bfloat16, device=dev)
    qlens = (p.cu_q_lens[1:] - p.cu_q_lens[:-1]).tolist()
    maxq = max(qlens)
    us = graph_us(torch, lambda: pkv.paged_attention_prefill_causal(
        out, q, k, v, t, l, cu, p.scale, maxq), steps, warmup)
    # visible (query, key) pairs: QK^T and PV, 2 flops per MAC, D = 64
    flops = sum(p.Hq * 2 * 2 * p.D * L * (L + 1) // 2 for L in qlens)
    tflops = flops / (us * 1e-6) / 1e12
    return {"workload": "causal paged prefill, prompts 4x512 + 2x2048, 32q/8kv heads, "
                        "head_dim 64, block_size 16, bf16",
            "us_per_call": round(us, 2), "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}}


def run_long_context(torch, pkv, wl, steps, warmup, copies=4):
    """Long-context split decode: 4 sequences of 32768 tokens, the query of each
    attending to its whole context, with fixed 512-token partitions merged by
    log-sum-exp (partition_size = 512), with the balanced split, and with the
    balanced split's plan (made once: the lengths and tables do not change).  `copies`
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
    del case, k_layers, v_layers
    torch.cuda.empty_cache()
    return res


def run_mixed_batch(torch, pkv, wl, steps, warmup):
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
    k, v = p.k_cache.to(dev), p.v_cache.to(dev)
    t, l, cu = p.block_tables.to(dev), p.context_lens.to(dev), p.cu_q_lens.to(dev)
    pkv.kv_append(k, v, p.k_new.to(dev), p.v_new.to(dev), t, l, cu)
    q = p.q.to(dev)
    out = torch.empty(tuple(p.q.shape), dtype=torch.bfloat16, device=dev)
    us = graph_us(torch, lambda: pkv.paged_attention_prefill_causal(
        out, q, k, v, t, l, cu, p.scale, max(prompts)), steps, warmup)
    # the same batch as two launches: the decode rows through
    # paged_attention_decode (balanced split), the chunks through the prefill
    nd = prompts.count(1)
    out2 = torch.empty_like(out)
    max_dec = max(h + 1 for h in history[:nd])
    ws = pkv.decode_workspace(nd, p.Hq, p.D, max_dec, pkv.PARTITION_AUTO, dev)
    cu_c = (cu[nd:] - cu[nd]).contiguous()

    def two_launches():
        pkv.paged_attention_decode(out2[:nd], q[:nd], k, v, t[:nd], l[:nd], p.scale, max_dec,
                                   pkv.PARTITION_AUTO, ws)
        pkv.paged_attention_prefill_causal(out2[nd:], q[nd:], k, v, t[nd:], l[nd:], cu_c,
                                           p.scale, max(prompts[nd:]))
    us2 = graph_us(torch, two_launches, steps, warmup)
    # the two launches on two streams (fork and join inside the graph): the
    # decode rows and the chunks write disjoint rows and only read the pools
    side = torch.cuda.Stream()

    def two_streams():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            pkv.paged_attention_decode(out2[:nd], q[:nd], k, v, t[:nd], l[:nd], p.scale,
                                       max_dec, pkv.PARTITION_AUTO, ws)
        pkv.paged_attention_prefill_causal(out2[nd:], q[nd:], k, v, t[nd:], l[nd:], cu_c,
                                           p.scale, max(prompts[nd:]))
        main.wait_stream(side)
    out2.zero_()
    us3 = graph_us(torch, two_streams, steps, warmup)
    if not torch.allclose(out.float(), out2.float(), atol=2e-2, rtol=0):
        raise RuntimeError("mixed batch: the two-stream form differs from the one-launch form")
    us2_dec = graph_us(torch, lambda: pkv.paged_attention_decode(
        out2[:nd], q[:nd], k, v, t[:nd], l[:nd], p.scale, max_dec, pkv.PARTITION_AUTO, ws),
        steps, warmup)
    us2_pre = graph_us(torch, lambda: pkv.paged_attention_prefill_causal(
        out2[nd:], q[nd:], k, v, t[nd:], l[nd:], cu_c, p.scale, max(prompts[nd:])), steps, warmup)
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
            "roofline_mfma": {"bound": "mfma", "achieved": round(tflops, 1),
                              "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(tflops / BF16_PEAK_TFLOPS, 4)},
            "roofline_hbm": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "two_launches_us": round(us2, 2),
            "two_streams_us": round(us3, 2),
            "two_launches_parts_us": {"decode_rows": round(us2_dec, 2),
                                      "prefill_chunks": round(us2_pre, 2)},
            "two_launches": "decode rows through paged_attention_decode (balanced split), "
                            "then the chunks through paged_attention_prefill_causal; "
                            "two_streams: the same two launches on two streams"}


def run_copy_blocks(torch, pkv, wl, steps, warmup):
    """kv_copy_blocks (copy on write of shared blocks): 64 and 2048 whole
    blocks (16 KiB of K and 16 KiB of V each, read and written) between
    disjoint random blocks of an 8192-block pool pair."""
    dev = "cuda"
    N, Hkv, bs, D = 8192, wl.HKV, wl.BLOCK_SIZE, wl.HEAD_DIM
    k = torch.zeros((N, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    perm = torch.randperm(N, generator=wl.generator(41)).to(torch.int32)
    res = {}
    for n in (64, 2048):
        src, dst = perm[:n].to(dev), perm[n:2 * n].to(dev)
        us = graph_us(torch, lambda: pkv.kv_copy_blocks(k, v, src, dst), steps, warmup)
        nbytes = n * Hkv * bs * D * 2 * 2 * 2
        gbs = nbytes / (us * 1e-6) / 1e9
        res[f"blocks_{n}"] = {"us_per_call": round(us, 2), "algorithmic_bytes": nbytes,
                              "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": round(gbs / HBM_PEAK_GBS, 4)}}
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


def run_rope_append(torch, pkv, wl, steps, warmup, decode_args):
    """kv_append_rope (RoPE of q and k fused with the append) for the decode step's
    new tokens (one per sequence, decode_args = pools, tables, lens of the step) and for
    the prefill workload's prompts (6144 new tokens); returns a dict."""
    dev = "cuda"
    res = {}
    k_pool, v_pool, tables, lens, B, Hq, Hkv, D = decode_args
    g = wl.generator(11)
    cases = {"decode_step": (k_pool, v_pool, wl.randn_bf16(g, (B, Hkv, D)).to(dev),
                             wl.randn_bf16(g, (B, Hkv, D)).to(dev), tables, lens, None,
                             wl.randn_bf16(g, (B, Hq, D)).to(dev), int(lens.max()) + 1)}
    p = wl.prefill_case()
    cases["prefill"] = (p.k_cache.to(dev), p.v_cache.to(dev), p.k_new.to(dev),
                        p.v_new.to(dev), p.block_tables.to(dev), p.context_lens.to(dev),
                        p.cu_new_lens.to(dev), p.q.to(dev), int(p.context_lens.max()))
    for name, (k, v, kn, vn, t, l, cu, q, max_pos) in cases.items():
        cos, sin = (x.to(dev) for x in wl.rope_tables(max_pos, D))
        def call():
            pkv.kv_append_rope(k, v, kn, vn, t, l, cos, sin, q=q, cu_new_lens=cu)
        us = graph_us(torch, call, steps, warmup)
        T = kn.shape[0]
        nbytes = rope_append_bytes(T, q.shape[1], Hkv, D)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"new_tokens": T, "us_per_call": round(us, 2), "algorithmic_bytes": nbytes,
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_193_amd as pkv
    from paged_kv_cache_193_amd import workloads as wl

    pkv.load_library()
    dev = "cuda"
    if args.only is not None:
        steps = max(args.steps, 10)
        fn = {"prefill": run_prefill, "long": run_long_context, "mixed": run_mixed_batch}[args.only]
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
                   "max_context": max_ctx, "partition_size": args.partition},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kernel,
                     "us_per_call": round(kernel_us, 2), "algorithmic_bytes": kernel_b,
                     "kernel_source_hash": khash},
        "other_step_forms_ms_per_step": other_ms,
        "decode_only_us_per_call": round(decode_us, 2),
    }

    if not args.no_prefill:
        try:
            result["prefill"] = run_prefill(torch, pkv, wl, max(args.steps, 10), args.warmup)
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
                (k_layers[0], v_layers[0], tables, lens, B, case.Hq, case.Hkv, case.D))
        except pkv.PagedKVError as e:
            result["rope_append"] = {"error": str(e)}

    if not args.no_cpu_baseline:
        gbs, secs, passes = cpu_baseline(case, k_layers, v_layers)
        result["cpu_baseline"] = {
            "value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} single-layer decode passes (all 64 sequences, layers taken in "
                      f"turn) of the same workload, {secs:.1f} s on one host core "
                      f"(single-threaded C oracle, fp64)"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
