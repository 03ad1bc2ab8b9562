"""Benchmark of the paged decode hot path on one MI355X.

One step = one decode step of the ragged continuous-batching workload:
64 sequences (context log-uniform in [16, 8192], block_size 16, 65536-block
bf16 pool per layer, Llama-3.2-1B attention shapes: 32 query heads, 8 KV
heads, head_dim 64), and for each of the 16 layers
    kv_append (one new token per sequence)  ->  paged_attention_decode
with the automatic balanced split and its log-sum-exp merge.

Prints ONE JSON line.  `value` is the whole step's algorithmic HBM bytes
divided by the step time (inputs resident in HBM).  `roofline` is for the
decode call (decode kernel + merge), timed with HIP events on the stream the
kernels run on.  `cpu_baseline` is the CPU oracle on a bounded sample of the
same workload.  `prefill` reports the causal paged prefill workload
(4 x 512 + 2 x 2048 prompts) on the bf16 MFMA roofline.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for counter scaling)")
    ap.add_argument("--partition", type=int, default=-1,
                    help="decode partition_size (-1 = automatic balanced split)")
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


def traffic_from_profiles(kernel_hash):
    """HBM bytes per decode call from committed counter runs, if they were
    taken on this exact kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "decode_ragged_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_hash:
        return None
    return rec.get("bytes_per_decode_call")


def cpu_baseline(case, k_layers, v_layers, layers):
    """The oracle (single-threaded C, fp64) on `layers` full layers of the
    workload; returns GB/s over the same algorithmic bytes."""
    import oracle
    from paged_kv_cache_193_amd import workloads as wl
    total_s, total_b = 0.0, 0
    for layer in range(layers):
        kc, vc, tc = wl.compact_for_oracle(case, k_layers[layer], v_layers[layer])
        q16, k16, v16 = wl.as_u16(case.q), wl.as_u16(kc), wl.as_u16(vc)
        t0 = time.perf_counter()
        oracle.decode(q16, k16, v16, tc.numpy(), case.context_lens.numpy(), case.scale)
        total_s += time.perf_counter() - t0
        total_b += decode_bytes(case.context_lens.tolist(), case.B, case.Hq, case.Hkv, case.D, 2)
    return total_b / total_s / 1e9, total_s


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
    for _ in range(warmup):
        pkv.paged_attention_prefill_causal(out, q, k, v, t, l, cu, p.scale, maxq)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        pkv.paged_attention_prefill_causal(out, q, k, v, t, l, cu, p.scale, maxq)
        b.record()
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in ev) / steps * 1e3
    # visible (query, key) pairs: QK^T and PV, 2 flops per MAC, D = 64
    flops = sum(p.Hq * 2 * 2 * p.D * L * (L + 1) // 2 for L in qlens)
    tflops = flops / (us * 1e-6) / 1e12
    return {"workload": "causal paged prefill, prompts 4x512 + 2x2048, 32q/8kv heads, "
                        "head_dim 64, block_size 16, bf16",
            "us_per_call": round(us, 2), "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}}


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
    case = wl.device_decode_case("ragged", dev, layers=LAYERS)
    k_layers, v_layers = case.extra["k_layers"], case.extra["v_layers"]
    B, Hq, Hkv, D = case.B, case.Hq, case.Hkv, case.D
    tables, lens, q = case.block_tables.to(dev), case.context_lens.to(dev), case.q.to(dev)
    k_new, v_new = case.k_new.to(dev), case.v_new.to(dev)
    max_ctx = case.max_context_len
    outs = [torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(LAYERS)]
    ws = pkv.decode_workspace(B, Hq, Hkv, D, 16, max_ctx, args.partition, dev)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(events=None):
        for layer in range(LAYERS):
            pkv.kv_append(k_layers[layer], v_layers[layer], k_new, v_new, tables, lens)
            if events is not None:
                events[layer][0].record()
            pkv.paged_attention_decode(outs[layer], q, k_layers[layer], v_layers[layer], tables,
                                       lens, case.scale, max_ctx, args.partition, ws)
            if events is not None:
                events[layer][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(LAYERS)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    decode_us = sum(a.elapsed_time(b) for st in evs for a, b in st) / (args.steps * LAYERS) * 1e3

    lens_list = case.context_lens.tolist()
    dec_b = decode_bytes(lens_list, B, Hq, Hkv, D, 2)
    step_b = LAYERS * (dec_b + append_bytes(B, Hkv, D))
    value = step_b / (ms_per_step * 1e-3) / 1e9
    achieved = dec_b / (decode_us * 1e-6) / 1e9
    khash = source_hash("decode.hip")
    traffic = traffic_from_profiles(khash)

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
                               "(kv_append + decode each)",
                   "batch": B, "layers": LAYERS, "context_tokens": sum(lens_list),
                   "max_context": max_ctx, "partition_size": args.partition},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "paged_attention_decode (decode + merge)",
                     "us_per_call": round(decode_us, 2), "algorithmic_bytes": dec_b,
                     "kernel_source_hash": khash},
    }

    if not args.no_prefill:
        try:
            result["prefill"] = run_prefill(torch, pkv, wl, max(args.steps, 10), args.warmup)
        except pkv.PagedKVError as e:
            result["prefill"] = {"error": str(e)}

    if not args.no_cpu_baseline:
        sample_layers = 4
        gbs, secs = cpu_baseline(case, k_layers, v_layers, sample_layers)
        result["cpu_baseline"] = {
            "value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{sample_layers} of the 16 layers, all 64 sequences, decode only "
                      f"(single-threaded C oracle, fp64), {secs:.1f} s"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
