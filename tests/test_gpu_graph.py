"""The library's launches captured in a HIP graph replay correctly.

A decode step (kv_append + decode with a split, and the combined
append + decode call) and a prefill are captured
once; the graph is replayed several times with eager work and
synchronisations in between, and every replay is checked against the eager
result (bit for bit: same kernels, same inputs)."""
import pytest
import torch

import paged_kv_cache_193_amd as pkv
from paged_kv_cache_193_amd import workloads as wl
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def test_decode_step_and_prefill_graph_replays():
    c = wl.decode_case("llama1b", with_append=True, poison=True)
    k, v = dev(c.k_cache), dev(c.v_cache)
    tables, lens, q = dev(c.block_tables), dev(c.context_lens), dev(c.q)
    kn, vn = dev(c.k_new), dev(c.v_new)
    out_a = torch.empty((c.B, c.Hq, c.D), dtype=torch.float32, device="cuda")
    out_f = torch.empty_like(out_a)
    ws_a = pkv.decode_workspace(c.B, c.Hq, c.D, c.max_context_len, -1, "cuda")
    ws_f = pkv.decode_workspace(c.B, c.Hq, c.D, c.max_context_len, 256, "cuda")
    p = wl.prefill_case(prompts=[70, 130], num_blocks=64, seed=81)
    kp, vp = dev(p.k_cache), dev(p.v_cache)
    tp, lp, cu, qp = dev(p.block_tables), dev(p.context_lens), dev(p.cu_q_lens), dev(p.q)
    pkv.kv_append(kp, vp, dev(p.k_new), dev(p.v_new), tp, lp, cu)
    out_p = torch.empty(tuple(p.q.shape), dtype=torch.float32, device="cuda")
    k2, v2 = dev(c.k_cache), dev(c.v_cache)
    out_c = torch.empty_like(out_a)
    ws_c = pkv.decode_workspace(c.B, c.Hq, c.D, c.max_context_len, -1, "cuda")

    def work():
        pkv.kv_append(k, v, kn, vn, tables, lens)
        pkv.paged_attention_decode(out_a, q, k, v, tables, lens, c.scale, c.max_context_len,
                                   pkv.PARTITION_AUTO, ws_a)
        pkv.paged_attention_decode(out_f, q, k, v, tables, lens, c.scale, c.max_context_len,
                                   256, ws_f)
        pkv.paged_attention_prefill_causal(out_p, qp, kp, vp, tp, lp, cu, p.scale, 130)
        pkv.paged_attention_decode_append(out_c, q, k2, v2, kn, vn, tables, lens, c.scale,
                                          c.max_context_len, pkv.PARTITION_AUTO, ws_c)

    outs = (out_a, out_f, out_p, out_c)
    work()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        # eager work between replays, on other buffers
        other = torch.empty_like(out_a)
        pkv.paged_attention_decode(other, q, k, v, tables, lens, c.scale, c.max_context_len,
                                   pkv.PARTITION_NONE)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), f"replay {rep} differs (output {i})"
