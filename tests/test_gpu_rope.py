"""kv_append_rope on the GPU against the oracle's steps (token positions,
RoPE in double precision, rounding to bf16, kv_append).

The GPU rounds each product and the difference to fp32 before rounding to
bf16; the oracle rounds the exact value once.  The fp32 steps are off by at
most 2^-23 (|x| + |y|) for a pair (x, y) (two products of magnitude at most
|x| and |y|, then their sum), so after rounding to bf16 the two results are
within one bf16 ulp plus that amount (twice it is allowed here): they differ
only where the exact value
lies that close to a bf16 rounding boundary, or where x cos and y sin nearly
cancel.  So: every rotated element within that bound, at most 0.1% of them
unequal at all, and V rows and every pool byte the call does not store
bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_193_amd as pkv
from paged_kv_cache_193_amd import workloads as wl
from tests.gpu_util import dev, u16

pytestmark = pytest.mark.gpu


def as_f64(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def assert_rotation_close(got, want, x, what):
    """Rotated rows [..][D] as bf16 bits against the oracle's, x the input
    rows (bf16 bits) they were rotated from."""
    g, w = as_f64(np.ascontiguousarray(got)), as_f64(np.ascontiguousarray(want))
    xf = as_f64(np.ascontiguousarray(x))
    half = xf.shape[-1] // 2
    partner = np.concatenate([xf[..., half:], xf[..., :half]], axis=-1)
    bound = (np.maximum(np.abs(w), np.abs(g)) * 2.0 ** -7 +
             2.0 ** -22 * (np.abs(xf) + np.abs(partner)))
    diff = np.abs(g - w)
    far = ~(diff <= bound)
    unequal = int((got != want).sum())
    print(f"  {what}: {unequal} of {got.size} differ (max {diff.max(initial=0):.3e})", flush=True)
    assert not far.any(), f"{what}: {far.sum()} values outside the bound"
    assert unequal <= max(1, got.size // 1000), f"{what}: {unequal} values differ"


def run_case(k_cache, v_cache, k_new, v_new, tables, lens, cu, q, cos, sin):
    """GPU call on device copies and the oracle's steps on host copies."""
    k_d, v_d = dev(k_cache), dev(v_cache)
    q_d = dev(q).contiguous() if q is not None else None
    pkv.kv_append_rope(k_d, v_d, dev(k_new), dev(v_new), dev(tables), dev(lens), dev(cos),
                       dev(sin), q=q_d, cu_new_lens=dev(cu))
    torch.cuda.synchronize()
    k_ref, v_ref = u16(k_cache).copy(), u16(v_cache).copy()
    q_ref = oracle.kv_append_rope(k_ref, v_ref, u16(k_new), u16(v_new), tables.numpy(),
                                  lens.numpy(), cos.numpy(), sin.numpy(),
                                  None if q is None else u16(q),
                                  None if cu is None else cu.numpy())
    got_q = None if q_d is None else u16(q_d.cpu())
    ctx = dict(k_new=u16(k_new), q=None if q is None else u16(q), tables=tables.numpy(),
               lens=lens.numpy(), cu=None if cu is None else cu.numpy(),
               max_position=cos.shape[0], bs=k_cache.shape[2], N=k_cache.shape[0])
    return (u16(k_d.cpu()), u16(v_d.cpu()), got_q), (k_ref, v_ref, q_ref), ctx


def stored_slots(ctx):
    """(token, block, row) of every token whose K/V the call stores."""
    T = ctx["k_new"].shape[0]
    pos, seq = oracle.token_positions(ctx["lens"], ctx["cu"], T)
    out = []
    for t in range(T):
        p = int(pos[t])
        if p < 0 or p >= ctx["max_position"]:
            continue
        lb = p // ctx["bs"]
        if lb >= ctx["tables"].shape[1]:
            continue
        blk = int(ctx["tables"][seq[t], lb])
        if 0 <= blk < ctx["N"]:
            out.append((t, blk, p % ctx["bs"]))
    return out


def check(result, what):
    (gk, gv, gq), (rk, rv, rq), ctx = result
    assert np.array_equal(gv, rv), f"{what}: V pool differs"
    slots = stored_slots(ctx)
    tok = np.array([s[0] for s in slots], dtype=np.int64)
    blk = np.array([s[1] for s in slots], dtype=np.int64)
    row = np.array([s[2] for s in slots], dtype=np.int64)
    # rotated K rows, element by element against the bound
    assert_rotation_close(gk[blk, :, row], rk[blk, :, row], ctx["k_new"][tok], f"{what} K rows")
    # every other K pool byte is bit-identical
    mask = np.ones(gk.shape[:3], dtype=bool)
    mask[blk, :, row] = False
    assert np.array_equal(gk[mask], rk[mask]), f"{what}: K pool outside the stored rows differs"
    if gq is not None:
        assert_rotation_close(gq, rq, ctx["q"], f"{what} q")


def ragged_case(seed, new, lens, num_blocks=256, max_blocks=16, Hq=32):
    g = wl.generator(seed)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    tables = wl.tables_from_permutation(g, lens_t, 16, num_blocks, max_blocks,
                                        filler=num_blocks - 1)
    cu = torch.zeros(len(new) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(new, dtype=torch.int32), 0)
    T = int(cu[-1])
    k_cache = wl.randn_bf16(g, (num_blocks, 8, 16, 64))
    v_cache = wl.randn_bf16(g, (num_blocks, 8, 16, 64))
    k_new, v_new = wl.randn_bf16(g, (T, 8, 64)), wl.randn_bf16(g, (T, 8, 64))
    q = wl.randn_bf16(g, (T, Hq, 64))
    return k_cache, v_cache, k_new, v_new, tables, lens_t, cu, q


@pytest.mark.parametrize("with_q", [True, False])
def test_ragged_new_tokens(with_q):
    """Several new tokens per sequence, one sequence without any, positions
    crossing block boundaries."""
    kc, vc, kn, vn, tables, lens, cu, q = ragged_case(91, [1, 7, 0, 16, 33], [10, 7, 3, 40, 100])
    cos, sin = wl.rope_tables(256)
    check(run_case(kc, vc, kn, vn, tables, lens, cu, q if with_q else None, cos, sin),
          f"ragged q={with_q}")


@pytest.mark.parametrize("B", [1, 2, 64, 65, 130])
def test_many_sequences(B):
    """Batch sizes on both sides of 64 sequences: up to 64 a wavefront finds
    each token's sequence from one read of the lengths, beyond that by
    binary search.  Sequences without new tokens, alone and in a run (equal
    consecutive cu_new_lens entries), must not capture any token."""
    g = np.random.default_rng(930 + B)
    new = g.integers(0, 6, B)
    if B > 8:
        new[::7] = 0
        new[B // 2:B // 2 + 5] = 0
    else:
        new = np.maximum(new, 1)
    lens = (new + g.integers(0, 60, B)).tolist()
    kc, vc, kn, vn, tables, lens_t, cu, q = ragged_case(93 + B, new.tolist(), lens,
                                                        num_blocks=1024, max_blocks=8)
    cos, sin = wl.rope_tables(64)
    check(run_case(kc, vc, kn, vn, tables, lens_t, cu, q, cos, sin), f"{B} sequences")


def test_one_token_per_sequence():
    """Decode-step form: cu_new_lens NULL, llama1b decode shapes."""
    c = wl.decode_case("llama1b", with_append=True)
    cos, sin = wl.rope_tables(int(c.context_lens.max()) + 1)
    q = c.q.clone()
    check(run_case(c.k_cache, c.v_cache, c.k_new, c.v_new, c.block_tables, c.context_lens,
                   None, q, cos, sin), "decode step")


def test_prefill_full_size():
    """The prefill workload's append (6144 new tokens over 6 prompts) with
    its queries, every row compared."""
    c = wl.prefill_case()
    cos, sin = wl.rope_tables(2048)
    check(run_case(c.k_cache, c.v_cache, c.k_new, c.v_new, c.block_tables, c.context_lens,
                   c.cu_new_lens, c.q, cos, sin), "prefill")


def test_positions_without_table_row_are_left_alone():
    """Tokens past the angle table: q rows unchanged, K/V not stored."""
    kc, vc, kn, vn, tables, lens, cu, q = ragged_case(92, [4, 9, 2], [30, 9, 200])
    cos, sin = wl.rope_tables(28)   # positions 26..29 and 198..199 have no row
    result = run_case(kc, vc, kn, vn, tables, lens, cu, q, cos, sin)
    check(result, "short table")
    pos, _ = oracle.token_positions(lens.numpy(), cu.numpy(), int(cu[-1]))
    off = pos >= 28
    assert off.any()
    assert np.array_equal(result[0][2][off], u16(q)[off])
    assert len(stored_slots(result[2])) == int((~off).sum())


def test_zero_angle_is_kv_append():
    """cos = 1, sin = 0: the pools equal plain kv_append (values compared, so
    a zero's sign may differ) and q is unchanged."""
    kc, vc, kn, vn, tables, lens, cu, q = ragged_case(93, [3, 5], [20, 5])
    cos = torch.ones(64, 32, dtype=torch.float32)
    sin = torch.zeros(64, 32, dtype=torch.float32)
    k1, v1, q1 = dev(kc), dev(vc), dev(q)
    pkv.kv_append_rope(k1, v1, dev(kn), dev(vn), dev(tables), dev(lens), dev(cos), dev(sin),
                       q=q1, cu_new_lens=dev(cu))
    k2, v2 = dev(kc), dev(vc)
    pkv.kv_append(k2, v2, dev(kn), dev(vn), dev(tables), dev(lens), dev(cu))
    torch.cuda.synchronize()
    assert torch.equal(k1.float(), k2.float()) and torch.equal(v1.view(torch.int16),
                                                               v2.view(torch.int16))
    assert torch.equal(q1.float(), dev(q).float())


def test_rejects_bad_tables():
    kc, vc, kn, vn, tables, lens, cu, q = ragged_case(94, [2], [5])
    cos, sin = wl.rope_tables(16)
    with pytest.raises(ValueError):
        pkv.kv_append_rope(dev(kc), dev(vc), dev(kn), dev(vn), dev(tables), dev(lens),
                           dev(cos[:, :16]), dev(sin[:, :16]), cu_new_lens=dev(cu))
    with pytest.raises(TypeError):
        pkv.kv_append_rope(dev(kc), dev(vc), dev(kn), dev(vn), dev(tables), dev(lens),
                           dev(cos.double()), dev(sin.double()), cu_new_lens=dev(cu))
