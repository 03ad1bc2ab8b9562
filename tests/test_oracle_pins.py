"""Pins of the CPU oracle against things other than itself.

The pages print no attention values, so the oracle is pinned by hand-derived
worked examples (tests/golden/worked_examples.json), closed forms, invariants
of the definition, and independent dense / library reconstructions
(tests/dense_ref.py).  Each pin is a plain function of an Oracle instance so
test_oracle_mutants.py can run the same battery against deliberately broken
builds of oracle.c and check that every planted mistake is caught.
"""
import math

import numpy as np
import pytest

import oracle
from tests import dense_ref as ref


# ----------------------------------------------------------------- inputs ---

def bits_normal(rng, shape, scale=1.0):
    """N(0, scale^2) rounded to bf16, as uint16 bit patterns."""
    import torch
    x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(shape)


def small_case(seed, B=3, Hq=8, Hkv=2, D=16, bs=4, lens=(5, 1, 13), spare=3):
    """Random paged problem: every sequence's blocks are a disjoint slice of
    a shuffled pool with `spare` unreferenced blocks."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    need = -(-lens // bs)
    N = int(need.sum()) + spare
    perm = rng.permutation(N).astype(np.int32)
    maxb = max(1, int(need.max()))
    tables = np.full((B, maxb), N - 1, dtype=np.int32)
    at = 0
    for b in range(B):
        tables[b, :need[b]] = perm[at:at + need[b]]
        at += need[b]
    q = bits_normal(rng, (B, Hq, D))
    k = bits_normal(rng, (N, Hkv, bs, D))
    v = bits_normal(rng, (N, Hkv, bs, D))
    return dict(q=q, k=k, v=v, tables=tables, lens=lens, scale=1 / math.sqrt(D))


def run_decode(orc, c, **kw):
    return orc.decode(c["q"], c["k"], c["v"], c["tables"], c["lens"], c["scale"], **kw)


def arr16(x):
    return ref.bf16_bits(np.asarray(x, dtype=np.float64))


# ------------------------------------------------------------------- pins ---

def pin_golden_decode(orc, golden):
    for ex in golden["decode"]:
        out = orc.decode(arr16(ex["q"]), arr16(ex["k_cache"]), arr16(ex["v_cache"]),
                         ex["block_tables"], ex["context_lens"], ex["scale"])
        np.testing.assert_allclose(out, ex["expected"], rtol=0, atol=1e-12, err_msg=ex["name"])


def pin_golden_prefill(orc, golden):
    for ex in golden["prefill"]:
        out = orc.prefill_causal(arr16(ex["q"]), arr16(ex["k_cache"]), arr16(ex["v_cache"]),
                                 ex["block_tables"], ex["context_lens"], ex["cu_q_lens"],
                                 ex["scale"])
        np.testing.assert_allclose(out, ex["expected"], rtol=0, atol=1e-12, err_msg=ex["name"])


def pin_golden_kv_append(orc, golden):
    for ex in golden["kv_append"]:
        shape = (ex["num_blocks"], ex["Hkv"], ex["block_size"], ex["D"])
        k = np.zeros(shape, dtype=np.uint16)
        v = np.zeros(shape, dtype=np.uint16)
        for st in ex["steps"]:
            orc.kv_append(k, v, arr16(st["k_new"]), arr16(st["v_new"]), ex["block_tables"],
                          st["context_lens"], st["cu_new_lens"])
        np.testing.assert_array_equal(k, arr16(ex["expected_k_cache"]), err_msg=ex["name"])
        np.testing.assert_array_equal(v, arr16(ex["expected_v_cache"]), err_msg=ex["name"])


def pin_golden_merge(orc, golden):
    for ex in golden["lse_merge"]:
        out = orc.lse_merge(np.array(ex["o"], float), np.array(ex["m"], float),
                            np.array(ex["l"], float))
        np.testing.assert_allclose(out, ex["expected"], rtol=0, atol=1e-12, err_msg=ex["name"])


def pin_context_one_returns_v(orc):
    """P1: a single key gets weight exactly 1, so the output is v_0 bit for bit."""
    c = small_case(11, lens=(1, 1, 1))
    out = run_decode(orc, c)
    for b in range(3):
        for h in range(8):
            blk = c["tables"][b, 0]
            expect = ref.widen(c["v"][blk, h // 4, 0])
            assert np.array_equal(out[b, h], expect)


def pin_identical_keys_give_mean(orc):
    """P2: equal scores (identical keys, or scale 0) -> arithmetic mean of V."""
    c = small_case(12, lens=(7, 16, 3))
    k = c["k"].copy()
    k[:] = k[0, :, 0:1, :]  # every slot holds the same key per KV head
    for kk, scale in ((k, c["scale"]), (c["k"], 0.0)):
        out = orc.decode(c["q"], kk, c["v"], c["tables"], c["lens"], scale)
        for b in range(3):
            n = int(c["lens"][b])
            V = ref.unpage(c["v"], c["tables"][b], n, 4)  # [Hkv][n][D]
            mean = V.mean(axis=1)
            np.testing.assert_allclose(out[b], np.repeat(mean, 4, axis=0), rtol=0, atol=1e-13)


def pin_block_permutation_invariance(orc):
    """P3: relabelling physical blocks together with the table is invisible."""
    c = small_case(13, lens=(9, 4, 15))
    base = run_decode(orc, c)
    rng = np.random.default_rng(99)
    N = c["k"].shape[0]
    perm = rng.permutation(N)
    inv = np.argsort(perm)
    k2 = c["k"][perm].copy()
    v2 = c["v"][perm].copy()
    t2 = inv[c["tables"]].astype(np.int32)
    out = orc.decode(c["q"], k2, v2, t2, c["lens"], c["scale"])
    assert np.array_equal(out, base)


def pin_online_matches_two_pass(orc):
    """P4: the online (running max / running sum) form equals the two-pass one."""
    c = small_case(14, lens=(37, 1, 64))
    a = run_decode(orc, c)
    b = run_decode(orc, c, online=True)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def pin_dense_reconstruction(orc):
    """P5: dense fp64 brute force with repeated KV heads agrees (decode)."""
    for seed, (Hq, Hkv) in ((15, (8, 2)), (16, (4, 4)), (17, (8, 1))):
        c = small_case(seed, Hq=Hq, Hkv=Hkv, lens=(6, 17, 12))
        out = run_decode(orc, c)
        exp = ref.dense_decode(c["q"], c["k"], c["v"], c["tables"], c["lens"], c["scale"])
        np.testing.assert_allclose(out, exp, rtol=0, atol=1e-12)


def prefill_small(seed, prompts=(5, 12, 1), history=(0, 0, 0), Hq=8, Hkv=2, D=16, bs=4):
    rng = np.random.default_rng(seed)
    qlens = np.asarray(prompts, dtype=np.int32)
    lens = qlens + np.asarray(history, dtype=np.int32)
    c = small_case(seed, B=len(prompts), Hq=Hq, Hkv=Hkv, D=D, bs=bs, lens=lens)
    T = int(qlens.sum())
    c["q"] = bits_normal(rng, (T, Hq, D))
    c["cu"] = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return c


def pin_prefill_dense_and_sdpa(orc):
    """P5 (prefill): explicit causal mask matrix, and torch SDPA(is_causal)."""
    c = prefill_small(18)
    args = (c["q"], c["k"], c["v"], c["tables"], c["lens"], c["cu"], c["scale"])
    out = orc.prefill_causal(*args)
    np.testing.assert_allclose(out, ref.dense_prefill(*args), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, ref.sdpa_prefill_fresh(*args), rtol=0, atol=1e-12)


def pin_prefill_with_history(orc):
    """Chunked prefill: query positions start after the cached history."""
    c = prefill_small(19, prompts=(3, 6), history=(5, 9))
    args = (c["q"], c["k"], c["v"], c["tables"], c["lens"], c["cu"], c["scale"])
    np.testing.assert_allclose(orc.prefill_causal(*args), ref.dense_prefill(*args),
                               rtol=0, atol=1e-12)


def pin_peaked_scores(orc):
    """P6: one key aligned with q at huge magnitude takes all the weight; the
    max subtraction keeps exp() finite even with scores in the thousands."""
    c = small_case(20, B=1, Hq=4, Hkv=1, lens=(10,))
    q = np.zeros_like(c["q"])
    q[0, :, :] = arr16(np.full(16, 8.0))
    k = c["k"].copy()
    blk = c["tables"][0, 2 // 4]
    k[blk, 0, 2 % 4, :] = arr16(np.full(16, 64.0))  # key 2: score 8*64*16*scale = 2048
    out = orc.decode(q, k, c["v"], c["tables"], c["lens"], c["scale"])
    assert np.all(np.isfinite(out))
    v_star = ref.widen(c["v"][blk, 0, 2 % 4])
    others = ref.unpage(k, c["tables"][0], 10, 4)[0]
    s = c["scale"] * others @ ref.widen(q[0, 0])
    bound = np.exp(s - s.max()).sum() - 1.0  # total weight of the other keys
    V = ref.unpage(c["v"], c["tables"][0], 10, 4)[0]
    np.testing.assert_allclose(out[0, 0], v_star, rtol=0, atol=2 * bound * np.abs(V).max() + 1e-12)


def pin_shift_invariance(orc):
    """P7: adding the same vector to every key shifts all scores equally."""
    rng = np.random.default_rng(21)
    c = small_case(21, lens=(9, 3, 14))
    kint = rng.integers(-4, 5, size=c["k"].shape).astype(np.float64)
    shift = rng.integers(-2, 3, size=(1, c["k"].shape[1], 1, c["k"].shape[3])).astype(np.float64)
    a = orc.decode(c["q"], arr16(kint), c["v"], c["tables"], c["lens"], c["scale"])
    b = orc.decode(c["q"], arr16(kint + shift), c["v"], c["tables"], c["lens"], c["scale"])
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def pin_affine_values_and_convexity(orc):
    """P8: v -> 2v + 1 maps the output the same way; each output lies between
    the per-dimension min and max of the visible values."""
    rng = np.random.default_rng(22)
    c = small_case(22, lens=(9, 3, 14))
    vint = rng.integers(-8, 9, size=c["v"].shape).astype(np.float64)
    a = orc.decode(c["q"], c["k"], arr16(vint), c["tables"], c["lens"], c["scale"])
    b = orc.decode(c["q"], c["k"], arr16(2 * vint + 1), c["tables"], c["lens"], c["scale"])
    np.testing.assert_allclose(b, 2 * a + 1, rtol=0, atol=1e-12)
    for bb in range(3):
        V = ref.unpage(arr16(vint), c["tables"][bb], int(c["lens"][bb]), 4)
        lo = np.repeat(V.min(axis=1), 4, axis=0)
        hi = np.repeat(V.max(axis=1), 4, axis=0)
        assert np.all(a[bb] >= lo - 1e-12) and np.all(a[bb] <= hi + 1e-12)


def relayout(pool, tables, lens, bs_old, bs_new, rng):
    """Same logical K/V, new block size, freshly shuffled physical blocks."""
    B = len(lens)
    need = [-(-int(n) // bs_new) for n in lens]
    N = sum(need) + 1
    Hkv, D = pool.shape[1], pool.shape[3]
    out = np.zeros((N, Hkv, bs_new, D), dtype=np.uint16)
    perm = rng.permutation(N - 1).astype(np.int32)
    tab = np.full((B, max(1, max(need))), N - 1, dtype=np.int32)
    at = 0
    for b in range(B):
        tab[b, :need[b]] = perm[at:at + need[b]]
        at += need[b]
        for j in range(int(lens[b])):
            src = pool[tables[b][j // bs_old], :, j % bs_old, :]
            out[tab[b, j // bs_new], :, j % bs_new, :] = src
    return out, tab


def pin_block_size_independence(orc):
    """P9: the same logical cache at block sizes 1, 4, 16, 32 -> identical bits."""
    c = small_case(23, lens=(9, 3, 33), bs=4)
    base = run_decode(orc, c)
    rng = np.random.default_rng(230)
    for bs in (1, 16, 32):
        k2, t2 = relayout(c["k"], c["tables"], c["lens"], 4, bs, rng)
        # V goes to the same slots as K under the new table
        v2 = np.zeros_like(k2)
        for b in range(3):
            for j in range(int(c["lens"][b])):
                v2[t2[b, j // bs], :, j % bs, :] = c["v"][c["tables"][b][j // 4], :, j % 4, :]
        out = orc.decode(c["q"], k2, v2, t2, c["lens"], c["scale"])
        assert np.array_equal(out, base), bs


def pin_batch_independence(orc):
    """P10: a sequence's output does not depend on the rest of the batch."""
    c = small_case(24, lens=(9, 3, 14))
    full = run_decode(orc, c)
    for b in range(3):
        alone = orc.decode(c["q"][b:b + 1], c["k"], c["v"], c["tables"][b:b + 1],
                           c["lens"][b:b + 1], c["scale"])
        assert np.array_equal(alone[0], full[b])


def pin_nan_outside_context(orc):
    """P11: NaN in slots past the context and in unreferenced blocks is never read."""
    c = small_case(25, lens=(9, 3, 14), spare=4)
    base = run_decode(orc, c)
    k, v = c["k"].copy(), c["v"].copy()
    nan = np.uint16(0x7FC0)
    used = set()
    for b in range(3):
        n = int(c["lens"][b])
        for i in range(-(-n // 4)):
            used.add(int(c["tables"][b, i]))
        if n % 4:
            last = c["tables"][b, n // 4]
            k[last, :, n % 4:, :] = nan
            v[last, :, n % 4:, :] = nan
    for blk in range(k.shape[0]):
        if blk not in used:
            k[blk], v[blk] = nan, nan
    out = orc.decode(c["q"], k, v, c["tables"], c["lens"], c["scale"])
    assert np.all(np.isfinite(out))
    assert np.array_equal(out, base)


def pin_split_merge(orc):
    """P12: per-partition partials merged by log-sum-exp equal the whole."""
    c = small_case(26, lens=(37, 5, 64))
    base = run_decode(orc, c)
    for part in (4, 8, 12, 64):
        o, m, l = orc.decode_partials(c["q"], c["k"], c["v"], c["tables"], c["lens"],
                                      c["scale"], part)
        np.testing.assert_allclose(orc.lse_merge(o, m, l), base, rtol=0, atol=1e-13)


def pin_prefill_row_is_decode(orc):
    """P13: prefill row t equals a decode whose context ends at t's position."""
    c = prefill_small(27, prompts=(6, 11), history=(3, 0))
    out = orc.prefill_causal(c["q"], c["k"], c["v"], c["tables"], c["lens"], c["cu"],
                             c["scale"])
    for b in range(2):
        qlen = int(c["cu"][b + 1] - c["cu"][b])
        for i in range(qlen):
            t = int(c["cu"][b]) + i
            pos = int(c["lens"][b]) - qlen + i
            d = orc.decode(c["q"][t:t + 1], c["k"], c["v"], c["tables"][b:b + 1],
                           [pos + 1], c["scale"])
            assert np.array_equal(d[0], out[t])


def pin_kv_append_roundtrip(orc):
    """P14: appended rows read back through the table; nothing else changes."""
    rng = np.random.default_rng(28)
    Hkv, D, bs, N = 2, 8, 4, 12
    lens_before = np.array([3, 0, 6], dtype=np.int32)
    new = np.array([2, 5, 1], dtype=np.int32)
    lens = lens_before + new
    perm = rng.permutation(N).astype(np.int32)
    tables = perm[:9].reshape(3, 3).copy()
    k = bits_normal(rng, (N, Hkv, bs, D))
    v = bits_normal(rng, (N, Hkv, bs, D))
    k0, v0 = k.copy(), v.copy()
    kn = bits_normal(rng, (int(new.sum()), Hkv, D))
    vn = bits_normal(rng, (int(new.sum()), Hkv, D))
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    orc.kv_append(k, v, kn, vn, tables, lens, cu)
    touched = np.zeros(k.shape[:3], dtype=bool)
    for b in range(3):
        for i in range(int(new[b])):
            pos = int(lens_before[b]) + i
            blk, row = tables[b, pos // bs], pos % bs
            assert np.array_equal(k[blk, :, row], kn[cu[b] + i])
            assert np.array_equal(v[blk, :, row], vn[cu[b] + i])
            touched[blk, :, row] = True
    assert np.array_equal(k[~touched], k0[~touched])
    assert np.array_equal(v[~touched], v0[~touched])
    assert touched.sum() == int(new.sum()) * Hkv
    # one-token-per-sequence form (no cu_new_lens)
    k1, v1 = k.copy(), v.copy()
    kn1 = bits_normal(rng, (3, Hkv, D))
    vn1 = bits_normal(rng, (3, Hkv, D))
    orc.kv_append(k1, v1, kn1, vn1, tables, lens + 1)
    for b in range(3):
        pos = int(lens[b])
        assert np.array_equal(k1[tables[b, pos // bs], :, pos % bs], kn1[b])


def pin_gqa(orc):
    """P15: one query head per KV head is per-head attention; duplicated query
    heads inside a group give identical rows."""
    c = small_case(29, Hq=8, Hkv=2, lens=(9, 3, 14))
    q = c["q"].copy()
    q[:, 1] = q[:, 0]
    q[:, 6] = q[:, 5]
    out = orc.decode(q, c["k"], c["v"], c["tables"], c["lens"], c["scale"])
    assert np.array_equal(out[:, 1], out[:, 0]) and np.array_equal(out[:, 6], out[:, 5])
    # MHA: split the 2 KV heads into 8 by repeating; query h must read copy h
    k8 = np.repeat(c["k"], 4, axis=1)
    v8 = np.repeat(c["v"], 4, axis=1)
    mha = orc.decode(q, k8, v8, c["tables"], c["lens"], c["scale"])
    assert np.array_equal(mha, out)


# ------------------------------------------------------------------ RoPE ---

def rope_tables(max_pos, D, base=10000.0):
    """fp32 cos/sin tables [max_pos][D/2] of the angles pos * base^(-2i/D)."""
    inv = base ** (-np.arange(D // 2, dtype=np.float64) * 2.0 / D)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def pin_rope_turns(orc):
    """Closed forms of the rotation of the pairs (i, i + D/2): a quarter turn
    maps (x, y) to (-y, x), a half turn to (-x, -y), angle 0 leaves x alone,
    and each pair takes its own table column.  An interleaved pairing, a
    flipped sign or a misplaced column changes these exact values."""
    import torch
    x = torch.tensor([[[1.0, 2.0, 3.0, 4.0]]] * 4).to(torch.bfloat16)
    x = x.view(torch.int16).numpy().view(np.uint16)
    cos = np.array([[1, 1], [0, 0], [-1, -1], [0, 1]], dtype=np.float32)
    sin = np.array([[0, 0], [1, 1], [0, 0], [1, 0]], dtype=np.float32)
    out = orc.rope(x, np.arange(4, dtype=np.int32), cos, sin)
    assert np.array_equal(out[0, 0], [1, 2, 3, 4])
    assert np.array_equal(out[1, 0], [-3, -4, 1, 2])
    assert np.array_equal(out[2, 0], [-1, -2, -3, -4])
    assert np.array_equal(out[3, 0], [-3, 2, 1, 4])


def pin_rope_is_complex_rotation(orc):
    """RoPE of the pair (a, b) is the complex product (a + ib)(cos + i sin):
    numpy's complex multiply of the same fp32 table entries agrees."""
    rng = np.random.default_rng(41)
    D, P = 16, 10
    ang = rng.uniform(-np.pi, np.pi, (P, D // 2))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    x = bits_normal(rng, (7, 3, D))
    pos = rng.integers(0, P, 7).astype(np.int32)
    out = orc.rope(x, pos, cos, sin)
    xf = ref.widen(x)
    z = (xf[..., :D // 2] + 1j * xf[..., D // 2:]) * \
        (cos[pos].astype(np.float64) + 1j * sin[pos].astype(np.float64))[:, None, :]
    assert np.allclose(out[..., :D // 2], z.real, rtol=0, atol=1e-12)
    assert np.allclose(out[..., D // 2:], z.imag, rtol=0, atol=1e-12)


def pin_rope_relative_position(orc):
    """With angles proportional to the position, q.k after RoPE depends only
    on the distance of the two positions (within the fp32 rounding of the
    tables)."""
    rng = np.random.default_rng(43)
    D = 64
    cos, sin = rope_tables(4096, D)
    q, k = bits_normal(rng, (1, 1, D)), bits_normal(rng, (1, 1, D))
    scale = float(np.linalg.norm(ref.widen(q)) * np.linalg.norm(ref.widen(k)))
    def dot(m, n):
        a = orc.rope(q, np.array([m], np.int32), cos, sin)
        b = orc.rope(k, np.array([n], np.int32), cos, sin)
        return float((a * b).sum())
    for m, n in ((7, 3), (100, 0), (2000, 1999)):
        base = dot(m, n)
        for shift in (1, 17, 1000):
            assert abs(dot(m + shift, n + shift) - base) <= 2e-5 * scale
    # and it does depend on the distance
    assert abs(dot(10, 0) - dot(0, 0)) > 1e-3 * scale


def pin_token_positions(orc):
    """New token t of the n_b new tokens of sequence b sits at
    context_lens[b] - n_b + t (the append rule); empty sequences own none."""
    pos, seq = orc.token_positions(np.array([10, 7, 3], np.int32),
                                   np.array([0, 2, 2, 5], np.int32), 5)
    assert pos.tolist() == [8, 9, 0, 1, 2] and seq.tolist() == [0, 0, 2, 2, 2]
    pos, seq = orc.token_positions(np.array([4, 1, 9], np.int32), None, 3)
    assert pos.tolist() == [3, 0, 8] and seq.tolist() == [0, 1, 2]


def pin_round_bf16(orc):
    """Rounding to bf16: torch's fp32 -> bf16 conversion (nearest even) for
    values an fp32 holds exactly, and direct rounding of the double where an
    intermediate fp32 would round twice."""
    import torch
    rng = np.random.default_rng(47)
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32),
        (rng.standard_normal(200) * 1e-39).astype(np.float32),   # fp32 subnormals
        np.float32([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 3.0e38, 3.4e38, np.inf, -np.inf,
                    0.0, -0.0, 2**-133 * 0.5, 2**-133 * 1.5])])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.round_bf16(vals.astype(np.float64)), want)
    # above the halfway point only in the double: rounds up, not to even
    assert orc.round_bf16(np.array([1 + 2**-8 + 2**-40]))[0] == 0x3F81
    assert orc.round_bf16(np.array([-(1 + 2**-8 + 2**-40)]))[0] == 0xBF81
    assert orc.round_bf16(np.array([np.nan]))[0] & 0x7FFF == 0x7FC0


def pin_kv_append_rope_steps(orc):
    """The fused operation stores round_bf16(rope(k)) and the unchanged v at
    the append slots, rotates q the same way, touches no other pool byte, and
    leaves alone a token whose position has no table row."""
    rng = np.random.default_rng(53)
    Hq, Hkv, D, bs, N = 4, 2, 8, 4, 12
    cos, sin = rope_tables(12, D)
    tables = rng.permutation(N).astype(np.int32).reshape(3, 4)
    lens = np.array([6, 13, 3], np.int32)           # after the append
    cu = np.array([0, 2, 5, 6], np.int32)           # 2, 3 and 1 new tokens
    kn, vn = bits_normal(rng, (6, Hkv, D)), bits_normal(rng, (6, Hkv, D))
    q = bits_normal(rng, (6, Hq, D))
    k = np.full((N, Hkv, bs, D), 0x7FC1, np.uint16)
    v = k.copy()
    q_rot = orc.kv_append_rope(k, v, kn, vn, tables, lens, cos, sin, q, cu)
    pos, _ = orc.token_positions(lens, cu, 6)
    assert pos.tolist() == [4, 5, 10, 11, 12, 2]
    ok = pos < 12                                    # position 12 has no table row
    touched = np.zeros((N, Hkv, bs), bool)
    for t, b in enumerate([0, 0, 1, 1, 1, 2]):
        if not ok[t]:
            assert np.array_equal(q_rot[t], q[t])
            continue
        blk, row = tables[b, pos[t] // bs], pos[t] % bs
        kr = orc.round_bf16(orc.rope(kn[t:t + 1], pos[t:t + 1], cos, sin))[0]
        qr = orc.round_bf16(orc.rope(q[t:t + 1], pos[t:t + 1], cos, sin))[0]
        assert np.array_equal(k[blk, :, row], kr) and np.array_equal(v[blk, :, row], vn[t])
        assert np.array_equal(q_rot[t], qr)
        touched[blk, :, row] = True
    assert (k[~touched] == 0x7FC1).all() and (v[~touched] == 0x7FC1).all()
    assert touched.sum() == int(ok.sum()) * Hkv


def pin_copy_blocks(orc):
    """Copy on write: the destination block holds the source's bytes in both
    pools afterwards, every other byte keeps its value, and pairs apply in
    order (a copy of a copy carries the first source)."""
    rng = np.random.default_rng(59)
    k = bits_normal(rng, (6, 2, 4, 8))
    v = bits_normal(rng, (6, 2, 4, 8))
    k0, v0 = k.copy(), v.copy()
    orc.copy_blocks(k, v, [4, 1, 2], [0, 5, 3])
    assert np.array_equal(k[0], k0[4]) and np.array_equal(v[0], v0[4])
    assert np.array_equal(k[5], k0[1]) and np.array_equal(v[5], v0[1])
    assert np.array_equal(k[3], k0[2]) and np.array_equal(v[3], v0[2])
    for blk in (1, 2, 4):
        assert np.array_equal(k[blk], k0[blk]) and np.array_equal(v[blk], v0[blk])
    orc.copy_blocks(k, v, [0, 3], [1, 0])
    assert np.array_equal(k[1], k0[4]) and np.array_equal(k[0], k0[2])
    with pytest.raises(ValueError):
        orc.copy_blocks(k, v, [6], [0])


PINS = [
    pin_golden_decode, pin_golden_prefill, pin_golden_kv_append, pin_golden_merge,
    pin_context_one_returns_v, pin_identical_keys_give_mean,
    pin_block_permutation_invariance, pin_online_matches_two_pass,
    pin_dense_reconstruction, pin_prefill_dense_and_sdpa, pin_prefill_with_history,
    pin_peaked_scores, pin_shift_invariance, pin_affine_values_and_convexity,
    pin_block_size_independence, pin_batch_independence, pin_nan_outside_context,
    pin_split_merge, pin_prefill_row_is_decode, pin_kv_append_roundtrip, pin_gqa,
    pin_rope_turns, pin_rope_is_complex_rotation, pin_rope_relative_position,
    pin_token_positions, pin_round_bf16, pin_kv_append_rope_steps, pin_copy_blocks,
]
NEEDS_GOLDEN = {pin_golden_decode, pin_golden_prefill, pin_golden_kv_append, pin_golden_merge}


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin, golden):
    orc = oracle.default()
    if pin in NEEDS_GOLDEN:
        pin(orc, golden)
    else:
        pin(orc)
