"""Independent dense reconstructions used to pin the oracle.

These take a different route from oracle.c on purpose: numpy fancy indexing
un-pages the cache into dense [L][D] matrices, GQA is done by repeating KV
heads, the causal rule is an explicit boolean mask matrix, and softmax is a
vectorised row operation.  torch's scaled_dot_product_attention on the CPU in
float64 is a second, library-side check.
"""
import numpy as np
import torch


def widen(u16) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits(x) -> np.ndarray:
    """float values (exactly representable in bf16) -> uint16 bit patterns."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    back = t.to(torch.float32).numpy()
    assert np.array_equal(back, np.asarray(x, dtype=np.float32)), "value not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def unpage(pool_u16, table_row, n, block_size) -> np.ndarray:
    """Dense [Hkv][n][D] float64 of the first n logical tokens of one sequence."""
    j = np.arange(n)
    blocks = np.asarray(table_row)[j // block_size]
    rows = j % block_size
    return widen(pool_u16[blocks, :, rows, :]).transpose(1, 0, 2)


def softmax_rows(s, mask=None):
    s = np.array(s, dtype=np.float64)
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    top = s.max(axis=-1, keepdims=True)
    top = np.where(np.isfinite(top), top, 0.0)
    e = np.exp(s - top)
    if mask is not None:
        e = np.where(mask, e, 0.0)
    tot = e.sum(axis=-1, keepdims=True)
    return np.divide(e, tot, out=np.zeros_like(e), where=tot > 0)


def dense_decode(q_u16, k_u16, v_u16, tables, lens, scale):
    """[B][Hq][D] via dense per-sequence matrices and repeated KV heads."""
    B, Hq, D = q_u16.shape
    Hkv, bs = k_u16.shape[1], k_u16.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        K = np.repeat(unpage(k_u16, tables[b], n, bs), G, axis=0)  # [Hq][n][D]
        V = np.repeat(unpage(v_u16, tables[b], n, bs), G, axis=0)
        q = widen(q_u16[b])                                         # [Hq][D]
        s = scale * np.einsum("hd,hnd->hn", q, K)
        out[b] = np.einsum("hn,hnd->hd", softmax_rows(s), V)
    return out


def dense_prefill(q_u16, k_u16, v_u16, tables, lens, cu_q, scale):
    """[T][Hq][D] with an explicit causal mask matrix (query position >= key)."""
    T, Hq, D = q_u16.shape
    Hkv, bs = k_u16.shape[1], k_u16.shape[2]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    for b in range(len(lens)):
        t0, t1 = int(cu_q[b]), int(cu_q[b + 1])
        n, qlen = int(lens[b]), t1 - t0
        K = np.repeat(unpage(k_u16, tables[b], n, bs), G, axis=0)
        V = np.repeat(unpage(v_u16, tables[b], n, bs), G, axis=0)
        q = widen(q_u16[t0:t1]).transpose(1, 0, 2)                  # [Hq][qlen][D]
        qpos = (n - qlen) + np.arange(qlen)
        mask = qpos[:, None] >= np.arange(n)[None, :]                # [qlen][n]
        s = scale * np.einsum("hqd,hnd->hqn", q, K)
        o = np.einsum("hqn,hnd->hqd", softmax_rows(s, mask[None]), V)
        out[t0:t1] = o.transpose(1, 0, 2)
    return out


def sdpa_prefill_fresh(q_u16, k_u16, v_u16, tables, lens, cu_q, scale):
    """torch SDPA (CPU, float64, is_causal) for prompts with no history."""
    T, Hq, D = q_u16.shape
    Hkv, bs = k_u16.shape[1], k_u16.shape[2]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    for b in range(len(lens)):
        t0, t1 = int(cu_q[b]), int(cu_q[b + 1])
        n = int(lens[b])
        assert n == t1 - t0
        K = torch.from_numpy(np.repeat(unpage(k_u16, tables[b], n, bs), G, axis=0))
        V = torch.from_numpy(np.repeat(unpage(v_u16, tables[b], n, bs), G, axis=0))
        q = torch.from_numpy(widen(q_u16[t0:t1]).transpose(1, 0, 2).copy())
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None], K[None], V[None], is_causal=True, scale=scale)[0]
        out[t0:t1] = o.permute(1, 0, 2).numpy()
    return out
