"""Seeded synthetic workloads for paged KV-cache attention.

This module only draws random numbers and builds block tables; it holds no
attention arithmetic.  Both the HIP path and the CPU oracle consume exactly
what it produces (bf16 tensors, int32 tables), so their results can be
compared element by element.

Draw order inside one case is fixed: context lengths, block permutation,
q, K pool, V pool, new K/V.  Normal draws are fp32 N(0,1) from a seeded
torch generator, rounded to bf16 (round-to-nearest-even by torch).

Workloads (Llama-3.2-1B attention shapes: 32 query heads, 8 KV heads,
head_dim 64, bf16; block_size 16):
  tiny      1 sequence, 4 query heads / 1 KV head, context 37, 8 physical
            blocks in a seeded permutation, scale 1/8
  llama1b   batch 8, context ~ U{128..2048}, 4096-block pool, tables are
            disjoint slices of a seeded permutation; one appended token per
            sequence
  ragged    batch 64, context log-uniform in [16, 8192], 65536-block pool per
            layer, 16 layers; one shared table for all layers
  long      batch 4, context 32768 each, 16384-block pool, 512-token
            partitions
  prefill   prompts 4 x 512 + 2 x 2048, K/V appended into shuffled blocks of a
            4096-block pool, causal
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

HQ, HKV, HEAD_DIM, BLOCK_SIZE = 32, 8, 64, 16
SCALE = 0.125  # 1 / sqrt(64)
# Base of the rotary frequencies in the synthetic angle tables (the value of
# the Llama 3 family; its long-context frequency scaling is left out: the
# library takes whatever tables the caller builds).
ROPE_BASE = 500000.0

CONFIGS = {
    "tiny": dict(B=1, Hq=4, Hkv=1, num_blocks=8, lens=("fixed", 37), seed=1),
    "llama1b": dict(B=8, Hq=HQ, Hkv=HKV, num_blocks=4096, lens=("uniform", 128, 2048),
                    max_blocks=128, seed=2),
    "ragged": dict(B=64, Hq=HQ, Hkv=HKV, num_blocks=65536,
                   lens=("loguniform", 16, 8192), max_blocks=512, layers=16, seed=3),
    "long": dict(B=4, Hq=HQ, Hkv=HKV, num_blocks=16384, lens=("fixed", 32768),
                 max_blocks=2048, partition=512, seed=4),
    "prefill": dict(prompts=[512, 512, 512, 512, 2048, 2048], Hq=HQ, Hkv=HKV,
                    num_blocks=4096, seed=5),
}


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def randn_bf16(gen: torch.Generator, shape, scale: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(torch.bfloat16)


def draw_lens(gen: torch.Generator, B: int, spec) -> torch.Tensor:
    kind = spec[0]
    if kind == "fixed":
        return torch.full((B,), spec[1], dtype=torch.int32)
    if kind == "uniform":  # integers lo..hi inclusive
        lo, hi = spec[1], spec[2]
        return torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)
    if kind == "loguniform":  # L = clamp(round(exp(U(ln lo, ln hi))), lo, hi)
        lo, hi = spec[1], spec[2]
        u = torch.rand(B, generator=gen, dtype=torch.float64)
        x = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
        return x.round().clamp(lo, hi).to(torch.int32)
    raise ValueError(kind)


def blocks_needed(lens: torch.Tensor, block_size: int) -> torch.Tensor:
    return (lens.to(torch.int64) + block_size - 1) // block_size


def tables_from_permutation(gen: torch.Generator, lens: torch.Tensor, block_size: int,
                            num_blocks: int, max_blocks: int, filler: int,
                            reserve_last: bool = True) -> torch.Tensor:
    """Disjoint slices of a seeded permutation of the physical block ids.

    If reserve_last, id num_blocks-1 is kept out of the permutation so callers
    can fill it with a sentinel and point unused table entries at it."""
    need = blocks_needed(lens, block_size)
    pool_ids = num_blocks - 1 if reserve_last else num_blocks
    if int(need.sum()) > pool_ids:
        raise ValueError("pool too small for the drawn lengths")
    if len(need) and int(need.max()) > max_blocks:
        raise ValueError("max_blocks too small for the drawn lengths")
    perm = torch.randperm(pool_ids, generator=gen).to(torch.int32)
    tables = torch.full((len(lens), max_blocks), filler, dtype=torch.int32)
    at = 0
    for b, n in enumerate(need.tolist()):
        tables[b, :n] = perm[at:at + n]
        at += n
    return tables


@dataclass
class PagedCase:
    """One paged-attention problem, all tensors on the CPU unless moved."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: torch.Tensor        # [B] int32, valid tokens after the append
    block_tables: torch.Tensor        # [B][max_blocks] int32
    q: torch.Tensor                   # decode [B][Hq][D] or prefill [T][Hq][D], bf16
    k_cache: Optional[torch.Tensor]   # [num_blocks][Hkv][bs][D] bf16
    v_cache: Optional[torch.Tensor]
    k_new: Optional[torch.Tensor] = None   # [T_new][Hkv][D] bf16
    v_new: Optional[torch.Tensor] = None
    cu_new_lens: Optional[torch.Tensor] = None  # [B+1] int32 or None (one per seq)
    cu_q_lens: Optional[torch.Tensor] = None    # prefill only
    sentinel_block: int = -1
    extra: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0


def rope_tables(max_position: int, D: int = HEAD_DIM, base: float = ROPE_BASE):
    """Angle tables for the rotary embedding: fp32 cos and sin [max_position][D/2]
    of pos * base^(-2i/D), computed in float64 and rounded once."""
    inv = base ** (-torch.arange(D // 2, dtype=torch.float64) * 2.0 / D)
    ang = torch.arange(max_position, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)


def poison_unused(case: PagedCase, value=float("nan")) -> None:
    """Fill every pool slot that no sequence may read (slots past the context
    in a last block, blocks no table references, the sentinel block) with
    `value`, in place."""
    used = torch.zeros(case.num_blocks, dtype=torch.bool)
    bs = case.block_size
    for b in range(case.B):
        n = int(blocks_needed(case.context_lens[b:b + 1], bs)[0])
        used[case.block_tables[b, :n].long()] = True
    for pool in (case.k_cache, case.v_cache):
        pool[~used] = value
        for b in range(case.B):
            L = int(case.context_lens[b])
            if L % bs:
                last = int(case.block_tables[b, L // bs])
                pool[last, :, L % bs:, :] = value


def decode_case(name: str, seed: Optional[int] = None, poison: bool = False,
                with_append: bool = False, **overrides) -> PagedCase:
    """A decode problem on the CPU (pools included) for the small workloads."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    seed = cfg["seed"] if seed is None else seed
    g = generator(seed)
    B, Hq, Hkv, N = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["num_blocks"]
    D, bs = cfg.get("D", HEAD_DIM), cfg.get("block_size", BLOCK_SIZE)
    lens = draw_lens(g, B, cfg["lens"])
    max_blocks = cfg.get("max_blocks", int(blocks_needed(lens, bs).max()))
    if name == "tiny":
        # all physical blocks in one seeded permutation; the first entries used
        perm = torch.randperm(N, generator=g).to(torch.int32)
        tables = perm.view(1, N)[:, :max(max_blocks, N)].clone()
        sentinel = -1
    else:
        tables = tables_from_permutation(g, lens, bs, N, max_blocks, filler=N - 1)
        sentinel = N - 1
    q = randn_bf16(g, (B, Hq, D), cfg.get("q_scale", 1.0))
    k_cache = randn_bf16(g, (N, Hkv, bs, D))
    v_cache = randn_bf16(g, (N, Hkv, bs, D))
    case = PagedCase(name, B, Hq, Hkv, D, bs, N, cfg.get("scale", SCALE), lens, tables, q,
                     k_cache, v_cache, sentinel_block=sentinel)
    if with_append:
        case.k_new = randn_bf16(g, (B, Hkv, D))
        case.v_new = randn_bf16(g, (B, Hkv, D))
    if poison:
        poison_unused(case)
    return case


def prefill_case(seed: Optional[int] = None, prompts: Optional[List[int]] = None,
                 num_blocks: Optional[int] = None, Hq: int = HQ, Hkv: int = HKV,
                 history: Optional[List[int]] = None, poison: bool = False) -> PagedCase:
    """Causal prefill: each prompt's K/V are new tokens to append (k_new/v_new,
    cu_new_lens) and the queries are packed [T][Hq][D] with cu_q_lens.

    history[b] optional tokens already in the cache before the prompt
    (chunked prefill); their K/V are drawn into the pool directly."""
    cfg = CONFIGS["prefill"]
    seed = cfg["seed"] if seed is None else seed
    prompts = list(cfg["prompts"] if prompts is None else prompts)
    N = cfg["num_blocks"] if num_blocks is None else num_blocks
    history = [0] * len(prompts) if history is None else list(history)
    g = generator(seed)
    B, D, bs = len(prompts), HEAD_DIM, BLOCK_SIZE
    q_lens = torch.tensor(prompts, dtype=torch.int32)
    lens = q_lens + torch.tensor(history, dtype=torch.int32)
    max_blocks = max(1, int(blocks_needed(lens, bs).max())) if len(lens) else 1
    tables = tables_from_permutation(g, lens, bs, N, max_blocks, filler=N - 1)
    T = int(q_lens.sum())
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(q_lens, 0)
    q = randn_bf16(g, (T, Hq, D))
    k_cache = randn_bf16(g, (N, Hkv, bs, D))
    v_cache = randn_bf16(g, (N, Hkv, bs, D))
    k_new = randn_bf16(g, (T, Hkv, D))
    v_new = randn_bf16(g, (T, Hkv, D))
    case = PagedCase("prefill", B, Hq, Hkv, D, bs, N, SCALE, lens, tables, q, k_cache, v_cache,
                     k_new=k_new, v_new=v_new, cu_new_lens=cu.clone(), cu_q_lens=cu,
                     sentinel_block=N - 1)
    if poison:
        poison_unused(case)
    return case


def device_decode_case(name: str, device, seed: Optional[int] = None, layers: int = 1,
                       **overrides) -> PagedCase:
    """Large decode problems built directly on the device.

    Lengths, tables and q come from the seeded CPU generator (same draw order
    as decode_case); each layer's K/V pools are filled only at the referenced
    blocks, from a seeded device generator (seed * 1000 + layer), and the
    unreferenced remainder is left as allocated.  k_cache/v_cache hold lists
    of per-layer pools in case.extra['k_layers'] / ['v_layers']."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    seed = cfg["seed"] if seed is None else seed
    g = generator(seed)
    B, Hq, Hkv, N = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["num_blocks"]
    D, bs = HEAD_DIM, BLOCK_SIZE
    lens = draw_lens(g, B, cfg["lens"])
    max_blocks = cfg.get("max_blocks", int(blocks_needed(lens, bs).max()))
    tables = tables_from_permutation(g, lens, bs, N, max_blocks, filler=N - 1)
    q = randn_bf16(g, (B, Hq, D))
    need = blocks_needed(lens, bs)
    used = torch.cat([tables[b, :int(n)] for b, n in enumerate(need.tolist())]).long()
    used_dev = used.to(device)
    k_layers, v_layers = [], []
    for layer in range(layers):
        dg = torch.Generator(device=device)
        dg.manual_seed(seed * 1000 + layer)
        pools = []
        for _ in range(2):
            pool = torch.empty((N, Hkv, bs, D), dtype=torch.bfloat16, device=device)
            vals = torch.randn((len(used), Hkv, bs, D), generator=dg, device=device,
                               dtype=torch.float32).to(torch.bfloat16)
            pool.index_copy_(0, used_dev, vals)
            del vals
            pools.append(pool)
        k_layers.append(pools[0])
        v_layers.append(pools[1])
    case = PagedCase(name, B, Hq, Hkv, D, bs, N, SCALE, lens, tables, q, k_layers[0],
                     v_layers[0], sentinel_block=N - 1)
    case.extra.update(k_layers=k_layers, v_layers=v_layers, used_blocks=used,
                      partition=cfg.get("partition", 512))
    # one new token per sequence for the append that precedes each decode
    case.k_new = randn_bf16(g, (B, Hkv, D))
    case.v_new = randn_bf16(g, (B, Hkv, D))
    return case


def compact_for_oracle(case: PagedCase, k_pool: torch.Tensor, v_pool: torch.Tensor):
    """Copy only the referenced blocks of (device) pools back to the host and
    renumber the tables to that compact pool.  Paging makes the result
    independent of where blocks sit, so the oracle sees the same problem."""
    bs = case.block_size
    need = blocks_needed(case.context_lens, bs)
    used = torch.cat([case.block_tables[b, :int(n)] for b, n in enumerate(need.tolist())])
    uniq, inverse = torch.unique(used.long(), return_inverse=True)
    k = k_pool.index_select(0, uniq.to(k_pool.device)).cpu()
    v = v_pool.index_select(0, uniq.to(v_pool.device)).cpu()
    tables = torch.zeros_like(case.block_tables)
    at = 0
    for b, n in enumerate(need.tolist()):
        tables[b, :n] = inverse[at:at + n].to(torch.int32)
        at += n
    return k, v, tables


def as_u16(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (no copy of values' meaning)."""
    return t.contiguous().cpu().view(torch.int16).numpy().view("uint16")
