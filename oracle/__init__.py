"""ctypes front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product package.  Arrays are numpy:
bf16 data as uint16 bit patterns, indices as int32, results as float64.

`Oracle(path)` binds one build of oracle.c (tests load deliberately mutated
builds through it); the module-level functions use the default build.
"""
import ctypes
import os

import numpy as np

from . import build as _build


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: inputs outside what the tables cover (rc={rc})")


def _balanced_groups(items, costs, n):
    """Deal items out to n groups, heaviest first onto the lightest group."""
    import heapq
    groups = [[] for _ in range(n)]
    heap = [(0, i) for i in range(n)]
    for c, it in sorted(zip(costs, items), reverse=True):
        load, i = heapq.heappop(heap)
        groups[i].append(it)
        heapq.heappush(heap, (load + max(int(c), 1), i))
    return [g for g in groups if g]


def _in_threads(fn, groups):
    """fn(group) for every group, one thread each; re-raises the first error."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=len(groups)) as ex:
        for f in [ex.submit(fn, g) for g in groups]:
            f.result()


class Oracle:
    def __init__(self, path):
        lib = ctypes.CDLL(path)
        P, I, Dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
        lib.oracle_kv_append.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I]
        lib.oracle_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, Dbl]
        lib.oracle_decode_online.argtypes = lib.oracle_decode.argtypes
        lib.oracle_prefill_causal.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I,
                                              I, I, Dbl, P, I]
        lib.oracle_decode_partials.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I,
                                               I, I, I, Dbl, I, I]
        lib.oracle_lse_merge.argtypes = [P, P, P, P, I, I, I]
        lib.oracle_token_positions.argtypes = [P, P, P, P, I, I]
        lib.oracle_rope.argtypes = [P, P, P, P, P, I, I, I, I]
        lib.oracle_round_bf16.argtypes = [P, P, ctypes.c_long]
        lib.oracle_copy_blocks.argtypes = [P, P, P, P, I, I, I, I, I]
        for f in (lib.oracle_kv_append, lib.oracle_decode, lib.oracle_decode_online,
                  lib.oracle_prefill_causal, lib.oracle_decode_partials,
                  lib.oracle_lse_merge, lib.oracle_token_positions, lib.oracle_rope,
                  lib.oracle_round_bf16, lib.oracle_copy_blocks):
            f.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def kv_append(self, k_cache, v_cache, k_new, v_new, block_tables, context_lens,
                  cu_new_lens=None):
        """In place on the numpy uint16 pools k_cache/v_cache [N][Hkv][bs][D]."""
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        assert k_cache.dtype == np.uint16 and v_cache.dtype == np.uint16
        N, Hkv, bs, D = k_cache.shape
        bt, cl = _i32(block_tables), _i32(context_lens)
        cu = None if cu_new_lens is None else _i32(cu_new_lens)
        kn, vn = _u16(k_new), _u16(v_new)
        rc = self.lib.oracle_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(kn), _ptr(vn),
                                       _ptr(bt), _ptr(cl), _ptr(cu), bt.shape[0], Hkv, D,
                                       bs, bt.shape[1], N)
        _check(rc, "kv_append")

    def decode(self, q, k_cache, v_cache, block_tables, context_lens, scale,
               online=False, threads=1):
        """q [B][Hq][D] uint16 -> out [B][Hq][D] float64.

        threads > 1 splits the sequences into that many groups of about equal
        context (each sequence whole, in one group) and runs the same
        single-threaded C routine on each group in its own thread (ctypes
        releases the GIL): the arithmetic of every output is unchanged."""
        q, k_cache, v_cache = _u16(q), _u16(k_cache), _u16(v_cache)
        B, Hq, D = q.shape
        N, Hkv, bs, _ = k_cache.shape
        bt, cl = _i32(block_tables), _i32(context_lens)
        out = np.zeros((B, Hq, D), dtype=np.float64)
        fn = self.lib.oracle_decode_online if online else self.lib.oracle_decode

        def run(seqs):
            for b in seqs:
                rc = fn(_ptr(out[b:b + 1]), _ptr(q[b:b + 1]), _ptr(k_cache), _ptr(v_cache),
                        _ptr(bt[b:b + 1]), _ptr(cl[b:b + 1]), 1, Hq, Hkv, D, bs, bt.shape[1],
                        N, float(scale))
                _check(rc, "decode")

        if threads <= 1 or B <= 1:
            rc = fn(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                    B, Hq, Hkv, D, bs, bt.shape[1], N, float(scale))
            _check(rc, "decode")
            return out
        _in_threads(run, _balanced_groups(list(range(B)), [int(x) + 1 for x in cl], threads))
        return out

    def prefill_causal(self, q, k_cache, v_cache, block_tables, context_lens, cu_q_lens,
                       scale, rows=None, threads=1):
        """q [T][Hq][D] uint16 -> out [T][Hq][D] float64 (unlisted rows stay NaN).

        threads > 1 deals the rows out to that many threads in groups of
        about equal cost (visible keys), each running the same single-threaded
        C routine on its rows; every row's arithmetic is unchanged."""
        q, k_cache, v_cache = _u16(q), _u16(k_cache), _u16(v_cache)
        T, Hq, D = q.shape
        N, Hkv, bs, _ = k_cache.shape
        bt, cl, cu = _i32(block_tables), _i32(context_lens), _i32(cu_q_lens)
        out = np.full((T, Hq, D), np.nan, dtype=np.float64)
        r = None if rows is None else _i32(rows)

        def run(rr):
            rr = _i32(rr)
            rc = self.lib.oracle_prefill_causal(
                _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                _ptr(cu), bt.shape[0], Hq, Hkv, D, bs, bt.shape[1], N, float(scale),
                _ptr(rr), len(rr))
            _check(rc, "prefill_causal")

        if threads <= 1:
            rc = self.lib.oracle_prefill_causal(
                _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                _ptr(cu), bt.shape[0], Hq, Hkv, D, bs, bt.shape[1], N, float(scale),
                _ptr(r), 0 if r is None else len(r))
            _check(rc, "prefill_causal")
            return out
        all_rows = list(range(T)) if r is None else [int(x) for x in r]
        seq = np.searchsorted(cu, np.asarray(all_rows), side="right") - 1
        qlen = cu[seq + 1] - cu[seq]
        cost = (cl[seq] - qlen + (np.asarray(all_rows) - cu[seq]) + 1).tolist()
        _in_threads(run, _balanced_groups(all_rows, cost, threads))
        return out

    def decode_partials(self, q, k_cache, v_cache, block_tables, context_lens, scale,
                        partition_size):
        """Per-partition (o, m, l) of the split-context formulation."""
        q, k_cache, v_cache = _u16(q), _u16(k_cache), _u16(v_cache)
        B, Hq, D = q.shape
        N, Hkv, bs, _ = k_cache.shape
        bt, cl = _i32(block_tables), _i32(context_lens)
        P = max(1, -(-int(cl.max(initial=0)) // partition_size))
        o = np.zeros((B, Hq, P, D))
        m = np.zeros((B, Hq, P))
        l = np.zeros((B, Hq, P))
        rc = self.lib.oracle_decode_partials(
            _ptr(o), _ptr(m), _ptr(l), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
            _ptr(cl), B, Hq, Hkv, D, bs, bt.shape[1], N, float(scale), partition_size, P)
        _check(rc, "decode_partials")
        return o, m, l

    def lse_merge(self, o, m, l):
        """Merge partials o [..][P][D], m/l [..][P] -> [..][D]."""
        lead = o.shape[:-2]
        P, D = o.shape[-2:]
        o2 = np.ascontiguousarray(o, dtype=np.float64).reshape(-1, P, D)
        m2 = np.ascontiguousarray(m, dtype=np.float64).reshape(-1, P)
        l2 = np.ascontiguousarray(l, dtype=np.float64).reshape(-1, P)
        out = np.zeros((o2.shape[0], D))
        rc = self.lib.oracle_lse_merge(_ptr(out), _ptr(o2), _ptr(m2), _ptr(l2),
                                       o2.shape[0], P, D)
        _check(rc, "lse_merge")
        return out.reshape(*lead, D)

    def token_positions(self, context_lens, cu_new_lens, T_new):
        """(pos, seq) int32 [T_new]: absolute position and sequence of every new token."""
        cl = _i32(context_lens)
        cu = None if cu_new_lens is None else _i32(cu_new_lens)
        pos = np.full(T_new, -1, dtype=np.int32)
        seq = np.full(T_new, -1, dtype=np.int32)
        rc = self.lib.oracle_token_positions(_ptr(pos), _ptr(seq), _ptr(cl), _ptr(cu),
                                             cl.shape[0], T_new)
        _check(rc, "token_positions")
        return pos, seq

    def rope(self, x, pos, rope_cos, rope_sin):
        """x [rows][heads][D] uint16 at positions pos [rows] -> float64 [rows][heads][D]."""
        x = _u16(x)
        rows, heads, D = x.shape
        p = _i32(pos)
        c = np.ascontiguousarray(rope_cos, dtype=np.float32)
        s = np.ascontiguousarray(rope_sin, dtype=np.float32)
        assert c.shape == s.shape and c.shape[1] * 2 == D and p.shape == (rows,)
        out = np.zeros((rows, heads, D), dtype=np.float64)
        rc = self.lib.oracle_rope(_ptr(out), _ptr(x), _ptr(p), _ptr(c), _ptr(s), rows, heads,
                                  D, c.shape[0])
        _check(rc, "rope")
        return out

    def round_bf16(self, x):
        """float64 array -> uint16 bf16 bit patterns (nearest, ties to even)."""
        xd = np.ascontiguousarray(x, dtype=np.float64)
        out = np.zeros(xd.shape, dtype=np.uint16)
        self.lib.oracle_round_bf16(_ptr(out), _ptr(xd), xd.size)
        return out

    def copy_blocks(self, k_cache, v_cache, src, dst):
        """Block dst[i] of both uint16 pools [N][Hkv][bs][D] gets block src[i], in place."""
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        N, Hkv, bs, D = k_cache.shape
        s, d = _i32(src), _i32(dst)
        rc = self.lib.oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(s), _ptr(d), len(s),
                                         Hkv, bs, D, N)
        _check(rc, "copy_blocks")

    def kv_append_rope(self, k_cache, v_cache, k_new, v_new, block_tables, context_lens,
                       rope_cos, rope_sin, q=None, cu_new_lens=None):
        """The fused operation written as its steps: positions of the new tokens, RoPE of
        k (and q) at those positions, rounding to bf16, then kv_append of the rotated K and
        the unchanged V.  Pools change in place; returns the rotated q (uint16) or None.
        Tokens whose position has no table row are left out, as the library does."""
        T_new = k_new.shape[0]
        pos, _ = self.token_positions(context_lens, cu_new_lens, T_new)
        ok = (pos >= 0) & (pos < rope_cos.shape[0])
        k_rot = np.array(_u16(k_new), copy=True)
        q_rot = None if q is None else np.array(_u16(q), copy=True)
        if ok.any():
            k_rot[ok] = self.round_bf16(self.rope(k_new[ok], pos[ok], rope_cos, rope_sin))
            if q is not None:
                q_rot[ok] = self.round_bf16(self.rope(q[ok], pos[ok], rope_cos, rope_sin))
        if ok.all():
            self.kv_append(k_cache, v_cache, k_rot, v_new, block_tables, context_lens,
                           cu_new_lens)
        else:
            # append the tokens with a table row one at a time (the others are skipped)
            cl = _i32(context_lens)
            _, seq = self.token_positions(context_lens, cu_new_lens, T_new)
            for t in np.nonzero(ok)[0]:
                b = int(seq[t])
                one_len = np.zeros_like(cl)
                one_len[b] = pos[t] + 1
                cu = np.zeros(cl.shape[0] + 1, dtype=np.int32)
                cu[b + 1:] = 1
                self.kv_append(k_cache, v_cache, k_rot[t:t + 1], v_new[t:t + 1], block_tables,
                               one_len, cu)
        return q_rot


_default = None


def default() -> Oracle:
    """The oracle build the module-level functions use: oracle/liboracle.so,
    or the build PKV_ORACLE_LIB names (the sanitizer build in the CPU tests)."""
    global _default
    if _default is None:
        path = os.environ.get("PKV_ORACLE_LIB")
        if not path:
            if not os.path.exists(_build.LIB):
                _build.build()
            path = _build.LIB
        _default = Oracle(path)
    return _default


def kv_append(*a, **k):
    return default().kv_append(*a, **k)


def decode(*a, **k):
    return default().decode(*a, **k)


def prefill_causal(*a, **k):
    return default().prefill_causal(*a, **k)


def decode_partials(*a, **k):
    return default().decode_partials(*a, **k)


def lse_merge(*a, **k):
    return default().lse_merge(*a, **k)


def token_positions(*a, **k):
    return default().token_positions(*a, **k)


def rope(*a, **k):
    return default().rope(*a, **k)


def round_bf16(*a, **k):
    return default().round_bf16(*a, **k)


def kv_append_rope(*a, **k):
    return default().kv_append_rope(*a, **k)


def copy_blocks(*a, **k):
    return default().copy_blocks(*a, **k)
