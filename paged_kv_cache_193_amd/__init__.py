"""MI355X-native paged KV-cache attention: Python binding of libpagedkv.so.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libpagedkv.so (built for gfx950 by build.py); torch supplies the
device memory and the current stream.  If the library is not built, every
call raises -- there is no CPU fallback.

Entry points (same names as the C ABI in include/pagedkv.h):
    kv_append(k_cache, v_cache, k_new, v_new, block_tables, context_lens,
              cu_new_lens=None)
    kv_append_rope(k_cache, v_cache, k_new, v_new, block_tables, context_lens,
              rope_cos, rope_sin, q=None, cu_new_lens=None)
    paged_attention_decode(out, q, k_cache, v_cache, block_tables,
              context_lens, scale, max_context_len, partition_size=AUTO,
              workspace=None)
    paged_attention_decode_append(out, q, k_cache, v_cache, k_new, v_new,
              block_tables, context_lens, scale, max_context_len,
              partition_size=AUTO, workspace=None)
    paged_attention_prefill_causal(out, q, k_cache, v_cache, block_tables,
              context_lens, cu_q_lens, scale, max_q_len)
    paged_attention_decode_plan(k_cache, block_tables, context_lens, Hq,
              max_context_len, workspace)
    paged_attention_decode_workspace_size(B, Hq, D, max_context_len, partition_size)
    Scheduler(num_blocks, block_size, max_blocks_per_seq, max_batch, max_step_tokens,
              static_batching=False)  -- pkv_sched_* (host control plane)
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libpagedkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_HIP = -4
PKV_OUT_BF16 = 0
PKV_OUT_F32 = 1
PARTITION_NONE = 0
PARTITION_AUTO = -1
PARTITION_PLANNED = -2
CHECK_READ = 0
CHECK_APPEND = 1
CHECK_PREFILL = 2

# every symbol include/pagedkv.h declares
ABI_SYMBOLS = ("pagedkv_last_error", "pagedkv_check_tables", "kv_append", "kv_append_rope", "kv_copy_blocks",
               "paged_attention_decode_workspace_size",
               "paged_attention_decode", "paged_attention_decode_append",
               "paged_attention_decode_noalloc",
               "paged_attention_decode_plan",
               "paged_attention_prefill_causal", "pagedkv_stream_blocks", "pagedkv_mfma_probe",
               "pkv_sched_create", "pkv_sched_destroy", "pkv_sched_add_request",
               "pkv_sched_step", "pkv_sched_events", "pkv_sched_stats",
               "pkv_sched_add_request_prefix", "pkv_sched_fork", "pkv_sched_copies")

PKV_SCHED_STATS = 16
SCHED_STAT_NAMES = ("steps", "tokens", "prefill_tokens", "decode_tokens", "preemptions",
                    "finished", "free_blocks", "running", "waiting", "cached_token_steps",
                    "paged_slot_steps", "static_request_slot_steps", "static_max_slot_steps",
                    "batch_row_steps", "block_copies", "shared_prefix_tokens")

_lib = None


class PagedKVError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"[{code}] {message}")
        self.code = code


def _bind_host(lib):
    """Argument types of the host-only entry points (status text, table
    checks, scheduler)."""
    P, I, L = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pagedkv_last_error.argtypes = []
    lib.pagedkv_last_error.restype = ctypes.c_char_p
    lib.pagedkv_check_tables.argtypes = [P, P, P, I, I, I, I, I, I]
    lib.pagedkv_check_tables.restype = ctypes.c_int
    lib.pkv_sched_create.argtypes = [I, I, I, I, I, I]
    lib.pkv_sched_create.restype = P
    lib.pkv_sched_destroy.argtypes = [P]
    lib.pkv_sched_destroy.restype = None
    lib.pkv_sched_add_request.argtypes = [P, L, I, I]
    lib.pkv_sched_add_request.restype = ctypes.c_int
    lib.pkv_sched_step.argtypes = [P, P, P, P, P, P]
    lib.pkv_sched_step.restype = ctypes.c_int
    lib.pkv_sched_events.argtypes = [P, I, P, I]
    lib.pkv_sched_events.restype = ctypes.c_int32
    lib.pkv_sched_stats.argtypes = [P, P]
    lib.pkv_sched_stats.restype = ctypes.c_int
    lib.pkv_sched_add_request_prefix.argtypes = [P, L, I, I, L, I]
    lib.pkv_sched_add_request_prefix.restype = ctypes.c_int
    lib.pkv_sched_fork.argtypes = [P, L, L, I]
    lib.pkv_sched_fork.restype = ctypes.c_int
    lib.pkv_sched_copies.argtypes = [P, P, P, I]
    lib.pkv_sched_copies.restype = ctypes.c_int32


_host_lib = None


def host_library():
    """The library the host-only calls (Scheduler, check_tables) go to:
    libpagedkv.so, or, when PKV_HOST_LIB names one, a host-only build of the
    same sources (the sanitizer build the CPU tests use)."""
    global _host_lib
    path = os.environ.get("PKV_HOST_LIB")
    if not path:
        return load_library()
    if _host_lib is None or _host_lib._name != path:
        lib = ctypes.CDLL(path)
        _bind_host(lib)
        _host_lib = lib
    return _host_lib


def _check_host(lib, rc):
    if rc != PKV_OK:
        raise PagedKVError(rc, lib.pagedkv_last_error().decode())


def load_library():
    """Load libpagedkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python __graft_entry__.py` "
                           "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.kv_append.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.kv_append.restype = ctypes.c_int
    lib.kv_append_rope.argtypes = [P, P, P, P, P, P, P, I, P, P, P, I, I, I, I, I, I, I, I, P]
    lib.kv_append_rope.restype = ctypes.c_int
    lib.kv_copy_blocks.argtypes = [P, P, P, P, I, I, I, I, I, P]
    lib.kv_copy_blocks.restype = ctypes.c_int
    lib.paged_attention_decode_workspace_size.argtypes = [I, I, I, I, I]
    lib.paged_attention_decode_workspace_size.restype = Z
    lib.paged_attention_decode.argtypes = [P, I, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I,
                                           P, Z, P]
    lib.paged_attention_decode.restype = ctypes.c_int
    lib.paged_attention_decode_noalloc.argtypes = [P, I, P, P, P, P, P, I, I, I, I, I, I, I, I, F,
                                                   I, P]
    lib.paged_attention_decode_noalloc.restype = ctypes.c_int
    lib.paged_attention_decode_append.argtypes = [P, I, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                                  I, F, I, P, Z, P]
    lib.paged_attention_decode_append.restype = ctypes.c_int
    lib.paged_attention_decode_plan.argtypes = [P, P, I, I, I, I, I, I, I, I, P, Z, P]
    lib.paged_attention_decode_plan.restype = ctypes.c_int
    lib.paged_attention_prefill_causal.argtypes = [P, I, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                                   I, I, F, P]
    lib.paged_attention_prefill_causal.restype = ctypes.c_int
    lib.pagedkv_stream_blocks.argtypes = [P, P, P, I, I, I, I, I, P, Z, P]
    lib.pagedkv_stream_blocks.restype = ctypes.c_int
    lib.pagedkv_mfma_probe.argtypes = [I, P, Z, P]
    lib.pagedkv_mfma_probe.restype = ctypes.c_int
    _bind_host(lib)
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().pagedkv_last_error().decode()


def _check(rc):
    if rc != PKV_OK:
        raise PagedKVError(rc, last_error())


def _torch():
    import torch
    return torch


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _out_dtype(out):
    torch = _torch()
    if out.dtype == torch.bfloat16:
        return PKV_OUT_BF16
    if out.dtype == torch.float32:
        return PKV_OUT_F32
    raise TypeError("out must be bfloat16 or float32")


def check_tables(block_tables, context_lens, kind=CHECK_READ, cu_lens=None, block_size=16,
                 num_blocks=None, T=None):
    """pagedkv_check_tables on host (numpy) arrays: raises PagedKVError naming
    the first out-of-range length, block id or prefix sum."""
    import numpy as np
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    cu = None if cu_lens is None else np.ascontiguousarray(cu_lens, dtype=np.int32)
    B, maxb = bt.shape
    if cl.shape != (B,) or (cu is not None and cu.shape != (B + 1,)):
        raise ValueError("context_lens must be [B] and cu_lens [B+1]")
    if T is None:
        T = int(cu[-1]) if cu is not None else B
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    lib = host_library()
    _check_host(lib, lib.pagedkv_check_tables(p(bt), p(cl), p(cu), B, int(T), maxb,
                                              int(num_blocks), int(block_size), int(kind)))


def _shape(t, n, name):
    """Shape of t as a tuple of n sizes (ValueError unless t has n dimensions)."""
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions (got shape {tuple(t.shape)})")
    return tuple(int(x) for x in t.shape)


def _pools(k_cache, v_cache):
    """(N, Hkv, bs, D) of a K/V pool pair of the same shape.  The C ABI sees
    only pointers, so every size the kernels index with is checked here."""
    shp = _shape(k_cache, 4, "k_cache")
    if _shape(v_cache, 4, "v_cache") != shp:
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} differs from k_cache {shp}")
    return shp


def _tables(block_tables, context_lens, B):
    """max_blocks_per_seq of a [B][max_blocks] table, with B context lengths."""
    nb, maxb = _shape(block_tables, 2, "block_tables")
    if nb != B:
        raise ValueError(f"block_tables has {nb} rows for a batch of {B}")
    if context_lens.numel() != B:
        raise ValueError(f"context_lens has {context_lens.numel()} entries for a batch of {B}")
    return maxb


def _rows(t, shape, name):
    if _shape(t, len(shape), name) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def kv_append(k_cache, v_cache, k_new, v_new, block_tables, context_lens, cu_new_lens=None):
    """Write new K/V rows [T_new][Hkv][D] into the pools [N][Hkv][bs][D] in place."""
    torch = _torch()
    N, Hkv, bs, D = _pools(k_cache, v_cache)
    B = _shape(block_tables, 2, "block_tables")[0]
    maxb = _tables(block_tables, context_lens, B)
    T_new = _shape(k_new, 3, "k_new")[0]
    _rows(k_new, (T_new, Hkv, D), "k_new")
    _rows(v_new, (T_new, Hkv, D), "v_new")
    cu_ptr = None
    if cu_new_lens is not None:
        if cu_new_lens.numel() != B + 1:
            raise ValueError("cu_new_lens must have B+1 entries")
        cu_ptr = _dev(cu_new_lens, torch.int32, "cu_new_lens")
    elif T_new != B:
        raise ValueError(f"without cu_new_lens there is one new row per sequence "
                         f"(T_new {T_new} != B {B})")
    _check(load_library().kv_append(
        _dev(k_cache, torch.bfloat16, "k_cache"), _dev(v_cache, torch.bfloat16, "v_cache"),
        _dev(k_new, torch.bfloat16, "k_new"), _dev(v_new, torch.bfloat16, "v_new"),
        _dev(block_tables, torch.int32, "block_tables"),
        _dev(context_lens, torch.int32, "context_lens"), cu_ptr, B, T_new, Hkv, D, bs, maxb, N,
        _stream()))


def kv_copy_blocks(k_cache, v_cache, src_blocks, dst_blocks):
    """Copy pool block src_blocks[i] onto dst_blocks[i] (int32 device tensors), K and V."""
    torch = _torch()
    N, Hkv, bs, D = _pools(k_cache, v_cache)
    n = src_blocks.numel()
    if dst_blocks.numel() != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    if n == 0:
        return
    _check(load_library().kv_copy_blocks(
        _dev(k_cache, torch.bfloat16, "k_cache"), _dev(v_cache, torch.bfloat16, "v_cache"),
        _dev(src_blocks, torch.int32, "src_blocks"), _dev(dst_blocks, torch.int32, "dst_blocks"),
        n, Hkv, D, bs, N, _stream()))


def kv_append_rope(k_cache, v_cache, k_new, v_new, block_tables, context_lens, rope_cos,
                   rope_sin, q=None, cu_new_lens=None):
    """kv_append of the RoPE-rotated new keys (k_new/v_new [T_new][Hkv][D]) and, when q
    ([T_new][Hq][D]) is given, the same rotation of q in place.  rope_cos/rope_sin are
    float32 [max_position][D/2] device tables."""
    torch = _torch()
    N, Hkv, bs, D = _pools(k_cache, v_cache)
    B = _shape(block_tables, 2, "block_tables")[0]
    maxb = _tables(block_tables, context_lens, B)
    T_new = _shape(k_new, 3, "k_new")[0]
    _rows(k_new, (T_new, Hkv, D), "k_new")
    _rows(v_new, (T_new, Hkv, D), "v_new")
    if cu_new_lens is None and T_new != B:
        raise ValueError(f"without cu_new_lens there is one new row per sequence "
                         f"(T_new {T_new} != B {B})")
    if rope_cos.dim() != 2 or tuple(rope_sin.shape) != tuple(rope_cos.shape) or \
            rope_cos.shape[1] * 2 != D:
        raise ValueError("rope_cos and rope_sin must both be [max_position][D/2]")
    q_ptr, Hq = None, 0
    if q is not None:
        if q.dim() != 3 or q.shape[0] != T_new or q.shape[2] != D:
            raise ValueError("q must be [T_new][Hq][D]")
        Hq = q.shape[1]
        q_ptr = _dev(q, torch.bfloat16, "q")
    cu_ptr = None
    if cu_new_lens is not None:
        if cu_new_lens.numel() != B + 1:
            raise ValueError("cu_new_lens must have B+1 entries")
        cu_ptr = _dev(cu_new_lens, torch.int32, "cu_new_lens")
    _check(load_library().kv_append_rope(
        _dev(k_cache, torch.bfloat16, "k_cache"), _dev(v_cache, torch.bfloat16, "v_cache"), q_ptr,
        _dev(k_new, torch.bfloat16, "k_new"), _dev(v_new, torch.bfloat16, "v_new"),
        _dev(rope_cos, torch.float32, "rope_cos"), _dev(rope_sin, torch.float32, "rope_sin"),
        rope_cos.shape[0], _dev(block_tables, torch.int32, "block_tables"),
        _dev(context_lens, torch.int32, "context_lens"), cu_ptr, B, T_new, Hq, Hkv, D, bs, maxb,
        N, _stream()))


def paged_attention_decode_workspace_size(B, Hq, D, max_context_len,
                                          partition_size=PARTITION_AUTO) -> int:
    return int(load_library().paged_attention_decode_workspace_size(
        int(B), int(Hq), int(D), int(max_context_len), int(partition_size)))


def _decode_shapes(out, q, k_cache, v_cache, block_tables, context_lens):
    """(B, Hq, D, N, Hkv, bs, max_blocks) of a decode call, every size checked."""
    B, Hq, D = _shape(q, 3, "q")
    N, Hkv, bs, Dk = _pools(k_cache, v_cache)
    if Dk != D:
        raise ValueError(f"pool head_dim {Dk} differs from q's {D}")
    _rows(out, (B, Hq, D), "out")
    maxb = _tables(block_tables, context_lens, B)
    return B, Hq, D, N, Hkv, bs, maxb


def _workspace(workspace):
    if workspace is None:
        return None, 0
    return _dev(workspace, _torch().uint8, "workspace"), workspace.numel()


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           max_context_len, partition_size=PARTITION_AUTO, workspace=None):
    """out[B][Hq][D] (bf16 or fp32) = paged decode attention of q[B][Hq][D].

    workspace: a device uint8 tensor of at least
    paged_attention_decode_workspace_size(...) bytes when a split is used."""
    torch = _torch()
    B, Hq, D, N, Hkv, bs, maxb = _decode_shapes(out, q, k_cache, v_cache, block_tables,
                                                context_lens)
    ws_ptr, ws_bytes = _workspace(workspace)
    _check(load_library().paged_attention_decode(
        _dev(out, out.dtype, "out"), _out_dtype(out), _dev(q, torch.bfloat16, "q"),
        _dev(k_cache, torch.bfloat16, "k_cache"), _dev(v_cache, torch.bfloat16, "v_cache"),
        _dev(block_tables, torch.int32, "block_tables"),
        _dev(context_lens, torch.int32, "context_lens"), B, Hq, Hkv, D, bs, maxb, N,
        int(max_context_len), float(scale), int(partition_size), ws_ptr, ws_bytes, _stream()))


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   max_context_len, partition_size=PARTITION_AUTO):
    """paged_attention_decode without a workspace: the split's scratch is the
    library's static device array (16 MiB per GPU), so the call allocates
    nothing.  Calls on one GPU share that array and must not overlap."""
    torch = _torch()
    B, Hq, D, N, Hkv, bs, maxb = _decode_shapes(out, q, k_cache, v_cache, block_tables,
                                                context_lens)
    _check(load_library().paged_attention_decode_noalloc(
        _dev(out, out.dtype, "out"), _out_dtype(out), _dev(q, torch.bfloat16, "q"),
        _dev(k_cache, torch.bfloat16, "k_cache"), _dev(v_cache, torch.bfloat16, "v_cache"),
        _dev(block_tables, torch.int32, "block_tables"),
        _dev(context_lens, torch.int32, "context_lens"), B, Hq, Hkv, D, bs, maxb, N,
        int(max_context_len), float(scale), int(partition_size), _stream()))


def paged_attention_decode_append(out, q, k_cache, v_cache, k_new, v_new, block_tables,
                                  context_lens, scale, max_context_len,
                                  partition_size=PARTITION_AUTO, workspace=None):
    """kv_append of one new token per sequence (k_new/v_new [B][Hkv][D]) followed by
    paged_attention_decode, in one launch for PARTITION_AUTO."""
    torch = _torch()
    B, Hq, D, N, Hkv, bs, maxb = _decode_shapes(out, q, k_cache, v_cache, block_tables,
                                                context_lens)
    _rows(k_new, (B, Hkv, D), "k_new")
    _rows(v_new, (B, Hkv, D), "v_new")
    ws_ptr, ws_bytes = _workspace(workspace)
    _check(load_library().paged_attention_decode_append(
        _dev(out, out.dtype, "out"), _out_dtype(out), _dev(q, torch.bfloat16, "q"),
        _dev(k_cache, torch.bfloat16, "k_cache"), _dev(v_cache, torch.bfloat16, "v_cache"),
        _dev(k_new, torch.bfloat16, "k_new"), _dev(v_new, torch.bfloat16, "v_new"),
        _dev(block_tables, torch.int32, "block_tables"),
        _dev(context_lens, torch.int32, "context_lens"), B, Hq, Hkv, D, bs, maxb, N,
        int(max_context_len), float(scale), int(partition_size), ws_ptr, ws_bytes, _stream()))


def paged_attention_decode_plan(k_cache, block_tables, context_lens, Hq, max_context_len,
                                workspace):
    """Store the automatic split's plan for these tables and lengths in
    `workspace` (sized for PARTITION_PLANNED), for decode calls with
    partition_size=PARTITION_PLANNED.  k_cache only supplies the pool shape."""
    torch = _torch()
    N, Hkv, bs, D = _shape(k_cache, 4, "k_cache")
    B = _shape(block_tables, 2, "block_tables")[0]
    maxb = _tables(block_tables, context_lens, B)
    _check(load_library().paged_attention_decode_plan(
        _dev(block_tables, torch.int32, "block_tables"),
        _dev(context_lens, torch.int32, "context_lens"), B, Hq, Hkv, D, bs, maxb, N,
        int(max_context_len), _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream()))


def paged_attention_prefill_causal(out, q, k_cache, v_cache, block_tables, context_lens,
                                   cu_q_lens, scale, max_q_len):
    """out[T][Hq][D] = causal paged prefill attention of packed q[T][Hq][D]."""
    torch = _torch()
    T, Hq, D = _shape(q, 3, "q")
    N, Hkv, bs, Dk = _pools(k_cache, v_cache)
    if Dk != D:
        raise ValueError(f"pool head_dim {Dk} differs from q's {D}")
    _rows(out, (T, Hq, D), "out")
    B = _shape(block_tables, 2, "block_tables")[0]
    maxb = _tables(block_tables, context_lens, B)
    if cu_q_lens.numel() != B + 1:
        raise ValueError("cu_q_lens must have B+1 entries")
    _check(load_library().paged_attention_prefill_causal(
        _dev(out, out.dtype, "out"), _out_dtype(out), _dev(q, torch.bfloat16, "q"),
        _dev(k_cache, torch.bfloat16, "k_cache"), _dev(v_cache, torch.bfloat16, "v_cache"),
        _dev(block_tables, torch.int32, "block_tables"),
        _dev(context_lens, torch.int32, "context_lens"),
        _dev(cu_q_lens, torch.int32, "cu_q_lens"), B, T, Hq, Hkv, D, bs, maxb, N,
        int(max_q_len), float(scale), _stream()))


STREAM_SINK_BYTES = 2048 * 64 * 4


def stream_blocks(k_cache, v_cache, block_ids, sink):
    """Measurement probe: read every KV head of the listed pool blocks (int32
    device tensor) from both pools and nothing else; sink is a uint8 device
    tensor of at least STREAM_SINK_BYTES."""
    torch = _torch()
    N, Hkv, bs, D = _pools(k_cache, v_cache)
    _check(load_library().pagedkv_stream_blocks(
        _dev(k_cache, torch.bfloat16, "k_cache"), _dev(v_cache, torch.bfloat16, "v_cache"),
        _dev(block_ids, torch.int32, "block_ids"), block_ids.numel(), Hkv, D, bs, N,
        _dev(sink, torch.uint8, "sink"), sink.numel(), _stream()))


MFMA_PROBE_MAX_ITERS = 1 << 18


def mfma_probe(iters, sink):
    """Measurement probe: 2048 wavefronts of bf16 MFMA chains, `iters` rounds
    each; sink is a float32 device tensor of at least STREAM_SINK_BYTES / 4
    elements and receives exactly 4 * iters in each."""
    torch = _torch()
    _check(load_library().pagedkv_mfma_probe(
        int(iters), _dev(sink, torch.float32, "sink"), sink.numel() * 4, _stream()))


def mfma_probe_flops(iters):
    """Flops of one mfma_probe launch: 2048 wavefronts x 4 chains x iters
    products of 32 x 32 x 16."""
    return 2048 * 4 * int(iters) * 2 * 32 * 32 * 16


class Scheduler:
    """Host block allocator + continuous-batching scheduler of libpagedkv.so
    (pkv_sched_*).  step() returns the next engine step as numpy arrays ready
    for the kernels: seq_ids [B], q_lens [B], context_lens [B], cu_q_lens
    [B+1] and block_tables [B][max_blocks_per_seq] (int32, -1 past the last
    block)."""

    def __init__(self, num_blocks, block_size, max_blocks_per_seq, max_batch,
                 max_step_tokens, static_batching=False):
        import numpy as np
        self._np = np
        self._lib = host_library()
        self.max_batch, self.max_blocks_per_seq = max_batch, max_blocks_per_seq
        self._h = self._lib.pkv_sched_create(num_blocks, block_size, max_blocks_per_seq,
                                             max_batch, max_step_tokens,
                                             1 if static_batching else 0)
        if not self._h:
            raise ValueError("pkv_sched_create: every size must be positive")
        self._ids = np.zeros(max_batch, dtype=np.int64)
        self._q = np.zeros(max_batch, dtype=np.int32)
        self._ctx = np.zeros(max_batch, dtype=np.int32)
        self._cu = np.zeros(max_batch + 1, dtype=np.int32)
        self._tab = np.zeros((max_batch, max_blocks_per_seq), dtype=np.int32)

    def close(self):
        if self._h:
            self._lib.pkv_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    def add_request(self, rid, prompt_len, max_new_tokens, prefix_owner=None, prefix_len=0):
        """Queue a request; with prefix_owner, its first prefix_len tokens are the
        owner's and their blocks are shared when it is admitted."""
        if prefix_owner is None:
            rc = self._lib.pkv_sched_add_request(self._h, int(rid), int(prompt_len),
                                                 int(max_new_tokens))
        else:
            rc = self._lib.pkv_sched_add_request_prefix(self._h, int(rid), int(prompt_len),
                                                        int(max_new_tokens), int(prefix_owner),
                                                        int(prefix_len))
        if rc != PKV_OK:
            raise PagedKVError(rc, f"request {rid}: prompt {prompt_len}, max_new "
                               f"{max_new_tokens} rejected")

    def fork(self, parent, child, extra_tokens):
        """Start `child` from the decoding sequence `parent`, sharing its blocks."""
        rc = self._lib.pkv_sched_fork(self._h, int(parent), int(child), int(extra_tokens))
        if rc != PKV_OK:
            raise PagedKVError(rc, f"fork {parent} -> {child} rejected")

    def copies(self):
        """(src, dst) int32 arrays of the block copies the last step needs first."""
        n = self._lib.pkv_sched_copies(self._h, None, None, 0)
        src = self._np.zeros(max(n, 1), dtype=self._np.int32)
        dst = self._np.zeros(max(n, 1), dtype=self._np.int32)
        self._lib.pkv_sched_copies(self._h, src.ctypes.data_as(ctypes.c_void_p),
                                   dst.ctypes.data_as(ctypes.c_void_p), n)
        return src[:n], dst[:n]

    def step(self):
        p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
        B = self._lib.pkv_sched_step(self._h, p(self._ids), p(self._q), p(self._ctx),
                                     p(self._cu), p(self._tab))
        if B < 0:
            raise PagedKVError(B, "pkv_sched_step")
        return dict(seq_ids=self._ids[:B].copy(), q_lens=self._q[:B].copy(),
                    context_lens=self._ctx[:B].copy(), cu_q_lens=self._cu[:B + 1].copy(),
                    block_tables=self._tab[:B].copy())

    def _events(self, which):
        n = self._lib.pkv_sched_events(self._h, which, None, 0)
        out = self._np.zeros(max(n, 1), dtype=self._np.int64)
        self._lib.pkv_sched_events(self._h, which, out.ctypes.data_as(ctypes.c_void_p), n)
        return out[:n].tolist()

    def finished(self):
        """Requests that finished in the last step."""
        return self._events(0)

    def preempted(self):
        """Requests preempted (blocks released, requeued) in the last step."""
        return self._events(1)

    def stats(self):
        out = self._np.zeros(PKV_SCHED_STATS, dtype=self._np.int64)
        _check_host(self._lib, self._lib.pkv_sched_stats(self._h,
                                                         out.ctypes.data_as(ctypes.c_void_p)))
        return {k: int(out[i]) for i, k in enumerate(SCHED_STAT_NAMES)}


def decode_workspace(B, Hq, D, max_context_len, partition_size, device):
    """Allocate (with torch) the zero-filled workspace a decode call needs, or
    None.  Later calls leave it zeroed, so it can be reused call after call."""
    n = paged_attention_decode_workspace_size(B, Hq, D, max_context_len, partition_size)
    if n == 0:
        return None
    return _torch().zeros(n, dtype=_torch().uint8, device=device)
