"""ctypes binding over libpagedattn.so (include/pagedattn.h).

Argument marshalling only: torch tensors supply device pointers and the current HIP
stream; every step of the computation runs in the library's kernels.  If the library is
not built, every call raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

F32, BF16, FP8_E4M3, FP8_E5M2, INT8 = 0, 1, 2, 3, 4
# A uint8 pool holds E4M3 codes; an E5M2 pool must be typed torch.float8_e5m2 and an INT8 pool
# torch.int8 (a uint8 buffer can be viewed as either).
_TORCH_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: FP8_E4M3,
               torch.float8_e4m3fn: FP8_E4M3, torch.float8_e5m2: FP8_E5M2, torch.int8: INT8}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")
_lib = None
_lock = threading.Lock()

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_NO_BLOCKS = range(6)


class BmStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("free_blocks", "evictable_blocks", "used_blocks", "cached_blocks",
                                              "lookups", "hits", "evictions", "cow_copies")]

# Every symbol include/pagedattn.h declares.
EXPORTS = (
    "pa_kv_cache_write", "pa_decode_workspace_size",
    "pa_paged_attention_decode", "pa_paged_attention_decode_phase", "pa_kv_bytes_per_token",
    "pa_pool_bytes", "pa_probe_tile_read", "pa_status_string", "pa_last_error",
    "pa_chunked_prefill_workspace_size", "pa_paged_attention_chunked_prefill", "pa_paged_attention_decode_append",
    "pa_paged_attention_decode_shared", "pa_copy_blocks", "pa_bm_create", "pa_bm_destroy", "pa_bm_add_sequence", "pa_bm_append_token", "pa_bm_fork",
    "pa_bm_free_sequence", "pa_bm_block_table", "pa_bm_refcount", "pa_bm_get_stats",
    "pa_paged_attention_decode_noalloc", "pa_decode_noalloc_max_workspace", "pa_validate_tables",
)


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


def library():
    """The loaded library (ctypes.CDLL) with its signatures declared."""
    global _lib
    lib = _lib
    if lib is not None:
        return lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpagedattn.so is not built (%s); run `python -m paged_kv_cache_461_amd.build`"
                               % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        lib.pa_kv_cache_write.restype = I32
        lib.pa_kv_cache_write.argtypes = [P, P, I32, P, P, I64, I32, P, I32, I32, I32, I32, P, P, P]
        lib.pa_decode_workspace_size.restype = I64
        lib.pa_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32]
        dec = [P, P, I32, P, P, I64, I32, P, I32, P, I32, I32, I32, I32, I32, I32, F, P, P, I32, P, SZ, P]
        lib.pa_paged_attention_decode.restype = I32
        lib.pa_paged_attention_decode.argtypes = dec
        lib.pa_paged_attention_decode_phase.restype = I32
        lib.pa_paged_attention_decode_phase.argtypes = [I32] + dec
        lib.pa_paged_attention_decode_shared.restype = I32
        lib.pa_paged_attention_decode_shared.argtypes = [I32] + dec[:10] + [P] + dec[10:]
        lib.pa_paged_attention_decode_noalloc.restype = I32
        lib.pa_paged_attention_decode_noalloc.argtypes = dec[:20] + [P]
        lib.pa_decode_noalloc_max_workspace.restype = I64
        lib.pa_decode_noalloc_max_workspace.argtypes = []
        lib.pa_paged_attention_decode_append.restype = I32
        lib.pa_paged_attention_decode_append.argtypes = [I32, P, P, I32, P, P] + dec[3:]
        lib.pa_chunked_prefill_workspace_size.restype = I64
        lib.pa_chunked_prefill_workspace_size.argtypes = [I32] * 9
        lib.pa_paged_attention_chunked_prefill.restype = I32
        lib.pa_paged_attention_chunked_prefill.argtypes = [P, P, I32, P, I32, I32, P, P, I64, I32, P, I32, P, I32, I32,
                                                           I32, I32, I32, I32, F, P, P, I32, P, SZ, P]
        lib.pa_kv_bytes_per_token.restype = I64
        lib.pa_kv_bytes_per_token.argtypes = [I32, I32, I32, I32]
        lib.pa_pool_bytes.restype = I64
        lib.pa_pool_bytes.argtypes = [I64, I32, I32, I32, I32]
        lib.pa_validate_tables.restype = I32
        lib.pa_validate_tables.argtypes = [P, I32, P, I32, I32, I32, I64, P, I32, P]
        lib.pa_probe_tile_read.restype = I32
        lib.pa_probe_tile_read.argtypes = [P, I64, P, I64, I32, P, P]
        lib.pa_copy_blocks.restype = I32
        lib.pa_copy_blocks.argtypes = [P, P, I64, I64, P, I32, P]
        lib.pa_bm_create.restype = P
        lib.pa_bm_create.argtypes = [I64, I32]
        lib.pa_bm_destroy.restype = None
        lib.pa_bm_destroy.argtypes = [P]
        lib.pa_bm_add_sequence.restype = I32
        lib.pa_bm_add_sequence.argtypes = [P, I64, P, I32, P]
        lib.pa_bm_append_token.restype = I32
        lib.pa_bm_append_token.argtypes = [P, I64, I32, P, P, P]
        lib.pa_bm_fork.restype = I32
        lib.pa_bm_fork.argtypes = [P, I64, I64]
        lib.pa_bm_free_sequence.restype = I32
        lib.pa_bm_free_sequence.argtypes = [P, I64]
        lib.pa_bm_block_table.restype = I32
        lib.pa_bm_block_table.argtypes = [P, I64, P, I32, P, P]
        lib.pa_bm_refcount.restype = I32
        lib.pa_bm_refcount.argtypes = [P, I32]
        lib.pa_bm_get_stats.restype = I32
        lib.pa_bm_get_stats.argtypes = [P, ctypes.POINTER(BmStats)]
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_status_string.argtypes = [I32]
        lib.pa_last_error.restype = ctypes.c_char_p
        lib.pa_last_error.argtypes = []
        _lib = lib
        return lib


def _check(status: int):
    if status != PA_OK:
        lib = library()
        raise PagedAttnError(status, "%s: %s" % (lib.pa_status_string(status).decode(),
                                                 lib.pa_last_error().decode()))


def dtype_code(t: torch.Tensor) -> int:
    try:
        return _TORCH_CODE[t.dtype]
    except KeyError:
        raise TypeError("unsupported tensor dtype %s" % t.dtype) from None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(name, t, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _check_scales(pool, k_scale, v_scale, num_kv_heads):
    """The kernels read k_scale[g] and v_scale[g] for every kv head g of a quantised cache: both must
    hold num_kv_heads values (a per-tensor scale is passed repeated per head)."""
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t is not None and t.numel() != num_kv_heads:
            raise ValueError("%s must hold one fp32 value per kv head (%d), got %d" % (name, num_kv_heads, t.numel()))


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


class PreparedCall:
    """One library call whose arguments were checked and converted once (prepare_* functions).
    Calling it launches with exactly those arguments: the tensors must stay alive, keep their
    storage and shapes, and hold the step's data when it is called; `stream` (a torch stream or
    a raw handle) replaces the stream chosen at preparation.  A repeated step (a decode loop, a
    benchmark) pays the argument checks and conversions once instead of on every launch."""

    __slots__ = ("_fn", "_args", "_keep")

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, tuple(args), keep

    def __call__(self, stream=None):
        if stream is None:
            st = self._fn(*self._args)
        else:
            st = self._fn(*self._args[:-1], _stream(stream))
        if st != PA_OK:
            _check(st)


def num_pool_blocks(pool: torch.Tensor, num_kv_heads: int, head_dim: int, block_size: int) -> int:
    tile = num_kv_heads * block_size * head_dim
    if pool.numel() % tile:
        raise ValueError("pool of %d elements is not a whole number of %d-element blocks" % (pool.numel(), tile))
    return pool.numel() // tile


def _kv_cache_write_args(key, value, k_pool, v_pool, slot_mapping, num_kv_heads, head_dim, block_size, k_scale,
                         v_scale, stream):
    for n, t in (("key", key), ("value", value), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(n, t)
    _dev("slot_mapping", slot_mapping, torch.int64)
    _dev("k_scale", k_scale, torch.float32)
    _dev("v_scale", v_scale, torch.float32)
    _check_scales(k_pool, k_scale, v_scale, num_kv_heads)
    nb = num_pool_blocks(k_pool, num_kv_heads, head_dim, block_size)
    T = slot_mapping.numel()
    if key.numel() != T * num_kv_heads * head_dim or value.shape != key.shape:
        raise ValueError("key/value must be [%d][%d][%d]" % (T, num_kv_heads, head_dim))
    return library().pa_kv_cache_write, (
        _ptr(key), _ptr(value), dtype_code(key), _ptr(k_pool), _ptr(v_pool), nb, dtype_code(k_pool),
        _ptr(slot_mapping), T, num_kv_heads, head_dim, block_size, _ptr(k_scale), _ptr(v_scale), _stream(stream))


def kv_cache_write(key, value, k_pool, v_pool, slot_mapping, *, num_kv_heads, head_dim, block_size=16,
                   k_scale=None, v_scale=None, stream=None):
    """Store key/value rows [T][Hkv][D] into their pool slots (pa_kv_cache_write)."""
    fn, args = _kv_cache_write_args(key, value, k_pool, v_pool, slot_mapping, num_kv_heads, head_dim, block_size,
                                    k_scale, v_scale, stream)
    _check(fn(*args))


def prepare_kv_cache_write(key, value, k_pool, v_pool, slot_mapping, *, num_kv_heads, head_dim, block_size=16,
                           k_scale=None, v_scale=None, stream=None) -> PreparedCall:
    """kv_cache_write with its arguments checked and converted once (PreparedCall)."""
    fn, args = _kv_cache_write_args(key, value, k_pool, v_pool, slot_mapping, num_kv_heads, head_dim, block_size,
                                    k_scale, v_scale, stream)
    return PreparedCall(fn, args, (key, value, k_pool, v_pool, slot_mapping, k_scale, v_scale))


def decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, block_size=16,
                          partition_size=0) -> int:
    n = int(library().pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                               max_context_len, partition_size))
    if n < 0:
        raise ValueError("invalid decode shape")
    return n


def decode_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, block_size=16,
                     partition_size=0, device="cuda"):
    """A workspace tensor of the required size (None for an empty batch)."""
    n = decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, block_size,
                              partition_size)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _decode_args(out, query, k_pool, v_pool, block_tables, context_lens, max_context_len, num_kv_heads, scale,
                 block_size, k_scale, v_scale, partition_size, workspace, phase, stream, shared_blocks):
    for n, t in (("out", out), ("query", query), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(n, t)
    _dev("block_tables", block_tables, torch.int32)
    _dev("context_lens", context_lens, torch.int32)
    _dev("k_scale", k_scale, torch.float32)
    _dev("v_scale", v_scale, torch.float32)
    _check_scales(k_pool, k_scale, v_scale, num_kv_heads)
    _dev("workspace", workspace)
    if query.dim() != 3 or out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("query and out must both be [num_seqs][num_heads][head_dim] of one dtype")
    S, Hq, D = query.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs][max_blocks] and context_lens [num_seqs]")
    nb = num_pool_blocks(k_pool, num_kv_heads, D, block_size)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (int(phase), _ptr(out), _ptr(query), dtype_code(query), _ptr(k_pool), _ptr(v_pool), nb,
            dtype_code(k_pool), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens))
    tail = (int(max_context_len), S, Hq, num_kv_heads, D, block_size, float(scale), _ptr(k_scale), _ptr(v_scale),
            int(partition_size), _ptr(workspace), ws_bytes, _stream(stream))
    if shared_blocks is not None:
        _dev("shared_blocks", shared_blocks, torch.int32)
        if shared_blocks.numel() != S:
            raise ValueError("shared_blocks must be [num_seqs]")
        return library().pa_paged_attention_decode_shared, head + (_ptr(shared_blocks),) + tail
    return library().pa_paged_attention_decode_phase, head + tail


def paged_attention_decode(out, query, k_pool, v_pool, block_tables, context_lens, *, max_context_len,
                           num_kv_heads, scale, block_size=16, k_scale=None, v_scale=None, partition_size=0,
                           workspace=None, phase=3, stream=None, shared_blocks=None):
    """One query row per sequence over its paged context (pa_paged_attention_decode[_phase]).
    query/out: [S][Hq][D]; block_tables: int32 [S][max_blocks]; context_lens: int32 [S].
    shared_blocks: optional int32 [S], the leading blocks of each sequence that other sequences
    share (pa_paged_attention_decode_shared: those are read with cached loads)."""
    fn, args = _decode_args(out, query, k_pool, v_pool, block_tables, context_lens, max_context_len, num_kv_heads,
                            scale, block_size, k_scale, v_scale, partition_size, workspace, phase, stream,
                            shared_blocks)
    _check(fn(*args))
    return out


def prepare_paged_attention_decode(out, query, k_pool, v_pool, block_tables, context_lens, *, max_context_len,
                                   num_kv_heads, scale, block_size=16, k_scale=None, v_scale=None,
                                   partition_size=0, workspace=None, phase=3, stream=None,
                                   shared_blocks=None) -> PreparedCall:
    """paged_attention_decode with its arguments checked and converted once (PreparedCall)."""
    fn, args = _decode_args(out, query, k_pool, v_pool, block_tables, context_lens, max_context_len, num_kv_heads,
                            scale, block_size, k_scale, v_scale, partition_size, workspace, phase, stream,
                            shared_blocks)
    return PreparedCall(fn, args, (out, query, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale,
                                   workspace, shared_blocks))


def paged_attention_decode_noalloc(out, query, k_pool, v_pool, block_tables, context_lens, *, max_context_len,
                                   num_kv_heads, scale, block_size=16, k_scale=None, v_scale=None, partition_size=0,
                                   stream=None):
    """pa_paged_attention_decode without a workspace: the library's static per-GPU scratch holds
    the split-K partial results (pa_paged_attention_decode_noalloc).  Calls that overlap on one
    GPU race."""
    for n, t in (("out", out), ("query", query), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(n, t)
    _dev("block_tables", block_tables, torch.int32)
    _dev("context_lens", context_lens, torch.int32)
    _dev("k_scale", k_scale, torch.float32)
    _dev("v_scale", v_scale, torch.float32)
    if query.dim() != 3 or out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("query and out must both be [num_seqs][num_heads][head_dim] of one dtype")
    S, Hq, D = query.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs][max_blocks] and context_lens [num_seqs]")
    _check_scales(k_pool, k_scale, v_scale, num_kv_heads)
    nb = num_pool_blocks(k_pool, num_kv_heads, D, block_size)
    _check(library().pa_paged_attention_decode_noalloc(
        _ptr(out), _ptr(query), dtype_code(query), _ptr(k_pool), _ptr(v_pool), nb, dtype_code(k_pool),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), int(max_context_len), S, Hq, num_kv_heads, D,
        block_size, float(scale), _ptr(k_scale), _ptr(v_scale), int(partition_size), _stream(stream)))
    return out


def decode_noalloc_max_workspace() -> int:
    return int(library().pa_decode_noalloc_max_workspace())


def chunked_prefill_workspace_size(num_query_rows, num_seqs, max_query_len, num_heads, num_kv_heads, head_dim,
                                   max_context_len, block_size=16, partition_size=0) -> int:
    n = int(library().pa_chunked_prefill_workspace_size(num_query_rows, num_seqs, max_query_len, num_heads,
                                                        num_kv_heads, head_dim, block_size, max_context_len,
                                                        partition_size))
    if n < 0:
        raise ValueError("invalid chunked-prefill shape")
    return n


def chunked_prefill_workspace(num_query_rows, num_seqs, max_query_len, num_heads, num_kv_heads, head_dim,
                              max_context_len, block_size=16, partition_size=0, device="cuda"):
    """A workspace tensor of the required size (None when the call needs none)."""
    n = chunked_prefill_workspace_size(num_query_rows, num_seqs, max_query_len, num_heads, num_kv_heads, head_dim,
                                       max_context_len, block_size, partition_size)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _prefill_args(out, query, cu_query_lens, k_pool, v_pool, block_tables, context_lens, max_query_len,
                  max_context_len, num_kv_heads, scale, block_size, k_scale, v_scale, partition_size, workspace,
                  stream):
    for n, t in (("out", out), ("query", query), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(n, t)
    _dev("cu_query_lens", cu_query_lens, torch.int32)
    _dev("block_tables", block_tables, torch.int32)
    _dev("context_lens", context_lens, torch.int32)
    _dev("k_scale", k_scale, torch.float32)
    _dev("v_scale", v_scale, torch.float32)
    _check_scales(k_pool, k_scale, v_scale, num_kv_heads)
    _dev("workspace", workspace)
    if query.dim() != 3 or out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("query and out must both be [num_query_rows][num_heads][head_dim] of one dtype")
    rows, Hq, D = query.shape
    S = context_lens.numel()
    if cu_query_lens.numel() != S + 1 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("cu_query_lens must be [S+1], block_tables [S][max_blocks], context_lens [S]")
    nb = num_pool_blocks(k_pool, num_kv_heads, D, block_size)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return library().pa_paged_attention_chunked_prefill, (
        _ptr(out), _ptr(query), dtype_code(query), _ptr(cu_query_lens), rows, int(max_query_len), _ptr(k_pool),
        _ptr(v_pool), nb, dtype_code(k_pool), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), S, Hq, num_kv_heads, D, block_size, float(scale), _ptr(k_scale), _ptr(v_scale),
        int(partition_size), _ptr(workspace), ws_bytes, _stream(stream))


def paged_attention_chunked_prefill(out, query, cu_query_lens, k_pool, v_pool, block_tables, context_lens, *,
                                    max_query_len, max_context_len, num_kv_heads, scale, block_size=16,
                                    k_scale=None, v_scale=None, partition_size=0, workspace=None, stream=None):
    """Causal attention of each sequence's last q_len positions over its paged context
    (pa_paged_attention_chunked_prefill).  query/out: [rows][Hq][D] bf16; cu_query_lens:
    int32 [S+1]; block_tables: int32 [S][max_blocks]; context_lens: int32 [S]."""
    fn, args = _prefill_args(out, query, cu_query_lens, k_pool, v_pool, block_tables, context_lens, max_query_len,
                             max_context_len, num_kv_heads, scale, block_size, k_scale, v_scale, partition_size,
                             workspace, stream)
    _check(fn(*args))
    return out


def prepare_paged_attention_chunked_prefill(out, query, cu_query_lens, k_pool, v_pool, block_tables,
                                            context_lens, *, max_query_len, max_context_len, num_kv_heads, scale,
                                            block_size=16, k_scale=None, v_scale=None, partition_size=0,
                                            workspace=None, stream=None) -> PreparedCall:
    """paged_attention_chunked_prefill with its arguments checked and converted once (PreparedCall)."""
    fn, args = _prefill_args(out, query, cu_query_lens, k_pool, v_pool, block_tables, context_lens, max_query_len,
                             max_context_len, num_kv_heads, scale, block_size, k_scale, v_scale, partition_size,
                             workspace, stream)
    return PreparedCall(fn, args, (out, query, cu_query_lens, k_pool, v_pool, block_tables, context_lens, k_scale,
                                   v_scale, workspace))


def _decode_append_args(out, query, new_key, new_value, k_pool, v_pool, block_tables, context_lens,
                        max_context_len, num_kv_heads, scale, block_size, k_scale, v_scale, partition_size,
                        workspace, phase, stream):
    for n, t in (("out", out), ("query", query), ("new_key", new_key), ("new_value", new_value),
                 ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(n, t)
    _dev("block_tables", block_tables, torch.int32)
    _dev("context_lens", context_lens, torch.int32)
    _dev("k_scale", k_scale, torch.float32)
    _dev("v_scale", v_scale, torch.float32)
    _check_scales(k_pool, k_scale, v_scale, num_kv_heads)
    _dev("workspace", workspace)
    if query.dim() != 3 or out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("query and out must both be [num_seqs][num_heads][head_dim] of one dtype")
    S, Hq, D = query.shape
    if new_key.shape != (S, num_kv_heads, D) or new_value.shape != new_key.shape or new_key.dtype != query.dtype \
            or new_value.dtype != query.dtype:
        raise ValueError("new_key/new_value must be [%d][%d][%d] in the query dtype" % (S, num_kv_heads, D))
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs][max_blocks] and context_lens [num_seqs]")
    nb = num_pool_blocks(k_pool, num_kv_heads, D, block_size)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return library().pa_paged_attention_decode_append, (
        int(phase), _ptr(out), _ptr(query), dtype_code(query), _ptr(new_key), _ptr(new_value), _ptr(k_pool),
        _ptr(v_pool), nb, dtype_code(k_pool), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), S, Hq, num_kv_heads, D, block_size, float(scale), _ptr(k_scale), _ptr(v_scale),
        int(partition_size), _ptr(workspace), ws_bytes, _stream(stream))


def paged_attention_decode_append(out, query, new_key, new_value, k_pool, v_pool, block_tables, context_lens, *,
                                  max_context_len, num_kv_heads, scale, block_size=16, k_scale=None, v_scale=None,
                                  partition_size=0, workspace=None, phase=3, stream=None):
    """Store each sequence's new K/V row at position context_lens[s] - 1, then decode
    (pa_paged_attention_decode_append).  new_key/new_value: [S][Hkv][D] in the query dtype."""
    fn, args = _decode_append_args(out, query, new_key, new_value, k_pool, v_pool, block_tables, context_lens,
                                   max_context_len, num_kv_heads, scale, block_size, k_scale, v_scale,
                                   partition_size, workspace, phase, stream)
    _check(fn(*args))
    return out


def prepare_paged_attention_decode_append(out, query, new_key, new_value, k_pool, v_pool, block_tables,
                                          context_lens, *, max_context_len, num_kv_heads, scale, block_size=16,
                                          k_scale=None, v_scale=None, partition_size=0, workspace=None, phase=3,
                                          stream=None) -> PreparedCall:
    """paged_attention_decode_append with its arguments checked and converted once (PreparedCall)."""
    fn, args = _decode_append_args(out, query, new_key, new_value, k_pool, v_pool, block_tables, context_lens,
                                   max_context_len, num_kv_heads, scale, block_size, k_scale, v_scale,
                                   partition_size, workspace, phase, stream)
    return PreparedCall(fn, args, (out, query, new_key, new_value, k_pool, v_pool, block_tables, context_lens,
                                   k_scale, v_scale, workspace))


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, cache_dtype) -> int:
    return int(library().pa_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, cache_dtype))


def pool_bytes(num_blocks, num_kv_heads, head_dim, block_size, cache_dtype) -> int:
    return int(library().pa_pool_bytes(num_blocks, num_kv_heads, head_dim, block_size, cache_dtype))


def validate_tables(block_tables, context_lens, max_context_len, block_size, num_blocks, slots=None,
                    block_refcounts=None):
    """Debug check of host copies of a call's block tables, context lengths and (optionally)
    write slots and the block manager's reference counts (pa_validate_tables).  Arrays are
    numpy arrays or CPU tensors; raises PagedAttnError naming the first violation."""
    import numpy as np

    def host(x, dt):
        if x is None:
            return None
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
        return np.ascontiguousarray(np.asarray(x), dtype=dt)

    bt = host(block_tables, np.int32)
    cl = host(context_lens, np.int32)
    sl = host(slots, np.int64)
    rc = host(block_refcounts, np.int32)
    if bt.ndim != 2 or cl.ndim != 1 or bt.shape[0] != cl.shape[0]:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq] and context_lens [num_seqs]")
    if rc is not None and (sl is None or rc.shape != (int(num_blocks),)):
        raise ValueError("block_refcounts needs slots and one count per block")
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p) if a is not None and a.size else None
    _check(library().pa_validate_tables(ptr(bt), bt.shape[1], ptr(cl), cl.shape[0], int(max_context_len),
                                        int(block_size), int(num_blocks), ptr(sl), 0 if sl is None else sl.size,
                                        ptr(rc)))


def probe_tile_read(buf, order, sink, grid_workgroups=2048, stream=None):
    """Read order.numel() 4 KiB tiles of buf in the given order (pa_probe_tile_read)."""
    _dev("buf", buf)
    _dev("order", order, torch.int32)
    _dev("sink", sink)
    _check(library().pa_probe_tile_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(order), order.numel(),
                                        int(grid_workgroups), _ptr(sink), _stream(stream)))


def copy_blocks(k_pool, v_pool, pairs, *, num_kv_heads, head_dim, block_size=16, stream=None):
    """Copy pool blocks pairs[i][0] -> pairs[i][1] in both pools (pa_copy_blocks); pairs is a
    device int32 tensor [n][2]."""
    _dev("k_pool", k_pool)
    _dev("v_pool", v_pool)
    _dev("pairs", pairs, torch.int32)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n][2]")
    nb = num_pool_blocks(k_pool, num_kv_heads, head_dim, block_size)
    block_bytes = num_kv_heads * block_size * head_dim * k_pool.element_size()
    _check(library().pa_copy_blocks(_ptr(k_pool), _ptr(v_pool), nb, block_bytes, _ptr(pairs), pairs.shape[0],
                                    _stream(stream)))


class BlockManager:
    """The library's host-side block manager (pa_bm_*): refcounted blocks, block-granular
    prefix caching, copy-on-write on append to a shared partial block."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self._lib = library()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError("bad block manager arguments (num_blocks %d, block_size %d)" % (num_blocks, block_size))
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self, seq_id: int, tokens) -> int:
        """Returns the number of leading prompt tokens served from the prefix cache."""
        t = (ctypes.c_int32 * len(tokens))(*[int(x) for x in tokens])
        cached = ctypes.c_int32(0)
        _check(self._lib.pa_bm_add_sequence(self._h, int(seq_id), t, len(tokens), ctypes.byref(cached)))
        return cached.value

    def append_token(self, seq_id: int, token: int):
        """Returns (slot, copy) where copy is None or the (source, destination) block pair."""
        slot, src, dst = ctypes.c_int64(0), ctypes.c_int32(-1), ctypes.c_int32(-1)
        _check(self._lib.pa_bm_append_token(self._h, int(seq_id), int(token), ctypes.byref(slot), ctypes.byref(src),
                                            ctypes.byref(dst)))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def fork(self, parent: int, child: int):
        _check(self._lib.pa_bm_fork(self._h, int(parent), int(child)))

    def free_sequence(self, seq_id: int):
        _check(self._lib.pa_bm_free_sequence(self._h, int(seq_id)))

    def block_table(self, seq_id: int):
        """(list of physical block ids, number of tokens)."""
        nb, nt = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(self._lib.pa_bm_block_table(self._h, int(seq_id), None, 0, ctypes.byref(nb), ctypes.byref(nt)))
        row = (ctypes.c_int32 * max(nb.value, 1))()
        _check(self._lib.pa_bm_block_table(self._h, int(seq_id), row, nb.value, None, None))
        return list(row)[:nb.value], nt.value

    def refcount(self, block: int) -> int:
        return self._lib.pa_bm_refcount(self._h, int(block))

    def stats(self) -> dict:
        st = BmStats()
        _check(self._lib.pa_bm_get_stats(self._h, ctypes.byref(st)))
        return {n: getattr(st, n) for n, _ in BmStats._fields_}
