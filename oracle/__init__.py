"""CPU float64 oracle for paged KV append and paged attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports, links or calls it, and it imports nothing from the
product package.  The arithmetic lives in ``pa_oracle.c`` (plain C99, float64, compiled
with gcc -O2, no fast-math); this module only builds it and marshals numpy arrays.

Element types are passed as numpy arrays of their raw bits: fp32 as ``float32``, bf16 as
``uint16``, OCP fp8 E4M3 / E5M2 and INT8 (two's complement) as ``uint8``.  Dtype codes: 0 fp32,
1 bf16, 2 fp8 e4m3, 3 fp8 e5m2, 4 int8.

Pins (tests/test_oracle_*.py check this module against what the pages and mathematics fix):
  * attention == torch scaled_dot_product_attention in float64 on the contiguous
    (un-paged) K/V with query head h reading kv head h // G, to 1e-12;
  * exact invariance under any relabelling of physical blocks, including the pages'
    worked logical->physical map 0->7, 1->2, 2->19, 3->4;
  * closed forms: one visible token gives that token's V; identical keys give the mean of
    V; adding one vector to every key leaves the output unchanged; a dominant key selects
    its value;
  * E4M3 decode table == torch.float8_e4m3fn for all 256 codes; encode == torch's
    round-to-nearest-even cast wherever that cast does not overflow, saturation to 448
    above it, and round trip on every finite code;
  * E5M2: the same three pins against torch.float8_e5m2 (saturation at 57344);
  * INT8: encode == numpy's binary32 division then round-half-even (numpy.rint), saturated to
    [-127, 127], over every bf16 pattern at several scales; decode == the int8 view of the byte;
  * KV bytes per token == 131072 for 32 layers x 8 kv heads x 128 x bf16.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F32, BF16, FP8_E4M3, FP8_E5M2, INT8 = 0, 1, 2, 3, 4
_NP_OF = {F32: np.float32, BF16: np.uint16, FP8_E4M3: np.uint8, FP8_E5M2: np.uint8, INT8: np.uint8}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_liboracle.so")
_lib = None
_lock = threading.Lock()

_ERRORS = {1: "invalid argument", 2: "unsupported dtype", 3: "index out of bounds", 4: "out of memory"}


def build(force: bool = True) -> str:
    """Compile pa_oracle.c into _liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_k_elem_index.restype = L
    lib.oracle_k_elem_index.argtypes = [L, I, I, I, I, I, I, I]
    lib.oracle_v_elem_index.restype = L
    lib.oracle_v_elem_index.argtypes = [L, I, I, I, I, I, I, I]
    lib.oracle_e4m3_to_double.restype = D
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_kv_cache_write.restype = I
    lib.oracle_kv_cache_write.argtypes = [P, P, I, P, P, I, L, P, L, I, I, I, P, P]
    lib.oracle_paged_attention.restype = I
    lib.oracle_paged_attention.argtypes = [P, P, I, P, P, I, L, P, I, P, P, I, I, I, I, I,
                                           D, P, P, I]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_e4m3_encode_array.argtypes = [P, P, L]
    lib.oracle_e4m3_decode_array.restype = None
    lib.oracle_e4m3_decode_array.argtypes = [P, P, L]
    lib.oracle_e5m2_to_double.restype = D
    lib.oracle_e5m2_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e5m2_encode.restype = ctypes.c_uint8
    lib.oracle_e5m2_encode.argtypes = [ctypes.c_float]
    lib.oracle_e5m2_encode_array.restype = None
    lib.oracle_e5m2_encode_array.argtypes = [P, P, L]
    lib.oracle_e5m2_decode_array.restype = None
    lib.oracle_e5m2_decode_array.argtypes = [P, P, L]
    lib.oracle_int8_to_double.restype = D
    lib.oracle_int8_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_int8_encode.restype = ctypes.c_uint8
    lib.oracle_int8_encode.argtypes = [ctypes.c_float]
    lib.oracle_int8_encode_array.restype = None
    lib.oracle_int8_encode_array.argtypes = [P, P, L]
    lib.oracle_int8_decode_array.restype = None
    lib.oracle_int8_decode_array.argtypes = [P, P, L]
    lib.oracle_kv_bytes_per_token.restype = L
    lib.oracle_kv_bytes_per_token.argtypes = [I, I, I, I]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
        return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(st):
    if st != 0:
        raise RuntimeError("oracle error %d: %s" % (st, _ERRORS.get(st, "?")))


def _as(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def k_elem_index(block, kv_head, token, d, num_kv_heads, head_dim, block_size, dtype):
    return _load().oracle_k_elem_index(block, kv_head, token, d, num_kv_heads, head_dim,
                                       block_size, dtype)


def v_elem_index(block, kv_head, token, d, num_kv_heads, head_dim, block_size, dtype):
    return _load().oracle_v_elem_index(block, kv_head, token, d, num_kv_heads, head_dim,
                                       block_size, dtype)


def e4m3_to_float64(codes) -> np.ndarray:
    """Value of each E4M3 code (NaN for S.1111.111)."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib.oracle_e4m3_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def e4m3_encode(y) -> np.ndarray:
    """Round binary32 values to E4M3 codes (nearest-even, saturating at +-448)."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib.oracle_e4m3_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def e5m2_to_float64(codes) -> np.ndarray:
    """Value of each E5M2 code (+-inf for S.11111.00, NaN for S.11111.mm with mm != 0)."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib.oracle_e5m2_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def e5m2_encode(y) -> np.ndarray:
    """Round binary32 values to E5M2 codes (nearest-even, saturating at +-57344)."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib.oracle_e5m2_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def int8_to_float64(codes) -> np.ndarray:
    """Integer value of each INT8 code byte (two's complement)."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib.oracle_int8_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def int8_encode(y) -> np.ndarray:
    """Round binary32 values to INT8 code bytes (nearest integer, ties to even, saturating at
    +-127, NaN -> 0)."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib.oracle_int8_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def kv_cache_write(key, value, src_dtype, k_pool, v_pool, cache_dtype, slot_mapping,
                   num_kv_heads, head_dim, block_size, k_scale=None, v_scale=None):
    """Append tokens to the pools in place.  key/value: [T][Hkv][D] raw-bit arrays of
    src_dtype; pools: raw-bit arrays of cache_dtype with num_blocks*Hkv*B*D elements;
    slot_mapping: int64 [T] (negative = skip)."""
    lib = _load()
    key = _as(key, _NP_OF[src_dtype])
    value = _as(value, _NP_OF[src_dtype])
    if not (k_pool.flags.c_contiguous and v_pool.flags.c_contiguous):
        raise ValueError("pools must be C-contiguous (written in place)")
    for p in (k_pool, v_pool):
        if p.dtype != _NP_OF[cache_dtype]:
            raise TypeError("pool dtype mismatch")
    slots = _as(slot_mapping, np.int64)
    T = slots.shape[0]
    if key.size != T * num_kv_heads * head_dim or value.size != key.size:
        raise ValueError("key/value size mismatch")
    tile = num_kv_heads * block_size * head_dim
    nb = k_pool.size // tile
    if v_pool.size != k_pool.size or k_pool.size % tile:
        raise ValueError("pool size mismatch")
    ks = None if k_scale is None else _as(k_scale, np.float32)
    vs = None if v_scale is None else _as(v_scale, np.float32)
    _check(lib.oracle_kv_cache_write(_ptr(key), _ptr(value), src_dtype, _ptr(k_pool), _ptr(v_pool),
                                     cache_dtype, nb, _ptr(slots), T, num_kv_heads, head_dim,
                                     block_size, _ptr(ks), _ptr(vs)))


def paged_attention(query, q_dtype, k_pool, v_pool, cache_dtype, block_tables, context_lens,
                    num_heads, num_kv_heads, head_dim, block_size, scale, cu_query_lens=None,
                    k_scale=None, v_scale=None, nthreads=None) -> np.ndarray:
    """float64 [rows][Hq][D].  Decode when cu_query_lens is None (one row per sequence);
    otherwise rows cu_query_lens[s]..cu_query_lens[s+1]-1 belong to sequence s and occupy
    its last q_len positions (causal)."""
    lib = _load()
    q = _as(query, _NP_OF[q_dtype])
    tables = _as(block_tables, np.int32)
    ctx = _as(context_lens, np.int32)
    S = ctx.shape[0]
    if cu_query_lens is None:
        cu = np.arange(S + 1, dtype=np.int32)
    else:
        cu = _as(cu_query_lens, np.int32)
    rows = int(cu[-1]) if S else 0
    if q.size != rows * num_heads * head_dim:
        raise ValueError("query size mismatch")
    if tables.ndim != 2 or tables.shape[0] != S:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    tile = num_kv_heads * block_size * head_dim
    nb = k_pool.size // tile
    ks = None if k_scale is None else _as(k_scale, np.float32)
    vs = None if v_scale is None else _as(v_scale, np.float32)
    out = np.zeros((rows, num_heads, head_dim), dtype=np.float64)
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    _check(lib.oracle_paged_attention(_ptr(out), _ptr(q), q_dtype, _ptr(np.ascontiguousarray(k_pool)),
                                      _ptr(np.ascontiguousarray(v_pool)), cache_dtype, nb, _ptr(tables),
                                      tables.shape[1], _ptr(ctx), _ptr(cu), S, num_heads, num_kv_heads,
                                      head_dim, block_size, float(scale), _ptr(ks), _ptr(vs),
                                      int(nthreads)))
    return out


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype) -> int:
    return int(_load().oracle_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype))
