"""Seeded synthetic inputs for paged KV append and paged attention.

This module is shared by the tests, the benchmark and the smoke check, and by both sides of
a parity comparison.  It generates inputs only: sequence lengths, block allocation with
refcounts, block tables, slot mappings, random token values and the calibration scales of a
quantised (fp8 / INT8) cache.  It
contains none of the attention or quantisation arithmetic.  It imports nothing from the
HIP binding or from the oracle.

Every random draw comes from ``numpy.random.default_rng`` seeded with a tuple
``(seed, stream, ...)``, so any one sequence's tokens can be regenerated on its own.

  stream 100  lengths, block allocation, unused-table filler
  stream 101  per-(layer, sequence) token K/V values  (positions after a shared prefix)
  stream 102  per-layer shared-prefix K/V values
  stream 103  query rows
  stream 104  calibration batch of a quantised (fp8 / INT8) cache's scales

Values are N(0, 1) drawn in float32, then rounded to the cache source dtype (bf16 with
round-to-nearest-even).  The workload shapes follow the pages' running example of a
Llama-3-8B-sized model: 32 layers, 32 query heads, 8 KV heads, head dim 128, bf16, with
16-token blocks (page 3, section 2.1; page 1, sections 2.1 and 10).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32, BF16, FP8_E4M3, FP8_E5M2, INT8 = 0, 1, 2, 3, 4
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8_E4M3: "fp8_e4m3", FP8_E5M2: "fp8_e5m2", INT8: "int8"}
ELEM_BYTES = {F32: 4, BF16: 2, FP8_E4M3: 1, FP8_E5M2: 1, INT8: 1}
RAW_NP = {F32: np.float32, BF16: np.uint16, FP8_E4M3: np.uint8, FP8_E5M2: np.uint8, INT8: np.uint8}
# Unused slots are filled with a value no append writes: NaN, or the INT8 code -128 (0x80).
POISON = {F32: np.float32(np.nan), BF16: np.uint16(0x7FC0), FP8_E4M3: np.uint8(0x7F), FP8_E5M2: np.uint8(0x7F),
          INT8: np.uint8(0x80)}
FP8_DTYPES = (FP8_E4M3, FP8_E5M2)
QUANT_DTYPES = (FP8_E4M3, FP8_E5M2, INT8)  # caches of codes times a per-head scale

# Largest code magnitude of each quantised format, used only to size calibration scales: the
# largest finite OCP E4M3 / E5M2 values and the symmetric INT8 range.
QUANT_MAX = {FP8_E4M3: 448.0, FP8_E5M2: 57344.0, INT8: 127.0}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # uint32 arithmetic cannot wrap for a non-NaN input (the largest is 0xFF800000)
    r = ((u + (np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1)))) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((x.view(np.uint32)[nan] >> 16) | 0x0040).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_raw(values_f32: np.ndarray, dtype: int) -> np.ndarray:
    """float32 values -> raw bits of a source dtype (fp32 or bf16)."""
    if dtype == F32:
        return np.ascontiguousarray(values_f32, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(values_f32)
    raise ValueError("token sources are fp32 or bf16")


def raw_to_f32(raw: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.asarray(raw, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits_to_f32(raw)
    raise ValueError("fp32 or bf16 expected")


class BlockAllocator:
    """Physical block pool with a free list and per-block refcounts.

    Blocks are handed out from a seeded random permutation of all block ids, so physically
    consecutive blocks are unrelated (page 1, section 4: logically contiguous, physically
    scattered).  ``share`` adds a reference (a common prefix); ``free`` drops one and
    returns the block to the pool when the count reaches zero.
    """

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.num_blocks = int(num_blocks)
        self.free_list = [int(b) for b in rng.permutation(self.num_blocks)[::-1]]
        self.refcount = np.zeros(self.num_blocks, dtype=np.int32)

    def alloc(self, n: int) -> list[int]:
        if n > len(self.free_list):
            raise MemoryError("block pool exhausted: need %d, have %d" % (n, len(self.free_list)))
        ids = [self.free_list.pop() for _ in range(n)]
        for b in ids:
            self.refcount[b] = 1
        return ids

    def share(self, ids) -> list[int]:
        for b in ids:
            if self.refcount[b] <= 0:
                raise ValueError("sharing a free block %d" % b)
            self.refcount[b] += 1
        return list(ids)

    def free(self, ids) -> None:
        for b in ids:
            if self.refcount[b] <= 0:
                raise ValueError("double free of block %d" % b)
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free_list.append(int(b))

    @property
    def num_free(self) -> int:
        return len(self.free_list)


@dataclass
class PagedBatch:
    """One batch of sequences over a paged KV pool (one layer unless stated)."""

    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: int
    src_dtype: int           # dtype of the K/V rows handed to kv_cache_write
    cache_dtype: int         # dtype stored in the pool
    context_lens: np.ndarray  # int32 [S]; includes this step's new positions
    query_lens: np.ndarray    # int32 [S]; 1 for a decode sequence
    block_tables: np.ndarray  # int32 [S][max_blocks_per_seq]
    num_blocks: int
    seed: int
    layer: int = 0
    shared_prefix_len: int = 0
    sharing: np.ndarray = field(default_factory=lambda: np.zeros(0, dtype=np.int64))
    refcount: np.ndarray = field(default_factory=lambda: np.zeros(0, dtype=np.int32))
    k_scale: np.ndarray | None = None  # float32 [Hkv] for a quantised (fp8 / INT8) cache
    v_scale: np.ndarray | None = None
    fp8_scale: str = "head"  # quantised-cache scale granularity: "head" or "tensor" (one value repeated
                             # per head)

    # -- shapes ------------------------------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def cu_query_lens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    @property
    def num_rows(self) -> int:
        return int(self.query_lens.sum())

    @property
    def gqa(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        """1/sqrt(head_dim) as a float32 value (page 1, section 2)."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def pool_elems(self) -> int:
        return self.num_blocks * self.num_kv_heads * self.block_size * self.head_dim

    @property
    def pool_bytes(self) -> int:
        return self.pool_elems * ELEM_BYTES[self.cache_dtype]

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.query_lens == 1))

    # -- values --------------------------------------------------------------------------
    def _prefix_values(self) -> np.ndarray:
        rng = np.random.default_rng([self.seed, 102, self.layer])
        return rng.standard_normal((self.shared_prefix_len, 2, self.num_kv_heads, self.head_dim),
                                   dtype=np.float32)

    def _own_values(self, s: int, n: int) -> np.ndarray:
        rng = np.random.default_rng([self.seed, 101, self.layer, s])
        return rng.standard_normal((n, 2, self.num_kv_heads, self.head_dim), dtype=np.float32)

    def _own_start(self, s: int) -> int:
        return self.shared_prefix_len if s in set(self.sharing.tolist()) else 0

    def token_values(self, s: int, t0: int = 0, t1: int | None = None):
        """float32 K and V values of positions [t0, t1) of sequence s, rounded to the source
        dtype, each [n][Hkv][D]."""
        kv = self._token_f32(s, t0, t1)
        kv = raw_to_f32(to_raw(kv, self.src_dtype), self.src_dtype)
        return np.ascontiguousarray(kv[:, 0]), np.ascontiguousarray(kv[:, 1])

    def _token_f32(self, s: int, t0: int, t1: int | None) -> np.ndarray:
        """Unrounded float32 draws [n][2][Hkv][D] of positions [t0, t1) of sequence s."""
        ctx = int(self.context_lens[s])
        t1 = ctx if t1 is None else t1
        start = self._own_start(s)
        parts = []
        if t0 < start:
            parts.append(self._prefix_values()[t0:min(t1, start)])
        if t1 > start:
            own = self._own_values(s, ctx - start)
            parts.append(own[max(t0, start) - start:t1 - start])
        if len(parts) == 1:
            return parts[0]
        return np.concatenate(parts, axis=0) if parts else np.zeros(
            (0, 2, self.num_kv_heads, self.head_dim), np.float32)

    def token_raw(self, s: int, t0: int = 0, t1: int | None = None):
        """Raw bits of token_values(s, t0, t1) in the source dtype."""
        kv = self._token_f32(s, t0, t1)
        return (np.ascontiguousarray(to_raw(kv[:, 0], self.src_dtype)),
                np.ascontiguousarray(to_raw(kv[:, 1], self.src_dtype)))

    def query_values(self) -> np.ndarray:
        rng = np.random.default_rng([self.seed, 103, self.layer])
        q = rng.standard_normal((self.num_rows, self.num_heads, self.head_dim), dtype=np.float32)
        return raw_to_f32(to_raw(q, self.q_dtype), self.q_dtype)

    def query_raw(self) -> np.ndarray:
        return to_raw(self.query_values(), self.q_dtype)

    # -- slots -----------------------------------------------------------------------------
    def slots(self, s: int, t0: int, t1: int) -> np.ndarray:
        """Pool slot (physical_block * block_size + offset) of positions [t0, t1) of seq s."""
        t = np.arange(t0, t1, dtype=np.int64)
        blocks = self.block_tables[s, t // self.block_size].astype(np.int64)
        return blocks * self.block_size + t % self.block_size

    def history_chunks(self, seqs=None, max_tokens: int = 1 << 16):
        """(key_raw, value_raw, slots) pieces covering every stored position that precedes
        this step's new rows, each shared-prefix position written once."""
        seqs = range(self.num_seqs) if seqs is None else seqs
        prefix_done = False
        sharing = set(self.sharing.tolist())
        for s in seqs:
            hist = int(self.context_lens[s]) - int(self.query_lens[s])
            t0 = 0
            if s in sharing:
                if prefix_done:
                    t0 = min(self.shared_prefix_len, hist)
                prefix_done = True
            for a in range(t0, hist, max_tokens):
                b = min(hist, a + max_tokens)
                k, v = self.token_raw(s, a, b)
                yield k, v, self.slots(s, a, b)

    def new_tokens(self, seqs=None):
        """(key_raw, value_raw, slots) of this step's new positions, concatenated over seqs."""
        seqs = range(self.num_seqs) if seqs is None else seqs
        ks, vs, ss = [], [], []
        for s in seqs:
            ctx, ql = int(self.context_lens[s]), int(self.query_lens[s])
            k, v = self.token_raw(s, ctx - ql, ctx)
            ks.append(k)
            vs.append(v)
            ss.append(self.slots(s, ctx - ql, ctx))
        return (np.ascontiguousarray(np.concatenate(ks)), np.ascontiguousarray(np.concatenate(vs)),
                np.concatenate(ss).astype(np.int64))

    def empty_pool(self, poison: bool = True) -> tuple[np.ndarray, np.ndarray]:
        """Host K and V pools (raw bits), filled with NaN so that unread slots are visible."""
        dt = RAW_NP[self.cache_dtype]
        fill = POISON[self.cache_dtype] if poison else dt(0)
        return np.full(self.pool_elems, fill, dtype=dt), np.full(self.pool_elems, fill, dtype=dt)

    def used_blocks(self) -> np.ndarray:
        ids = [self.block_tables[s, :(int(c) + self.block_size - 1) // self.block_size]
               for s, c in enumerate(self.context_lens)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)

    # -- algorithmic bytes -------------------------------------------------------------------
    def kv_read_bytes(self, unique: bool = True) -> int:
        """K+V bytes attention must read: every visible position once per kv head; with
        unique=True a physical block shared by several sequences counts once."""
        e = ELEM_BYTES[self.cache_dtype]
        per_tok = self.num_kv_heads * self.head_dim * 2 * e
        if not unique or len(self.sharing) <= 1:
            return int(self.context_lens.astype(np.int64).sum()) * per_tok
        dup = (len(self.sharing) - 1) * self.shared_prefix_len
        return (int(self.context_lens.astype(np.int64).sum()) - dup) * per_tok

    def decode_bytes(self, unique: bool = True) -> int:
        """Algorithmic bytes of one attention call: KV + query + output + tables + lengths
        (+ the scales of a quantised cache)."""
        eq = ELEM_BYTES[self.q_dtype]
        nblk = (self.context_lens.astype(np.int64) + self.block_size - 1) // self.block_size
        b = self.kv_read_bytes(unique)
        b += self.num_rows * self.num_heads * self.head_dim * 2 * eq
        b += int(nblk.sum()) * 4 + self.num_seqs * 4
        if self.cache_dtype in QUANT_DTYPES:
            b += 2 * 4 * self.num_kv_heads
        return int(b)

    def shared_block_counts(self) -> np.ndarray:
        """int32 [S]: the leading blocks of each sequence whose refcount is above 1 -- the blocks
        it shares with other sequences, as a prefix cache's host side knows them (the hint that
        pa_paged_attention_decode_shared takes)."""
        B = self.block_size
        counts = np.zeros(self.num_seqs, np.int32)
        if self.refcount.size == 0:
            return counts
        for s in range(self.num_seqs):
            nb = -(-int(self.context_lens[s]) // B)
            row = self.block_tables[s, :nb]
            shared = self.refcount[row] > 1
            counts[s] = nb if shared.all() else int(np.argmin(shared))
        return counts

    def write_bytes(self) -> int:
        """Algorithmic bytes of appending this step's new rows: read K,V rows in the source
        dtype, write them in the cache dtype, read the slot ids."""
        T = self.num_rows
        per = self.num_kv_heads * self.head_dim * 2
        return int(T * per * (ELEM_BYTES[self.src_dtype] + ELEM_BYTES[self.cache_dtype]) + 8 * T)


def build_batch(context_lens, *, num_heads, num_kv_heads, head_dim, block_size=16, q_dtype=BF16,
                cache_dtype=BF16, src_dtype=None, seed=0, query_lens=None, shared_prefix_len=0,
                sharing=(), num_blocks=None, pool_slack=0.10, max_blocks_per_seq=None, layer=0,
                name="custom", quant_calibration_tokens=4096, fp8_scale="head") -> PagedBatch:
    ctx = np.asarray(context_lens, dtype=np.int32)
    S = ctx.shape[0]
    ql = np.ones(S, np.int32) if query_lens is None else np.asarray(query_lens, np.int32)
    if np.any(ql > np.maximum(ctx, 0)) or np.any(ql < 0):
        raise ValueError("query_lens must lie in [0, context_len]")
    if src_dtype is None:
        src_dtype = q_dtype if cache_dtype in QUANT_DTYPES else cache_dtype
    B = block_size
    sharing = np.asarray(sorted(set(int(s) for s in sharing)), dtype=np.int64)
    if shared_prefix_len % B:
        raise ValueError("a shared prefix must end on a block boundary")
    nblk = (ctx.astype(np.int64) + B - 1) // B
    pblk = shared_prefix_len // B
    for s in sharing:
        if ctx[s] - ql[s] < shared_prefix_len:
            raise ValueError("sharing sequence shorter than the prefix")
    unique = int(nblk.sum()) - (max(len(sharing), 1) - 1) * pblk if len(sharing) else int(nblk.sum())
    if num_blocks is None:
        num_blocks = int(math.ceil((1.0 + pool_slack) * unique)) if unique else 1
    rng = np.random.default_rng([seed, 100, layer])
    alloc = BlockAllocator(num_blocks, rng)
    mbps = int(max(nblk.max() if S else 1, 1)) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    tables = np.zeros((S, mbps), dtype=np.int32)
    prefix_ids = alloc.alloc(pblk) if len(sharing) and pblk else []
    first_sharer = True
    for s in range(S):
        own = int(nblk[s])
        ids = []
        if s in set(sharing.tolist()):
            ids = alloc.share(prefix_ids) if not first_sharer else list(prefix_ids)
            first_sharer = False
            own -= pblk
        ids += alloc.alloc(own)
        tables[s, :len(ids)] = ids
    # Entries past a sequence's last block are never read; point them at free (poisoned)
    # blocks so a stray read shows up as NaN instead of an out-of-bounds access.
    free = np.array(alloc.free_list if alloc.num_free else [0], dtype=np.int32)
    for s in range(S):
        n = int(nblk[s])
        if n < mbps:
            tables[s, n:] = rng.choice(free, size=mbps - n)
    batch = PagedBatch(name=name, num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                       block_size=B, q_dtype=q_dtype, src_dtype=src_dtype, cache_dtype=cache_dtype,
                       context_lens=ctx, query_lens=ql, block_tables=tables, num_blocks=num_blocks,
                       seed=seed, layer=layer, shared_prefix_len=shared_prefix_len if len(sharing) else 0,
                       sharing=sharing, refcount=alloc.refcount.copy(), fp8_scale=fp8_scale)
    if cache_dtype in QUANT_DTYPES:
        batch.k_scale, batch.v_scale = quant_calibration_scales(
            num_kv_heads, head_dim, seed, layer, src_dtype, quant_calibration_tokens, cache_dtype, fp8_scale)
    return batch


def quant_calibration_scales(num_kv_heads, head_dim, seed, layer, src_dtype, tokens=4096, cache_dtype=FP8_E4M3,
                             granularity="head"):
    """Scales of a quantised cache for one layer: amax over a seeded calibration batch of K
    (resp. V) rows drawn like the workload, divided by the format's largest code magnitude
    (448 E4M3, 57344 E5M2, 127 INT8), as float32.
    granularity "head" takes the amax per kv head; "tensor" takes one amax over all heads and
    repeats it per head (a per-tensor scale)."""
    if granularity not in ("head", "tensor"):
        raise ValueError("scale granularity must be 'head' or 'tensor'")
    rng = np.random.default_rng([seed, 104, layer])
    cal = rng.standard_normal((tokens, 2, num_kv_heads, head_dim), dtype=np.float32)
    cal = raw_to_f32(to_raw(cal, src_dtype), src_dtype)
    amax = np.abs(cal).max(axis=(0, 3))  # [2][Hkv]
    if granularity == "tensor":
        amax = np.repeat(amax.max(axis=1, keepdims=True), num_kv_heads, axis=1)
    sc = (amax.astype(np.float64) / QUANT_MAX[cache_dtype]).astype(np.float32)
    return np.ascontiguousarray(sc[0]), np.ascontiguousarray(sc[1])


# ---- the five workloads ------------------------------------------------------------------

def tiny_fp32(seed=0, block_size=16) -> PagedBatch:
    """4 sequences, contexts {17, 33, 64, 100} (the new token included), 8 query / 2 KV
    heads, head dim 64, 16-token blocks, fp32, a 32-block pool handed out by a seeded
    permutation."""
    return build_batch([17, 33, 64, 100], num_heads=8, num_kv_heads=2, head_dim=64, block_size=block_size,
                       q_dtype=F32, cache_dtype=F32, seed=seed, num_blocks=32, name="tiny_fp32")


def llama3_8b_decode(seed=0, num_seqs=64, ctx_range=(512, 4096), layer=0, block_size=16) -> PagedBatch:
    """Llama-3-8B-shaped decode layer: 64 sequences, contexts uniform in [512, 4096],
    32 query / 8 KV heads, head dim 128, bf16, 16-token blocks, pool = used blocks + 10%."""
    rng = np.random.default_rng([seed, 100, 9999])
    ctx = rng.integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs)
    return build_batch(ctx, num_heads=32, num_kv_heads=8, head_dim=128, block_size=block_size, q_dtype=BF16,
                       cache_dtype=BF16, seed=seed, layer=layer, name="llama3_8b_decode")


def long_context(seed=0, num_seqs=16, ctx=8192, layer=0, block_size=16) -> PagedBatch:
    """Long-context split-K decode: 16 sequences of 8192 tokens (512 scattered blocks
    each), 32 query / 8 KV heads, head dim 128, bf16; one layer of the 32."""
    return build_batch([ctx] * num_seqs, num_heads=32, num_kv_heads=8, head_dim=128, block_size=block_size,
                       q_dtype=BF16, cache_dtype=BF16, seed=seed, layer=layer, name="long_context")


def mixed_continuous_batch(seed=0, num_seqs=256, num_sharing=64, prefix=2048,
                           median=1024, sigma=1.0, clip=(32, 32768), layer=0, block_size=16) -> PagedBatch:
    """Continuous-batching decode step: 256 sequences with log-normal contexts (median
    1024, sigma 1.0, clipped to [32, 32768]); 64 of them share a 2048-token prefix through
    the same leading physical blocks (refcount 64) and extend it by their own log-normal
    sample (clipped again)."""
    rng = np.random.default_rng([seed, 100, 9998])
    own = np.clip(np.round(rng.lognormal(math.log(median), sigma, size=num_seqs)), clip[0], clip[1])
    sharing = np.sort(rng.choice(num_seqs, size=num_sharing, replace=False))
    ctx = own.astype(np.int64)
    ctx[sharing] = np.minimum(prefix + ctx[sharing], clip[1])
    return build_batch(ctx, num_heads=32, num_kv_heads=8, head_dim=128, block_size=block_size, q_dtype=BF16,
                       cache_dtype=BF16, seed=seed, layer=layer, shared_prefix_len=prefix,
                       sharing=sharing, name="mixed_continuous_batch")


def fp8_chunked_prefill(seed=0, num_decode=128, chunk=512, chunk_ctx=8192,
                        decode_range=(256, 8192), layer=0, cache_dtype=FP8_E4M3, fp8_scale="head",
                        name="fp8_chunked_prefill", block_size=16) -> PagedBatch:
    """Quantised KV cache (fp8 E4M3 unless cache_dtype says E5M2 or INT8) with per-(layer, kv head)
    scales (fp8_scale="tensor": one scale per layer, repeated per head): sequence 0 is a 512-row prefill
    chunk that is the last 512 positions of an 8192-token context; sequences 1..128 are
    decode rows with contexts uniform in [256, 8192].  32 query / 8 KV heads, head dim 128,
    bf16 queries and K/V rows."""
    rng = np.random.default_rng([seed, 100, 9997])
    dec = rng.integers(decode_range[0], decode_range[1] + 1, size=num_decode)
    ctx = np.concatenate([[chunk_ctx], dec])
    ql = np.concatenate([[chunk], np.ones(num_decode, np.int64)])
    return build_batch(ctx, num_heads=32, num_kv_heads=8, head_dim=128, block_size=block_size, q_dtype=BF16,
                       cache_dtype=cache_dtype, src_dtype=BF16, seed=seed, layer=layer, query_lens=ql,
                       name=name, fp8_scale=fp8_scale)


WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "llama3_8b_decode": llama3_8b_decode,
    "long_context": long_context,
    "mixed_continuous_batch": mixed_continuous_batch,
    "fp8_chunked_prefill": fp8_chunked_prefill,
    # the same step over an E5M2 cache with one scale per layer (per-tensor)
    "fp8_e5m2_chunked_prefill": lambda seed=0, layer=0, block_size=16: fp8_chunked_prefill(
        seed=seed, layer=layer, cache_dtype=FP8_E5M2, fp8_scale="tensor", name="fp8_e5m2_chunked_prefill",
        block_size=block_size),
    # the same step over an INT8 cache with per-head scales (page 4, section 4.5, step 4)
    "int8_chunked_prefill": lambda seed=0, layer=0, block_size=16: fp8_chunked_prefill(
        seed=seed, layer=layer, cache_dtype=INT8, name="int8_chunked_prefill", block_size=block_size),
}
