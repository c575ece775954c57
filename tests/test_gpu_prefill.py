"""GPU parity: chunked-prefill PagedAttention through the C ABI vs the CPU oracle.

Each sequence's last q_len positions are this step's rows: their K/V are appended by the GPU
(checked bit-exact against the oracle's append), then every row attends causally over the
paged context.  Sizes span several 64-key iterations, several 128-row workgroups, partial
MFMA tiles, ragged last blocks and decode rows (q_len 1) mixed with chunks.  The bar is the
same as decode: 2e-2 absolute for a bf16 cache, 6e-2 for fp8, against the oracle run on the
same cache bytes.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_461_amd import workloads as W
from tests.gpu_util import DeviceBatch, assert_close, oracle_attention, oracle_pool, out_to_f64, to_dev, to_host_raw

pytestmark = pytest.mark.gpu


def prefill_and_compare(batch, partition_size=0, poison=True):
    kp_h, vp_h = oracle_pool(batch, include_new=False, poison=poison)
    db = DeviceBatch(batch)
    kp, vp = to_dev(kp_h, batch.cache_dtype), to_dev(vp_h, batch.cache_dtype)
    db.write_new_tokens(kp, vp)
    k, v, slots = batch.new_tokens()
    oracle.kv_cache_write(k, v, batch.src_dtype, kp_h, vp_h, batch.cache_dtype, slots, batch.num_kv_heads,
                          batch.head_dim, batch.block_size, batch.k_scale, batch.v_scale)
    assert np.array_equal(to_host_raw(kp).view(np.uint8), kp_h.view(np.uint8)), "K pool differs after append"
    assert np.array_equal(to_host_raw(vp).view(np.uint8), vp_h.view(np.uint8)), "V pool differs after append"
    out = db.prefill(kp, vp, partition_size=partition_size)
    got = out_to_f64(out)
    ref = oracle_attention(batch, kp_h, vp_h)
    assert_close(batch, got, ref)
    return db, kp, vp, out, kp_h, vp_h


# (context length, rows) per sequence: whole prompts from position 0, chunks at the end of a
# longer context, decode rows, an exact 64-key multiple and ragged tails.
MIXED = ([300, 1, 64, 700, 129, 40, 1000], [37, 1, 64, 200, 1, 40, 130])


@pytest.mark.parametrize("cache", [W.BF16, W.FP8_E4M3, W.FP8_E5M2, W.INT8])
@pytest.mark.parametrize("gqa", [1, 2, 4, 8])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_mixed_chunks(cache, gqa, head_dim):
    hkv = 2 if gqa < 8 else 1
    b = W.build_batch(MIXED[0], num_heads=hkv * gqa, num_kv_heads=hkv, head_dim=head_dim, q_dtype=W.BF16,
                      cache_dtype=cache, seed=100 + 10 * gqa + head_dim, query_lens=MIXED[1])
    prefill_and_compare(b)


@pytest.mark.parametrize("cache", [W.BF16, W.FP8_E4M3, W.INT8])
@pytest.mark.parametrize("P", [0, 24, 64])
def test_block_size_8(cache, P):
    """8-token blocks: every 16-token unit of an iteration comes from two blocks (an 8-bit
    cache's V piece of a channel is 8 bytes of each); split ranges of 24 keys start inside a
    unit."""
    b = W.build_batch(MIXED[0], num_heads=16, num_kv_heads=4, head_dim=128, block_size=8, q_dtype=W.BF16,
                      cache_dtype=cache, seed=80 + P, query_lens=MIXED[1])
    prefill_and_compare(b, partition_size=P)


@pytest.mark.parametrize("cache", [W.BF16, W.FP8_E4M3, W.INT8])
@pytest.mark.parametrize("P", [0, 32, 96])
def test_block_size_32(cache, P):
    """32-token blocks: a 64-key iteration spans two blocks (four 16-token units); split
    ranges of 32 / 96 keys start in either half of a block pair."""
    b = W.build_batch(MIXED[0], num_heads=16, num_kv_heads=4, head_dim=128, block_size=32, q_dtype=W.BF16,
                      cache_dtype=cache, seed=320 + P, query_lens=MIXED[1])
    prefill_and_compare(b, partition_size=P)


@pytest.mark.parametrize("P", [16, 48, 64, 256, 1024, 0])
def test_split_k_partition_sweep(P):
    """Fixed key ranges of every size (one block .. no split) give the same rows."""
    b = W.build_batch([900, 2000, 70], num_heads=32, num_kv_heads=8, head_dim=128, q_dtype=W.BF16,
                      cache_dtype=W.FP8_E4M3, seed=11, query_lens=[300, 33, 70])
    prefill_and_compare(b, partition_size=P)


def test_chunk_shaped_like_the_fp8_step():
    """One 512-row chunk ending a 2048-token context, fp8 cache, 32/8 heads, head dim 128:
    the automatic plan splits the keys (16 row blocks x 8 kv heads < 512 workgroups)."""
    b = W.build_batch([2048], num_heads=32, num_kv_heads=8, head_dim=128, q_dtype=W.BF16,
                      cache_dtype=W.FP8_E4M3, seed=5, query_lens=[512])
    prefill_and_compare(b)


def test_rows_equal_decode_rows():
    """Row i of a chunk is the decode of position p_i = ctx - q_len + i over ctx' = p_i + 1
    positions: the GPU prefill and the GPU decode agree within the bf16 bar."""
    b = W.build_batch([600], num_heads=16, num_kv_heads=4, head_dim=128, q_dtype=W.BF16, cache_dtype=W.BF16,
                      seed=8, query_lens=[150])
    db, kp, vp, out, _, _ = prefill_and_compare(b)
    rows = [0, 1, 63, 64, 100, 149]
    pos = [600 - 150 + i for i in rows]
    d = W.build_batch([p + 1 for p in pos], num_heads=16, num_kv_heads=4, head_dim=128, q_dtype=W.BF16,
                      cache_dtype=W.BF16, seed=8, max_blocks_per_seq=b.block_tables.shape[1])
    dd = DeviceBatch(d)
    dd.tables = db.tables[[0] * len(rows)].contiguous()
    dd.query = db.query[rows].contiguous()
    dec = dd.decode(kp, vp)
    assert float((dec.float() - out[rows].float()).abs().max()) <= 2e-2


def test_physical_block_relabelling_is_bit_identical():
    b = W.build_batch([500, 130], num_heads=16, num_kv_heads=4, head_dim=128, q_dtype=W.BF16, cache_dtype=W.BF16,
                      seed=3, query_lens=[200, 130])
    kp_h, vp_h = oracle_pool(b, include_new=True)
    db = DeviceBatch(b)
    base = db.prefill(to_dev(kp_h, b.cache_dtype), to_dev(vp_h, b.cache_dtype))
    perm = np.random.default_rng(6).permutation(b.num_blocks)
    tile = b.num_kv_heads * b.block_size * b.head_dim
    kp2, vp2 = np.empty_like(kp_h), np.empty_like(vp_h)
    kp2.reshape(-1, tile)[perm] = kp_h.reshape(-1, tile)
    vp2.reshape(-1, tile)[perm] = vp_h.reshape(-1, tile)
    db.tables = torch.from_numpy(perm[b.block_tables].astype(np.int32)).cuda()
    again = db.prefill(to_dev(kp2, b.cache_dtype), to_dev(vp2, b.cache_dtype))
    assert torch.equal(base.view(torch.int16), again.view(torch.int16))


@pytest.mark.parametrize("cache", [W.BF16, W.FP8_E4M3, W.FP8_E5M2, W.INT8])
def test_unused_slots_never_read(cache):
    """NaN in every unwritten slot, free block and stale table entry: same bits as zeros."""
    b = W.build_batch([7, 17, 300], num_heads=8, num_kv_heads=2, head_dim=128, q_dtype=W.BF16, cache_dtype=cache,
                      seed=9, max_blocks_per_seq=40, query_lens=[7, 3, 90])
    outs = []
    for poison in (True, False):
        kp_h, vp_h = oracle_pool(b, include_new=True, poison=poison)
        db = DeviceBatch(b)
        outs.append(db.prefill(to_dev(kp_h, b.cache_dtype), to_dev(vp_h, b.cache_dtype), partition_size=64))
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_single_position_is_its_value():
    """A one-position prompt sees only itself: the output is that token's V exactly."""
    b = W.build_batch([1, 1], num_heads=8, num_kv_heads=2, head_dim=128, q_dtype=W.BF16, cache_dtype=W.BF16,
                      seed=2, query_lens=[1, 1])
    _, _, _, out, _, _ = prefill_and_compare(b)
    got = to_host_raw(out)
    for s in range(2):
        _, v0 = b.token_raw(s, 0, 1)
        for h in range(8):
            assert np.array_equal(got[s, h], v0[0, h // 4])


def test_empty_sequences_and_rows_are_skipped():
    """q_len 0 sequences own no rows; the others are unaffected."""
    b = W.build_batch([50, 80, 30], num_heads=8, num_kv_heads=2, head_dim=64, q_dtype=W.BF16, cache_dtype=W.BF16,
                      seed=4, query_lens=[0, 20, 0])
    prefill_and_compare(b)


def test_rows_before_the_context_start_are_zero():
    """q_len above the context length (outside the contract): rows whose position would be
    negative get zeros, the others attend over the positions that exist (as the oracle)."""
    b = W.build_batch([8], num_heads=8, num_kv_heads=2, head_dim=64, q_dtype=W.BF16, cache_dtype=W.BF16,
                      seed=12, query_lens=[8])
    kp_h, vp_h = oracle_pool(b, include_new=True)
    db = DeviceBatch(b)
    db.ctx = torch.tensor([5], dtype=torch.int32, device="cuda")
    out = db.prefill(to_dev(kp_h, b.cache_dtype), to_dev(vp_h, b.cache_dtype))
    ref = oracle.paged_attention(b.query_raw(), b.q_dtype, kp_h, vp_h, b.cache_dtype, b.block_tables,
                                 np.array([5], dtype=np.int32), b.num_heads, b.num_kv_heads, b.head_dim,
                                 b.block_size, b.scale, cu_query_lens=b.cu_query_lens)
    got = out_to_f64(out)
    assert np.all(got[:3] == 0.0)
    assert_close(b, got, ref)
