"""The sampled-row oracle used by the full-size GPU tests equals the full oracle on batches
small enough for both: compact relabelled pool, chunk rows as decode rows of their position,
shared prefixes and fp8 scales included (CPU only)."""
import numpy as np

from paged_kv_cache_461_amd import workloads as W
from tests.gpu_util import oracle_attention, oracle_pool, oracle_sampled_rows


def check(batch, picks):
    kp, vp = oracle_pool(batch, include_new=True)
    full = oracle_attention(batch, kp, vp)
    ref, used, _, _ = oracle_sampled_rows(batch, picks)
    rows = [int(batch.cu_query_lens[s]) + i for s, i in picks]
    assert np.array_equal(ref, full[rows])
    assert len(used) <= batch.num_blocks


def test_sampled_decode_rows():
    b = W.build_batch([5, 40, 300, 17], num_heads=8, num_kv_heads=2, head_dim=64, q_dtype=W.BF16,
                      cache_dtype=W.BF16, seed=1)
    check(b, [(0, 0), (2, 0), (3, 0)])


def test_sampled_chunk_rows_fp8():
    b = W.build_batch([200, 64, 90], num_heads=8, num_kv_heads=2, head_dim=128, q_dtype=W.BF16,
                      cache_dtype=W.FP8_E4M3, seed=2, query_lens=[50, 1, 90])
    check(b, [(0, 0), (0, 49), (0, 17), (1, 0), (2, 0), (2, 89)])


def test_sampled_rows_with_shared_prefix():
    b = W.build_batch([40, 70, 33, 100], num_heads=4, num_kv_heads=1, head_dim=64, q_dtype=W.BF16,
                      cache_dtype=W.BF16, seed=3, shared_prefix_len=32, sharing=[0, 1, 3])
    check(b, [(0, 0), (1, 0), (2, 0), (3, 0)])
