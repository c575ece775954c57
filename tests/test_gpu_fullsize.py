"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The GPU fills each full-size pool through the library's append (as the benchmark does) and
runs the whole step over the whole batch.  The oracle cannot afford the whole batch, so it
computes sampled rows one by one -- first, last, shortest, longest and seeded random
sequences, prefix sharers, chunk rows at both ends -- from its own compact pool written by
its own append; the GPU pool tiles of those sequences must equal the oracle's bit for bit.
Tolerances as elsewhere: 2e-2 absolute (bf16 cache), 6e-2 absolute (fp8 cache).
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_461_amd import ops
from paged_kv_cache_461_amd import workloads as W
from tests.gpu_util import (DeviceBatch, assert_close, byte_view, device_step, oracle_sampled_rows, out_to_f64,
                            to_dev, to_host_raw)

pytestmark = pytest.mark.gpu


def sample_seqs(batch, k=3, seed=0):
    ctx = batch.context_lens
    dec = [s for s in range(batch.num_seqs) if batch.query_lens[s] == 1]
    pick = {dec[0], dec[-1], dec[int(np.argmin(ctx[dec]))], dec[int(np.argmax(ctx[dec]))]}
    rng = np.random.default_rng(seed)
    pick.update(int(x) for x in rng.choice(dec, size=min(k, len(dec)), replace=False))
    return sorted(pick)


def full_step_and_check(batch, picks, partitions=(0,)):
    db = DeviceBatch(batch)
    kp, vp = db.empty_pools(poison=False)
    db.fill_history(kp, vp)
    db.write_new_tokens(kp, vp)
    ref, used, kp_h, vp_h = oracle_sampled_rows(batch, picks)
    tile = batch.num_kv_heads * batch.block_size * batch.head_dim
    ids = torch.from_numpy(used).cuda()
    for dev_pool, host_pool, name in ((kp, kp_h, "K"), (vp, vp_h, "V")):
        got = to_host_raw(byte_view(dev_pool).view(-1, tile * dev_pool.element_size())[ids]).reshape(-1)
        assert np.array_equal(got.view(np.uint8), host_pool.view(np.uint8)), "%s tiles differ from the oracle" % name
    rows = [int(batch.cu_query_lens[s]) + i for s, i in picks]
    worst = 0.0
    for P in partitions:
        out = device_step(batch, db, kp, vp, partition_size=P)
        got = out_to_f64(out)[rows]
        worst = max(worst, assert_close(batch, got, ref))
    return worst


def test_llama3_8b_decode_full():
    b = W.llama3_8b_decode()
    full_step_and_check(b, [(s, 0) for s in sample_seqs(b)])


def test_long_context_full_partition_sweep():
    """16 x 8192 tokens; automatic split and the 256 / 512 / 1024 partition sweep."""
    b = W.long_context()
    full_step_and_check(b, [(s, 0) for s in (0, 7, 15)], partitions=(0, 256, 512, 1024))


def test_mixed_continuous_batch_full():
    """256 log-normal contexts up to 32768, 64 sharing a 2048-token prefix (same physical blocks),
    decoded with the shared-block hint as the benchmark runs it."""
    b = W.mixed_continuous_batch()
    seqs = set(sample_seqs(b))
    seqs.update(int(s) for s in b.sharing[:2])
    assert b.shared_block_counts().max() == 2048 // b.block_size
    full_step_and_check(b, [(s, 0) for s in sorted(seqs)])


@pytest.mark.parametrize("cache,granularity", [(W.FP8_E4M3, "head"), (W.FP8_E5M2, "tensor")])
def test_fp8_chunked_prefill_full(cache, granularity):
    """512-row chunk ending an 8192-token context (fp8 cache) plus 128 decode rows."""
    b = W.fp8_chunked_prefill(cache_dtype=cache, fp8_scale=granularity)
    picks = [(0, i) for i in (0, 1, 127, 128, 255, 384, 510, 511)]
    picks += [(s, 0) for s in sample_seqs(b)]
    full_step_and_check(b, picks)


def test_llama3_8b_decode_full_fused_append():
    """The fused append + decode call as bench.py times it, at full size."""
    b = W.llama3_8b_decode()
    db = DeviceBatch(b)
    kp, vp = db.empty_pools(poison=False)
    db.fill_history(kp, vp)
    k, v, _ = b.new_tokens()
    shape = (b.num_seqs, b.num_kv_heads, b.head_dim)
    nk, nv = to_dev(k, b.src_dtype).view(shape), to_dev(v, b.src_dtype).view(shape)
    out = torch.empty_like(db.query)
    ws = ops.decode_workspace(b.num_seqs, b.num_heads, b.num_kv_heads, b.head_dim, b.max_context_len, b.block_size)
    ops.paged_attention_decode_append(out, db.query, nk, nv, kp, vp, db.tables, db.ctx,
                                      max_context_len=b.max_context_len, num_kv_heads=b.num_kv_heads, scale=b.scale,
                                      block_size=b.block_size, workspace=ws)
    picks = [(s, 0) for s in sample_seqs(b)]
    ref, used, kp_h, vp_h = oracle_sampled_rows(b, picks)
    tile = b.num_kv_heads * b.block_size * b.head_dim
    ids = torch.from_numpy(used).cuda()
    for dev_pool, host_pool in ((kp, kp_h), (vp, vp_h)):
        got = to_host_raw(dev_pool.view(-1, tile)[ids]).reshape(-1)
        assert np.array_equal(got.view(np.uint8), host_pool.view(np.uint8))
    assert_close(b, out_to_f64(out)[[s for s, _ in picks]], ref)
