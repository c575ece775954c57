"""pa_paged_attention_decode_noalloc: the decode that allocates nothing (its split-K partial
results live in the library's static per-GPU scratch array) gives the same output bits as
pa_paged_attention_decode with a caller workspace, on two calls in a row -- the second with a
smaller batch, so it runs over what the first left in the scratch -- and both are within the
bf16 / fp8 bar of the oracle."""
import numpy as np
import pytest
import torch

from paged_kv_cache_461_amd import ops
from paged_kv_cache_461_amd import workloads as W
from tests.gpu_util import DeviceBatch, assert_close, oracle_attention, oracle_pool, out_to_f64, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(db, kp, vp, partition_size):
    b = db.b
    out = torch.full_like(db.query, float("nan"))
    ops.paged_attention_decode_noalloc(out, db.query, kp, vp, db.tables, db.ctx, max_context_len=b.max_context_len,
                                       num_kv_heads=b.num_kv_heads, scale=b.scale, block_size=b.block_size,
                                       k_scale=db.k_scale, v_scale=db.v_scale, partition_size=partition_size)
    return out


CASES = [
    # (cache dtype, contexts of the first call, of the second (smaller) call, partition size of each)
    (W.BF16, dict(n=48, lo=1, hi=3000, seed=3), dict(n=9, lo=1, hi=700, seed=4), (0, 0)),
    (W.BF16, dict(n=40, lo=200, hi=2500, seed=5), dict(n=12, lo=17, hi=900, seed=6), (256, 0)),
    (W.FP8_E4M3, dict(n=33, lo=100, hi=4000, seed=7), dict(n=5, lo=1, hi=300, seed=8), (0, 64)),
]


@pytest.mark.parametrize("cache,first,second,parts", CASES)
def test_noalloc_matches_workspace_decode_twice(cache, first, second, parts):
    print("noalloc case: cache %d first %s second %s partitions %s" % (cache, first, second, parts), flush=True)
    for spec, P in ((first, parts[0]), (second, parts[1])):
        rng = np.random.default_rng([spec["seed"], 77])
        ctx = rng.integers(spec["lo"], spec["hi"] + 1, size=spec["n"])
        b = W.build_batch(ctx, num_heads=32, num_kv_heads=8, head_dim=128, q_dtype=W.BF16, cache_dtype=cache,
                          seed=spec["seed"])
        kp_h, vp_h = oracle_pool(b, include_new=True)
        db = DeviceBatch(b)
        kp, vp = to_dev(kp_h, b.cache_dtype), to_dev(vp_h, b.cache_dtype)
        want = db.decode(kp, vp, partition_size=P)
        got = _noalloc(db, kp, vp, P)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "no-alloc output differs from the " \
                                                                           "workspace call"
        assert_close(b, out_to_f64(got), oracle_attention(b, kp_h, vp_h))


def test_noalloc_rejects_oversized_request_without_launch():
    b = W.build_batch([16] * 4, num_heads=8, num_kv_heads=2, head_dim=64, q_dtype=W.BF16, cache_dtype=W.BF16)
    db = DeviceBatch(b)
    kp, vp = db.empty_pools()
    out = torch.empty_like(db.query)
    # 16-token partitions over 4 sequences of up to 2^21 tokens: far more split-K pieces than the
    # scratch holds (the table bound is a host argument only; nothing is launched)
    big = 1 << 21
    tables = torch.zeros((4, big // 16), dtype=torch.int32, device="cuda")
    with pytest.raises(ops.PagedAttnError) as ei:
        ops.paged_attention_decode_noalloc(out, db.query, kp, vp, tables, db.ctx, max_context_len=big, num_kv_heads=2,
                                           scale=b.scale, block_size=16, partition_size=16)
    assert ei.value.status == ops.PA_ERR_WORKSPACE
