"""GPU: a whole step (append + decode, or append + chunked prefill + decode) captured in a HIP
graph and replayed gives the eager step's bits on every replay, with eager work and host
synchronisation between the replays; the library's launches allocate nothing and record no
memset, so they can sit in a graph.  Small steps are launch-bound, which is what graphs are for."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_461_amd import ops
from paged_kv_cache_461_amd import workloads as W
from tests.gpu_util import (DeviceBatch, assert_close, device_step, oracle_attention, oracle_pool, out_to_f64, to_dev,
                            to_host_raw)

pytestmark = pytest.mark.gpu


def _graph_case(batch):
    kp_h, vp_h = oracle_pool(batch, include_new=False)
    db = DeviceBatch(batch)
    kp, vp = to_dev(kp_h, batch.cache_dtype), to_dev(vp_h, batch.cache_dtype)
    k, v, slots = batch.new_tokens()
    nk, nv = to_dev(k, batch.src_dtype), to_dev(v, batch.src_dtype)  # device inputs made before capture
    ns = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).cuda()

    def step():
        ops.kv_cache_write(nk, nv, kp, vp, ns, num_kv_heads=batch.num_kv_heads, head_dim=batch.head_dim,
                           block_size=batch.block_size, k_scale=db.k_scale, v_scale=db.v_scale)
        return device_step(batch, db, kp, vp)

    eager = step()
    torch.cuda.synchronize()
    want = to_host_raw(eager).view(np.uint8).copy()
    pools = to_host_raw(kp).view(np.uint8).copy(), to_host_raw(vp).view(np.uint8).copy()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            out = step()
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_raw(out).view(np.uint8), want), "replay %d differs from the eager step" % i
        assert np.array_equal(to_host_raw(kp).view(np.uint8), pools[0])
        assert np.array_equal(to_host_raw(vp).view(np.uint8), pools[1])
        del junk
    # and the eager step itself matches the oracle
    oracle.kv_cache_write(k, v, batch.src_dtype, kp_h, vp_h, batch.cache_dtype, slots, batch.num_kv_heads,
                          batch.head_dim, batch.block_size, batch.k_scale, batch.v_scale)
    assert_close(batch, out_to_f64(eager), oracle_attention(batch, kp_h, vp_h))


def test_graph_replay_tiny_fp32():
    """The 4-sequence fp32 configuration: 4 contexts {17, 33, 64, 100}, GQA 4, head dim 64."""
    _graph_case(W.tiny_fp32())


@pytest.mark.parametrize("cache", [W.BF16, W.FP8_E4M3])
def test_graph_replay_mixed_step(cache):
    """A chunk (prefill call with split keys) plus decode rows (decode call with split runs)."""
    b = W.build_batch([900, 40, 333, 1200, 64], num_heads=16, num_kv_heads=4, head_dim=128, q_dtype=W.BF16,
                      cache_dtype=cache, seed=77, query_lens=[130, 1, 1, 1, 1])
    _graph_case(b)
