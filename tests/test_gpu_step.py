"""Decode steps captured per batch-size bucket (pakv_decode_step).

* A small stack (bf16 sliding and full owners, an int8 owner, a K=V owner,
  shared layers) with a bucket ladder: a batch runs in the smallest bucket
  that holds it, its rows match the oracle, the padded rows (kv_len 1, page
  rows -1) write nothing, and replays are bit-identical to the same calls
  made eagerly on the bucket's rows.
* The benchmark's own step at full size (the E2B-like stack, batch 64, 35
  layers: one plan per kind of layer, store-and-decode on the 15 owners,
  planned decode on the 20 shared layers, replayed from a graph), checked
  against the oracle on the longest, shortest and median sequences of every
  layer, new rows included.
"""

import numpy as np
import pytest
import torch

from oracle import attend
from workloads import (DeviceDraws, LayerSpec, bf16_to_f32, e2b_decode_workload, make_page_pool, normal_bf16)

from gpu_helpers import Scenario, assert_close, dev_bits, host_bits, i32, need_gpu

pytestmark = pytest.mark.gpu


def test_step_buckets_match_oracle_and_eager():
    need_gpu()
    # owners of every kind (int8, K=V, bf16 full and sliding), then two
    # layers sharing the last owner of their type (layers 3 and 2)
    specs = [LayerSpec("full", 256, 16, 2, 0, kv_dtype="int8"), LayerSpec("full", 512, 16, 2, 0, k_eq_v=True),
             LayerSpec("sliding", 256, 8, 1, 64), LayerSpec("full", 512, 8, 1, 0),
             LayerSpec("sliding", 256, 8, 1, 64), LayerSpec("full", 512, 8, 1, 0)]
    max_batch = 8
    lens = [300, 65, 1000, 17, 129, 700, 1]              # seven sequences
    caps = lens + [1]
    sc = Scenario(specs, 4, caps, seed=301)
    n = len(specs)
    for layer in range(n):
        sc.store(layer, [0] * len(caps), [max(L - 1, 0) for L in caps])
    rng = np.random.default_rng(4)
    q = [normal_bf16(rng, (max_batch, s.num_q_heads, s.head_dim)) for s in specs]
    kn = [normal_bf16(rng, (max_batch, s.num_kv_heads, s.head_dim)) for s in specs]
    vn = [normal_bf16(rng, (max_batch, s.num_kv_heads, s.head_dim)) for s in specs]
    qd = [dev_bits(x) for x in q]
    knd = [dev_bits(x) for x in kn]
    vnd = [dev_bits(x) for x in vn]
    outs = [torch.zeros_like(x) for x in qd]
    kv = i32(lens + [1])
    table = sc.pool.page_table.copy()
    table[7:] = -1                                        # the padded row holds no page
    sc.cache.set_page_table(table)
    io = [(l, qd[l], outs[l], knd[l], vnd[l]) for l in range(n)]
    step = sc.cache.capture_decode_step(kv, max(lens), io, [2, 4, 8], max_batch=max_batch)
    assert step.bucket(7) == 8 and step.bucket(3) == 4 and step.bucket(1) == 2 and step.bucket(9) == -1
    step.run(7)
    torch.cuda.synchronize()
    for l in range(n):
        for b in range(7):
            sc.oracle.store(l, b, lens[b] - 1, kn[l][b:b + 1], vn[l][b:b + 1])
        ref = np.stack([sc.oracle.decode(l, b, q[l][b], lens[b]) for b in range(7)])
        assert_close(host_bits(outs[l])[:7], ref, f"step layer {l}")
    # the padded row's slot of page 0 was not written: page 0 is unchanged
    # by a replay (the new rows were written once already); replay and compare
    first = [host_bits(o).copy() for o in outs]
    def bits(t):                       # compared as bits: the sentinels are NaN
        return t.view(torch.int32) if t.dtype == torch.float32 else t

    slabs = [[bits(t).clone() for t in sc.cache.slab_of(l) if t is not None] for l in range(n)]
    for o in outs:
        o.zero_()
    step.run(5)        # bucket 8 again
    torch.cuda.synchronize()
    for l in range(n):
        assert np.array_equal(host_bits(outs[l])[:7], first[l][:7]), f"replay layer {l}"
        for a, b in zip(slabs[l], [bits(t) for t in sc.cache.slab_of(l) if t is not None]):
            assert torch.equal(a, b), f"slab of layer {l} changed on replay"
    # bucket 4: rows 0..3 as computed by eager calls on 4 rows
    step.run(3)
    torch.cuda.synchronize()
    kv4 = i32(lens[:4])
    for l in range(n):
        plan = sc.cache.decode_plan(l, kv4, max(lens))
        eager = host_bits(sc.cache.decode(l, kv4, qd[l][:4], max(lens), plan=plan))
        assert np.array_equal(host_bits(outs[l])[:4], eager), f"bucket 4 layer {l}"


def test_bench_step_full_size_matches_oracle():
    """The E2B-like decode step exactly as the benchmark replays it."""
    need_gpu()
    from full_attention_amd.cache import PagedKVCache
    wl = e2b_decode_workload()
    B = wl.num_seqs
    L = np.array(wl.cached_lens, dtype=np.int64)
    kv_len = L + 1
    pool = make_page_pool(np.random.default_rng(wl.seed), kv_len)
    cache = PagedKVCache(wl.layers, wl.first_shared, pool.num_pages)
    cache.set_page_table(pool.page_table)
    draws = DeviceDraws(wl.seed)
    order = np.argsort(L, kind="stable")
    sample = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2])})
    owners = [l for l in range(len(wl.layers)) if cache.sources[l] == l]
    kept = {}
    for l in owners:
        s = wl.layers[l]
        lo = np.maximum(0, kv_len - s.window) if s.window else np.zeros(B, np.int64)
        counts = L - lo
        cu = np.concatenate([[0], np.cumsum(counts)])
        k = draws.bf16((int(cu[-1]), 1, s.head_dim))
        v = draws.bf16((int(cu[-1]), 1, s.head_dim))
        cache.store(l, i32(cu), i32(lo), k, v)
        for b in sample:
            kept[(l, b)] = (np.arange(lo[b], L[b]), bf16_to_f32(host_bits(k[cu[b]:cu[b + 1]])),
                            bf16_to_f32(host_bits(v[cu[b]:cu[b + 1]])))
        del k, v
    q, out, kn, vn = [], [], {}, {}
    for l, s in enumerate(wl.layers):
        q.append(draws.bf16((B, 8, s.head_dim)))
        out.append(torch.empty_like(q[-1]))
        if l in owners:
            kn[l] = draws.bf16((B, 1, s.head_dim))
            vn[l] = draws.bf16((B, 1, s.head_dim))
    kv_t = i32(kv_len)
    io = [(l, q[l], out[l], kn.get(l), vn.get(l)) for l in range(len(wl.layers))]
    step = cache.capture_decode_step(kv_t, int(kv_len.max()), io, [64])
    step.run(B)
    torch.cuda.synchronize()
    for l, s in enumerate(wl.layers):
        src = cache.sources[l]
        got = host_bits(out[l])
        qf = bf16_to_f32(host_bits(q[l])).astype(np.float64)
        for b in sample:
            pos, k, v = kept[(src, b)]
            knew = bf16_to_f32(host_bits(kn[src][b:b + 1]))
            vnew = bf16_to_f32(host_bits(vn[src][b:b + 1]))
            pos = np.concatenate([pos, [L[b]]])
            k = np.concatenate([k, knew]).astype(np.float64)
            v = np.concatenate([v, vnew]).astype(np.float64)
            ref = attend(qf[b:b + 1], np.array([L[b]]), k, v, pos, s.window, s.sm_scale)[0]
            assert_close(got[b], ref, f"bench step layer {l} seq {b} (L {kv_len[b]})", report=(l in (0, 4, 15, 19)))
