"""Sliding layers on a window pool with its own page table, the full layers on
a full pool (pegainfer issue #807, Description, first paragraph: the sliding
group releases pages the full group still reads).  Sequences are prefilled in
64-token chunks and then decoded step by step; before every call each pool
reserves what the next queries can see, and every page the window pool gives
back is poisoned with NaN in the sliding slab and soon handed to another
sequence.  Every extend and decode output of all four layers (two owners, and
a shared layer of each kind reading its source's slab through its group's
table) matches the oracle, which keeps every row and knows nothing of pages.
The window pool never holds more than the window's pages plus the chunk's."""

import numpy as np
import pytest
import torch

from full_attention_amd import pakv
from oracle import LogicalCache
from workloads import LayerSpec, normal_bf16

from gpu_helpers import assert_close, dev_bits, host_bits, i32, need_gpu

pytestmark = pytest.mark.gpu

W = 48
CHUNK = 64


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_window_pool_prefill_then_decode(fmt):
    need_gpu()
    from full_attention_amd.cache import PagedKVCache
    specs = [LayerSpec("sliding", 256, 8, 1, W, kv_dtype=fmt), LayerSpec("full", 512, 8, 1, 0, kv_dtype=fmt),
             LayerSpec("sliding", 256, 8, 1, W, kv_dtype=fmt), LayerSpec("full", 512, 8, 1, 0, kv_dtype=fmt)]
    first_shared = 2
    prefill = [150, 97, 64]
    steps = 40
    B = len(prefill)
    max_len = max(prefill) + steps
    max_pages = (max_len + 15) // 16
    per_seq_window = (W - 1 + CHUNK + 15) // 16 + 1          # the most a sequence can hold at once
    n_window = B * per_seq_window
    n_full = B * max_pages
    wpool = pakv.PagePool(n_window, B, max_pages, W)
    fpool = pakv.PagePool(n_full, B, max_pages, 0)
    cache = PagedKVCache(specs, first_shared, {"sliding": n_window, "full": n_full})
    oracle = LogicalCache([s.as_dict() for s in specs], first_shared, B)
    rng = np.random.default_rng(5 if fmt == "bf16" else 6)
    poisoned = 0

    def reserve(b, first_query, end):
        nonlocal poisoned
        fpool.reserve(b, first_query, end)
        wpool.reserve(b, first_query, end)
        for p in wpool.released():
            for t in cache.slab_of(0)[:2]:
                t[p].fill_(0x7FC0 if fmt == "bf16" else -128)        # poison what was given back
            if fmt != "bf16":
                for t in cache.slab_of(0)[2:]:
                    t[p].fill_(float("nan"))
            poisoned += 1

    def upload():
        cache.set_page_table(wpool.table(), "sliding")
        cache.set_page_table(fpool.table(), "full")
        assert wpool.free_pages() >= 0

    def store_all(starts, counts):
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        for layer in (0, 1):
            s = specs[layer]
            k = normal_bf16(rng, (int(cu[-1]), s.num_kv_heads, s.head_dim))
            v = normal_bf16(rng, (int(cu[-1]), s.num_kv_heads, s.head_dim))
            cache.store(layer, i32(cu), i32(starts), dev_bits(k), dev_bits(v))
            for b in range(B):
                if counts[b]:
                    oracle.store(layer, b, int(starts[b]), k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]])

    # prefill, chunk by chunk, the sequences interleaved
    done = [0] * B
    while any(d < p for d, p in zip(done, prefill)):
        counts = [min(CHUNK, p - d) for d, p in zip(done, prefill)]
        for b in range(B):
            if counts[b]:
                reserve(b, done[b], done[b] + counts[b])
        upload()
        store_all(done, counts)
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        max_kv = max(d + c for d, c in zip(done, counts))
        for layer in range(4):
            s = specs[layer]
            q = normal_bf16(rng, (int(cu[-1]), s.num_q_heads, s.head_dim))
            out = host_bits(cache.extend(layer, i32(cu), i32(done), dev_bits(q), max(counts), max_kv))
            torch.cuda.synchronize()
            for b in range(B):
                if counts[b]:
                    ref = oracle.extend(layer, b, q[cu[b]:cu[b + 1]], done[b])
                    assert_close(out[cu[b]:cu[b + 1]], ref, f"{fmt} prefill layer {layer} seq {b} at {done[b]}")
        done = [d + c for d, c in zip(done, counts)]
    # decode steps: the new token is stored, then every layer decodes
    lens = list(prefill)
    for step in range(steps):
        lens = [L + 1 for L in lens]
        for b in range(B):
            reserve(b, lens[b] - 1, lens[b])
        upload()
        store_all([L - 1 for L in lens], [1] * B)
        for layer in range(4):
            s = specs[layer]
            q = normal_bf16(rng, (B, s.num_q_heads, s.head_dim))
            out = host_bits(cache.decode(layer, i32(lens), dev_bits(q), max(lens)))
            torch.cuda.synchronize()
            if step % 8 == 0 or step == steps - 1:
                ref = np.stack([oracle.decode(layer, b, q[b], lens[b]) for b in range(B)])
                assert_close(out, ref, f"{fmt} decode step {step} layer {layer}")
    # a sliding sequence holds its window's pages and no more
    t = wpool.table()
    for b in range(B):
        held = np.nonzero(t[b] >= 0)[0]
        assert held.min() == (lens[b] - W) // 16 and held.max() == (lens[b] - 1) // 16
    assert poisoned > 2 * B
