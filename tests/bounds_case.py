"""Child process of test_gpu_debug_bounds.py, run with PAKV_LIBRARY naming the
PAKV_DEBUG_BOUNDS build: stores, decodes and extends with a clean page table,
then with two bad entries, and prints the library's page-id counters after
each phase as one JSON line.  Bad entries are read as page 0 (decode, extend)
or dropped (store) in every build, so nothing here leaves a slab.

Layers: one full and one sliding (W 32) layer, D 256, Hq 8, Hkv 1; sequences
of 70, 40 and 100 positions.  The bad table has page 1 of sequence 1
(positions 16..31) outside the pool and page 0 of sequence 2 (positions
0..15) set to -1.
"""

import json
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

from full_attention_amd import pakv  # noqa: E402
from full_attention_amd.cache import PagedKVCache  # noqa: E402
from gpu_helpers import dev_bits, i32  # noqa: E402
from workloads import LayerSpec, make_page_pool, normal_bf16  # noqa: E402


def main():
    assert os.path.basename(pakv.LIB_PATH) == "libpakv_bounds.so", pakv.LIB_PATH
    torch.cuda.set_device(0)
    rng = np.random.default_rng(3)
    specs = [LayerSpec("full", 256, 8, 1, 0), LayerSpec("sliding", 256, 8, 1, 32)]
    caps = [70, 40, 100]
    pool = make_page_pool(rng, caps)
    cache = PagedKVCache(specs, None, pool.num_pages)
    cache.set_page_table(pool.page_table)
    res = {}

    def mark(name):
        torch.cuda.synchronize()
        res[name] = list(pakv.debug_bounds_counts())

    def store(layer, starts, counts):
        total = int(sum(counts))
        k = normal_bf16(rng, (total, 1, 256))
        v = normal_bf16(rng, (total, 1, 256))
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        cache.store(layer, i32(cu), i32(starts), dev_bits(k), dev_bits(v))

    def decode(layer, lens):
        q = normal_bf16(rng, (len(lens), 8, 256))
        cache.decode(layer, i32(lens), dev_bits(q), int(max(lens)))

    def extend(layer, prefixes, chunks):
        q = normal_bf16(rng, (int(sum(chunks)), 8, 256))
        cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
        cache.extend(layer, i32(cu), i32(prefixes), dev_bits(q), int(max(chunks)),
                     int(max(p + n for p, n in zip(prefixes, chunks))))

    pakv.debug_bounds_reset()
    mark("reset")
    for layer in (0, 1):
        store(layer, [0, 0, 0], caps)                       # chunk store kernel
    store(0, [c - 1 for c in caps], [1, 1, 1])              # row store kernel (rewrites the last rows)
    mark("clean_store")
    for layer in (0, 1):
        decode(layer, caps)
        extend(layer, [c - 8 for c in caps], [8, 8, 8])
    mark("clean_attend")

    bad = pool.page_table.copy()
    bad[1, 1] = pool.num_pages + 7
    bad[2, 0] = -1
    cache.set_page_table(bad)
    store(0, [0, 16, 0], [10, 16, 4])                       # 20 rows without a page, chunk kernel
    mark("bad_chunk_store")
    store(0, [3, 20, 5], [1, 1, 1])                         # 2 more, row kernel
    mark("bad_row_store")
    decode(0, caps)                                         # full layer: both bad pages visible
    mark("bad_full_decode")
    decode(1, caps)                                         # W 32: only sequence 1's is visible
    mark("bad_sliding_decode")
    extend(0, [0, 32, 90], [0, 8, 10])                      # sequences 1 and 2 read their bad pages
    mark("bad_extend")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
