"""pakv_paged_attn_decode_noalloc (decode with the library's own static device
workspace) against pakv_paged_attn_decode with a caller workspace: the same
kernels and the same plan, so the outputs must be bit-identical.  Two calls in
a row, the second with fewer sequences and shorter lengths (its arrival
counters and plan reuse the first call's memory), on layers of both head
dims; and the oracle."""

import numpy as np
import pytest
import torch

from workloads import LayerSpec, normal_bf16

from gpu_helpers import Scenario, assert_close, dev_bits, host_bits, i32, need_gpu

pytestmark = pytest.mark.gpu


def _noalloc(cache, layer, kv_lens, q, max_kv_len):
    from full_attention_amd import pakv
    out = torch.empty_like(q)
    pakv.paged_attn_decode_noalloc(cache.map, layer, cache.pages, kv_lens, q, out, q.shape[0], max_kv_len)
    return out


def test_noalloc_decode_equals_workspace_decode_twice():
    need_gpu()
    specs = [LayerSpec("full", 512, 8, 1, 0), LayerSpec("sliding", 256, 16, 2, 64)]
    big = [1, 17, 513, 4097, 9000, 700, 33]
    small = [1, 5, 300]          # within what the first three sequences hold
    sc = Scenario(specs, None, big, seed=211)
    for layer in range(2):
        sc.store(layer, [0] * len(big), big)
    for lens in (big, small):
        B = len(lens)
        kv, maxl = i32(lens), max(lens)
        for layer in range(2):
            s = specs[layer]
            qh = normal_bf16(sc.rng, (B, s.num_q_heads, s.head_dim))
            q = dev_bits(qh)
            ref_ws = host_bits(sc.cache.decode(layer, kv, q, maxl))
            got = host_bits(_noalloc(sc.cache, layer, kv, q, maxl))
            torch.cuda.synchronize()
            assert np.array_equal(got, ref_ws), f"B={B} layer {layer}"
            ref = np.stack([sc.oracle.decode(layer, b, qh[b], L) for b, L in enumerate(lens)])
            assert_close(got, ref, f"noalloc B={B} layer {layer}")
