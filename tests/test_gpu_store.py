"""paged_kv_store on the GPU: bit-exact against the draws (bf16) and against the
oracle's int8 encoding, through an independent host page walk; pages no
sequence owns and slots nobody wrote keep their sentinel; a shared layer's store
changes nothing (FreeToken PR #898, description: store_kv returns early for a
shared layer)."""

import numpy as np
import pytest
import torch

from oracle import quantise_rows
from workloads import LayerSpec, bf16_to_f32, normal_bf16

from gpu_helpers import Scenario, dev_bits, host_bits, i32, need_gpu, page_walk_k, page_walk_v

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,hkv", [(256, 1), (512, 1), (256, 8), (512, 2)])
def test_store_bf16_bit_exact(d, hkv):
    need_gpu()
    spec = LayerSpec("full", d, hkv, hkv, 0)
    caps = [1, 15, 16, 17, 100, 33]
    sc = Scenario([spec], None, caps, seed=11 + d + hkv)
    starts = [0, 3, 0, 9, 40, 32]
    counts = [1, 12, 16, 8, 60, 1]
    k, v, = sc.store(0, starts, counts)[:2]
    torch.cuda.synchronize()
    ks, vs = sc.cache.slabs[0][0], sc.cache.slabs[0][1]
    kh, vh = host_bits(ks), host_bits(vs)
    table = sc.pool.page_table
    cu = np.concatenate([[0], np.cumsum(counts)])
    written = np.zeros((sc.pool.num_pages, 16), dtype=bool)
    for b in range(len(caps)):
        for i in range(counts[b]):
            pos = starts[b] + i
            written[table[b, pos // 16], pos % 16] = True
            for h in range(hkv):
                assert np.array_equal(page_walk_k(kh, table, b, pos, h), k[cu[b] + i, h])
                assert np.array_equal(page_walk_v(vh, table, b, pos, h), v[cu[b] + i, h])
    # every slot nobody wrote (spare pages included) still holds the sentinel
    assert (kh.transpose(0, 2, 1, 3)[~written] == 0x7FC0).all()
    assert (vh.transpose(0, 3, 1, 2)[~written] == 0x7FC0).all()


@pytest.mark.parametrize("d", [256, 512])
def test_store_int8_matches_oracle_encoding(d):
    need_gpu()
    spec = LayerSpec("sliding", d, 8, 1, 64, kv_dtype="int8")
    caps = [40, 70]
    sc = Scenario([spec], None, caps, seed=21 + d)
    starts, counts = [0, 5], [40, 65]
    total = sum(counts)
    k = normal_bf16(sc.rng, (total, 1, d))
    v = normal_bf16(sc.rng, (total, 1, d))
    # special rows: all zero, amax exactly 127 and 254, halves that must round to even
    k[0] = 0
    row = np.zeros(d, np.float32); row[:4] = [1.0, -2.0, 0.5, 127.0]
    from workloads import bf16_from_f32
    k[1, 0] = bf16_from_f32(row)
    row = np.zeros(d, np.float32); row[:4] = [1.0, 3.0, 5.0, -254.0]
    v[2, 0] = bf16_from_f32(row)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sc.cache.store(0, i32(cu), i32(starts), dev_bits(k), dev_bits(v))
    torch.cuda.synchronize()
    kc, vc, ksc, vsc = [t.cpu().numpy() for t in sc.cache.slabs[0]]
    kq, kscale = quantise_rows(bf16_to_f32(k))
    vq, vscale = quantise_rows(bf16_to_f32(v))
    table = sc.pool.page_table
    for b in range(2):
        for i in range(counts[b]):
            pos, t = starts[b] + i, cu[b] + i
            page, slot = table[b, pos // 16], pos % 16
            assert np.array_equal(kc[page, 0, slot, :], kq[t, 0])
            assert np.array_equal(vc[page, 0, :, slot], vq[t, 0])
            assert kscale[t, 0].tobytes() == ksc[page, 0, slot].tobytes()
            assert vscale[t, 0].tobytes() == vsc[page, 0, slot].tobytes()
    assert kc[table[0, 0], 0, 1, :4].tolist() == [1, -2, 0, 127]


def test_shared_layer_store_changes_nothing():
    need_gpu()
    specs = [LayerSpec("sliding", 256, 8, 1, 32), LayerSpec("full", 512, 8, 1, 0),
             LayerSpec("sliding", 256, 8, 1, 32), LayerSpec("full", 512, 8, 1, 0)]
    sc = Scenario(specs, 2, [50, 20], seed=31)
    sc.store(0, [0, 0], [50, 20])
    sc.store(1, [0, 0], [50, 20])
    torch.cuda.synchronize()
    before = [t.clone() for l in (0, 1) for t in sc.cache.slabs[l][:2]]
    for layer in (2, 3):
        d = specs[layer].head_dim
        nan_rows = torch.full((70, 1, d), 0x7FC0, dtype=torch.int16, device="cuda")
        sc.cache.store(layer, i32([0, 50, 70]), i32([0, 0]), nan_rows, nan_rows)
    torch.cuda.synchronize()
    after = [t for l in (0, 1) for t in sc.cache.slabs[l][:2]]
    for x, y in zip(before, after):
        assert torch.equal(x, y)
    assert set(sc.cache.slabs) == {0, 1}
