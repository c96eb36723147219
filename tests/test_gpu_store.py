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


def _check_bf16_slab(sc, k, v, starts, counts, table, hkv, dropped=()):
    """Every stored row bit for bit where its page walk leads (rows of `dropped`
    (b, i) pairs nowhere), and the NaN sentinel in every other slot."""
    ks = host_bits(sc.cache.slabs[0][0])
    vs = host_bits(sc.cache.slabs[0][1]) if v is not None else None
    cu = np.concatenate([[0], np.cumsum(counts)])
    written = np.zeros((sc.pool.num_pages, 16), dtype=bool)
    for b in range(len(counts)):
        for i in range(counts[b]):
            if (b, i) in dropped:
                continue
            pos = starts[b] + i
            written[table[b, pos // 16], pos % 16] = True
            for h in range(hkv):
                assert np.array_equal(page_walk_k(ks, table, b, pos, h), k[cu[b] + i, h])
                if vs is not None:
                    assert np.array_equal(page_walk_v(vs, table, b, pos, h), v[cu[b] + i, h])
    assert (ks.transpose(0, 2, 1, 3)[~written] == 0x7FC0).all()
    if vs is not None:
        assert (vs.transpose(0, 3, 1, 2)[~written] == 0x7FC0).all()


@pytest.mark.parametrize("case", ["whole_pages", "ragged", "one_token_each", "k_eq_v"])
@pytest.mark.parametrize("d,hkv", [(256, 1), (512, 2)])
def test_store_bf16_paths_bit_exact(case, d, hkv):
    """Chunks of four or more tokens per sequence on average go through the
    kernel that writes whole V pages (32-byte dim rows when 16 tokens fill a
    page, single values otherwise); fewer go through the row kernel.  Both
    are bit-exact: whole pages only (page-aligned starts and counts), ragged
    starts and ends with blocks of 16 tokens that cross sequences, one token
    per sequence, and a K=V layer (keys only)."""
    need_gpu()
    if case == "whole_pages":
        caps, starts, counts = [64, 32, 96, 16], [0, 16, 32, 0], [64, 16, 48, 16]
    elif case == "one_token_each":
        caps = [1, 17, 33, 16, 5, 200, 31, 2]
        starts, counts = [c - 1 for c in caps], [1] * 8
    else:
        caps, starts, counts = [40, 7, 100, 33, 19], [3, 0, 21, 32, 2], [37, 7, 79, 1, 17]
    spec = LayerSpec("full", d, hkv, hkv, 0, k_eq_v=(case == "k_eq_v"))
    sc = Scenario([spec], None, caps, seed=61 + d + len(case))
    k, v = sc.store(0, starts, counts)
    torch.cuda.synchronize()
    _check_bf16_slab(sc, k, None if case == "k_eq_v" else v, starts, counts, sc.pool.page_table, hkv)


@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("chunk", [True, False])
def test_store_drops_rows_without_a_page(d, chunk):
    """A position whose page-table entry lies outside the pool, or whose page
    index lies past the table's width, is dropped; every other row lands, in
    both store kernels."""
    need_gpu()
    caps = [48, 40, 64]
    spec = LayerSpec("full", d, 1, 1, 0)
    sc = Scenario([spec], None, caps, seed=73 + d)
    table = sc.pool.page_table.copy()
    table[0, 1] = sc.pool.num_pages + 3          # page 1 of sequence 0: outside the pool
    table[2, 2] = -1                             # page 2 of sequence 2: no page
    sc.cache.set_page_table(table)
    width = table.shape[1]
    if chunk:
        starts, counts = [0, 8, 16], [48, 32, 48]
    else:
        starts, counts = [20, 39, 40], [1, 1, 1]
    # one more sequence: the last slot of the table's last page, then a row
    # past the table's width
    starts2 = starts + [width * 16 - (1 if chunk else 0)]
    counts2 = counts + [2 if chunk else 1]
    B = len(starts2)
    table4 = np.concatenate([table, np.full((1, width), -1, np.int32)], axis=0)
    table4[3, width - 1] = sc.pool.spare_pages[0]   # the last page in the table: a spare one
    sc.cache.set_page_table(table4)
    total = sum(counts2)
    k = normal_bf16(sc.rng, (total, 1, d))
    v = normal_bf16(sc.rng, (total, 1, d))
    cu = np.concatenate([[0], np.cumsum(counts2)]).astype(np.int32)
    sc.cache.store(0, i32(cu), i32(starts2), dev_bits(k), dev_bits(v))
    torch.cuda.synchronize()
    dropped = set()
    for b in range(B):
        for i in range(counts2[b]):
            pos = starts2[b] + i
            if pos // 16 >= width or not (0 <= table4[b, pos // 16] < sc.pool.num_pages):
                dropped.add((b, i))
    assert dropped                                  # the case drops something
    assert len(dropped) < total                     # and stores the rest
    ks, vs = host_bits(sc.cache.slabs[0][0]), host_bits(sc.cache.slabs[0][1])
    written = np.zeros((sc.pool.num_pages, 16), dtype=bool)
    for b in range(B):
        for i in range(counts2[b]):
            if (b, i) in dropped:
                continue
            pos = starts2[b] + i
            page = table4[b, pos // 16]
            written[page, pos % 16] = True
            assert np.array_equal(ks[page, 0, pos % 16], k[cu[b] + i, 0])
            assert np.array_equal(vs[page, 0, :, pos % 16], v[cu[b] + i, 0])
    assert (ks.transpose(0, 2, 1, 3)[~written] == 0x7FC0).all()
    assert (vs.transpose(0, 3, 1, 2)[~written] == 0x7FC0).all()


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


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("case", ["whole_pages", "ragged", "one_token_each", "dropped"])
@pytest.mark.parametrize("d,hkv", [(256, 1), (512, 2)])
def test_store_q8_paths_bit_exact(fmt, case, d, hkv):
    """8-bit chunks (four or more tokens per sequence on average) go through the
    kernel that writes whole V pages (16-byte dim rows when 16 tokens fill a
    page, single codes otherwise), fewer through the row kernel: codes and
    scales equal the oracle's encoding of every row either way, rows without a
    page are dropped, and unwritten slots keep their sentinel."""
    from oracle import fp8_pth
    need_gpu()
    if case == "whole_pages":
        caps, starts, counts = [64, 32, 96, 16], [0, 16, 32, 0], [64, 16, 48, 16]
    elif case == "one_token_each":
        caps = [1, 17, 33, 16, 5, 200, 31, 2]
        starts, counts = [c - 1 for c in caps], [1] * 8
    else:
        caps, starts, counts = [40, 7, 100, 33, 19], [3, 0, 21, 32, 2], [37, 7, 79, 1, 17]
    spec = LayerSpec("full", d, hkv, hkv, 0, kv_dtype=fmt)
    sc = Scenario([spec], None, caps, seed=91 + d + len(case) + len(fmt))
    table = sc.pool.page_table.copy()
    if case == "dropped":
        table[0, 1] = sc.pool.num_pages + 3           # outside the pool
        table[2, 3] = -1                              # no page
        sc.cache.set_page_table(table)
    kc0, vc0 = [t.clone() for t in sc.cache.slabs[0][:2]]
    total = sum(counts)
    k = normal_bf16(sc.rng, (total, hkv, d))
    v = normal_bf16(sc.rng, (total, hkv, d))
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sc.cache.store(0, i32(cu), i32(starts), dev_bits(k), dev_bits(v))
    torch.cuda.synchronize()
    u8 = lambda t: t.cpu().numpy().view(np.uint8)
    kc, vc = u8(sc.cache.slabs[0][0]), u8(sc.cache.slabs[0][1])
    ksc, vsc = sc.cache.slabs[0][2].cpu().numpy(), sc.cache.slabs[0][3].cpu().numpy()
    quant = fp8_pth.quantise_rows if fmt == "fp8" else quantise_rows
    kq, kscale = quant(bf16_to_f32(k))
    vq, vscale = quant(bf16_to_f32(v))
    kq, vq = kq.view(np.uint8), vq.view(np.uint8)
    written = np.zeros((sc.pool.num_pages, 16), dtype=bool)
    stored = 0
    for b in range(len(caps)):
        for i in range(counts[b]):
            pos, t = starts[b] + i, cu[b] + i
            page = table[b, pos // 16]
            if not (0 <= page < sc.pool.num_pages):
                continue
            written[page, pos % 16] = True
            stored += 1
            for h in range(hkv):
                assert np.array_equal(kc[page, h, pos % 16, :], kq[t, h]), (b, i, h)
                assert np.array_equal(vc[page, h, :, pos % 16], vq[t, h]), (b, i, h)
                assert kscale[t, h].tobytes() == ksc[page, h, pos % 16].tobytes()
                assert vscale[t, h].tobytes() == vsc[page, h, pos % 16].tobytes()
    assert stored == total or case == "dropped"
    assert case != "dropped" or 0 < stored < total
    k0, v0 = u8(kc0), u8(vc0)
    assert np.array_equal(kc.transpose(0, 2, 1, 3)[~written], k0.transpose(0, 2, 1, 3)[~written])
    assert np.array_equal(vc.transpose(0, 3, 1, 2)[~written], v0.transpose(0, 3, 1, 2)[~written])
