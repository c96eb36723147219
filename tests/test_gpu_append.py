"""paged_attn_decode_append (store this step's row, then decode, in one launch)
against the two calls it replaces: the outputs and every byte of the slab must
be identical to pakv_paged_kv_store at position kv_len - 1 followed by the
planned decode, for the slot positions a page can give the new token (0, 15,
and in between), one-chunk units, runs that cross units, sliding windows and
several KV heads; and against the oracle directly.  Slabs start filled with NaN,
so a slot the fused call failed to fill would show."""

import numpy as np
import pytest
import torch

from workloads import LayerSpec, normal_bf16

from gpu_helpers import Scenario, assert_close, dev_bits, host_bits, i32, need_gpu

pytestmark = pytest.mark.gpu


def _pair(specs, first_shared, lens, seed):
    """Two identical scenarios (same draws), every layer's rows [0, L - 1) stored."""
    scs = [Scenario(specs, first_shared, lens, seed=seed) for _ in range(2)]
    for sc in scs:
        for layer in range(len(specs)):
            sc.store(layer, [0] * len(lens), [L - 1 for L in lens])
    return scs


def _slab_bits(sc, layer):
    k, v, _, _ = sc.cache.slab_of(layer)
    return host_bits(k), host_bits(v)


def _new_rows(rng, spec, B):
    k = normal_bf16(rng, (B, spec.num_kv_heads, spec.head_dim))
    v = normal_bf16(rng, (B, spec.num_kv_heads, spec.head_dim))
    return k, v


LENS = [1, 16, 17, 2, 15, 33, 100, 513, 530, 1000, 4097]


@pytest.mark.parametrize("d,hq,hkv,window", [(256, 8, 1, 512), (512, 8, 1, 0), (256, 16, 2, 32), (512, 16, 8, 0),
                                             (256, 4, 4, 7), (512, 16, 1, 1)])
def test_append_matches_store_then_decode(d, hq, hkv, window):
    need_gpu()
    kind = "sliding" if window else "full"
    spec = LayerSpec(kind, d, hq, hkv, window)
    a, b = _pair([spec], None, LENS, seed=71 + d + hq + window)
    rng = np.random.default_rng(5)
    kn, vn = _new_rows(rng, spec, len(LENS))
    q = normal_bf16(rng, (len(LENS), hq, d))
    kv, maxl = i32(LENS), max(LENS)
    # two calls
    a.cache.store(0, i32(np.arange(len(LENS) + 1)), i32([L - 1 for L in LENS]), dev_bits(kn), dev_bits(vn))
    plan_a = a.cache.decode_plan(0, kv, maxl)
    out_a = host_bits(a.cache.decode(0, kv, dev_bits(q), maxl, plan=plan_a))
    # one call
    plan_b = b.cache.decode_plan(0, kv, maxl)
    out_b = host_bits(b.cache.decode_append(0, plan_b, dev_bits(kn), dev_bits(vn), dev_bits(q), maxl))
    torch.cuda.synchronize()
    assert np.array_equal(out_a, out_b)
    ka, va = _slab_bits(a, 0)
    kb, vb = _slab_bits(b, 0)
    assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    # and the oracle, with the new rows appended to its logical cache
    for bb, L in enumerate(LENS):
        b.oracle.store(0, bb, L - 1, kn[bb:bb + 1], vn[bb:bb + 1])
    ref = np.stack([b.oracle.decode(0, bb, q[bb], L) for bb, L in enumerate(LENS)])
    assert_close(out_b, ref)


def test_append_on_a_stack_with_shared_layers():
    """Owners store and decode; shared layers only decode, reading the rows
    their source's append stored, in the bench step's order (one plan per kind
    of layer); outputs equal store + decode layer by layer."""
    need_gpu()
    specs = [LayerSpec("sliding", 256, 8, 1, 512), LayerSpec("full", 512, 8, 1, 0),
             LayerSpec("sliding", 256, 8, 1, 512), LayerSpec("full", 512, 8, 1, 0)]
    lens = [1, 17, 513, 700, 2049, 16, 31]
    a, b = _pair(specs, 2, lens, seed=83)
    rng = np.random.default_rng(9)
    kv, maxl = i32(lens), max(lens)
    plans_a, plans_b = {}, {}
    for layer in range(4):
        key = a.cache.plan_key(layer)
        if key not in plans_a:
            plans_a[key] = a.cache.decode_plan(layer, kv, maxl)
            plans_b[key] = b.cache.decode_plan(layer, kv, maxl)
    for layer in range(4):
        s = specs[layer]
        kn, vn = _new_rows(rng, s, len(lens))
        q = normal_bf16(rng, (len(lens), s.num_q_heads, s.head_dim))
        a.cache.store(layer, i32(np.arange(len(lens) + 1)), i32([L - 1 for L in lens]), dev_bits(kn),
                      dev_bits(vn))
        out_a = host_bits(a.cache.decode(layer, kv, dev_bits(q), maxl, plan=plans_a[a.cache.plan_key(layer)]))
        shared = b.cache.sources[layer] != layer
        out_b = host_bits(b.cache.decode_append(layer, plans_b[b.cache.plan_key(layer)],
                                                None if shared else dev_bits(kn), None if shared else dev_bits(vn),
                                                dev_bits(q), maxl))
        torch.cuda.synchronize()
        assert np.array_equal(out_a, out_b), f"layer {layer}"
    for layer in (0, 1):
        ka, va = _slab_bits(a, layer)
        kb, vb = _slab_bits(b, layer)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb), f"slab {layer}"


def test_append_refuses_int8_owner_before_launch():
    need_gpu()
    from full_attention_amd import pakv
    spec = LayerSpec("full", 256, 8, 1, 0, kv_dtype="int8")
    lens = [5, 40]
    sc = Scenario([spec], None, lens, seed=3)
    sc.store(0, [0, 0], [4, 39])
    before = host_bits(sc.cache.slab_of(0)[0]).copy()
    kn, vn = _new_rows(np.random.default_rng(1), spec, 2)
    q = normal_bf16(np.random.default_rng(2), (2, 8, 256))
    plan = sc.cache.decode_plan(0, i32(lens), 40)
    with pytest.raises(pakv.PakvError) as e:
        sc.cache.decode_append(0, plan, dev_bits(kn), dev_bits(vn), dev_bits(q), 40)
    assert e.value.status == pakv.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert np.array_equal(before, host_bits(sc.cache.slab_of(0)[0]))


def test_append_in_graph_replays():
    """Captured once, replayed with the program's own work between replays: each
    replay stores the same rows again and gives the eager output."""
    need_gpu()
    specs = [LayerSpec("sliding", 256, 8, 1, 512), LayerSpec("full", 512, 8, 1, 0)]
    lens = [3, 600, 1500, 16]
    sc = Scenario(specs, None, lens, seed=91)
    for layer in range(2):
        sc.store(layer, [0] * len(lens), [L - 1 for L in lens])
    rng = np.random.default_rng(4)
    kv, maxl = i32(lens), max(lens)
    news = [_new_rows(rng, s, len(lens)) for s in specs]
    qs = [dev_bits(normal_bf16(rng, (len(lens), 8, s.head_dim))) for s in specs]
    kns = [(dev_bits(k), dev_bits(v)) for k, v in news]
    outs = [torch.empty_like(q) for q in qs]
    plans = [sc.cache.decode_plan(l, kv, maxl) for l in range(2)]

    def step():
        for l in range(2):
            sc.cache.decode_append(l, plans[l], kns[l][0], kns[l][1], qs[l], maxl, out=outs[l])

    step()
    torch.cuda.synchronize()
    eager = [host_bits(o).copy() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert np.array_equal(e, host_bits(o))
