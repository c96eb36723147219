"""Pins for oracle.cache: shared layers store nothing and read their source's
rows (FreeToken PR #898, description: store_kv's early return; outputs
unchanged because the copies held the source's rows), and a shared sliding
layer keeps its own window (unsloth commit dee9371 and commit ca9dbce: the
earlier cut lost the window on shared sliding layers)."""

import numpy as np

from oracle import LogicalCache, quantise_rows, attend
from oracle.cache import bf16_bits_to_f32
from workloads import normal_bf16, bf16_to_f32


def _layers(d=16, hq=4, hkv=1, w=8, fmt="bf16"):
    mk = lambda t, win: dict(type=t, head_dim=d, num_q_heads=hq, num_kv_heads=hkv, window=win,
                             kv_dtype=fmt, sm_scale=1.0 / np.sqrt(d))
    # 0: sliding, 1: full (owners); 2: sliding, 3: full (shared)
    return [mk("sliding", w), mk("full", 0), mk("sliding", w), mk("full", 0)]


def _fill(cache, rng, n, hkv=1, d=16, layers=(0, 1, 2, 3)):
    data = {}
    for layer in layers:
        k = normal_bf16(rng, (n, hkv, d))
        v = normal_bf16(rng, (n, hkv, d))
        cache.store(layer, 0, 0, k, v)
        data[layer] = (k, v)
    return data


def test_shared_layer_output_equals_source_output():
    rng = np.random.default_rng(0)
    c = LogicalCache(_layers(), 2, 1)
    _fill(c, rng, 40)
    q = normal_bf16(rng, (4, 16))
    assert np.array_equal(c.decode(2, 0, q, 40), c.decode(0, 0, q, 40))
    assert np.array_equal(c.decode(3, 0, q, 40), c.decode(1, 0, q, 40))
    qe = normal_bf16(rng, (10, 4, 16))
    assert np.array_equal(c.extend(3, 0, qe, 30), c.extend(1, 0, qe, 30))


def test_shared_layer_store_is_a_no_op():
    rng = np.random.default_rng(1)
    c = LogicalCache(_layers(), 2, 1)
    data = _fill(c, rng, 20)
    pos, k, v = c.values(0, 0)
    assert np.array_equal(k, bf16_to_f32(data[0][0]).astype(np.float64))
    assert np.array_equal(v, bf16_to_f32(data[0][1]).astype(np.float64))
    assert set(c._rows) == {(0, 0), (1, 0)}


def test_shared_sliding_layer_keeps_its_window():
    rng = np.random.default_rng(2)
    c = LogicalCache(_layers(w=8), 2, 1)
    _fill(c, rng, 40)
    q = normal_bf16(rng, (4, 16))
    shared_sliding = c.decode(2, 0, q, 40)
    pos, k, v = c.values(2, 0)
    qf = bf16_bits_to_f32(q)[None]
    full = attend(qf, np.array([39]), k, v, pos, 0, 0.25)[0]
    windowed = attend(qf, np.array([39]), k, v, pos, 8, 0.25)[0]
    assert np.array_equal(shared_sliding, windowed)
    assert not np.allclose(shared_sliding, full)


def test_int8_layer_stores_codes_and_scales():
    rng = np.random.default_rng(3)
    c = LogicalCache(_layers(fmt="int8"), 2, 1)
    data = _fill(c, rng, 12)
    pos, rows = c.stored(2, 0)           # shared sliding layer reads layer 0
    kq, ks = quantise_rows(bf16_to_f32(data[0][0]))
    assert np.array_equal(np.stack([r[0] for r in rows]), kq)
    assert np.array_equal(np.stack([r[2] for r in rows]), ks)
    q = normal_bf16(rng, (4, 16))
    out = c.decode(0, 0, q, 12)
    _, k, v = c.values(0, 0)
    assert np.allclose(k, bf16_to_f32(data[0][0]), atol=np.abs(ks).max())
    assert np.isfinite(out).all()


def test_positions_past_kv_len_are_ignored():
    rng = np.random.default_rng(4)
    c = LogicalCache(_layers(), None, 1)
    _fill(c, rng, 30)
    q = normal_bf16(rng, (4, 16))
    a = c.decode(1, 0, q, 20)
    c2 = LogicalCache(_layers(), None, 1)
    rng = np.random.default_rng(4)
    data = _fill(c2, rng, 30)
    pos, k, v = c2.values(1, 0)
    want = attend(bf16_bits_to_f32(q)[None], np.array([19]), k[:20], v[:20], pos[:20], 0, 0.25)[0]
    assert np.array_equal(a, want)
