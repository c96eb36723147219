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


# ---- extend positions and the key cut (hand-worked) -------------------------
# An extend chunk of n queries after a cached prefix of P tokens sits at
# positions P .. P + n - 1 (FreeToken PR #898, description, fourth bullet: the
# chunk follows what the cache already holds); the tiny workload's chunk after
# its decode token starts at 101 and ends at 164.

from oracle import extend_positions


def test_extend_positions_hand_typed():
    assert extend_positions(3, 2).tolist() == [3, 4]
    assert extend_positions(0, 1).tolist() == [0]
    assert extend_positions(5, 0).tolist() == []
    pos = extend_positions(101, 64)
    assert pos[0] == 101 and pos[-1] == 164 and len(pos) == 64


def _scalar_layers(window):
    # D = 1, one head; sm_scale irrelevant once q = 0
    return [dict(type="sliding" if window else "full", head_dim=1, num_q_heads=1, num_kv_heads=1,
                 window=window, kv_dtype="bf16", sm_scale=1.0)]


def _bits(vals):
    from workloads import bf16_from_f32
    return bf16_from_f32(np.asarray(vals, dtype=np.float32).reshape(-1, 1, 1))


def test_extend_chunk_hand_worked_window_two():
    """Values 10, 20, 30, 40, 50 at positions 0..4, a position-5 row of 1000
    that no query may see, q = 0 (so the output is the mean of the visible
    values).  Prefix 3, chunk 2: the queries sit at 3 and 4; with W = 2 they
    see {2, 3} and {3, 4}: (30 + 40) / 2 = 35 and (40 + 50) / 2 = 45.  A chunk
    placed one position early gives 25 and 35; a window taken as an inclusive
    distance gives 30 and 40."""
    c = LogicalCache(_scalar_layers(2), None, 1)
    c.store(0, 0, 0, _bits([10, 20, 30, 40, 50, 1000]), _bits([10, 20, 30, 40, 50, 1000]))
    out = c.extend(0, 0, _bits([0, 0]).reshape(2, 1, 1), 3)
    assert out.shape == (2, 1, 1)
    assert out[:, 0, 0].tolist() == [35.0, 45.0]


def test_extend_chunk_hand_worked_full():
    """Same rows, full causal layer: the queries at 3 and 4 see 0..3 and 0..4:
    means 25 and 30.  The row at position 5 is cut."""
    c = LogicalCache(_scalar_layers(0), None, 1)
    c.store(0, 0, 0, _bits([10, 20, 30, 40, 50, 1000]), _bits([10, 20, 30, 40, 50, 1000]))
    out = c.extend(0, 0, _bits([0, 0]).reshape(2, 1, 1), 3)
    assert out[:, 0, 0].tolist() == [25.0, 30.0]


def test_extend_chunk_of_tiny_workload_counts_its_keys():
    """Tiny workload, chunk after the decode token: prefix 101, 64 queries at
    101..164.  With q = 0 and value v_j = j, the query at p sees j in
    [max(0, p - W + 1), p]: the mean is the midpoint of that range (W = 32:
    p - 15.5; full: p / 2)."""
    vals = np.arange(165, dtype=np.float32)
    for window in (32, 0):
        c = LogicalCache(_scalar_layers(window), None, 1)
        c.store(0, 0, 0, _bits(vals), _bits(vals))
        out = c.extend(0, 0, _bits(np.zeros(64)).reshape(64, 1, 1), 101)[:, 0, 0]
        p = np.arange(101, 165, dtype=np.float64)
        want = p - 15.5 if window else p / 2
        assert np.array_equal(out, want), window


# ---- K=V layers (value = RMS-normalised key) and packed extend chunks -------

from oracle import v_from_k


def _kv_layer(d, eps, fmt="bf16", window=0):
    return dict(type="sliding" if window else "full", head_dim=d, num_q_heads=1, num_kv_heads=1,
                window=window, kv_dtype=fmt, sm_scale=1.0, k_eq_v=True, v_norm_eps=eps)


def test_v_from_k_closed_forms():
    # mean of squares 25 -> root 5: [1, 7] / 5
    assert v_from_k(np.array([[1.0, 7.0]]), 0.0).tolist() == [[0.2, 1.4]]
    # a constant row normalises to ones (sign kept); a one-hot row to sqrt(D)
    assert v_from_k(np.array([[-3.0, -3.0, -3.0, -3.0]]), 0.0).tolist() == [[-1.0] * 4]
    assert v_from_k(np.array([[0.0, 2.0, 0.0, 0.0]]), 0.0).tolist() == [[0.0, 2.0, 0.0, 0.0]]
    # eps sits under the root: [1, 7] with eps 1 -> [1, 7] / sqrt(26)
    assert np.allclose(v_from_k(np.array([[1.0, 7.0]]), 1.0), np.array([[1.0, 7.0]]) / np.sqrt(26.0), rtol=1e-15)
    # scale invariance when eps = 0, and unit mean square
    k = np.random.default_rng(0).standard_normal((5, 64))
    assert np.allclose(v_from_k(3.5 * k, 0.0), v_from_k(k, 0.0), rtol=1e-13)
    assert np.allclose(np.mean(v_from_k(k, 0.0) ** 2, axis=-1), 1.0, rtol=1e-13)


def test_k_eq_v_layer_stores_keys_only_and_derives_values():
    """D = 2, q = 0: the decode output is the mean of the visible value rows.
    Keys [1, 7] and [5, 5] (eps 0) give values [0.2, 1.4] and [1, 1]: the
    query at position 1 sees both, mean [0.6, 1.2]; a shared layer reads the
    same rows."""
    layers = [_kv_layer(2, 0.0), dict(_kv_layer(2, 0.0))]
    c = LogicalCache(layers, 1, 1)
    k = _bits([[1.0, 7.0], [5.0, 5.0]]).reshape(2, 1, 2)
    c.store(0, 0, 0, k, None)
    pos, rows = c.stored(0, 0)
    assert all(r[1] is None for r in rows)          # no value rows kept
    q = _bits([0.0, 0.0]).reshape(1, 2)
    out = c.decode(0, 0, q, 2)
    assert np.allclose(out[0], [0.6, 1.2], rtol=1e-15)
    assert np.array_equal(c.decode(1, 0, q, 2), out)


def test_k_eq_v_int8_layer_normalises_the_decoded_key():
    """int8 K=V: the value is the decoded key row, normalised.  Key [127, -127]
    quantises exactly (scale 1), so its value is [1, -1] (eps 0)."""
    c = LogicalCache([_kv_layer(2, 0.0, fmt="int8")], None, 1)
    c.store(0, 0, 0, _bits([[127.0, -127.0]]).reshape(1, 1, 2), None)
    out = c.decode(0, 0, _bits([0.0, 0.0]).reshape(1, 2), 1)
    assert out[0].tolist() == [1.0, -1.0]


def test_extend_packed_takes_the_chunk_as_given():
    """D = 1, q = 0.  Stored 10, 20, 30 at positions 0..2 and a stale 1000 at 3;
    the chunk at prefix 3 comes as packed rows 40, 50: the queries at 3 and 4
    see (10 + 20 + 30 + 40) / 4 = 25 and 30.  The stored row at position 3
    is not used."""
    c = LogicalCache(_scalar_layers(0), None, 1)
    c.store(0, 0, 0, _bits([10, 20, 30, 1000]), _bits([10, 20, 30, 1000]))
    out = c.extend_packed(0, 0, _bits([0, 0]).reshape(2, 1, 1), 3, _bits([40, 50]), _bits([40, 50]))
    assert out[:, 0, 0].tolist() == [25.0, 30.0]
    # no prefix at all
    c2 = LogicalCache(_scalar_layers(2), None, 1)
    out = c2.extend_packed(0, 0, _bits([0, 0, 0]).reshape(3, 1, 1), 0, _bits([4, 8, 16]), _bits([4, 8, 16]))
    assert out[:, 0, 0].tolist() == [4.0, 6.0, 12.0]


def test_extend_packed_chunk_stays_exact_over_an_int8_prefix():
    """An int8 cache: the stored prefix is decoded (127 and 254 quantise to code
    127 with scales 1 and 2, exactly), the packed chunk row 3 is taken as given
    (bf16, not quantised): means (127 + 254 + 3) / 3 = 128."""
    layers = [dict(type="full", head_dim=1, num_q_heads=1, num_kv_heads=1, window=0, kv_dtype="int8",
                   sm_scale=1.0)]
    c = LogicalCache(layers, None, 1)
    c.store(0, 0, 0, _bits([127, 254]), _bits([127, 254]))
    out = c.extend_packed(0, 0, _bits([0]).reshape(1, 1, 1), 2, _bits([3]), _bits([3]))
    assert out[0, 0, 0] == 128.0
