"""Pins for oracle.attention.

Each pin is written so that a plausible mistake in the oracle fails at least
one of them; ``test_planted_mistakes_are_caught`` plants such mistakes in a
copy of the oracle (on the CPU) and checks exactly that.

* a hand-typed mask (window W = 3) and brute-force row counts min(p + 1, W);
* the window edge: a marker W - 1 positions back is seen, one W back is not
  (pegainfer issue #807, Description: the current token counts inside W);
* closed forms: W = 1 returns the query's own value row; a zero query or equal
  keys average the visible value rows; the first position sees only itself;
* a library routine: torch's scaled_dot_product_attention in float64 on the
  CPU, given the boolean mask and KV heads repeated over their query groups,
  with its default 1/sqrt(D) scale;
* brute force: scalar Python loops with math.exp on tiny inputs;
* numerically large logits stay finite and agree with the library routine.
"""

import math

import numpy as np
import pytest
import torch

import oracle.attention as oa
from oracle import attend, visibility_mask


# ---------------------------------------------------------------- references

def sdpa_reference(q, q_pos, k, v, kv_pos, window):
    """torch SDPA, float64, CPU, explicit boolean mask, default scale."""
    hq, hkv = q.shape[1], k.shape[1]
    p = torch.as_tensor(np.asarray(q_pos))[:, None]
    j = torch.as_tensor(np.asarray(kv_pos))[None, :]
    mask = j <= p
    if window:
        mask = mask & (p - j < window)
    qt = torch.as_tensor(q, dtype=torch.float64).permute(1, 0, 2)
    kt = torch.as_tensor(k, dtype=torch.float64).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    vt = torch.as_tensor(v, dtype=torch.float64).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(), attn_mask=mask)
    return out.permute(1, 0, 2).numpy()


def scalar_reference(q, q_pos, k, v, kv_pos, window, scale):
    nq, hq, d = q.shape
    hkv = k.shape[1]
    out = np.zeros((nq, hq, d))
    for i in range(nq):
        for h in range(hq):
            g = h // (hq // hkv)
            logits = []
            for r in range(len(kv_pos)):
                dist = int(q_pos[i]) - int(kv_pos[r])
                if dist < 0 or (window and dist >= window):
                    continue
                logits.append((r, scale * sum(float(q[i, h, t]) * float(k[r, g, t]) for t in range(d))))
            top = max(s for _, s in logits)
            ws = [(r, math.exp(s - top)) for r, s in logits]
            total = sum(w for _, w in ws)
            for t in range(d):
                out[i, h, t] = sum(w * float(v[r, g, t]) for r, w in ws) / total
    return out


def rand_case(rng, nq=5, hq=4, hkv=2, d=8, n_kv=30, window=0, shuffle=False):
    kv_pos = np.arange(n_kv)
    if shuffle:
        kv_pos = rng.permutation(n_kv)
    q_pos = np.sort(rng.choice(np.arange(n_kv), size=nq, replace=False))
    q = rng.standard_normal((nq, hq, d))
    k = rng.standard_normal((n_kv, hkv, d))
    v = rng.standard_normal((n_kv, hkv, d))
    return q, q_pos, k, v, kv_pos, window


# ---------------------------------------------------------------- pins, parametrised by implementation

def pin_window_edge(fn):
    d, p, w = 4, 40, 8
    q = np.zeros((1, 1, d))
    k = np.ones((p + 1, 1, d))
    pos = np.arange(p + 1)
    v_in = np.zeros((p + 1, 1, d)); v_in[p - (w - 1), 0, :] = 1000.0
    v_out = np.zeros((p + 1, 1, d)); v_out[p - w, 0, :] = 1000.0
    a = fn(q, np.array([p]), k, v_in, pos, w, 0.5)
    b = fn(q, np.array([p]), k, v_out, pos, w, 0.5)
    return np.allclose(a, 1000.0 / w, rtol=0, atol=1e-12) and np.allclose(b, 0.0, atol=1e-12)


def pin_window_one(fn):
    rng = np.random.default_rng(1)
    q, q_pos, k, v, kv_pos, _ = rand_case(rng, window=1)
    out = fn(q, q_pos, k, v, kv_pos, 1, 0.3)
    hq, hkv = q.shape[1], k.shape[1]
    want = np.stack([np.repeat(v[p], hq // hkv, axis=0) for p in q_pos])
    return np.array_equal(out, want)


def pin_uniform_weights(fn):
    rng = np.random.default_rng(2)
    ok = True
    for window in (0, 6):
        q, q_pos, k, v, kv_pos, _ = rand_case(rng, window=window)
        out = fn(np.zeros_like(q), q_pos, k, v, kv_pos, window, 0.7)
        for i, p in enumerate(q_pos):
            lo = 0 if window == 0 else max(0, p - window + 1)
            mean = v[lo:p + 1].mean(axis=0)          # [hkv, d]
            want = np.repeat(mean, q.shape[1] // k.shape[1], axis=0)
            ok &= np.allclose(out[i], want, rtol=0, atol=1e-12)
        # equal keys: any query gives the same average
        k_eq = np.broadcast_to(k[:1], k.shape).copy()
        out2 = fn(q, q_pos, k_eq, v, kv_pos, window, 0.7)
        ok &= np.allclose(out2, out, rtol=0, atol=1e-12)
    return bool(ok)


def pin_first_position(fn):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((10, 2, 8))
    v = rng.standard_normal((10, 2, 8))
    out = fn(q, np.array([0]), k, v, np.arange(10), 0, 0.35)
    return np.array_equal(out[0], np.repeat(v[0], 2, axis=0))


def pin_library(fn):
    rng = np.random.default_rng(4)
    ok = True
    for window in (0, 1, 5, 64):
        for hq, hkv in ((4, 1), (8, 2), (4, 4)):
            q, q_pos, k, v, kv_pos, _ = rand_case(rng, hq=hq, hkv=hkv, d=16, n_kv=40, nq=7,
                                                  window=window, shuffle=True)
            out = fn(q, q_pos, k, v, kv_pos, window, 1.0 / math.sqrt(16))
            ok &= np.allclose(out, sdpa_reference(q, q_pos, k, v, kv_pos, window), rtol=0, atol=1e-12)
    return bool(ok)


def pin_large_logits(fn):
    rng = np.random.default_rng(5)
    q, q_pos, k, v, kv_pos, _ = rand_case(rng, d=16, n_kv=24)
    q = q * 300.0
    out = fn(q, q_pos, k, v, kv_pos, 0, 1.0 / math.sqrt(16))
    return bool(np.isfinite(out).all() and
                np.allclose(out, sdpa_reference(q, q_pos, k, v, kv_pos, 0), rtol=0, atol=1e-10))


PINS = [pin_window_edge, pin_window_one, pin_uniform_weights, pin_first_position,
        pin_library, pin_large_logits]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(attend)


# ---------------------------------------------------------------- mask

def test_hand_typed_mask_w3():
    want = np.array([
        [1, 0, 0, 0, 0, 0],
        [1, 1, 0, 0, 0, 0],
        [1, 1, 1, 0, 0, 0],
        [0, 1, 1, 1, 0, 0],
        [0, 0, 1, 1, 1, 0],
        [0, 0, 0, 1, 1, 1],
    ], dtype=bool)
    assert np.array_equal(visibility_mask(np.arange(6), np.arange(6), 3), want)
    assert np.array_equal(visibility_mask(np.arange(6), np.arange(6), 0), np.tril(np.ones((6, 6), bool)))


def test_mask_row_counts_brute_force():
    for w in (0, 1, 2, 7, 32, 512):
        for p in (0, 1, 5, 31, 32, 33, 600):
            row = visibility_mask(np.array([p]), np.arange(p + 50), w)[0]
            assert row.sum() == (p + 1 if w == 0 else min(p + 1, w))
            vis = [j for j in range(p + 50) if j <= p and (w == 0 or p - j < w)]
            assert np.flatnonzero(row).tolist() == vis


def test_window_at_least_length_equals_full():
    rng = np.random.default_rng(6)
    q, q_pos, k, v, kv_pos, _ = rand_case(rng, n_kv=20)
    assert np.array_equal(attend(q, q_pos, k, v, kv_pos, 20, 0.4), attend(q, q_pos, k, v, kv_pos, 0, 0.4))
    assert np.array_equal(attend(q, q_pos, k, v, kv_pos, 1000, 0.4), attend(q, q_pos, k, v, kv_pos, 0, 0.4))


def test_brute_force_scalar_loops():
    rng = np.random.default_rng(8)
    for window in (0, 3, 9):
        q, q_pos, k, v, kv_pos, _ = rand_case(rng, nq=4, hq=4, hkv=2, d=6, n_kv=25,
                                              window=window, shuffle=True)
        out = attend(q, q_pos, k, v, kv_pos, window, 0.45)
        assert np.allclose(out, scalar_reference(q, q_pos, k, v, kv_pos, window, 0.45), rtol=0, atol=1e-12)


def test_row_order_does_not_matter():
    rng = np.random.default_rng(9)
    q, q_pos, k, v, kv_pos, _ = rand_case(rng, n_kv=33, window=7)
    perm = rng.permutation(33)
    a = attend(q, q_pos, k, v, kv_pos, 7, 0.5)
    b = attend(q, q_pos, k[perm], v[perm], kv_pos[perm], 7, 0.5)
    assert np.allclose(a, b, rtol=0, atol=1e-14)


def test_rows_nobody_sees_may_hold_nan():
    rng = np.random.default_rng(10)
    q, q_pos, k, v, kv_pos, _ = rand_case(rng, n_kv=30, window=4)
    lo = int(q_pos.min()) - 4
    k2, v2 = k.copy(), v.copy()
    if lo >= 0:
        k2[: lo + 1] = np.nan
        v2[: lo + 1] = np.nan
    assert np.array_equal(attend(q, q_pos, k2, v2, kv_pos, 4, 0.5), attend(q, q_pos, k, v, kv_pos, 4, 0.5))


def test_query_without_keys_is_an_error():
    with pytest.raises(ValueError):
        attend(np.zeros((1, 1, 4)), np.array([5]), np.zeros((2, 1, 4)), np.zeros((2, 1, 4)),
               np.array([6, 7]), 0, 1.0)


# ---------------------------------------------------------------- planted mistakes

def _mutant(kind):
    def fn(q, q_pos, k, v, kv_pos, window, sm_scale):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        nq, hq, d = q.shape
        hkv = k.shape[1]
        p = np.asarray(q_pos)[:, None]
        j = np.asarray(kv_pos)[None, :]
        mask = j <= p
        if window > 0:
            mask = mask & (((p - j) <= window) if kind == "window_le" else ((p - j) < window))
        if kind == "not_causal":
            mask = (p - j < window) if window else np.ones_like(mask)
        out = np.empty((nq, hq, d))
        for h in range(hq):
            g = (h % hkv) if kind == "gqa_mod" else h // (hq // hkv)
            scale = 1.0 if kind == "no_scale" else sm_scale
            s = scale * (q[:, h] @ k[:, g].T)
            s = np.where(mask, s, -np.inf)
            top = 0.0 if kind == "no_max" else s.max(axis=1, keepdims=True)
            w = np.exp(s - top)
            vv = k[:, g] if kind == "k_for_v" else v[:, g]
            denom = 1.0 if kind == "no_norm" else w.sum(axis=1, keepdims=True)
            out[:, h] = (w @ vv) / denom
        return out
    return fn


@pytest.mark.parametrize("kind", ["window_le", "not_causal", "gqa_mod", "no_scale", "no_max",
                                  "k_for_v", "no_norm"])
def test_planted_mistakes_are_caught(kind):
    fn = _mutant(kind)
    with np.errstate(all="ignore"):
        results = []
        for pin in PINS:
            try:
                results.append(pin(fn))
            except Exception:
                results.append(False)
    assert not all(results), f"no pin catches the planted mistake {kind!r}"
