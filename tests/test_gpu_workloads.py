"""The five workloads at full size, run the way bench.py runs them (same
kernels, same grid), checked against the oracle on sampled outputs.

Rows are drawn on the device by a seeded generator (workloads.DeviceDraws),
stored through paged_kv_store, and the rows of the sampled sequences are
copied back to the host for the oracle: the oracle's inputs are the draws,
never the slabs.  Tolerance: |gpu - ref| <= 2e-2 + 1e-2 |ref| per element.
"""

import numpy as np
import pytest
import torch

from oracle import attend, quantise_rows, dequantise_rows
from workloads import (DeviceDraws, bf16_to_f32, e2b_decode_workload, e2b_extend_workload,
                       int8_long_workload, make_page_pool, moe26b_decode_workload, tiny_workload)

from gpu_helpers import assert_close, host_bits, i32, need_gpu

pytestmark = pytest.mark.gpu


def f64(bits_dev):
    return bf16_to_f32(host_bits(bits_dev)).astype(np.float64)


class DeviceScenario:
    """Slabs for a workload, rows drawn on the device; keeps host copies of
    the rows of the sampled sequences only."""

    def __init__(self, wl, capacities, sample):
        from full_attention_amd.cache import PagedKVCache
        self.wl = wl
        self.B = len(capacities)
        self.pool = make_page_pool(np.random.default_rng(wl.seed), capacities)
        self.cache = PagedKVCache(wl.layers, wl.first_shared, self.pool.num_pages)
        self.cache.set_page_table(self.pool.page_table)
        self.draws = DeviceDraws(wl.seed)
        self.sample = list(sample)
        self.kept = {}      # (owner layer, seq) -> (positions, k f32, v f32) on the host

    def store(self, layer, starts, counts):
        if self.cache.sources[layer] != layer:
            return
        s = self.wl.layers[layer]
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        k = self.draws.bf16((int(cu[-1]), s.num_kv_heads, s.head_dim))
        v = self.draws.rms_normalised(k) if s.k_eq_v else self.draws.bf16((int(cu[-1]), s.num_kv_heads, s.head_dim))
        self.cache.store(layer, i32(cu), i32(starts), k, v)
        for b in self.sample:
            if counts[b] == 0:
                continue
            pos = np.arange(starts[b], starts[b] + counts[b])
            kb = bf16_to_f32(host_bits(k[cu[b]:cu[b + 1]]))
            vb = bf16_to_f32(host_bits(v[cu[b]:cu[b + 1]]))
            old = self.kept.get((layer, b))
            if old is not None:
                pos = np.concatenate([old[0], pos])
                kb = np.concatenate([old[1], kb])
                vb = np.concatenate([old[2], vb])
            self.kept[(layer, b)] = (pos, kb, vb)
        del k, v

    def rows(self, layer, b):
        """(positions, k, v) float64 of the slab `layer` reads, as the oracle
        sees it (int8 layers: the oracle's own encoding of the drawn rows)."""
        pos, k, v = self.kept[(self.cache.sources[layer], b)]
        if self.wl.layers[layer].kv_dtype == "int8":
            kq, ks = quantise_rows(k)
            vq, vs = quantise_rows(v)
            return pos, dequantise_rows(kq, ks), dequantise_rows(vq, vs)
        return pos, k.astype(np.float64), v.astype(np.float64)


def _decode_workload(wl, n_sample=3, layers=None):
    lens = np.array(wl.cached_lens, dtype=np.int64)
    kv = lens + 1
    order = np.argsort(lens)
    sample = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2])})[:n_sample]
    sc = DeviceScenario(wl, kv, sample)
    for l, s in enumerate(wl.layers):
        lo = np.maximum(0, kv - s.window) if s.window else np.zeros_like(kv)
        sc.store(l, lo, kv - lo)
    q_all = []
    outs = []
    for l, s in enumerate(wl.layers):
        q = sc.draws.bf16((sc.B, s.num_q_heads, s.head_dim))
        outs.append(sc.cache.decode(l, i32(kv), q, int(kv.max())))
        q_all.append(q)
    torch.cuda.synchronize()
    worst = 0.0
    check_layers = range(len(wl.layers)) if layers is None else layers
    for l in check_layers:
        s = wl.layers[l]
        got = host_bits(outs[l])
        qf = f64(q_all[l])
        for b in sample:
            pos, k, v = sc.rows(l, b)
            ref = attend(qf[b:b + 1], np.array([kv[b] - 1]), k, v, pos, s.window, s.sm_scale)[0]
            worst = max(worst, assert_close(got[b], ref, f"{wl.name} layer {l} seq {b}"))
    return worst


def test_tiny_workload_both_readings():
    """2 sequences cached to 100 and 37; decode one token each, then a 64-token
    chunk on sequence 0, (a) after the decode token (positions 101..164) and
    (b) from the same cached state (positions 100..163)."""
    need_gpu()
    wl = tiny_workload()
    lens = np.array(wl.cached_lens)
    for reading in ("after", "same"):
        sc = DeviceScenario(wl, [lens[0] + 1 + 64, lens[1] + 1], [0, 1])
        for l, s in enumerate(wl.layers):
            sc.store(l, [0, 0], [lens[0] + 1, lens[1] + 1])
        for l, s in enumerate(wl.layers):
            q = sc.draws.bf16((2, s.num_q_heads, s.head_dim))
            out = host_bits(sc.cache.decode(l, i32(lens + 1), q, int(lens.max() + 1)))
            for b in range(2):
                pos, k, v = sc.rows(l, b)
                ref = attend(f64(q)[b:b + 1], np.array([lens[b]]), k, v, pos, s.window, s.sm_scale)[0]
                assert_close(out[b], ref, f"tiny decode layer {l} seq {b}")
        start = lens[0] + 1 if reading == "after" else lens[0]
        for l, s in enumerate(wl.layers):
            # the chunk's K/V (over the decode token's slot in the "same" reading)
            sc.store(l, [start, 0], [64, 0])
            q = sc.draws.bf16((64, s.num_q_heads, s.head_dim))
            out = host_bits(sc.cache.extend(l, i32([0, 64, 64]), i32([start, lens[1] + 1]), q, 64, start + 64))
            pos, k, v = sc.rows(l, 0)
            # a later store of a position replaces the earlier row
            last = {p: i for i, p in enumerate(pos)}
            idx = np.array(sorted(last.values()))
            ref = attend(f64(q), np.arange(start, start + 64), k[idx], v[idx], pos[idx], s.window, s.sm_scale)
            assert_close(out, ref, f"tiny extend ({reading}) layer {l}")


def test_e2b_decode_full_size():
    need_gpu()
    _decode_workload(e2b_decode_workload())


def test_moe26b_decode_full_size():
    need_gpu()
    _decode_workload(moe26b_decode_workload(), n_sample=2)


def test_int8_long_context_full_size():
    need_gpu()
    _decode_workload(int8_long_workload(), n_sample=2)


def test_e2b_extend_full_size():
    need_gpu()
    wl = e2b_extend_workload()
    P = np.array(wl.cached_lens, dtype=np.int64)
    n = np.array(wl.extend_lens, dtype=np.int64)
    sc = DeviceScenario(wl, P + n, range(len(P)))
    for l, s in enumerate(wl.layers):
        lo = np.maximum(0, P - s.window + 1) if s.window else np.zeros_like(P)
        sc.store(l, lo, P - lo)          # cached prefix (rows a chunk query can see)
    cu = np.concatenate([[0], np.cumsum(n)])
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 511, 512, 513, 1023, 2047], rng.integers(0, 2048, 7)]))
    for l, s in enumerate(wl.layers):
        sc.store(l, P, n)                # the chunk, through paged_kv_store (owners only)
        q = sc.draws.bf16((int(cu[-1]), s.num_q_heads, s.head_dim))
        out = host_bits(sc.cache.extend(l, i32(cu), i32(P), q, int(n.max()), int((P + n).max())))
        qf = f64(q)
        for b in range(len(P)):
            pos, k, v = sc.rows(l, b)
            ref = attend(qf[cu[b] + rows], P[b] + rows, k, v, pos, s.window, s.sm_scale)
            assert_close(out[cu[b] + rows], ref, f"E2B extend layer {l} seq {b}")
