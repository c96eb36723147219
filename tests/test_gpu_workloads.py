"""The five workloads at full size (and the long-context one with fp8 KV),
run the way bench.py runs them (same kernels, same grid), checked against the
oracle on sampled outputs.

Rows are drawn on the device by a seeded generator (workloads.DeviceDraws),
stored through paged_kv_store, and the rows of the sampled sequences are
copied back to the host for the oracle: the oracle's inputs are the draws,
never the slabs.  Tolerance: |gpu - ref| <= 2e-2 + 1e-2 |ref| per element.
"""

import numpy as np
import pytest
import torch

from oracle import attend, fp8_pth, quantise_rows, dequantise_rows, v_from_k
from workloads.configs import V_NORM_EPS
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

    def store(self, layer, starts, counts, make_rows=None):
        """make_rows(layer, positions [T] int64 device tensor, k) -> (k, v) device
        bf16 bits, to replace the N(0, 1) draws (v may be None: drawn)."""
        if self.cache.sources[layer] != layer:
            return
        s = self.wl.layers[layer]
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        k = self.draws.bf16((int(cu[-1]), s.num_kv_heads, s.head_dim))
        v = None
        if make_rows is not None:
            pos = torch.cat([torch.arange(st, st + c, device="cuda", dtype=torch.int64)
                             for st, c in zip(starts, counts)])
            k, v = make_rows(layer, pos, k)
        if v is None:
            v = self.draws.rms_normalised(k) if s.k_eq_v else self.draws.bf16((int(cu[-1]), s.num_kv_heads,
                                                                               s.head_dim))
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
        spec = self.wl.layers[layer]
        if spec.kv_dtype == "int8":
            kq, ks = quantise_rows(k)
            vq, vs = quantise_rows(v)
            k, v = dequantise_rows(kq, ks), dequantise_rows(vq, vs)
        elif spec.kv_dtype == "fp8":
            kq, ks = fp8_pth.quantise_rows(k)
            vq, vs = fp8_pth.quantise_rows(v)
            k, v = fp8_pth.dequantise_rows(kq, ks), fp8_pth.dequantise_rows(vq, vs)
        if spec.k_eq_v and self.cache.specs[layer]["k_eq_v"]:
            # one slab: the library derives the values from the stored keys
            return pos, k.astype(np.float64), v_from_k(k, V_NORM_EPS)
        return pos, k.astype(np.float64), v.astype(np.float64)


def _sample(lens, n_sample):
    """The longest sequence always, then the shortest, then the median one."""
    order = np.argsort(lens, kind="stable")
    picks = []
    for i in (int(order[-1]), int(order[0]), int(order[len(order) // 2])):
        if i not in picks:
            picks.append(i)
    return sorted(picks[:n_sample])


def _decode_workload(wl, n_sample=3, layers=None):
    lens = np.array(wl.cached_lens, dtype=np.int64)
    kv = lens + 1
    sample = _sample(lens, n_sample)
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
            worst = max(worst, assert_close(got[b], ref, f"{wl.name} layer {l} seq {b} (L {kv[b]})",
                                            report=(l < 2)))
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


def test_fp8_long_context_full_size():
    """The long-context workload with fp8 E4M3 per-token-head KV, as
    bench.py's decode_fp8_long runs it (the oracle on its own E4M3 encoding
    of the drawn rows)."""
    import dataclasses
    need_gpu()
    wl = int8_long_workload()
    wl = dataclasses.replace(wl, name=wl.name + " (fp8)",
                             layers=[dataclasses.replace(s, kv_dtype="fp8") for s in wl.layers])
    _decode_workload(wl, n_sample=2)


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
            assert_close(out[cu[b] + rows], ref, f"E2B extend layer {l} seq {b}", report=(l in (0, 4)))


def test_e2b_extend_int8_staged_full_size():
    """The extend stack with int8 per-token-head KV on every layer, in the
    launch configuration bench.py times for it: the staged call, one staging
    pass per owner, the KV-shared layers reusing their source's workspace.
    Sampled rows of every sequence against the oracle (on the oracle's own
    int8 encoding of the drawn rows); row 0 of the empty-prefix sequence sees
    one key, so its output is that key's value row."""
    import dataclasses
    need_gpu()
    wl = e2b_extend_workload()
    wl = dataclasses.replace(wl, layers=[dataclasses.replace(s, kv_dtype="int8") for s in wl.layers])
    P = np.array(wl.cached_lens, dtype=np.int64)
    n = np.array(wl.extend_lens, dtype=np.int64)
    sc = DeviceScenario(wl, P + n, range(len(P)))
    for l, s in enumerate(wl.layers):
        lo = np.maximum(0, P - s.window + 1) if s.window else np.zeros_like(P)
        sc.store(l, lo, P - lo)
    cu = np.concatenate([[0], np.cumsum(n)])
    max_q, max_kv = int(n.max()), int((P + n).max())
    ws = {}
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 511, 512, 513, 1023, 2047], rng.integers(0, 2048, 7)]))
    for l, s in enumerate(wl.layers):
        sc.store(l, P, n)
        src = sc.cache.sources[l]
        if src == l:
            ws[l] = torch.empty(sc.cache.staging_bytes(l, len(P), max_q, max_kv), dtype=torch.uint8, device="cuda")
        q = sc.draws.bf16((int(cu[-1]), s.num_q_heads, s.head_dim))
        out = host_bits(sc.cache.extend_staged(l, i32(cu), i32(P), q, max_q, max_kv, workspace=ws[src],
                                               stage=src == l))
        qf = f64(q)
        for b in range(len(P)):
            pos, k, v = sc.rows(l, b)
            ref = attend(qf[cu[b] + rows], P[b] + rows, k, v, pos, s.window, s.sm_scale)
            assert_close(out[cu[b] + rows], ref, f"E2B int8 staged extend layer {l} seq {b}",
                         report=(l in (0, 4, 20)))


# ---- closed forms at full size ------------------------------------------------
# With q = 0 every visible key scores 0, so the output is the plain mean of the
# visible value rows, whatever the keys hold.  Value row j carries A = D in one
# dimension, (j // s) mod D with s = n_visible // D, and 0 elsewhere, so every
# dimension of the output is A * (its keys) / n_visible, about 1; a page (16
# keys) dropped, counted twice or taken from the wrong place moves some
# dimension by at least A * 16 / n_visible (0.06 at 131,073 keys), past the
# tolerance.  Every page of every split of the stream counts.

def _bucket_rows(wl, lens_visible):
    """make_rows for DeviceScenario.store: one-hot value rows by position."""
    def make(layer, pos, k):
        s = wl.layers[layer]
        d = s.head_dim
        step = max(1, int(lens_visible[layer]) // d)
        v = torch.zeros((pos.numel(), s.num_kv_heads, d), dtype=torch.bfloat16, device="cuda")
        dim = (pos // step) % d
        v[torch.arange(pos.numel(), device="cuda"), :, dim] = float(d)
        return k, v.view(torch.int16)
    return make


def _closed_form_mean(window, kv_len, d, lens_visible):
    lo = max(0, kv_len - window) if window else 0
    step = max(1, int(lens_visible) // d)
    dims = (np.arange(lo, kv_len) // step) % d
    return np.bincount(dims, minlength=d).astype(np.float64) * d / (kv_len - lo)


def _check_bucket_decode(wl, sample, seqs_label):
    lens = np.array(wl.cached_lens, dtype=np.int64)
    kv = lens + 1
    n_vis = {l: (min(int(kv.max()), s.window) if s.window else int(kv.max())) for l, s in enumerate(wl.layers)}
    sc = DeviceScenario(wl, kv, sample)
    for l, s in enumerate(wl.layers):
        lo = np.maximum(0, kv - s.window) if s.window else np.zeros_like(kv)
        sc.store(l, lo, kv - lo, make_rows=_bucket_rows(wl, n_vis))
    for l, s in enumerate(wl.layers):
        if sc.cache.sources[l] != l:
            continue
        q = torch.zeros((sc.B, s.num_q_heads, s.head_dim), dtype=torch.int16, device="cuda")
        got = host_bits(sc.cache.decode(l, i32(kv), q, int(kv.max())))
        torch.cuda.synchronize()
        for b in sample:
            pos, k, v = sc.rows(l, b)
            ref = attend(np.zeros((1, s.num_q_heads, s.head_dim)), np.array([kv[b] - 1]), k, v, pos, s.window,
                         s.sm_scale)[0]
            closed = _closed_form_mean(s.window, int(kv[b]), s.head_dim, n_vis[l])
            # the oracle agrees with the closed form (8-bit: to the encoding's error)
            tol = 1e-3 if s.kv_dtype in ("int8", "fp8") else 1e-9
            assert np.abs(ref - closed[None, :]).max() < tol
            assert_close(got[b], ref, f"{wl.name} {seqs_label} layer {l} seq {b}: q = 0, one-hot values", report=True)


def test_int8_long_context_every_page_counts():
    """131,073 keys per sequence, all 8 sequences, both int8 layers."""
    need_gpu()
    _check_bucket_decode(int8_long_workload(), list(range(8)), "all sequences")


def test_fp8_long_context_every_page_counts():
    """The same with fp8 E4M3 per-token-head KV (bench.py's decode_fp8_long)."""
    import dataclasses
    need_gpu()
    wl = int8_long_workload()
    wl = dataclasses.replace(wl, name=wl.name + " (fp8)",
                             layers=[dataclasses.replace(s, kv_dtype="fp8") for s in wl.layers])
    _check_bucket_decode(wl, list(range(8)), "all sequences")


def test_moe26b_longest_sequence_every_page_counts():
    """The 26B-like stack's sliding layers (V free), on its longest sequence."""
    need_gpu()
    wl = moe26b_decode_workload()
    keep = [l for l, s in enumerate(wl.layers) if not s.k_eq_v]
    import copy
    sub = copy.copy(wl)
    sub.layers = [wl.layers[l] for l in keep[:3]]
    _check_bucket_decode(sub, _sample(np.array(wl.cached_lens), 1), "longest sequence")


def test_moe26b_longest_sequence_planted_keys():
    """The 26B-like full layers (V = RMS-normalised K) on their full stack:
    keys planted every 1,000 positions (first page, page edges, the last
    position) point along their own dimension d_m with length 544, and every
    query is the sum of those directions, so each planted key scores about 24
    and all other keys about 0 +- 0.2: the output is the mean of the planted
    keys' value rows (sqrt(D) along d_m), about 1.4 in each d_m; a split that
    is dropped or merged twice moves some d_m by 0.1 or more."""
    need_gpu()
    wl = moe26b_decode_workload()
    lens = np.array(wl.cached_lens, dtype=np.int64)
    kv = lens + 1
    longest = _sample(lens, 1)
    marks = sorted(set([0, 15, 16] + list(range(1000, int(kv.max()), 1000)) + [int(kv[longest[0]]) - 1]))
    marks_t = torch.tensor(marks, device="cuda", dtype=torch.int64)

    def dims_of(n, d):
        return [(7 + 29 * m) % d for m in range(n)]

    def make(layer, pos, k):
        s = wl.layers[layer]
        if not s.k_eq_v:
            return k, None
        hit = torch.isin(pos, marks_t)
        idx = torch.nonzero(hit).flatten()
        m = torch.searchsorted(marks_t, pos[idx])
        dims = torch.tensor(dims_of(len(marks), s.head_dim), device="cuda")[m]
        kb = k.view(torch.bfloat16)
        kb[idx] = 0
        kb[idx, :, dims] = 544.0
        return kb.view(torch.int16), None

    sc = DeviceScenario(wl, kv, longest)
    full = [l for l, s in enumerate(wl.layers) if s.k_eq_v]
    for l in full:
        sc.store(l, np.zeros_like(kv), kv, make_rows=make)
    b = longest[0]
    for l in full:
        s = wl.layers[l]
        qv = np.zeros((sc.B, s.num_q_heads, s.head_dim), dtype=np.float32)
        for m, dm in enumerate(dims_of(len(marks), s.head_dim)):
            if marks[m] < kv[b]:
                qv[:, :, dm] = 1.0
        from workloads import bf16_from_f32
        qb = bf16_from_f32(qv)
        q = torch.from_numpy(qb.view(np.int16)).cuda()
        got = host_bits(sc.cache.decode(l, i32(kv), q, int(kv.max())))
        torch.cuda.synchronize()
        pos, k, v = sc.rows(l, b)
        ref = attend(bf16_to_f32(qb[b:b + 1]).astype(np.float64), np.array([kv[b] - 1]), k, v, pos, 0,
                     s.sm_scale)[0]
        assert ref.max() > 1.0                       # the planted keys carry the output
        assert_close(got[b], ref, f"26B full layer {l} seq {b} (L {kv[b]}): planted keys", report=True)
