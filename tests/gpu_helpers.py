"""Shared helpers for the GPU parity tests (imported only by tests marked gpu).

The oracle gets its inputs from the same seeded generators as the GPU path
(workloads); nothing read back from the GPU is ever fed to the oracle.  Slab
bytes read back from the GPU are only compared, through an independent host
page walk that follows the layout documented in include/pakv.h.
"""

import numpy as np
import pytest
import torch

from oracle import LogicalCache
from workloads import PAGE_SIZE, bf16_to_f32, make_page_pool, normal_bf16, rms_normalise_bf16

ATOL = 2e-2
RTOL = 1e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from full_attention_amd import pakv  # noqa: F401  (fails loudly if the library is missing)


def dev_bits(bits):
    """uint16 numpy bf16 bits -> int16 cuda tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host_bits(t):
    return t.cpu().numpy().view(np.uint16)


def i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), dtype=torch.int32).cuda()


def error_stats(gpu_bits, ref):
    """(max abs err, RMS(err) / RMS(ref)) of bf16 outputs against float64."""
    got = bf16_to_f32(gpu_bits).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = got - ref
    rms_ref = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    rel = float(np.sqrt(np.mean(err * err)) / rms_ref) if rms_ref > 0 else float("nan")
    return float(np.abs(err).max()) if err.size else 0.0, rel


def assert_close(gpu_bits, ref, what="", report=False):
    """Elementwise |gpu - ref| <= ATOL + RTOL * |ref| (bf16 outputs vs float64).
    report: print the max abs error and RMS(err) / RMS(ref)."""
    got = bf16_to_f32(gpu_bits).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; "
                           f"max abs err {err.max():.3e}")
    if report:
        mx, rel = error_stats(gpu_bits, ref)
        print(f"[parity] {what}: max abs err {mx:.3e}, RMS(err)/RMS(ref) {rel:.3e}, "
              f"RMS(ref) {np.sqrt(np.mean(ref * ref)):.3e}", flush=True)
    return float(err.max())


def page_walk_k(k_slab, page_table, b, pos, head):
    """K row of (sequence b, position pos, KV head) from a host copy of the slab
    [num_pages][Hkv][16][D]."""
    page = page_table[b, pos // PAGE_SIZE]
    return k_slab[page, head, pos % PAGE_SIZE, :]


def page_walk_v(v_slab, page_table, b, pos, head):
    """V row from a host copy of a dim-major slab [num_pages][Hkv][D][16]."""
    page = page_table[b, pos // PAGE_SIZE]
    return v_slab[page, head, :, pos % PAGE_SIZE]


class Scenario:
    """Layers, a page pool and stored rows, mirrored on the GPU (through the
    library's store) and in the oracle's logical cache (from the same draws).

    rows_from[b] (optional): first position stored per sequence; positions
    below it are never written (they keep the NaN sentinel)."""

    def __init__(self, specs, first_shared, capacities, seed, spare=4):
        from full_attention_amd.cache import PagedKVCache
        self.rng = np.random.default_rng(seed)
        self.specs = specs
        self.first_shared = first_shared
        self.capacities = list(capacities)
        self.B = len(capacities)
        self.pool = make_page_pool(self.rng, capacities, spare=spare)
        self.cache = PagedKVCache(specs, first_shared, self.pool.num_pages)
        self.cache.set_page_table(self.pool.page_table)
        self.oracle = LogicalCache([s.as_dict() for s in specs], first_shared, self.B)
        self.rows = {}

    def store(self, layer, starts, counts):
        """Draw and store counts[b] rows at positions starts[b].. for every sequence
        (on every layer, shared ones included: a shared layer's store is a no-op on
        both sides)."""
        s = self.specs[layer]
        total = int(sum(counts))
        k = normal_bf16(self.rng, (total, s.num_kv_heads, s.head_dim))
        v = rms_normalise_bf16(k) if s.k_eq_v else normal_bf16(self.rng, (total, s.num_kv_heads, s.head_dim))
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        self.cache.store(layer, i32(cu), i32(starts), dev_bits(k), dev_bits(v))
        for b in range(self.B):
            if counts[b]:
                self.oracle.store(layer, b, int(starts[b]), k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]])
        self.rows[layer] = (k, v, cu, list(starts))
        return k, v

    def store_rows(self, layer, starts, counts, k, v):
        """Stores given rows (uint16 bf16 bits [T, Hkv, D]) on both sides."""
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        self.cache.store(layer, i32(cu), i32(starts), dev_bits(k), dev_bits(v))
        for b in range(self.B):
            if counts[b]:
                self.oracle.store(layer, b, int(starts[b]), k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]])
        self.rows[layer] = (k, v, cu, list(starts))

    def decode(self, layer, kv_lens, seqs=None):
        s = self.specs[layer]
        q = normal_bf16(self.rng, (self.B, s.num_q_heads, s.head_dim))
        out = self.cache.decode(layer, i32(kv_lens), dev_bits(q), int(max(kv_lens)))
        torch.cuda.synchronize()
        got = host_bits(out)
        seqs = range(self.B) if seqs is None else seqs
        ref = np.stack([self.oracle.decode(layer, b, q[b], int(kv_lens[b])) for b in seqs])
        return got[list(seqs)], ref, q

    def extend(self, layer, prefixes, chunks, seqs=None, q=None):
        s = self.specs[layer]
        total = int(sum(chunks))
        if q is None:
            q = normal_bf16(self.rng, (max(total, 1), s.num_q_heads, s.head_dim))[:total]
        cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
        max_kv = int(max(p + n for p, n in zip(prefixes, chunks)))
        out = self.cache.extend(layer, i32(cu), i32(prefixes), dev_bits(q), int(max(chunks)), max_kv)
        torch.cuda.synchronize()
        got = host_bits(out)
        seqs = range(self.B) if seqs is None else seqs
        pairs = []
        for b in seqs:
            if chunks[b] == 0:
                continue
            ref = self.oracle.extend(layer, b, q[cu[b]:cu[b + 1]], int(prefixes[b]))
            pairs.append((got[cu[b]:cu[b + 1]], ref, b))
        return pairs
