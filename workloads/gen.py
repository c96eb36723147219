"""Random draws and page pools.

* Values are N(0, 1) float32 draws from numpy's PCG64, rounded to bf16 with
  round-to-nearest-even; they travel as uint16 bit patterns.
* A page pool holds ceil(capacity_b / 16) pages per sequence plus spare pages
  that no sequence owns (canaries).  Physical page ids are a seeded
  permutation of the pool; sequence b takes the next ceil(capacity_b / 16)
  ids in order.  Every layer uses the same page table.
"""

from dataclasses import dataclass

import numpy as np

PAGE_SIZE = 16


def bf16_from_f32(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even.
    NaN maps to the quiet NaN 0x7FC0."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), rounded).astype(np.uint16)


def bf16_to_f32(bits):
    """bf16 bit patterns -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def normal_bf16(rng, shape):
    """N(0, 1) float32 draws rounded to bf16, as uint16 bits."""
    return bf16_from_f32(rng.standard_normal(shape, dtype=np.float32))


def rms_normalise_bf16(k_bits, eps=1e-6):
    """Value rows of a layer whose V is its RMS-normalised K without a learned
    scale: v = bf16(k / sqrt(mean_d k^2 + eps)), computed in float64 from the
    bf16 k rows.  eps is not on the pages; at D = 512 with N(0, 1) rows it
    moves nothing."""
    k = bf16_to_f32(k_bits).astype(np.float64)
    r = np.sqrt(np.mean(k * k, axis=-1, keepdims=True) + eps)
    return bf16_from_f32((k / r).astype(np.float32))


@dataclass
class PagePool:
    page_table: np.ndarray     # int32 [B, max_pages_per_seq]; -1 past a sequence's pages
    num_pages: int             # pool size, spare pages included
    pages_per_seq: np.ndarray  # int64 [B]
    spare_pages: np.ndarray    # ids no sequence owns


def make_page_pool(rng, capacities, spare=4):
    """capacities[b] = largest number of positions sequence b will hold."""
    caps = np.asarray(capacities, dtype=np.int64)
    per_seq = (caps + PAGE_SIZE - 1) // PAGE_SIZE
    used = int(per_seq.sum())
    total = used + spare
    perm = rng.permutation(total).astype(np.int32)
    max_pages = max(1, int(per_seq.max()) if len(per_seq) else 1)
    table = np.full((len(caps), max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(per_seq):
        table[b, :n] = perm[off:off + n]
        off += n
    return PagePool(table, total, per_seq, perm[used:])
