"""Logical KV cache (test infrastructure only).

Per owning layer and sequence, the K/V rows a paged cache would hold, kept in
position order with no pages.  A KV-shared layer stores nothing and reads its
source's rows (FreeToken PR #898, description: the store returns early for a
shared layer because its source already stored the same rows; reads go through
the one layer mapping, scales included).
"""

import numpy as np

from .attention import attend, decode_positions, extend_positions
from .int8_pth import quantise_rows, dequantise_rows
from .layers import kv_sources


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32, exact: the bf16 bits are the top
    half of the float32 word."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


class LogicalCache:
    """layers: list of dicts with keys type ("full"/"sliding"), head_dim,
    num_q_heads, num_kv_heads, window, kv_dtype ("bf16"/"int8"), sm_scale.
    first_shared: index of the first KV-shared layer (None: no sharing)."""

    def __init__(self, layers, first_shared, num_seqs):
        self.layers = layers
        self.sources = kv_sources([l["type"] for l in layers], first_shared)
        self.num_seqs = num_seqs
        # (owner, seq) -> {pos: (k_row, v_row, k_scale, v_scale)}
        self._rows = {}

    def source(self, layer):
        return self.sources[layer]

    def store(self, layer, seq, start_pos, k_bits, v_bits):
        """Write rows k_bits[i], v_bits[i] ([T, Hkv, D] bf16 bit patterns) at
        positions start_pos + i.  A shared layer stores nothing."""
        if self.sources[layer] != layer:
            return
        desc = self.layers[layer]
        k = bf16_bits_to_f32(k_bits)
        v = bf16_bits_to_f32(v_bits)
        slot = self._rows.setdefault((layer, seq), {})
        if desc["kv_dtype"] == "int8":
            kq, ks = quantise_rows(k)
            vq, vs = quantise_rows(v)
            for i in range(k.shape[0]):
                slot[start_pos + i] = (kq[i], vq[i], ks[i], vs[i])
        else:
            for i in range(k.shape[0]):
                slot[start_pos + i] = (k[i], v[i], None, None)

    def stored(self, layer, seq):
        """(positions, rows) of the slab a layer reads: codes and scales for
        int8, float32 rows for bf16."""
        slot = self._rows.get((self.sources[layer], seq), {})
        pos = np.array(sorted(slot), dtype=np.int64)
        return pos, [slot[p] for p in pos]

    def values(self, layer, seq):
        """(kv_pos, k, v) in float64: exact bf16 values, or code * scale."""
        pos, rows = self.stored(layer, seq)
        if not rows:
            raise ValueError("nothing stored for this layer and sequence")
        if rows[0][2] is None:
            k = np.stack([r[0] for r in rows]).astype(np.float64)
            v = np.stack([r[1] for r in rows]).astype(np.float64)
        else:
            k = dequantise_rows(np.stack([r[0] for r in rows]), np.stack([r[2] for r in rows]))
            v = dequantise_rows(np.stack([r[1] for r in rows]), np.stack([r[3] for r in rows]))
        return pos, k, v

    def decode(self, layer, seq, q_bits, kv_len):
        """One decode query per sequence at position kv_len - 1.
        q_bits: [Hq, D] bf16 bits -> [Hq, D] float64."""
        desc = self.layers[layer]
        pos, k, v = self.values(layer, seq)
        keep = pos < kv_len
        q = bf16_bits_to_f32(q_bits)[None]
        out = attend(q, decode_positions(kv_len), k[keep], v[keep], pos[keep],
                     desc["window"], desc["sm_scale"])
        return out[0]

    def extend(self, layer, seq, q_bits, prefix_len):
        """A chunk of queries at positions prefix_len + i.
        q_bits: [n, Hq, D] bf16 bits -> [n, Hq, D] float64."""
        desc = self.layers[layer]
        n = q_bits.shape[0]
        pos, k, v = self.values(layer, seq)
        keep = pos < prefix_len + n
        q = bf16_bits_to_f32(q_bits)
        return attend(q, extend_positions(prefix_len, n), k[keep], v[keep], pos[keep],
                      desc["window"], desc["sm_scale"])
