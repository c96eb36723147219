"""Logical KV cache (test infrastructure only).

Per owning layer and sequence, the K/V rows a paged cache would hold, kept in
position order with no pages.  A KV-shared layer stores nothing and reads its
source's rows (FreeToken PR #898, description: the store returns early for a
shared layer because its source already stored the same rows; reads go through
the one layer mapping, scales included).

Layers whose values are their own keys, RMS-normalised without a learned
scale (unsloth commit 749fb75: attention_k_eq_v on the full layers, the value
being the key projection followed only by a scale-free v_norm), store K alone;
their value row is v = k / sqrt(mean_d k_d^2 + eps), computed here in float64
from the stored key row (dequantised first for 8-bit formats).  eps comes with
the layer ("v_norm_eps"; Gemma's RMS norms use 1e-6); the pages do not print
it.

An extend chunk may also come as packed rows beside the cache (FreeToken PR
#898, description, fourth bullet: the extend kernel takes the current chunk
from k_extend / v_extend): ``extend_packed`` attends the stored rows before
the chunk plus the given chunk rows, taken exactly as given (bf16), whatever
format the cache stores.
"""

import numpy as np

from .attention import attend, decode_positions, extend_positions
from . import int8_pth, fp8_pth
from .layers import kv_sources

_CODECS = {"int8": int8_pth, "fp8": fp8_pth}


def v_from_k(k, eps):
    """Value rows of a K=V layer: each key row divided by its root mean square
    (plus eps under the root), in float64."""
    k = np.asarray(k, dtype=np.float64)
    return k / np.sqrt(np.mean(k * k, axis=-1, keepdims=True) + eps)


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

    def _k_eq_v(self, layer):
        return bool(self.layers[self.sources[layer]].get("k_eq_v", False))

    def store(self, layer, seq, start_pos, k_bits, v_bits):
        """Write rows k_bits[i], v_bits[i] ([T, Hkv, D] bf16 bit patterns) at
        positions start_pos + i.  A shared layer stores nothing; a K=V layer
        keeps the key rows only (v_bits may be None)."""
        if self.sources[layer] != layer:
            return
        desc = self.layers[layer]
        k = bf16_bits_to_f32(k_bits)
        v = None if self._k_eq_v(layer) else bf16_bits_to_f32(v_bits)
        slot = self._rows.setdefault((layer, seq), {})
        if desc["kv_dtype"] in _CODECS:
            codec = _CODECS[desc["kv_dtype"]]
            kq, ks = codec.quantise_rows(k)
            vq, vs = codec.quantise_rows(v) if v is not None else (None, None)
            for i in range(k.shape[0]):
                slot[start_pos + i] = (kq[i], None if v is None else vq[i], ks[i], None if v is None else vs[i])
        else:
            for i in range(k.shape[0]):
                slot[start_pos + i] = (k[i], None if v is None else v[i], None, None)

    def stored(self, layer, seq):
        """(positions, rows) of the slab a layer reads: codes and scales for
        int8, float32 rows for bf16."""
        slot = self._rows.get((self.sources[layer], seq), {})
        pos = np.array(sorted(slot), dtype=np.int64)
        return pos, [slot[p] for p in pos]

    def values(self, layer, seq):
        """(kv_pos, k, v) in float64: exact bf16 values, or the decoded codes;
        for a K=V layer v is derived from k."""
        pos, rows = self.stored(layer, seq)
        if not rows:
            raise ValueError("nothing stored for this layer and sequence")
        desc = self.layers[self.sources[layer]]
        kve = self._k_eq_v(layer)
        if rows[0][2] is None:
            k = np.stack([r[0] for r in rows]).astype(np.float64)
            v = None if kve else np.stack([r[1] for r in rows]).astype(np.float64)
        else:
            codec = _CODECS[desc["kv_dtype"]]
            k = codec.dequantise_rows(np.stack([r[0] for r in rows]), np.stack([r[2] for r in rows]))
            v = None if kve else codec.dequantise_rows(np.stack([r[1] for r in rows]), np.stack([r[3] for r in rows]))
        if kve:
            v = v_from_k(k, desc.get("v_norm_eps", 1e-6))
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

    def extend_packed(self, layer, seq, q_bits, prefix_len, k_bits, v_bits):
        """A chunk of queries at positions prefix_len + i whose own key / value
        rows are given ([n, Hkv, D] bf16 bits; v_bits None for a K=V layer)
        rather than stored: the stored rows below prefix_len, then the chunk's
        rows exactly as given.  q_bits: [n, Hq, D] -> [n, Hq, D] float64."""
        desc = self.layers[layer]
        n = q_bits.shape[0]
        src = self.layers[self.sources[layer]]
        try:
            pos, k, v = self.values(layer, seq)
            keep = pos < prefix_len
            pos, k, v = pos[keep], k[keep], v[keep]
        except ValueError:                     # nothing stored yet: an empty prefix
            d, hkv = src["head_dim"], src["num_kv_heads"]
            pos, k, v = np.zeros(0, np.int64), np.zeros((0, hkv, d)), np.zeros((0, hkv, d))
        kc = bf16_bits_to_f32(k_bits).astype(np.float64)
        if self._k_eq_v(layer):
            vc = v_from_k(kc, src.get("v_norm_eps", 1e-6))
        else:
            vc = bf16_bits_to_f32(v_bits).astype(np.float64)
        pos = np.concatenate([pos, extend_positions(prefix_len, n)])
        k = np.concatenate([k, kc])
        v = np.concatenate([v, vc])
        q = bf16_bits_to_f32(q_bits)
        return attend(q, extend_positions(prefix_len, n), k, v, pos, desc["window"], desc["sm_scale"])
