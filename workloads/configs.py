"""The five synthetic workloads, by shape.

Layer-type patterns are not printed on the pages.  For an E2B-like stack
(35 layers, 7 full and 28 sliding, shared from layer 15) the only period that
gives sources 14 / 13 and 3 + 12 owning slabs is "full iff l % 5 == 4"; for
an E4B-like stack (42 layers, shared from layer 24) it is "full iff
l % 6 == 5" (sources 23 / 22, 4 + 20 owners).  The 26B-A4B-like stack
(25 sliding, 5 full, no sharing) uses the same period of 6.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


# eps of the value norm of K=V layers (Gemma's RMS norms use 1e-6; the pages
# do not print it)
V_NORM_EPS = 1e-6


@dataclass
class LayerSpec:
    type: str            # "full" or "sliding"
    head_dim: int
    num_q_heads: int
    num_kv_heads: int
    window: int          # 0 for full layers
    kv_dtype: str = "bf16"   # "bf16", "int8" or "fp8"
    k_eq_v: bool = False     # value rows are the RMS-normalised key rows

    @property
    def sm_scale(self):
        return 1.0 / float(np.sqrt(self.head_dim))

    def as_dict(self):
        return dict(type=self.type, head_dim=self.head_dim, num_q_heads=self.num_q_heads,
                    num_kv_heads=self.num_kv_heads, window=self.window,
                    kv_dtype=self.kv_dtype, sm_scale=self.sm_scale, k_eq_v=self.k_eq_v,
                    v_norm_eps=V_NORM_EPS)


@dataclass
class Workload:
    name: str
    seed: int
    layers: List[LayerSpec]
    first_shared: Optional[int]
    kind: str                       # "decode", "extend", "decode+extend"
    cached_lens: List[int] = field(default_factory=list)     # L_b before the step
    extend_lens: List[int] = field(default_factory=list)     # n_b for extend
    notes: str = ""

    @property
    def layer_types(self):
        return [l.type for l in self.layers]

    @property
    def num_seqs(self):
        return len(self.cached_lens)


def e2b_layer_types():
    return ["full" if l % 5 == 4 else "sliding" for l in range(35)]


def e4b_layer_types():
    return ["full" if l % 6 == 5 else "sliding" for l in range(42)]


def _e2b_layers(window=512):
    out = []
    for t in e2b_layer_types():
        if t == "full":
            out.append(LayerSpec("full", 512, 8, 1, 0))
        else:
            out.append(LayerSpec("sliding", 256, 8, 1, window))
    return out


def tiny_workload():
    """2 sequences cached to 100 and 37; Hq 8, Hkv 1, D 256; one sliding layer
    (W 32) and one full layer, both owners; one decode token per sequence,
    then a 64-token extend chunk on sequence 0."""
    layers = [LayerSpec("sliding", 256, 8, 1, 32), LayerSpec("full", 256, 8, 1, 0)]
    return Workload("tiny decode+extend", 1001, layers, None, "decode+extend",
                    cached_lens=[100, 37], extend_lens=[64, 0])


def e2b_decode_workload(batch=64, lo=512, hi=4096):
    rng = np.random.default_rng(1002)
    lens = rng.integers(lo, hi + 1, size=batch).tolist()
    return Workload("E2B-like decode, 35 layers, batch 64", 1002, _e2b_layers(), 15,
                    "decode", cached_lens=lens)


def e2b_extend_workload(prefixes=(0, 1024, 2048, 4096), chunk=2048):
    return Workload("E2B-like extend, 4 x 2048-token chunks", 1003, _e2b_layers(), 15,
                    "extend", cached_lens=list(prefixes), extend_lens=[chunk] * len(prefixes))


def moe26b_decode_workload(batch=48, lo=2048, hi=16384):
    rng = np.random.default_rng(1004)
    lens = rng.integers(lo, hi + 1, size=batch).tolist()
    layers = []
    for l in range(30):
        if l % 6 == 5:
            layers.append(LayerSpec("full", 512, 16, 2, 0, k_eq_v=True))
        else:
            layers.append(LayerSpec("sliding", 256, 16, 8, 1024))
    return Workload("26B-A4B-like decode, 30 layers, batch 48", 1004, layers, None,
                    "decode", cached_lens=lens)


def int8_long_workload(batch=8, length=131072):
    layers = [LayerSpec("full", 512, 8, 1, 0, kv_dtype="int8"),
              LayerSpec("sliding", 256, 8, 1, 1024, kv_dtype="int8")]
    return Workload("int8 long-context decode, batch 8 x 131072", 1005, layers, None,
                    "decode", cached_lens=[length] * batch)


WORKLOADS = {
    1: tiny_workload,
    2: e2b_decode_workload,
    3: e2b_extend_workload,
    4: moe26b_decode_workload,
    5: int8_long_workload,
}
