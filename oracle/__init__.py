"""Plain CPU oracle for paged KV-cache attention with per-layer mask regimes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
anything in this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library (no
kernels, headers, helpers, tables or constants); the only module both sides
use is ``workloads``, which draws seeded synthetic inputs and holds none of the
method's arithmetic.

What it computes, and the pages each part follows:

* ``layers``    -- which layer owns a KV slab and which layer a KV-shared layer
                   reads (FreeToken PR #898, description: the (layer, source)
                   list and the pool's owner-only slabs), and the KV bytes per
                   token that follow from it (same PR, "End to end").
* ``int8_pth``  -- the int8 per-token-head KV encoding (same PR, description
                   bullet on the per-token-head formats; the 4-byte scale is
                   fixed by the bytes-per-token figures in "End to end").  The
                   rounding and the clamp are this oracle's reading; the pages
                   do not print them.
* ``fp8_pth``   -- the fp8 per-token-head sibling format (same bullet; same
                   D + 4 bytes per row): E4M3 codes, scale amax / 448, round
                   to nearest even, saturating (this oracle's reading).
* ``attention`` -- dense attention in float64 over an explicitly materialised
                   visibility mask (full causal, or causal and inside a window
                   of W positions that counts the query's own position),
                   unsloth commit ca9dbce (the block-mask-per-regime change)
                   and pegainfer issue #807 (Description: the window_left
                   conversion).
* ``cache``     -- logical, position-ordered K/V arrays per owning layer and
                   sequence: what a paged cache holds, without pages; K=V
                   layers (value = RMS-normalised key, unsloth commit 749fb75)
                   and extend chunks given as packed rows (FreeToken PR #898,
                   description, fourth bullet).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms, brute force and a library
routine; none is "parity unpinned".
"""

from .attention import visibility_mask, attend, decode_positions, extend_positions
from .int8_pth import quantise_rows, dequantise_rows
from . import fp8_pth
from .fp8_pth import e4m3_encode, e4m3_value
from .layers import kv_sources, owner_layers, kv_bytes_per_token, AliasError
from .cache import LogicalCache, v_from_k

__all__ = [
    "visibility_mask", "attend", "decode_positions", "extend_positions",
    "quantise_rows", "dequantise_rows", "fp8_pth", "e4m3_encode", "e4m3_value", "v_from_k",
    "kv_sources", "owner_layers", "kv_bytes_per_token", "AliasError",
    "LogicalCache",
]
