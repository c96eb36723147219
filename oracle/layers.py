"""KV-slab ownership and KV-source resolution (test infrastructure only).

Rules followed (FreeToken PR #898, "perf(gemma4): read the source layer's kv
slab on kv-shared layers"):

* Description, first bullet: every KV-shared layer reads the last layer before
  the shared block that has the same attention type; a shared layer with no
  such earlier layer is refused (the review asks for a NotImplementedError,
  and the author's reply confirms it went in).
* Description, third bullet: the pool allocates slabs, and the cost model
  prices bytes, only for layers that own KV.
* "End to end": bytes per token are the sum over owning layers of
  Hkv * 2 (K and V) * row bytes, row = 2*D for bf16 and D + 4 for the 8-bit
  per-token-head formats (D codes and one 4-byte scale).
"""


class AliasError(ValueError):
    """A KV-shared layer has no earlier layer of its attention type."""


def kv_sources(layer_types, first_shared):
    """Source layer of every layer: itself for an owner (index < first_shared),
    else the last owner with the same attention type."""
    n = len(layer_types)
    if first_shared is None or first_shared >= n:
        return list(range(n))
    out = []
    for layer, kind in enumerate(layer_types):
        if layer < first_shared:
            out.append(layer)
            continue
        earlier = [i for i in range(first_shared) if layer_types[i] == kind]
        if not earlier:
            raise AliasError(f"layer {layer} ({kind}) has no earlier layer of its type")
        out.append(max(earlier))
    return out


def owner_layers(layer_types, first_shared, share=True):
    """Layers that own a slab: all of them when sharing is off (every layer
    stores its own copy), else those below first_shared."""
    if not share or first_shared is None:
        return list(range(len(layer_types)))
    return [l for l in range(len(layer_types)) if l < first_shared]


def kv_bytes_per_token(layer_types, first_shared, head_dim, kv_heads, fmt="bf16", share=True):
    """(full_bytes, window_bytes) per token over owning layers.

    head_dim / kv_heads map an attention type ("full" or "sliding") to D / Hkv.
    fmt is "bf16", or "int8" / "fp8" (8-bit codes and one 4-byte scale per
    token-head row).
    """
    totals = {"full": 0, "sliding": 0}
    for layer in owner_layers(layer_types, first_shared, share):
        kind = layer_types[layer]
        d = head_dim[kind]
        row = 2 * d if fmt == "bf16" else d + 4
        totals[kind] += kv_heads[kind] * 2 * row
    return totals["full"], totals["sliding"]
