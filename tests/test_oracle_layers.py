"""Pins for oracle.layers against integer facts the pages print.

Fixtures: tests/golden/freetoken_pr898_*.txt (FreeToken PR #898).  The layer
patterns (full iff l % 5 == 4 on the 35-layer E2B stack, l % 6 == 5 on the
42-layer E4B stack), Hkv (1 / 2) and the head dims (512 full / 256 sliding) are
readings; the pins check that these readings reproduce every printed figure.
"""

import os
from fractions import Fraction

import pytest

from oracle import kv_sources, owner_layers, kv_bytes_per_token, AliasError
from workloads import e2b_layer_types, e4b_layer_types

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MODELS = {
    "E2B": dict(types=e2b_layer_types(), first_shared=15,
                head_dim={"full": 512, "sliding": 256}, kv_heads={"full": 1, "sliding": 1}),
    "E4B": dict(types=e4b_layer_types(), first_shared=24,
                head_dim={"full": 512, "sliding": 256}, kv_heads={"full": 2, "sliding": 2}),
}


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                out.append(line)
    return out


def _facts():
    facts = {}
    for row in _rows("freetoken_pr898_sharing.txt"):
        facts[(row[0], row[1])] = [int(x) for x in row[2:]]
    return facts


@pytest.mark.parametrize("row", _rows("freetoken_pr898_unit_bytes.txt"), ids=lambda r: "-".join(r[:3]))
def test_bytes_per_token_match_printed_unit_bytes(row):
    model, fmt, arm, full, window = row[0], row[1], row[2], int(row[3]), int(row[4])
    m = MODELS[model]
    got = kv_bytes_per_token(m["types"], m["first_shared"], m["head_dim"], m["kv_heads"],
                             fmt=fmt, share=(arm == "shared"))
    assert got == (full, window)


@pytest.mark.parametrize("model", ["E2B", "E4B"])
def test_sources_are_last_earlier_layer_of_same_type(model):
    m = MODELS[model]
    facts = _facts()
    src = kv_sources(m["types"], m["first_shared"])
    want_full, want_sliding = facts[("source", model)]
    for layer in range(m["first_shared"], len(m["types"])):
        want = want_full if m["types"][layer] == "full" else want_sliding
        assert src[layer] == want
    for layer in range(m["first_shared"]):
        assert src[layer] == layer
    assert len(m["types"]) - m["first_shared"] == facts[("shared_layers", model)][0]


@pytest.mark.parametrize("model", ["E2B", "E4B"])
def test_slab_counts_with_and_without_sharing(model):
    m = MODELS[model]
    facts = _facts()
    types = m["types"]
    main = owner_layers(types, m["first_shared"], share=False)
    assert [sum(types[l] == "full" for l in main), sum(types[l] == "sliding" for l in main)] == \
        facts[("main_slabs", model)]
    own = owner_layers(types, m["first_shared"], share=True)
    n_full = sum(types[l] == "full" for l in own)
    n_sliding = sum(types[l] == "sliding" for l in own)
    # every shared layer's source is an owner, and there are no other owners
    src = kv_sources(types, m["first_shared"])
    assert set(src) == set(own)
    assert n_full + n_sliding == m["first_shared"]


@pytest.mark.parametrize("model", ["E2B", "E4B"])
def test_shared_fraction_and_capacity_gain(model):
    m = MODELS[model]
    facts = _facts()
    main = sum(kv_bytes_per_token(m["types"], m["first_shared"], m["head_dim"], m["kv_heads"], share=False))
    shared = sum(kv_bytes_per_token(m["types"], m["first_shared"], m["head_dim"], m["kv_heads"], share=True))
    assert round(100 * (main - shared) / main) == facts[("shared_pct", model)][0]
    num, den = facts[("gain", model)]
    assert Fraction(main, shared) == Fraction(num, den)


def test_hand_worked_source_rule():
    # types:   0:s 1:f 2:s 3:s | 4:f 5:s 6:f   (shared from 4)
    types = ["sliding", "full", "sliding", "sliding", "full", "sliding", "full"]
    assert kv_sources(types, 4) == [0, 1, 2, 3, 1, 3, 1]
    assert kv_sources(types, None) == list(range(7))


def test_unsourced_shared_layer_is_refused():
    with pytest.raises(AliasError):
        kv_sources(["sliding", "sliding", "full"], 2)
    with pytest.raises(AliasError):
        kv_sources(["full", "sliding"], 0)
