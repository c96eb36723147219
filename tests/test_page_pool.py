"""Page pools (host bookkeeping, no GPU) and the capacity arithmetic.

* A window pool keeps, for a sequence whose next queries start at position p,
  the pages holding positions p - W + 1 onwards, and gives the rest back
  (pegainfer issue #807, Description, first paragraph: the sliding group
  releases pages the full group still reads); a full pool keeps everything.
  Released pages are handed out again, last released first; a reservation the
  pool cannot meet changes nothing.
* Capacity (FreeToken PR #898, "End to end", the capacity table): every
  printed window pool holds one token per five of its full pool; with that
  share, the bytes per token of the owning layers give exactly 7/3 (E2B) and
  7/4 (E4B) more tokens after sharing, the printed gains lie a little above
  (the page: the window pool's fixed floor shrinks too), and each printed arm's
  own budget gives back its printed pools to one token; the printed gains
  are within 3 % above 7/3 and 7/4.
"""

import os

import numpy as np
import pytest

from full_attention_amd import pakv
from workloads import e2b_layer_types, e4b_layer_types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_window_pool_keeps_only_what_later_queries_see():
    pool = pakv.PagePool(num_pages=12, max_seqs=2, max_pages_per_seq=20, window=40)
    pool.reserve(0, 0, 100)               # prefill of 100 tokens: first query at 0 -> keep all 7 pages
    t = pool.table()
    assert (t[0, :7] >= 0).all() and (t[0, 7:] == -1).all()
    assert pool.free_pages() == 5
    # decode at kv_len 101: query at 100 sees 61..100 -> pages 3.. kept, 0..2 released
    pool.reserve(0, 100, 101)
    t = pool.table()
    assert (t[0, :3] == -1).all() and (t[0, 3:7] >= 0).all()
    released = pool.released()
    assert len(released) == 3 and pool.free_pages() == 8
    # the next sequence gets the last released page first
    pool.reserve(1, 0, 16)
    assert pool.table()[1, 0] == released[-1]
    # a query at 200 (keys 161..) and end 220: pages 10..13 held, everything below given back
    pool.reserve(0, 200, 220)
    t = pool.table()
    assert (t[0, :10] == -1).all() and (t[0, 10:14] >= 0).all() and (t[0, 14:] == -1).all()
    # every held page is distinct
    held = t[t >= 0]
    assert len(set(held.tolist())) == len(held)
    pool.release_seq(0)
    assert (pool.table()[0] == -1).all() and pool.free_pages() == 11


def test_full_pool_keeps_everything_and_refuses_without_change():
    pool = pakv.PagePool(num_pages=5, max_seqs=2, max_pages_per_seq=8, window=0)
    pool.reserve(0, 60, 64)
    before = pool.table()
    assert (before[0, :4] >= 0).all()
    with pytest.raises(pakv.PakvError) as e:
        pool.reserve(1, 0, 40)            # 3 pages needed, 1 free
    assert e.value.status == pakv.ERR_WORKSPACE
    assert np.array_equal(pool.table(), before) and pool.free_pages() == 1
    with pytest.raises(pakv.PakvError):
        pool.reserve(0, 10, 5)            # first query past the end
    with pytest.raises(pakv.PakvError):
        pool.reserve(2, 0, 5)             # no such sequence


def _rows():
    out = []
    for line in open(os.path.join(ROOT, "tests", "golden", "freetoken_pr898_capacity.txt")):
        line = line.split("#", 1)[0].split()
        if line:
            out.append(line)
    return out


@pytest.mark.parametrize("row", _rows(), ids=lambda r: "-".join(r[:2]))
def test_printed_window_pools_hold_a_fifth_of_the_full_pool(row):
    mf, mw, pf, pw = (int(x) for x in row[2:6])
    assert abs(mw / mf - 0.2) < 1e-4 and abs(pw / pf - 0.2) < 1e-4
    assert round(pf / mf, 2) == float(row[6])


def _map(name, fmt, share):
    types = e2b_layer_types() if name == "E2B" else e4b_layer_types()
    first = 15 if name == "E2B" else 24
    hkv = 1 if name == "E2B" else 2
    tags = [1 if t == "full" else 0 for t in types]
    src = pakv.resolve_kv_sources(tags, first if share else len(types))
    dtype = pakv.KV_BF16 if fmt == "bf16" else pakv.KV_INT8_PTH
    descs = []
    for l, t in enumerate(types):
        d, w = (512, 0) if t == "full" else (256, 512)
        descs.append(pakv.LayerDesc(d, 8, hkv, w, -1 if src[l] == l else src[l], dtype, 1.0 / np.sqrt(d)))
    return pakv.LayerMap(descs)


@pytest.mark.parametrize("row", [r for r in _rows() if "draft" not in r[1]], ids=lambda r: "-".join(r[:2]))
def test_capacity_arithmetic_against_the_printed_table(row):
    name, setup = row[0], row[1]
    fmt = "int8" if setup == "int8" else "bf16"
    main, shared = _map(name, fmt, False), _map(name, fmt, True)
    mf, mw, pf, pw = (int(x) for x in row[2:6])
    # each arm's own budget (its printed pools times its bytes per token) gives
    # its printed pools back
    for m, f, w in ((main, mf, mw), (shared, pf, pw)):
        fb, wb = m.kv_bytes_per_token()
        budget = f * fb + w * wb
        full, window = pakv.pool_tokens(m, budget, 0.2)
        assert abs(full - f) <= 1 and abs(window - w) <= 1, (full, f, window, w)
    # on one budget, sharing gives exactly 7/3 (E2B) or 7/4 (E4B) more tokens
    budget = 10 ** 13
    gain = pakv.pool_tokens(shared, budget, 0.2)[0] / pakv.pool_tokens(main, budget, 0.2)[0]
    want = 7 / 3 if name == "E2B" else 7 / 4
    assert abs(gain - want) < 1e-6
    # the printed gain lies a little above it
    assert want <= pf / mf <= want * 1.03
