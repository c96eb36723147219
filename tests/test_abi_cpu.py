"""Host-side checks of libpakv.so that need no GPU: every symbol the header
declares is exported, the layer-map rules, the bytes-per-token figures the
pages print (FreeToken PR #898, "End to end"), and argument errors that are
returned before anything is launched."""

import ctypes
import os
import re
import subprocess

import pytest

from full_attention_amd import pakv
from workloads import e2b_layer_types, e4b_layer_types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "pakv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pakv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_symbols()
    for required in ("pakv_paged_kv_store", "pakv_paged_attn_decode", "pakv_paged_attn_extend",
                     "pakv_layer_map_create", "pakv_resolve_kv_sources"):
        assert required in names


@pytest.mark.parametrize("name", declared_symbols())
def test_every_declared_symbol_is_exported(name):
    assert hasattr(pakv.lib, name)
    assert name in pakv.EXPORTED


def _desc(d=256, hq=8, hkv=1, w=0, src=-1, dtype=pakv.KV_BF16, scale=0.0625):
    return pakv.LayerDesc(d, hq, hkv, w, src, dtype, scale)


def _model(name, fmt, share):
    types = e2b_layer_types() if name == "E2B" else e4b_layer_types()
    first = 15 if name == "E2B" else 24
    hkv = 1 if name == "E2B" else 2
    tags = [1 if t == "full" else 0 for t in types]
    src = pakv.resolve_kv_sources(tags, first if share else len(types))
    dtype = {"bf16": pakv.KV_BF16, "int8": pakv.KV_INT8_PTH, "fp8": pakv.KV_FP8_PTH}[fmt]
    descs = []
    for l, t in enumerate(types):
        d, w = (512, 0) if t == "full" else (256, 512)
        descs.append(_desc(d, 8, hkv, w, -1 if src[l] == l else src[l], dtype))
    return pakv.LayerMap(descs), src, types


def _golden_rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].split()
        if line:
            out.append(line)
    return out


@pytest.mark.parametrize("row", _golden_rows("freetoken_pr898_unit_bytes.txt"), ids=lambda r: "-".join(r[:3]))
def test_library_bytes_per_token_match_printed(row):
    m, _, _ = _model(row[0], row[1], row[2] == "shared")
    assert m.kv_bytes_per_token() == (int(row[3]), int(row[4]))


@pytest.mark.parametrize("model,full,sliding", [("E2B", 14, 13), ("E4B", 23, 22)])
def test_library_source_rule_matches_printed(model, full, sliding):
    m, src, types = _model(model, "bf16", True)
    first = 15 if model == "E2B" else 24
    for l, t in enumerate(types):
        want = l if l < first else (full if t == "full" else sliding)
        assert src[l] == want and m.source(l) == want


def test_unsourced_shared_layer_refused():
    with pytest.raises(pakv.PakvError) as e:
        pakv.resolve_kv_sources([0, 0, 1], 2)
    assert e.value.status == pakv.ERR_ALIAS
    assert "no earlier layer" in str(e.value)


@pytest.mark.parametrize("descs,status", [
    ([_desc(), _desc(src=2)], pakv.ERR_ALIAS),                        # source not earlier
    ([_desc(), _desc(src=0), _desc(src=1)], pakv.ERR_ALIAS),          # source itself shared
    ([_desc(d=256), _desc(d=512, src=0)], pakv.ERR_ALIAS),            # different head_dim
    ([_desc(w=32), _desc(w=0, src=0)], pakv.ERR_ALIAS),               # different window
    ([_desc(hkv=1), _desc(hkv=2, hq=8, src=0)], pakv.ERR_ALIAS),      # different Hkv
    ([_desc(), _desc(src=0, dtype=pakv.KV_INT8_PTH)], pakv.ERR_ALIAS),  # different dtype
    ([_desc(d=128)], pakv.ERR_UNSUPPORTED),
    ([_desc(hq=7, hkv=2)], pakv.ERR_INVALID),
    ([_desc(hq=32, hkv=1)], pakv.ERR_UNSUPPORTED),
    ([_desc(w=-1)], pakv.ERR_INVALID),
    ([_desc(scale=0.0)], pakv.ERR_INVALID),
    ([_desc(dtype=7)], pakv.ERR_INVALID),
])
def test_layer_map_rules(descs, status):
    with pytest.raises(pakv.PakvError) as e:
        pakv.LayerMap(descs)
    assert e.value.status == status


def test_shared_layer_cannot_own_a_slab():
    m = pakv.LayerMap([_desc(), _desc(src=0)])
    with pytest.raises(pakv.PakvError) as e:
        m.bind_slab(1, 0x1000, 0x2000, 4)
    assert e.value.status == pakv.ERR_ALIAS
    m.bind_slab(0, 0x1000, 0x2000, 4)        # host bookkeeping only; nothing is dereferenced
    with pytest.raises(pakv.PakvError):
        m.bind_slab(0, 0x1000, 0x2000, 0)
    m8 = pakv.LayerMap([_desc(dtype=pakv.KV_INT8_PTH)])
    with pytest.raises(pakv.PakvError):
        m8.bind_slab(0, 0x1000, 0x2000, 4)    # int8 needs scales


def test_slab_bytes():
    m = pakv.LayerMap([_desc(d=512, hkv=2), _desc(d=256, hkv=1, dtype=pakv.KV_INT8_PTH)])
    assert m.slab_bytes(0, 10) == (10 * 2 * 16 * 512 * 2, 0)
    assert m.slab_bytes(1, 10) == (10 * 1 * 16 * 256, 10 * 16 * 4)


def _bound_map():
    m = pakv.LayerMap([_desc(), _desc(src=0), _desc(dtype=pakv.KV_INT8_PTH)])
    m.bind_slab(0, 0x1000, 0x2000, 8)
    m.bind_slab(2, 0x1000, 0x2000, 8, 0x3000, 0x4000)
    return m


def test_store_on_shared_layer_returns_ok_without_launch():
    m = _bound_map()
    pages = pakv.Pages(0x5000, 2, 4)
    # null device pointers: a shared layer must return before touching anything
    assert pakv.lib.pakv_paged_kv_store(m.handle, 1, ctypes.byref(pages), None, None, None, None, 2, 5, None) == 0


def test_argument_errors_are_returned_before_launch():
    m = _bound_map()
    pages = pakv.Pages(0x5000, 2, 4)
    lib = pakv.lib
    # decode: null q
    assert lib.pakv_paged_attn_decode(m.handle, 0, ctypes.byref(pages), 0x6000, None, 0x7000, 2, 40,
                                      0x8000, 1 << 20, None) == pakv.ERR_INVALID
    # decode: length bound beyond the page table (4 pages = 64 positions)
    assert lib.pakv_paged_attn_decode(m.handle, 0, ctypes.byref(pages), 0x6000, 0x6100, 0x7000, 2, 65,
                                      0x8000, 1 << 20, None) == pakv.ERR_INVALID
    # decode: workspace too small
    need = lib.pakv_decode_workspace_bytes(m.handle, 0, 2, 40)
    assert need > 0
    assert lib.pakv_paged_attn_decode(m.handle, 0, ctypes.byref(pages), 0x6000, 0x6100, 0x7000, 2, 40,
                                      0x8000, need - 1, None) == pakv.ERR_WORKSPACE
    assert "workspace" in pakv.last_error()
    # decode: more sequences than the page table holds
    assert lib.pakv_paged_attn_decode(m.handle, 0, ctypes.byref(pages), 0x6000, 0x6100, 0x7000, 3, 40,
                                      0x8000, 1 << 20, None) == pakv.ERR_INVALID
    # decode: no sequences -> nothing to do
    assert lib.pakv_paged_attn_decode(m.handle, 0, ctypes.byref(pages), None, None, None, 0, 40,
                                      None, 0, None) == pakv.OK
    # packed extend without its key rows (or values, on a layer that stores V)
    assert lib.pakv_paged_attn_extend_packed(m.handle, 2, ctypes.byref(pages), 0x6000, 0x6100, 0x6200, None,
                                             0x6300, 0x7000, 2, 10, 5, 40, None) == pakv.ERR_INVALID
    assert lib.pakv_paged_attn_extend_packed(m.handle, 0, ctypes.byref(pages), 0x6000, 0x6100, 0x6200, 0x6300,
                                             None, 0x7000, 2, 10, 5, 40, None) == pakv.ERR_INVALID
    # extend: empty chunk -> nothing to do
    assert lib.pakv_paged_attn_extend(m.handle, 0, ctypes.byref(pages), None, None, None, None,
                                      2, 0, 0, 40, None) == pakv.OK
    # store: unbound layer map entry / bad layer index
    assert lib.pakv_paged_kv_store(m.handle, 9, ctypes.byref(pages), 0x6000, 0x6100, 0x6200, 0x6300,
                                   2, 5, None) == pakv.ERR_INVALID
    # store: null k
    assert lib.pakv_paged_kv_store(m.handle, 0, ctypes.byref(pages), 0x6000, 0x6100, None, 0x6300,
                                   2, 5, None) == pakv.ERR_INVALID


def test_extend_staging_sizes_and_refusals():
    """The staged extend's workspace: none for a bf16 layer's own chunk; for
    8-bit layers and packed chunks, two bf16 page sets and two scale arrays
    over the pages a chunk's rows see (whole context on a full layer, window
    plus chunk on a sliding one); a missing or short workspace is refused
    before any launch."""
    m = _bound_map()
    assert pakv.extend_staging_bytes(m, 0, 2, 5, 40, False) == 0        # bf16, chunk from the slab
    assert pakv.extend_staging_bytes(m, 1, 2, 5, 40, False) == 0        # shared bf16
    al = lambda x: (x + 255) // 256 * 256
    stride = 2 * ((40 + 30) // 32 + 1)          # whole 32-key tiles over 40 positions, one more for the start
    blocks = 2 * stride * 1
    for packed in (False, True):
        want = 2 * al(blocks * 16 * 256 * 2) + al((blocks + 1) * 32 * 4)
        assert pakv.extend_staging_bytes(m, 2, 2, 5, 40, packed) == want
    assert pakv.extend_staging_bytes(m, 0, 2, 5, 40, True) == 2 * al(blocks * 16 * 512) + al((blocks + 1) * 128)
    ms = pakv.LayerMap([_desc(w=512, dtype=pakv.KV_INT8_PTH)])
    span = lambda q, kv: pakv.extend_staging_bytes(ms, 0, 1, q, kv, False)
    assert span(64, 8192) == span(64, 4096) < span(64, 576) * 10           # window + chunk, not the context
    assert span(64, 100) < span(64, 8192)
    assert pakv.extend_staging_bytes(m, 7, 2, 5, 40, False) == 0        # bad layer
    assert pakv.extend_staging_bytes(m, 2, 0, 5, 40, False) == 0        # nothing to stage
    pages = pakv.Pages(0x5000, 2, 4)
    lib = pakv.lib
    need = pakv.extend_staging_bytes(m, 2, 2, 5, 40, False)
    assert lib.pakv_paged_attn_extend_staged(m.handle, 2, ctypes.byref(pages), 0x6000, 0x6100, 0x6200, None, None,
                                             0x7000, 2, 10, 5, 40, None, 0, 1, None) == pakv.ERR_WORKSPACE
    assert lib.pakv_paged_attn_extend_staged(m.handle, 2, ctypes.byref(pages), 0x6000, 0x6100, 0x6200, None, None,
                                             0x7000, 2, 10, 5, 40, 0x9000, need - 1, 1, None) == pakv.ERR_WORKSPACE
    assert "staging" in pakv.last_error()
    # packed on a bf16 layer needs staging too; without its value rows it is refused
    assert lib.pakv_paged_attn_extend_staged(m.handle, 0, ctypes.byref(pages), 0x6000, 0x6100, 0x6200, 0x6300, None,
                                             0x7000, 2, 10, 5, 40, 0x9000, 1 << 30, 1, None) == pakv.ERR_INVALID
    # empty chunk: nothing to do, no workspace needed
    assert lib.pakv_paged_attn_extend_staged(m.handle, 2, ctypes.byref(pages), None, None, None, None, None,
                                             None, 2, 0, 0, 40, None, 0, 1, None) == pakv.OK


def test_unbound_source_slab_is_an_error():
    m = pakv.LayerMap([_desc(), _desc(src=0)])
    pages = pakv.Pages(0x5000, 1, 4)
    st = pakv.lib.pakv_paged_attn_decode(m.handle, 1, ctypes.byref(pages), 0x6000, 0x6100, 0x7000, 1, 40,
                                         0x8000, 1 << 20, None)
    assert st == pakv.ERR_INVALID and "not bound" in pakv.last_error()


def test_workspace_and_plan_sizes():
    m = pakv.LayerMap([_desc(d=512), _desc(d=256, w=512)])
    p_short = pakv.decode_plan_bytes(m, 0, 64, 4097)
    p_long = pakv.decode_plan_bytes(m, 0, 64, 131073)
    # the plan holds a page id per 16 keys of every sequence
    assert p_long - p_short >= 64 * ((131073 + 15) // 16 - (4097 + 15) // 16) * 4 - 256
    # the partials (the rest of the workspace) depend on the batch, not the context
    part = lambda layer, nseq, ctx: (pakv.decode_workspace_bytes(m, layer, nseq, ctx)
                                     - pakv.decode_plan_bytes(m, layer, nseq, ctx))
    assert part(0, 64, 4097) == part(0, 64, 131073) > 0
    assert 0 < part(0, 8, 4097) < part(0, 64, 4097)
    assert part(1, 64, 4097) < part(0, 64, 4097)     # D 256 partials are half the size
    assert pakv.decode_plan_bytes(m, 0, 64, 0) == 0 and pakv.decode_plan_bytes(m, 5, 64, 10) == 0


def test_plan_argument_errors_are_returned_before_launch():
    m = _bound_map()
    pages = pakv.Pages(0x5000, 2, 4)
    lib = pakv.lib
    need = lib.pakv_decode_plan_bytes(m.handle, 0, 2, 40)
    assert need > 0
    # plan: buffer too small, null kv_lens
    assert lib.pakv_decode_plan(m.handle, 0, ctypes.byref(pages), 0x6000, 2, 40, 0x9000, need - 1,
                                None) == pakv.ERR_WORKSPACE
    assert lib.pakv_decode_plan(m.handle, 0, ctypes.byref(pages), None, 2, 40, 0x9000, need,
                                None) == pakv.ERR_INVALID
    # planned decode: missing plan, small workspace, null q
    ws = lib.pakv_decode_workspace_bytes(m.handle, 0, 2, 40)
    assert lib.pakv_paged_attn_decode_planned(m.handle, 0, ctypes.byref(pages), None, 0, 0x6100, 0x7000, 2, 40,
                                              0x8000, ws, None) == pakv.ERR_WORKSPACE
    assert lib.pakv_paged_attn_decode_planned(m.handle, 0, ctypes.byref(pages), 0x9000, need, 0x6100, 0x7000,
                                              2, 40, 0x8000, 16, None) == pakv.ERR_WORKSPACE
    assert lib.pakv_paged_attn_decode_planned(m.handle, 0, ctypes.byref(pages), 0x9000, need, None, 0x7000,
                                              2, 40, 0x8000, ws, None) == pakv.ERR_INVALID
    # no sequences -> nothing to do
    assert lib.pakv_decode_plan(m.handle, 0, ctypes.byref(pages), None, 0, 40, None, 0, None) == pakv.OK


def test_append_argument_errors_are_returned_before_launch():
    """Every refusal of pakv_paged_attn_decode_append comes back on the host (no
    GPU here: a launch would fail with PAKV_ERR_HIP instead)."""
    m = _bound_map()           # 0: bf16 owner, 1: shared (source 0), 2: int8 owner
    pages = pakv.Pages(0x5000, 2, 4)
    lib = pakv.lib
    need = lib.pakv_decode_plan_bytes(m.handle, 0, 2, 40)
    ws = lib.pakv_decode_workspace_bytes(m.handle, 0, 2, 40)
    f = lib.pakv_paged_attn_decode_append
    P = ctypes.byref(pages)
    # int8 owner: not built, whatever the other arguments
    assert f(m.handle, 2, P, 0x9000, need, 0x6200, 0x6300, 0x6100, 0x7000, 2, 40, 0x8000, ws, None) == \
        pakv.ERR_UNSUPPORTED
    # bf16 owner without the new rows
    assert f(m.handle, 0, P, 0x9000, need, None, 0x6300, 0x6100, 0x7000, 2, 40, 0x8000, ws, None) == pakv.ERR_INVALID
    assert f(m.handle, 0, P, 0x9000, need, 0x6200, None, 0x6100, 0x7000, 2, 40, 0x8000, ws, None) == pakv.ERR_INVALID
    # plan and workspace sizes, null q
    assert f(m.handle, 0, P, 0x9000, need - 1, 0x6200, 0x6300, 0x6100, 0x7000, 2, 40, 0x8000, ws, None) == \
        pakv.ERR_WORKSPACE
    assert f(m.handle, 0, P, 0x9000, need, 0x6200, 0x6300, 0x6100, 0x7000, 2, 40, 0x8000, 16, None) == \
        pakv.ERR_WORKSPACE
    assert f(m.handle, 0, P, 0x9000, need, 0x6200, 0x6300, None, 0x7000, 2, 40, 0x8000, ws, None) == pakv.ERR_INVALID
    # a shared layer needs no new rows; no sequences: nothing to do
    assert f(m.handle, 1, P, 0x9000, need, None, None, None, 0x7000, 2, 40, 0x8000, ws, None) == pakv.ERR_INVALID
    assert f(m.handle, 0, P, None, 0, None, None, None, None, 0, 40, None, 0, None) == pakv.OK


def test_too_many_sequences_or_units_per_decode_call_are_refused():
    m = pakv.LayerMap([_desc(hq=16, hkv=8)])
    m.bind_slab(0, 0x1000, 0x2000, 8)
    for nseq in (1024, 1100):
        pages = pakv.Pages(0x5000, nseq, 4)
        st = pakv.lib.pakv_paged_attn_decode(m.handle, 0, ctypes.byref(pages), 0x6000, 0x6100, 0x7000, nseq, 40,
                                             0x8000, 1 << 30, None)
        assert st == pakv.ERR_UNSUPPORTED, nseq


def test_one_hip_runtime_per_process():
    """The library must bind to the HIP runtime torch loaded (same soname), not
    load a second one: torch's streams are only valid in its own runtime."""
    maps = open("/proc/self/maps").read()
    runtimes = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(runtimes) == 1, runtimes


def test_workgroup_xcds_argument_errors_are_returned_before_launch():
    from full_attention_amd import pakv
    assert pakv.lib.pakv_workgroup_xcds(None, 8, None) == pakv.ERR_INVALID
    assert pakv.lib.pakv_workgroup_xcds(0x8000, 0, None) == pakv.ERR_INVALID
    assert pakv.lib.pakv_workgroup_xcds(0x8000, 65536, None) == pakv.ERR_INVALID


def test_noalloc_decode_refuses_what_its_scratch_cannot_hold():
    """pakv_paged_attn_decode_noalloc checks the workspace it would need against
    its static scratch (64 MiB) before any GPU call; arguments as for decode."""
    lib = pakv.lib
    assert lib.pakv_decode_noalloc_max_bytes() == 64 << 20
    m = pakv.LayerMap([_desc(d=512, hq=16, hkv=1)])
    m.bind_slab(0, 0x1000, 0x2000, 8)
    nseq, max_len = 1000, 1 << 17
    pages = pakv.Pages(0x5000, nseq, max_len // 16)
    need = lib.pakv_decode_workspace_bytes(m.handle, 0, nseq, max_len)
    assert need > 64 << 20
    st = lib.pakv_paged_attn_decode_noalloc(m.handle, 0, ctypes.byref(pages), 0x6000, 0x6100, 0x7000, nseq,
                                            max_len, None)
    assert st == pakv.ERR_WORKSPACE and "scratch" in pakv.last_error()
    # the decode checks come first
    assert lib.pakv_paged_attn_decode_noalloc(m.handle, 0, ctypes.byref(pages), None, 0x6100, 0x7000, 2, 40,
                                              None) == pakv.ERR_INVALID
    assert lib.pakv_paged_attn_decode_noalloc(m.handle, 0, ctypes.byref(pages), None, None, None, 0, 40,
                                              None) == pakv.OK


def test_k_eq_v_layers_store_keys_only():
    """A K=V layer binds no V buffer, prices one row per token and head, may
    only be read by shared layers of the same kind, and is built for bf16."""
    eps = 1e-6
    kv = lambda src=-1, dtype=pakv.KV_BF16, e=eps: pakv.LayerDesc(512, 16, 2, 0, src, dtype, 0.044, 1, e)
    m = pakv.LayerMap([kv(), kv(src=0)])
    m.bind_slab(0, 0x1000, None, 8)
    assert m.kv_bytes_per_token() == (2 * 1 * 1024, 0)
    with pytest.raises(pakv.PakvError) as e:
        pakv.LayerMap([kv(), pakv.LayerDesc(512, 16, 2, 0, 0, pakv.KV_BF16, 0.044)])    # source stores K only
    assert e.value.status == pakv.ERR_ALIAS
    with pytest.raises(pakv.PakvError) as e:
        pakv.LayerMap([kv(), kv(src=0, e=1e-5)])
    assert e.value.status == pakv.ERR_ALIAS
    with pytest.raises(pakv.PakvError) as e:
        pakv.LayerMap([kv(dtype=pakv.KV_INT8_PTH)])
    assert e.value.status == pakv.ERR_UNSUPPORTED
    with pytest.raises(pakv.PakvError) as e:
        pakv.LayerMap([kv(e=-1.0)])
    assert e.value.status == pakv.ERR_INVALID
    # a layer that stores V still needs its V buffer
    m2 = pakv.LayerMap([_desc()])
    with pytest.raises(pakv.PakvError):
        m2.bind_slab(0, 0x1000, None, 8)


def test_fp8_layers_need_scales_and_share_only_with_fp8():
    m = pakv.LayerMap([_desc(dtype=pakv.KV_FP8_PTH)])
    with pytest.raises(pakv.PakvError):
        m.bind_slab(0, 0x1000, 0x2000, 8)
    m.bind_slab(0, 0x1000, 0x2000, 8, 0x3000, 0x4000)
    assert m.kv_bytes_per_token() == (2 * (256 + 4), 0)
    with pytest.raises(pakv.PakvError) as e:
        pakv.LayerMap([_desc(dtype=pakv.KV_FP8_PTH), _desc(src=0, dtype=pakv.KV_INT8_PTH)])
    assert e.value.status == pakv.ERR_ALIAS


def test_decode_checks_flags():
    assert pakv.lib.pakv_set_decode_checks(1 << 5) == pakv.ERR_INVALID
    pakv.set_decode_checks(pakv.CHECK_XCD_PLACEMENT)
    pakv.set_decode_checks(0)


def test_debug_bounds_calls_refused_by_the_product_build():
    """The page-id counters exist only in a PAKV_DEBUG_BOUNDS build; the
    product library refuses both calls on the host, touching no device."""
    if os.path.basename(pakv.LIB_PATH) == "libpakv_bounds.so":
        pytest.skip("this process loaded the PAKV_DEBUG_BOUNDS build")
    with pytest.raises(pakv.PakvError) as e:
        pakv.debug_bounds_counts()
    assert e.value.status == pakv.ERR_UNSUPPORTED
    with pytest.raises(pakv.PakvError) as e:
        pakv.debug_bounds_reset()
    assert e.value.status == pakv.ERR_UNSUPPORTED


@pytest.mark.parametrize("variant", ["bounds", "hostsan"])
def test_diagnostic_builds_export_every_declared_symbol(variant):
    """libpakv_bounds.so (PAKV_DEBUG_BOUNDS) and libpakv_hostsan.so (host code
    under ASan/UBSan) are the same ABI: every symbol the header declares."""
    from full_attention_amd.build import library_path
    path = library_path(variant)
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} is not built (__graft_entry__.build() builds it)")
    nm = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pakv_[a-z0-9_]+)\b", nm))
    missing = [n for n in declared_symbols() if n not in exported]
    assert not missing, missing


def test_pages_struct_keeps_its_table_alive():
    """make_pages holds a reference to the table tensor, so a temporary table
    cannot be freed (and its memory reused) while the struct is in use."""
    import gc
    import weakref
    import torch
    t = torch.zeros((3, 4), dtype=torch.int32)
    ref = weakref.ref(t)
    pages = pakv.make_pages(t)
    del t
    gc.collect()
    assert ref() is not None and pages.num_seqs == 3 and pages.max_pages_per_seq == 4
    del pages
    gc.collect()
    assert ref() is None
