"""The decode workspace's status word, and rows an append cannot place.

* A plan made for another shape is refused inside the kernel: nothing is
  written, the arrival counters stay zero, and PAKV_DECODE_PLAN_MISMATCH is
  set.
* After ordinary decodes (units merged inside one XCD's L2 and through
  memory) the status word is clear and the arrival counters are zero again.
* An append whose new row has no page (a page-table entry outside the pool)
  writes nothing, as pakv_paged_kv_store drops such a row: the slab after the
  fused call equals the slab after store-then-decode, byte for byte.
"""

import numpy as np
import pytest
import torch

from workloads import LayerSpec, e2b_decode_workload, normal_bf16

from gpu_helpers import Scenario, assert_close, dev_bits, host_bits, i32, need_gpu

pytestmark = pytest.mark.gpu


def _workspace_zero_past_status(cache):
    """The status block past its word and the arrival counters (bytes 4 ..
    256 + 4 * 8192) are zero: what must be zero between calls."""
    w = cache._workspace.cpu().numpy()
    return not w[4:256 + 4 * 8192].any()


def test_status_clear_after_local_and_cross_xcd_merges():
    """With the placement check on (pakv_set_decode_checks)."""
    need_gpu()
    from full_attention_amd import pakv
    pakv.set_decode_checks(pakv.CHECK_XCD_PLACEMENT)
    try:
        _run_local_and_cross_merges()
    finally:
        pakv.set_decode_checks(0)


def _run_local_and_cross_merges():
    from full_attention_amd import pakv
    lens = list(np.array(e2b_decode_workload().cached_lens[:60]) + 1) + [5, 17, 100, 250]
    specs = [LayerSpec("full", 512, 8, 1, 0), LayerSpec("sliding", 256, 8, 1, 512)]
    sc = Scenario(specs, None, lens, seed=147)
    for layer in range(2):
        sc.store(layer, [0] * len(lens), lens)
    kv, maxl = i32(lens), max(lens)
    for layer in range(2):
        plan = sc.cache.decode_plan(layer, kv, maxl)
        for _ in range(3):
            got, ref, _ = sc.decode(layer, lens)
            assert_close(got, ref, f"layer {layer}")
            q = normal_bf16(sc.rng, (len(lens), 8, specs[layer].head_dim))
            sc.cache.decode(layer, kv, dev_bits(q), maxl, plan=plan)
    assert sc.cache.status() == 0
    assert _workspace_zero_past_status(sc.cache)
    assert pakv.DECODE_PLAN_MISMATCH == 1 and pakv.DECODE_XCD_SPLIT == 2


@pytest.mark.parametrize("wrong", ["window", "max_kv_len"])
def test_plan_of_another_shape_is_refused_in_kernel(wrong):
    need_gpu()
    from full_attention_amd import pakv
    specs = [LayerSpec("sliding", 256, 8, 1, 64), LayerSpec("full", 256, 8, 1, 0)]
    lens = [300, 65, 1000, 17]
    sc = Scenario(specs, None, lens, seed=151)
    for layer in range(2):
        sc.store(layer, [0] * len(lens), lens)
    kv, maxl = i32(lens), max(lens)
    if wrong == "window":
        plan = sc.cache.decode_plan(0, kv, maxl)          # sliding plan, used on the full layer
        call_max = maxl
    else:                                                 # made for another length bound
        nbytes = pakv.decode_plan_bytes(sc.cache.map, 1, len(lens), maxl)
        plan = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        pakv.decode_plan(sc.cache.map, 1, sc.cache.pages, kv, len(lens), maxl - 16, plan, nbytes)
        call_max = maxl
    q = dev_bits(normal_bf16(sc.rng, (len(lens), 8, 256)))
    out = torch.full_like(q, 0x1234)
    sc.cache.decode(1, kv, q, call_max, out=out, plan=plan)
    torch.cuda.synchronize()
    assert sc.cache.status() == pakv.DECODE_PLAN_MISMATCH
    assert (out == 0x1234).all(), "a refused call wrote outputs"
    assert _workspace_zero_past_status(sc.cache)
    sc.cache.clear_status()
    good = sc.cache.decode_plan(1, kv, maxl)
    got = host_bits(sc.cache.decode(1, kv, q, maxl, plan=good))
    torch.cuda.synchronize()
    assert sc.cache.status() == 0
    ref = np.stack([sc.oracle.decode(1, b, host_bits(q)[b], L) for b, L in enumerate(lens)])
    assert_close(got, ref)


def test_append_drops_a_row_without_a_page():
    need_gpu()
    spec = LayerSpec("full", 256, 8, 1, 0)
    lens = [40, 17, 33, 100]          # the new rows sit at 39, 16, 32, 99
    scs = [Scenario([spec], None, lens, seed=157) for _ in range(2)]
    for sc in scs:
        sc.store(0, [0] * len(lens), [L - 1 for L in lens])
    bad = 1                            # sequence whose new row's page is missing
    for sc in scs:
        table = sc.pool.page_table.copy()
        table[bad, (lens[bad] - 1) // 16] = -1
        sc.cache.set_page_table(table)
    rng = np.random.default_rng(3)
    kn = normal_bf16(rng, (len(lens), 1, 256))
    vn = normal_bf16(rng, (len(lens), 1, 256))
    q = normal_bf16(rng, (len(lens), 8, 256))
    kv, maxl = i32(lens), max(lens)
    a, b = scs
    a.cache.store(0, i32(np.arange(len(lens) + 1)), i32([L - 1 for L in lens]), dev_bits(kn), dev_bits(vn))
    out_a = host_bits(a.cache.decode(0, kv, dev_bits(q), maxl, plan=a.cache.decode_plan(0, kv, maxl)))
    out_b = host_bits(b.cache.decode_append(0, b.cache.decode_plan(0, kv, maxl), dev_bits(kn), dev_bits(vn),
                                            dev_bits(q), maxl))
    torch.cuda.synchronize()
    for layer_slab_a, layer_slab_b in zip(a.cache.slab_of(0)[:2], b.cache.slab_of(0)[:2]):
        assert np.array_equal(host_bits(layer_slab_a), host_bits(layer_slab_b))
    good = [s for s in range(len(lens)) if s != bad]
    assert np.array_equal(out_a[good], out_b[good])
    for s in good:
        b.oracle.store(0, s, lens[s] - 1, kn[s:s + 1], vn[s:s + 1])
        assert_close(out_b[s], b.oracle.decode(0, s, q[s], lens[s]), f"seq {s}")
