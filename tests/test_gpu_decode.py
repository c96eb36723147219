"""paged_attn_decode on the GPU against the oracle, within |err| <= 2e-2 + 1e-2|ref|
(bf16 outputs, fp32 accumulation), plus the exact properties the method has:
W = 1 returns the query's own value row; outputs are bit-identical from run to
run, across page placements and across batch compositions; a shared layer's
output is bit-identical to its source's and a shared sliding layer keeps its
window.  Unwritten slots hold NaN throughout."""

import zlib

import numpy as np
import pytest
import torch

from workloads import LayerSpec, bf16_from_f32, bf16_to_f32, normal_bf16

from gpu_helpers import Scenario, assert_close, dev_bits, host_bits, i32, need_gpu

pytestmark = pytest.mark.gpu


def _decode_case(d, hq, hkv, window, kv_dtype, lens, seed, only_visible=True):
    kind = "sliding" if window else "full"
    spec = LayerSpec(kind, d, hq, hkv, window, kv_dtype=kv_dtype)
    sc = Scenario([spec], None, lens, seed=seed)
    starts = [max(0, L - window) if (window and only_visible) else 0 for L in lens]
    counts = [L - s for L, s in zip(lens, starts)]
    sc.store(0, starts, counts)
    return sc


LENS = [1, 2, 15, 16, 17, 31, 33, 100, 129, 257, 700]


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("hq,hkv", [(8, 1), (16, 8), (16, 2), (4, 4), (16, 1)])
@pytest.mark.parametrize("window", [0, 1, 7, 32, 512])
def test_decode_matches_oracle(kv_dtype, d, hq, hkv, window):
    need_gpu()
    seed = zlib.crc32(repr((kv_dtype, d, hq, hkv, window)).encode()) % 10000
    sc = _decode_case(d, hq, hkv, window, kv_dtype, LENS, seed)
    got, ref, _ = sc.decode(0, LENS)
    assert_close(got, ref, f"decode d={d} hq={hq} hkv={hkv} W={window} {kv_dtype}")


@pytest.mark.parametrize("d", [256, 512])
def test_window_one_returns_own_value_row(d):
    need_gpu()
    lens = [1, 5, 16, 17, 300]
    sc = _decode_case(d, 8, 1, 1, "bf16", lens, seed=5)
    got, _, _ = sc.decode(0, lens)
    k, v, cu, starts = sc.rows[0]
    for b, L in enumerate(lens):
        own = v[cu[b + 1] - 1, 0]            # row of position L - 1
        assert np.array_equal(got[b], np.broadcast_to(own, got[b].shape))


def test_long_context_many_splits():
    need_gpu()
    lens = [9000, 40000, 3]
    for kv_dtype in ("bf16", "int8"):
        sc = _decode_case(512, 8, 1, 0, kv_dtype, lens, seed=9)
        got, ref, _ = sc.decode(0, lens)
        assert_close(got, ref, f"long {kv_dtype}")


@pytest.mark.parametrize("window,hkv", [(0, 1), (32, 8)])
def test_largest_batch_per_call(window, hkv):
    """1023 sequences, the most one decode call takes (the per-sequence table
    the kernels keep in LDS is then full), of lengths 1..60; at Hkv 8 that is
    8184 (sequence, KV head) units, near the 8192 a call takes.  Every output
    matches the oracle."""
    need_gpu()
    rng = np.random.default_rng(91 + hkv)
    lens = [int(x) for x in rng.integers(1, 61, 1023)]
    sc = _decode_case(256, 8, hkv, window, "bf16", lens, seed=93 + hkv)
    got, ref, _ = sc.decode(0, lens)
    assert_close(got, ref, f"1023 sequences, W {window}, Hkv {hkv}")


def test_deterministic_and_page_placement_invariant():
    need_gpu()
    lens = [37, 1000, 513, 4096]
    outs = []
    for pool_seed in (1, 2):
        spec = LayerSpec("full", 512, 8, 1, 0)
        sc = Scenario([spec], None, lens, seed=100)
        # same draws, different page permutation: re-seed the pool only
        rng = np.random.default_rng(pool_seed)
        from workloads import make_page_pool
        sc.pool = make_page_pool(rng, lens, spare=4 + pool_seed)
        from full_attention_amd.cache import PagedKVCache
        sc.cache = PagedKVCache([spec], None, sc.pool.num_pages)
        sc.cache.set_page_table(sc.pool.page_table)
        sc.store(0, [0] * 4, lens)
        q = np.random.default_rng(7).standard_normal((4, 8, 512)).astype(np.float32)
        from workloads import bf16_from_f32
        qb = dev_bits(bf16_from_f32(q))
        a = host_bits(sc.cache.decode(0, i32(lens), qb, 4096))
        b = host_bits(sc.cache.decode(0, i32(lens), qb, 4096))
        assert np.array_equal(a, b)
        outs.append(a)
    assert np.array_equal(outs[0], outs[1])


def test_other_sequences_change_nothing_but_the_partition():
    """A sequence's output with other sequences in the batch stays within
    tolerance of the oracle and of its output alone (the chunk stream is
    partitioned over the whole batch, so bits may differ)."""
    need_gpu()
    spec = LayerSpec("sliding", 256, 8, 1, 512)
    lens = [2000, 777, 3000]
    sc = Scenario([spec], None, lens, seed=12)
    sc.store(0, [0, 0, 0], lens)
    from workloads import normal_bf16
    q = normal_bf16(np.random.default_rng(3), (3, 8, 256))
    full = host_bits(sc.cache.decode(0, i32(lens), dev_bits(q), 3000))
    from full_attention_amd import pakv
    table = torch.as_tensor(sc.pool.page_table[1:2], dtype=torch.int32).cuda()
    saved = sc.cache.pages
    sc.cache.pages = pakv.make_pages(table)
    alone = host_bits(sc.cache.decode(0, i32([777]), dev_bits(q[1:2]), 3000))
    sc.cache.pages = saved
    ref = sc.oracle.decode(0, 1, q[1], 777)
    assert_close(full[1], ref, "in batch")
    assert_close(alone[0], ref, "alone")


@pytest.mark.parametrize("window", [0, 512])
def test_same_split_gives_the_same_bits_in_any_batch(window):
    """A unit's split depends only on its length and on the batch's chunks per
    run.  Batches with the same lengths (so the same split) give a sequence
    bit-identical output wherever it sits in the batch and whatever its
    neighbours hold, although its runs land on other workgroups (and its merge
    may go through one XCD's L2 in one batch and through memory in another)."""
    need_gpu()
    from full_attention_amd import pakv
    from workloads import normal_bf16
    d = 512 if window == 0 else 256
    spec = LayerSpec("full" if window == 0 else "sliding", d, 8, 1, window)
    lens = [1800, 900, 3100, 2600, 700, 1300]      # sequence 0 is the one followed
    alt = lens[1:]                                  # neighbours of the same lengths, other data
    every = lens + alt
    sc = Scenario([spec], None, every, seed=81)
    sc.store(0, [0] * len(every), every)
    q_all = normal_bf16(np.random.default_rng(82), (len(every), 8, d))
    table = sc.pool.page_table

    def run(rows):
        L = [every[r] for r in rows]
        saved = sc.cache.pages
        sc.cache.pages = pakv.make_pages(torch.as_tensor(table[rows], dtype=torch.int32).cuda())
        out = host_bits(sc.cache.decode(0, i32(L), dev_bits(q_all[rows]), max(L)))
        torch.cuda.synchronize()
        sc.cache.pages = saved
        return out

    n = len(lens)
    a = run([0, 1, 2, 3, 4, 5])
    b = run([3, 5, 1, 0, 2, 4])                     # the same sequences in another order
    c = run([0] + [n + i for i in range(len(alt))])  # sequence 0 beside other data
    assert np.array_equal(a[0], b[3]), "another position in the batch changed the bits"
    assert np.array_equal(a[0], c[0]), "other neighbours changed the bits"
    assert_close(a[0], sc.oracle.decode(0, 0, q_all[0], lens[0]))


def test_shared_layers_read_their_source():
    need_gpu()
    specs = [LayerSpec("sliding", 256, 8, 1, 64), LayerSpec("full", 512, 8, 1, 0),
             LayerSpec("sliding", 256, 8, 1, 64), LayerSpec("full", 512, 8, 1, 0)]
    lens = [300, 65, 64, 1]
    sc = Scenario(specs, 2, lens, seed=44)
    for layer in range(4):
        sc.store(layer, [0] * 4, lens)
    from workloads import normal_bf16
    for src, shared in ((0, 2), (1, 3)):
        q = dev_bits(normal_bf16(sc.rng, (4, 8, specs[src].head_dim)))
        a = host_bits(sc.cache.decode(src, i32(lens), q, 300))
        b = host_bits(sc.cache.decode(shared, i32(lens), q, 300))
        assert np.array_equal(a, b)
    # the shared sliding layer keeps its window: differs from full attention over the same rows
    got, ref, q = sc.decode(2, lens)
    assert_close(got, ref, "shared sliding")
    from oracle import attend
    k, v, cu, _ = sc.rows[0]
    qf = bf16_to_f32(q).astype(np.float64)
    kf = bf16_to_f32(k).astype(np.float64)
    vf = bf16_to_f32(v).astype(np.float64)
    full = attend(qf[0:1], np.array([299]), kf[:300], vf[:300], np.arange(300), 0, specs[2].sm_scale)
    assert np.abs(bf16_to_f32(got[0]) - full[0]).max() > 0.05


def test_unwritten_slots_do_not_leak_into_sliding_output():
    need_gpu()
    # only the visible rows are written; everything before the window is NaN
    lens = [1000, 1030, 17]
    sc = _decode_case(256, 8, 1, 32, "bf16", lens, seed=77, only_visible=True)
    got, ref, _ = sc.decode(0, lens)
    assert_close(got, ref, "sentinel")
    sc8 = _decode_case(512, 8, 1, 32, "int8", lens, seed=78, only_visible=True)
    got, ref, _ = sc8.decode(0, lens)
    assert_close(got, ref, "sentinel int8")


def test_graph_replay_matches_eager():
    """Decode and store captured into a HIP graph: every replay (with eager work
    and synchronisations between replays) equals the eager result bit for bit."""
    need_gpu()
    specs = [LayerSpec("sliding", 256, 8, 1, 64), LayerSpec("full", 512, 8, 1, 0)]
    lens = [300, 65, 1000]
    sc = Scenario(specs, None, [L + 1 for L in lens], seed=90)
    for layer in range(2):
        sc.store(layer, [0] * 3, lens)
    from workloads import normal_bf16
    kv = i32([L + 1 for L in lens])
    cu, pos = i32([0, 1, 2, 3]), i32(lens)
    new = {l: (dev_bits(normal_bf16(sc.rng, (3, 1, specs[l].head_dim))),
               dev_bits(normal_bf16(sc.rng, (3, 1, specs[l].head_dim)))) for l in range(2)}
    qs = [dev_bits(normal_bf16(sc.rng, (3, 8, specs[l].head_dim))) for l in range(2)]
    outs = [torch.empty_like(q) for q in qs]
    ws, need = sc.cache.workspace(1, 3, 1001)
    sc.cache._workspace = torch.zeros(4 * need, dtype=torch.uint8, device="cuda")

    def step():
        for l in range(2):
            sc.cache.store(l, cu, pos, *new[l])
            sc.cache.decode(l, kv, qs[l], 1001, out=outs[l])

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outs:
            o.fill_(0)
        torch.randn(1000, device="cuda").sum()          # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs"


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_planned_decode_matches_unplanned_bitwise(kv_dtype):
    """One plan per (window, Hkv), shared by every layer of that kind, gives the
    same bits as the one-call decode, including runs that cross units and
    batches of page ids past the first 64."""
    need_gpu()
    specs = [LayerSpec("sliding", 256, 8, 1, 512, kv_dtype=kv_dtype), LayerSpec("full", 512, 8, 1, 0,
                                                                                  kv_dtype=kv_dtype),
             LayerSpec("sliding", 256, 8, 1, 512, kv_dtype=kv_dtype), LayerSpec("full", 512, 8, 1, 0,
                                                                                  kv_dtype=kv_dtype)]
    lens = [1, 17, 513, 4097, 30000, 700, 2]
    sc = Scenario(specs, None, lens, seed=61 if kv_dtype == "bf16" else 62)
    for layer in range(4):
        sc.store(layer, [0] * len(lens), lens)
    from workloads import normal_bf16
    kv, maxl = i32(lens), max(lens)
    plans = {}
    for layer in range(4):
        key = sc.cache.plan_key(layer)
        if key not in plans:
            plans[key] = sc.cache.decode_plan(layer, kv, maxl)
    for layer in range(4):
        q = dev_bits(normal_bf16(sc.rng, (len(lens), 8, specs[layer].head_dim)))
        a = host_bits(sc.cache.decode(layer, kv, q, maxl))
        b = host_bits(sc.cache.decode(layer, kv, q, maxl, plan=plans[sc.cache.plan_key(layer)]))
        assert np.array_equal(a, b), f"layer {layer}"


def test_planned_decode_in_graph_replays():
    """Plans and planned decodes captured into a HIP graph: every replay equals
    the eager result bit for bit, and the oracle within tolerance."""
    need_gpu()
    specs = [LayerSpec("sliding", 256, 8, 1, 64), LayerSpec("full", 512, 8, 1, 0)]
    lens = [300, 65, 1000]
    sc = Scenario(specs, None, lens, seed=93)
    for layer in range(2):
        sc.store(layer, [0] * 3, lens)
    from workloads import normal_bf16
    kv = i32(lens)
    qh = [normal_bf16(sc.rng, (3, 8, specs[l].head_dim)) for l in range(2)]
    qs = [dev_bits(q) for q in qh]
    outs = [torch.empty_like(q) for q in qs]
    plans = [sc.cache.decode_plan(l, kv, 1000) for l in range(2)]
    ws, need = sc.cache.workspace(1, 3, 1000)

    def step():
        from full_attention_amd import pakv
        for l in range(2):
            pakv.decode_plan(sc.cache.map, l, sc.cache.pages, kv, 3, 1000, plans[l], plans[l].numel())
            sc.cache.decode(l, kv, qs[l], 1000, out=outs[l], plan=plans[l])

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for l in range(2):
        ref = np.stack([sc.oracle.decode(l, b, qh[l][b], lens[b]) for b in range(3)])
        assert_close(host_bits(eager[l]), ref, f"planned layer {l}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outs:
            o.fill_(0)
        torch.randn(1000, device="cuda").sum()          # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs"


def _read_plan(plan, B, max_kv_len, hkv=1, by_workgroup=False):
    """Header and records of a decode plan (the schedule layout the plan and
    decode kernels share; grid 512).  The plan stores each run's record at the
    decode workgroup that takes it, with the run's number in word 7; the
    records come back in run order (words 0..8), or in workgroup order."""
    w = plan.cpu().numpy().view(np.int32)
    soff, slen = 16, 16 + B + 1
    rec = (slen + B + 15) & ~15
    head = w[:8]
    by_wg = w[rec:rec + 512 * 80].reshape(512, 80)[:, :9]
    if by_workgroup:
        return head, by_wg, w[soff:soff + B + 1], w[slen:slen + B]
    assert sorted(by_wg[:, 7].tolist()) == list(range(512))    # one record per run
    recs = np.empty_like(by_wg)
    recs[by_wg[:, 7]] = by_wg
    return head, recs, w[soff:soff + B + 1], w[slen:slen + B]


@pytest.mark.parametrize("case", ["sliding", "full", "skewed"])
def test_plan_runs_partition_the_stream(case):
    """The plan's runs cover the key stream once, in workgroup order, none longer
    than the chunks-per-workgroup bound plus a half; with the unit-aligned
    split (chosen when every unit can have its own workgroups) no run crosses a
    unit and each unit's record names exactly the workgroups that cover it."""
    need_gpu()
    from workloads import e2b_decode_workload
    rng = np.random.default_rng(5)
    if case == "skewed":
        lens = [100000] + [20] * 700
        window = 0
    else:
        lens = list(np.array(e2b_decode_workload().cached_lens) + 1)
        window = 512 if case == "sliding" else 0
    spec = LayerSpec("sliding" if window else "full", 256, 8, 1, window)
    from full_attention_amd.cache import PagedKVCache
    from workloads import make_page_pool
    pool = make_page_pool(rng, lens)
    cache = PagedKVCache([spec], None, pool.num_pages, sentinel=False)
    cache.set_page_table(pool.page_table)
    B, maxl = len(lens), max(lens)
    plan = cache.decode_plan(0, i32(lens), maxl)
    torch.cuda.synchronize()
    head, recs, soff, slen = _read_plan(plan, B, maxl)
    T = int(head[1])
    L = np.array(lens)
    lo = np.maximum(0, L - window) if window else np.zeros(B, np.int64)
    n = (L + 15) // 16 - lo // 16
    assert T == int(n.sum()) and soff[B] == T
    per0 = -(-T // 512)
    cb, ce = recs[:, 0], recs[:, 1]
    busy = cb < ce
    # cover [0, T) exactly once, in workgroup order
    order = np.argsort(cb[busy], kind="stable")
    assert np.all(order == np.arange(busy.sum()))
    starts, ends = cb[busy], ce[busy]
    assert starts[0] == 0 and ends[-1] == T and np.all(starts[1:] == ends[:-1])
    aligned = head[2] == 0
    assert aligned == (case != "skewed")
    longest = int((ends - starts).max())
    assert longest <= (per0 + max(per0 // 2, 1) if aligned else per0)
    if aligned:
        unit_first = soff[:B]                         # one KV head: unit b starts at soff[b]
        for wg in np.nonzero(busy)[0]:
            c0, c1, u, kc, per, w0, w1 = (int(x) for x in recs[wg, :7])
            assert per == 0 and w0 <= wg <= w1
            assert c0 - unit_first[u] == kc and c1 <= unit_first[u] + n[u]       # inside its unit
            assert all(recs[x, 2] == u for x in range(w0, w1 + 1))               # the unit's workgroups
            assert recs[w0, 0] == unit_first[u] and recs[w1, 1] == unit_first[u] + n[u]


@pytest.mark.parametrize("case", ["sliding", "full", "skewed"])
def test_plan_gives_each_xcd_a_block_of_runs(case):
    """Workgroup i runs on XCD i mod 8.  Aligned split (sliding, full): the R
    busy runs are shared out evenly, the workgroups of class x taking runs
    [R x / 8, R (x + 1) / 8) in order and empty records after them, and a
    record's local flag says whether its unit's runs lie in one such block.
    Stream-K (skewed): workgroup i takes run (i mod 8) * 64 + i / 8."""
    need_gpu()
    from workloads import e2b_decode_workload, make_page_pool
    from full_attention_amd.cache import PagedKVCache
    rng = np.random.default_rng(6)
    if case == "skewed":
        lens, window = [100000] + [20] * 700, 0
    else:
        lens = list(np.array(e2b_decode_workload().cached_lens) + 1)
        window = 512 if case == "sliding" else 0
    spec = LayerSpec("sliding" if window else "full", 256, 8, 1, window)
    pool = make_page_pool(rng, lens)
    cache = PagedKVCache([spec], None, pool.num_pages, sentinel=False)
    cache.set_page_table(pool.page_table)
    B, maxl = len(lens), max(lens)
    plan = cache.decode_plan(0, i32(lens), maxl)
    torch.cuda.synchronize()
    head, wg, _, _ = _read_plan(plan, B, maxl, by_workgroup=True)
    runs = wg[:, 7]
    if head[2] != 0:
        assert case == "skewed"
        i = np.arange(512)
        assert np.array_equal(runs, (i % 8) * 64 + i // 8)
        return
    busy = wg[:, 0] < wg[:, 1]
    R = int(busy.sum())
    start = [(R * x) // 8 for x in range(9)]
    if case == "sliding":
        assert R == 448 and all(start[x + 1] - start[x] == 56 for x in range(8))   # every XCD busy
    block = lambda r: max(x for x in range(8) if start[x] <= r)
    for x in range(8):
        cls = runs[x::8]
        n = start[x + 1] - start[x]
        assert np.array_equal(cls[:n], np.arange(start[x], start[x + 1]))
        assert np.all(~busy[x::8][n:]) and np.all(cls[n:] >= R)
    for i in np.nonzero(busy)[0]:
        w0, w1 = int(wg[i, 5]), int(wg[i, 6])
        assert wg[i, 8] == (1 if block(w0) == block(w1) else 0)


@pytest.mark.parametrize("window,lens,cap", [(0, [4000], 32), (0, [3000, 700, 5], 32), (512, [2000, 600], 16)])
def test_small_batches_cap_the_runs_of_a_unit(window, lens, cap):
    """Under 4 chunks per workgroup on average, no unit is cut into more than
    16 runs on a sliding layer, 32 on a full one (checked on the plan), and the
    outputs match the oracle."""
    need_gpu()
    from full_attention_amd.cache import PagedKVCache
    from workloads import make_page_pool, normal_bf16
    d = 256 if window else 512
    spec = LayerSpec("sliding" if window else "full", d, 8, 1, window)
    sc = Scenario([spec], None, lens, seed=97)
    starts = [max(0, L - window) if window else 0 for L in lens]
    sc.store(0, starts, [L - s0 for L, s0 in zip(lens, starts)])
    B, maxl = len(lens), max(lens)
    kv = i32(lens)
    plan = sc.cache.decode_plan(0, kv, maxl)
    q = normal_bf16(np.random.default_rng(98), (B, 8, d))
    out = host_bits(sc.cache.decode(0, kv, dev_bits(q), maxl, plan=plan))
    torch.cuda.synchronize()
    head, recs, soff, _ = _read_plan(plan, B, maxl)
    assert head[2] == 0                                   # unit-aligned
    busy = recs[:, 0] < recs[:, 1]
    units = recs[busy, 2]
    runs = np.bincount(units, minlength=B)
    L = np.array(lens)
    n = (L + 15) // 16 - (np.maximum(0, L - window) // 16 if window else 0)
    assert -(-int(n.sum()) // 512) < 4                     # the small-batch case
    assert runs.max() <= cap and (runs[n > cap] > 1).all(), runs
    ref = np.stack([sc.oracle.decode(0, b, q[b], Lb) for b, Lb in enumerate(lens)])
    assert_close(out, ref)


def test_merges_inside_and_across_xcd_blocks():
    """The plan gives each XCD (the workgroups of one class mod 8) a block of
    consecutive runs, the busy runs shared out evenly; a unit whose runs lie in
    one block merges through that XCD's L2, the others through memory.  The
    E2B full-layer length mix has units of both kinds (checked on the plan);
    four short sequences added to it give single-workgroup units.  Every output
    matches the oracle."""
    need_gpu()
    from workloads import e2b_decode_workload
    lens = list(np.array(e2b_decode_workload().cached_lens[:60]) + 1) + [5, 17, 100, 250]
    spec = LayerSpec("full", 512, 8, 1, 0)
    sc = Scenario([spec], None, lens, seed=47)
    sc.store(0, [0] * len(lens), lens)
    B, maxl = len(lens), max(lens)
    kv = i32(lens)
    plan = sc.cache.decode_plan(0, kv, maxl)
    q = normal_bf16(np.random.default_rng(8), (B, 8, 512))
    out = host_bits(sc.cache.decode(0, kv, dev_bits(q), maxl, plan=plan))
    torch.cuda.synchronize()
    head, recs, _, _ = _read_plan(plan, B, maxl)
    assert head[2] == 0                                   # the unit-aligned split
    busy = recs[:, 0] < recs[:, 1]
    spans = {(int(recs[w, 5]), int(recs[w, 6]), int(recs[w, 8])) for w in np.nonzero(busy)[0]}
    inside = [s for s in spans if s[0] < s[1] and s[2] == 1]
    across = [s for s in spans if s[0] < s[1] and s[2] == 0]
    single = [s for s in spans if s[0] == s[1]]
    assert inside and across and single, (len(inside), len(across), len(single))
    ref = np.stack([sc.oracle.decode(0, b, q[b], L) for b, L in enumerate(lens)])
    assert_close(out, ref)


@pytest.mark.parametrize("d,hq,hkv,kv_dtype,lens,local", [
    (512, 16, 1, "bf16", [4000] * 8, 1),        # 63 runs a unit, each unit in one XCD block
    (256, 16, 2, "int8", [4000] * 8, 1),        # 32 runs a unit, two units a block
    (512, 8, 1, "bf16", [4000], 0),             # 32 runs over every block
    (256, 8, 1, "fp8", [9000, 3000, 700], 0),   # 32 + 11 + 3 runs
])
def test_units_of_many_runs_merge(d, hq, hkv, kv_dtype, lens, local):
    """Units cut into many runs (up to 63, so that the merge takes several
    batches of 7 partials at D 512, 8 at 256, with a ragged last one), merged
    inside one XCD's L2 or across XCDs as the case says (checked on the plan).
    The outputs match the oracle and are bit-identical over three calls, the
    placement check finds nothing, and the arrival counters are zero after
    each call."""
    need_gpu()
    from full_attention_amd import pakv
    gs = 7 if d == 512 else 8
    sc = _decode_case(d, hq, hkv, 0, kv_dtype, lens, seed=59)
    B, maxl = len(lens), max(lens)
    kv = i32(lens)
    plan = sc.cache.decode_plan(0, kv, maxl)
    torch.cuda.synchronize()
    head, recs, _, _ = _read_plan(plan, B, maxl, hkv=hkv)
    assert head[2] == 0                                   # unit-aligned
    busy = recs[:, 0] < recs[:, 1]
    spans = {(int(recs[w, 5]), int(recs[w, 6]), int(recs[w, 8])) for w in np.nonzero(busy)[0]}
    many = [sp for sp in spans if sp[1] - sp[0] + 1 > 2 * gs]
    assert many and all(sp[2] == local for sp in many), sorted(spans)
    q = normal_bf16(np.random.default_rng(60), (B, hq, d))
    ref = np.stack([sc.oracle.decode(0, b, q[b], L) for b, L in enumerate(lens)])
    pakv.set_decode_checks(pakv.CHECK_XCD_PLACEMENT)
    try:
        first = None
        for _ in range(3):
            out = host_bits(sc.cache.decode(0, kv, dev_bits(q), maxl, plan=plan))
            torch.cuda.synchronize()
            if first is None:
                assert_close(out, ref)
                first = out
            else:
                assert np.array_equal(out, first)
            assert sc.cache.status() == 0
            w = sc.cache._workspace.cpu().numpy()
            assert not w[4:256 + 4 * 8192].any()
    finally:
        pakv.set_decode_checks(0)


def test_workgroups_of_one_class_mod_8_share_an_xcd():
    """The decode merge keeps a unit's partials in one XCD's L2 when all of its
    workgroups lie in one class of i mod 8, which is correct only if those
    workgroups always run on one XCD (the dispatcher hands workgroups to the
    XCDs in turn).  Checked over 20 launches of the decode grid's size."""
    need_gpu()
    from full_attention_amd import pakv
    n = 512
    out = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    for _ in range(20):
        out.fill_(-1)
        pakv.workgroup_xcds(out, n)
        ids = out.cpu().numpy()
        assert (ids >= 0).all()
        for c in range(8):
            assert len(set(ids[c::8].tolist())) == 1, (c, sorted(set(ids[c::8].tolist())))


def test_stream_k_runs_cross_units_and_xcd_blocks():
    """Many short sequences and one long one: no unit-aligned split fits the
    grid, so runs are equal pieces of the stream that cross units (a run
    writes a partial for each unit it touches).  Units merged inside one XCD's
    block of 64 workgroups and units spread over two blocks both occur (checked
    on the plan); every output matches the oracle."""
    need_gpu()
    lens = [3000] + [40 + (i % 7) for i in range(700)]
    spec = LayerSpec("full", 256, 8, 1, 0)
    sc = Scenario([spec], None, lens, seed=53)
    sc.store(0, [0] * len(lens), lens)
    B, maxl = len(lens), max(lens)
    kv = i32(lens)
    plan = sc.cache.decode_plan(0, kv, maxl)
    q = normal_bf16(np.random.default_rng(12), (B, 8, 256))
    out = host_bits(sc.cache.decode(0, kv, dev_bits(q), maxl, plan=plan))
    torch.cuda.synchronize()
    head, _, soff, _ = _read_plan(plan, B, maxl)
    per = int(head[2])
    assert per > 0                                        # stream-K
    n = (np.array(lens) + 15) // 16
    w0, w1 = soff[:B] // per, (soff[:B] + n - 1) // per
    assert np.any((w0 != w1) & (w0 // 64 == w1 // 64)) and np.any(w0 // 64 != w1 // 64)
    ref = np.stack([sc.oracle.decode(0, b, q[b], L) for b, L in enumerate(lens)])
    assert_close(out, ref)


@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("q_scale", [2.0 ** -20, 2.0 ** 6, 2.0 ** 80])
def test_int8_decode_with_tiny_and_large_queries(d, q_scale):
    """int8 scores run on fp16 MFMAs with Q scaled per wavefront by a power of
    two: queries 2^20 times smaller (near-uniform weights), 2^6 times larger
    (peaked weights) or 2^80 times larger (far past fp16's range: one-hot
    weights) than N(0, 1) still match the oracle; heads of one unit differ in
    magnitude by 2^10."""
    need_gpu()
    spec = LayerSpec("full", d, 8, 1, 0, kv_dtype="int8")
    lens = [1, 33, 700, 2049]
    sc = Scenario([spec], None, lens, seed=417 if q_scale < 1 else 418)
    sc.store(0, [0] * len(lens), lens)
    q = normal_bf16(sc.rng, (len(lens), 8, d))
    qf = bf16_to_f32(q) * np.float32(q_scale)
    qf[:, :4] *= np.float32(2.0 ** 10) if q_scale < 1 else np.float32(2.0 ** -10)
    q = bf16_from_f32(qf)                       # power-of-two scaling: the same bf16 mantissas
    out = host_bits(sc.cache.decode(0, i32(lens), dev_bits(q), max(lens)))
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        assert_close(out[b], sc.oracle.decode(0, b, q[b], L), f"int8 d={d} q x {q_scale} seq {b}")
