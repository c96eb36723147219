"""The staged extend (pakv_paged_attn_extend_staged): 8-bit slabs, K=V layers
and packed chunks staged into a workspace, then run on the bf16 MFMA kernel
with per-token key and value scales, against the oracle.

* every format, both head dims, full and sliding layers (windows 1, 5, 32),
  GQA groups, ragged chunks (an empty one among them), a context of several
  32-key tiles with a ragged tail;
* packed chunks (the chunk's slab slots hold the NaN sentinel, so a read of
  them would show), a shared layer given its source's rows;
* the workspace is filled with NaN bytes before each call: pages the staging
  pass does not write must never reach the arithmetic;
* a smaller call after a larger one on the same (stale) workspace;
* agreement with the unstaged call's kernel and bit-identical repeats.
"""

import zlib

import numpy as np
import pytest
import torch

from workloads import LayerSpec, bf16_to_f32, normal_bf16

from gpu_helpers import Scenario, assert_close, dev_bits, host_bits, i32, need_gpu

pytestmark = pytest.mark.gpu

EXT_PREFIXES = [0, 17, 100, 5, 64]
EXT_CHUNKS = [64, 33, 1, 0, 70]
LONG_PREFIXES = [0, 700, 300, 1000, 33]
LONG_CHUNKS = [300, 129, 257, 0, 200]


def _spec(fmt, d, hq, hkv, window):
    kw = dict(k_eq_v=True) if fmt == "keqv" else dict(kv_dtype=fmt)
    return LayerSpec("sliding" if window else "full", d, hq, hkv, window, **kw)


def _poison_workspace(sc, layer, nseq, max_q, max_kv, packed):
    """A NaN-filled workspace (0xFF bytes: NaN as bf16 and as float32) of the
    size the call needs, for the cache to use."""
    from full_attention_amd import pakv
    need = pakv.extend_staging_bytes(sc.cache.map, layer, nseq, max_q, max_kv, packed)
    sc.cache._stage_ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    return need


def _staged(sc, layer, prefixes, chunks, poison=True, q=None):
    s = sc.specs[layer]
    total = int(sum(chunks))
    if q is None:
        q = normal_bf16(sc.rng, (max(total, 1), s.num_q_heads, s.head_dim))[:total]
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    max_kv = int(max(p + n for p, n in zip(prefixes, chunks)))
    if poison:
        _poison_workspace(sc, layer, len(chunks), int(max(chunks)), max_kv, False)
    out = sc.cache.extend_staged(layer, i32(cu), i32(prefixes), dev_bits(q), int(max(chunks)), max_kv)
    torch.cuda.synchronize()
    return host_bits(out), q, cu


def _check(sc, layer, prefixes, chunks, got, q, cu, what):
    for b, n in enumerate(chunks):
        if n == 0:
            continue
        ref = sc.oracle.extend(layer, b, q[cu[b]:cu[b + 1]], int(prefixes[b]))
        assert_close(got[cu[b]:cu[b + 1]], ref, f"{what} seq {b}")


@pytest.mark.parametrize("fmt", ["int8", "fp8", "keqv"])
@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("hq,hkv,window", [(8, 1, 0), (16, 2, 32), (3, 1, 5), (8, 1, 1)])
def test_staged_formats_match_oracle(fmt, d, hq, hkv, window):
    need_gpu()
    caps = [p + n for p, n in zip(EXT_PREFIXES, EXT_CHUNKS)]
    sc = Scenario([_spec(fmt, d, hq, hkv, window)], None, [max(c, 1) for c in caps],
                  seed=zlib.crc32(repr(("staged", fmt, d, hq, hkv, window)).encode()) % 1000)
    sc.store(0, [0] * len(caps), caps)
    got, q, cu = _staged(sc, 0, EXT_PREFIXES, EXT_CHUNKS)
    _check(sc, 0, EXT_PREFIXES, EXT_CHUNKS, got, q, cu, f"staged {fmt} d={d} hq={hq} hkv={hkv} W={window}")


@pytest.mark.parametrize("fmt", ["int8", "fp8", "keqv"])
@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("window", [0, 512])
def test_staged_long_context_matches_oracle(fmt, d, window):
    """Contexts of up to 1000 keys (many tiles, pages of the window's start
    not aligned to a tile), chunks of up to 300 rows (several row blocks)."""
    need_gpu()
    caps = [p + n for p, n in zip(LONG_PREFIXES, LONG_CHUNKS)]
    sc = Scenario([_spec(fmt, d, 8, 1, window)], None, caps,
                  seed=zlib.crc32(repr(("staged-long", fmt, d, window)).encode()) % 1000)
    sc.store(0, [0] * len(caps), caps)
    got, q, cu = _staged(sc, 0, LONG_PREFIXES, LONG_CHUNKS)
    _check(sc, 0, LONG_PREFIXES, LONG_CHUNKS, got, q, cu, f"staged long {fmt} d={d} W={window}")


def _packed_staged(spec_kw, d, hq, hkv, window, seed, shared=False):
    kind = "sliding" if window else "full"
    specs = [LayerSpec(kind, d, hq, hkv, window, **spec_kw)]
    if shared:
        specs.append(LayerSpec(kind, d, hq, hkv, window, **spec_kw))
    sc = Scenario(specs, 1 if shared else None, [max(p + n, 1) for p, n in zip(EXT_PREFIXES, EXT_CHUNKS)], seed=seed)
    sc.store(0, [0] * len(EXT_PREFIXES), EXT_PREFIXES)     # the chunks' slots keep the NaN sentinel
    layer = 1 if shared else 0
    total = sum(EXT_CHUNKS)
    k = normal_bf16(sc.rng, (total, hkv, d))
    v = normal_bf16(sc.rng, (total, hkv, d))
    q = normal_bf16(sc.rng, (total, hq, d))
    cu = np.concatenate([[0], np.cumsum(EXT_CHUNKS)]).astype(np.int32)
    max_kv = max(p + n for p, n in zip(EXT_PREFIXES, EXT_CHUNKS))
    kve = spec_kw.get("k_eq_v", False)
    _poison_workspace(sc, layer, len(EXT_CHUNKS), max(EXT_CHUNKS), max_kv, True)
    out = host_bits(sc.cache.extend_staged(layer, i32(cu), i32(EXT_PREFIXES), dev_bits(q), max(EXT_CHUNKS), max_kv,
                                           k_ext=dev_bits(k), v_ext=None if kve else dev_bits(v)))
    torch.cuda.synchronize()
    for b, n in enumerate(EXT_CHUNKS):
        if n == 0:
            continue
        ref = sc.oracle.extend_packed(layer, b, q[cu[b]:cu[b + 1]], EXT_PREFIXES[b], k[cu[b]:cu[b + 1]],
                                      None if kve else v[cu[b]:cu[b + 1]])
        assert_close(out[cu[b]:cu[b + 1]], ref, f"staged packed {spec_kw} d={d} W={window} seq {b}")


@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("fmt", ["bf16", "int8", "fp8", "keqv"])
@pytest.mark.parametrize("hq,hkv,window", [(8, 1, 0), (16, 2, 24)])
def test_staged_packed_reads_only_the_prefix_from_the_slab(d, fmt, hq, hkv, window):
    need_gpu()
    kw = dict(k_eq_v=True) if fmt == "keqv" else dict(kv_dtype=fmt)
    _packed_staged(kw, d, hq, hkv, window, seed=zlib.crc32(repr(("staged-packed", d, fmt, hq, window)).encode()) % 1000)


def test_staged_packed_on_a_shared_layer():
    need_gpu()
    _packed_staged(dict(kv_dtype="int8"), 256, 8, 1, 32, seed=78, shared=True)


@pytest.mark.parametrize("fmt", ["int8", "keqv"])
def test_staged_smaller_call_after_a_larger_one(fmt):
    """The cache keeps the larger call's workspace; the smaller call's pages
    sit elsewhere in it, over stale staged data."""
    need_gpu()
    caps = [p + n for p, n in zip(LONG_PREFIXES, LONG_CHUNKS)]
    sc = Scenario([_spec(fmt, 512, 8, 1, 0)], None, caps, seed=91)
    sc.store(0, [0] * len(caps), caps)
    got, q, cu = _staged(sc, 0, LONG_PREFIXES, LONG_CHUNKS)
    _check(sc, 0, LONG_PREFIXES, LONG_CHUNKS, got, q, cu, f"{fmt} large")
    small_p, small_n = [5, 0, 40], [20, 7, 0]
    got, q, cu = _staged(sc, 0, small_p, small_n, poison=False)
    _check(sc, 0, small_p, small_n, got, q, cu, f"{fmt} small after large")


@pytest.mark.parametrize("fmt", ["int8", "fp8", "keqv"])
@pytest.mark.parametrize("d,window", [(256, 512), (512, 0)])
def test_staged_agrees_with_the_unstaged_kernel_and_repeats_exactly(fmt, d, window):
    """The two kernels apply the same scales in different places (the general
    kernel scales the value rows, the staged one the weights before they are
    rounded to bf16); their outputs agree within the oracle tolerance, and
    repeats of the staged call are bit-identical."""
    need_gpu()
    caps = [p + n for p, n in zip(LONG_PREFIXES, LONG_CHUNKS)]
    sc = Scenario([_spec(fmt, d, 8, 1, window)], None, caps, seed=zlib.crc32(repr(("agree", fmt, d)).encode()) % 1000)
    sc.store(0, [0] * len(caps), caps)
    s = sc.specs[0]
    total = sum(LONG_CHUNKS)
    q = normal_bf16(sc.rng, (total, s.num_q_heads, d))
    cu = np.concatenate([[0], np.cumsum(LONG_CHUNKS)]).astype(np.int32)
    max_kv = max(p + n for p, n in zip(LONG_PREFIXES, LONG_CHUNKS))
    general = host_bits(sc.cache.extend(0, i32(cu), i32(LONG_PREFIXES), dev_bits(q), max(LONG_CHUNKS), max_kv))
    runs = [host_bits(sc.cache.extend_staged(0, i32(cu), i32(LONG_PREFIXES), dev_bits(q), max(LONG_CHUNKS), max_kv))
            for _ in range(3)]
    torch.cuda.synchronize()
    assert all(np.array_equal(runs[0], r) for r in runs[1:])
    a = bf16_to_f32(runs[0]).astype(np.float64)
    g = bf16_to_f32(general).astype(np.float64)
    assert (np.abs(a - g) <= 2e-2 + 1e-2 * np.abs(g)).all(), np.abs(a - g).max()


@pytest.mark.parametrize("fmt,d,window", [("int8", 256, 32), ("keqv", 512, 0), ("fp8", 512, 0)])
def test_shared_layer_reuses_its_source_staging(fmt, d, window):
    """A KV-shared layer called with stage=False on the workspace its source's
    call staged: bit-identical to its own staging pass, and matches the
    oracle."""
    need_gpu()
    caps = [p + n for p, n in zip(LONG_PREFIXES, LONG_CHUNKS)]
    specs = [_spec(fmt, d, 8, 1, window), _spec(fmt, d, 8, 1, window)]
    sc = Scenario(specs, 1, caps, seed=zlib.crc32(repr(("reuse", fmt, d)).encode()) % 1000)
    sc.store(0, [0] * len(caps), caps)
    total = sum(LONG_CHUNKS)
    cu = np.concatenate([[0], np.cumsum(LONG_CHUNKS)]).astype(np.int32)
    max_q, max_kv = max(LONG_CHUNKS), max(p + n for p, n in zip(LONG_PREFIXES, LONG_CHUNKS))
    need = sc.cache.staging_bytes(0, len(caps), max_q, max_kv)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    args = (i32(cu), i32(LONG_PREFIXES))
    q0 = normal_bf16(sc.rng, (total, 8, d))
    q1 = normal_bf16(sc.rng, (total, 8, d))
    sc.cache.extend_staged(0, *args, dev_bits(q0), max_q, max_kv, workspace=ws, stage=True)
    reused = host_bits(sc.cache.extend_staged(1, *args, dev_bits(q1), max_q, max_kv, workspace=ws, stage=False))
    fresh = host_bits(sc.cache.extend_staged(1, *args, dev_bits(q1), max_q, max_kv))
    torch.cuda.synchronize()
    assert np.array_equal(reused, fresh)
    _check(sc, 1, LONG_PREFIXES, LONG_CHUNKS, reused, q1, cu, f"reused staging {fmt} d={d} W={window}")


def _random_case(seed):
    """A seeded random staged-extend case: format, head dim, GQA shape,
    window, batch, prefixes and chunk lengths (an empty chunk possible),
    packed or not."""
    r = np.random.default_rng(seed)
    fmt = ["int8", "fp8", "keqv", "bf16"][r.integers(0, 4)]
    packed = fmt == "bf16" or bool(r.integers(0, 2))
    d = int(r.choice([256, 512]))
    hkv = int(r.choice([1, 2, 4]))
    hq = hkv * int(r.choice([1, 2, 3, 8]))
    window = int(r.choice([0, 0, 1, 2, 17, 32, 33, 100, 512]))
    B = int(r.integers(1, 6))
    prefixes = [int(x) for x in r.integers(0, 300, B)]
    chunks = [int(x) for x in r.integers(0, 120, B)]
    if r.integers(0, 3) == 0:
        chunks[int(r.integers(0, B))] = 0
    if sum(chunks) == 0:
        chunks[0] = 1
    return fmt, packed, d, hq, hkv, window, prefixes, chunks


@pytest.mark.parametrize("seed", range(24))
def test_staged_random_shapes_match_oracle(seed):
    need_gpu()
    fmt, packed, d, hq, hkv, window, prefixes, chunks = _random_case(9000 + seed)
    what = f"seed {seed}: {fmt} packed={packed} d={d} hq={hq} hkv={hkv} W={window} P={prefixes} n={chunks}"
    print(what, flush=True)
    caps = [max(p + n, 1) for p, n in zip(prefixes, chunks)]
    sc = Scenario([_spec(fmt, d, hq, hkv, window)], None, caps, seed=seed)
    kve = fmt == "keqv"
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    total = int(cu[-1])
    max_q, max_kv = max(chunks), max(p + n for p, n in zip(prefixes, chunks))
    q = normal_bf16(sc.rng, (total, hq, d))
    if packed:
        sc.store(0, [0] * len(caps), prefixes)
        k = normal_bf16(sc.rng, (total, hkv, d))
        v = normal_bf16(sc.rng, (total, hkv, d))
        _poison_workspace(sc, 0, len(chunks), max_q, max_kv, True)
        got = host_bits(sc.cache.extend_staged(0, i32(cu), i32(prefixes), dev_bits(q), max_q, max_kv,
                                               k_ext=dev_bits(k), v_ext=None if kve else dev_bits(v)))
    else:
        sc.store(0, [0] * len(caps), [p + n for p, n in zip(prefixes, chunks)])
        _poison_workspace(sc, 0, len(chunks), max_q, max_kv, False)
        got = host_bits(sc.cache.extend_staged(0, i32(cu), i32(prefixes), dev_bits(q), max_q, max_kv))
    torch.cuda.synchronize()
    for b, n in enumerate(chunks):
        if n == 0:
            continue
        if packed:
            ref = sc.oracle.extend_packed(0, b, q[cu[b]:cu[b + 1]], prefixes[b], k[cu[b]:cu[b + 1]],
                                          None if kve else v[cu[b]:cu[b + 1]])
        else:
            ref = sc.oracle.extend(0, b, q[cu[b]:cu[b + 1]], prefixes[b])
        assert_close(got[cu[b]:cu[b + 1]], ref, f"{what} seq {b}")


@pytest.mark.parametrize("fmt,packed", [("int8", False), ("keqv", True)])
def test_staged_extend_in_graph_replays(fmt, packed):
    """The staged call (staging pass + scaled kernel) captured into a HIP graph:
    every replay, with unrelated eager work between replays, gives the eager
    call's bits (the call launches no memset and allocates nothing)."""
    need_gpu()
    caps = [p + n for p, n in zip(LONG_PREFIXES, LONG_CHUNKS)]
    sc = Scenario([_spec(fmt, 512, 8, 1, 0)], None, caps, seed=303 if packed else 302)
    sc.store(0, [0] * len(caps), LONG_PREFIXES if packed else caps)
    total = sum(LONG_CHUNKS)
    cu = i32(np.concatenate([[0], np.cumsum(LONG_CHUNKS)]))
    pre = i32(LONG_PREFIXES)
    max_q, max_kv = max(LONG_CHUNKS), max(p + n for p, n in zip(LONG_PREFIXES, LONG_CHUNKS))
    q = dev_bits(normal_bf16(sc.rng, (total, 8, 512)))
    kx = dev_bits(normal_bf16(sc.rng, (total, 1, 512))) if packed else None
    ws = torch.empty(sc.cache.staging_bytes(0, len(caps), max_q, max_kv, packed), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def call():
        sc.cache.extend_staged(0, cu, pre, q, max_q, max_kv, k_ext=kx, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.fill_(0)
        ws.fill_(0xFF)                                   # the replay must restage
        torch.randn(1000, device="cuda").sum()          # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
