"""The fp8 per-token-head format, K=V layers (one slab, values derived from
the keys in-kernel), 8-bit and K=V extend, and extend with the chunk given as
packed rows, against the oracle.

* fp8 store: codes and scales bit-exact against the oracle's encoding
  (oracle/fp8_pth.py), special rows included.
* fp8 decode of every code: a value page holding all 254 finite E4M3 codes
  with scale 1, read by a one-key decode, returns each code's value exactly.
* decode and extend parity (2e-2 abs + 1e-2 rel) for fp8, int8 extend, K=V
  at both head dims, with sliding windows and GQA groups.
* packed extend: the chunk's slab slots are never written (they hold NaN), so
  any read of them would show; 8-bit prefixes with exact bf16 chunks; K=V; a
  shared layer given its source's rows.
"""

import zlib

import numpy as np
import pytest
import torch

from oracle import e4m3_value, fp8_pth
from workloads import LayerSpec, bf16_from_f32, bf16_to_f32, normal_bf16

from gpu_helpers import Scenario, assert_close, dev_bits, host_bits, i32, need_gpu

pytestmark = pytest.mark.gpu

LENS = [1, 2, 15, 16, 17, 31, 33, 100, 129, 257, 700]


@pytest.mark.parametrize("d", [256, 512])
def test_store_fp8_matches_oracle_encoding(d):
    need_gpu()
    spec = LayerSpec("sliding", d, 8, 1, 64, kv_dtype="fp8")
    caps = [40, 70]
    sc = Scenario([spec], None, caps, seed=521 + d)
    starts, counts = [0, 5], [40, 65]
    total = sum(counts)
    k = normal_bf16(sc.rng, (total, 1, d))
    v = normal_bf16(sc.rng, (total, 1, d))
    k[0] = 0                                             # all-zero row
    row = np.zeros(d, np.float32)
    row[:6] = [448.0, 1.0625, -1.1875, 2.0 ** -9, 2.0 ** -10, -3.3]   # amax 448: scale 1
    k[1, 0] = bf16_from_f32(row)
    v[2, 0, :] = bf16_from_f32(np.full(d, -0.0, np.float32))           # negative zeros
    v[2, 0, 0] = bf16_from_f32(np.float32(5.0))
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sc.cache.store(0, i32(cu), i32(starts), dev_bits(k), dev_bits(v))
    torch.cuda.synchronize()
    kc, vc, ksc, vsc = [t.cpu().numpy().view(np.uint8) if t.dtype == torch.int8 else t.cpu().numpy()
                        for t in sc.cache.slabs[0]]
    kq, kscale = fp8_pth.quantise_rows(bf16_to_f32(k))
    vq, vscale = fp8_pth.quantise_rows(bf16_to_f32(v))
    table = sc.pool.page_table
    for b in range(2):
        for i in range(counts[b]):
            pos, t = starts[b] + i, cu[b] + i
            page, slot = table[b, pos // 16], pos % 16
            assert np.array_equal(kc[page, 0, slot, :], kq[t, 0]), (b, i)
            assert np.array_equal(vc[page, 0, :, slot], vq[t, 0]), (b, i)
            assert kscale[t, 0].tobytes() == ksc[page, 0, slot].tobytes()
            assert vscale[t, 0].tobytes() == vsc[page, 0, slot].tobytes()
    assert kc[table[0, 0], 0, 1, :6].tolist() == [0x7E, 0x38, 0xBA, 0x01, 0x00, 0xC5]


@pytest.mark.parametrize("d", [256, 512])
def test_fp8_decode_reads_every_code_exactly(d):
    """One key per sequence: the output is that key's value row, code * 1."""
    need_gpu()
    spec = LayerSpec("full", d, 8, 1, 0, kv_dtype="fp8")
    sc = Scenario([spec], None, [1], seed=7)
    k, v, ks, vs = sc.cache.slabs[0]
    page = int(sc.pool.page_table[0][0])
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    codes = np.array([finite[i % len(finite)] for i in range(d)], dtype=np.uint8)
    vv = v.view(torch.uint8)
    vv[page, 0, :, 0] = torch.from_numpy(codes).cuda()
    k.view(torch.uint8)[page, 0, 0, :] = 0x38         # key codes 1.0
    ks[page, 0, 0] = 1.0
    vs[page, 0, 0] = 1.0
    q = dev_bits(normal_bf16(np.random.default_rng(1), (1, 8, d)))
    out = host_bits(sc.cache.decode(0, i32([1]), q, 1))
    torch.cuda.synchronize()
    want = e4m3_value(codes)                 # every E4M3 value is a bf16 value
    for h in range(8):
        # compared as numbers: code 0x80 (-0) comes out as +0 (the
        # accumulator starts at +0)
        assert np.array_equal(bf16_to_f32(out[0, h]).astype(np.float64), want), h


@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("hq,hkv", [(8, 1), (16, 8), (16, 2)])
@pytest.mark.parametrize("window", [0, 7, 32])
def test_fp8_decode_matches_oracle(d, hq, hkv, window):
    need_gpu()
    spec = LayerSpec("sliding" if window else "full", d, hq, hkv, window, kv_dtype="fp8")
    sc = Scenario([spec], None, LENS, seed=zlib.crc32(repr(("fp8", d, hq, hkv, window)).encode()) % 10000)
    starts = [max(0, L - window) if window else 0 for L in LENS]
    sc.store(0, starts, [L - s for L, s in zip(LENS, starts)])
    got, ref, _ = sc.decode(0, LENS)
    assert_close(got, ref, f"fp8 decode d={d} hq={hq} hkv={hkv} W={window}")


@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("hq,hkv", [(8, 1), (16, 2), (4, 4)])
@pytest.mark.parametrize("window", [0, 1, 32])
def test_k_eq_v_decode_matches_oracle(d, hq, hkv, window):
    """K=V layers store keys only; the values are the keys divided by their root
    mean square (eps 1e-6), derived in the kernel."""
    need_gpu()
    spec = LayerSpec("sliding" if window else "full", d, hq, hkv, window, k_eq_v=True)
    sc = Scenario([spec], None, LENS, seed=zlib.crc32(repr(("keqv", d, hq, hkv, window)).encode()) % 10000)
    assert sc.cache.slabs[0][1] is None                  # no V slab
    starts = [max(0, L - window) if window else 0 for L in LENS]
    sc.store(0, starts, [L - s for L, s in zip(LENS, starts)])
    got, ref, _ = sc.decode(0, LENS)
    assert_close(got, ref, f"K=V decode d={d} hq={hq} hkv={hkv} W={window}")


EXT_PREFIXES = [0, 17, 100, 5, 64]
EXT_CHUNKS = [64, 33, 1, 0, 70]


@pytest.mark.parametrize("fmt", ["int8", "fp8", "keqv"])
@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("hq,hkv,window", [(8, 1, 0), (16, 2, 32), (3, 1, 5), (8, 1, 1)])
def test_extend_formats_match_oracle(fmt, d, hq, hkv, window):
    need_gpu()
    kw = dict(k_eq_v=True) if fmt == "keqv" else dict(kv_dtype=fmt)
    spec = LayerSpec("sliding" if window else "full", d, hq, hkv, window, **kw)
    caps = [p + n for p, n in zip(EXT_PREFIXES, EXT_CHUNKS)]
    sc = Scenario([spec], None, [max(c, 1) for c in caps],
                  seed=zlib.crc32(repr(("ext", fmt, d, hq, hkv, window)).encode()) % 1000)
    sc.store(0, [0] * len(caps), caps)
    for got, ref, b in sc.extend(0, EXT_PREFIXES, EXT_CHUNKS):
        assert_close(got, ref, f"{fmt} extend d={d} hq={hq} hkv={hkv} W={window} seq {b}")


def _packed_case(spec_kw, d, hq, hkv, window, seed, shared=False):
    """Prefix rows stored; the chunk's rows drawn but never stored (their slab
    slots keep the NaN sentinel); extend_packed against the oracle's."""
    kind = "sliding" if window else "full"
    specs = [LayerSpec(kind, d, hq, hkv, window, **spec_kw)]
    if shared:
        specs.append(LayerSpec(kind, d, hq, hkv, window, **spec_kw))
    sc = Scenario(specs, 1 if shared else None, [max(p + n, 1) for p, n in zip(EXT_PREFIXES, EXT_CHUNKS)], seed=seed)
    sc.store(0, [0] * len(EXT_PREFIXES), EXT_PREFIXES)
    layer = 1 if shared else 0
    total = sum(EXT_CHUNKS)
    k = normal_bf16(sc.rng, (total, hkv, d))
    v = normal_bf16(sc.rng, (total, hkv, d))
    q = normal_bf16(sc.rng, (total, hq, d))
    cu = np.concatenate([[0], np.cumsum(EXT_CHUNKS)]).astype(np.int32)
    max_kv = max(p + n for p, n in zip(EXT_PREFIXES, EXT_CHUNKS))
    kve = spec_kw.get("k_eq_v", False)
    out = host_bits(sc.cache.extend_packed(layer, i32(cu), i32(EXT_PREFIXES), dev_bits(q), dev_bits(k),
                                           None if kve else dev_bits(v), max(EXT_CHUNKS), max_kv))
    torch.cuda.synchronize()
    for b, n in enumerate(EXT_CHUNKS):
        if n == 0:
            continue
        ref = sc.oracle.extend_packed(layer, b, q[cu[b]:cu[b + 1]], EXT_PREFIXES[b], k[cu[b]:cu[b + 1]],
                                      None if kve else v[cu[b]:cu[b + 1]])
        assert_close(out[cu[b]:cu[b + 1]], ref, f"packed {spec_kw} d={d} W={window} seq {b}")


@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("fmt", ["bf16", "int8", "fp8", "keqv"])
@pytest.mark.parametrize("hq,hkv,window", [(8, 1, 0), (16, 2, 24)])
def test_extend_packed_reads_only_the_prefix_from_the_slab(d, fmt, hq, hkv, window):
    need_gpu()
    kw = dict(k_eq_v=True) if fmt == "keqv" else dict(kv_dtype=fmt)
    _packed_case(kw, d, hq, hkv, window, seed=zlib.crc32(repr(("packed", d, fmt, hq, window)).encode()) % 1000)


def test_extend_packed_on_a_shared_layer():
    need_gpu()
    _packed_case(dict(kv_dtype="int8"), 256, 8, 1, 32, seed=77, shared=True)
