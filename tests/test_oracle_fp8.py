"""Pins for oracle.fp8_pth (the fp8 per-token-head reading: OCP E4M3 codes,
scale = amax / 448, nearest even, saturating).

* Hand-worked codes from the E4M3 definition: the largest value, one, the
  smallest subnormal, halfway cases that go to the even mantissa, and the
  saturation of values past 448.
* A library routine: torch's float8_e4m3fn conversion (CPU) gives the same
  codes on every bf16 value within [-448, 448] and on a million float32 draws
  (torch turns values past 480 into NaN; the reading saturates instead, so
  the comparison stops at the range where both are defined).
* Exhaustive decode: the 254 finite codes are strictly ordered and every one
  re-encodes to itself.
* Per-row properties: the largest magnitude of a row maps to +-448 exactly,
  the reconstruction error stays within half a step of the E4M3 grid, an
  all-zero row gives zero scale and codes, and the row costs D + 4 bytes.
"""

import numpy as np
import pytest
import torch

from oracle.fp8_pth import FP8_MAX, dequantise_rows, e4m3_encode, e4m3_value, quantise_rows
from workloads import bf16_to_f32, normal_bf16


def test_hand_worked_codes():
    y = np.array([448.0, -448.0, 1.0, 2.0 ** -9, 2.0 ** -10, 0.75 * 2.0 ** -9, 1.0625, 1.1875, -3.3, 0.0,
                  464.0, 470.0, 1000.0, 2.0 ** -6, 15.0 * 2.0 ** -10], dtype=np.float32)
    want = [0x7E, 0xFE, 0x38, 0x01, 0x00, 0x01, 0x38, 0x3A, 0xC5, 0x00,
            0x7E, 0x7E, 0x7E, 0x08, 0x08]
    # 1.0625 lies halfway between 1.0 (mantissa 000) and 1.125 (001): even, 1.0
    # 1.1875 lies halfway between 1.125 (001) and 1.25 (010): even, 1.25
    # -3.3 -> -3.25 = -(1 + 5/8) * 2; 15 * 2^-10 rounds up to 2^-6, the first normal
    # 464, 470, 1000: past 448 they saturate
    assert e4m3_encode(y).tolist() == want
    assert e4m3_value(np.array([0x7E, 0x38, 0x01, 0x08, 0xC5], dtype=np.uint8)).tolist() == \
        [448.0, 1.0, 2.0 ** -9, 2.0 ** -6, -3.25]


def test_matches_torch_float8_e4m3fn_where_both_are_defined():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(b)
    f = f[np.isfinite(f) & (np.abs(f) <= FP8_MAX)]
    theirs = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(f), theirs)
    r = (np.random.default_rng(0).standard_normal(1_000_000) * 100).astype(np.float32)
    r = r[np.abs(r) <= FP8_MAX]
    theirs = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(r), theirs)


def test_every_finite_code_decodes_and_reencodes_to_itself():
    codes = np.arange(256, dtype=np.uint8)
    v = e4m3_value(codes)
    finite = np.isfinite(v)
    assert (~finite).sum() == 2 and set(codes[~finite].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(e4m3_encode(v[finite]), codes[finite])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0 and pos[1] == 2.0 ** -9


@pytest.mark.parametrize("d", [256, 512])
def test_row_properties(d):
    rng = np.random.default_rng(d)
    x = bf16_to_f32(normal_bf16(rng, (300, d)))
    codes, scale = quantise_rows(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    vals = e4m3_value(codes)
    assert np.all(np.abs(vals).max(axis=1) == FP8_MAX)
    xh = dequantise_rows(codes, scale)
    # half a step of the grid at the value's binade (relative 2^-4), or half a
    # subnormal step (2^-10) times the scale
    y = np.abs(x.astype(np.float64)) / scale[:, None]
    step = np.where(y >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(x - xh) <= (0.5 * step + 1e-6 * y) * scale[:, None])
    # bytes per row: D one-byte codes and one float32 scale
    assert codes[0].nbytes + scale[:1].nbytes == d + 4


def test_zero_row():
    codes, scale = quantise_rows(np.zeros((2, 16), dtype=np.float32))
    assert not codes.any() and not scale.any()
    assert not dequantise_rows(codes, scale).any()
