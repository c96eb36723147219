"""Pins for oracle.int8_pth: hand-worked rows (round half to even, the
symmetric clamp, the all-zero row), error bounds, and the row size that the
bytes-per-token figures fix (FreeToken PR #898, "End to end": D + 4 bytes)."""

import numpy as np
import pytest

from oracle import quantise_rows, dequantise_rows
from workloads import normal_bf16, bf16_to_f32


def test_hand_worked_rows():
    # amax 127 -> scale exactly 1; 0.5 rounds to the even code 0.
    q, s = quantise_rows(np.array([[1.0, -2.0, 0.5, 127.0]], dtype=np.float32))
    assert s.tolist() == [1.0]
    assert q.tolist() == [[1, -2, 0, 127]]
    # amax 254 -> scale 2; x / scale = 0.5, 1.5, 2.5, -127 -> 0, 2, 2, -127.
    q, s = quantise_rows(np.array([[1.0, 3.0, 5.0, -254.0]], dtype=np.float32))
    assert s.tolist() == [2.0]
    assert q.tolist() == [[0, 2, 2, -127]]
    # all-zero row
    q, s = quantise_rows(np.zeros((1, 8), dtype=np.float32))
    assert s.tolist() == [0.0] and not q.any()
    # a negative extreme maps to -127, never -128
    q, s = quantise_rows(np.array([[-6.0, 1.0]], dtype=np.float32))
    assert q[0, 0] == -127


@pytest.mark.parametrize("d", [256, 512])
def test_properties_on_normal_rows(d):
    rng = np.random.default_rng(7)
    x = bf16_to_f32(normal_bf16(rng, (500, d)))
    x[3] = 0.0
    q, s = quantise_rows(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.abs(q.astype(np.int32)).max() <= 127
    assert (q != -128).all()
    nz = np.abs(x).max(axis=1) > 0
    assert (np.abs(q[nz].astype(np.int32)).max(axis=1) == 127).all()
    assert not q[3].any() and s[3] == 0
    err = np.abs(x.astype(np.float64) - dequantise_rows(q, s))
    bound = s.astype(np.float64)[:, None] * (0.5 + 128 * 2.0 ** -23)
    assert (err <= bound).all()
    # scale is the float32 quotient amax / 127
    amax = np.abs(x).max(axis=1)
    assert (s == (amax / np.float32(127)).astype(np.float32)).all()


@pytest.mark.parametrize("d,row_bytes", [(512, 516), (256, 260)])
def test_row_bytes(d, row_bytes):
    q, s = quantise_rows(np.ones((1, d), dtype=np.float32))
    assert q.nbytes + s.nbytes == row_bytes
