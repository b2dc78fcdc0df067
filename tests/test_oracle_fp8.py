"""Pins of the oracle's FP8 checkpoint dequantisation (O11): the E4M3 decode
against torch's own float8_e4m3fn conversion (an independent implementation
of the format) and the format's closed forms, the 128x128 block scaling
against numpy on ragged shapes with a non-square block grid, and the
requantisation against a hand-worked case."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def torch_e4m3(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(
        torch.float8_e4m3fn).float().numpy()


def test_every_code_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    mine = np.array([orc.e4m3_value(int(c)) for c in codes], np.float32)
    ref = torch_e4m3(codes)
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok].view(np.uint32), ref[ok].view(np.uint32))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x30, 0.5), (0x3C, 1.5), (0x7E, 448.0),
    (0xFE, -448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x0F, 1.875 * 2.0 ** -6), (0xB8, -1.0),
])
def test_closed_forms(orc, code, value):
    assert orc.e4m3_value(code) == value


def test_format_invariants(orc):
    v = np.array([orc.e4m3_value(c) for c in range(256)])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()                      # magnitude grows with the code
    np.testing.assert_array_equal(v[0x80:0xFF], -pos)    # sign bit
    assert np.signbit(v[0x80]) and v[0x80] == 0.0        # negative zero


def test_block_scaling_ragged_shape(orc):
    rng = np.random.default_rng(11)
    rows, cols = 200, 300                      # a 2 x 3 grid of 128x128 blocks
    w8 = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    w8[(w8 & 0x7F) == 0x7F] = 0x38             # no NaN codes
    bs = np.array([[0.5, 2.0, 0.25], [4.0, 0.125, 8.0]], np.float32)
    out = orc.dequant_fp8_block(w8, bs)
    per = np.repeat(np.repeat(bs, 128, axis=0), 128, axis=1)[:rows, :cols].astype(np.float64)
    ref = (torch_e4m3(w8).astype(np.float64) * per).astype(np.float32)  # powers of two: exact
    np.testing.assert_array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_block_scale_product_rounds_once(orc):
    rng = np.random.default_rng(12)
    w8 = rng.integers(0, 0x7F, size=(130, 160), dtype=np.uint8)
    bs = rng.uniform(0.001, 0.01, size=(2, 2)).astype(np.float32)
    out = orc.dequant_fp8_block(w8, bs)
    per = np.repeat(np.repeat(bs, 128, axis=0), 128, axis=1)[:130, :160].astype(np.float64)
    ref = (torch_e4m3(w8).astype(np.float64) * per).astype(np.float32)
    np.testing.assert_array_equal(out, ref)


def test_requant_hand_worked(orc):
    """One block of 1.0 codes at scale 0.5, into int4: every value is 0.5, so
    the row scale is fl32(0.5 / 7) and every code is +7 (nibbles 0x7)."""
    w8 = np.full((3, 64), 0x38, np.uint8)
    packed, scales = orc.requant_fp8_block(4, w8, np.array([[0.5]], np.float32))
    np.testing.assert_array_equal(scales, np.full(3, np.float32(0.5) / np.float32(7), np.float32))
    np.testing.assert_array_equal(packed, np.full((3, 32), 0x77, np.uint8))


def test_rejects_mismatched_block_grid(orc):
    with pytest.raises(ValueError):
        orc.dequant_fp8_block(np.zeros((129, 32), np.uint8), np.ones((1, 1), np.float32))
