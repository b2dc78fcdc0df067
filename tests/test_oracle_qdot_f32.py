"""Pins of the oracle's f32-activation product O12 (the variant of the
quantised product whose activations stay binary32): exact integer closed
forms, bit-equality with O4 where Q8_0 represents the activations exactly,
exact rational arithmetic on a small case, and the packed-int4 == int8
container identity."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

from exact import matches_f32

F32 = np.float32


def _codes(rng, bits, R, C):
    q = {8: 127, 4: 7, 2: 1}[bits]
    return rng.integers(-q, q + 1, size=(R, C)).astype(np.int8)


def _pack(orc, bits, codes):
    """Pack codes by the oracle's own O1/O2 path: a row of codes times 2^-6,
    with one +-qmax entry, quantises back to exactly those codes at scale
    2^-6 (the grid closed form the packing pins establish)."""
    q = {8: 127, 4: 7, 2: 1}[bits]
    w = codes.astype(np.float32) * F32(2.0 ** -6)
    w[:, 0] = q * 2.0 ** -6
    packed, scale = orc.quant_pack(bits, w)
    np.testing.assert_array_equal(scale, np.full(len(w), F32(2.0 ** -6)))
    c = codes.copy()
    c[:, 0] = q
    return packed, scale, c


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_integer_closed_form(orc, bits):
    """Integer activations and scale 2^-6: y = 2^-6 * (codes @ x) exactly."""
    rng = np.random.default_rng(bits)
    packed, scale, codes = _pack(orc, bits, _codes(rng, bits, 40, 256))
    x = rng.integers(-50, 51, size=(3, 256)).astype(np.float32)
    y = orc.qdot_f32act(bits, packed, scale, 256, x)
    ref = (x.astype(np.int64) @ codes.astype(np.int64).T).astype(np.float64) * 2.0 ** -6
    np.testing.assert_array_equal(y, ref.astype(np.float32))


@pytest.mark.parametrize("bits", [4, 2])
def test_equals_q8_0_product_on_representable_activations(orc, bits):
    """x = q * 2^-5 with integer |q| <= 127 is its own Q8_0 encoding when every
    block holds a +-127 (d = 2^-5 exactly); then O12 and O4 compute the same
    exact real and round it once: bit-identical."""
    rng = np.random.default_rng(10 + bits)
    R, C = 24, 192
    codes = _codes(rng, bits, R, C)
    w = codes.astype(np.float32) * F32(0.013)
    packed, scale = orc.quant_pack(bits, w)
    xq = rng.integers(-127, 128, size=(2, C)).astype(np.int8)
    xq[:, ::32] = 127
    x = xq.astype(np.float32) * F32(2.0 ** -5)
    q8, d = orc.q8_0(x)
    np.testing.assert_array_equal(q8, xq)
    np.testing.assert_array_equal(d, np.full_like(d, F32(2.0 ** -5)))
    _, y4 = orc.qdot(bits, packed, scale, C, q8, d, want_acc=False)
    y12 = orc.qdot_f32act(bits, packed, scale, C, x)
    np.testing.assert_array_equal(y12.view(np.uint32), y4.view(np.uint32))


def test_exact_rational(orc):
    rng = np.random.default_rng(3)
    R, C, T = 5, 64, 2
    w = rng.normal(0, 0.02, size=(R, C)).astype(np.float32)
    packed, scale = orc.quant_pack(4, w)
    codes = orc.unpack(4, packed, C)
    x = rng.normal(0, 1, size=(T, C)).astype(np.float32)
    y = orc.qdot_f32act(4, packed, scale, C, x)
    for t in range(T):
        for r in range(R):
            q = Fraction(float(scale[r])) * sum(Fraction(int(codes[r, c])) * Fraction(float(x[t, c]))
                                                for c in range(C))
            assert matches_f32(y[t, r], q), (t, r)


def test_int4_container_identity(orc):
    """The same int4-level codes packed as int4 and held in the int8 container
    give bit-identical products."""
    rng = np.random.default_rng(4)
    codes = _codes(rng, 4, 16, 128)
    p4, s4, c = _pack(orc, 4, codes)
    p8 = c.view(np.uint8).copy()  # the int8 container: one code per byte
    x = rng.normal(0, 1, size=(2, 128)).astype(np.float32)
    y4 = orc.qdot_f32act(4, p4, s4, 128, x)
    y8 = orc.qdot_f32act(8, p8, s4, 128, x)
    np.testing.assert_array_equal(y4, y8)


def test_rejects_bad_arguments(orc):
    with pytest.raises(Exception):
        orc.qdot_f32act(3, np.zeros((1, 16), np.uint8), np.ones(1, np.float32), 32,
                        np.zeros((1, 32), np.float32))
