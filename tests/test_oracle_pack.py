"""Pins of the oracle's containers (O1 quantisation, O2 packing).

Pins: exhaustive unpack of every byte against sign extension done by
arithmetic shifts; every code in every field position against the place-value
definition; pack(unpack(b)) == b; the packed int4 container decodes to the
same bytes as the int8 container holding the same codes (colibrì README,
"Implemented features": packing checked bit-identical to the int8 container);
grid closed forms for the per-row scale; round-half-even cases; the absmax
error bound; hand-worked fixtures in tests/golden/.
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _signext_shift(field: np.ndarray, bits: int) -> np.ndarray:
    """Sign-extend b-bit fields by moving them to the top of an int8 and
    shifting back arithmetically (a mechanism unlike the oracle's)."""
    top = (field.astype(np.uint8) << np.uint8(8 - bits)).view(np.int8)
    return (top >> np.int8(8 - bits)).astype(np.int8)


@pytest.mark.parametrize("bits", [4, 2])
def test_unpack_every_byte(orc, bits):
    per = 8 // bits
    allb = np.arange(256, dtype=np.uint8).reshape(256, 1)
    codes = orc.unpack(bits, allb, per)
    mask = (1 << bits) - 1
    for m in range(per):
        field = (allb[:, 0] >> np.uint8(bits * m)) & np.uint8(mask)
        np.testing.assert_array_equal(codes[:, m], _signext_shift(field, bits))
    # round trip on every byte
    np.testing.assert_array_equal(orc.pack(bits, codes), allb)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_every_code_every_position(orc, bits):
    per = 8 // bits
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    cols = 32 if bits != 8 else 4
    for m in range(min(per * 2, cols)):
        for v in range(lo, hi + 1):
            row = np.zeros((1, cols), np.int8)
            row[0, m] = v
            packed = orc.pack(bits, row)
            want = np.zeros(cols * bits // 8, np.uint8)
            # place value: field (v mod 2^b) at bit offset b*(m mod per) of byte m//per
            want[m // per] = ((v % (1 << bits)) << (bits * (m % per))) & 0xFF
            np.testing.assert_array_equal(packed[0], want, err_msg=f"bits={bits} m={m} v={v}")
            np.testing.assert_array_equal(orc.unpack(bits, packed, cols), row)


def test_int8_pack_is_the_code_bytes(orc):
    rng = np.random.default_rng(1)
    codes = rng.integers(-128, 128, size=(5, 64), dtype=np.int8)
    np.testing.assert_array_equal(orc.pack(8, codes), codes.view(np.uint8))


@pytest.mark.parametrize("bits", [4, 2])
def test_packed_equals_int8_container(orc, bits):
    """Packing is bit-identical to the int8 container: codes of the b-bit
    grid stored one per byte, and the packed bytes, decode to the same
    codes; quantising through either gives the same scales."""
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.02, size=(64, 256)).astype(np.float32)
    codes, s = orc.quant_rows(bits, w)
    packed, s2 = orc.quant_pack(bits, w)
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(orc.unpack(bits, packed, 256), codes)
    container8 = orc.pack(8, codes)  # the same codes in the int8 container
    np.testing.assert_array_equal(orc.unpack(8, container8, 256), orc.unpack(bits, packed, 256))
    assert packed.nbytes * (8 // bits) == container8.nbytes


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_quant_grid_closed_form(orc, bits):
    """w = q * 2^-e with one element per row at +-qmax*2^-e: quantisation
    returns s = 2^-e and q unchanged (every division is exact)."""
    qm = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(3)
    R, C = 40, 96
    q = rng.integers(-qm, qm + 1, size=(R, C)).astype(np.int8)
    pos = rng.integers(0, C, size=R)
    sign = rng.choice([-1, 1], size=R)
    q[np.arange(R), pos] = sign * qm
    e = rng.integers(-20, 20, size=R)
    scale = np.ldexp(np.ones(R, np.float32), -e).astype(np.float32)
    w = (q.astype(np.float32) * scale[:, None]).astype(np.float32)
    codes, s = orc.quant_rows(bits, w)
    np.testing.assert_array_equal(s, scale)
    np.testing.assert_array_equal(codes, q)


def test_quant_zero_row(orc):
    for bits in (8, 4, 2):
        codes, s = orc.quant_rows(bits, np.zeros((2, 32), np.float32))
        assert (s == 0).all() and (codes == 0).all()


def test_quant_round_half_even(orc):
    # int8: amax 127 -> s = 1 exactly, so codes are round_half_even(w)
    w = np.zeros((1, 32), np.float32)
    w[0, :8] = [127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]
    codes, s = orc.quant_rows(8, w)
    assert s[0] == 1.0
    np.testing.assert_array_equal(codes[0, :8], [127, 2, 4, -2, -4, 0, 2, 0])
    # int4: amax 7 -> s = 1
    w4 = np.zeros((1, 32), np.float32)
    w4[0, :6] = [7, 2.5, -3.5, 6.5, -6.5, 0.5]
    codes4, s4 = orc.quant_rows(4, w4)
    assert s4[0] == 1.0
    np.testing.assert_array_equal(codes4[0, :6], [7, 2, -4, 6, -6, 0])
    # int2 ternary: amax 1 -> s = 1; 0.5 ties to 0, 0.75 -> 1
    w2 = np.zeros((1, 32), np.float32)
    w2[0, :4] = [1, 0.5, -0.75, -0.5]
    codes2, _ = orc.quant_rows(2, w2)
    np.testing.assert_array_equal(codes2[0, :4], [1, 0, -1, 0])


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_quant_error_bound(orc, bits):
    """Absmax quantisation: |w - s*q| <= s/2 (plus a few ulps) and the row's
    largest |w| maps to +-qmax."""
    qm = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(4)
    w = rng.normal(0, 0.02, size=(50, 256)).astype(np.float32)
    codes, s = orc.quant_rows(bits, w)
    err = np.abs(w.astype(np.float64) - s[:, None].astype(np.float64) * codes)
    assert (err <= s[:, None] * (0.5 + 1e-6)).all()
    am = np.abs(w).argmax(1)
    np.testing.assert_array_equal(np.abs(codes[np.arange(50), am]), qm)
    assert np.abs(codes).max() <= qm


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split("|"))
    return rows


def test_golden_pack(orc):
    for bits, codes, packed in _read_golden("pack_examples.txt"):
        bits = int(bits)
        c = np.array([int(v) for v in codes.split()], np.int8).reshape(1, -1)
        want = np.array([int(v, 16) for v in packed.split()], np.uint8)
        np.testing.assert_array_equal(orc.pack(bits, c)[0], want)
        np.testing.assert_array_equal(orc.unpack(bits, want.reshape(1, -1), c.shape[1]), c)
