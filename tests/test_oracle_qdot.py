"""Pins of the oracle's Q8_0 activation quantisation (O3), quantised product
(O4) and router logits (O5).

Pins: Q8_0 grid closed form and hand-worked rounding; block independence;
the int32 block accumulators against numpy's integer einsum over codes decoded
by shifts (not the oracle's decoder); the fp32 outputs against exact rational
arithmetic rounded once; outputs exactly representable when every scale is a
power of two; the int4 packed and int8 containers give identical accumulators
and outputs (colibrì README, "Implemented features": packing bit-identical to
the int8 container); logits against exact rational dot products.
"""
from fractions import Fraction

import numpy as np
import pytest

from exact import f32_nearest, matches_f32


def _decode_shift(packed: np.ndarray, bits: int, cols: int) -> np.ndarray:
    """Decode packed fields with numpy shifts (independent of the oracle)."""
    per = 8 // bits
    R = packed.shape[0]
    out = np.empty((R, cols), np.int8)
    for m in range(per):
        top = (packed << np.uint8(8 - bits * (m + 1))).view(np.int8)
        out[:, m::per] = top >> np.int8(8 - bits)
    return out


def test_q8_0_grid_closed_form(orc):
    rng = np.random.default_rng(10)
    T, n = 6, 256
    q = rng.integers(-127, 128, size=(T, n)).astype(np.int8)
    nb = n // 32
    for t in range(T):
        for b in range(nb):
            q[t, b * 32 + rng.integers(0, 32)] = rng.choice([-127, 127])
    e = rng.integers(-30, 30, size=(T, nb))
    d = np.ldexp(np.ones((T, nb), np.float32), -e).astype(np.float32)
    x = (q.astype(np.float32).reshape(T, nb, 32) * d[..., None]).reshape(T, n).astype(np.float32)
    q2, d2 = orc.q8_0(x)
    np.testing.assert_array_equal(d2, d)
    np.testing.assert_array_equal(q2, q)


def test_q8_0_rounding_and_zero_block(orc):
    x = np.zeros((1, 64), np.float32)
    x[0, :7] = [127, 2.5, 3.5, -2.5, -3.5, 126.5, -0.5]  # d = 1
    q, d = orc.q8_0(x)
    assert d[0, 0] == 1.0 and d[0, 1] == 0.0
    np.testing.assert_array_equal(q[0, :7], [127, 2, 4, -2, -4, 126, 0])
    assert (q[0, 32:] == 0).all()


def test_q8_0_blocks_independent_and_bound(orc):
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, size=(3, 192)).astype(np.float32)
    q, d = orc.q8_0(x)
    x2 = x.copy()
    x2[:, 32:64] *= 1000.0
    q2, d2 = orc.q8_0(x2)
    keep = np.r_[0:32, 64:192]
    np.testing.assert_array_equal(q[:, keep], q2[:, keep])
    err = np.abs(x.reshape(3, 6, 32).astype(np.float64) - q.reshape(3, 6, 32) * d[..., None].astype(np.float64))
    assert (err <= d[..., None] * (0.5 + 1e-6)).all()
    amax_pos = np.abs(x.reshape(3, 6, 32)).argmax(-1)
    assert (np.abs(np.take_along_axis(q.reshape(3, 6, 32), amax_pos[..., None], -1)) == 127).all()


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_qdot_acc_matches_integer_einsum(orc, bits):
    rng = np.random.default_rng(12 + bits)
    R, C, T = 24, 192, 3
    w = rng.normal(0, 0.02, size=(R, C)).astype(np.float32)
    packed, s = orc.quant_pack(bits, w)
    x = rng.normal(0, 1, size=(T, C)).astype(np.float32)
    xq, xd = orc.q8_0(x)
    acc, y = orc.qdot(bits, packed, s, C, xq, xd)
    wc = _decode_shift(packed, bits, C).astype(np.int64).reshape(R, C // 32, 32)
    want = np.einsum("rbi,tbi->trb", wc, xq.astype(np.int64).reshape(T, C // 32, 32))
    np.testing.assert_array_equal(acc, want)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_qdot_y_exact_rational(orc, bits):
    rng = np.random.default_rng(20 + bits)
    R, C, T = 6, 96, 2
    w = rng.normal(0, 0.02, size=(R, C)).astype(np.float32)
    packed, s = orc.quant_pack(bits, w)
    x = rng.normal(0, 1, size=(T, C)).astype(np.float32)
    xq, xd = orc.q8_0(x)
    acc, y = orc.qdot(bits, packed, s, C, xq, xd)
    for t in range(T):
        for r in range(R):
            exact = sum(Fraction(float(s[r])) * Fraction(float(xd[t, b])) * int(acc[t, r, b])
                        for b in range(C // 32))
            assert matches_f32(y[t, r], exact), (t, r, y[t, r], float(exact))


def test_qdot_power_of_two_scales_exact(orc):
    """With power-of-two row and block scales (one block scale per token)
    and |sum acc| < 2^24, y is exactly s*d*sum(acc) -- a value every
    summation order reproduces."""
    rng = np.random.default_rng(30)
    R, C, T = 16, 6144, 2
    codes = rng.integers(-7, 8, size=(R, C)).astype(np.int8)
    codes[:, 0] = 7
    sc = np.ldexp(np.ones(R, np.float32), -rng.integers(3, 9, size=R)).astype(np.float32)
    w = (codes.astype(np.float32) * sc[:, None]).astype(np.float32)
    packed, s = orc.quant_pack(4, w)
    np.testing.assert_array_equal(s, sc)
    xq = rng.integers(-127, 128, size=(T, C)).astype(np.int8)
    dt = np.ldexp(np.ones(T, np.float32), -rng.integers(1, 6, size=T)).astype(np.float32)
    xd = np.repeat(dt[:, None], C // 32, axis=1).astype(np.float32)
    _, y = orc.qdot(4, packed, s, C, xq, xd, want_acc=False)
    tot = codes.astype(np.int64) @ xq.astype(np.int64).T  # [R, T]
    assert np.abs(tot).max() < 2 ** 24
    want = (sc[:, None].astype(np.float64) * dt[None, :] * tot).T
    np.testing.assert_array_equal(y.astype(np.float64), want)


@pytest.mark.parametrize("bits", [4, 2])
def test_container_identity_through_qdot(orc, bits):
    """int4 (int2) codes stored in the int8 container give the same int32
    accumulators and the same fp32 outputs as the packed container."""
    rng = np.random.default_rng(40 + bits)
    R, C, T = 32, 512, 4
    w = rng.normal(0, 0.02, size=(R, C)).astype(np.float32)
    codes, s = orc.quant_rows(bits, w)
    packed = orc.pack(bits, codes)
    cont8 = orc.pack(8, codes)
    x = rng.normal(0, 1, size=(T, C)).astype(np.float32)
    xq, xd = orc.q8_0(x)
    a1, y1 = orc.qdot(bits, packed, s, C, xq, xd)
    a2, y2 = orc.qdot(8, cont8, s, C, xq, xd)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(y1, y2)


def test_logits_exact_rational(orc):
    rng = np.random.default_rng(50)
    T, E, H = 2, 5, 64
    x = rng.normal(0, 1, size=(T, H)).astype(np.float32)
    g = rng.normal(0, 0.02, size=(E, H)).astype(np.float32)
    lg = orc.logits(x, g)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], g[e]))
            assert matches_f32(lg[t, e], exact)


def test_logits_one_hot(orc):
    E, H = 7, 32
    rng = np.random.default_rng(51)
    g = rng.normal(0, 0.02, size=(E, H)).astype(np.float32)
    x = np.zeros((H, H), np.float32)
    np.fill_diagonal(x, 1.0)
    np.testing.assert_array_equal(orc.logits(x, g), g.T)
    assert f32_nearest(Fraction(1, 3)) == np.float32(1 / 3)
