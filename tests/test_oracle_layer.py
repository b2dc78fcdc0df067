"""Pins of the oracle's expert FFN (O8), layer (O9) and union tables (O10).

Source: colibrì README, "Implemented features" (DeepSeek-V3-like MoE with a
shared expert and a sigmoid router; int kernels against Q8_0-style int8
activations; batch-union MoE reading each unique expert of a batch once).
Pins: a SwiGLU expert built from scaled identities, whose output is
silu(a x) * b x up to one Q8_0 rounding of h (catches a swapped gate/up, a
missing activation or a wrong down operand); h against a 60-digit silu;
closed forms (x = 0, rsf = 0, identical experts); token-permutation and
in-group expert-relabelling equivariance, bit-exact; the combine against an
exact rational sum of the per-expert outputs; the union tables against a
Python sort of (expert, token, slot).
"""
from fractions import Fraction

import numpy as np
import pytest

from exact import matches_f32, silu_exact
from quantized_moe_coli_amd import inputs

F32 = np.float32


def _layer(orc, shape, seed=0, bits=None, experts=None):
    bits = shape.bits if bits is None else bits
    exs = []
    E = shape.n_experts
    for e in range(E + 1):
        g, u, d = (t.numpy() for t in inputs.expert_weights(shape, seed, e))
        exs.append(orc.Expert.from_float(bits, g, u, d))
    cfg = orc.make_cfg(E, shape.top_k, shape.n_group, shape.topk_group, 1, shape.rsf,
                       shape.top_p, 1)
    return orc.Layer(shape.hidden, shape.inter, bits, cfg,
                     exs[:E] if experts is None else experts, exs[E],
                     inputs.gate_weight(shape, seed).numpy(),
                     inputs.gate_bias(shape, seed).numpy())


SMALL = inputs.Shape(hidden=128, inter=64, n_experts=16, top_k=4, n_group=4,
                     topk_group=2, rsf=2.5, bias_std=0.01, bits=4)


def test_swiglu_identity_construction(orc):
    """gate = a*I, up = b*I, down = c*I (H = I = 64), x on the Q8_0 grid:
    g = a x and u = b x exactly, h = fl32(silu(a x) * b x), and
    o = c * dequant(Q8_0(h)), within c*d_h/2 of c*h."""
    H = I = 64
    a, b, c = F32(0.5), F32(0.25), F32(2.0)
    eye = np.eye(H, dtype=F32)
    ex = orc.Expert.from_float(8, a * eye, b * eye, c * eye)
    np.testing.assert_array_equal(ex.s_gate, np.full(I, a / F32(127), F32))
    rng = np.random.default_rng(70)
    q = rng.integers(-127, 128, size=(3, H)).astype(F32)
    q[:, 0] = 127
    q[:, 32] = -127
    x = (q * F32(2.0 ** -5)).astype(F32)  # d = 2^-5 exactly
    o, h = orc.expert_ffn(8, H, I, ex, x, want_h=True)
    for t in range(3):
        for i in range(I):
            g = Fraction(float(x[t, i])) * Fraction(float(a))
            u = Fraction(float(x[t, i])) * Fraction(float(b))
            want = silu_exact(float(g)) * u
            assert matches_f32(h[t, i], want), (t, i)
    hq, hd = orc.q8_0(h)
    dh = np.repeat(hd, 32, axis=1)
    np.testing.assert_allclose(o, c * h, rtol=0, atol=float(c) * dh.max() * 0.5 * 1.0001)
    # swapping gate and up must change the result
    ex_sw = orc.Expert.from_float(8, b * eye, a * eye, c * eye)
    assert not np.allclose(orc.expert_ffn(8, H, I, ex_sw, x), o)


def test_h_matches_exact_silu(orc):
    H, I = 128, 64
    rng = np.random.default_rng(71)
    ex = orc.Expert.from_float(4, rng.normal(0, .02, (I, H)).astype(F32),
                               rng.normal(0, .02, (I, H)).astype(F32),
                               rng.normal(0, .02, (H, I)).astype(F32))
    x = rng.normal(0, 1, (2, H)).astype(F32)
    o, h = orc.expert_ffn(4, H, I, ex, x, want_h=True)
    xq, xd = orc.q8_0(x)
    _, g = orc.qdot(4, ex.w_gate, ex.s_gate, H, xq, xd, want_acc=False)
    _, u = orc.qdot(4, ex.w_up, ex.s_up, H, xq, xd, want_acc=False)
    for t in range(2):
        for i in range(I):
            assert matches_f32(h[t, i], silu_exact(g[t, i]) * Fraction(float(u[t, i])))
    hq, hd = orc.q8_0(h)
    _, o2 = orc.qdot(4, ex.w_down, ex.s_down, I, hq, hd, want_acc=False)
    np.testing.assert_array_equal(o, o2)


def test_zero_input_gives_zero(orc):
    L = _layer(orc, SMALL)
    y, idx, w, _ = orc.moe_forward(L, np.zeros((3, SMALL.hidden), F32))
    assert (y == 0).all()


def test_rsf_zero_gives_shared(orc):
    L = _layer(orc, SMALL.with_(rsf=0.0))
    x = inputs.tokens(SMALL, 0, 0, 4).numpy()
    y, _, w, _ = orc.moe_forward(L, x)
    assert (w == 0).all()
    np.testing.assert_array_equal(y, orc.expert_ffn(4, SMALL.hidden, SMALL.inter, L.shared, x))


def test_identical_experts(orc):
    base = _layer(orc, SMALL)
    same = [base.experts[3]] * SMALL.n_experts
    L = _layer(orc, SMALL, experts=same)
    x = inputs.tokens(SMALL, 0, 1, 5).numpy()
    y, _, w, _ = orc.moe_forward(L, x)
    o_sh = orc.expert_ffn(4, SMALL.hidden, SMALL.inter, L.shared, x)
    o_e = orc.expert_ffn(4, SMALL.hidden, SMALL.inter, same[0], x)
    np.testing.assert_allclose(y, o_sh + SMALL.rsf * o_e, rtol=1e-5, atol=1e-6)


def test_combine_exact_rational(orc):
    L = _layer(orc, SMALL)
    x = inputs.tokens(SMALL, 0, 2, 3).numpy()
    y, idx, w, _ = orc.moe_forward(L, x)
    H = SMALL.hidden
    for t in range(3):
        o_sh = orc.expert_ffn(4, H, SMALL.inter, L.shared, x[t:t + 1])[0]
        outs = [orc.expert_ffn(4, H, SMALL.inter, L.experts[e], x[t:t + 1])[0] for e in idx[t]]
        for r in range(0, H, 7):
            exact = Fraction(float(o_sh[r])) + sum(
                Fraction(float(w[t, j])) * Fraction(float(outs[j][r])) for j in range(SMALL.top_k))
            assert matches_f32(y[t, r], exact)


def test_token_permutation_equivariance(orc):
    L = _layer(orc, SMALL)
    x = inputs.tokens(SMALL, 0, 3, 6).numpy()
    y, idx, w, lg = orc.moe_forward(L, x)
    perm = np.array([3, 0, 5, 1, 4, 2])
    y2, idx2, w2, lg2 = orc.moe_forward(L, x[perm])
    np.testing.assert_array_equal(y2, y[perm])
    np.testing.assert_array_equal(idx2, idx[perm])
    np.testing.assert_array_equal(w2, w[perm])


def test_expert_relabelling_within_groups(orc):
    L = _layer(orc, SMALL)
    E, per = SMALL.n_experts, SMALL.n_experts // SMALL.n_group
    rng = np.random.default_rng(72)
    sigma = np.concatenate([g * per + rng.permutation(per) for g in range(SMALL.n_group)])
    # new expert i is old expert sigma[i]
    L2 = orc.Layer(L.hidden, L.inter, L.bits, L.cfg, [L.experts[s] for s in sigma], L.shared,
                   L.gate_w[sigma], L.gate_bias[sigma])
    x = inputs.tokens(SMALL, 0, 4, 5).numpy()
    y, idx, w, _ = orc.moe_forward(L, x)
    y2, idx2, w2, _ = orc.moe_forward(L2, x)
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(sigma[idx2], idx)
    np.testing.assert_array_equal(w2, w)


def test_logits_in_matches_gate(orc):
    L = _layer(orc, SMALL)
    x = inputs.tokens(SMALL, 0, 5, 4).numpy()
    y, idx, w, lg = orc.moe_forward(L, x)
    y2, idx2, w2, lg2 = orc.moe_forward(L, x, logits_in=lg)
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(idx2, idx)
    np.testing.assert_array_equal(lg2, orc.logits(x, L.gate_w))


def test_missing_selected_expert_is_rejected(orc):
    L = _layer(orc, SMALL)
    x = inputs.tokens(SMALL, 0, 6, 2).numpy()
    _, idx, _, _ = orc.moe_forward(L, x)
    holes = list(L.experts)
    holes[int(idx[0, 0])] = None
    with pytest.raises(ValueError):
        orc.moe_forward(orc.Layer(L.hidden, L.inter, L.bits, L.cfg, holes, L.shared,
                                  L.gate_w, L.gate_bias), x)
    # experts nobody selects may be absent
    used = set(idx.ravel().tolist())
    sparse = [ex if e in used else None for e, ex in enumerate(L.experts)]
    y2, _, _, _ = orc.moe_forward(orc.Layer(L.hidden, L.inter, L.bits, L.cfg, sparse, L.shared,
                                            L.gate_w, L.gate_bias), x)
    np.testing.assert_array_equal(y2, orc.moe_forward(L, x)[0])


def test_top_p_layer_drops_experts(orc):
    s = SMALL.with_(top_p=0.5)
    L = _layer(orc, s)
    x = inputs.tokens(s, 0, 7, 8).numpy()
    y, idx, w, _ = orc.moe_forward(L, x)
    assert (idx == -1).any()
    # the output equals the layer restricted to the kept experts
    H = s.hidden
    for t in range(8):
        acc = orc.expert_ffn(4, H, s.inter, L.shared, x[t:t + 1])[0].astype(np.float64)
        for j in range(s.top_k):
            if idx[t, j] >= 0:
                acc += float(w[t, j]) * orc.expert_ffn(4, H, s.inter, L.experts[idx[t, j]],
                                                       x[t:t + 1])[0]
        np.testing.assert_allclose(y[t], acc, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("T,k,E,drop", [(1, 8, 256, 0.0), (3, 8, 256, 0.0), (64, 4, 16, 0.0),
                                        (50, 8, 64, 0.3), (0, 2, 4, 0.0)])
def test_union_tables_against_sort(orc, T, k, E, drop):
    rng = np.random.default_rng(T * 7 + k)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]) if T else \
        np.zeros((0, k), np.int64)
    idx = idx.astype(np.int32)
    if drop:
        idx[rng.random(idx.shape) < drop] = -1
    counts, offs, perm, uniq = orc.union_tables(idx, E)
    pairs = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k) if idx[t, j] >= 0)
    np.testing.assert_array_equal(perm, [t * k + j for _, t, j in pairs])
    np.testing.assert_array_equal(counts, np.bincount(idx[idx >= 0].ravel(), minlength=E))
    np.testing.assert_array_equal(offs, np.r_[0, np.cumsum(counts)])
    np.testing.assert_array_equal(uniq, np.unique(idx[idx >= 0]))
