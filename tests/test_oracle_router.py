"""Pins of the oracle's router (O6 selection and weights, O7 expert top-p).

Source: colibrì README, "Implemented features" (DeepSeek-V3-like sigmoid
router, noaux_tc, routed_scaling_factor) and "Quick start" (adaptive expert
top-p knob).  Pins: sigmoid against a 60-digit evaluation; brute-force
selection on tiny routers, characterised by dominance over every subset
instead of the oracle's repeated argmax; group scores by enumerating pairs;
plain top-k against a stable argsort; a +1 bias forces a chosen set;
invariants of the weights; top-p special cases; hand-worked fixtures.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from exact import matches_f32, sigmoid_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _cfg(orc, E, k, G=1, TG=1, norm=1, rsf=2.5, top_p=0.0, renorm=1):
    return orc.make_cfg(E, k, G, TG, norm, rsf, top_p, renorm)


def test_sigmoid_exact(orc):
    rng = np.random.default_rng(60)
    lg = np.concatenate([rng.normal(0, 2, size=200), [0.0, 1e-8, -1e-8, 30.0, -30.0, 80.0, -80.0]])
    lg = lg.astype(F32).reshape(1, -1)
    E = lg.shape[1]
    _, _, sig = orc.route(_cfg(orc, E, 1), lg, want_sigma=True)
    assert sig[0, E - 7] == 0.5
    for e in range(E):
        assert matches_f32(sig[0, e], sigmoid_exact(lg[0, e])), (lg[0, e], sig[0, e])


def _dominates(a_val, a_idx, b_val, b_idx):
    """Total order of the selection: larger value first, lower index on ties."""
    return a_val > b_val or (a_val == b_val and a_idx < b_idx)


def _brute_select(c, E, k, G, TG):
    """The selection as the unique (group set, expert set) whose members each
    dominate every non-member, found by enumerating all subsets."""
    per = E // G
    gscore = []
    for g in range(G):
        mem = range(g * per, (g + 1) * per)
        if per >= 2:
            # the best pair sum: fp32 addition is monotone, so the max over
            # all pairs is the sum of the two largest
            gscore.append(max(F32(c[a]) + F32(c[b]) for a, b in itertools.combinations(mem, 2)))
        else:
            gscore.append(F32(c[g]))
    gsets = [S for S in itertools.combinations(range(G), TG)
             if all(_dominates(gscore[a], a, gscore[b], b) for a in S for b in range(G) if b not in S)]
    assert len(gsets) == 1
    allowed = [e for e in range(E) if e // per in gsets[0]]
    esets = [S for S in itertools.combinations(allowed, k)
             if all(_dominates(c[a], a, c[b], b) for a in S for b in allowed if b not in S)]
    assert len(esets) == 1
    return set(esets[0]), gsets[0]


@pytest.mark.parametrize("E,k,G,TG", [(8, 2, 1, 1), (8, 3, 2, 1), (12, 4, 4, 2), (16, 4, 4, 2),
                                      (16, 3, 8, 3), (16, 4, 2, 2), (16, 2, 16, 2)])
def test_router_brute_force(orc, E, k, G, TG):
    rng = np.random.default_rng(E * 100 + k * 10 + G)
    for trial in range(40):
        lg = rng.normal(0, 1.5, size=(1, E)).astype(F32)
        if trial % 5 == 0:  # inject ties
            lg[0, rng.integers(0, E)] = lg[0, rng.integers(0, E)]
        bias = (rng.normal(0, 0.05, size=E) if trial % 2 else np.zeros(E)).astype(F32)
        idx, w, sig = orc.route(_cfg(orc, E, k, G, TG), lg, bias, want_sigma=True)
        c = (sig[0] + bias).astype(F32)
        want, gsel = _brute_select(c, E, k, G, TG)
        assert set(idx[0].tolist()) == want, (trial, idx, want)
        # rank order: every slot dominates the next
        for j in range(k - 1):
            a, b = idx[0, j], idx[0, j + 1]
            assert _dominates(c[a], a, c[b], b)


def test_plain_topk_matches_stable_argsort(orc):
    rng = np.random.default_rng(61)
    E, k, T = 64, 6, 50
    lg = rng.normal(0, 1, size=(T, E)).astype(F32)
    idx, _ = orc.route(_cfg(orc, E, k), lg)
    order = np.argsort(-lg, axis=1, kind="stable")[:, :k]  # sigmoid is monotone
    np.testing.assert_array_equal(idx, order)


def test_bias_forces_chosen_set(orc):
    rng = np.random.default_rng(62)
    E, k, G, TG = 16, 4, 4, 2
    for _ in range(20):
        lg = rng.normal(0, 2, size=(1, E)).astype(F32)
        groups = rng.choice(G, size=TG, replace=False)
        pool = [e for e in range(E) if e // (E // G) in groups]
        chosen = rng.choice(pool, size=k, replace=False)
        bias = np.zeros(E, F32)
        bias[chosen] = 1.0
        idx, w = orc.route(_cfg(orc, E, k, G, TG), lg, bias)
        assert set(idx[0].tolist()) == set(chosen.tolist())
        # weights use the unbiased sigmoid
        sig = np.array([float(sigmoid_exact(lg[0, e])) for e in idx[0]])
        np.testing.assert_allclose(w[0] / w[0].sum(), sig / sig.sum(), rtol=1e-6)


@pytest.mark.parametrize("rsf", [2.5, 1.0])
def test_router_invariants(orc, rsf):
    rng = np.random.default_rng(63)
    E, k, G, TG, T = 256, 8, 8, 4, 64
    lg = rng.normal(0, 1.57, size=(T, E)).astype(F32)
    bias = rng.normal(0, 0.01, size=E).astype(F32)
    idx, w, sig = orc.route(_cfg(orc, E, k, G, TG, rsf=rsf), lg, bias, want_sigma=True)
    for t in range(T):
        assert len(set(idx[t].tolist())) == k
        assert len({e // (E // G) for e in idx[t]}) <= TG
        assert (w[t] > 0).all()
        assert abs(float(w[t].astype(np.float64).sum()) - rsf) <= 8 * rsf * 2 ** -23
        s = sig[t, idx[t]].astype(np.float64)
        np.testing.assert_allclose(w[t] / w[t].sum(), s / s.sum(), rtol=1e-6)
    # without bias the rank order follows sigma
    idx0, _, sig0 = orc.route(_cfg(orc, E, k, G, TG), lg, None, want_sigma=True)
    for t in range(T):
        s = sig0[t, idx0[t]]
        assert (np.diff(s) <= 0).all()


def test_no_normalisation(orc):
    rng = np.random.default_rng(64)
    E, k = 32, 4
    lg = rng.normal(0, 1, size=(5, E)).astype(F32)
    idx, w, sig = orc.route(_cfg(orc, E, k, norm=0, rsf=2.5), lg, want_sigma=True)
    for t in range(5):
        # sigma*2.5 is exact up to one rounding of the product
        np.testing.assert_allclose(w[t], sig[t, idx[t]] * 2.5, rtol=2 ** -23)


def test_top_p_off_values(orc):
    rng = np.random.default_rng(65)
    E, k, G, TG = 256, 8, 8, 4
    lg = rng.normal(0, 1.57, size=(16, E)).astype(F32)
    bias = rng.normal(0, 0.01, size=E).astype(F32)
    i0, w0 = orc.route(_cfg(orc, E, k, G, TG), lg, bias)
    for p in (0.0, 1.0, 1.5, -0.3):
        i1, w1 = orc.route(_cfg(orc, E, k, G, TG, top_p=p), lg, bias)
        np.testing.assert_array_equal(i0, i1)
        np.testing.assert_array_equal(w0, w1)


def test_top_p_tiny_keeps_one(orc):
    rng = np.random.default_rng(66)
    E, k, G, TG = 256, 8, 8, 4
    lg = rng.normal(0, 1.57, size=(16, E)).astype(F32)
    bias = rng.normal(0, 0.01, size=E).astype(F32)
    i0, w0, sig = orc.route(_cfg(orc, E, k, G, TG), lg, bias, want_sigma=True)
    i1, w1 = orc.route(_cfg(orc, E, k, G, TG, top_p=1e-7), lg, bias)
    for t in range(16):
        kept = np.nonzero(i1[t] >= 0)[0]
        assert len(kept) == 1
        j = kept[0]
        # the kept slot is the largest unbiased weight of the selection
        assert sig[t, i1[t, j]] == sig[t, i0[t]].max()
        assert i1[t, j] == i0[t, j]
        assert w1[t, j] == np.float32(2.5)  # sigma/sigma * rsf, exact
        assert (w1[t][i1[t] < 0] == 0).all()


@pytest.mark.parametrize("renorm", [1, 0])
def test_top_p_minimal_prefix(orc, renorm):
    rng = np.random.default_rng(67 + renorm)
    E, k, G, TG = 256, 8, 8, 4
    lg = rng.normal(0, 1.57, size=(64, E)).astype(F32)
    bias = rng.normal(0, 0.01, size=E).astype(F32)
    p = 0.7
    i0, w0, sig = orc.route(_cfg(orc, E, k, G, TG), lg, bias, want_sigma=True)
    i1, w1 = orc.route(_cfg(orc, E, k, G, TG, top_p=p, renorm=renorm), lg, bias)
    for t in range(64):
        s = sig[t, i0[t]].astype(np.float64)
        pn = s / s.sum()
        kept = i1[t] >= 0
        np.testing.assert_array_equal(i1[t][kept], i0[t][kept])  # slots keep their rank position
        # kept = the largest normalised weights, a minimal prefix reaching p
        order = sorted(range(k), key=lambda j: (-pn[j], j))
        n_keep = int(kept.sum())
        assert set(np.nonzero(kept)[0].tolist()) == set(order[:n_keep])
        assert pn[order[:n_keep]].sum() >= p - 1e-6
        if n_keep > 1:
            assert pn[order[:n_keep - 1]].sum() < p + 1e-6
        if renorm:
            assert abs(float(w1[t].astype(np.float64).sum()) - 2.5) < 1e-5
        else:
            np.testing.assert_array_equal(w1[t][kept], w0[t][kept])
        assert (w1[t][~kept] == 0).all()


def _golden_router_cases():
    out = []
    with open(os.path.join(GOLDEN, "router_examples.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            cfg, lg, bias, idx, w = [p.strip() for p in line.split("|")]
            out.append((dict(kv.split("=") for kv in cfg.split()), lg, bias, idx, w))
    return out


def test_golden_router(orc):
    cases = _golden_router_cases()
    assert cases
    for cfg, lg, bias, idx, w in cases:
        E, k = int(cfg["E"]), int(cfg["k"])
        c = _cfg(orc, E, k, int(cfg.get("G", 1)), int(cfg.get("TG", 1)),
                 rsf=float(cfg.get("rsf", 2.5)), top_p=float(cfg.get("top_p", 0)))
        lgv = np.array([[eval(v, {"ln": math.log}) for v in lg.split()]], F32)
        b = None if bias == "-" else np.array([float(v) for v in bias.split()], F32)
        got_i, got_w = orc.route(c, lgv, b)
        np.testing.assert_array_equal(got_i[0], [int(v) for v in idx.split()])
        np.testing.assert_array_equal(got_w[0], np.array([float(v) for v in w.split()], F32))
    assert Fraction(1, 2) == Fraction(float(np.float32(0.5)))
