"""Accuracy of the Q8_0 activation path (O4) against the f32-activation
product (O12) at GLM-5.2 shape: the error that quantising the activations
to Q8_0 adds, for each weight container, on a gate-shaped matrix (2048 x
6144, fed a token's hidden state) and a down-shaped one (6144 x 2048, fed
the expert's SwiGLU output h).  Both sides are the oracle's; the table this
prints is the measurement behind the per-(container, batch) choice of the
product (colibrì README, "Implemented features", integer dot-product item:
the choice by shape, with f32 activations kept for a single int4 row).

Properties checked: the Q8_0 error is small (RMS relative error below 1.5%)
and is the larger of the two against the exact product of the same codes
in binary64, so the table measures the activation quantisation, not the
f32 path's rounding."""
from __future__ import annotations

import numpy as np
import pytest

from quantized_moe_coli_amd import inputs

S = inputs.GLM
T = 4


def _rel(a, ref):
    a = a.astype(np.float64)
    ref = ref.astype(np.float64)
    rms = float(np.sqrt(((a - ref) ** 2).sum() / (ref ** 2).sum()))
    mx = float((np.abs(a - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())
    return rms, mx


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_q8_0_error_against_f32_activations(orc, bits):
    H, I = S.hidden, S.inter
    w_gate = inputs.normal((I, H), S.w_std, "cpu", 900, 0, bits).numpy()
    w_down = inputs.normal((H, I), S.w_std, "cpu", 900, 1, bits).numpy()
    x = inputs.tokens(S, 900, 0, T).numpy()
    gq, gs = orc.quant_pack(bits, w_gate)
    dq, ds = orc.quant_pack(bits, w_down)
    # a realistic input for the down projection: SwiGLU of two gate-shaped
    # products of x (fp32, as the layer forms h before its Q8_0 step)
    w_up = inputs.normal((I, H), S.w_std, "cpu", 900, 2, bits).numpy()
    uq, us = orc.quant_pack(bits, w_up)
    g = orc.qdot_f32act(bits, gq, gs, H, x)
    u = orc.qdot_f32act(bits, uq, us, H, x)
    gd = g.astype(np.float64)
    h = ((gd / (1.0 + np.exp(-gd))) * u.astype(np.float64)).astype(np.float32)
    rows = []
    for name, wq, ws, cols, inp in (("gate-shaped 2048x6144", gq, gs, H, x),
                                    ("down-shaped 6144x2048", dq, ds, I, h)):
        xq, xd = orc.q8_0(inp)
        _, y_q8 = orc.qdot(bits, wq, ws, cols, xq, xd, want_acc=False)
        y_f32 = orc.qdot_f32act(bits, wq, ws, cols, inp)
        # the exact product of the same codes with the fp32 activations
        codes = orc.unpack(bits, wq, cols).astype(np.float64)
        y_ex = (inp.astype(np.float64) @ codes.T) * ws.astype(np.float64)[None, :]
        q8_rms, q8_max = _rel(y_q8, y_f32)
        f_rms, _ = _rel(y_f32, y_ex)
        e_rms, _ = _rel(y_q8, y_ex)
        rows.append((name, q8_rms, q8_max, f_rms))
        assert q8_rms < 1.5e-2, (name, q8_rms)
        assert f_rms < e_rms, (name, f_rms, e_rms)
    print(f"\nint{bits}: Q8_0 vs f32 activations (RMS rel, max rel per row); f32 path vs exact (RMS rel)")
    for name, a, b, c in rows:
        print(f"  {name}: {a:.3e} {b:.3e}; {c:.1e}")
