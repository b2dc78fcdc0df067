"""The 40-layer GLM-5.2-shaped stack (40 x 257 int4 experts resident, ~195
GB) with Zipf-skewed expert popularity and expert top-p 0.7, decoded one
token at a time through HIP graphs.

Layer parity: layers 0, 19 and 39 of the resident stack, on the stack's step
inputs (steps 0, 1, 255) fed straight to the layer, against the oracle (its
logits from the gate plus the layer's offsets, routed and combined by its own
code).  The oracle takes no input from the GPU, so the chained hidden state
is not handed to it; the chain is checked by what holds at any size: graph
replays equal eager runs bit for bit, every layer's routing keeps distinct
experts whose weights sum to the scaling factor, the popularity skew shows in
the selections, and the hidden state stays finite and bounded."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_coli_amd import binding as B
from quantized_moe_coli_amd import inputs, stack

from gpu_util import assert_close_layer, orc_cfg

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N_LAYERS = 40
N_STEPS = 256


@pytest.fixture(scope="module")
def stk():
    torch.cuda.empty_cache()
    st = stack.build(N_LAYERS)
    yield st
    del st
    torch.cuda.empty_cache()


def _oracle_layer(st, li, x: np.ndarray):
    """The oracle's forward of layer li on x [1, H]: O5 logits plus the
    layer's offsets (one binary32 addition), then the layer on them."""
    s = st.s
    L = st.layers[li]
    gate_w = L.gate_w.cpu().numpy()
    bias = L.gate_bias.cpu().numpy()
    off = st.offsets[li].cpu().numpy()
    lg = (oracle.logits(x, gate_w) + off[None, :]).astype(np.float32)
    cfg = orc_cfg(s)
    idx, _ = oracle.route(cfg, lg, bias)
    experts = [None] * s.n_experts

    def ex(e):
        g, u, d = (t.cpu().numpy() for t in
                   inputs.expert_weights(s, stack.layer_seed(li), e, "cuda"))
        return oracle.Expert.from_float(s.bits, g, u, d)

    for e in set(idx.ravel().tolist()):
        if e >= 0:
            experts[e] = ex(e)
    layer = oracle.Layer(s.hidden, s.inter, s.bits, cfg, experts, ex(s.n_experts), gate_w, bias)
    y, idx_r, w_r, _ = oracle.moe_forward(layer, x, lg)
    return y, idx_r, w_r, lg


@pytest.mark.parametrize("li", [0, 19, 39])
def test_stack_layer_parity(stk, li):
    s = stk.s
    ws = B.workspace(stk.layers[li], 1)
    for step in (0, 1, N_STEPS - 1):
        x = inputs.tokens(s, stack.token_seed(), step, 1, "cuda")
        y = torch.empty(1, s.hidden, device="cuda")
        idx = torch.empty(1, s.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(1, s.top_k, device="cuda")
        lg = torch.empty(1, s.n_experts, device="cuda")
        B.coli_moe_forward(stk.layers[li], x, y, ws, idx_out=idx, w_out=w, logits_out=lg)
        torch.cuda.synchronize()
        y_r, idx_r, w_r, lg_r = _oracle_layer(stk, li, x.cpu().numpy())
        # the summed logit within one unit in the last place of its larger
        # addend (the binary64 dot products agree to far below that)
        l_raw = oracle.logits(x.cpu().numpy(), stk.layers[li].gate_w.cpu().numpy())
        bound = 2.0 ** -23 * np.maximum(np.abs(l_raw), np.abs(stk.offsets[li].cpu().numpy()))
        assert (np.abs(lg.cpu().numpy() - lg_r) <= bound).all()
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_r)
        np.testing.assert_array_equal(w.cpu().numpy(), w_r)
        assert_close_layer(y.cpu().numpy(), y_r)
        # top-p keeps between 1 and k of the selected experts
        kept = int((idx_r >= 0).sum())
        assert 1 <= kept <= s.top_k



@pytest.mark.parametrize("li", [0, 39])
def test_stack_verify_batch_parity(stk, li):
    """An MTP verify batch (the current token and two drafts, drawn as the
    stack's 3-token step inputs) through layer li as one batch union, against
    the oracle, which computes each token on its own."""
    s = stk.s
    ws = B.workspace(stk.layers[li], 3)
    for step in (0, N_STEPS - 1):
        x = inputs.tokens(s, stack.token_seed(), step, 3, "cuda")
        y = torch.empty(3, s.hidden, device="cuda")
        idx = torch.empty(3, s.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(3, s.top_k, device="cuda")
        lg = torch.empty(3, s.n_experts, device="cuda")
        B.coli_moe_forward(stk.layers[li], x, y, ws, idx_out=idx, w_out=w, logits_out=lg)
        torch.cuda.synchronize()
        y_r, idx_r, w_r, lg_r = _oracle_layer(stk, li, x.cpu().numpy())
        l_raw = oracle.logits(x.cpu().numpy(), stk.layers[li].gate_w.cpu().numpy())
        bound = 2.0 ** -23 * np.maximum(np.abs(l_raw), np.abs(stk.offsets[li].cpu().numpy())[None, :])
        assert (np.abs(lg.cpu().numpy() - lg_r) <= bound).all()
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_r)
        np.testing.assert_array_equal(w.cpu().numpy(), w_r)
        assert_close_layer(y.cpu().numpy(), y_r)
        kept = (idx_r >= 0).sum(axis=1)
        assert ((kept >= 1) & (kept <= s.top_k)).all()

def _chain_eager(st, x, ws, y, idx_rec, w_rec):
    h = x.clone()
    stack.step(st, h, ws, y, idx_rec, w_rec)
    torch.cuda.synchronize()
    return h


def test_stack_chain(stk):
    s, nl = stk.s, stk.n_layers
    ws = B.workspace(stk.layers[0], 1)
    xs = torch.stack([inputs.tokens(s, stack.token_seed(), t, 1, "cuda") for t in range(N_STEPS)])
    h = torch.empty(1, s.hidden, device="cuda")
    y = torch.empty(1, s.hidden, device="cuda")
    idx_g = torch.empty(nl, 1, s.top_k, dtype=torch.int32, device="cuda")
    w_g = torch.empty(nl, 1, s.top_k, device="cuda")

    # one graph for one step, replayed per step on a fresh token
    h.copy_(xs[0])
    stack.step(stk, h, ws, y, idx_g, w_g)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            stack.step(stk, h, ws, y, idx_g, w_g)
    torch.cuda.synchronize()

    idx_all = torch.empty(N_STEPS, nl, s.top_k, dtype=torch.int32, device="cuda")
    w_all = torch.empty(N_STEPS, nl, s.top_k, device="cuda")
    h_all = torch.empty(N_STEPS, s.hidden, device="cuda")
    for t in range(N_STEPS):
        h.copy_(xs[t])
        g.replay()
        idx_all[t].copy_(idx_g[:, 0])
        w_all[t].copy_(w_g[:, 0])
        h_all[t].copy_(h[0])
    torch.cuda.synchronize()

    # replays equal eager runs, bit for bit, with eager work in between
    idx_e = torch.empty_like(idx_g)
    w_e = torch.empty_like(w_g)
    for t in (0, 1, 17, N_STEPS - 1):
        he = _chain_eager(stk, xs[t], ws, y, idx_e, w_e)
        np.testing.assert_array_equal(he[0].cpu().numpy(), h_all[t].cpu().numpy(),
                                      err_msg=f"step {t}")
        np.testing.assert_array_equal(idx_e[:, 0].cpu().numpy(), idx_all[t].cpu().numpy())
        np.testing.assert_array_equal(w_e[:, 0].cpu().numpy(), w_all[t].cpu().numpy())

    idx = idx_all.cpu().numpy()
    w = w_all.cpu().numpy()
    hh = h_all.cpu().numpy()
    assert np.isfinite(hh).all()
    rms = np.sqrt((hh.astype(np.float64) ** 2).mean(axis=1))
    assert (rms > 0.1).all() and (rms < 1e3).all(), (rms.min(), rms.max())

    # every layer's routing: top-p keeps the highest-weight experts and marks
    # the other slots in place (-1, weight 0); kept weights sum to rsf
    kept = idx >= 0
    n_kept = kept.sum(axis=2)
    assert (n_kept >= 1).all() and (n_kept <= s.top_k).all()
    assert (w[~kept] == 0).all() and (w[kept] > 0).all()
    wsum = np.where(kept, w, 0.0).astype(np.float64).sum(axis=2)
    np.testing.assert_allclose(wsum, s.rsf, rtol=1e-5)
    for t in range(0, N_STEPS, 37):
        for li in range(nl):
            row = idx[t, li][kept[t, li]]
            assert len(set(row.tolist())) == len(row)
            assert (row < s.n_experts).all()
    # top-p keeps fewer than k experts on average
    assert n_kept.mean() < s.top_k

    # the popularity skew: each layer's 8 highest-ranked experts take far
    # more than their uniform share (8/256) of the selections
    share = []
    for li in range(nl):
        off = stk.offsets[li].cpu().numpy()
        top = set(np.argsort(-off, kind="stable")[:8].tolist())
        sel = idx[:, li][kept[:, li]]
        share.append(np.isin(sel, list(top)).mean())
    assert min(share) > 4 * 8 / s.n_experts, share
    print(f"stack: mean kept experts {n_kept.mean():.2f}; top-8 share {np.mean(share):.2f}")
