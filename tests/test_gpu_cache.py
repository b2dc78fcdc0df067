"""Tiered expert residency on the GPU through the C ABI.

The cache moves bytes, not arithmetic: with the same logits, a forward
through the cache must give outputs bit-identical to coli_moe_forward on the
fully resident layer, and the cache's device state after every call must
equal the reference model's (oracle/cache_model.py) fed the same routing.
Without supplied logits, the cached path's routing must equal the oracle's
on the logits it reports, and its outputs must match the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import LayerPair, assert_close_layer, gpu_cfg, orc_cfg, to_dev, ulp_diff
from oracle.cache_model import ExpertCacheModel
from quantized_moe_coli_amd import binding as B
from quantized_moe_coli_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "needs a GPU"
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name


def cached_twin(pair: LayerPair, n_slots: int):
    """The pair's layer with its routed experts moved to a host tier and
    n_slots empty HBM slots in front of it (gate, bias, offsets and shared
    expert shared with the resident layer)."""
    s, g = pair.s, pair.gpu
    tier = B.HostTier(s.n_experts, s.hidden, s.inter, s.bits)
    tier.load_experts(g)
    slots = B.MoeLayer.empty(s.hidden, s.inter, s.bits, gpu_cfg(s), gate=False, n_slots=n_slots)
    lay = B.MoeLayer(s.hidden, s.inter, s.bits, gpu_cfg(s), g.gate_w, g.gate_bias,
                     slots.w_gate, slots.s_gate, slots.w_up, slots.s_up, slots.w_down, slots.s_down,
                     g.sh_gate, g.sh_s_gate, g.sh_up, g.sh_s_up, g.sh_down, g.sh_s_down,
                     g.mfma_min_tokens, g.gate_offset)
    cache = B.ExpertCache(tier, n_slots)
    cache.init()
    return lay, cache


def assert_state(cache: B.ExpertCache, m: ExpertCacheModel):
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cache.slot_of.cpu().numpy(), m.slot_of)
    np.testing.assert_array_equal(cache.expert_of.cpu().numpy(), m.expert_of)
    np.testing.assert_array_equal(cache.last_use.cpu().numpy(), m.last_use)
    np.testing.assert_array_equal(cache.pinned.cpu().numpy(), m.pinned)
    np.testing.assert_array_equal(cache.use_count.cpu().numpy(), m.use_count)
    st = cache.stats()
    assert (st["clock"], st["copied"], st["error"]) == (m.clock, len(m.copies), m.error)
    assert (st["hits"], st["misses"]) == (m.hits, m.misses)


def run_pair(pair, lay, cache, x, logits=None):
    """Resident forward (its own logits, reported), then the cached forward
    on those logits; returns both sides' (y, idx, w) and the logits."""
    s = pair.s
    T = x.shape[0]
    ws = B.workspace(pair.gpu, T)
    out = []
    lg = torch.empty(T, s.n_experts, device="cuda")
    for which in ("resident", "cached"):
        y = torch.empty(T, s.hidden, device="cuda")
        idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, s.top_k, device="cuda")
        if which == "resident":
            B.coli_moe_forward(pair.gpu, x, y, ws, logits_in=logits, idx_out=idx, w_out=w,
                               logits_out=lg)
        else:
            B.coli_moe_forward_cached(lay, cache, x, y, ws, logits_in=lg, idx_out=idx, w_out=w)
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()))
    return out[0], out[1], lg


SMALL = inputs.Shape(hidden=256, inter=128, n_experts=16, top_k=4, n_group=4, topk_group=2,
                     rsf=2.5, bias_std=0.01, bits=4)


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_cached_decode_matches_resident_and_model(bits):
    s = SMALL.with_(bits=bits)
    pair = LayerPair(s, seed=3)
    S = 6
    lay, cache = cached_twin(pair, S)
    m = ExpertCacheModel(s.n_experts, S)
    for step in range(40):
        x = inputs.tokens(s, 9, step, 1, "cuda")
        (y_r, i_r, w_r), (y_c, i_c, w_c), _ = run_pair(pair, lay, cache, x)
        np.testing.assert_array_equal(i_c, i_r)
        np.testing.assert_array_equal(w_c.view(np.uint32), w_r.view(np.uint32))
        np.testing.assert_array_equal(y_c.view(np.uint32), y_r.view(np.uint32))
        m.step(i_r.ravel())
        assert_state(cache, m)
    st = cache.stats()
    assert st["misses"] > S and st["hits"] > 0  # the run evicted and reused


def test_cached_decode_own_logits_against_oracle():
    """No supplied logits: the cached path computes them (gate plus
    offsets), routes, fills and runs; routing equals the oracle's on the
    logits it reports and the outputs match the oracle's."""
    s = SMALL
    rng = np.random.default_rng(4)
    off = rng.normal(0, 1.0, size=s.n_experts).astype(np.float32)
    pair = LayerPair(s, seed=5, gate_offset=off)
    lay, cache = cached_twin(pair, 5)
    ws = B.workspace(lay, 1)
    for step in range(12):
        x = inputs.tokens(s, 6, step, 1, "cuda")
        y = torch.empty(1, s.hidden, device="cuda")
        idx = torch.empty(1, s.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(1, s.top_k, device="cuda")
        lg = torch.empty(1, s.n_experts, device="cuda")
        B.coli_moe_forward_cached(lay, cache, x, y, ws, idx_out=idx, w_out=w, logits_out=lg)
        torch.cuda.synchronize()
        lg_np = lg.cpu().numpy()
        lg_ref = (oracle.logits(x.cpu().numpy(), pair.gate_w) + off[None, :]).astype(np.float32)
        assert ulp_diff(lg_np, lg_ref).max() <= 1
        i_ref, w_ref = oracle.route(orc_cfg(s), lg_np, pair.gate_bias)
        np.testing.assert_array_equal(idx.cpu().numpy(), i_ref)
        np.testing.assert_array_equal(w.cpu().numpy(), w_ref)
        y_ref, _, _, _ = pair.oracle_forward(x.cpu().numpy(), logits_in=lg_np)
        assert_close_layer(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("T", [2, 3, 4, 8])
def test_cached_union_matches_resident_and_model(T):
    """Batches (MTP verify, a short prefill) through the cache: the union
    path reads each unique expert from its slot.  Resident batches of 2-4
    tokens run as one kernel, whose arithmetic is the union path's: the
    outputs agree bit for bit."""
    s = SMALL.with_(n_experts=64, n_group=8, topk_group=4)
    pair = LayerPair(s, seed=8)
    S = min(s.n_experts, T * s.top_k) + 4
    lay, cache = cached_twin(pair, S)
    m = ExpertCacheModel(s.n_experts, S)
    for step in range(10):
        x = inputs.tokens(s, 2, step, T, "cuda")
        (y_r, i_r, w_r), (y_c, i_c, w_c), _ = run_pair(pair, lay, cache, x)
        np.testing.assert_array_equal(i_c, i_r)
        np.testing.assert_array_equal(w_c.view(np.uint32), w_r.view(np.uint32))
        np.testing.assert_array_equal(y_c.view(np.uint32), y_r.view(np.uint32))
        m.step(i_r.ravel())
        assert_state(cache, m)


def test_repin_and_usage_profile(tmp_path):
    s = SMALL
    pair = LayerPair(s, seed=12)
    S = 8
    lay, cache = cached_twin(pair, S)
    m = ExpertCacheModel(s.n_experts, S)
    for step in range(15):
        x = inputs.tokens(s, 13, step, 1, "cuda")
        (_, i_r, _), (y_c, i_c, _), _ = run_pair(pair, lay, cache, x)
        m.step(i_r.ravel())
    assert_state(cache, m)
    cache.repin(lay, 3)
    m.repin(3)
    assert_state(cache, m)
    assert cache.c.n_pinned == 3
    pinned_experts = {e for e, p in zip(m.expert_of, m.pinned) if p}
    for step in range(15, 35):
        x = inputs.tokens(s, 13, step, 1, "cuda")
        (y_r, i_r, _), (y_c, i_c, _), _ = run_pair(pair, lay, cache, x)
        np.testing.assert_array_equal(y_c.view(np.uint32), y_r.view(np.uint32))
        m.step(i_r.ravel())
        assert_state(cache, m)
        assert pinned_experts <= {int(e) for e in cache.expert_of.cpu().numpy()}
    # the usage profile survives a save, an init and a load
    p = tmp_path / "usage.txt"
    cache.save_usage(str(p))
    before = cache.use_count.cpu().numpy().copy()
    cache.init()
    assert cache.use_count.cpu().numpy().sum() == 0 and cache.c.n_pinned == 0
    cache.load_usage(str(p))
    np.testing.assert_array_equal(cache.use_count.cpu().numpy(), before)


def test_glm_decode_through_a_small_cache():
    """GLM-5.2 shape (256 experts of ~19 MB int4) with a Zipf-skewed gate and
    32 HBM slots: outputs bit-identical to the resident layer, state equal
    to the model, and the host-link copies land whole experts."""
    s = inputs.GLM
    off = inputs.zipf_logit_offsets(0, 0, s.n_experts, 1.1, "cpu").numpy()
    pair = LayerPair(s, seed=0, device_gen=True, gate_offset=off)
    S = 32
    lay, cache = cached_twin(pair, S)
    m = ExpertCacheModel(s.n_experts, S)
    for step in range(24):
        x = inputs.tokens(s, 1, step, 1, "cuda")
        (y_r, i_r, w_r), (y_c, i_c, w_c), _ = run_pair(pair, lay, cache, x)
        np.testing.assert_array_equal(i_c, i_r)
        np.testing.assert_array_equal(y_c.view(np.uint32), y_r.view(np.uint32))
        m.step(i_r.ravel())
        assert_state(cache, m)
    # every resident slot holds its expert's bytes exactly
    eo = cache.expert_of.cpu().numpy()
    for sl in range(0, S, 5):
        e = int(eo[sl])
        if e < 0:
            continue
        for name in ("w_gate", "w_down", "s_up"):
            a = getattr(lay, name)[sl].cpu()
            b = getattr(pair.gpu, name)[e].cpu()
            assert torch.equal(a, b), (name, sl, e)


def test_cache_rejects_batches_that_do_not_fit_and_foreign_host_memory():
    s = SMALL
    pair = LayerPair(s, seed=1)
    lay, cache = cached_twin(pair, 6)
    x = inputs.tokens(s, 0, 0, 2, "cuda")  # 2 tokens x 4 experts > 6 slots
    y = torch.empty(2, s.hidden, device="cuda")
    ws = B.workspace(lay, 2)
    with pytest.raises(B.ColiError) as ei:
        B.coli_moe_forward_cached(lay, cache, x, y, ws)
    assert ei.value.status == B.COLI_ERR_UNSUPPORTED
    cache.repin(lay, 3)
    with pytest.raises(B.ColiError) as ei:  # 4 experts > 6 - 3 unpinned slots
        B.coli_moe_forward_cached(lay, cache, x[:1], y[:1], ws)
    assert ei.value.status == B.COLI_ERR_UNSUPPORTED
    # a host tier that did not come from coli_host_alloc is refused
    foreign = torch.empty(cache.tier.w_gate.numel(), dtype=torch.uint8).pin_memory()
    bad = B.ExpertCache(cache.tier, 6)
    bad.c.host_w_gate = foreign.data_ptr()
    with pytest.raises(B.ColiError) as ei:
        B.coli_moe_forward_cached(lay, bad, x[:1], y[:1], ws)
    assert ei.value.status == B.COLI_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert cache.stats()["error"] == 0
