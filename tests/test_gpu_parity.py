"""GPU parity: every step of the layer on gfx950 through the C ABI, against
the CPU oracle on the same seeded inputs.

Bar: bit-exact for packed codes, scales, Q8_0 codes, int32 block
accumulators, routing indices and weights (when both sides take the same
fp32 logits) and the union tables; router logits within 1 ulp (binary64
accumulation in a different order, rounded once); layer outputs within
1e-3 of the token's largest |y| (the GPU accumulates in fp32).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (LayerPair, assert_close_layer, gpu_cfg, orc_cfg, to_dev, ulp_diff)
from quantized_moe_coli_amd import binding as B
from quantized_moe_coli_amd import inputs

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "needs a GPU"
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name


def _special_rows(rng, R, C):
    w = rng.normal(0, 0.02, size=(R, C)).astype(F32)
    w[0] = 0.0                                     # zero row
    w[1] = rng.integers(-7, 8, size=C) * F32(2.0 ** -6)  # grid row
    w[1, 0] = 7 * 2.0 ** -6
    w[2] *= F32(1e-30)                             # tiny values
    w[3] *= F32(1e30)                              # huge values
    w[4, :] = 0.0
    w[4, 5] = -3.0                                 # single negative spike
    return w


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("R,C", [(37, 96), (64, 256), (8, 6144)])
def test_quant_pack_bit_exact(orc, bits, R, C):
    rng = np.random.default_rng(R * C + bits)
    w = _special_rows(rng, R, C)
    q_ref, s_ref = orc.quant_pack(bits, w)
    q = torch.empty(R, C * bits // 8, dtype=torch.uint8, device="cuda")
    s = torch.empty(R, device="cuda")
    B.coli_quant_pack(bits, to_dev(w), q, s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_quant_pack_full_expert(orc, bits):
    """A GLM-5.2-shaped expert matrix, 2048 x 6144, drawn on the device."""
    w = inputs.normal((2048, 6144), 0.02, "cuda", 77, bits)
    q = torch.empty(2048, 6144 * bits // 8, dtype=torch.uint8, device="cuda")
    s = torch.empty(2048, device="cuda")
    B.coli_quant_pack(bits, w, q, s)
    q_ref, s_ref = orc.quant_pack(bits, w.cpu().numpy())
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


def _fp8_requant_gpu(bits, codes, bs):
    R, C = codes.shape
    q = torch.empty(R, C * bits // 8, dtype=torch.uint8, device="cuda")
    s = torch.empty(R, device="cuda")
    B.coli_quant_pack_fp8(bits, codes.cuda(), bs.cuda(), q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("R,C", [(1, 32), (200, 96), (130, 288), (256, 1024), (40, 4096), (5, 8224),
                                 (3, 16416), (129, 2080)])
def test_fp8_requant_bit_exact(orc, bits, R, C):
    """FP8 block-scaled codes -> container on the GPU equals the oracle's
    dequantisation followed by its quantisation and packing.  The shapes put
    rows and columns across ragged 128x128 tiles; special rows hold zeros of
    both signs only (scale 0), the format's extreme codes, and subnormals."""
    codes, bs = inputs.fp8_checkpoint(R, C, 5, "cpu")
    c = codes.numpy().copy()
    if R >= 4:
        c[0] = 0x80                                  # -0.0 everywhere: zero row
        c[1, :] = 0x00
        c[1, 3] = 0x7E                               # +448 spike
        c[2] = np.resize(np.array([0x01, 0x81, 0x07, 0x87, 0x08], np.uint8), C)  # subnormals
        c[3, ::2] = 0xFE                             # -448 and random codes
    codes = torch.from_numpy(c)
    q, s = _fp8_requant_gpu(bits, codes, bs)
    q_ref, s_ref = orc.requant_fp8_block(bits, c, bs.numpy())
    np.testing.assert_array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(q, q_ref)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("R,C", [(2048, 6144), (6144, 2048)])
def test_fp8_requant_full_expert(orc, bits, R, C):
    """GLM-5.2-shaped expert matrices (gate/up 2048 x 6144, down 6144 x 2048)."""
    codes, bs = inputs.fp8_checkpoint(R, C, 6, "cpu")
    q, s = _fp8_requant_gpu(bits, codes, bs)
    q_ref, s_ref = orc.requant_fp8_block(bits, codes.numpy(), bs.numpy())
    np.testing.assert_array_equal(s, s_ref)
    np.testing.assert_array_equal(q, q_ref)


def test_fp8_requant_equals_fp32_pack_on_device(orc):
    """Through the oracle's dequantised fp32 matrix, the FP8 entry point and
    coli_quant_pack write the same bytes and scales."""
    codes, bs = inputs.fp8_checkpoint(384, 640, 7, "cpu")
    q, s = _fp8_requant_gpu(4, codes, bs)
    w = to_dev(orc.dequant_fp8_block(codes.numpy(), bs.numpy()))
    q2 = torch.empty(384, 320, dtype=torch.uint8, device="cuda")
    s2 = torch.empty(384, device="cuda")
    B.coli_quant_pack(4, w, q2, s2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q, q2.cpu().numpy())
    np.testing.assert_array_equal(s.view(np.uint32), s2.cpu().numpy().view(np.uint32))


def _gemv_f32_case(orc, bits, R, C, seed, integer_x):
    rng = np.random.default_rng(seed)
    if integer_x:
        # power-of-two scales and integer activations: every fp32 summation
        # order is exact, so the GPU must match the oracle bit for bit
        q = {8: 127, 4: 7, 2: 1}[bits]
        codes = rng.integers(-q, q + 1, size=(R, C)).astype(np.float32)
        codes[:, 0] = q
        w = codes * F32(2.0 ** -7)
        x = rng.integers(-8, 9, size=C).astype(np.float32)
    else:
        w = rng.normal(0, 0.02, size=(R, C)).astype(F32)
        x = rng.normal(0, 1, size=C).astype(F32)
    packed, scale = orc.quant_pack(bits, w)
    y_ref = orc.qdot_f32act(bits, packed, scale, C, x[None, :])[0]
    y = torch.empty(R, device="cuda")
    B.coli_gemv_f32act(bits, to_dev(packed), to_dev(scale), to_dev(x), y)
    torch.cuda.synchronize()
    return y.cpu().numpy(), y_ref


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("R,C", [(1, 64), (37, 128), (130, 1088), (21, 4096)])
def test_gemv_f32act_exact_on_integer_activations(orc, bits, R, C):
    y, y_ref = _gemv_f32_case(orc, bits, R, C, R + C + bits, True)
    np.testing.assert_array_equal(y.view(np.uint32), y_ref.view(np.uint32))


@pytest.mark.parametrize("bits,R,C", [(4, 2048, 6144), (4, 6144, 2048), (2, 2048, 6144),
                                      (8, 2048, 6144), (8, 9, 8192), (2, 5, 16384),
                                      (4, 19, 16384), (8, 131, 3072)])
def test_gemv_f32act_glm_rows(orc, bits, R, C):
    """GLM-5.2 expert rows and the longest rows of each container: fp32 sums
    within 1e-4 of the row block's largest |y| (the oracle sums in binary64)."""
    y, y_ref = _gemv_f32_case(orc, bits, R, C, 7 * bits + R, False)
    assert np.abs(y.astype(np.float64) - y_ref).max() <= 1e-4 * np.abs(y_ref).max()


@pytest.mark.parametrize("T,n", [(1, 32), (3, 256), (17, 6144), (512, 2048)])
def test_act_quant_bit_exact(orc, T, n):
    rng = np.random.default_rng(T + n)
    x = rng.normal(0, 1, size=(T, n)).astype(F32)
    x[0, :32] = 0.0
    if n >= 64:
        x[0, 32:64] = rng.integers(-127, 128, size=32) * F32(2.0 ** -9)
        x[0, 32] = 127 * 2.0 ** -9
    q_ref, d_ref = orc.q8_0(x)
    q = torch.empty(T, n, dtype=torch.int8, device="cuda")
    d = torch.empty(T, n // 32, device="cuda")
    B.coli_quant_act_q8_0(to_dev(x), q, d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d.cpu().numpy(), d_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("R,C,T", [(16, 128, 1), (40, 6144, 3), (6144, 2048, 1), (7, 256, 8)])
def test_int32_block_accumulators_exact(orc, bits, R, C, T):
    rng = np.random.default_rng(bits * 1000 + R + C + T)
    # arbitrary bytes: every field value, including -8 (int4) and -2 (int2)
    packed = rng.integers(0, 256, size=(R, C * bits // 8), dtype=np.uint8)
    xq = rng.integers(-128, 128, size=(T, C)).astype(np.int8)
    xd = np.ones((T, C // 32), F32)
    acc_ref, _ = orc.qdot(bits, packed, np.ones(R, F32), C, xq, xd)
    acc = torch.empty(T, R, C // 32, dtype=torch.int32, device="cuda")
    B.coli_debug_qgemv_blocks(bits, to_dev(packed), C, to_dev(xq), acc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)


@pytest.mark.parametrize("bits", [4, 2])
def test_container_identity_on_gpu(orc, bits):
    """int4 (int2) codes in the int8 container and in the packed container
    give identical int32 block sums through the GPU kernels."""
    rng = np.random.default_rng(90 + bits)
    R, C, T = 64, 6144, 2
    w = rng.normal(0, 0.02, size=(R, C)).astype(F32)
    codes, _ = orc.quant_rows(bits, w)
    packed, cont8 = orc.pack(bits, codes), orc.pack(8, codes)
    xq = rng.integers(-127, 128, size=(T, C)).astype(np.int8)
    a_p = torch.empty(T, R, C // 32, dtype=torch.int32, device="cuda")
    a_8 = torch.empty_like(a_p)
    B.coli_debug_qgemv_blocks(bits, to_dev(packed), C, to_dev(xq), a_p)
    B.coli_debug_qgemv_blocks(8, to_dev(cont8), C, to_dev(xq), a_8)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a_p.cpu().numpy(), a_8.cpu().numpy())
    acc_ref, _ = orc.qdot(bits, packed, np.ones(R, F32), C, xq, np.ones((T, C // 32), F32))
    np.testing.assert_array_equal(a_p.cpu().numpy(), acc_ref)


@pytest.mark.parametrize("T", [1, 3, 4, 5, 37, 512])
def test_logits_within_one_ulp(orc, T):
    s = inputs.GLM
    gw = inputs.gate_weight(s, 0)
    x = inputs.tokens(s, 0, T, T)
    ref = orc.logits(x.numpy(), gw.numpy())
    out = torch.empty(T, s.n_experts, device="cuda")
    B.coli_moe_logits(x.cuda(), gw.cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert ulp_diff(got, ref).max() <= 1
    assert (got == ref).mean() > 0.99


ROUTERS = {
    "tiny": dict(E=16, k=2, G=1, TG=1, bias=0.0, top_p=0.0),
    "grouped": dict(E=16, k=4, G=4, TG=2, bias=0.05, top_p=0.0),
    "glm": dict(E=256, k=8, G=8, TG=4, bias=0.01, top_p=0.0),
    "glm_top_p": dict(E=256, k=8, G=8, TG=4, bias=0.01, top_p=0.7),
    "glm_top_p_norenorm": dict(E=256, k=8, G=8, TG=4, bias=0.01, top_p=0.7, renorm=0),
    "glm_nonorm": dict(E=256, k=8, G=8, TG=4, bias=0.01, top_p=0.0, norm=0),
    "wide": dict(E=1024, k=32, G=64, TG=8, bias=0.01, top_p=0.0),
}


@pytest.mark.parametrize("name", list(ROUTERS))
@pytest.mark.parametrize("T,rho", [(1, 0.0), (3, 0.0), (512, 0.9)])
def test_route_bit_exact(orc, name, T, rho):
    r = ROUTERS[name]
    norm, renorm = r.get("norm", 1), r.get("renorm", 1)
    lg = inputs.correlated_logits(5, T, r["E"], rho).numpy()
    rng = np.random.default_rng(T)
    bias = (rng.normal(0, r["bias"], size=r["E"]) if r["bias"] else np.zeros(r["E"])).astype(F32)
    if T > 1:
        lg[1, :] = lg[0, :]  # duplicate token
        lg[-1, : r["E"] // 2] = 0.0  # many exact ties
    oc = oracle.make_cfg(r["E"], r["k"], r["G"], r["TG"], norm, 2.5, r["top_p"], renorm)
    idx_ref, w_ref = orc.route(oc, lg, bias)
    gc = B.router_cfg(r["E"], r["k"], r["G"], r["TG"], norm, 2.5, r["top_p"], renorm)
    idx = torch.empty(T, r["k"], dtype=torch.int32, device="cuda")
    w = torch.empty(T, r["k"], device="cuda")
    B.coli_moe_route(gc, to_dev(lg), to_dev(bias), idx, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    np.testing.assert_array_equal(w.cpu().numpy(), w_ref)


@pytest.mark.parametrize("T,k,E,drop,dup", [(1, 8, 256, 0.0, False), (3, 8, 256, 0.0, False),
                                            (512, 8, 256, 0.0, False), (77, 4, 16, 0.3, False),
                                            (300, 8, 1024, 0.1, True), (2, 32, 64, 0.0, False),
                                            (600, 8, 256, 0.05, True), (50, 6, 100, 0.2, True),
                                            (4096, 8, 256, 0.0, False)])
def test_dispatch_tables_bit_exact(orc, T, k, E, drop, dup):
    rng = np.random.default_rng(T * 31 + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if dup:
        idx[::5, 1] = idx[::5, 0]  # a token naming an expert twice
    if drop:
        idx[rng.random(idx.shape) < drop] = -1
    counts_r, offs_r, perm_r, uniq_r = orc.union_tables(idx, E)
    dev = lambda n: torch.full((n,), -7, dtype=torch.int32, device="cuda")  # noqa: E731
    counts, offs, perm, uniq, nu = dev(E), dev(E + 1), dev(T * k), dev(E), dev(1)
    B.coli_moe_dispatch(to_dev(idx), E, counts, offs, perm, uniq, nu)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(counts.cpu().numpy(), counts_r)
    np.testing.assert_array_equal(offs.cpu().numpy(), offs_r)
    n = int(offs_r[-1])
    np.testing.assert_array_equal(perm.cpu().numpy()[:n], perm_r)
    assert int(nu.item()) == len(uniq_r)
    np.testing.assert_array_equal(uniq.cpu().numpy()[: len(uniq_r)], uniq_r)


# ------------------------------------------------------------------ layer --
TINY_VARIANTS = {
    "tiny_int8": inputs.TINY,                                              # the small layer, int8
    "tiny_int4": inputs.TINY.with_(bits=4),
    "tiny_int2": inputs.TINY.with_(bits=2),
    "tiny_grouped": inputs.TINY.with_(n_group=4, topk_group=2, top_k=4, bias_std=0.05, bits=4),
    "tiny_top_p": inputs.TINY.with_(n_group=4, topk_group=2, top_k=4, top_p=0.5, bits=4),
    "tiny_rsf1": inputs.TINY.with_(rsf=1.0),
    # groups of 3 experts: the selection's general group path
    "tiny_odd_groups": inputs.TINY.with_(n_experts=24, n_group=8, topk_group=3, top_k=5,
                                         bias_std=0.05, bits=4),
    # more experts than the decode workgroup has threads
    "tiny_wide": inputs.TINY.with_(n_experts=640, n_group=10, topk_group=4, top_k=6,
                                   bias_std=0.05, bits=2),
}


@pytest.fixture(scope="module")
def tiny_pairs():
    return {}


def _pair(cache, name):
    if name not in cache:
        cache[name] = LayerPair(TINY_VARIANTS[name], seed=0)
    return cache[name]


@pytest.mark.parametrize("name", list(TINY_VARIANTS))
@pytest.mark.parametrize("T", [1, 4, 5, 33])
def test_layer_tiny(tiny_pairs, name, T):
    p = _pair(tiny_pairs, name)
    x = inputs.tokens(p.s, 0, 100 + T, T)
    y_r, idx_r, w_r, lg_r = p.oracle_forward(x.numpy())
    y, idx, w, lg = p.gpu_forward(x.cuda())
    assert ulp_diff(lg, lg_r).max() <= 1
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    assert_close_layer(y, y_r)


@pytest.mark.parametrize("T", [1, 9])
def test_layer_tiny_supplied_logits(tiny_pairs, T):
    p = _pair(tiny_pairs, "tiny_grouped")
    x = inputs.tokens(p.s, 0, 7, T)
    lg = inputs.correlated_logits(3, T, p.s.n_experts, 0.5).numpy()
    y_r, idx_r, w_r, _ = p.oracle_forward(x.numpy(), lg)
    y, idx, w, lg_out = p.gpu_forward(x.cuda(), to_dev(lg))
    np.testing.assert_array_equal(lg_out, lg)
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    assert_close_layer(y, y_r)


@pytest.mark.parametrize("T", [1, 5, 40])
def test_layer_gate_offsets(T):
    """Per-expert logit offsets (a Zipf-like popularity over a random expert
    ranking) added to the computed logits, with expert top-p: batch 1 (the
    decode kernel), 5 and 40 (the two logits kernels of the union path)."""
    s = inputs.TINY.with_(n_experts=64, top_k=6, n_group=4, topk_group=2, bias_std=0.05,
                          bits=4, top_p=0.7)
    off = inputs.zipf_logit_offsets(0, 7, s.n_experts).numpy()
    p = LayerPair(s, seed=9, gate_offset=off)
    x = inputs.tokens(s, 0, 700 + T, T)
    y_r, idx_r, w_r, lg_r = p.oracle_forward(x.numpy())
    y, idx, w, lg = p.gpu_forward(x.cuda())
    l_raw = oracle.logits(x.numpy(), p.gate_w)
    assert (np.abs(lg - lg_r) <= 2.0 ** -23 * np.maximum(np.abs(l_raw), np.abs(off))).all()
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    assert_close_layer(y, y_r)


def test_layer_zero_input_and_zero_rsf(tiny_pairs):
    p = _pair(tiny_pairs, "tiny_int8")
    y, _, _, _ = p.gpu_forward(torch.zeros(3, p.s.hidden, device="cuda"))
    assert (y == 0).all()
    s0 = inputs.TINY.with_(rsf=0.0)
    p0 = LayerPair(s0, seed=0)
    x = inputs.tokens(s0, 0, 3, 5)
    y, _, w, _ = p0.gpu_forward(x.cuda())
    assert (w == 0).all()
    # with zero weights the layer is the shared expert alone
    y_sh = oracle.expert_ffn(s0.bits, s0.hidden, s0.inter, p0.orc_expert(s0.n_experts), x.numpy())
    assert_close_layer(y, y_sh)


def test_layer_empty_batch(tiny_pairs):
    p = _pair(tiny_pairs, "tiny_int8")
    y = torch.full((1, p.s.hidden), 5.0, device="cuda")
    ws = B.workspace(p.gpu, 1)
    B.coli_moe_forward(p.gpu, torch.empty(0, p.s.hidden, device="cuda"), y[:0], ws)
    torch.cuda.synchronize()
    assert (y == 5.0).all()


def test_union_equals_per_token(tiny_pairs):
    """A batch grouped by expert gives each token what it gets alone."""
    p = _pair(tiny_pairs, "tiny_int4")
    T = 12
    x = inputs.tokens(p.s, 0, 55, T).cuda()
    yb, idxb, wb, _ = p.gpu_forward(x)
    for t in range(T):
        y1, idx1, w1, _ = p.gpu_forward(x[t:t + 1].contiguous())
        np.testing.assert_array_equal(idx1[0], idxb[t])
        np.testing.assert_array_equal(w1[0], wb[t])
        assert_close_layer(y1, yb[t:t + 1], tol=1e-5)


def test_determinism(tiny_pairs):
    p = _pair(tiny_pairs, "tiny_grouped")
    x = inputs.tokens(p.s, 0, 9, 17).cuda()
    a = p.gpu_forward(x)
    b = p.gpu_forward(x)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_decode_workspace_reuse(tiny_pairs):
    """Many single-token calls on one workspace (the decode kernel's counters
    must return to zero after every call) match calls on fresh workspaces."""
    p = _pair(tiny_pairs, "tiny_grouped")
    ws = B.workspace(p.gpu, 1)
    x = inputs.tokens(p.s, 0, 77, 40).cuda()
    for t in range(40):
        a = p.gpu_forward(x[t:t + 1].contiguous(), ws=ws)
        b = p.gpu_forward(x[t:t + 1].contiguous())
        for u, v in zip(a, b):
            np.testing.assert_array_equal(u, v)
    hdr = ws[:B.WORKSPACE_COUNTER_BYTES].cpu().numpy()
    assert (hdr == 0).all()  # the status word too: no wait gave up


@pytest.mark.parametrize("T", [1, 3])
def test_graph_replay_matches_eager(tiny_pairs, T):
    """The forward captured in a HIP graph and replayed several times, with
    eager work between replays, gives the eager result every time."""
    p = _pair(tiny_pairs, "tiny_int4")
    s = p.s
    x = inputs.tokens(s, 0, 88 + T, T).cuda()
    ref = p.gpu_forward(x)[0]
    ws = B.workspace(p.gpu, T)
    y = torch.empty(T, s.hidden, device="cuda")
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            B.coli_moe_forward(p.gpu, x, y, ws)
    torch.cuda.synchronize()
    for rep in range(5):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), ref, err_msg=f"replay {rep}")
        p.gpu_forward(inputs.tokens(s, 0, 500 + rep, 2).cuda())  # eager work in between


# ------------------------------------------------ GLM-5.2-shaped layer --
@pytest.fixture(scope="module")
def glm():
    return LayerPair(inputs.GLM, seed=0, device_gen=True)


@pytest.mark.slow
def test_glm_decode(glm):
    """Batch-1 decode of the full-size layer (computed logits), 4 tokens."""
    errs = []
    for step in range(4):
        x = inputs.tokens(glm.s, 0, step, 1, "cuda")
        y, idx, w, lg = glm.gpu_forward(x)
        y_r, idx_r, w_r, lg_r = glm.oracle_forward(x.cpu().numpy())
        assert ulp_diff(lg, lg_r).max() <= 1
        np.testing.assert_array_equal(idx, idx_r)
        np.testing.assert_array_equal(w, w_r)
        errs.append(assert_close_layer(y, y_r))
    print("glm decode max rel err", max(errs))


@pytest.mark.slow
def test_glm_mtp_verify_union(glm):
    """The 3-token verify batch with supplied logits, every token checked."""
    T = 3
    x = inputs.tokens(glm.s, 0, 1000, T, "cuda")
    lg = inputs.correlated_logits(11, T, glm.s.n_experts, 0.0)
    y, idx, w, _ = glm.gpu_forward(x, lg.cuda())
    y_r, idx_r, w_r, _ = glm.oracle_forward(x.cpu().numpy(), lg.numpy())
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    assert_close_layer(y, y_r)


@pytest.mark.slow
@pytest.mark.parametrize("T", [2, 4])
def test_glm_small_batch_computed_logits(glm, T):
    """Batches of 2 and 4 tokens (one kernel: logit slices for every token,
    per-token selection, the batch union, the combine), computed logits."""
    x = inputs.tokens(glm.s, 0, 2000 + T, T, "cuda")
    y, idx, w, lg = glm.gpu_forward(x)
    y_r, idx_r, w_r, lg_r = glm.oracle_forward(x.cpu().numpy())
    assert ulp_diff(lg, lg_r).max() <= 1
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    assert_close_layer(y, y_r)


@pytest.mark.slow
def test_small_batch_wait_giveup_is_reported(glm):
    """The small-batch kernel's bounded waits (scores, selections, slots)
    forced to give up from the host, as for the decode kernel: the call
    completes, the status word records it, the header is left clear and the
    next call is bit-identical to one on a fresh workspace."""
    T = 3
    x = inputs.tokens(glm.s, 0, 7, T, "cuda")
    ref = glm.gpu_forward(x)
    ws = B.workspace(glm.gpu, T)
    off = B.WORKSPACE_SPIN_LIMIT_OFFSET
    ws[off:off + 4].copy_(torch.tensor([1, 0, 0, 0x80], dtype=torch.uint8))  # 0x80000001
    glm.gpu_forward(x, ws=ws)  # outputs undefined
    st = _ws_status(ws, clear=True)
    assert st == B.WAIT_SCORES | B.WAIT_SLOTS, st
    hdr = ws[:B.WORKSPACE_COUNTER_BYTES].cpu().numpy()
    assert (hdr == 0).all()
    b = glm.gpu_forward(x, ws=ws)
    for u, v in zip(b, ref):
        np.testing.assert_array_equal(u, v)
    assert _ws_status(ws) == 0


@pytest.mark.slow
@pytest.mark.parametrize("T", [8, 64])
def test_glm_union_sampled(glm, T):
    """Computed logits; a union batch of T tokens, 3 sampled tokens checked
    against the oracle, the routing of all tokens checked."""
    x = inputs.tokens(glm.s, 0, 2000 + T, T, "cuda")
    y, idx, w, lg = glm.gpu_forward(x)
    xh = x.cpu().numpy()
    lg_r = oracle.logits(xh, glm.gate_w)
    assert ulp_diff(lg, lg_r).max() <= 1
    idx_r, w_r = oracle.route(orc_cfg(glm.s), lg_r, glm.gate_bias)
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    for t in (0, T // 2, T - 1):
        y_r, _, _, _ = glm.oracle_forward(xh[t:t + 1])
        assert_close_layer(y[t:t + 1], y_r)


def _ws_status(ws, clear=False) -> int:
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    B.coli_moe_workspace_status(ws, st, clear=clear)
    torch.cuda.synchronize()
    return int(st.item())


@pytest.mark.slow
def test_decode_wait_giveup_is_reported(glm):
    """Failure handling of the decode kernel's bounded waits, forced from the
    host: the workspace's test hook (one polling round, every wait treating
    its data as absent) makes every wait give up.  The call completes (every
    workgroup exits), the sticky status word records the give-ups, the call
    clears the hook, and after the status is cleared the next call on the
    same workspace is bit-identical to one on a fresh workspace."""
    x = inputs.tokens(glm.s, 0, 6, 1, "cuda")
    ref = glm.gpu_forward(x)
    ws = B.workspace(glm.gpu, 1)
    assert _ws_status(ws) == 0
    a = glm.gpu_forward(x, ws=ws)
    for u, v in zip(a, ref):
        np.testing.assert_array_equal(u, v)
    assert _ws_status(ws) == 0
    off = B.WORKSPACE_SPIN_LIMIT_OFFSET
    ws[off:off + 4].copy_(torch.tensor([1, 0, 0, 0x80], dtype=torch.uint8))  # 0x80000001
    glm.gpu_forward(x, ws=ws)  # outputs undefined
    st = _ws_status(ws, clear=True)
    assert st == B.WAIT_SCORES | B.WAIT_SLOTS, st
    assert _ws_status(ws) == 0
    hdr = ws[:B.WORKSPACE_COUNTER_BYTES].cpu().numpy()
    assert (hdr == 0).all()  # counters, scores and the hook cleared by the call
    b = glm.gpu_forward(x, ws=ws)
    for u, v in zip(b, ref):
        np.testing.assert_array_equal(u, v)
    assert _ws_status(ws) == 0


def test_decode_garbage_ticket_counters_stay_in_bounds(glm):
    """A workspace whose work-queue counters hold garbage (a caller that let
    the memory be reused: nonzero words, values with the sign bit set, float
    bit patterns) must not make the decode kernel index outside its items:
    the call completes, its last workgroup clears the header, and the next
    call is bit-identical to one on a fresh workspace.  Only the eight ticket
    words are planted; the polling bound and status words stay zero."""
    x = inputs.tokens(glm.s, 0, 9, 1, "cuda")
    ref = glm.gpu_forward(x)
    ws = B.workspace(glm.gpu, 1)
    words = ws[:B.WORKSPACE_COUNTER_BYTES].view(torch.int32)
    garbage = [0x3F800000, -0x40800000, 0x7FFFFFFF, -1, -0x80000000, 1, 0x40000000, -0x21524111]
    for q, v in enumerate(garbage):
        words[64 * q] = v  # queue q's ticket counter (one 256-byte line per counter)
    torch.cuda.synchronize()
    glm.gpu_forward(x, ws=ws)  # outputs undefined: items were skipped
    torch.cuda.synchronize()
    hdr = ws[:B.WORKSPACE_COUNTER_BYTES].cpu().numpy()
    assert (hdr == 0).all()
    b = glm.gpu_forward(x, ws=ws)
    for u, v in zip(b, ref):
        np.testing.assert_array_equal(u, v)
    assert _ws_status(ws) == 0


# The full-size layer (256 experts, computed logits) in the int8 and int2
# containers at batch 1, 8 and 64 (the int4 container is covered above): the
# precision-by-batch grid.  Routing of every token is checked; outputs for
# every token at T = 1 and for three sampled tokens of larger batches.
@pytest.fixture(scope="module")
def glm_containers():
    return {}


@pytest.mark.slow
@pytest.mark.parametrize("bits", [8, 2])
@pytest.mark.parametrize("T", [1, 8, 64])
def test_glm_full_containers(glm_containers, bits, T):
    if bits not in glm_containers:
        glm_containers.clear()  # one full-size layer resident at a time
        glm_containers[bits] = LayerPair(inputs.GLM.with_(bits=bits), seed=4, device_gen=True)
    p = glm_containers[bits]
    x = inputs.tokens(p.s, 0, 3000 + T, T, "cuda")
    y, idx, w, lg = p.gpu_forward(x)
    xh = x.cpu().numpy()
    lg_r = oracle.logits(xh, p.gate_w)
    assert ulp_diff(lg, lg_r).max() <= 1
    idx_r, w_r = oracle.route(orc_cfg(p.s), lg_r, p.gate_bias)
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    for t in sorted({0, T // 2, T - 1}):
        y_r, _, _, _ = p.oracle_forward(xh[t:t + 1])
        assert_close_layer(y[t:t + 1], y_r)


# GLM-5.2 row shapes (H 6144, I 2048) in the int8 and int2 containers, with
# 16 experts so the layer packs quickly: the decode kernel's other row
# layouts and the union path at full row length.
@pytest.fixture(scope="module")
def glm_rows():
    return {}


@pytest.mark.slow
@pytest.mark.parametrize("bits", [8, 2])
@pytest.mark.parametrize("T", [1, 3])
def test_glm_rows_other_containers(glm_rows, bits, T):
    if bits not in glm_rows:
        s = inputs.GLM.with_(n_experts=16, top_k=4, n_group=4, topk_group=2, bits=bits)
        glm_rows[bits] = LayerPair(s, seed=3, device_gen=True)
    p = glm_rows[bits]
    x = inputs.tokens(p.s, 0, 40 + T, T, "cuda")
    y, idx, w, lg = p.gpu_forward(x)
    y_r, idx_r, w_r, lg_r = p.oracle_forward(x.cpu().numpy())
    assert ulp_diff(lg, lg_r).max() <= 1
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    assert_close_layer(y, y_r)


# The matrix-core union path (experts with at least mfma_min_tokens tokens
# run on v_mfma_i32_16x16x32_i8) against the oracle, with every slot forced
# onto it (min 1), with none on it (min large), and at the library default.
@pytest.fixture(scope="module")
def mfma_pairs():
    return {}


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("mfma_min", [1, 0, 1 << 30])
@pytest.mark.parametrize("T", [2, 33, 130])
def test_union_matrix_cores(mfma_pairs, bits, mfma_min, T):
    key = (bits, mfma_min)
    if key not in mfma_pairs:
        s = inputs.TINY.with_(n_experts=16, top_k=4, n_group=4, topk_group=2, bias_std=0.05,
                              bits=bits)
        mfma_pairs[key] = LayerPair(s, seed=5, mfma_min_tokens=mfma_min)
    p = mfma_pairs[key]
    x = inputs.tokens(p.s, 0, 300 + T, T)
    y_r, idx_r, w_r, _ = p.oracle_forward(x.numpy())
    y, idx, w, _ = p.gpu_forward(x.cuda())
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    assert_close_layer(y, y_r)


@pytest.mark.slow
@pytest.mark.parametrize("bits", [4, 2])
def test_glm_rows_matrix_cores(glm_rows, bits):
    """GLM-5.2 row lengths on the matrix cores: 96 tokens over 16 experts
    (about 24 per expert, shared expert 96) with every slot on MFMA."""
    if bits not in glm_rows:
        s = inputs.GLM.with_(n_experts=16, top_k=4, n_group=4, topk_group=2, bits=bits)
        glm_rows[bits] = LayerPair(s, seed=3, device_gen=True)
    p = glm_rows[bits]
    p.gpu.mfma_min_tokens = 1
    try:
        T = 96
        x = inputs.tokens(p.s, 0, 900, T, "cuda")
        y, idx, w, lg = p.gpu_forward(x)
        xh = x.cpu().numpy()
        lg_r = oracle.logits(xh, p.gate_w)
        idx_r, w_r = oracle.route(orc_cfg(p.s), lg_r, p.gate_bias)
        np.testing.assert_array_equal(idx, idx_r)
        for t in (0, 47, 95):
            y_r, _, _, _ = p.oracle_forward(xh[t:t + 1])
            assert_close_layer(y[t:t + 1], y_r)
    finally:
        p.gpu.mfma_min_tokens = 0


# Matrix-core work items cover up to 64 tokens of one expert; an expert with
# more runs as several token groups (first token n0 = 0, 64, 128, ...).
@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("mfma_min", [1, 0])
def test_union_matrix_cores_long_groups(bits, mfma_min):
    """4 experts top-2 over 300 tokens: every routed expert receives 139-165
    tokens, so each runs as three 64-token groups on the matrix cores, and
    the shared expert (300 tokens) as five."""
    s = inputs.TINY.with_(n_experts=4, top_k=2, n_group=1, topk_group=1, bits=bits)
    p = LayerPair(s, seed=5, mfma_min_tokens=mfma_min)
    T = 300
    x = inputs.tokens(s, 0, 301, T)
    y_r, idx_r, w_r, _ = p.oracle_forward(x.numpy())
    counts = np.bincount(idx_r.ravel(), minlength=s.n_experts)
    assert counts.min() > 128, counts  # the case this test is for
    y, idx, w, _ = p.gpu_forward(x.cuda())
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    assert_close_layer(y, y_r)


def _prefill_picks(idx: np.ndarray, E: int, T: int, n_experts_checked: int = 3) -> list[int]:
    """Tokens to check against the oracle in a long batch: every 73rd token
    (spread over the batch and over the shared expert's 64-token groups),
    the last one, and in the batch's most loaded experts the tokens at
    union positions 64, 130 and the last (past the first and second 64-token
    group of that expert's matrix-core work)."""
    counts = np.bincount(idx[idx >= 0], minlength=E)
    picks = set(range(0, T, 73)) | {T - 1}
    for e in np.argsort(-counts, kind="stable")[:n_experts_checked]:
        toks = np.nonzero((idx == e).any(axis=1))[0]
        for pos in (64, 130, len(toks) - 1):
            if pos < len(toks):
                picks.add(int(toks[pos]))
    return sorted(picks)


@pytest.mark.slow
@pytest.mark.parametrize("rho", [0.0, 0.99])
def test_glm_prefill512(glm, rho):
    """The 512-token prefill batch at full GLM-5.2 shape (256 int4 experts,
    logits supplied with correlation rho across the batch): routing of every
    token bit-exact, and the outputs of sampled tokens within the layer
    tolerance.  rho = 0 gives ~256 unique experts of ~16 tokens each; rho =
    0.99 gives ~20-30 unique experts, the busiest with up to 512 tokens, so
    routed experts run as several 64-token matrix-core groups."""
    T = 512
    E = glm.s.n_experts
    x = inputs.tokens(glm.s, 0, 4000, T, "cuda")
    lg = inputs.correlated_logits(21, T, E, rho)
    y, idx, w, _ = glm.gpu_forward(x, lg.cuda())
    lgh = lg.numpy()
    idx_r, w_r = oracle.route(orc_cfg(glm.s), lgh, glm.gate_bias)
    np.testing.assert_array_equal(idx, idx_r)
    np.testing.assert_array_equal(w, w_r)
    counts = np.bincount(idx_r[idx_r >= 0], minlength=E)
    if rho > 0.9:
        assert counts.max() > 128, counts.max()  # routed multi-group items run
    picks = _prefill_picks(idx_r, E, T)
    assert len(picks) >= 8, picks
    xh = x.cpu().numpy()
    errs = []
    for t in picks:
        y_r, _, _, _ = glm.oracle_forward(xh[t:t + 1], lgh[t:t + 1])
        errs.append(assert_close_layer(y[t:t + 1], y_r))
    print(f"prefill512 rho {rho}: U {int((counts > 0).sum())}, max tokens/expert "
          f"{counts.max()}, {len(picks)} tokens checked, max rel err {max(errs):.2e}")
