"""Host-side checks of the C-ABI library (no kernel runs here).

The library loads, exports every function include/coli_moe.h declares, and
rejects bad arguments with the documented status before touching a device;
on a host without a GPU a well-formed call reports COLI_ERR_DEVICE instead of
crashing.
"""
import ctypes

import pytest
import torch

from quantized_moe_coli_amd import binding as B

P = ctypes.c_void_p


def _fake(addr):  # aligned, never dereferenced on the host
    return ctypes.c_void_p(addr)


def _layer_struct(H=6144, I=2048, q=4, E=256, k=8, G=8, TG=4):
    cfg = B.router_cfg(E, k, G, TG)
    p = [_fake(0x10000 * (i + 1)) for i in range(16)]
    return B.MoeLayerC(H, I, q, cfg, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8],
                       p[9], p[10], p[11], p[12], p[13], 0)


def test_library_loads_and_exports_every_declared_symbol():
    L = B.lib()
    names = B.declared_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert B.coli_abi_version() == 1


def test_status_strings():
    L = B.lib()
    for s in range(5):
        assert L.coli_status_str(s)
    assert L.coli_status_str(99) == b"unknown status"


def test_invalid_arguments_rejected_before_device():
    L = B.lib()
    # bad qtype / null pointers / bad shapes
    assert L.coli_quant_pack(3, _fake(16), 4, 32, _fake(16), _fake(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_quant_pack(4, None, 4, 32, _fake(16), _fake(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_quant_pack(4, _fake(16), 4, 48, _fake(16), _fake(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_quant_act_q8_0(_fake(16), 1, 33, _fake(16), _fake(16), None) == B.COLI_ERR_INVALID_ARG
    f = _fake
    # f32-activation GEMV: bad qtype, ragged columns, misaligned x, rows too long
    assert L.coli_gemv_f32act(3, f(16), f(16), 4, 64, f(16), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_gemv_f32act(2, f(16), f(16), 4, 32, f(16), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_gemv_f32act(4, f(16), f(16), 4, 64, f(8), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_gemv_f32act(4, f(16), None, 4, 64, f(16), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_gemv_f32act(4, f(16), f(16), 4, 16384 + 32, f(16), f(16), None) \
        == B.COLI_ERR_UNSUPPORTED
    assert L.coli_gemv_f32act(8, f(16), f(16), 4, 8192 + 32, f(16), f(16), None) \
        == B.COLI_ERR_UNSUPPORTED
    # FP8 requantisation: bad qtype, null scales, ragged columns, misaligned codes or output
    f = _fake
    assert L.coli_quant_pack_fp8(5, f(16), f(16), 4, 32, f(16), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_quant_pack_fp8(4, f(16), None, 4, 32, f(16), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_quant_pack_fp8(4, f(16), f(16), 4, 40, f(16), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_quant_pack_fp8(4, f(8), f(16), 4, 32, f(16), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_quant_pack_fp8(4, f(16), f(16), 4, 32, f(8), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_quant_pack_fp8(4, f(16), f(16), -1, 32, f(16), f(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_quant_act_q8_0(_fake(8), 1, 32, _fake(16), _fake(16), None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_moe_logits(_fake(16), _fake(16), 1, 0, 64, _fake(16), None) == B.COLI_ERR_INVALID_ARG
    bad = B.router_cfg(256, 8, 7, 4)  # 256 % 7 != 0
    assert L.coli_moe_route(ctypes.byref(bad), _fake(16), None, 1, _fake(16), _fake(16), None) \
        == B.COLI_ERR_INVALID_ARG
    bad = B.router_cfg(256, 40, 8, 8)  # k > 32
    assert L.coli_moe_route(ctypes.byref(bad), _fake(16), None, 1, _fake(16), _fake(16), None) \
        == B.COLI_ERR_INVALID_ARG
    bad = B.router_cfg(16, 5, 4, 1)  # k > topk_group * E / n_group
    assert L.coli_moe_route(ctypes.byref(bad), _fake(16), None, 1, _fake(16), _fake(16), None) \
        == B.COLI_ERR_INVALID_ARG
    assert L.coli_moe_dispatch(_fake(16), 4, 0, 16, *[_fake(16)] * 5, None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_debug_qgemv_blocks(4, _fake(16), 4, 96, _fake(16), 1, _fake(16), None) \
        == B.COLI_ERR_INVALID_ARG


def test_forward_argument_checks():
    L = B.lib()
    good = _layer_struct()
    ws = L.coli_moe_workspace_bytes(ctypes.byref(good), 1)
    assert ws > 0
    x, y = _fake(0x100000), _fake(0x200000)
    # workspace missing / too small / misaligned
    assert L.coli_moe_forward(ctypes.byref(good), x, 1, None, y, None, None, None, None, 0, None) \
        == B.COLI_ERR_WORKSPACE
    assert L.coli_moe_forward(ctypes.byref(good), x, 1, None, y, None, None, None,
                              _fake(0x300000), ws - 1, None) == B.COLI_ERR_WORKSPACE
    assert L.coli_moe_forward(ctypes.byref(good), x, 1, None, y, None, None, None,
                              _fake(0x300010), ws, None) == B.COLI_ERR_WORKSPACE
    # bad shapes / qtype / pointers
    for kw in (dict(H=6000), dict(I=100), dict(q=3), dict(E=1025, G=1, TG=1), dict(H=16384)):
        s = _layer_struct(**kw)
        assert L.coli_moe_workspace_bytes(ctypes.byref(s), 1) == 0
        assert L.coli_moe_forward(ctypes.byref(s), x, 1, None, y, None, None, None,
                                  _fake(0x300000), ws, None) == B.COLI_ERR_INVALID_ARG
    s = _layer_struct()
    s.w_down = None
    assert L.coli_moe_forward(ctypes.byref(s), x, 1, None, y, None, None, None,
                              _fake(0x300000), ws, None) == B.COLI_ERR_INVALID_ARG
    s = _layer_struct()
    s.w_up = _fake(0x10008)  # not 16-byte aligned
    assert L.coli_moe_forward(ctypes.byref(s), x, 1, None, y, None, None, None,
                              _fake(0x300000), ws, None) == B.COLI_ERR_INVALID_ARG
    s = _layer_struct()
    s.gate_w = None  # no gate and no logits
    assert L.coli_moe_forward(ctypes.byref(s), x, 1, None, y, None, None, None,
                              _fake(0x300000), ws, None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_moe_forward(ctypes.byref(good), x, -1, None, y, None, None, None,
                              _fake(0x300000), ws, None) == B.COLI_ERR_INVALID_ARG


def test_counter_header_size_matches_c_header():
    import pathlib
    import re
    h = (pathlib.Path(__file__).resolve().parents[1] / "include" / "coli_moe.h").read_text()
    m = re.search(r"#define COLI_WORKSPACE_COUNTER_BYTES (\d+)", h)
    assert m and int(m.group(1)) == B.WORKSPACE_COUNTER_BYTES
    for name, val in (("COLI_WORKSPACE_STATUS_OFFSET", B.WORKSPACE_STATUS_OFFSET),
                      ("COLI_WORKSPACE_SPIN_LIMIT_OFFSET", B.WORKSPACE_SPIN_LIMIT_OFFSET)):
        m = re.search(rf"#define {name} (\d+)", h)
        assert m and int(m.group(1)) == val, name
        assert val % 256 == 0 and val < B.WORKSPACE_COUNTER_BYTES  # own 256-byte line
    for name, val in (("COLI_WAIT_SCORES", B.WAIT_SCORES), ("COLI_WAIT_SLOTS", B.WAIT_SLOTS)):
        m = re.search(rf"#define {name} (\d+)u", h)
        assert m and int(m.group(1)) == val, name
    s = _layer_struct()
    assert B.lib().coli_moe_workspace_bytes(ctypes.byref(s), 1) > B.WORKSPACE_COUNTER_BYTES


def test_workspace_status_rejects_bad_arguments():
    L = B.lib()
    assert L.coli_moe_workspace_status(None, _fake(16), 0, None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_moe_workspace_status(_fake(0x300010), _fake(16), 0, None) \
        == B.COLI_ERR_INVALID_ARG  # not 256-byte aligned
    assert L.coli_moe_workspace_status(_fake(0x300000), None, 1, None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_moe_workspace_status(_fake(0x300000), _fake(0x10002), 1, None) \
        == B.COLI_ERR_INVALID_ARG


def test_workspace_grows_with_tokens():
    L = B.lib()
    s = _layer_struct()
    sizes = [L.coli_moe_workspace_bytes(ctypes.byref(s), t) for t in (1, 2, 3, 64, 512)]
    assert all(b > a for a, b in zip(sizes, sizes[1:]))
    assert all(v % 256 == 0 for v in sizes)
    # the union buffer of per-(token, slot) outputs dominates at 512 tokens
    assert sizes[-1] >= 512 * 9 * 6144 * 4
    assert L.coli_moe_workspace_bytes(ctypes.byref(s), -1) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_no_device_reports_device_error():
    L = B.lib()
    good = _layer_struct()
    ws = L.coli_moe_workspace_bytes(ctypes.byref(good), 1)
    assert L.coli_moe_forward(ctypes.byref(good), _fake(0x100000), 1, None, _fake(0x200000),
                              None, None, None, _fake(0x300000), ws, None) == B.COLI_ERR_DEVICE
    assert L.coli_quant_pack(4, _fake(16), 4, 32, _fake(16), _fake(16), None) == B.COLI_ERR_DEVICE
    assert L.coli_quant_pack_fp8(4, _fake(16), _fake(16), 4, 32, _fake(16), _fake(16), None) \
        == B.COLI_ERR_DEVICE
    assert L.coli_gemv_f32act(4, _fake(16), _fake(16), 4, 64, _fake(16), _fake(16), None) \
        == B.COLI_ERR_DEVICE
    cfg = B.router_cfg(16, 2)
    assert L.coli_moe_route(ctypes.byref(cfg), _fake(16), None, 1, _fake(16), _fake(16), None) \
        == B.COLI_ERR_DEVICE


def _cache_struct(E=256, S=32, state=0x400000, host=0x800000):
    h = [_fake(host + 0x100000 * i) for i in range(6)]
    return B.ExpertCacheC(E, S, 0, 0, *h, _fake(state))


def test_expert_cache_layout():
    L = B.lib()
    lo = B.CacheLayoutC()
    assert L.coli_expert_cache_layout_of(256, 32, ctypes.byref(lo)) == B.COLI_OK
    offs = [lo.ctl, lo.slot_of, lo.expert_of, lo.last_use, lo.pinned, lo.use_count, lo.copy_list]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs) and lo.total % 256 == 0
    assert lo.slot_of - lo.ctl >= 64 * 4
    assert lo.expert_of - lo.slot_of >= 256 * 4 and lo.total - lo.copy_list >= 32 * 8
    for E, S in ((0, 1), (16, 0), (16, 17), (1025, 8), (-1, -1)):
        assert L.coli_expert_cache_layout_of(E, S, ctypes.byref(lo)) == B.COLI_ERR_INVALID_ARG
    assert L.coli_expert_cache_layout_of(16, 8, None) == B.COLI_ERR_INVALID_ARG


def test_expert_cache_calls_reject_bad_arguments_before_device():
    L = B.lib()
    c = _cache_struct()
    good = _layer_struct()
    ws = L.coli_moe_workspace_bytes(ctypes.byref(good), 1)
    x, y, wsp = _fake(0x100000), _fake(0x200000), _fake(0x300000)
    assert L.coli_expert_cache_init(None, None) == B.COLI_ERR_INVALID_ARG
    bad = _cache_struct(state=0x400010)  # state not 256-byte aligned
    assert L.coli_expert_cache_init(ctypes.byref(bad), None) == B.COLI_ERR_INVALID_ARG
    bad = _cache_struct(S=300)  # more slots than experts
    assert L.coli_expert_cache_init(ctypes.byref(bad), None) == B.COLI_ERR_INVALID_ARG
    # host tier outside any coli_host_alloc allocation
    assert L.coli_moe_forward_cached(ctypes.byref(good), ctypes.byref(c), x, 1, None, y, None,
                                     None, None, wsp, ws, None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_expert_cache_repin(ctypes.byref(c), ctypes.byref(good), 2, None) \
        == B.COLI_ERR_INVALID_ARG
    # expert count differing from the layer's router
    c16 = _cache_struct(E=16, S=8)
    assert L.coli_moe_forward_cached(ctypes.byref(good), ctypes.byref(c16), x, 1, None, y, None,
                                     None, None, wsp, ws, None) == B.COLI_ERR_INVALID_ARG
    assert L.coli_host_free(None) == B.COLI_OK
    assert L.coli_host_free(_fake(0x12345000)) == B.COLI_ERR_INVALID_ARG
    p = ctypes.c_void_p()
    assert L.coli_host_alloc(0, ctypes.byref(p)) == B.COLI_ERR_INVALID_ARG
    assert L.coli_host_alloc(64, None) == B.COLI_ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_host_alloc_without_device_reports_device_error():
    p = ctypes.c_void_p(1)
    assert B.lib().coli_host_alloc(4096, ctypes.byref(p)) == B.COLI_ERR_DEVICE
    assert not p.value
