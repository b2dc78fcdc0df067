"""Thin Python binding over ``libcoli_moe.so`` (include/coli_moe.h).

Argument marshalling only: every function checks tensor dtypes, devices and
shapes, passes raw device pointers and the current HIP stream to the C ABI of
the same name, and raises ``ColiError`` on a non-OK status.  All computation
happens in the library's gfx950 kernels; there is no fallback.  PyTorch is
used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcoli_moe.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "coli_moe.h")

COLI_OK, COLI_ERR_INVALID_ARG, COLI_ERR_UNSUPPORTED, COLI_ERR_WORKSPACE, COLI_ERR_DEVICE = range(5)
COLI_Q8, COLI_Q4, COLI_Q2 = 8, 4, 2


class ColiError(RuntimeError):
    def __init__(self, name: str, status: int, msg: str):
        super().__init__(f"{name}: status {status} ({msg})")
        self.status = status


class RouterCfg(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("expert_top_p", ctypes.c_float), ("top_p_renorm", ctypes.c_int32)]


_P = ctypes.c_void_p


class MoeLayerC(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("qtype", ctypes.c_int32),
                ("router", RouterCfg),
                ("gate_w", _P), ("gate_bias", _P),
                ("w_gate", _P), ("w_up", _P), ("w_down", _P),
                ("s_gate", _P), ("s_up", _P), ("s_down", _P),
                ("sh_gate", _P), ("sh_up", _P), ("sh_down", _P),
                ("sh_s_gate", _P), ("sh_s_up", _P), ("sh_s_down", _P),
                ("mfma_min_tokens", ctypes.c_int32), ("gate_offset", _P)]


class ExpertCacheC(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("n_pinned", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("host_w_gate", _P), ("host_w_up", _P), ("host_w_down", _P),
                ("host_s_gate", _P), ("host_s_up", _P), ("host_s_down", _P),
                ("state", _P)]


class SpecGuardC(ctypes.Structure):
    _fields_ = [("max_draft", ctypes.c_int32), ("probe_every", ctypes.c_int32),
                ("ema", ctypes.c_float), ("margin", ctypes.c_float),
                ("cost_draft", ctypes.c_double), ("cost_plain", ctypes.c_double),
                ("sum_cost", ctypes.c_double * 2), ("sum_tokens", ctypes.c_double * 2),
                ("next_draft", ctypes.c_int32), ("since_probe", ctypes.c_int32),
                ("steps", ctypes.c_int64), ("draft_steps", ctypes.c_int64),
                ("tokens", ctypes.c_int64)]


class CacheLayoutC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("ctl", "slot_of", "expert_of", "last_use", "pinned", "use_count", "copy_list",
                 "total")]


# The timeline build (decode kernel with timeline records compiled in), for
# coli_debug_decode_trace only.
TRACE_LIB_PATH = os.path.join(_PKG, "libcoli_moe_trace.so")

_lib = None
_trace_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def trace_lib() -> ctypes.CDLL:
    """Load the timeline build of the library."""
    global _trace_lib
    if _trace_lib is None:
        _trace_lib = _load(TRACE_LIB_PATH)
    return _trace_lib


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(python -m quantized_moe_coli_amd.build)")
    L = ctypes.CDLL(path)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "coli_abi_version": ([], ctypes.c_int),
        "coli_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "coli_quant_pack": ([i32, _P, i64, i64, _P, _P, _P], ctypes.c_int),
        "coli_quant_pack_fp8": ([i32, _P, _P, i64, i64, _P, _P, _P], ctypes.c_int),
        "coli_gemv_f32act": ([i32, _P, _P, i64, i64, _P, _P, _P], ctypes.c_int),
        "coli_quant_act_q8_0": ([_P, i32, i32, _P, _P, _P], ctypes.c_int),
        "coli_moe_logits": ([_P, _P, i32, i32, i32, _P, _P], ctypes.c_int),
        "coli_moe_route": ([ctypes.POINTER(RouterCfg), _P, _P, i32, _P, _P, _P], ctypes.c_int),
        "coli_moe_dispatch": ([_P, i32, i32, i32, _P, _P, _P, _P, _P, _P], ctypes.c_int),
        "coli_moe_workspace_bytes": ([ctypes.POINTER(MoeLayerC), i32], sz),
        "coli_moe_forward": ([ctypes.POINTER(MoeLayerC), _P, i32, _P, _P, _P, _P, _P, _P, sz,
                              _P], ctypes.c_int),
        "coli_moe_forward_profiled": ([ctypes.POINTER(MoeLayerC), _P, i32, _P, _P, _P, _P, _P,
                                       _P, sz, _P, ctypes.POINTER(_P), i32], ctypes.c_int),
        "coli_debug_qgemv_blocks": ([i32, _P, i32, i32, _P, i32, _P, _P], ctypes.c_int),
        "coli_moe_workspace_status": ([_P, _P, i32, _P], ctypes.c_int),
        "coli_debug_decode_trace": ([ctypes.POINTER(MoeLayerC), _P, _P, _P, sz, _P, i32,
                                     ctypes.POINTER(i32), _P], ctypes.c_int),
        "coli_debug_stream_read": ([_P, sz, _P, ctypes.POINTER(i32), _P], ctypes.c_int),
        "coli_moe_forward_noalloc": ([ctypes.POINTER(MoeLayerC), _P, i32, _P, _P, _P, _P, _P,
                                      _P, _P], ctypes.c_int),
        "coli_host_alloc": ([sz, ctypes.POINTER(_P)], ctypes.c_int),
        "coli_host_free": ([_P], ctypes.c_int),
        "coli_expert_cache_layout_of": ([i32, i32, ctypes.POINTER(CacheLayoutC)], ctypes.c_int),
        "coli_expert_cache_init": ([ctypes.POINTER(ExpertCacheC), _P], ctypes.c_int),
        "coli_expert_cache_repin": ([ctypes.POINTER(ExpertCacheC), ctypes.POINTER(MoeLayerC), i32,
                                     _P], ctypes.c_int),
        "coli_moe_forward_cached": ([ctypes.POINTER(MoeLayerC), ctypes.POINTER(ExpertCacheC), _P,
                                     i32, _P, _P, _P, _P, _P, _P, sz, _P], ctypes.c_int),
        "coli_spec_guard_init": ([ctypes.POINTER(SpecGuardC), i32, i32, ctypes.c_float,
                                  ctypes.c_float], ctypes.c_int),
        "coli_spec_guard_step": ([ctypes.POINTER(SpecGuardC), i32, i32, ctypes.c_double], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def declared_symbols() -> list[str]:
    """Function names declared in include/coli_moe.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(coli_[a-z0-9_]+)\s*\(", text)))


def _check(name: str, status: int) -> None:
    if status != COLI_OK:
        raise ColiError(name, status, lib().coli_status_str(status).decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t: torch.Tensor | None, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def router_cfg(n_experts, top_k, n_group=1, topk_group=1, norm_topk_prob=1,
               routed_scaling_factor=2.5, expert_top_p=0.0, top_p_renorm=1) -> RouterCfg:
    return RouterCfg(n_experts, top_k, n_group, topk_group, norm_topk_prob,
                     routed_scaling_factor, expert_top_p, top_p_renorm)


def coli_abi_version() -> int:
    return lib().coli_abi_version()


def coli_quant_pack(qtype: int, w: torch.Tensor, q_out: torch.Tensor, scale_out: torch.Tensor,
                    stream=None) -> None:
    """w fp32 [rows, cols] -> q_out uint8 [rows, cols*qtype/8], scale_out fp32 [rows]."""
    rows, cols = w.shape
    if q_out.numel() != rows * cols * qtype // 8 or scale_out.numel() != rows:
        raise ValueError("output sizes do not match")
    _check("coli_quant_pack", lib().coli_quant_pack(
        qtype, _ptr(w, torch.float32, "w"), rows, cols, _ptr(q_out, torch.uint8, "q_out"),
        _ptr(scale_out, torch.float32, "scale_out"), _stream(stream)))


def coli_quant_pack_fp8(qtype: int, w8: torch.Tensor, block_scale: torch.Tensor,
                        q_out: torch.Tensor, scale_out: torch.Tensor, stream=None) -> None:
    """w8 uint8 FP8 E4M3 codes [rows, cols], block_scale fp32 [ceil(rows/128),
    ceil(cols/128)] -> q_out uint8 [rows, cols*qtype/8], scale_out fp32 [rows]."""
    rows, cols = w8.shape
    if tuple(block_scale.shape) != ((rows + 127) // 128, (cols + 127) // 128):
        raise ValueError("block scales do not tile the matrix in 128x128 blocks")
    if q_out.numel() != rows * cols * qtype // 8 or scale_out.numel() != rows:
        raise ValueError("output sizes do not match")
    _check("coli_quant_pack_fp8", lib().coli_quant_pack_fp8(
        qtype, _ptr(w8, torch.uint8, "w8"), _ptr(block_scale, torch.float32, "block_scale"),
        rows, cols, _ptr(q_out, torch.uint8, "q_out"),
        _ptr(scale_out, torch.float32, "scale_out"), _stream(stream)))


def coli_gemv_f32act(qtype: int, w: torch.Tensor, scale: torch.Tensor, x: torch.Tensor,
                     y: torch.Tensor, stream=None) -> None:
    """w uint8 [rows, cols*qtype/8] packed codes, scale fp32 [rows], x fp32
    [cols] -> y fp32 [rows] = scale * (codes @ x)."""
    rows = w.shape[0]
    cols = x.numel()
    if w.shape[1] * 8 != cols * qtype or scale.numel() != rows or y.numel() != rows:
        raise ValueError("shapes do not match")
    _check("coli_gemv_f32act", lib().coli_gemv_f32act(
        qtype, _ptr(w, torch.uint8, "w"), _ptr(scale, torch.float32, "scale"), rows, cols,
        _ptr(x, torch.float32, "x"), _ptr(y, torch.float32, "y"), _stream(stream)))


def coli_quant_act_q8_0(x: torch.Tensor, q: torch.Tensor, d: torch.Tensor, stream=None) -> None:
    """x fp32 [T, n] -> q int8 [T, n] (natural order), d fp32 [T, n/32]."""
    T, n = x.shape
    if q.numel() != T * n or d.numel() != T * (n // 32):
        raise ValueError("output sizes do not match")
    _check("coli_quant_act_q8_0", lib().coli_quant_act_q8_0(
        _ptr(x, torch.float32, "x"), T, n, _ptr(q, torch.int8, "q"), _ptr(d, torch.float32, "d"),
        _stream(stream)))


def coli_moe_logits(x: torch.Tensor, gate_w: torch.Tensor, logits: torch.Tensor, stream=None) -> None:
    T, H = x.shape
    E = gate_w.shape[0]
    if gate_w.shape[1] != H or logits.numel() != T * E:
        raise ValueError("shape mismatch")
    _check("coli_moe_logits", lib().coli_moe_logits(
        _ptr(x, torch.float32, "x"), _ptr(gate_w, torch.float32, "gate_w"), T, E, H,
        _ptr(logits, torch.float32, "logits"), _stream(stream)))


def coli_moe_route(cfg: RouterCfg, logits: torch.Tensor, bias: torch.Tensor | None,
                   idx: torch.Tensor, w: torch.Tensor, stream=None) -> None:
    T = logits.shape[0]
    if logits.shape[1] != cfg.n_experts or idx.numel() != T * cfg.top_k or w.numel() != T * cfg.top_k:
        raise ValueError("shape mismatch")
    _check("coli_moe_route", lib().coli_moe_route(
        ctypes.byref(cfg), _ptr(logits, torch.float32, "logits"),
        _ptr(bias, torch.float32, "bias"), T, _ptr(idx, torch.int32, "idx"),
        _ptr(w, torch.float32, "w"), _stream(stream)))


def coli_moe_dispatch(idx: torch.Tensor, E: int, counts, offs, perm, uniq, n_uniq,
                      stream=None) -> None:
    T, k = idx.shape
    _check("coli_moe_dispatch", lib().coli_moe_dispatch(
        _ptr(idx, torch.int32, "idx"), T, k, E, _ptr(counts, torch.int32, "counts"),
        _ptr(offs, torch.int32, "offs"), _ptr(perm, torch.int32, "perm"),
        _ptr(uniq, torch.int32, "uniq"), _ptr(n_uniq, torch.int32, "n_uniq"), _stream(stream)))


class MoeLayer:
    """A layer's device tensors plus the C descriptor that points at them.

    Routed tensors are stacked: w_gate/w_up uint8 [E, I, H*b/8], s_gate/s_up
    fp32 [E, I], w_down uint8 [E, H, I*b/8], s_down fp32 [E, H]; the shared
    expert's tensors have no leading E.  The object keeps the tensors alive.
    """

    def __init__(self, hidden, inter, qtype, cfg: RouterCfg, gate_w, gate_bias,
                 w_gate, s_gate, w_up, s_up, w_down, s_down,
                 sh_gate, sh_s_gate, sh_up, sh_s_up, sh_down, sh_s_down, mfma_min_tokens=0,
                 gate_offset=None):
        self.hidden, self.inter, self.qtype, self.cfg = hidden, inter, qtype, cfg
        self.gate_w, self.gate_bias = gate_w, gate_bias
        self.w_gate, self.s_gate, self.w_up, self.s_up = w_gate, s_gate, w_up, s_up
        self.w_down, self.s_down = w_down, s_down
        self.sh_gate, self.sh_s_gate, self.sh_up, self.sh_s_up = sh_gate, sh_s_gate, sh_up, sh_s_up
        self.sh_down, self.sh_s_down = sh_down, sh_s_down
        self.mfma_min_tokens = mfma_min_tokens
        self.gate_offset = gate_offset  # optional fp32 [E] added to computed logits

    def c_struct(self) -> MoeLayerC:
        u8, f32 = torch.uint8, torch.float32
        return MoeLayerC(self.hidden, self.inter, self.qtype, self.cfg,
                         _ptr(self.gate_w, f32, "gate_w"), _ptr(self.gate_bias, f32, "gate_bias"),
                         _ptr(self.w_gate, u8, "w_gate"), _ptr(self.w_up, u8, "w_up"),
                         _ptr(self.w_down, u8, "w_down"),
                         _ptr(self.s_gate, f32, "s_gate"), _ptr(self.s_up, f32, "s_up"),
                         _ptr(self.s_down, f32, "s_down"),
                         _ptr(self.sh_gate, u8, "sh_gate"), _ptr(self.sh_up, u8, "sh_up"),
                         _ptr(self.sh_down, u8, "sh_down"),
                         _ptr(self.sh_s_gate, f32, "sh_s_gate"), _ptr(self.sh_s_up, f32, "sh_s_up"),
                         _ptr(self.sh_s_down, f32, "sh_s_down"), self.mfma_min_tokens,
                         _ptr(self.gate_offset, f32, "gate_offset"))

    @staticmethod
    def empty(hidden, inter, qtype, cfg: RouterCfg, device="cuda", gate=True,
              n_slots: int | None = None) -> "MoeLayer":
        """Uninitialised device storage for a layer (filled by coli_quant_pack).
        With ``n_slots`` the routed arrays hold that many expert-cache slots
        instead of all E experts."""
        E, H, I = cfg.n_experts, hidden, inter
        R = E if n_slots is None else n_slots  # routed entries: experts or slots
        gb, db = H * qtype // 8, I * qtype // 8
        u8, f32 = torch.uint8, torch.float32
        z = lambda *s, dt: torch.empty(*s, dtype=dt, device=device)  # noqa: E731
        return MoeLayer(H, I, qtype, cfg,
                        z(E, H, dt=f32) if gate else None, z(E, dt=f32),
                        z(R, I, gb, dt=u8), z(R, I, dt=f32), z(R, I, gb, dt=u8), z(R, I, dt=f32),
                        z(R, H, db, dt=u8), z(R, H, dt=f32),
                        z(I, gb, dt=u8), z(I, dt=f32), z(I, gb, dt=u8), z(I, dt=f32),
                        z(H, db, dt=u8), z(H, dt=f32))

    def pack_expert(self, e: int, gate: torch.Tensor, up: torch.Tensor, down: torch.Tensor,
                    stream=None) -> None:
        """Quantise fp32 gate [I, H], up [I, H], down [H, I] of routed expert e
        (e == n_experts: the shared expert) into this layer's storage."""
        if e == self.cfg.n_experts:
            dst = ((self.sh_gate, self.sh_s_gate), (self.sh_up, self.sh_s_up),
                   (self.sh_down, self.sh_s_down))
        else:
            dst = ((self.w_gate[e], self.s_gate[e]), (self.w_up[e], self.s_up[e]),
                   (self.w_down[e], self.s_down[e]))
        for src, (q, s) in zip((gate, up, down), dst):
            coli_quant_pack(self.qtype, src, q, s, stream)


def coli_moe_workspace_bytes(layer: MoeLayer, max_tokens: int) -> int:
    c = layer.c_struct()
    return lib().coli_moe_workspace_bytes(ctypes.byref(c), max_tokens)


# Leading workspace bytes holding the decode kernel's counters, and the byte
# offsets of its sticky status word and polling-bound test hook
# (COLI_WORKSPACE_* in include/coli_moe.h), with the status bits.
WORKSPACE_COUNTER_BYTES = 20480
WORKSPACE_STATUS_OFFSET = 10752
WORKSPACE_SPIN_LIMIT_OFFSET = 11008
WAIT_SCORES, WAIT_SLOTS = 1, 2


def workspace(layer: MoeLayer, max_tokens: int, device="cuda") -> torch.Tensor:
    """A zeroed device workspace big enough for ``max_tokens`` (256-byte
    aligned; its counter header must start at zero)."""
    n = coli_moe_workspace_bytes(layer, max_tokens)
    if n == 0:
        raise ValueError("invalid layer descriptor")
    buf = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + n]


def coli_moe_forward(layer: MoeLayer, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor,
                     logits_in=None, idx_out=None, w_out=None, logits_out=None,
                     stream=None, c_layer: MoeLayerC | None = None) -> None:
    """y [T, H] = the layer on x [T, H]; optional routing outputs."""
    T = x.shape[0]
    c = c_layer if c_layer is not None else layer.c_struct()
    _check("coli_moe_forward", lib().coli_moe_forward(
        ctypes.byref(c), _ptr(x, torch.float32, "x"), T,
        _ptr(logits_in, torch.float32, "logits_in"), _ptr(y, torch.float32, "y"),
        _ptr(idx_out, torch.int32, "idx_out"), _ptr(w_out, torch.float32, "w_out"),
        _ptr(logits_out, torch.float32, "logits_out"), ctypes.c_void_p(ws.data_ptr()),
        ws.numel(), _stream(stream)))


# Bytes of the library's static per-GPU scratch behind coli_moe_forward_noalloc
# (COLI_NOALLOC_SCRATCH_BYTES in include/coli_moe.h).
NOALLOC_SCRATCH_BYTES = 32 << 20


def coli_moe_forward_noalloc(layer: MoeLayer, x: torch.Tensor, y: torch.Tensor, logits_in=None,
                             idx_out=None, w_out=None, logits_out=None, wait_status_out=None,
                             stream=None, c_layer: MoeLayerC | None = None) -> None:
    """coli_moe_forward without a workspace argument: the library's static
    per-GPU scratch serves as the workspace (calls on one GPU must not
    overlap); optional ``wait_status_out`` int32 [1] receives the status word."""
    T = x.shape[0]
    c = c_layer if c_layer is not None else layer.c_struct()
    _check("coli_moe_forward_noalloc", lib().coli_moe_forward_noalloc(
        ctypes.byref(c), _ptr(x, torch.float32, "x"), T,
        _ptr(logits_in, torch.float32, "logits_in"), _ptr(y, torch.float32, "y"),
        _ptr(idx_out, torch.int32, "idx_out"), _ptr(w_out, torch.float32, "w_out"),
        _ptr(logits_out, torch.float32, "logits_out"),
        _ptr(wait_status_out, torch.int32, "wait_status_out"), _stream(stream)))


def coli_moe_forward_profiled(layer: MoeLayer, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor,
                              events, logits_in=None, stream=None,
                              c_layer: MoeLayerC | None = None) -> None:
    """coli_moe_forward recording the hipEvent_t handles ``events`` (ints)
    at its stage boundaries."""
    T = x.shape[0]
    c = c_layer if c_layer is not None else layer.c_struct()
    ev = (_P * len(events))(*events)
    _check("coli_moe_forward_profiled", lib().coli_moe_forward_profiled(
        ctypes.byref(c), _ptr(x, torch.float32, "x"), T,
        _ptr(logits_in, torch.float32, "logits_in"), _ptr(y, torch.float32, "y"),
        None, None, None, ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream),
        ev, len(events)))


def coli_moe_workspace_status(ws: torch.Tensor, status_out: torch.Tensor, clear: bool = False,
                              stream=None) -> None:
    """status_out int32 [1] (device) <- the workspace's status word; cleared
    afterwards when ``clear``."""
    if status_out.numel() != 1:
        raise ValueError("status_out must hold one int32")
    _check("coli_moe_workspace_status", lib().coli_moe_workspace_status(
        ctypes.c_void_p(ws.data_ptr()), _ptr(status_out, torch.int32, "status_out"),
        1 if clear else 0, _stream(stream)))


TRACE_RECORDS = 64  # COLI_TRACE_RECORDS in include/coli_moe.h


def coli_debug_decode_trace(layer: MoeLayer, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor,
                            trace: torch.Tensor, stream=None, c_layer: MoeLayerC | None = None) -> int:
    """One-token decode recording its timeline into ``trace`` (int64
    [wgs, TRACE_RECORDS, 2], zeroed by the caller); returns the grid size."""
    c = c_layer if c_layer is not None else layer.c_struct()
    if trace.dim() != 3 or trace.shape[1:] != (TRACE_RECORDS, 2):
        raise ValueError("trace must be [wgs, TRACE_RECORDS, 2]")
    grid = ctypes.c_int32(0)
    _check("coli_debug_decode_trace", trace_lib().coli_debug_decode_trace(
        ctypes.byref(c), _ptr(x, torch.float32, "x"), _ptr(y, torch.float32, "y"),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _ptr(trace, torch.int64, "trace"),
        trace.shape[0], ctypes.byref(grid), _stream(stream)))
    return grid.value


def coli_debug_stream_read(buf: torch.Tensor, out: torch.Tensor, stream=None) -> int:
    """Streaming read of every byte of ``buf``; returns the grid size."""
    grid = ctypes.c_int32(0)
    _check("coli_debug_stream_read", lib().coli_debug_stream_read(
        ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
        _ptr(out, torch.int32, "out"), ctypes.byref(grid), _stream(stream)))
    return grid.value


def coli_debug_qgemv_blocks(qtype: int, Wq: torch.Tensor, cols: int, xq: torch.Tensor,
                            acc_out: torch.Tensor, stream=None) -> None:
    rows = Wq.shape[0]
    T = xq.shape[0]
    _check("coli_debug_qgemv_blocks", lib().coli_debug_qgemv_blocks(
        qtype, _ptr(Wq, torch.uint8, "Wq"), rows, cols, _ptr(xq, torch.int8, "xq"), T,
        _ptr(acc_out, torch.int32, "acc_out"), _stream(stream)))


# ---------------------------------------------------------------------------
# Tiered expert residency: a host tier in pinned host memory, and per-layer
# expert caches of HBM slots over it.
# ---------------------------------------------------------------------------
class HostBuffer:
    """Pinned host memory from coli_host_alloc (valid on host and device);
    freed by close() or when collected.  Views must not outlive it."""

    def __init__(self, nbytes: int):
        p = _P()
        _check("coli_host_alloc", lib().coli_host_alloc(nbytes, ctypes.byref(p)))
        self.ptr, self.nbytes = p.value, nbytes

    def view(self, offset: int, shape, dtype) -> torch.Tensor:
        """A CPU tensor over bytes [offset, offset + numel*itemsize)."""
        import numpy as np
        n = 1
        for d in shape:
            n *= d
        nb = n * torch.empty((), dtype=dtype).element_size()
        if offset < 0 or offset + nb > self.nbytes:
            raise ValueError("view outside the buffer")
        arr = np.ctypeslib.as_array((ctypes.c_uint8 * nb).from_address(self.ptr + offset))
        return torch.from_numpy(arr).view(dtype).reshape(shape)

    def close(self) -> None:
        if self.ptr:
            _check("coli_host_free", lib().coli_host_free(_P(self.ptr)))
            self.ptr = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class HostTier:
    """Every routed expert of one layer in pinned host memory, stacked over E
    in the layer's layouts: w_gate/w_up uint8 [E, I, H*b/8], s_gate/s_up fp32
    [E, I], w_down uint8 [E, H, I*b/8], s_down fp32 [E, H]."""

    def __init__(self, n_experts: int, hidden: int, inter: int, qtype: int):
        E, H, I, b = n_experts, hidden, inter, qtype
        self.n_experts, self.hidden, self.inter, self.qtype = E, H, I, b
        u8, f32 = torch.uint8, torch.float32
        specs = [("w_gate", (E, I, H * b // 8), u8), ("w_up", (E, I, H * b // 8), u8),
                 ("w_down", (E, H, I * b // 8), u8), ("s_gate", (E, I), f32),
                 ("s_up", (E, I), f32), ("s_down", (E, H), f32)]
        offs, off = [], 0
        for _, shp, dt in specs:
            offs.append(off)
            n = torch.empty((), dtype=dt).element_size()
            for d in shp:
                n *= d
            off = (off + n + 255) // 256 * 256
        self.buf = HostBuffer(off)
        for (name, shp, dt), o in zip(specs, offs):
            setattr(self, name, self.buf.view(o, shp, dt))

    def load_experts(self, layer: "MoeLayer", first: int = 0) -> None:
        """Copy the routed experts of a device layer (stacked over its own
        count n) into host-tier experts first .. first+n-1."""
        n = layer.w_gate.shape[0]
        for name in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
            getattr(self, name)[first:first + n].copy_(getattr(layer, name))

    def close(self) -> None:
        self.buf.close()


class ExpertCache:
    """One layer's expert cache: ``n_slots`` HBM slots (the routed arrays of
    the layer it serves) over a HostTier, with its device state."""

    def __init__(self, tier: HostTier, n_slots: int, device="cuda"):
        E = tier.n_experts
        self.tier, self.n_slots = tier, n_slots
        lo = CacheLayoutC()
        _check("coli_expert_cache_layout_of", lib().coli_expert_cache_layout_of(E, n_slots, ctypes.byref(lo)))
        self.layout = lo
        raw = torch.zeros(lo.total + 256, dtype=torch.uint8, device=device)
        off = (-raw.data_ptr()) % 256
        self._raw = raw
        self.state = raw[off:off + lo.total]
        h = lambda t: _P(t.data_ptr())  # noqa: E731 -- pinned host views
        self.c = ExpertCacheC(E, n_slots, 0, 0, h(tier.w_gate), h(tier.w_up), h(tier.w_down),
                              h(tier.s_gate), h(tier.s_up), h(tier.s_down), _P(self.state.data_ptr()))

    def _words(self, off: int, n: int, dtype=torch.int32) -> torch.Tensor:
        return self.state[off:off + 4 * n].view(dtype)

    @property
    def slot_of(self) -> torch.Tensor:
        return self._words(self.layout.slot_of, self.c.n_experts)

    @property
    def expert_of(self) -> torch.Tensor:
        return self._words(self.layout.expert_of, self.n_slots)

    @property
    def last_use(self) -> torch.Tensor:
        return self._words(self.layout.last_use, self.n_slots)

    @property
    def pinned(self) -> torch.Tensor:
        return self._words(self.layout.pinned, self.n_slots)

    @property
    def use_count(self) -> torch.Tensor:
        return self._words(self.layout.use_count, self.c.n_experts)

    def init(self, stream=None) -> None:
        _check("coli_expert_cache_init", lib().coli_expert_cache_init(ctypes.byref(self.c), _stream(stream)))

    def repin(self, layer: "MoeLayer", n_pin: int, stream=None, c_layer=None) -> None:
        c = c_layer if c_layer is not None else layer.c_struct()
        _check("coli_expert_cache_repin", lib().coli_expert_cache_repin(
            ctypes.byref(self.c), ctypes.byref(c), n_pin, _stream(stream)))

    def stats(self) -> dict:
        """clock, last call's copies, error bits, hits and misses (host ints;
        synchronises the device)."""
        ctl = self.state[self.layout.ctl:self.layout.ctl + 64 * 4].view(torch.int64).cpu()
        w = ctl.view(torch.int32)
        return {"clock": int(w[0]) & 0xFFFFFFFF, "copied": int(w[1]), "error": int(w[2]),
                "hits": int(ctl[2]), "misses": int(ctl[3])}

    def save_usage(self, path: str) -> None:
        """Write the learned usage profile (one count per expert)."""
        with open(path, "w") as f:
            f.write(" ".join(str(int(v)) for v in self.use_count.cpu().tolist()) + "\n")

    def load_usage(self, path: str) -> None:
        """Restore a usage profile written by save_usage (after init)."""
        with open(path) as f:
            vals = [int(v) for v in f.read().split()]
        if len(vals) != self.c.n_experts:
            raise ValueError("usage profile has the wrong expert count")
        self.use_count.copy_(torch.tensor(vals, dtype=torch.int32))


def coli_moe_forward_cached(layer: MoeLayer, cache: ExpertCache, x: torch.Tensor, y: torch.Tensor,
                            ws: torch.Tensor, logits_in=None, idx_out=None, w_out=None,
                            logits_out=None, stream=None, c_layer: MoeLayerC | None = None) -> None:
    """coli_moe_forward with the layer's routed experts read from ``cache``'s
    slots (``layer``'s routed arrays hold the slots)."""
    T = x.shape[0]
    c = c_layer if c_layer is not None else layer.c_struct()
    _check("coli_moe_forward_cached", lib().coli_moe_forward_cached(
        ctypes.byref(c), ctypes.byref(cache.c), _ptr(x, torch.float32, "x"), T,
        _ptr(logits_in, torch.float32, "logits_in"), _ptr(y, torch.float32, "y"),
        _ptr(idx_out, torch.int32, "idx_out"), _ptr(w_out, torch.float32, "w_out"),
        _ptr(logits_out, torch.float32, "logits_out"), ctypes.c_void_p(ws.data_ptr()),
        ws.numel(), _stream(stream)))


class SpecGuard:
    """The adaptive speculation guard (coli_spec_guard_*): report each step,
    get the drafts for the next one."""

    def __init__(self, max_draft: int, probe_every: int = 16, ema: float = 0.25,
                 margin: float = 0.0):
        self.c = SpecGuardC()
        _check("coli_spec_guard_init", lib().coli_spec_guard_init(
            ctypes.byref(self.c), max_draft, probe_every, ema, margin))

    @property
    def next_draft(self) -> int:
        return self.c.next_draft

    def step(self, drafted: int, accepted: int, cost: float) -> int:
        r = lib().coli_spec_guard_step(ctypes.byref(self.c), drafted, accepted, float(cost))
        if r < 0:
            raise ValueError("malformed guard report")
        return r
