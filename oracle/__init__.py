"""The CPU oracle for colibrì's routed-expert MoE layer -- TEST INFRASTRUCTURE.

Only the test suite, the package entry module's ``smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It wraps the plain
C oracle in ``coli_oracle.c`` (numpy in, numpy out) and shares no code with
the GPU library.  Each function names the definition it follows; the
definitions and their citations are in ``coli_oracle.c``.

Parity unpinned: the weight-quantisation rule, the Q8_0 scale type, the
group score and top-p renormalisation are this oracle's readings of the
pages (stated in ``coli_oracle.c``), pinned against mathematics, not against
colibrì's own numbers, which the pages do not print.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coli_oracle.c")
_HDR = os.path.join(_HERE, "coli_oracle.h")
LIB_PATH = os.path.join(_HERE, "libcoli_oracle.so")

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``libcoli_oracle.so``."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    return any(os.path.getmtime(p) > t for p in (_SRC, _HDR))


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if _stale():
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


class RouterCfg(ctypes.Structure):
    _fields_ = [("n_experts", _I32), ("top_k", _I32), ("n_group", _I32),
                ("topk_group", _I32), ("norm_topk_prob", _I32),
                ("routed_scaling_factor", ctypes.c_float),
                ("top_p", ctypes.c_float), ("top_p_renorm", _I32)]


class _Layer(ctypes.Structure):
    _fields_ = [("hidden", _I32), ("inter", _I32), ("bits", _I32),
                ("router", RouterCfg),
                ("gate_w", _P), ("gate_bias", _P),
                ("w_gate", _P), ("s_gate", _P),
                ("w_up", _P), ("s_up", _P),
                ("w_down", _P), ("s_down", _P),
                ("sh_gate", _P), ("sh_up", _P), ("sh_down", _P),
                ("sh_s_gate", _P), ("sh_s_up", _P), ("sh_s_down", _P)]


def _declare(L: ctypes.CDLL) -> None:
    sig = {
        "orc_qmax": [ctypes.c_int],
        "orc_quant_rows": [ctypes.c_int, _P, _I64, _I64, _P, _P],
        "orc_pack": [ctypes.c_int, _P, _I64, _I64, _P],
        "orc_unpack": [ctypes.c_int, _P, _I64, _I64, _P],
        "orc_quant_pack": [ctypes.c_int, _P, _I64, _I64, _P, _P],
        "orc_q8_0": [_P, _I64, _I64, _P, _P],
        "orc_qdot": [ctypes.c_int, _P, _P, _I64, _I64, _P, _P, _I64, _P, _P],
        "orc_logits": [_P, _P, _I64, _I64, _I64, _P],
        "orc_route": [ctypes.POINTER(RouterCfg), _P, _P, _I64, _P, _P, _P],
        "orc_expert_ffn": [ctypes.c_int, _I64, _I64, _P, _P, _P, _P, _P, _P,
                           _P, _I64, _P, _P],
        "orc_moe_forward": [ctypes.POINTER(_Layer), _P, _I64, _P, _P, _P, _P, _P],
        "orc_union_tables": [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P],
        "orc_num_threads": [],
        "orc_set_num_threads": [ctypes.c_int],
        "orc_dequant_fp8_block": [_P, _P, _I64, _I64, _P],
        "orc_qdot_f32act": [ctypes.c_int, _P, _P, _I64, _I64, _P, _I64, _P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.orc_set_num_threads.restype = None
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_value.restype = ctypes.c_float


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    """A C-contiguous array of the given dtype (no copy when already so)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (rc={rc})")


def qmax(bits: int) -> int:
    return lib().orc_qmax(bits)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Thread count of later oracle calls; results do not depend on it."""
    lib().orc_set_num_threads(int(n))


def quant_rows(bits: int, w: np.ndarray):
    """O1: fp32 [R, C] -> (int8 codes [R, C], fp32 scales [R])."""
    w = _c(w, np.float32)
    R, C = w.shape
    codes = np.empty((R, C), np.int8)
    s = np.empty(R, np.float32)
    _check(lib().orc_quant_rows(bits, _ptr(w), R, C, _ptr(codes), _ptr(s)), "quant_rows")
    return codes, s


def pack(bits: int, codes: np.ndarray) -> np.ndarray:
    """O2: int8 codes [R, C] -> packed bytes [R, C*bits/8]."""
    codes = _c(codes, np.int8)
    R, C = codes.shape
    out = np.empty((R, C * bits // 8), np.uint8)
    _check(lib().orc_pack(bits, _ptr(codes), R, C, _ptr(out)), "pack")
    return out


def unpack(bits: int, packed: np.ndarray, cols: int) -> np.ndarray:
    """O2 inverse: packed bytes [R, cols*bits/8] -> int8 codes [R, cols]."""
    packed = _c(packed, np.uint8)
    R = packed.shape[0]
    out = np.empty((R, cols), np.int8)
    _check(lib().orc_unpack(bits, _ptr(packed), R, cols, _ptr(out)), "unpack")
    return out


def quant_pack(bits: int, w: np.ndarray):
    """O1 then O2: fp32 [R, C] -> (packed [R, C*bits/8], scales [R])."""
    w = _c(w, np.float32)
    R, C = w.shape
    out = np.empty((R, C * bits // 8), np.uint8)
    s = np.empty(R, np.float32)
    _check(lib().orc_quant_pack(bits, _ptr(w), R, C, _ptr(out), _ptr(s)), "quant_pack")
    return out, s


def q8_0(x: np.ndarray):
    """O3: fp32 [T, n] -> (int8 [T, n], fp32 block scales [T, n/32])."""
    x = _c(x, np.float32)
    T, n = x.shape
    q = np.empty((T, n), np.int8)
    d = np.empty((T, n // 32), np.float32)
    _check(lib().orc_q8_0(_ptr(x), T, n, _ptr(q), _ptr(d)), "q8_0")
    return q, d


def qdot(bits: int, w_packed: np.ndarray, w_scale: np.ndarray, cols: int,
         xq: np.ndarray, xd: np.ndarray, want_acc: bool = True):
    """O4: returns (acc int32 [T, R, cols/32] or None, y fp32 [T, R])."""
    w_packed = _c(w_packed, np.uint8)
    w_scale = _c(w_scale, np.float32)
    xq = _c(xq, np.int8)
    xd = _c(xd, np.float32)
    R = w_packed.shape[0]
    T = xq.shape[0]
    acc = np.empty((T, R, cols // 32), np.int32) if want_acc else None
    y = np.empty((T, R), np.float32)
    _check(lib().orc_qdot(bits, _ptr(w_packed), _ptr(w_scale), R, cols, _ptr(xq),
                          _ptr(xd), T, _ptr(acc), _ptr(y)), "qdot")
    return acc, y


def qdot_f32act(bits: int, w_packed: np.ndarray, w_scale: np.ndarray, cols: int,
                x: np.ndarray) -> np.ndarray:
    """O12: packed codes [R, cols*bits/8], row scales [R], fp32 x [T, cols]
    -> fp32 y [T, R]."""
    w_packed = _c(w_packed, np.uint8)
    w_scale = _c(w_scale, np.float32)
    x = _c(x, np.float32)
    R, T = w_packed.shape[0], x.shape[0]
    y = np.empty((T, R), np.float32)
    _check(lib().orc_qdot_f32act(bits, _ptr(w_packed), _ptr(w_scale), R, cols, _ptr(x), T,
                                 _ptr(y)), "qdot_f32act")
    return y


def logits(x: np.ndarray, gate_w: np.ndarray) -> np.ndarray:
    """O5: fp32 x [T, H], gate [E, H] -> fp32 [T, E]."""
    x = _c(x, np.float32)
    gate_w = _c(gate_w, np.float32)
    T, H = x.shape
    E = gate_w.shape[0]
    out = np.empty((T, E), np.float32)
    _check(lib().orc_logits(_ptr(x), _ptr(gate_w), T, E, H, _ptr(out)), "logits")
    return out


def e4m3_value(code: int) -> float:
    """O11: the value of one OCP FP8 E4M3 (e4m3fn) code."""
    return float(lib().orc_e4m3_value(code & 0xFF))


def dequant_fp8_block(w8: np.ndarray, block_scale: np.ndarray) -> np.ndarray:
    """O11: uint8 codes [rows, cols] and fp32 scales [ceil(rows/128),
    ceil(cols/128)] -> fp32 [rows, cols]."""
    w8 = _c(w8, np.uint8)
    rows, cols = w8.shape
    bs = _c(block_scale, np.float32)
    if bs.shape != ((rows + 127) // 128, (cols + 127) // 128):
        raise ValueError(f"block scales {bs.shape} do not tile {w8.shape} in 128x128 blocks")
    out = np.empty((rows, cols), np.float32)
    _check(lib().orc_dequant_fp8_block(_ptr(w8), _ptr(bs), rows, cols, _ptr(out)), "dequant_fp8_block")
    return out


def requant_fp8_block(bits: int, w8: np.ndarray, block_scale: np.ndarray):
    """O11 then O1 + O2: the converter's FP8 -> container step; returns
    (packed codes, row scales)."""
    return quant_pack(bits, dequant_fp8_block(w8, block_scale))


def make_cfg(n_experts, top_k, n_group=1, topk_group=1, norm_topk_prob=1,
             routed_scaling_factor=2.5, top_p=0.0, top_p_renorm=1) -> RouterCfg:
    return RouterCfg(n_experts, top_k, n_group, topk_group, norm_topk_prob,
                     routed_scaling_factor, top_p, top_p_renorm)


def route(cfg: RouterCfg, logits_: np.ndarray, bias: np.ndarray | None = None,
          want_sigma: bool = False):
    """O6/O7: returns (idx int32 [T, k], w fp32 [T, k][, sigma fp32 [T, E]])."""
    logits_ = _c(logits_, np.float32)
    T = logits_.shape[0]
    k = cfg.top_k
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    sig = np.empty((T, cfg.n_experts), np.float32) if want_sigma else None
    b = None if bias is None else _c(bias, np.float32)
    _check(lib().orc_route(ctypes.byref(cfg), _ptr(logits_), _ptr(b), T, _ptr(idx),
                           _ptr(w), _ptr(sig)), "route")
    return (idx, w, sig) if want_sigma else (idx, w)


@dataclass
class Expert:
    """One expert's quantised container: packed codes and per-row scales."""
    w_gate: np.ndarray
    s_gate: np.ndarray
    w_up: np.ndarray
    s_up: np.ndarray
    w_down: np.ndarray
    s_down: np.ndarray

    @staticmethod
    def from_float(bits: int, gate: np.ndarray, up: np.ndarray, down: np.ndarray) -> "Expert":
        """Quantise fp32 gate [I, H], up [I, H], down [H, I] with O1/O2."""
        wg, sg = quant_pack(bits, gate)
        wu, su = quant_pack(bits, up)
        wd, sd = quant_pack(bits, down)
        return Expert(wg, sg, wu, su, wd, sd)


def expert_ffn(bits: int, H: int, I: int, ex: Expert, x: np.ndarray,
               want_h: bool = False):
    """O8: x fp32 [T, H] -> o fp32 [T, H] (and h fp32 [T, I])."""
    x = _c(x, np.float32)
    T = x.shape[0]
    o = np.empty((T, H), np.float32)
    h = np.empty((T, I), np.float32) if want_h else None
    parts = [_c(a, t) for a, t in ((ex.w_gate, np.uint8), (ex.s_gate, np.float32),
                                   (ex.w_up, np.uint8), (ex.s_up, np.float32),
                                   (ex.w_down, np.uint8), (ex.s_down, np.float32))]
    _check(lib().orc_expert_ffn(bits, H, I, *[_ptr(p) for p in parts], _ptr(x), T,
                                _ptr(o), _ptr(h)), "expert_ffn")
    return (o, h) if want_h else o


@dataclass
class Layer:
    """A layer for the oracle.  ``experts[e]`` may be None for an expert a
    call never selects (the oracle then refuses a token that selects it)."""
    hidden: int
    inter: int
    bits: int
    cfg: RouterCfg
    experts: list
    shared: Expert
    gate_w: np.ndarray | None = None
    gate_bias: np.ndarray | None = None
    _keep: list = field(default_factory=list, repr=False)


def moe_forward(layer: Layer, x: np.ndarray, logits_in: np.ndarray | None = None):
    """O9: returns (y fp32 [T, H], idx int32 [T, k], w fp32 [T, k], logits fp32 [T, E])."""
    x = _c(x, np.float32)
    T = x.shape[0]
    E, k, H = layer.cfg.n_experts, layer.cfg.top_k, layer.hidden
    keep = []

    def hold(a, dt):
        if a is None:
            return None
        a = _c(a, dt)
        keep.append(a)
        return a.ctypes.data

    def table(attr, dt):
        arr = (ctypes.c_void_p * E)()
        for e, ex in enumerate(layer.experts):
            arr[e] = None if ex is None else hold(getattr(ex, attr), dt)
        keep.append(arr)
        return ctypes.cast(arr, ctypes.c_void_p).value

    sh = layer.shared
    L = _Layer(H, layer.inter, layer.bits, layer.cfg,
               hold(layer.gate_w, np.float32), hold(layer.gate_bias, np.float32),
               table("w_gate", np.uint8), table("s_gate", np.float32),
               table("w_up", np.uint8), table("s_up", np.float32),
               table("w_down", np.uint8), table("s_down", np.float32),
               hold(sh.w_gate, np.uint8), hold(sh.w_up, np.uint8), hold(sh.w_down, np.uint8),
               hold(sh.s_gate, np.float32), hold(sh.s_up, np.float32),
               hold(sh.s_down, np.float32))
    lin = None if logits_in is None else _c(logits_in, np.float32)
    y = np.empty((T, H), np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lg = np.empty((T, E), np.float32)
    _check(lib().orc_moe_forward(ctypes.byref(L), _ptr(x), T, _ptr(lin), _ptr(y),
                                 _ptr(idx), _ptr(w), _ptr(lg)), "moe_forward")
    return y, idx, w, lg


def union_tables(idx: np.ndarray, E: int):
    """O10: returns (counts [E], offs [E+1], perm [n], uniq [U])."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offs = np.empty(E + 1, np.int32)
    perm = np.empty(max(T * k, 1), np.int32)
    uniq = np.empty(E, np.int32)
    n = np.zeros(1, np.int32)
    _check(lib().orc_union_tables(_ptr(idx), T, k, E, _ptr(counts), _ptr(offs),
                                  _ptr(perm), _ptr(uniq), _ptr(n)), "union_tables")
    return counts, offs, perm[: int(offs[-1])], uniq[: int(n[0])]
