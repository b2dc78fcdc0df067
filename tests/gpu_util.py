"""Helpers for the GPU parity tests: build the same layer on both sides (the
GPU library packs fp32 weights on the device with coli_quant_pack; the oracle
packs the same fp32 values on the host with its own code) and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from quantized_moe_coli_amd import binding as B
from quantized_moe_coli_amd import inputs

REL_TOL = 1e-3  # per token: max |dy| / max |y_oracle|


def to_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_cfg(s: inputs.Shape) -> B.RouterCfg:
    return B.router_cfg(s.n_experts, s.top_k, s.n_group, s.topk_group, 1, s.rsf, s.top_p, 1)


def orc_cfg(s: inputs.Shape):
    return oracle.make_cfg(s.n_experts, s.top_k, s.n_group, s.topk_group, 1, s.rsf, s.top_p, 1)


class LayerPair:
    """One layer on both sides.  ``device_gen``: fp32 weights are drawn on
    the GPU (full-size layers) and copied to the host only for the experts
    the oracle needs; otherwise they are drawn on the CPU."""

    def __init__(self, s: inputs.Shape, seed: int = 0, device_gen: bool = False,
                 mfma_min_tokens: int = 0, gate_offset: np.ndarray | None = None):
        self.s, self.seed, self.device_gen = s, seed, device_gen
        self.gate_offset = gate_offset
        gdev = "cuda" if device_gen else "cpu"
        self.gpu = B.MoeLayer.empty(s.hidden, s.inter, s.bits, gpu_cfg(s))
        self.gpu.mfma_min_tokens = mfma_min_tokens
        if gate_offset is not None:
            self.gpu.gate_offset = to_dev(gate_offset.astype(np.float32))
        gw = inputs.gate_weight(s, seed, gdev)
        gb = inputs.gate_bias(s, seed, gdev)
        self.gpu.gate_w.copy_(gw)
        self.gpu.gate_bias.copy_(gb)
        self.gate_w = gw.cpu().numpy()
        self.gate_bias = gb.cpu().numpy()
        self._orc_experts: dict[int, oracle.Expert] = {}
        for e in range(s.n_experts + 1):
            g, u, d = inputs.expert_weights(s, seed, e, gdev)
            self.gpu.pack_expert(e, g.cuda(), u.cuda(), d.cuda())
            if not device_gen:
                self._orc_experts[e] = oracle.Expert.from_float(
                    s.bits, g.numpy(), u.numpy(), d.numpy())
        torch.cuda.synchronize()

    def orc_expert(self, e: int) -> oracle.Expert:
        if e not in self._orc_experts:
            g, u, d = (t.cpu().numpy() for t in
                       inputs.expert_weights(self.s, self.seed, e, "cuda" if self.device_gen else "cpu"))
            self._orc_experts[e] = oracle.Expert.from_float(self.s.bits, g, u, d)
        return self._orc_experts[e]

    def orc_layer(self, needed=None) -> oracle.Layer:
        E = self.s.n_experts
        need = range(E) if needed is None else needed
        experts = [None] * E
        for e in need:
            if e >= 0:
                experts[e] = self.orc_expert(int(e))
        return oracle.Layer(self.s.hidden, self.s.inter, self.s.bits, orc_cfg(self.s), experts,
                            self.orc_expert(E), self.gate_w, self.gate_bias)

    def oracle_forward(self, x: np.ndarray, logits_in: np.ndarray | None = None):
        """The oracle on x, supplying only the experts its own routing picks.
        With per-expert logit offsets, the oracle's logits from the gate plus
        the offsets (one binary32 addition) are handed to it as supplied."""
        if logits_in is None and self.gate_offset is not None:
            logits_in = (oracle.logits(x, self.gate_w) +
                         self.gate_offset.astype(np.float32)[None, :]).astype(np.float32)
        lg = oracle.logits(x, self.gate_w) if logits_in is None else logits_in
        idx, _ = oracle.route(orc_cfg(self.s), lg, self.gate_bias)
        return oracle.moe_forward(self.orc_layer(set(idx.ravel().tolist())), x, logits_in)

    def gpu_forward(self, x: torch.Tensor, logits_in: torch.Tensor | None = None, ws=None):
        T = x.shape[0]
        s = self.s
        y = torch.empty(T, s.hidden, device="cuda")
        idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, s.top_k, device="cuda")
        lg = torch.empty(T, s.n_experts, device="cuda")
        ws = ws if ws is not None else B.workspace(self.gpu, T)
        B.coli_moe_forward(self.gpu, x, y, ws, logits_in=logits_in, idx_out=idx, w_out=w,
                           logits_out=lg)
        torch.cuda.synchronize()
        return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


def rel_err_per_token(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    d = np.abs(y.astype(np.float64) - ref.astype(np.float64)).max(axis=1)
    m = np.abs(ref.astype(np.float64)).max(axis=1)
    return np.where(m > 0, d / np.where(m > 0, m, 1), d)


def assert_close_layer(y, ref, tol=REL_TOL):
    err = rel_err_per_token(y, ref)
    assert (err <= tol).all(), f"per-token rel err max {err.max():.3e} (tol {tol})"
    return float(err.max())


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)
