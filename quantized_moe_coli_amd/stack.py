"""A stack of routed-MoE layers resident in HBM, decoded one token at a time.

The colibrì pages run GLM-5.2 by streaming each layer's selected experts for
every generated token, with a learned cache that pins the most-used experts
(README "Quick start"; CSDN feature, "冷启动与热缓存的辩证法") and an
adaptive expert top-p (README "Quick start").  On one MI355X a 40-layer int4 stack
(40 x 257 experts, ~195 GB) fits in HBM, so this driver measures the routed
layers back to back at the popularity skew and top-p of that workload.

Glue between layers: ``h <- h + MoE_l(rmsnorm(h))`` with a weightless
RMSNorm (eps 1e-6).  It stands in for the attention blocks the pages' model
has between its MoE layers, only to keep the hidden state's magnitude stable
from layer to layer; it is plain torch and not part of the MoE path.

Per layer l the router gets per-expert logit offsets -1.1*ln(rank_l(e)+1)
over a random ranking of the experts (a Zipf-like popularity), added to the
logits computed from the gate (the layer's ``gate_offset``), and an expert
top-p of 0.7 over the normalised weights with renormalisation.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import binding as B
from . import inputs

RMS_EPS = 1e-6
STACK_SHAPE = inputs.GLM.with_(top_p=0.7)
ZIPF_S = 1.1


def layer_seed(layer: int) -> int:
    """Generator seed of layer ``layer``'s weights, gate and bias."""
    return inputs.seed_of(0, layer)


def token_seed() -> int:
    """Generator seed of the per-step input tokens (step s draws index s)."""
    return 1


@dataclass
class Stack:
    s: inputs.Shape
    layers: list
    offsets: list
    c_layers: list = field(default_factory=list)

    @property
    def n_layers(self) -> int:
        return len(self.layers)


def build(n_layers: int = 40, s: inputs.Shape = STACK_SHAPE, device="cuda") -> Stack:
    """Draw and pack every layer on the device (weights drawn per expert,
    packed by coli_quant_pack in place, then freed)."""
    cfg = B.router_cfg(s.n_experts, s.top_k, s.n_group, s.topk_group, 1, s.rsf, s.top_p, 1)
    layers, offsets = [], []
    for li in range(n_layers):
        seed = layer_seed(li)
        L = B.MoeLayer.empty(s.hidden, s.inter, s.bits, cfg, device)
        L.gate_w.copy_(inputs.gate_weight(s, seed, device))
        L.gate_bias.copy_(inputs.gate_bias(s, seed, device))
        off = inputs.zipf_logit_offsets(0, li, s.n_experts, ZIPF_S, device)
        L.gate_offset = off
        for e in range(s.n_experts + 1):
            g, u, d = inputs.expert_weights(s, seed, e, device)
            L.pack_expert(e, g, u, d)
            del g, u, d
        layers.append(L)
        offsets.append(off)
        torch.cuda.synchronize()
    st = Stack(s, layers, offsets)
    st.c_layers = [L.c_struct() for L in layers]
    return st


def rmsnorm(h: torch.Tensor) -> torch.Tensor:
    return torch.nn.functional.rms_norm(h, (h.shape[-1],), eps=RMS_EPS)


def step(st: Stack, h: torch.Tensor, ws: torch.Tensor, y: torch.Tensor,
         idx_rec: torch.Tensor | None = None, w_rec: torch.Tensor | None = None) -> None:
    """One token through every layer, in place on h [T, H].  idx_rec/w_rec
    [n_layers, T, k] receive each layer's routing when given."""
    for li, L in enumerate(st.layers):
        B.coli_moe_forward(L, rmsnorm(h), y, ws,
                           idx_out=None if idx_rec is None else idx_rec[li],
                           w_out=None if w_rec is None else w_rec[li],
                           c_layer=st.c_layers[li])
        h.add_(y)


@dataclass
class TieredStack:
    """The same stack with each layer's routed experts in a pinned host tier
    and ``n_slots`` HBM slots per layer in front of it (per-layer expert
    caches); gates, offsets and shared experts stay in HBM."""
    s: inputs.Shape
    layers: list
    caches: list
    offsets: list
    n_slots: int
    c_layers: list = field(default_factory=list)

    @property
    def n_layers(self) -> int:
        return len(self.layers)


def build_tiered(n_layers: int, n_slots: int, s: inputs.Shape = STACK_SHAPE,
                 device="cuda", log=None) -> TieredStack:
    """Draw and pack every layer as ``build`` does; each layer's routed
    experts are packed into one reused HBM staging layer and copied to the
    layer's host tier, and the layer keeps ``n_slots`` empty slots."""
    cfg = B.router_cfg(s.n_experts, s.top_k, s.n_group, s.topk_group, 1, s.rsf, s.top_p, 1)
    staging = B.MoeLayer.empty(s.hidden, s.inter, s.bits, cfg, device, gate=False)
    layers, caches, offsets = [], [], []
    for li in range(n_layers):
        seed = layer_seed(li)
        L = B.MoeLayer.empty(s.hidden, s.inter, s.bits, cfg, device, n_slots=n_slots)
        L.gate_w.copy_(inputs.gate_weight(s, seed, device))
        L.gate_bias.copy_(inputs.gate_bias(s, seed, device))
        off = inputs.zipf_logit_offsets(0, li, s.n_experts, ZIPF_S, device)
        L.gate_offset = off
        for e in range(s.n_experts):
            g, u, d = inputs.expert_weights(s, seed, e, device)
            staging.pack_expert(e, g, u, d)
        g, u, d = inputs.expert_weights(s, seed, s.n_experts, device)
        L.pack_expert(s.n_experts, g, u, d)
        del g, u, d
        torch.cuda.synchronize()
        try:
            tier = B.HostTier(s.n_experts, s.hidden, s.inter, s.bits)
        except B.ColiError as e:
            pinned = sum(c.tier.buf.nbytes for c in caches)
            raise RuntimeError(f"pinned host allocation failed after {li} layers "
                               f"({pinned / 1e9:.1f} GB pinned): the host limits pinned "
                               f"memory per process; build fewer layers") from e
        tier.load_experts(staging)
        cache = B.ExpertCache(tier, n_slots, device)
        cache.init()
        layers.append(L)
        caches.append(cache)
        offsets.append(off)
        if log is not None and (li % 8 == 7 or li == n_layers - 1):
            log(f"[stack] {li + 1}/{n_layers} layers to the host tier")
    del staging
    torch.cuda.synchronize()
    st = TieredStack(s, layers, caches, offsets, n_slots)
    st.c_layers = [L.c_struct() for L in layers]
    return st


def step_tiered(st: TieredStack, h: torch.Tensor, ws: torch.Tensor, y: torch.Tensor,
                idx_rec: torch.Tensor | None = None) -> None:
    """One token through every layer of a tiered stack, in place on h."""
    for li, L in enumerate(st.layers):
        B.coli_moe_forward_cached(L, st.caches[li], rmsnorm(h), y, ws,
                                  idx_out=None if idx_rec is None else idx_rec[li],
                                  c_layer=st.c_layers[li])
        h.add_(y)
