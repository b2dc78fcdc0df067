"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only draws random numbers.  It holds no step of the layer's
arithmetic (no quantisation, routing, expert math or combine), so both the
GPU library's tests and the CPU oracle may take their inputs from it.

Every tensor has its own generator, seeded from (seed, role, index), so any
single expert or token batch can be regenerated on its own -- on the device
for the full-size layers, on the CPU for the small ones.  The same seed on
two different device types gives different numbers: a fixture draws once and
hands the same values to both sides.

Shapes (the GLM-5.2 layer the colibrì pages describe: 256 routed experts,
top-8, one shared expert, ~19 MB per int4 expert => H=6144, I=2048):
  * ``TINY``  H 256, I 128, E 16, top-2, no groups, zero router bias, int8.
  * ``GLM``   H 6144, I 2048, E 256, top-8, 8 groups keep 4, rsf 2.5,
              router bias N(0, 0.01), int4 by default.
Weights N(0, 0.02) (fp32, quantised by the layer's own packing step),
activations N(0, 1).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, replace

import torch

# roles: distinct streams for each kind of tensor
_ROLE = {"gate_w": 1, "bias": 2, "w_gate": 3, "w_up": 4, "w_down": 5,
         "x": 6, "logit_z": 7, "logit_eps": 8, "zipf": 9, "fp8_codes": 10, "fp8_scale": 11}


@dataclass(frozen=True)
class Shape:
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    n_group: int = 1
    topk_group: int = 1
    rsf: float = 2.5
    bias_std: float = 0.0
    bits: int = 4
    w_std: float = 0.02
    x_std: float = 1.0
    top_p: float = 0.0

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)


TINY = Shape(hidden=256, inter=128, n_experts=16, top_k=2, n_group=1,
             topk_group=1, rsf=2.5, bias_std=0.0, bits=8)
GLM = Shape(hidden=6144, inter=2048, n_experts=256, top_k=8, n_group=8,
            topk_group=4, rsf=2.5, bias_std=0.01, bits=4)


def seed_of(*parts: int) -> int:
    """Mix integers into a 63-bit generator seed (stable across runs)."""
    h = hashlib.blake2b(repr(tuple(int(p) for p in parts)).encode(), digest_size=8)
    return int.from_bytes(h.digest(), "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def normal(shape_, std, device, *parts) -> torch.Tensor:
    """N(0, std^2) fp32 tensor from the stream named by ``parts``."""
    g = _gen(device, *parts)
    t = torch.randn(shape_, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def gate_weight(s: Shape, seed: int, device="cpu") -> torch.Tensor:
    """Router gate [E, H] fp32."""
    return normal((s.n_experts, s.hidden), s.w_std, device, seed, _ROLE["gate_w"])


def gate_bias(s: Shape, seed: int, device="cpu") -> torch.Tensor:
    """Router selection bias [E] fp32 (zeros when the shape has none)."""
    if s.bias_std == 0.0:
        return torch.zeros(s.n_experts, dtype=torch.float32, device=device)
    return normal((s.n_experts,), s.bias_std, device, seed, _ROLE["bias"])


def expert_weights(s: Shape, seed: int, e: int, device="cpu"):
    """fp32 (gate [I, H], up [I, H], down [H, I]) of expert ``e``;
    ``e == n_experts`` is the shared expert."""
    H, I = s.hidden, s.inter
    return (normal((I, H), s.w_std, device, seed, _ROLE["w_gate"], e),
            normal((I, H), s.w_std, device, seed, _ROLE["w_up"], e),
            normal((H, I), s.w_std, device, seed, _ROLE["w_down"], e))


def tokens(s: Shape, seed: int, step: int, T: int, device="cpu") -> torch.Tensor:
    """Activations [T, H] fp32 ~ N(0, x_std^2)."""
    return normal((T, s.hidden), s.x_std, device, seed, _ROLE["x"], step)


def correlated_logits(seed: int, T: int, E: int, rho: float, scale: float = 1.57,
                      device="cpu") -> torch.Tensor:
    """Router logits [T, E] whose tokens share a common component:
    scale * (rho * z_e + sqrt(1 - rho^2) * eps_te), z, eps ~ N(0, 1).
    rho = 0 gives independent tokens (many unique experts per batch), rho near
    1 makes the batch agree (few unique experts).  scale 1.57 ~ 0.02*sqrt(6144)
    is the spread of logits a N(0, 0.02) gate gives on N(0, 1) inputs."""
    z = normal((1, E), 1.0, device, seed, _ROLE["logit_z"])
    eps = normal((T, E), 1.0, device, seed, _ROLE["logit_eps"], T)
    return (scale * (rho * z + math.sqrt(max(0.0, 1.0 - rho * rho)) * eps)).float()


def zipf_logit_offsets(seed: int, layer: int, E: int, s_exp: float = 1.1,
                       device="cpu") -> torch.Tensor:
    """Per-expert logit offsets -s*ln(rank+1) over a random ranking of the
    experts: a Zipf(s)-skewed expert popularity for one layer."""
    g = _gen("cpu", seed, _ROLE["zipf"], layer)
    rank = torch.randperm(E, generator=g)
    return (-s_exp * torch.log(rank.double() + 1.0)).float().to(device)


def fp8_checkpoint(rows: int, cols: int, seed: int, device="cpu"):
    """A synthetic FP8 checkpoint matrix as a block-scaled FP8 checkpoint
    stores it: uint8 OCP E4M3 codes [rows, cols] and fp32 scales
    [ceil(rows/128), ceil(cols/128)].  The codes are torch's float8_e4m3fn
    storage of N(0, 100^2) draws clipped to the format's +-448 (so they span
    the format's normal and subnormal codes and both zeros); the block scales
    are uniform in [1e-4, 4e-4], which puts the weights at the N(0, 0.02)
    scale of the layer's other weights.  No NaN code is produced."""
    g = _gen(device, seed, _ROLE["fp8_codes"], rows, cols)
    v = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    v.mul_(100.0).clamp_(-448.0, 448.0)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8)
    g = _gen(device, seed, _ROLE["fp8_scale"], rows, cols)
    bs = torch.rand(((rows + 127) // 128, (cols + 127) // 128), generator=g, device=device,
                    dtype=torch.float32)
    bs.mul_(3e-4).add_(1e-4)
    return codes.contiguous(), bs
