"""Seeded generators of the layer's inputs (hidden states and all weights).

Distributions (one recipe for every workload):

* x: N(0, 1) per element, rounded to bf16 (round to nearest even).
* router weight W_r [E, H]: fp32 N(0, 1/H), so that a logit is ~N(0, 1).
* routed expert weights: fp32 N(0, 0.02^2), gate/up [2I, H] and down [H, I]
  per expert, encoded to MXFP4 by :func:`mxfp4_encode` (or to MXFP8 by
  :func:`mxfp8_encode` when the workload's expert format is "mxfp8").
* shared expert weights: N(0, 0.02^2) rounded to bf16.
* optional Zipf selection bias: b_e = alpha * r_e^-s with r a seeded random
  permutation of 1..E (rank 1 is the hottest expert).
* with the pre-FFN norm on: x rows of very different sizes, the draw above
  times 2^u per row with u uniform in [-4, 8) (a residual stream's rows are
  not normalised), and a bf16 gain gamma ~ N(1, 0.1^2) per channel.

Every tensor has its own seed, derived from (seed, config id, tensor id,
expert, weight set) by numpy's ``SeedSequence`` hashing, so one expert can be
regenerated alone and a second weight set ("another layer") is independent.
Tensors are drawn with torch's generator on the device they are made on: the
same seed gives different (but fixed) values on CPU and on the GPU, and every
consumer takes its inputs from one call.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import LayerConfig

TENSOR_X, TENSOR_ROUTER, TENSOR_BIAS, TENSOR_GU, TENSOR_DN, TENSOR_SH_GU, TENSOR_SH_DN, TENSOR_GAMMA = range(8)


def derive_seed(*parts: int) -> int:
    """A 63-bit seed from integer parts (numpy SeedSequence hashing)."""
    ss = np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts])
    return int(ss.generate_state(1, np.uint64)[0]) & ((1 << 63) - 1)


def _randn(shape, seed: int, device, std: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


def f32_to_bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """Round fp32 to bf16 (nearest even) and return the raw bits as int16."""
    return t.to(torch.bfloat16).view(torch.int16)


def pack_nibbles(codes: torch.Tensor) -> torch.Tensor:
    """Pack 4-bit codes [..., K] to bytes [..., K/2]: even element in the low nibble."""
    lo = codes[..., 0::2].to(torch.uint8)
    hi = codes[..., 1::2].to(torch.uint8)
    return lo | (hi << 4)


# Magnitude thresholds of round-to-nearest-even onto E2M1 {0,.5,1,1.5,2,3,4,6}.
# A magnitude equal to a midpoint goes to the neighbour whose code is even:
# 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4; above 5 saturates
# to 6.  torch.bucketize(right=False) puts x in bucket i when b[i-1] < x <= b[i],
# so a midpoint that rounds up uses the float just below it as its boundary.
def _e2m1_boundaries(device) -> torch.Tensor:
    below = lambda v: float(np.nextafter(np.float32(v), np.float32(-np.inf)))  # noqa: E731
    return torch.tensor([0.25, below(0.75), 1.25, below(1.75), 2.5, below(3.5), 5.0],
                        dtype=torch.float32, device=device)


def _block_amax(blocks: torch.Tensor) -> torch.Tensor:
    """max |x| over the last dimension (32) by pairwise elementwise maxima.

    The same values as ``blocks.abs().amax(dim=-1)`` (a maximum is exact in any
    order), without a reduction kernel: under rocprofv3 counter collection the
    host process crashed inside the launch of torch's reduce kernel for amax.
    """
    a = blocks.abs()
    while a.shape[-1] > 1:
        a = torch.maximum(a[..., 0::2], a[..., 1::2])
    return a.squeeze(-1)


def mxfp4_encode(w: torch.Tensor):
    """Encode fp32 rows [R, K] (K % 32 == 0) to MXFP4 (OCP Microscaling v1.0 rule).

    Per block of 32 consecutive elements of a row: shared exponent
    floor(log2(amax)) - 2 (2 = emax of E2M1), stored biased by 127 and clamped
    to [0, 254]; an all-zero block gets 127.  Elements are divided by the block
    scale and rounded to nearest even onto E2M1, saturating at +-6.  Returns
    (packed uint8 [R, K/2], scales uint8 [R, K/32]).
    """
    rows, k = w.shape
    assert k % 32 == 0
    blocks = w.reshape(rows, k // 32, 32)
    amax = _block_amax(blocks)
    _, exp = torch.frexp(amax)  # amax = m * 2^exp, m in [0.5, 1)
    code = (exp.to(torch.int32) - 1 - 2 + 127).clamp(0, 254)
    code = torch.where(amax == 0, torch.full_like(code, 127), code)
    scale = torch.ldexp(torch.ones_like(amax), (code - 127).to(torch.float32))
    scaled = blocks / scale.unsqueeze(-1)
    mag_code = torch.bucketize(scaled.abs(), _e2m1_boundaries(w.device), right=False).to(torch.int32)
    sign = torch.signbit(scaled).to(torch.int32) << 3
    codes = (mag_code | sign).reshape(rows, k)
    return pack_nibbles(codes), code.to(torch.uint8)


def mxfp8_encode(w: torch.Tensor):
    """Encode fp32 rows [R, K] (K % 32 == 0) to MXFP8 with E4M3 elements (OCP rule).

    Per block of 32: shared exponent floor(log2(amax)) - 8 (8 = emax of E4M3),
    biased by 127 and clamped to [0, 254], 127 for an all-zero block;
    elements divided by the block scale, held within +-448 and rounded to
    nearest even by torch's float8_e4m3fn cast.  Returns (codes uint8 [R, K],
    scales uint8 [R, K/32]).
    """
    rows, k = w.shape
    assert k % 32 == 0
    blocks = w.reshape(rows, k // 32, 32)
    amax = _block_amax(blocks)
    _, exp = torch.frexp(amax)
    code = (exp.to(torch.int32) - 1 - 8 + 127).clamp(0, 254)
    code = torch.where(amax == 0, torch.full_like(code, 127), code)
    scale = torch.ldexp(torch.ones_like(amax), (code - 127).to(torch.float32))
    scaled = (blocks / scale.unsqueeze(-1)).clamp(-448.0, 448.0)
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(rows, k)
    return codes, code.to(torch.uint8)


class ExpertTensor:
    """Per-expert read access ``t[e]`` to a device tensor [E, ...] as numpy arrays."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)

    def __len__(self) -> int:
        return self.shape[0]

    def __getitem__(self, e):
        return self.t[e].detach().cpu().numpy()


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: torch.Tensor            # int16 bf16 bits [T, H]
    router_w: torch.Tensor     # float32 [E, H]
    router_bias: Optional[torch.Tensor]  # float32 [E] or None
    gu_q: torch.Tensor         # uint8 [E, 2I, H/2] (MXFP8: [E, 2I, H])
    gu_s: torch.Tensor         # uint8 [E, 2I, H/32]
    dn_q: torch.Tensor         # uint8 [E, H, I/2] (MXFP8: [E, H, I])
    dn_s: torch.Tensor         # uint8 [E, H, I/32]
    sh_gu: Optional[torch.Tensor]  # int16 bf16 bits [2Is, H] or None
    sh_dn: Optional[torch.Tensor]  # int16 bf16 bits [H, Is] or None
    norm_gamma: Optional[torch.Tensor] = None  # int16 bf16 bits [H] or None (no norm)

    def to(self, device) -> "LayerInputs":
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return LayerInputs(self.cfg, mv(self.x), mv(self.router_w), mv(self.router_bias), mv(self.gu_q),
                           mv(self.gu_s), mv(self.dn_q), mv(self.dn_s), mv(self.sh_gu), mv(self.sh_dn),
                           mv(self.norm_gamma))

    def oracle_args(self) -> dict:
        """Keyword arguments of the oracle's ``layer_forward`` (numpy on the host)."""
        npy = lambda t: None if t is None else t.detach().cpu().numpy()  # noqa: E731
        return dict(x_bits=npy(self.x).view(np.uint16), router_w=npy(self.router_w),
                    router_bias=npy(self.router_bias),
                    gu_q=ExpertTensor(self.gu_q), gu_s=ExpertTensor(self.gu_s),
                    dn_q=ExpertTensor(self.dn_q), dn_s=ExpertTensor(self.dn_s),
                    sh_gu=None if self.sh_gu is None else npy(self.sh_gu).view(np.uint16),
                    sh_dn=None if self.sh_dn is None else npy(self.sh_dn).view(np.uint16),
                    top_k=self.cfg.top_k, route_scale=self.cfg.route_scale,
                    swiglu_limit=self.cfg.swiglu_limit,
                    norm_gamma=None if self.norm_gamma is None else npy(self.norm_gamma).view(np.uint16),
                    norm_eps=self.cfg.norm_eps, expert_format=self.cfg.expert_format)


def zipf_bias(cfg: LayerConfig, seed: int, weight_set: int = 0) -> torch.Tensor:
    """b_e = alpha * rank_e^-s over a seeded random ranking of the experts."""
    g = torch.Generator(device="cpu")
    g.manual_seed(derive_seed(seed, cfg.cfg_id, TENSOR_BIAS, 0, weight_set))
    rank = torch.randperm(cfg.n_experts, generator=g).to(torch.float64) + 1.0
    return (cfg.zipf_alpha * rank.pow(-cfg.zipf_s)).to(torch.float32)


def make_router_inputs(cfg: LayerConfig, seed: int = 0, device="cpu", weight_set: int = 0,
                       x_seed: Optional[int] = None):
    """(x bits [T, H], W_r [E, H], bias [E] or None): the same tensors make_inputs draws."""
    dev = torch.device(device)
    xs = seed if x_seed is None else x_seed
    x = _randn((cfg.tokens, cfg.hidden), derive_seed(xs, cfg.cfg_id, TENSOR_X, 0, 0), dev, cfg.x_std)
    if cfg.norm:
        g = torch.Generator(device=dev)
        g.manual_seed(derive_seed(xs, cfg.cfg_id, TENSOR_X, 1, 0))
        x = x * torch.exp2(torch.randint(-4, 8, (cfg.tokens, 1), generator=g, device=dev).to(torch.float32))
    x = f32_to_bf16_bits(x)
    router_w = _randn((cfg.n_experts, cfg.hidden), derive_seed(seed, cfg.cfg_id, TENSOR_ROUTER, 0, weight_set),
                      dev, 1.0 / math.sqrt(cfg.hidden))
    bias = zipf_bias(cfg, seed, weight_set).to(dev) if cfg.bias == "zipf" else None
    return x, router_w, bias


def make_inputs(cfg: LayerConfig, seed: int = 0, device="cpu", weight_set: int = 0,
                x_seed: Optional[int] = None) -> LayerInputs:
    """All inputs of one layer, generated on ``device``.

    ``weight_set`` selects an independent draw of every weight tensor (a
    different layer of the same shape); ``x_seed`` (default ``seed``) selects
    the hidden states.
    """
    dev = torch.device(device)
    t, h, e, inter = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.inter
    x, router_w, bias = make_router_inputs(cfg, seed, device, weight_set, x_seed)
    per_byte = {"mxfp4": 2, "mxfp8": 1}[cfg.expert_format]
    encode = mxfp4_encode if cfg.expert_format == "mxfp4" else mxfp8_encode
    gu_q = torch.empty((e, 2 * inter, h // per_byte), dtype=torch.uint8, device=dev)
    gu_s = torch.empty((e, 2 * inter, h // 32), dtype=torch.uint8, device=dev)
    dn_q = torch.empty((e, h, inter // per_byte), dtype=torch.uint8, device=dev)
    dn_s = torch.empty((e, h, inter // 32), dtype=torch.uint8, device=dev)
    for ex in range(e):
        w = _randn((2 * inter, h), derive_seed(seed, cfg.cfg_id, TENSOR_GU, ex, weight_set), dev, cfg.expert_std)
        gu_q[ex], gu_s[ex] = encode(w)
        w = _randn((h, inter), derive_seed(seed, cfg.cfg_id, TENSOR_DN, ex, weight_set), dev, cfg.expert_std)
        dn_q[ex], dn_s[ex] = encode(w)
        del w
    sh_gu = sh_dn = None
    if cfg.n_shared:
        i_s = cfg.shared_inter
        sh_gu = f32_to_bf16_bits(_randn((2 * i_s, h), derive_seed(seed, cfg.cfg_id, TENSOR_SH_GU, 0, weight_set),
                                        dev, cfg.expert_std))
        sh_dn = f32_to_bf16_bits(_randn((h, i_s), derive_seed(seed, cfg.cfg_id, TENSOR_SH_DN, 0, weight_set),
                                        dev, cfg.expert_std))
    gamma = None
    if cfg.norm:
        gamma = f32_to_bf16_bits(1.0 + _randn((h,), derive_seed(seed, cfg.cfg_id, TENSOR_GAMMA, 0, weight_set), dev,
                                              0.1))
    return LayerInputs(cfg, x, router_w, bias, gu_q, gu_s, dn_q, dn_s, sh_gu, sh_dn, gamma)
