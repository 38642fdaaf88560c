"""Layer shapes of the synthetic workloads.

The full-size shapes are the DeepSeek-V4.1-Flash MoE layer (hidden 5120, 384
routed experts, top-6, 1 shared expert, expert width 2304, route scale 1.5,
swiglu limit 10) from the checkpoint ``config.json`` on the "DeepSeek V4.1"
atlas page, and the drafter-style MoE (128 routed experts, top-3) from the
same file's ``dspark_n_routed_experts`` / ``dspark_n_activated_experts``.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    tokens: int
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    n_shared: int = 1
    shared_inter: int = 0
    route_scale: float = 1.5
    swiglu_limit: float = 10.0
    #: "none" or "zipf": a per-expert selection bias that skews the load
    bias: str = "none"
    zipf_s: float = 1.2
    #: bias amplitude: b_e = zipf_alpha * rank_e ** -zipf_s
    zipf_alpha: float = 0.626
    #: numeric id used to derive per-tensor seeds
    cfg_id: int = 0
    x_std: float = 1.0
    expert_std: float = 0.02
    #: pre-FFN RMSNorm in front of the layer (bf16 gain, eps norm_eps)
    norm: bool = False
    norm_eps: float = 1e-20
    #: routed expert weights: "mxfp4" (E2M1) or "mxfp8" (E4M3), E8M0 scale per 32
    expert_format: str = "mxfp4"
    extra: dict = field(default_factory=dict, compare=False)

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    @property
    def slots(self) -> int:
        return self.tokens * self.top_k


CONFIGS = {
    # 8 tokens on a small layer: the case the oracle finishes in seconds
    "tiny_t8_h512_e32": LayerConfig("tiny_t8_h512_e32", 8, 512, 32, 6, 256, 1, 256, cfg_id=1),
    # full-size decode, one token
    "decode_t1_h5120_e384": LayerConfig("decode_t1_h5120_e384", 1, 5120, 384, 6, 2304, 1, 2304, cfg_id=2),
    # full-size decode, 64 tokens
    "decode_t64_h5120_e384": LayerConfig("decode_t64_h5120_e384", 64, 5120, 384, 6, 2304, 1, 2304, cfg_id=3),
    # full-size prefill, 4096 tokens
    "prefill_t4096_h5120_e384": LayerConfig("prefill_t4096_h5120_e384", 4096, 5120, 384, 6, 2304, 1, 2304,
                                            cfg_id=4),
    # speculative-verify decode: one sequence with a 5-token draft block, and 64 sequences of 5
    "verify_t5_h5120_e384": LayerConfig("verify_t5_h5120_e384", 5, 5120, 384, 6, 2304, 1, 2304, cfg_id=6),
    "verify_t320_h5120_e384": LayerConfig("verify_t320_h5120_e384", 320, 5120, 384, 6, 2304, 1, 2304, cfg_id=7),
    # DeepSeek-V4-Pro MoE dimensions (hidden 7168, expert width 3072), one decode token
    "pro_t1_h7168_e384": LayerConfig("pro_t1_h7168_e384", 1, 7168, 384, 6, 3072, 1, 3072, cfg_id=8),
    # the one-token decode layer with the pre-FFN RMSNorm in front (eps 1e-20)
    "decode_t1_h5120_e384_norm": LayerConfig("decode_t1_h5120_e384_norm", 1, 5120, 384, 6, 2304, 1, 2304,
                                             cfg_id=9, norm=True),
    # MXFP8 (E4M3) routed experts: one decode token and the 4096-token prefill
    "decode_t1_h5120_e384_fp8": LayerConfig("decode_t1_h5120_e384_fp8", 1, 5120, 384, 6, 2304, 1, 2304,
                                            cfg_id=10, expert_format="mxfp8"),
    "prefill_t4096_h5120_e384_fp8": LayerConfig("prefill_t4096_h5120_e384_fp8", 4096, 5120, 384, 6, 2304, 1,
                                                2304, cfg_id=11, expert_format="mxfp8"),
    # skewed routing on the drafter-style MoE, 16384 tokens
    "skew_t16384_h5120_e128": LayerConfig("skew_t16384_h5120_e128", 16384, 5120, 128, 3, 2304, 1, 2304,
                                          bias="zipf", cfg_id=5),
}
