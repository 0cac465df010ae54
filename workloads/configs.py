"""Layer shapes: the workloads plus reduced shapes for full-oracle tests."""
from dataclasses import dataclass, replace
from typing import Optional

SOFTMAX = "softmax"
SIGMOID = "sigmoid"
SQRTSOFTPLUS = "sqrtsoftplus"


@dataclass(frozen=True)
class LayerShape:
    name: str
    T: int                      # tokens in the batch
    H: int                      # hidden size
    E: int                      # routed experts
    S: int                      # shared experts (always active, unweighted)
    k: int                      # experts chosen per token
    I: int                      # expert intermediate size (routed and shared)
    G: int = 1                  # expert groups
    topk_group: int = 1         # groups kept per token
    scoring: str = SOFTMAX      # "softmax" | "sigmoid" | "sqrtsoftplus"
    renorm: bool = True         # renormalise the selected gates
    scale: float = 1.0          # routed scaling factor applied to the gates
    capacity_factor: float = 0.0  # <= 0: unlimited
    drop_tokens: bool = False   # with a capacity: drop overflow instead of re-routing
    dtype: str = "bf16"         # "bf16" | "f32" for x and every weight; "fp8": bf16 x and
                                # router, E4M3 expert weights with 128 x 128 UE8M0 block scales
    sel_bias: Optional[float] = None   # selection bias ~ U(-a, a) when set
    zipf_s: Optional[float] = None     # Zipf exponent of the per-expert logit offset
    hash_vocab: int = 0         # > 0: hash routing through a [hash_vocab, k] token-id table
    seed: int = 0

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)

    @property
    def rows(self) -> int:
        """Upper bound of expert rows: every (token, slot) plus S*T shared rows."""
        return self.T * self.k + self.S * self.T

    def flops(self, assigned_slots: Optional[int] = None) -> float:
        """Algorithmic FLOPs of one layer call: router GEMM + 3 expert GEMMs
        over assigned (non-dropped) rows and all shared rows."""
        a = self.T * self.k if assigned_slots is None else assigned_slots
        return 2.0 * self.T * self.H * self.E + 6.0 * self.H * self.I * (a + self.S * self.T)


CONFIGS = {
    # Tiny Mixtral-style layer in fp32.
    "tiny_mixtral_fp32": LayerShape("tiny_mixtral_fp32", T=64, H=256, E=8, S=0, k=2, I=512,
                                    dtype="f32", seed=101),
    # Mixtral-8x7B-shaped layer.
    "mixtral_8x7b": LayerShape("mixtral_8x7b", T=4096, H=4096, E=8, S=0, k=2, I=14336, seed=202),
    # DeepSeek-V2-shaped layer: softmax without renormalisation.
    "deepseek_v2": LayerShape("deepseek_v2", T=8192, H=5120, E=160, S=2, k=6, I=1536,
                              renorm=False, seed=303),
    # DeepSeek-V3-shaped layer, prefill size.
    "deepseek_v3_prefill": LayerShape("deepseek_v3_prefill", T=16384, H=7168, E=256, S=1, k=8,
                                      I=2048, G=8, topk_group=4, scoring=SIGMOID, renorm=True,
                                      scale=2.5, sel_bias=0.05, seed=404),
    # DeepSeek-V3-shaped layer, decode size, Zipf-skewed load and expert capacity.
    "deepseek_v3_decode": LayerShape("deepseek_v3_decode", T=128, H=7168, E=256, S=1, k=8,
                                     I=2048, G=8, topk_group=4, scoring=SIGMOID, renorm=True,
                                     scale=2.5, sel_bias=0.05, zipf_s=1.1, capacity_factor=1.25,
                                     seed=505),
    # DeepSeek-V4-Flash-shaped layer, prefill size: sqrt(softplus) scores with
    # the selection bias, no group limit.  The page gives H, E, S and k; the
    # expert width is not printed, 2048 (V3's) makes the experts of its 43
    # layers 278B of the 284B total it states.
    "deepseek_v4_flash": LayerShape("deepseek_v4_flash", T=16384, H=4096, E=256, S=1, k=6, I=2048,
                                    scoring=SQRTSOFTPLUS, renorm=True, scale=1.0, sel_bias=0.05, seed=606),
    # The same layer with hash routing (V4's first layers): a fixed table over
    # the 129,280-entry vocabulary chooses, the router only weights.
    "deepseek_v4_flash_hash": LayerShape("deepseek_v4_flash_hash", T=16384, H=4096, E=256, S=1, k=6, I=2048,
                                         scoring=SQRTSOFTPLUS, renorm=True, scale=1.0, hash_vocab=129280,
                                         seed=707),
}
# The DeepSeek-V3-shaped layers with FP8 experts (E4M3 codes, 128 x 128 UE8M0
# block scales; "15. DeepSeek：MLA、MoE 与 MTP", section on FP8 as a training
# recipe): x and the router stay bf16.
CONFIGS["deepseek_v3_prefill_fp8"] = CONFIGS["deepseek_v3_prefill"].with_(name="deepseek_v3_prefill_fp8", dtype="fp8",
                                                                          seed=808)
CONFIGS["deepseek_v3_decode_fp8"] = CONFIGS["deepseek_v3_decode"].with_(name="deepseek_v3_decode_fp8", dtype="fp8",
                                                                        seed=909)

# Reduced shapes with the same routing structure, small enough for the full
# fp64 oracle to finish in seconds while still spanning several GEMM tiles and
# ragged tails (T not a multiple of any tile height).
TEST_SHAPES = {
    "tiny_mixtral_fp32": CONFIGS["tiny_mixtral_fp32"],
    "mixtral_small": CONFIGS["mixtral_8x7b"].with_(name="mixtral_small", T=389, H=512, I=1024),
    "v2_small": CONFIGS["deepseek_v2"].with_(name="v2_small", T=301, H=512, I=384),
    "v3_small": CONFIGS["deepseek_v3_prefill"].with_(name="v3_small", T=517, H=512, I=256),
    "v3_decode_small": CONFIGS["deepseek_v3_decode"].with_(name="v3_decode_small", H=512, I=256),
    "v4_small": CONFIGS["deepseek_v4_flash"].with_(name="v4_small", T=517, H=512, I=256),
    "v4_hash_small": CONFIGS["deepseek_v4_flash_hash"].with_(name="v4_hash_small", T=389, H=512, I=256,
                                                             hash_vocab=3000),
    "v3_fp8_small": CONFIGS["deepseek_v3_prefill_fp8"].with_(name="v3_fp8_small", T=517, H=512, I=384),
    "v3_decode_fp8_small": CONFIGS["deepseek_v3_decode_fp8"].with_(name="v3_decode_fp8_small", H=512, I=256),
}


def get_config(name: str) -> LayerShape:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in TEST_SHAPES:
        return TEST_SHAPES[name]
    raise KeyError(name)
