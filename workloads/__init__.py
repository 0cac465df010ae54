"""Layer shapes and seeded synthetic inputs for the sparse MoE FFN layer.

This package is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It holds *no* arithmetic of the method itself (no routing, no scoring,
no FFN): only shape descriptions and seeded random tensors.

Shapes follow the pages' statements of the layer:
  * Mixtral-style 8 experts / top-2 softmax ("MoE on KnightLi的博客", the MoE
    section; "MoE架构揭秘", section 3.1 on the router),
  * DeepSeek-V2: 160 routed + 2 shared experts, top-6, intermediate 1536
    ("15. DeepSeek：MLA、MoE 与 MTP", section "V2：MLA 和 DeepSeekMoE 第一次组合"),
  * DeepSeek-V3: 256 routed + 1 shared, top-8, 8 groups / 4 kept, sigmoid +
    selection bias, gates renormalised x 2.5, intermediate 2048, hidden 7168
    (same page, section "V3 的 MoE：256 个专家怎样选 8 个"),
  * DeepSeek-V4-Flash: 256 routed + 1 shared, top-6, hidden 4096,
    sqrt(softplus) scores with the selection bias and no group limit, or hash
    routing over the 129,280-token vocabulary (same page, section
    "V4：放弃潜向量，改用压缩注意力", and its table of generations).
"""
from .configs import LayerShape, CONFIGS, TEST_SHAPES, get_config  # noqa: F401
from .generate import hash_table, make_inputs, zipf_logit_offsets, zipf_token_ids  # noqa: F401
