"""CPU oracle for MoE dispatch layout, dispatch and combine.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously
correct statement of what the GPU path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  The product package ``combine_ep_dispatch_amd`` never
imports it and shares no code with it.

Sources (the pages describe DeepSeek's DeepEP library; they fix *what* is
moved, not a kernel design):

* [P1] "DeepSeek 开源周第二弹：DeepEP —— 首个 MoE 模型训练和推理的 EP 通信库"
  (m.youleyou.com), sections "DeepEP 的核心功能" and
  "DeepEP 的常规内核和低延迟内核": tokens are sent to the experts they
  activate and the expert outputs are merged back; dispatch travels in
  FP8 and the merge is in BF16; the prefill setting is 4096 tokens,
  hidden 7168, top-4 groups, top-8 experts, the decode setting 128
  tokens.
* [P4] DeepEP article on deepseek.csdn.net, section "使用示例 › MoE 训练中的
  应用": ``dispatch(x, topk_idx, topk_weights, num_experts)`` returns the
  received rows, their routing and a ``handle``; section
  "推理解码阶段的应用": the low-latency form also returns the per-expert
  received count.
* [P5] "deepseek-ai/DeepEP" (agentlenshq.com), section "典型工作流程":
  dispatch routes tokens to their experts, the expert GEMM runs on the
  received rows, combine reduces the expert outputs back to the source.

Where the pages leave a step open (order inside an expert, FP8 variant,
scale granularity and formula, combine arithmetic) the oracle takes one
plain reading and states it in the function that implements it.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against brute force, exact rational arithmetic, library casts or
invariants.  The choice of scale convention (one FP32 scale per 128
channels, s = amax/448) and of the OCP E4M3FN variant is not fixed by the
pages, so against DeepEP itself those two conventions are parity
unpinned; they are pinned only against their own definitions.
"""

from .codecs import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_rne,
    f32_to_e4m3_rne_sat,
    e4m3_to_f32,
    E4M3_MAX,
)
from .ep_oracle import (  # noqa: F401
    dispatch_layout,
    dispatch_layout_padded,
    group_scales,
    quantize_tokens_fp8,
    dispatch_fp8,
    dispatch_bf16,
    combine,
    dequantize_rows,
    dispatch_backward,
    combine_backward,
    dot_rn32,
)
