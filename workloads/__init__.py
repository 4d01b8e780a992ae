"""Seeded synthetic inputs for MoE dispatch/combine.

This module draws inputs only; it holds none of the dispatch/combine
arithmetic, and both the GPU path's tests and the oracle take their inputs
from it.  Routing (which experts a token picks and with what weight) is
upstream gating, not part of the measured path, so it lives here as an
input generator.

The pages measure on DeepSeek-V3/R1 settings, not on a dataset
([P1] "DeepSeek 开源周第二弹：DeepEP —— 首个 MoE 模型训练和推理的 EP 通信库",
section "DeepEP 的常规内核和低延迟内核": prefill batches of 4096 tokens,
hidden 7168, top-4 groups, top-8 experts; decode batches of 128 tokens).
Trained router statistics are not available, so gate logits are N(0, 1).
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    make_workload,
    make_x_bits,
    make_y_bits,
    route_softmax_topk,
    route_group_limited,
    route_zipf,
    to_bf16_bits,
)
