"""Oracle for the MoE dispatch/combine hot path (test infrastructure only).

Plain numpy, no blocking, fusion or reordering beyond what each definition
states.  Floating point is binary32 where the method fixes binary32
(the quantiser and the combine accumulator); numpy float32 ``+ * /`` are
single IEEE operations with round-to-nearest-even and are never fused.

Terminology: T tokens, H hidden channels, E experts, K experts per token
(top-k), R = T*K receive rows, G = H/128 scale groups per row.
"""

import math

import numpy as np

from .codecs import bf16_bits_to_f32, f32_to_bf16_rne, f32_to_e4m3_rne_sat, e4m3_to_f32

GROUP = 128  # channels per FP8 scale group
SCALE_FLOOR = np.float32(2.0 ** -126)  # smallest normal binary32


def dispatch_layout(topk_idx, num_experts):
    """Routing layout of one dispatch: counts, offsets, slots and sources.

    [P4 "使用示例 › MoE 训练中的应用"] dispatch takes ``topk_idx`` and
    ``num_experts`` and returns a ``handle`` that combine uses to bring the
    rows back; [P4 "推理解码阶段的应用"] the per-expert received count is
    part of what dispatch reports.  The pages do not say how rows are
    ordered inside an expert; the reading taken here is a stable counting
    sort of the (t, k) entries by expert, i.e. rows of one expert appear in
    ascending token order, and entries of one token in ascending k.

    Entries whose expert id is outside [0, num_experts) (for example -1)
    are masked: not counted, ``slot = -1``.  They sort behind every real
    row, so ``src_token`` has -1 in rows ``offsets[E] .. T*K-1``.

    Returns
      counts  int32[E]      entries routed to each expert
      offsets int32[E+1]    exclusive prefix sum of counts (offsets[0] = 0)
      slot    int32[T, K]   receive row of entry (t, k), or -1 if masked
      src     int32[T*K]    token that receive row r came from, or -1
    """
    idx = np.asarray(topk_idx)
    if idx.ndim != 2:
        raise ValueError("topk_idx must be [T, K]")
    T, K = idx.shape
    E = int(num_experts)
    flat = idx.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)

    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)

    # Stable sort: entries enumerated in (t, k) order, keyed by expert.
    valid_pos = np.flatnonzero(valid)
    order = valid_pos[np.argsort(flat[valid_pos], kind="stable")]

    slot = np.full(T * K, -1, dtype=np.int64)
    slot[order] = np.arange(order.size, dtype=np.int64)
    src = np.full(T * K, -1, dtype=np.int64)
    src[: order.size] = order // K
    return (counts.astype(np.int32), offsets.astype(np.int32),
            slot.reshape(T, K).astype(np.int32), src.astype(np.int32))


def dispatch_layout_padded(topk_idx, num_experts, capacity):
    """Low-latency (padded) layout: expert e owns rows e*capacity ..
    (e+1)*capacity - 1 of the receive buffer.

    [P4 "推理解码阶段的应用"]: the low-latency buffer is sized
    num_max_tokens * hidden * num_experts, i.e. a fixed per-expert capacity
    of num_max_tokens rows, and the low-latency dispatch reports the number
    of tokens each expert received (recv_expert_count).  Reading taken: the
    entry's rank inside its expert is the same stable (t, k) rank as in
    ``dispatch_layout``; its row is e*capacity + rank.  The pages give no
    overflow rule; here an entry whose rank is >= capacity is dropped
    (slot -1, skipped by dispatch and combine) and recv_expert_count[e] =
    min(count, capacity).  With capacity >= T and distinct experts per token
    nothing is ever dropped.

    Returns
      recv_count int32[E]          rows used in each expert's block
      slot       int32[T, K]       receive row of (t, k), or -1
      src        int32[E*capacity] token of each used row; -1 elsewhere (the
                 GPU path leaves unused rows untouched; compare used rows)
    """
    idx = np.asarray(topk_idx)
    T, K = idx.shape
    E, cap = int(num_experts), int(capacity)
    counts, offsets, slot_packed, _ = dispatch_layout(idx, E)
    flat = idx.reshape(-1).astype(np.int64)
    sp = slot_packed.reshape(-1).astype(np.int64)
    valid = sp >= 0
    rank = np.where(valid, sp - offsets[np.clip(flat, 0, E - 1)], 0)
    keep = valid & (rank < cap)
    slot = np.where(keep, np.clip(flat, 0, E - 1) * cap + rank, -1)
    src = np.full(E * cap, -1, dtype=np.int64)
    pos = np.flatnonzero(keep)
    src[slot[pos]] = pos // K
    recv_count = np.minimum(counts.astype(np.int64), cap)
    return recv_count.astype(np.int32), slot.reshape(T, K).astype(np.int32), src.astype(np.int32)


def group_scales(xf):
    """One FP32 scale per (token, 128-channel group).

    [P1 "DeepEP 的核心功能"] dispatch supports FP8 in the manner of the
    DeepSeek-V3 technical report; the pages do not give the granularity or
    the formula.  Reading taken: a = max |x| over the group (exact in
    binary32), s = RN32(a / 448) so that the largest element maps to the
    top of the E4M3 range.  Two degenerate groups need a rule the pages do
    not give: an all-zero group gets s = 1 (its codes are signed zeros), and
    a group so small that a / 448 would be subnormal gets s = 2**-126, the
    smallest normal binary32, so no scale is ever subnormal or zero.

    xf: float32[T, H] with H a multiple of 128.  Returns (amax, s) as
    float32[T, H/128].
    """
    T, H = xf.shape
    g = xf.reshape(T, H // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2).astype(np.float32)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s = np.where(s < SCALE_FLOOR, SCALE_FLOOR, s).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    return amax, s


def quantize_tokens_fp8(x_bits):
    """Per-token FP8 E4M3 codes and scales (before the fan-out to rows).

    q[t, c] = E4M3_RNE_sat(RN32(f32(x[t, c]) / s[t, c // 128])).  The
    division is one correctly rounded binary32 division; its result is then
    rounded once more to E4M3.  Returns (q uint8[T, H], s float32[T, G]).
    """
    xb = np.asarray(x_bits, dtype=np.uint16)
    T, H = xb.shape
    if H % GROUP:
        raise ValueError("hidden size must be a multiple of 128 for FP8")
    xf = bf16_bits_to_f32(xb)
    _, s = group_scales(xf)
    v = (xf.reshape(T, H // GROUP, GROUP) / s[:, :, None]).astype(np.float32)
    q = f32_to_e4m3_rne_sat(v).reshape(T, H)
    return q, s


def _fan_out(rows_out, per_token, slot):
    """rows_out[slot[t, k]] = per_token[t] for every unmasked (t, k)."""
    T, K = slot.shape
    for k in range(K):
        r = slot[:, k].astype(np.int64)
        m = r >= 0
        rows_out[r[m]] = per_token[m]


def dispatch_fp8(x_bits, slot, num_rows=None, topk_weights=None):
    """FP8 dispatch: permute tokens into expert-major rows, cast to E4M3.

    [P1 "DeepEP 的常规内核和低延迟内核"] dispatch sends each token to the
    experts it is routed to, in FP8; on one device the "send" is the copy
    of token t into receive row slot[t, k] for each of its K experts.  Each
    copy carries the token's codes and its per-group scales; optionally the
    routing weight of that (t, k) entry rides along ([P4 "使用示例 › MoE 训练
    中的应用"]: dispatch also returns the received routing weights).

    Rows that no entry maps to are returned as zeros here (the GPU path
    leaves them untouched); callers compare only rows < offsets[E].

    Returns (recv uint8[R, H], recv_scale float32[R, G], recv_weight
    float32[R] or None).
    """
    q, s = quantize_tokens_fp8(x_bits)
    slot = np.asarray(slot)
    T, K = slot.shape
    H = q.shape[1]
    R = T * K if num_rows is None else int(num_rows)
    recv = np.zeros((R, H), dtype=np.uint8)
    recv_scale = np.zeros((R, H // GROUP), dtype=np.float32)
    _fan_out(recv, q, slot)
    _fan_out(recv_scale, s, slot)
    recv_weight = None
    if topk_weights is not None:
        w = np.asarray(topk_weights, dtype=np.float32)
        recv_weight = np.zeros(R, dtype=np.float32)
        for k in range(K):
            r = slot[:, k].astype(np.int64)
            m = r >= 0
            recv_weight[r[m]] = w[m, k]
    return recv, recv_scale, recv_weight


def dispatch_bf16(x_bits, slot, num_rows=None):
    """BF16 dispatch: the same permutation with the token bits copied as-is."""
    xb = np.asarray(x_bits, dtype=np.uint16)
    slot = np.asarray(slot)
    T, K = slot.shape
    R = T * K if num_rows is None else int(num_rows)
    recv = np.zeros((R, xb.shape[1]), dtype=np.uint16)
    _fan_out(recv, xb, slot)
    return recv


def combine(y_bits, slot, topk_weights):
    """Combine: gather each token's K expert rows and reduce them to BF16.

    [P5 "典型工作流程"] combine reduces the expert outputs back to where the
    tokens came from; [P1 "DeepEP 的常规内核和低延迟内核"] the merge is in
    BF16.  The pages do not fix the arithmetic.  Reading taken: the weights
    are applied here as a weighted sum, accumulated in binary32 in
    ascending k, each product rounded before it is added (no fused
    multiply-add), starting from +0.0, and the sum rounded once to BF16:

        acc = +0.0
        for k = 0 .. K-1 with slot[t, k] >= 0:
            acc = RN32(acc + RN32(w[t, k] * f32(y[slot[t, k], c])))
        out[t, c] = BF16_RNE(acc)

    y_bits: uint16[>=R, H] receive-row-ordered expert outputs; slot:
    int32[T, K]; topk_weights: float32[T, K].  Returns uint16[T, H].
    """
    yb = np.asarray(y_bits, dtype=np.uint16)
    slot = np.asarray(slot)
    w = np.asarray(topk_weights, dtype=np.float32)
    T, K = slot.shape
    H = yb.shape[1]
    acc = np.zeros((T, H), dtype=np.float32)
    for k in range(K):
        r = slot[:, k].astype(np.int64)
        m = r >= 0
        yk = bf16_bits_to_f32(yb[r[m]])
        p = (w[m, k][:, None] * yk).astype(np.float32)
        acc[m] = (acc[m] + p).astype(np.float32)
    return f32_to_bf16_rne(acc)


def dequantize_rows(recv, recv_scale):
    """An identity expert on FP8 rows: y = BF16_RNE(f32(q) * s).

    Used by the round-trip invariant (dispatch -> identity expert ->
    combine with weights summing to 1 reproduces x within the FP8 bound).
    """
    R, H = recv.shape
    qf = e4m3_to_f32(recv).reshape(R, H // GROUP, GROUP)
    y = (qf * np.asarray(recv_scale, dtype=np.float32)[:, :, None]).astype(np.float32)
    return f32_to_bf16_rne(y.reshape(R, H))


# ---- backward helpers --------------------------------------------------------
# [P5 "典型工作流程"]: besides combine, the library offers backward helper
# functions for training.  The pages give no arithmetic for them; the
# readings below follow the forward definitions.

def dispatch_backward(grad_recv_bits, slot):
    """Gradient of dispatch w.r.t. x: the K copies' gradients summed.

    Dispatch copies token t into K rows, so d x[t] = sum_k d recv[slot[t,k]]
    (the FP8 cast is passed straight through).  Same arithmetic as combine
    with unit weights: binary32, ascending k, from +0.0, BF16 RNE.
    """
    slot = np.asarray(slot)
    return combine(grad_recv_bits, slot, np.ones(slot.shape, dtype=np.float32))


def dot_rn32(a, b):
    """The dot product of two BF16-valued vectors, rounded once to binary32.

    Every product of two BF16 values is exact in binary64 (8-bit
    significands give a 16-bit product, far inside binary64's range), and
    math.fsum returns the binary64 value nearest the exact sum of its
    terms.  Rounding that to binary32 is a second rounding, which differs
    from rounding the exact sum only where the binary64 value lies exactly
    halfway between two binary32 values while the exact sum does not; the
    sign of the exact remainder (another fsum) then picks the neighbour.
    An exact zero sum is +0.0.
    """
    p = (np.asarray(a, dtype=np.float64) * np.asarray(b, dtype=np.float64)).tolist()
    s = math.fsum(p)
    if s == 0.0:
        return np.float32(0.0)
    r = np.float32(s)
    lo = r if float(r) <= s else np.nextafter(r, np.float32(-np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    if (float(lo) + float(hi)) / 2.0 == s:  # a binary32 midpoint: the exact remainder decides
        rem = math.fsum(p + [-s])
        if rem > 0:
            r = hi
        elif rem < 0:
            r = lo
    return np.float32(r)


def combine_backward(grad_out_bits, y_bits, slot, topk_weights, num_rows=None):
    """Gradients of combine w.r.t. the expert outputs y and the weights.

    combine computes out[t] = sum_k w[t,k] * y[slot[t,k]], so
      grad_y[slot[t,k], c] = BF16_RNE(RN32(w[t,k] * grad_out[t,c]))
      grad_w[t,k]          = RN32(sum_c grad_out[t,c] * y[slot[t,k], c])
    grad_y is the forward product rounded as combine rounds its products,
    then to BF16 like every row the library writes.  grad_w is the dot
    product itself, exact and rounded once to binary32 (``dot_rn32``): the
    pages fix no order for it, so the oracle takes none.  Masked entries
    (slot -1) get grad_w = +0.0 and no grad_y row; grad_y rows no entry
    maps to are returned as zeros (the GPU leaves them untouched).

    Returns (grad_y uint16[num_rows, H], grad_w float32[T, K]).
    """
    g = bf16_bits_to_f32(np.asarray(grad_out_bits, dtype=np.uint16))
    yb = np.asarray(y_bits, dtype=np.uint16)
    slot = np.asarray(slot)
    w = np.asarray(topk_weights, dtype=np.float32)
    T, K = slot.shape
    H = g.shape[1]
    R = T * K if num_rows is None else int(num_rows)
    grad_y = np.zeros((R, H), dtype=np.uint16)
    grad_w = np.zeros((T, K), dtype=np.float32)
    for k in range(K):
        r = slot[:, k].astype(np.int64)
        m = r >= 0
        gy = (w[m, k][:, None] * g[m]).astype(np.float32)
        grad_y[r[m]] = f32_to_bf16_rne(gy)
    for t in range(T):
        for k in range(K):
            if slot[t, k] >= 0:
                grad_w[t, k] = dot_rn32(g[t], bf16_bits_to_f32(yb[slot[t, k]]))
    return grad_y, grad_w
