"""Python face of the C ABI: the same three calls, taking torch tensors.

Each ``ep_*`` function checks dtypes, devices, shapes and contiguity (the C
side trusts buffer sizes), then passes raw device pointers and the current
HIP stream to libep.so.  Every step of the computation runs in the
library's kernels; torch only owns the memory and the stream.

``dispatch`` / ``combine`` mirror the pages' call shape
``dispatch(x, topk_idx, topk_weights, num_experts)`` returning received rows
and a handle, and ``combine(...)`` reducing back ([P4] "使用示例 › MoE 训练中
的应用"; [P5] "典型工作流程").
"""

import os
from collections import namedtuple

import torch

from ._lib import (EP_MAX_EXPERTS, EP_MAX_TOPK, EP_RECV_BF16, EP_RECV_FP8_E4M3_G128, LIB, check)

Handle = namedtuple("Handle", "tokens_per_expert expert_offset slot src_token num_experts")
# low-latency (padded) handle: expert e owns rows e*capacity .. e*capacity+capacity-1
PaddedHandle = namedtuple("PaddedHandle", "recv_expert_count slot src_token num_experts capacity")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# EP_DEBUG_CHECK=1: reject expert ids outside [-1, E) before launching.  The
# kernels mask every id outside [0, E), so such ids are legal; an id other
# than -1 out there is usually a caller bug.  The check reads the ids'
# range back to the host (a synchronisation), so it is off by default.
DEBUG_CHECK = os.environ.get("EP_DEBUG_CHECK") == "1"


def _debug_check_ids(topk_idx, num_experts):
    if not DEBUG_CHECK or topk_idx.numel() == 0:
        return
    lo, hi = int(topk_idx.min()), int(topk_idx.max())
    if lo < -1 or hi >= num_experts:
        raise ValueError("EP_DEBUG_CHECK: topk_idx holds ids in [%d, %d], outside [-1, %d)" % (lo, hi, num_experts))


def _need(t, name, dtypes, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_cuda:  # (a ROCm device tensor reports is_cuda; cheaper than t.device.type)
        raise ValueError("%s must be on a GPU device" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and t.shape != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


_I32 = (torch.int32,)
_IDX = (torch.int32, torch.int64)  # expert ids: int32, or int64 as routers produce them
_F32 = (torch.float32,)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8, torch.float8_e4m3fn)


def _ids_fn(name, topk_idx):
    """The C entry point for these ids: NAME, or NAME_i64 for int64 ids."""
    return getattr(LIB, name + "_i64") if topk_idx.dtype == torch.int64 else getattr(LIB, name)


def _as_ids(topk_idx):
    """int32 and int64 ids go to the library as they are; other integer
    types are widened to int32."""
    if topk_idx.dtype not in _IDX:
        topk_idx = topk_idx.to(torch.int32)
    return topk_idx.contiguous()


def ep_layout_workspace_bytes(num_tokens, top_k, num_experts):
    """Bytes of device workspace the layout calls need for this shape (0 up
    to 65536 entries, T*K)."""
    return int(LIB.ep_layout_workspace_bytes(int(num_tokens), int(top_k), int(num_experts)))


def ep_dispatch_layout(topk_idx, num_experts, tokens_per_expert, expert_offset, slot, src_token,
                       workspace=None, stream=None):
    """Routing layout into caller-owned int32 tensors: tokens_per_expert [E],
    expert_offset [E+1] (exclusive scan), slot [T, K] (receive row of entry
    (t, k), -1 if masked), src_token [T*K] (token of each row, -1 past
    expert_offset[E]).  Rows of one expert are in ascending token order.
    workspace: uint8/int32 device tensor of ep_layout_workspace_bytes bytes
    (only needed past 65536 entries)."""
    _need(topk_idx, "topk_idx", _IDX)
    _debug_check_ids(topk_idx, num_experts)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, K]")
    T, K = topk_idx.shape
    E = int(num_experts)
    _need(tokens_per_expert, "tokens_per_expert", _I32, (E,))
    _need(expert_offset, "expert_offset", _I32, (E + 1,))
    _need(slot, "slot", _I32, (T, K))
    _need(src_token, "src_token", _I32, (T * K,))
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8, torch.int32))
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check("ep_dispatch_layout", _ids_fn("ep_dispatch_layout", topk_idx)(
        topk_idx.data_ptr(), T, K, E, tokens_per_expert.data_ptr(), expert_offset.data_ptr(),
        slot.data_ptr(), src_token.data_ptr(), ws_ptr, ws_bytes, _stream(stream)))


def ep_dispatch_layout_padded(topk_idx, num_experts, capacity, recv_expert_count, slot, src_token,
                              workspace=None, stream=None):
    """Low-latency layout: expert e owns rows e*capacity .. e*capacity +
    capacity - 1; recv_expert_count [E] = min(count, capacity), slot [T, K]
    (-1 for masked or dropped entries), src_token [E*capacity] (unused rows
    are not written)."""
    _need(topk_idx, "topk_idx", _IDX)
    _debug_check_ids(topk_idx, num_experts)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, K]")
    T, K = topk_idx.shape
    E, cap = int(num_experts), int(capacity)
    _need(recv_expert_count, "recv_expert_count", _I32, (E,))
    _need(slot, "slot", _I32, (T, K))
    _need(src_token, "src_token", _I32, (E * cap,))
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8, torch.int32))
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check("ep_dispatch_layout_padded", _ids_fn("ep_dispatch_layout_padded", topk_idx)(
        topk_idx.data_ptr(), T, K, E, cap, recv_expert_count.data_ptr(), slot.data_ptr(), src_token.data_ptr(),
        ws_ptr, ws_bytes, _stream(stream)))


def ep_dispatch(x, slot, topk_weights, format, recv_x, recv_scale=None, recv_weight=None, stream=None,
                num_rows=None):
    """Copy every token x [T, H] (bf16) into its K receive rows given by slot:
    EP_RECV_FP8_E4M3_G128 writes E4M3FN codes to recv_x (uint8 [rows, H])
    and one float32 scale per 128 channels to recv_scale [rows, H/128];
    EP_RECV_BF16 copies the bf16 bits to recv_x (bf16 [rows, H]).
    recv_weight [rows] (optional) receives topk_weights[t, k].  num_rows:
    rows of the receive buffers (T*K by default; E*capacity for a padded
    slot)."""
    _need(x, "x", _BF16)
    if x.dim() != 2:
        raise ValueError("x must be [T, H]")
    T, H = x.shape
    _need(slot, "slot", _I32)
    if slot.dim() != 2 or slot.shape[0] != T:
        raise ValueError("slot must be [T, K]")
    K = slot.shape[1]
    R = T * K if num_rows is None else int(num_rows)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", _F32, (T, K))
    if format == EP_RECV_FP8_E4M3_G128:
        _need(recv_x, "recv_x", _U8, (R, H))
        if H % 128:
            raise ValueError("FP8 dispatch needs hidden % 128 == 0")
        _need(recv_scale, "recv_scale", _F32, (R, H // 128))
    elif format == EP_RECV_BF16:
        _need(recv_x, "recv_x", _BF16, (R, H))
    else:
        raise ValueError("unknown receive format %r" % (format,))
    if recv_weight is not None:
        _need(recv_weight, "recv_weight", _F32, (R,))
    check("ep_dispatch", LIB.ep_dispatch(
        x.data_ptr(), T, H, K, slot.data_ptr(),
        topk_weights.data_ptr() if topk_weights is not None else None, int(format), recv_x.data_ptr(),
        recv_scale.data_ptr() if recv_scale is not None else None,
        recv_weight.data_ptr() if recv_weight is not None else None, _stream(stream)))


def _check_layout_dispatch(topk_idx, x, topk_weights, num_experts, capacity, format, tokens_per_expert,
                           expert_offset, slot, src_token, recv_x, recv_scale, recv_weight):
    """Shape and dtype checks of ep_layout_dispatch's tensors; returns T, H, K."""
    _need(topk_idx, "topk_idx", _IDX)
    _debug_check_ids(topk_idx, num_experts)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, K]")
    T, K = topk_idx.shape
    E, cap = int(num_experts), int(capacity)
    if cap < 0:
        raise ValueError("capacity must be >= 0")
    R = E * cap if cap else T * K
    _need(x, "x", _BF16)
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, H]")
    H = x.shape[1]
    _need(tokens_per_expert, "tokens_per_expert", _I32, (E,))
    if cap == 0:
        _need(expert_offset, "expert_offset", _I32, (E + 1,))
    elif expert_offset is not None:
        raise ValueError("expert_offset is not used by the padded layout; pass None")
    _need(slot, "slot", _I32, (T, K))
    _need(src_token, "src_token", _I32, (R,))
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", _F32, (T, K))
    if format == EP_RECV_FP8_E4M3_G128:
        if H % 128:
            raise ValueError("FP8 dispatch needs hidden % 128 == 0")
        _need(recv_x, "recv_x", _U8, (R, H))
        _need(recv_scale, "recv_scale", _F32, (R, H // 128))
    elif format == EP_RECV_BF16:
        _need(recv_x, "recv_x", _BF16, (R, H))
    else:
        raise ValueError("unknown receive format %r" % (format,))
    if recv_weight is not None:
        _need(recv_weight, "recv_weight", _F32, (R,))
    return T, H, K


def ep_layout_dispatch(topk_idx, x, topk_weights, num_experts, capacity, format, tokens_per_expert,
                       expert_offset, slot, src_token, recv_x, recv_scale=None, recv_weight=None, workspace=None,
                       stream=None):
    """Layout and dispatch in one call (one launch up to 65536 entries).
    capacity 0: packed layout (expert_offset [E+1], src_token [T*K], T*K
    receive rows); capacity > 0: padded layout (expert_offset None,
    src_token [E*capacity], E*capacity receive rows)."""
    T, H, K = _check_layout_dispatch(topk_idx, x, topk_weights, num_experts, capacity, format, tokens_per_expert,
                                     expert_offset, slot, src_token, recv_x, recv_scale, recv_weight)
    E, cap = int(num_experts), int(capacity)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8, torch.int32))
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check("ep_layout_dispatch", _ids_fn("ep_layout_dispatch", topk_idx)(
        topk_idx.data_ptr(), x.data_ptr(), topk_weights.data_ptr() if topk_weights is not None else None, T, H, K,
        E, cap, int(format), tokens_per_expert.data_ptr(),
        expert_offset.data_ptr() if expert_offset is not None else None, slot.data_ptr(), src_token.data_ptr(),
        recv_x.data_ptr(), recv_scale.data_ptr() if recv_scale is not None else None,
        recv_weight.data_ptr() if recv_weight is not None else None, ws_ptr, ws_bytes, _stream(stream)))


def ep_layout_dispatch_noalloc(topk_idx, x, topk_weights, num_experts, capacity, format, tokens_per_expert,
                               expert_offset, slot, src_token, recv_x, recv_scale=None, recv_weight=None,
                               stream=None):
    """ep_layout_dispatch without a workspace: the library's own per-GPU
    scratch (EP_NOALLOC_SCRATCH_BYTES) holds the layout's histograms, so the
    call allocates nothing.  int32 ids only.  Calls that overlap on one GPU
    race on that scratch; issue them on one stream."""
    if topk_idx.dtype != torch.int32:
        raise TypeError("ep_layout_dispatch_noalloc takes int32 topk_idx")
    T, H, K = _check_layout_dispatch(topk_idx, x, topk_weights, num_experts, capacity, format, tokens_per_expert,
                                     expert_offset, slot, src_token, recv_x, recv_scale, recv_weight)
    check("ep_layout_dispatch_noalloc", LIB.ep_layout_dispatch_noalloc(
        topk_idx.data_ptr(), x.data_ptr(), topk_weights.data_ptr() if topk_weights is not None else None, T, H, K,
        int(num_experts), int(capacity), int(format), tokens_per_expert.data_ptr(),
        expert_offset.data_ptr() if expert_offset is not None else None, slot.data_ptr(), src_token.data_ptr(),
        recv_x.data_ptr(), recv_scale.data_ptr() if recv_scale is not None else None,
        recv_weight.data_ptr() if recv_weight is not None else None, _stream(stream)))


def ep_combine(y, slot, topk_weights, out, stream=None, num_rows=None):
    """out[t] = BF16(sum over k of topk_weights[t, k] * y[slot[t, k]]), in
    binary32, ascending k, each product rounded before it is added.
    y: bf16 [rows, H] in receive order; out: bf16 [T, H].  num_rows: rows
    of y (T*K by default; E*capacity for a padded slot)."""
    _need(slot, "slot", _I32)
    if slot.dim() != 2:
        raise ValueError("slot must be [T, K]")
    T, K = slot.shape
    _need(y, "y", _BF16)
    R = T * K if num_rows is None else int(num_rows)
    if y.dim() != 2 or y.shape[0] != R:
        raise ValueError("y must be [%d, H]" % R)
    H = y.shape[1]
    _need(topk_weights, "topk_weights", _F32, (T, K))
    _need(out, "out", _BF16, (T, H))
    check("ep_combine", LIB.ep_combine(y.data_ptr(), slot.data_ptr(), topk_weights.data_ptr(), T, H, K,
                                       out.data_ptr(), _stream(stream)))


def ep_dispatch_backward(grad_recv, slot, grad_x, stream=None, num_rows=None):
    """grad_x [T, H] = sum over k of grad_recv[slot[t, k]] (bf16)."""
    _need(slot, "slot", _I32)
    if slot.dim() != 2:
        raise ValueError("slot must be [T, K]")
    T, K = slot.shape
    _need(grad_recv, "grad_recv", _BF16)
    R = T * K if num_rows is None else int(num_rows)
    if grad_recv.dim() != 2 or grad_recv.shape[0] != R:
        raise ValueError("grad_recv must be [%d, H]" % R)
    H = grad_recv.shape[1]
    _need(grad_x, "grad_x", _BF16, (T, H))
    check("ep_dispatch_backward", LIB.ep_dispatch_backward(grad_recv.data_ptr(), slot.data_ptr(), T, H, K,
                                                           grad_x.data_ptr(), _stream(stream)))


def ep_combine_backward(grad_out, y, slot, topk_weights, grad_y, grad_w=None, stream=None, num_rows=None):
    """grad_y rows = w * grad_out (bf16); grad_w [T, K] = row dot products
    (float32), or skipped when grad_w is None (y may then be None)."""
    _need(slot, "slot", _I32)
    if slot.dim() != 2:
        raise ValueError("slot must be [T, K]")
    T, K = slot.shape
    _need(grad_out, "grad_out", _BF16)
    if grad_out.dim() != 2 or grad_out.shape[0] != T:
        raise ValueError("grad_out must be [T, H]")
    H = grad_out.shape[1]
    R = T * K if num_rows is None else int(num_rows)
    _need(topk_weights, "topk_weights", _F32, (T, K))
    _need(grad_y, "grad_y", _BF16, (R, H))
    if grad_w is not None:
        _need(y, "y", _BF16, (R, H))
        _need(grad_w, "grad_w", _F32, (T, K))
    check("ep_combine_backward", LIB.ep_combine_backward(
        grad_out.data_ptr(), y.data_ptr() if y is not None else None, slot.data_ptr(), topk_weights.data_ptr(),
        T, H, K, grad_y.data_ptr(), grad_w.data_ptr() if grad_w is not None else None, _stream(stream)))


def ep_cast_fp8_e4m3(inp, out, stream=None):
    """The binary32 -> E4M3FN conversion dispatch uses (round to nearest
    even, saturating at +-448), elementwise: inp float32, out uint8 of the
    same shape."""
    _need(inp, "in", _F32)
    _need(out, "out", _U8, tuple(inp.shape))
    check("ep_cast_fp8_e4m3", LIB.ep_cast_fp8_e4m3(inp.data_ptr(), out.data_ptr(), inp.numel(),
                                                   _stream(stream)))


# ---- convenience wrappers that allocate their outputs ----------------------

def layout(topk_idx, num_experts, stream=None):
    """Routing layout of ``topk_idx`` [T, K] (int32 or int64) -> Handle."""
    topk_idx = _as_ids(topk_idx)
    T, K = topk_idx.shape
    E = int(num_experts)
    if not 1 <= E <= EP_MAX_EXPERTS or not 1 <= K <= EP_MAX_TOPK:
        raise ValueError("unsupported num_experts=%d / top_k=%d" % (E, K))
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = torch.empty(T * K, dtype=torch.int32, device=dev)
    nb = ep_layout_workspace_bytes(T, K, E)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    ep_dispatch_layout(topk_idx, E, counts, offsets, slot, src, ws, stream)
    return Handle(counts, offsets, slot, src, E)


def dispatch(x, topk_idx, topk_weights, num_experts, fp8=True, handle=None, stream=None):
    """Permute tokens into expert-major rows.

    Returns (recv_x, recv_scale, recv_weight, handle): recv_x is uint8 E4M3FN
    [T*K, H] with recv_scale float32 [T*K, H/128] when ``fp8``, else bfloat16
    [T*K, H] with recv_scale None; recv_weight float32 [T*K] (None if
    ``topk_weights`` is None).  Rows expert_offset[e] .. expert_offset[e+1]-1
    belong to expert e.
    """
    T, H = x.shape
    dev = x.device
    if handle is None:
        topk_idx = _as_ids(topk_idx)
    K = handle.slot.shape[1] if handle is not None else topk_idx.shape[1]
    recv_weight = None
    if topk_weights is not None:
        topk_weights = topk_weights.to(torch.float32).contiguous()
        recv_weight = torch.empty(T * K, dtype=torch.float32, device=dev)
    fmt = EP_RECV_FP8_E4M3_G128 if fp8 else EP_RECV_BF16
    if fp8:
        recv_x = torch.empty((T * K, H), dtype=torch.uint8, device=dev)
        recv_scale = torch.empty((T * K, H // 128), dtype=torch.float32, device=dev)
    else:
        recv_x = torch.empty((T * K, H), dtype=torch.bfloat16, device=dev)
        recv_scale = None
    if handle is not None:
        ep_dispatch(x, handle.slot, topk_weights, fmt, recv_x, recv_scale, recv_weight, stream)
        return recv_x, recv_scale, recv_weight, handle
    E = int(num_experts)
    if not 1 <= E <= EP_MAX_EXPERTS or not 1 <= K <= EP_MAX_TOPK:
        raise ValueError("unsupported num_experts=%d / top_k=%d" % (E, K))
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = torch.empty(T * K, dtype=torch.int32, device=dev)
    nb = ep_layout_workspace_bytes(T, K, E)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    ep_layout_dispatch(topk_idx, x, topk_weights, E, 0, fmt, counts, offsets, slot, src, recv_x, recv_scale,
                       recv_weight, ws, stream)
    return recv_x, recv_scale, recv_weight, Handle(counts, offsets, slot, src, E)


def combine(y, handle, topk_weights, stream=None):
    """Weighted reduction of expert outputs ``y`` [T*K, H] (bf16, receive
    order) back to token order -> bfloat16 [T, H]."""
    T = handle.slot.shape[0]
    out = torch.empty((T, y.shape[1]), dtype=torch.bfloat16, device=y.device)
    ep_combine(y, handle.slot, topk_weights.to(torch.float32).contiguous(), out, stream)
    return out


def layout_padded(topk_idx, num_experts, capacity, stream=None):
    """Low-latency layout with ``capacity`` rows per expert -> PaddedHandle."""
    topk_idx = _as_ids(topk_idx)
    T, K = topk_idx.shape
    E, cap = int(num_experts), int(capacity)
    dev = topk_idx.device
    count = torch.empty(E, dtype=torch.int32, device=dev)
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = torch.empty(E * cap, dtype=torch.int32, device=dev)
    nb = ep_layout_workspace_bytes(T, K, E)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    ep_dispatch_layout_padded(topk_idx, E, cap, count, slot, src, ws, stream)
    return PaddedHandle(count, slot, src, E, cap)


def low_latency_dispatch(x, topk_idx, num_max_tokens, num_experts, fp8=True, stream=None):
    """Decode-time dispatch into a padded buffer, shaped like the pages'
    ``low_latency_dispatch(hidden_states, topk_idx, num_max_tokens,
    num_experts)`` ([P4] "使用示例 › 推理解码阶段的应用").

    Returns (recv_x [E, num_max_tokens, H], recv_scale [E, num_max_tokens,
    H/128] or None, recv_expert_count [E], handle).
    """
    topk_idx = _as_ids(topk_idx)
    T, H = x.shape
    K = topk_idx.shape[1]
    E, cap = int(num_experts), int(num_max_tokens)
    if cap < 1:
        raise ValueError("num_max_tokens must be >= 1")
    dev = x.device
    count = torch.empty(E, dtype=torch.int32, device=dev)
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = torch.empty(E * cap, dtype=torch.int32, device=dev)
    nb = ep_layout_workspace_bytes(T, K, E)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    if fp8:
        recv_x = torch.empty((E * cap, H), dtype=torch.uint8, device=dev)
        recv_scale = torch.empty((E * cap, H // 128), dtype=torch.float32, device=dev)
    else:
        recv_x = torch.empty((E * cap, H), dtype=torch.bfloat16, device=dev)
        recv_scale = None
    ep_layout_dispatch(topk_idx, x, None, E, cap, EP_RECV_FP8_E4M3_G128 if fp8 else EP_RECV_BF16, count, None,
                       slot, src, recv_x, recv_scale, None, ws, stream)
    if recv_scale is not None:
        recv_scale = recv_scale.view(E, cap, H // 128)
    return recv_x.view(E, cap, H), recv_scale, count, PaddedHandle(count, slot, src, E, cap)


def low_latency_combine(y, handle, topk_weights, stream=None):
    """Weighted reduction of padded expert outputs y [E, capacity, H] (bf16)
    back to token order -> bfloat16 [T, H]."""
    E, cap = handle.num_experts, handle.capacity
    H = y.shape[-1]
    y2 = y.reshape(E * cap, H)
    T = handle.slot.shape[0]
    out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    ep_combine(y2, handle.slot, topk_weights.to(torch.float32).contiguous(), out, stream, num_rows=E * cap)
    return out


def dispatch_backward(grad_recv, handle, stream=None):
    """Gradient of dispatch w.r.t. x: the K copies' gradients summed -> bf16 [T, H]."""
    T = handle.slot.shape[0]
    R = grad_recv.shape[0]
    out = torch.empty((T, grad_recv.shape[1]), dtype=torch.bfloat16, device=grad_recv.device)
    ep_dispatch_backward(grad_recv, handle.slot, out, stream, num_rows=R)
    return out


def combine_backward(grad_out, y, handle, topk_weights, stream=None):
    """Gradients of combine -> (grad_y bf16 [rows, H], grad_w float32 [T, K]).
    Rows no entry maps to are zero-filled first (a torch fill)."""
    T, K = handle.slot.shape
    R, H = y.shape
    grad_y = torch.zeros((R, H), dtype=torch.bfloat16, device=y.device)
    grad_w = torch.empty((T, K), dtype=torch.float32, device=y.device)
    ep_combine_backward(grad_out, y, handle.slot, topk_weights.to(torch.float32).contiguous(), grad_y, grad_w,
                        stream, num_rows=R)
    return grad_y, grad_w
