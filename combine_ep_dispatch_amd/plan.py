"""Pre-validated launches for a fixed set of buffers.

A serving loop calls layout -> dispatch -> combine on the same buffers every
step.  ``StepPlan`` checks dtypes, shapes and devices once, allocates the
layout workspace once, and has the library check the raw arguments once
into an ``ep_step_plan`` (C storage held here), so a step costs two C calls
of one pointer argument each: layout+dispatch and combine.
The kernels are the same ones the ``ep_*`` functions launch.
"""

import ctypes

import torch

from . import api
from ._lib import EP_RECV_BF16, EP_RECV_FP8_E4M3_G128, LIB, STEP_PLAN_WORDS, check


class StepPlan:
    """One MoE step's buffers: routing, tokens, receive rows, expert outputs
    and the combined output.

    topk_idx int32 or int64 [T, K]; topk_weights float32 [T, K]; x bf16 [T, H];
    capacity 0 for the packed layout (T*K receive rows) or the rows per
    expert of the low-latency layout (E*capacity rows); fp8 selects the
    receive format.  y (expert outputs, bf16 [rows, H]) defaults to a new
    tensor; all other buffers are allocated here.  The stream is fixed at
    construction (the current stream by default).  To replay a step as a
    HIP graph, build the plan on a side stream and capture on it:
    ``torch.cuda.graph(g, stream=that_stream)``; the plan's input tensors
    can be refilled between replays.  The library keeps no state, so plans
    on different streams may run at the same time.
    """

    def __init__(self, topk_idx, topk_weights, x, num_experts, capacity=0, fp8=True, y=None, stream=None):
        api._need(topk_idx, "topk_idx", api._IDX)
        if topk_idx.dim() != 2:
            raise ValueError("topk_idx must be [T, K]")
        T, K = topk_idx.shape
        api._need(topk_weights, "topk_weights", (torch.float32,), (T, K))
        api._need(x, "x", (torch.bfloat16, torch.int16, torch.uint16))
        if x.dim() != 2 or x.shape[0] != T:
            raise ValueError("x must be [T, H]")
        H = x.shape[1]
        E = int(num_experts)
        if fp8 and H % 128:
            raise ValueError("FP8 dispatch needs hidden % 128 == 0")
        if int(capacity) < 0:
            raise ValueError("capacity must be >= 0")
        self.T, self.H, self.K, self.E, self.capacity = T, H, K, E, int(capacity)
        rows = E * self.capacity if self.capacity else T * K
        self.rows = rows
        dev = x.device
        self.topk_idx, self.topk_weights, self.x = topk_idx, topk_weights, x
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.slot = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.src = torch.empty(rows, dtype=torch.int32, device=dev)
        nb = api.ep_layout_workspace_bytes(T, K, E)
        self.workspace = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        self.fmt = EP_RECV_FP8_E4M3_G128 if fp8 else EP_RECV_BF16
        if fp8:
            self.recv_x = torch.empty((rows, H), dtype=torch.uint8, device=dev)
            self.recv_scale = torch.empty((rows, H // 128), dtype=torch.float32, device=dev)
        else:
            self.recv_x = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
            self.recv_scale = None
        self.y = y if y is not None else torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
        api._need(self.y, "y", (torch.bfloat16, torch.int16, torch.uint16), (rows, H))
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.stream = api._stream(stream)

        # the three-call form's entry points for these ids, and argument
        # tuples built once; the C side still checks them on every call
        self._fn_layout = api._ids_fn("ep_dispatch_layout", topk_idx)
        self._fn_layout_padded = api._ids_fn("ep_dispatch_layout_padded", topk_idx)
        self._layout_args = self._make_layout_args()
        self._dispatch_args = (x.data_ptr(), T, H, K, self.slot.data_ptr(), None, self.fmt, self.recv_x.data_ptr(),
                               self.recv_scale.data_ptr() if self.recv_scale is not None else None, None,
                               self.stream)
        ws = self.workspace
        # the library's own plan of the two per-step launches
        self._plan = (ctypes.c_uint64 * STEP_PLAN_WORDS)()
        self._plan_ptr = ctypes.c_void_p(ctypes.addressof(self._plan))
        check("ep_step_plan_init", LIB.ep_step_plan_init(
            self._plan_ptr, topk_idx.data_ptr(), topk_idx.element_size(), x.data_ptr(), topk_weights.data_ptr(), T,
            H, K, E, self.capacity, self.fmt, self.counts.data_ptr(),
            None if self.capacity else self.offsets.data_ptr(), self.slot.data_ptr(), self.src.data_ptr(),
            self.recv_x.data_ptr(), self.recv_scale.data_ptr() if self.recv_scale is not None else None, None,
            ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0, self.y.data_ptr(),
            self.out.data_ptr(), self.stream))
        self._plan_layout_dispatch = LIB.ep_step_plan_layout_dispatch
        self._plan_combine = LIB.ep_step_plan_combine

    def _make_layout_args(self):
        ws = self.workspace
        ws_ptr = ws.data_ptr() if ws is not None else None
        ws_bytes = ws.numel() if ws is not None else 0
        if self.capacity:
            return (True, (self.topk_idx.data_ptr(), self.T, self.K, self.E, self.capacity, self.counts.data_ptr(),
                           self.slot.data_ptr(), self.src.data_ptr(), ws_ptr, ws_bytes, self.stream))
        return (False, (self.topk_idx.data_ptr(), self.T, self.K, self.E, self.counts.data_ptr(),
                        self.offsets.data_ptr(), self.slot.data_ptr(), self.src.data_ptr(), ws_ptr, ws_bytes,
                        self.stream))

    def layout(self):
        padded, args = self._layout_args
        if padded:
            check("ep_dispatch_layout_padded", self._fn_layout_padded(*args))
        else:
            check("ep_dispatch_layout", self._fn_layout(*args))

    def dispatch(self):
        check("ep_dispatch", LIB.ep_dispatch(*self._dispatch_args))

    def layout_dispatch(self):
        """layout() and dispatch() as one call (one launch up to 65536 entries)."""
        status = self._plan_layout_dispatch(self._plan_ptr)
        if status:
            check("ep_step_plan_layout_dispatch", status)

    def combine(self):
        status = self._plan_combine(self._plan_ptr)
        if status:
            check("ep_step_plan_combine", status)

    def step(self):
        """layout_dispatch() then combine(), with no Python call between the
        two launches (at decode sizes the host's submit time paces a step)."""
        status = self._plan_layout_dispatch(self._plan_ptr)
        if status:
            check("ep_step_plan_layout_dispatch", status)
        status = self._plan_combine(self._plan_ptr)
        if status:
            check("ep_step_plan_combine", status)
