"""MoE token dispatch / combine for one MI355X (gfx950).

The kernels live in libep.so (HIP, built by ``combine_ep_dispatch_amd.build``)
behind the C ABI of include/ep.h; this package is a thin ctypes binding
with the same entry-point names.  Importing it raises ImportError when the
library has not been built.
"""

from ._lib import (  # noqa: F401
    EP_ERR_HIP,
    EP_ERR_INVALID_ARG,
    EP_ERR_UNSUPPORTED,
    EP_MAX_EXPERTS,
    EP_MAX_TOPK,
    EP_NOALLOC_SCRATCH_BYTES,
    EP_OK,
    EP_RECV_BF16,
    EP_RECV_FP8_E4M3_G128,
    LIB,
    LIB_PATH,
    EpError,
)
from .api import (  # noqa: F401
    Handle,
    PaddedHandle,
    combine,
    combine_backward,
    dispatch,
    dispatch_backward,
    ep_cast_fp8_e4m3,
    ep_combine,
    ep_combine_backward,
    ep_dispatch_backward,
    ep_dispatch,
    ep_dispatch_layout,
    ep_dispatch_layout_padded,
    ep_layout_dispatch,
    ep_layout_dispatch_noalloc,
    ep_layout_workspace_bytes,
    layout,
    layout_padded,
    low_latency_combine,
    low_latency_dispatch,
)
from .plan import StepPlan  # noqa: F401
