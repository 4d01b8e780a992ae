"""Run the three C-ABI calls on the GPU through the binding (test helper).

Outputs are pre-filled with sentinels so that rows the kernels must not
touch, and rows they forget, both show up.
"""

import numpy as np
import torch

SENT_I32 = -7
SENT_U8 = 0xA5
SENT_F32 = -12345.0
SENT_BF16 = 0x7FA5  # a NaN pattern no kernel writes


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def gpu_layout(ep, idx, E, misalign=False):
    """misalign: pass topk_idx 4 bytes past a 16-byte boundary."""
    T, K = idx.shape
    if misalign:
        flat = np.concatenate([np.zeros(1, np.int32), idx.astype(np.int32).ravel()])
        d_idx = to_dev(flat)[1:].view(T, K)
        assert d_idx.data_ptr() % 16 == 4
    else:
        d_idx = to_dev(idx.astype(np.int32))
    counts = torch.full((E,), SENT_I32, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), SENT_I32, dtype=torch.int32, device="cuda")
    slot = torch.full((T, K), SENT_I32, dtype=torch.int32, device="cuda")
    src = torch.full((T * K,), SENT_I32, dtype=torch.int32, device="cuda")
    nb = ep.ep_layout_workspace_bytes(T, K, E)
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda") if nb else None
    ep.ep_dispatch_layout(d_idx, E, counts, offsets, slot, src, ws)
    return counts, offsets, slot, src


def gpu_dispatch(ep, x_bits, slot, w=None, fp8=True, with_weight=True):
    T, H = x_bits.shape
    K = slot.shape[1]
    d_x = to_dev(x_bits.view(np.int16), None) if isinstance(x_bits, np.ndarray) else x_bits
    d_w = to_dev(w.astype(np.float32)) if w is not None else None
    rw = torch.full((T * K,), SENT_F32, dtype=torch.float32, device="cuda") if (with_weight and w is not None) else None
    if fp8:
        recv = torch.full((T * K, H), SENT_U8, dtype=torch.uint8, device="cuda")
        scale = torch.full((T * K, H // 128), SENT_F32, dtype=torch.float32, device="cuda")
        ep.ep_dispatch(d_x, slot, d_w, ep.EP_RECV_FP8_E4M3_G128, recv, scale, rw)
        return recv, scale, rw
    recv = torch.full((T * K, H), SENT_BF16, dtype=torch.int16, device="cuda")
    ep.ep_dispatch(d_x, slot, d_w, ep.EP_RECV_BF16, recv, None, rw)
    return recv, None, rw


def gpu_combine(ep, y, slot, w):
    T, K = slot.shape
    d_y = to_dev(y.view(np.int16)) if isinstance(y, np.ndarray) else y
    d_w = to_dev(w.astype(np.float32)) if isinstance(w, np.ndarray) else w
    out = torch.full((T, d_y.shape[1]), SENT_BF16, dtype=torch.int16, device="cuda")
    ep.ep_combine(d_y, slot, d_w, out)
    return out


def host(t):
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a
