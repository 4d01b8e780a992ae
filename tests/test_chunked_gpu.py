"""ep_layout_dispatch past the decode kernel's 3072 entries, up to the
one-launch layout's 65536: the chunked kernel (each workgroup lays out and
dispatches its own tokens), against the oracle.

Bar: every output bit-exact (counts, offsets, slot, src, receive rows,
scales, received weights); rows and entries the contract leaves alone still
hold their sentinels.  Cases cover the prefill workload, both id widths with
aligned and misaligned ids (16-byte or 4-/8-byte id loads), scale buffers
that do or do not take the wavefront scale stores, top-k from 1 to 16,
1024 experts (8-wave workgroups), the padded layout with drops, masked ids,
a last workgroup with fewer tokens, and BF16.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import SENT_BF16, SENT_F32, SENT_I32, SENT_U8, host, to_dev
from workloads import make_workload, to_bf16_bits

pytestmark = pytest.mark.gpu


def dev_view(a, offset, torch_dtype):
    """`a` on the device starting `offset` elements past a 256-byte aligned
    allocation (offset 1: ids not 16-byte aligned)."""
    flat = torch.empty(a.size + offset, dtype=torch_dtype, device="cuda")
    view = flat[offset:offset + a.size].view(a.shape)
    view.copy_(torch.from_numpy(np.ascontiguousarray(a)))
    return view


def run_and_check(ep, idx, x_bits, w, E, cap=0, fp8=True, id_offset=0, scale_offset=0):
    T, K = idx.shape
    H = x_bits.shape[1]
    R = E * cap if cap else T * K
    tdt = torch.int64 if idx.dtype == np.int64 else torch.int32
    d_idx = dev_view(idx, id_offset, tdt)
    assert (d_idx.data_ptr() % 16 == 0) == (id_offset == 0)
    d_x = to_dev(x_bits.view(np.int16))
    d_w = to_dev(w.astype(np.float32)) if w is not None else None
    counts = torch.full((E,), SENT_I32, dtype=torch.int32, device="cuda")
    offsets = None if cap else torch.full((E + 1,), SENT_I32, dtype=torch.int32, device="cuda")
    slot = torch.full((T, K), SENT_I32, dtype=torch.int32, device="cuda")
    src = torch.full((R,), SENT_I32, dtype=torch.int32, device="cuda")
    nb = ep.ep_layout_workspace_bytes(T, K, E)
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda") if nb else None
    G = H // 128
    if fp8:
        recv = torch.full((R, H), SENT_U8, dtype=torch.uint8, device="cuda")
        store = torch.full((R * G + 4,), SENT_F32, dtype=torch.float32, device="cuda")
        scale = store[scale_offset:scale_offset + R * G].view(R, G)
        fmt = ep.EP_RECV_FP8_E4M3_G128
    else:
        recv = torch.full((R, H), SENT_BF16, dtype=torch.int16, device="cuda")
        store = scale = None
        fmt = ep.EP_RECV_BF16
    rw = torch.full((R,), SENT_F32, dtype=torch.float32, device="cuda") if w is not None else None
    ep.ep_layout_dispatch(d_idx, d_x, d_w, E, cap, fmt, counts, offsets, slot, src, recv, scale, rw, ws)

    if cap:
        oc, oslot, osrc = oracle.dispatch_layout_padded(idx, E, cap)
        used = (np.arange(cap)[None, :] < oc[:, None]).ravel()
        hs = host(src)
        assert np.array_equal(host(counts), oc)
        assert np.array_equal(host(slot), oslot)
        assert np.array_equal(hs[used], osrc[used]) and np.all(hs[~used] == SENT_I32)
    else:
        oc, oo, oslot, osrc = oracle.dispatch_layout(idx, E)
        used = np.arange(R) < oo[-1]
        assert np.array_equal(host(counts), oc) and np.array_equal(host(offsets), oo)
        assert np.array_equal(host(slot), oslot)
        assert np.array_equal(host(src), osrc)
    hr = host(recv)
    if fp8:
        orecv, oscale, orw = oracle.dispatch_fp8(x_bits, oslot, num_rows=R, topk_weights=w)
        assert np.array_equal(hr[used], orecv[used]) and np.all(hr[~used] == SENT_U8)
        hsc = host(scale)
        assert np.array_equal(hsc[used].view(np.uint32), oscale[used].view(np.uint32))
        assert np.all(hsc[~used] == SENT_F32)
        rest = host(store)
        assert np.all(rest[:scale_offset] == SENT_F32) and np.all(rest[scale_offset + R * G:] == SENT_F32)
    else:
        orecv = oracle.dispatch_bf16(x_bits, oslot, num_rows=R)
        assert np.array_equal(hr[used], orecv[used]) and np.all(hr[~used] == SENT_BF16)
        orw = oracle.dispatch_fp8(x_bits[:, :128], oslot, num_rows=R, topk_weights=w)[2] if w is not None else None
    if rw is not None:
        hw = host(rw)
        assert np.array_equal(hw[used], orw[used]) and np.all(hw[~used] == SENT_F32)


def routing(rng, T, K, E, distinct=True, mask_frac=0.0, dtype=np.int32):
    if distinct and E >= K:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K]
    else:
        idx = rng.integers(0, E, size=(T, K))
    mask = rng.random((T, K)) < mask_frac
    bad = rng.choice(np.array([-1, E, E + 5, -7, 2 ** 31 - 1, -(2 ** 31)], dtype=np.int64), size=(T, K))
    if dtype == np.int64:
        bad = np.where(bad == -1, bad, bad * 3 + (1 << 40))  # wide ids that wrap in 32 bits
    return np.where(mask, bad, idx).astype(dtype)


def tokens(rng, T, H, scale=1.0):
    return to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32) * np.float32(scale))


@pytest.mark.parametrize("fp8", [True, False])
def test_prefill_workload(gpu, fp8):
    """4096 tokens x 7168, 256 experts (group-limited top-8): the shape the
    step is measured on."""
    wl = make_workload("prefill", seed=11)
    print("case chunked prefill fp8=%s" % fp8, flush=True)
    run_and_check(gpu, wl.topk_idx, wl.x_bits, wl.topk_weights, wl.E, 0, fp8)


def test_skewed_prefill(gpu):
    wl = make_workload("skew", seed=12)
    print("case chunked skew", flush=True)
    run_and_check(gpu, wl.topk_idx, wl.x_bits, wl.topk_weights, wl.E, 0, True)


@pytest.mark.parametrize("T,K,E,H,cap,mask", [
    (3073, 1, 256, 512, 0, 0.05),    # K=1: 16 tokens per workgroup for 16-byte id loads
    (385, 8, 256, 2048, 0, 0.0),     # 3080 entries: 2 tokens per workgroup
    (1000, 6, 64, 1536, 0, 0.1),     # K=6; 96 items per token: per-lane scale stores
    (2000, 10, 300, 1024, 0, 0.05),  # K=10, odd E, 64 items per token: wavefront scale stores
    (3001, 2, 16, 1152, 0, 0.02),    # the last workgroup holds one token
    (4096, 16, 1024, 256, 0, 0.0),   # 65536 entries with 1024 experts: 8-wave workgroups
    (8192, 8, 256, 128, 0, 0.0),     # 65536 entries: 32 tokens per workgroup
    (600, 8, 256, 2048, 40, 0.05),   # padded with drops
    (1500, 8, 256, 7168, 128, 0.0),  # padded, full hidden size
    (4100, 1, 16, 128, 0, 0.5),      # half the entries masked
    (500, 16, 8, 640, 0, 0.0),       # K=16 over 8 experts: repeated experts in a token
    (200, 32, 64, 1024, 0, 0.05),    # K at its maximum: one token per workgroup
    (2000, 3, 256, 1152, 0, 0.05),   # odd K: 8 tokens per workgroup for 16-byte id loads
    (1025, 3, 64, 2048, 0, 0.0),     # odd K, the last workgroup holds one token
])
def test_shapes(gpu, T, K, E, H, cap, mask):
    rng = np.random.default_rng(T * 7919 + K * 31 + E + H)
    idx = routing(rng, T, K, E, distinct=E >= K, mask_frac=mask)
    x = tokens(rng, T, H, float(rng.choice([1e-3, 1.0, 300.0])))
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case chunked T=%d K=%d E=%d H=%d cap=%d" % (T, K, E, H, cap), flush=True)
    run_and_check(gpu, idx, x, w, E, cap, True)
    run_and_check(gpu, idx, x, w, E, cap, False)


@pytest.mark.parametrize("dtype", [np.int32, np.int64])
@pytest.mark.parametrize("id_offset", [0, 1])
@pytest.mark.parametrize("K", [8, 5])
def test_id_widths_and_alignment(gpu, dtype, id_offset, K):
    """16-byte id loads when the ids are 16-byte aligned, else element loads;
    int64 ids that wrap in 32 bits stay masked; odd K makes the chunk size
    a multiple of 4 (int32) or 2 (int64) ids only by the token count."""
    rng = np.random.default_rng(77 + id_offset + (dtype == np.int64) + K)
    T, E, H = 1800, 256, 1024
    idx = routing(rng, T, K, E, mask_frac=0.05, dtype=dtype)
    x = tokens(rng, T, H)
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case chunked ids %s offset=%d K=%d" % (np.dtype(dtype).name, id_offset, K), flush=True)
    run_and_check(gpu, idx, x, w, E, 0, True, id_offset=id_offset)
    run_and_check(gpu, idx, x, w, E, 16, True, id_offset=id_offset)


@pytest.mark.parametrize("scale_offset", [0, 1, 2])
def test_scale_alignment_and_no_weights(gpu, scale_offset):
    """recv_scale 16-byte aligned (wavefront scale stores) or not (per-lane
    stores); no routing weights."""
    rng = np.random.default_rng(90 + scale_offset)
    T, K, E, H = 1200, 8, 128, 2048
    idx = routing(rng, T, K, E, mask_frac=0.02)
    x = tokens(rng, T, H, 5.0)
    print("case chunked scale offset=%d" % scale_offset, flush=True)
    run_and_check(gpu, idx, x, None, E, 0, True, scale_offset=scale_offset)


def test_matches_the_separate_calls(gpu):
    """The one call and ep_layout + ep_dispatch give the same bits at the
    prefill size (both checked against the oracle elsewhere; here the
    chunked kernel against the kernels the step uses otherwise)."""
    ep = gpu
    wl = make_workload("prefill", seed=13)
    T, K, E, H = wl.T, wl.K, wl.E, wl.H
    R, G = T * K, H // 128
    d_idx = to_dev(wl.topk_idx)
    d_x = to_dev(wl.x_bits.view(np.int16))
    d_w = to_dev(wl.topk_weights)
    outs = []
    for fused in (True, False):
        counts = torch.full((E,), SENT_I32, dtype=torch.int32, device="cuda")
        offsets = torch.full((E + 1,), SENT_I32, dtype=torch.int32, device="cuda")
        slot = torch.full((T, K), SENT_I32, dtype=torch.int32, device="cuda")
        src = torch.full((R,), SENT_I32, dtype=torch.int32, device="cuda")
        recv = torch.full((R, H), SENT_U8, dtype=torch.uint8, device="cuda")
        scale = torch.full((R, G), SENT_F32, dtype=torch.float32, device="cuda")
        rw = torch.full((R,), SENT_F32, dtype=torch.float32, device="cuda")
        if fused:
            ep.ep_layout_dispatch(d_idx, d_x, d_w, E, 0, ep.EP_RECV_FP8_E4M3_G128, counts, offsets, slot, src,
                                  recv, scale, rw, None)
        else:
            ep.ep_dispatch_layout(d_idx, E, counts, offsets, slot, src)
            ep.ep_dispatch(d_x, slot, d_w, ep.EP_RECV_FP8_E4M3_G128, recv, scale, rw)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (counts, offsets, slot, src, recv, scale, rw)])
    print("case chunked vs separate calls", flush=True)
    for a, b in zip(*outs):
        assert torch.equal(a, b)
