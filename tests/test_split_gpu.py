"""ep_layout_dispatch on the split layout + dispatch kernel (the large
one-launch batches: 7 or 8 FP8 or 13 or 14 BF16 work items per lane of a
1024-lane workgroup, one workgroup per CU), against the oracle bit for bit.

On a 256-CU device every case below takes that kernel: 3329 to 4608 tokens
of hidden 7168 (FP8), 3329 to 4096 (BF16), or 6145 to 8192 tokens of
hidden 4096 (FP8).  Cases: int64 ids, the padded layout with drops, top-k
6 and 16, 300 and 1024 experts, masked ids, scale buffers with and without
the wavefront scale stores, with and without routing weights, a last
workgroup with fewer tokens.
"""

import numpy as np
import pytest

from tests.test_chunked_gpu import routing, run_and_check, tokens

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,K,E,H,cap,mask,dtype,fp8,weights,scale_offset", [
    (3900, 8, 256, 7168, 0, 0.05, np.int64, True, True, 0),    # int64 ids, ragged last workgroup
    (3900, 8, 256, 7168, 100, 0.02, np.int32, True, True, 0),  # padded layout, entries dropped
    (3600, 6, 300, 7168, 0, 0.05, np.int32, True, False, 0),   # K=6: 16 tokens per workgroup
    (4096, 8, 256, 7168, 0, 0.0, np.int32, True, True, 1),     # scales not 16-byte aligned
    (4096, 8, 1024, 7168, 0, 0.1, np.int32, True, True, 0),    # 1024 experts
    (4000, 8, 256, 7168, 0, 0.05, np.int64, False, True, 0),   # BF16, 14 items per lane
    (3500, 8, 256, 7168, 0, 0.5, np.int32, False, False, 0),   # BF16, half the entries masked
    (7000, 8, 256, 4096, 0, 0.05, np.int32, True, True, 0),    # hidden 4096, 28 tokens per workgroup
    (4096, 16, 64, 7168, 0, 0.0, np.int32, True, True, 0),     # K=16: 256 entries per workgroup
])
def test_split_shapes(gpu, T, K, E, H, cap, mask, dtype, fp8, weights, scale_offset):
    rng = np.random.default_rng(T * 31 + K * 7 + E + H + cap)
    idx = routing(rng, T, K, E, distinct=E >= K, mask_frac=mask, dtype=dtype)
    x = tokens(rng, T, H, float(rng.choice([1e-3, 1.0, 300.0])))
    w = rng.standard_normal((T, K)).astype(np.float32) if weights else None
    print("case split T=%d K=%d E=%d H=%d cap=%d %s fp8=%d" % (T, K, E, H, cap, np.dtype(dtype).name, fp8),
          flush=True)
    run_and_check(gpu, idx, x, w, E, cap, fp8, scale_offset=scale_offset)
