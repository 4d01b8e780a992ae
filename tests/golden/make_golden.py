"""Write the oracle regression digests in this folder.

Calls only the oracle and the seeded input generators.  Run from the
repository root:  python tests/golden/make_golden.py
A change to these digests is a change to the oracle's arithmetic: the
commit that makes it names the passage (or the reading of it) behind it.
"""

import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from workloads import make_workload  # noqa: E402


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode() + str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()


def compute():
    out = {}
    for name, seed, T in (("tiny", 0, None), ("decode", 1, None), ("skew", 0, 256)):
        wl = make_workload(name, seed=seed, T=T)
        counts, offsets, slot, src = oracle.dispatch_layout(wl.topk_idx, wl.E)
        recv, scale, rw = oracle.dispatch_fp8(wl.x_bits, slot, topk_weights=wl.topk_weights)
        comb = oracle.combine(wl.y_bits, slot, wl.topk_weights)
        pc, pslot, psrc = oracle.dispatch_layout_padded(wl.topk_idx, wl.E, max(1, wl.T // 8))
        gx = oracle.dispatch_backward(wl.y_bits, slot)
        gy, gw = oracle.combine_backward(wl.x_bits, wl.y_bits, slot, wl.topk_weights)
        key = "%s_seed%d_T%d" % (name, seed, wl.T)
        out[key] = {
            "inputs": digest(wl.topk_idx, wl.topk_weights, wl.x_bits, wl.y_bits),
            "layout": digest(counts, offsets, slot, src),
            "dispatch_fp8": digest(recv, scale, rw),
            "combine": digest(comb),
            "layout_padded": digest(pc, pslot, psrc),
            "dispatch_backward": digest(gx),
            "combine_backward": digest(gy, gw),
        }
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_digests.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)
