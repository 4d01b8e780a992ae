"""Seeded generators for the five MoE dispatch/combine workloads.

Recipe (every array is a pure function of (config, seed)):

* ``np.random.SeedSequence(seed).spawn(3)`` gives three independent
  streams: ``rx`` for the tokens x, ``rg`` for the gate and ``ry`` for the
  expert outputs y.
* x: ``rx.standard_normal((T, H), float32)`` rounded to BF16 by torch's CPU
  cast (a library call; this module implements no rounding of its own).
* Gate logits ~ N(0, 1) in float64; routing per config (below); weights are
  computed in float64 and cast to float32 once.
* y (expert outputs for combine parity and timing): an independent
  N(0, 1) BF16 tensor of R = T*K rows drawn from ``ry``.

Configurations (sizes are those of the pages' prefill and decode settings;
see the package docstring):

=========  =====  ====  ===  =  ==================================  =====
name       T      H     E    K  routing                             recv
=========  =====  ====  ===  =  ==================================  =====
tiny       64     256   16   2  softmax, top-2, renormalised        fp8
decode     128    7168  256  8  group-limited (8 groups, top-4)     fp8
prefill    4096   7168  256  8  group-limited (8 groups, top-4)     fp8
skew       4096   7168  256  8  Zipf(1.2) popularity, Dirichlet w   fp8
hbm        32768  7168  256  8  group-limited (8 groups, top-4)     bf16
=========  =====  ====  ===  =  ==================================  =====

Group-limited routing: sigma = sigmoid(logit); a group's score is the sum
of its two largest sigma; the 4 best groups are kept; the top 8 experts by
sigma inside them are picked and their weights are sigma / sum(sigma).
Ties go to the lower index (stable sorts).  Experts of one token are listed
by descending weight.
"""

from dataclasses import dataclass, field

import numpy as np


def to_bf16_bits(x32):
    """float32 array -> BF16 bit patterns (uint16) via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _streams(seed):
    ss = np.random.SeedSequence(int(seed))
    return [np.random.default_rng(s) for s in ss.spawn(3)]


def route_softmax_topk(logits, k):
    """Softmax gate, top-k by probability, weights renormalised to sum 1."""
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    idx = np.argsort(-p, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(p, idx, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w.astype(np.float32)


def route_group_limited(logits, n_group, topk_group, k):
    """Sigmoid gate with group-limited top-k (see the module docstring)."""
    T, E = logits.shape
    sig = 1.0 / (1.0 + np.exp(-logits))
    g = sig.reshape(T, n_group, E // n_group)
    top2 = np.sort(g, axis=2)[:, :, -2:].sum(axis=2)
    keep = np.argsort(-top2, axis=1, kind="stable")[:, :topk_group]
    gmask = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(gmask, keep, True, axis=1)
    masked = np.where(np.repeat(gmask, E // n_group, axis=1), sig, -np.inf)
    idx = np.argsort(-masked, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(sig, idx, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w.astype(np.float32)


def route_zipf(rng, T, E, k, s=1.2, holes_frac=0.0):
    """k distinct experts per token from a Zipf(s) popularity; Dirichlet(1) weights.

    Popularity p_e is proportional to rank**-s over a seeded rank->expert
    permutation.  Drawing k distinct experts with probability proportional
    to p (sampling without replacement) is done with Gumbel-top-k.  With
    ``holes_frac`` > 0 that fraction of experts gets popularity 0 and so
    receives no token.
    """
    perm = rng.permutation(E)
    pop = np.empty(E)
    pop[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    if holes_frac > 0:
        holes = rng.choice(E, size=int(round(holes_frac * E)), replace=False)
        pop[holes] = 0.0
    with np.errstate(divide="ignore"):
        logp = np.log(pop / pop.sum())
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    w = rng.dirichlet(np.ones(k), size=T)
    order = np.argsort(-w, axis=1, kind="stable")
    w = np.take_along_axis(w, order, axis=1)
    return idx.astype(np.int32), w.astype(np.float32)


WORKLOADS = {
    "tiny": dict(T=64, H=256, E=16, K=2, routing="softmax", fp8=True),
    "decode": dict(T=128, H=7168, E=256, K=8, routing="group", fp8=True),
    "prefill": dict(T=4096, H=7168, E=256, K=8, routing="group", fp8=True),
    "skew": dict(T=4096, H=7168, E=256, K=8, routing="zipf", fp8=True),
    "hbm": dict(T=32768, H=7168, E=256, K=8, routing="group", fp8=False),
}


def make_x_bits(rx, T, H, chunk=2048):
    out = np.empty((T, H), dtype=np.uint16)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        out[t0:t1] = to_bf16_bits(rx.standard_normal((t1 - t0, H), dtype=np.float32))
    return out


def make_y_bits(ry, R, H, chunk=4096):
    return make_x_bits(ry, R, H, chunk)


@dataclass
class Workload:
    name: str
    seed: int
    T: int
    H: int
    E: int
    K: int
    fp8: bool
    topk_idx: np.ndarray
    topk_weights: np.ndarray
    _rx: object = field(repr=False, default=None)
    _ry: object = field(repr=False, default=None)
    _x: object = field(repr=False, default=None)
    _y: object = field(repr=False, default=None)

    @property
    def x_bits(self):
        if self._x is None:
            self._x = make_x_bits(self._rx, self.T, self.H)
        return self._x

    @property
    def y_bits(self):
        """Independent N(0,1) BF16 expert outputs, one per receive row."""
        if self._y is None:
            self._y = make_y_bits(self._ry, self.T * self.K, self.H)
        return self._y


def make_routing(name, seed, T=None, **over):
    cfg = dict(WORKLOADS[name])
    cfg.update(over)
    if T is not None:
        cfg["T"] = T
    rx, rg, ry = _streams(seed)
    T, E, K = cfg["T"], cfg["E"], cfg["K"]
    if cfg["routing"] == "softmax":
        idx, w = route_softmax_topk(rg.standard_normal((T, E)), K)
    elif cfg["routing"] == "group":
        idx, w = route_group_limited(rg.standard_normal((T, E)), 8, 4, K)
    elif cfg["routing"] == "zipf":
        idx, w = route_zipf(rg, T, E, K, s=1.2, holes_frac=cfg.get("holes_frac", 0.0))
    else:
        raise ValueError(cfg["routing"])
    return cfg, rx, ry, idx, w


def make_workload(name, seed=0, T=None, **over):
    """Build the seeded workload ``name`` (a key of WORKLOADS).

    ``T`` overrides the token count (same routing recipe); other keyword
    overrides replace config fields (e.g. ``holes_frac=0.25`` for the
    skew-with-empty-experts variant).  x and y are drawn lazily.
    """
    cfg, rx, ry, idx, w = make_routing(name, seed, T=T, **over)
    return Workload(name=name, seed=seed, T=cfg["T"], H=cfg["H"], E=cfg["E"], K=cfg["K"],
                    fp8=cfg["fp8"], topk_idx=idx, topk_weights=w, _rx=rx, _ry=ry)
