"""Pins for the oracle's dispatch layout (CPU only)."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import dispatch_layout
from tests.pins import brute_layout
from workloads import make_workload


def check_invariants(idx, E, counts, offsets, slot, src):
    T, K = idx.shape
    valid = (idx >= 0) & (idx < E)
    nv = int(valid.sum())
    assert counts.sum() == nv
    assert offsets[0] == 0 and offsets[-1] == nv
    assert np.all(np.diff(offsets.astype(np.int64)) == counts)
    # slot is a bijection of the valid entries onto [0, nv)
    assert np.array_equal(np.sort(slot[valid]), np.arange(nv))
    assert np.all(slot[~valid] == -1)
    # src inverts slot, and is -1 past the valid rows
    tt = np.broadcast_to(np.arange(T)[:, None], (T, K))
    assert np.array_equal(src[slot[valid]], tt[valid])
    assert np.all(src[nv:] == -1)
    # each row lies in the segment of an expert its token picked, and
    # inside a segment tokens ascend (strictly when a token lists an expert once)
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) >= 0)
        if seg.size:
            assert np.all((idx[seg] == e).any(axis=1))


def test_hand_worked_example():
    """Three tokens, two picks each, four experts, one masked pick.

    Entries in (t, k) order: (0,0)->2 (0,1)->0 (1,0)->2 (1,1)->-1
    (2,0)->0 (2,1)->3.  Counts: e0 two, e1 none, e2 two, e3 one, so the
    offsets are 0,2,2,4,5.  Expert 0 receives token 0 then token 2 (rows 0,
    1); expert 2 receives token 0 then token 1 (rows 2, 3); expert 3
    receives token 2 (row 4); the masked pick has no row, and row 5 is past
    the valid rows.
    """
    idx = np.array([[2, 0], [2, -1], [0, 3]], dtype=np.int32)
    counts, offsets, slot, src = dispatch_layout(idx, 4)
    assert counts.tolist() == [2, 0, 2, 1]
    assert offsets.tolist() == [0, 2, 2, 4, 5]
    assert slot.tolist() == [[2, 0], [3, -1], [1, 4]]
    assert src.tolist() == [0, 2, 0, 1, 2, -1]


def test_duplicate_expert_in_one_token_orders_by_k():
    idx = np.array([[1, 1], [0, 1]], dtype=np.int32)
    counts, offsets, slot, src = dispatch_layout(idx, 2)
    assert slot.tolist() == [[1, 2], [0, 3]]
    assert src.tolist() == [1, 0, 0, 1]


def test_empty_and_all_masked():
    c, o, s, r = dispatch_layout(np.zeros((0, 3), np.int32), 5)
    assert c.tolist() == [0] * 5 and o.tolist() == [0] * 6 and s.shape == (0, 3) and r.size == 0
    c, o, s, r = dispatch_layout(np.full((4, 2), -1, np.int32), 3)
    assert c.tolist() == [0, 0, 0] and o.tolist() == [0, 0, 0, 0]
    assert np.all(s == -1) and np.all(r == -1)


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 9).flatmap(lambda E: st.tuples(
    st.just(E),
    st.integers(0, 12).flatmap(lambda T: st.integers(1, 4).flatmap(lambda K: st.lists(
        st.lists(st.integers(-2, E + 1), min_size=K, max_size=K), min_size=T, max_size=T).map(
            lambda rows: np.array(rows, dtype=np.int32).reshape(T, K)))))))
def test_matches_brute_force(args):
    E, idx = args
    counts, offsets, slot, src = dispatch_layout(idx, E)
    bc, bo, bs, bsrc = brute_layout(idx.tolist(), E)
    assert counts.tolist() == bc
    assert offsets.tolist() == bo
    assert slot.tolist() == (bs if idx.shape[0] else [])
    assert src.tolist() == bsrc
    check_invariants(idx, E, counts, offsets, slot, src)


def test_brute_force_on_tiny_config():
    wl = make_workload("tiny", seed=0)
    counts, offsets, slot, src = dispatch_layout(wl.topk_idx, wl.E)
    bc, bo, bs, bsrc = brute_layout(wl.topk_idx.tolist(), wl.E)
    assert counts.tolist() == bc and offsets.tolist() == bo
    assert slot.tolist() == bs and src.tolist() == bsrc


def test_textbook_counting_sort():
    """Special case: with no masked entries the layout is a textbook stable
    counting sort by expert: histogram, exclusive scan, then one pass in
    (t, k) order placing each entry at its expert's running cursor."""
    rng = np.random.default_rng(1)
    T, K, E = 300, 6, 40
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    hist = [0] * E
    for v in idx.ravel():
        hist[v] += 1
    cursor, run = [], 0
    for h in hist:
        cursor.append(run)
        run += h
    want_slot = np.empty((T, K), np.int64)
    for t in range(T):
        for k in range(K):
            e = idx[t, k]
            want_slot[t, k] = cursor[e]
            cursor[e] += 1
    counts, offsets, slot, src = dispatch_layout(idx, E)
    assert counts.tolist() == hist
    assert np.array_equal(slot, want_slot)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skew", "hbm"])
def test_invariants_on_workloads(name):
    wl = make_workload(name, seed=0)
    idx = wl.topk_idx
    counts, offsets, slot, src = dispatch_layout(idx, wl.E)
    assert counts.sum() == wl.T * wl.K
    # distinct experts per token in every configuration
    assert all(len(set(r)) == wl.K for r in idx[:: max(1, wl.T // 512)].tolist())
    if wl.T <= 4096:
        check_invariants(idx, wl.E, counts, offsets, slot, src)
    else:
        assert np.array_equal(np.sort(slot.ravel()), np.arange(wl.T * wl.K))
        tt = np.repeat(np.arange(wl.T), wl.K)
        assert np.array_equal(src[slot.ravel()], tt)


def test_skew_has_hot_experts_and_holes_variant_has_empty_experts():
    c = dispatch_layout(make_workload("skew", seed=0).topk_idx, 256)[0]
    assert c.max() > 1000 and c.min() >= 0
    c2 = dispatch_layout(make_workload("skew", seed=0, holes_frac=0.25).topk_idx, 256)[0]
    assert (c2 == 0).sum() == 64


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 6).flatmap(lambda E: st.tuples(
    st.just(E), st.integers(1, 5),
    st.integers(0, 10).flatmap(lambda T: st.integers(1, 3).flatmap(lambda K: st.lists(
        st.lists(st.integers(-2, E), min_size=K, max_size=K), min_size=T, max_size=T).map(
            lambda rows: np.array(rows, dtype=np.int32).reshape(T, K)))))))
def test_padded_matches_brute_force(args):
    from oracle import dispatch_layout_padded
    from tests.pins import brute_layout_padded

    E, cap, idx = args
    rc, slot, src = dispatch_layout_padded(idx, E, cap)
    bc, bs, bsrc = brute_layout_padded(idx.tolist(), E, cap)
    assert rc.tolist() == bc
    assert slot.tolist() == (bs if idx.shape[0] else [])
    assert src.tolist() == bsrc


def test_padded_with_enough_capacity_is_the_packed_layout_rebased():
    """Special case: capacity >= every count drops nothing, and each row is
    the packed row moved from offsets[e] to e*capacity."""
    from oracle import dispatch_layout_padded

    wl = make_workload("decode", seed=0)
    counts, offsets, slot, src = dispatch_layout(wl.topk_idx, wl.E)
    rc, pslot, psrc = dispatch_layout_padded(wl.topk_idx, wl.E, wl.T)
    assert np.array_equal(rc, counts)
    e = wl.topk_idx
    assert np.array_equal(pslot, e * wl.T + (slot - offsets[e]))
    for ex in range(wl.E):
        assert np.array_equal(psrc[ex * wl.T: ex * wl.T + counts[ex]], src[offsets[ex]:offsets[ex + 1]])
        assert np.all(psrc[ex * wl.T + counts[ex]:(ex + 1) * wl.T] == -1)
