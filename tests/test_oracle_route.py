"""Pins for the oracle's routing: top-k selection, gate weights and the route map.

Each check uses something other than the oracle's own code: a brute-force
full sort, torch.topk, numpy's stable argsort, a different formula for the
gate weights, or invariants the route map must satisfy (tutorial, routing-tax
section: per-expert counts, row counts and a per-expert permutation).
"""
import numpy as np
import pytest
import torch


def _brute_topk(l, k):
    # full sort by (larger logit first, then lower index)
    return sorted(range(len(l)), key=lambda e: (-float(l[e]), e))[:k]


@pytest.mark.parametrize("T,E,k", [(40, 10, 3), (33, 8, 8), (17, 5, 1), (64, 16, 4)])
def test_topk_matches_brute_force_with_ties(oracle_lib, T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)   # many ties
    r = oracle_lib.route(logits, k)
    for t in range(T):
        assert list(r["topk_idx"][t]) == _brute_topk(logits[t], k)


def test_topk_negative_zero_ties_positive_zero(oracle_lib):
    logits = np.array([[0.0, -0.0, 0.0, -1.0]], np.float32)
    logits[0, 0] = -0.0
    r = oracle_lib.route(logits, 3)
    assert list(r["topk_idx"][0]) == [0, 1, 2]


def test_topk_matches_torch_topk_tie_free(oracle_lib):
    g = torch.Generator().manual_seed(7)
    logits = torch.randn(200, 32, generator=g)
    r = oracle_lib.route(logits.numpy(), 4)
    ref = torch.topk(logits, 4, dim=1, sorted=True).indices.numpy()
    np.testing.assert_array_equal(r["topk_idx"], ref)


def test_gate_weights_equal_renormalised_full_softmax(oracle_lib):
    g = torch.Generator().manual_seed(3)
    logits = torch.randn(300, 16, generator=g) * 3
    r = oracle_lib.route(logits.numpy(), 4)
    # different formula: softmax over all E, gather the selected, renormalise
    p = torch.softmax(logits.double(), dim=1)
    sel = torch.gather(p, 1, torch.from_numpy(r["topk_idx"]).long())
    ref = (sel / sel.sum(1, keepdim=True)).numpy()
    np.testing.assert_allclose(r["topk_w"], ref, rtol=2e-7, atol=1e-9)
    np.testing.assert_allclose(r["topk_w"].astype(np.float64).sum(1), 1.0, atol=1e-6)
    # descending logits give non-increasing weights
    assert np.all(np.diff(r["topk_w"], axis=1) <= 0)


def test_top1_weight_is_exactly_one(oracle_lib):
    logits = np.random.default_rng(0).standard_normal((50, 7)).astype(np.float32)
    r = oracle_lib.route(logits, 1)
    assert np.all(r["topk_w"] == 1.0)


@pytest.mark.parametrize("T,E,k", [(100, 8, 2), (257, 13, 4), (64, 64, 8)])
def test_route_map_against_stable_sort(oracle_lib, T, E, k):
    logits = np.random.default_rng(T + E + k).standard_normal((T, E)).astype(np.float32)
    r = oracle_lib.route(logits, k)
    idx = r["topk_idx"]
    # each token k distinct experts
    assert all(len(set(row)) == k for row in idx)
    np.testing.assert_array_equal(r["counts"], np.bincount(idx.ravel(), minlength=E))
    assert r["counts"].sum() == T * k
    np.testing.assert_array_equal(r["offsets"], np.concatenate([[0], np.cumsum(r["counts"])]))
    # a stable sort of the flattened pairs by expert is the per-expert permutation
    order = np.argsort(idx.ravel(), kind="stable")
    np.testing.assert_array_equal(r["src_slot"], order)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    np.testing.assert_array_equal(r["dst_row"], inv)
    # bijection onto [0, T*k) and increasing token order inside each group
    assert sorted(r["dst_row"].tolist()) == list(range(T * k))
    for e in range(E):
        toks = r["src_slot"][r["offsets"][e]:r["offsets"][e + 1]] // k
        assert np.all(np.diff(toks) > 0)


def test_padded_route_large_capacity_equals_unpadded(oracle_lib):
    T, E, k = 120, 6, 2
    logits = np.random.default_rng(11).standard_normal((T, E)).astype(np.float32)
    u = oracle_lib.route(logits, k)
    C = int(u["counts"].max()) + 3
    p = oracle_lib.route(logits, k, capacity=C)
    e = u["topk_idx"].ravel()
    np.testing.assert_array_equal(p["dst_row"], e * C + (u["dst_row"] - u["offsets"][e]))
    assert p["src_slot"].size == E * C
    filled = p["src_slot"] >= 0
    assert filled.sum() == T * k


def test_padded_route_drops_first_come_overflow(oracle_lib):
    T, E, k = 200, 4, 2
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 0] += 2.0                                     # expert 0 oversubscribed
    C = 60
    p = oracle_lib.route(logits, k, capacity=C)
    counts = p["counts"]
    assert (p["dst_row"] < 0).sum() == np.maximum(counts - C, 0).sum()
    # brute force: the first C pairs (token order) of each expert are kept
    seen = np.zeros(E, int)
    for t in range(T):
        for j in range(k):
            e = p["topk_idx"][t, j]
            want = e * C + seen[e] if seen[e] < C else -1
            assert p["dst_row"][t * k + j] == want
            seen[e] += 1
    # empty capacity rows are marked -1
    for e in range(E):
        used = min(counts[e], C)
        assert np.all(p["src_slot"][e * C + used:(e + 1) * C] == -1)
        assert np.all(p["src_slot"][e * C:e * C + used] >= 0)


def test_nonfinite_logit_rejected(oracle_lib):
    logits = np.zeros((4, 4), np.float32)
    logits[2, 1] = np.nan
    with pytest.raises(ValueError):
        oracle_lib.route(logits, 2)
