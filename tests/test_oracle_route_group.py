"""Pins of the oracle's routing (top-k + gates) and grouping (stable counting sort).

Each check compares the C oracle with something other than itself: a
lexicographic brute-force sort, a float64 softmax over all experts, closed-form
special cases, and the invariants any valid grouping must satisfy.
"""
import numpy as np
import pytest

import oracle
from oracle.dense import topk_mask_gates


def brute_topk(logits, k):
    T, E = logits.shape
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        out[t] = np.lexsort((np.arange(E), -logits[t]))[:k]
    return out


@pytest.mark.parametrize("T,E,k", [(8, 16, 2), (37, 64, 10), (5, 512, 10), (3, 100, 100),
                                   (9, 7, 1), (4, 129, 33)])
def test_topk_matches_lexsort(T, E, k):
    rng = np.random.default_rng(T * 1000 + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, gates = oracle.route(logits, k)
    assert np.array_equal(idx, brute_topk(logits, k))


def test_topk_ties_go_to_lower_index():
    rng = np.random.default_rng(1)
    logits = rng.integers(0, 4, size=(50, 40)).astype(np.float32)   # ties everywhere
    for k in (1, 3, 10, 40):
        idx, _ = oracle.route(logits, k)
        assert np.array_equal(idx, brute_topk(logits, k))


def test_all_equal_logits():
    logits = np.full((6, 16), 0.75, dtype=np.float32)
    for k in (1, 2, 5, 16):
        idx, gates = oracle.route(logits, k)
        assert np.array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (6, 1)))
        assert np.all(gates == np.float32(1.0 / k))


def test_k_equals_E_is_full_sort():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((4, 33)).astype(np.float32)
    idx, gates = oracle.route(logits, 33)
    for t in range(4):
        assert sorted(idx[t]) == list(range(33))
        assert np.all(np.diff(logits[t][idx[t]]) <= 0)
    assert np.allclose(gates.sum(axis=1), 1.0, atol=33 * 2 ** -23)


def test_signed_zero_and_nan_order():
    logits = np.array([[-0.0, 0.0, np.nan, -1.0, np.nan, 0.5]], dtype=np.float32)
    idx, _ = oracle.route(logits, 6)
    # 0.5 first; -0 == +0 tie -> lower index 0 then 1; -1; NaNs last by index
    assert idx.tolist() == [[5, 0, 1, 3, 2, 4]]


def test_k1_gate_is_one():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((20, 50)).astype(np.float32) * 10
    idx, gates = oracle.route(logits, 1)
    assert np.all(gates == 1.0)


def test_gates_equal_full_softmax_renormalised():
    rng = np.random.default_rng(4)
    logits = (rng.standard_normal((64, 512)) * 2).astype(np.float32)
    k = 10
    idx, gates = oracle.route(logits, k)
    mask, g_full = topk_mask_gates(logits, k)
    for t in range(64):
        assert set(idx[t]) == set(np.nonzero(mask[t])[0])
        ref = g_full[t, idx[t]]
        assert np.max(np.abs(gates[t] - ref)) < 1e-7
    assert np.all(np.abs(gates.sum(axis=1) - 1) <= k * 2 ** -23)
    assert np.all(np.diff(gates, axis=1) <= 0)        # rank order -> non-increasing


def test_gates_closed_form_two_experts():
    # k=2 with logits a > b: gates = 1/(1+e^(b-a)), e^(b-a)/(1+e^(b-a))
    a, b = 1.25, -0.5
    logits = np.array([[b, a, -3.0]], dtype=np.float32)
    idx, gates = oracle.route(logits, 2)
    assert idx.tolist() == [[1, 0]]
    r = np.exp(b - a)
    assert abs(gates[0, 0] - 1 / (1 + r)) < 1e-7 and abs(gates[0, 1] - r / (1 + r)) < 1e-7


# ---------------------------------------------------------------- grouping


def check_grouping(idx, E, has_shared, counts, offsets, perm, slot_of):
    T, k = idx.shape
    A = T * (k + int(has_shared))
    expert_of = np.concatenate([idx.reshape(-1), np.full(T if has_shared else 0, E)])
    assert counts.sum() == A
    assert np.array_equal(counts, np.bincount(expert_of, minlength=E + 1))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert sorted(perm.tolist()) == list(range(A))           # a permutation
    assert np.array_equal(slot_of[perm], np.arange(A))       # inverse map
    # each token appears exactly k (+1) times
    tok = np.where(perm < T * k, perm // max(k, 1), perm - T * k)
    assert np.all(np.bincount(tok, minlength=T) == k + int(has_shared))
    # stable: equals the stable argsort of the expert of each flat id
    assert np.array_equal(perm, np.argsort(expert_of, kind="stable"))


@pytest.mark.parametrize("T,E,k,shared", [(8, 16, 2, 0), (1024, 512, 10, 1), (4, 512, 10, 1),
                                          (1, 5, 5, 1), (300, 3, 2, 0)])
def test_grouping_invariants(T, E, k, shared):
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = oracle.route(logits, k)
    check_grouping(idx, E, shared, *oracle.group(idx, E, shared))


def test_grouping_one_expert_takes_all():
    T, E, k = 64, 32, 3
    idx = np.tile(np.array([7, 0, 31], dtype=np.int32), (T, 1))
    counts, offsets, perm, slot_of = oracle.group(idx, E, True)
    check_grouping(idx, E, True, counts, offsets, perm, slot_of)
    assert counts[7] == T and counts[0] == T and counts[31] == T and counts[E] == T
    assert counts.sum() == T * (k + 1)


def test_grouping_empty():
    idx = np.zeros((0, 4), dtype=np.int32)
    counts, offsets, perm, slot_of = oracle.group(idx, 8, True)
    assert counts.sum() == 0 and perm.size == 0 and offsets[-1] == 0
