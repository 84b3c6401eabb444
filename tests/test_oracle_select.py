"""Pins of the oracle's indexer scores, top-k and blockwise pooling against
closed forms, an O(n^2) rank-count definition and brute force."""
import itertools
import math

import numpy as np

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


# ----------------------------------------------------------------- scores

def test_score_one_hot_keys_give_query_components():
    rng = np.random.default_rng(0)
    q = bf16(rng.standard_normal(64))
    keys = bf16(np.eye(64) * 1.0)
    s = oracle.scores(q, keys)
    assert np.array_equal(s, bf16_bits_to_f32(q))


def test_score_keys_proportional_to_query():
    # halves and small integers: every product and sum is exact
    rng = np.random.default_rng(1)
    qv = rng.integers(-8, 9, size=64) / 2.0
    q = bf16(qv)
    cs = np.array([0.0, 1.0, -2.0, 0.5, 3.0])
    keys = bf16(cs[:, None] * qv[None, :])
    s = oracle.scores(q, keys)
    want = (cs * float(np.sum(qv * qv))).astype(np.float32)
    assert np.array_equal(s, want)


def test_score_is_exactly_rounded_sum():
    rng = np.random.default_rng(2)
    q = bf16(rng.standard_normal(64))
    keys = bf16(rng.standard_normal((200, 64)))
    s = oracle.scores(q, keys)
    qf = bf16_bits_to_f32(q).astype(np.float64)
    kf = bf16_bits_to_f32(keys).astype(np.float64)
    want = np.array([math.fsum(qf * kf[j]) for j in range(200)], np.float64).astype(np.float32)
    assert np.array_equal(s, want)


# ------------------------------------------------------------------ top-k

def rank_count_select(s, k, ids=None):
    """j is chosen iff fewer than k candidates precede it (higher score, or
    equal score at a lower position).  O(n^2), no sorting."""
    n = len(s)
    ids = np.arange(n) if ids is None else np.asarray(ids)
    valid = ids >= 0
    chosen = []
    for j in range(n):
        if not valid[j]:
            continue
        before = 0
        for i in range(n):
            if not valid[i] or i == j:
                continue
            if s[i] > s[j] or (s[i] == s[j] and ids[i] < ids[j]):
                before += 1
        if before < k:
            chosen.append(int(ids[j]))
    out = sorted(chosen)
    return np.array(out + [-1] * (k - len(out)), np.int32)


def test_topk_matches_rank_count_with_heavy_ties():
    rng = np.random.default_rng(3)
    for n, k in [(1, 1), (7, 3), (300, 17), (1200, 64), (40, 40), (40, 55)]:
        s = rng.integers(-5, 6, size=n).astype(np.float32) * 0.5
        s[rng.random(n) < 0.1] = -0.0  # -0 and +0 are equal
        got = oracle.topk(s, k)
        assert np.array_equal(got, rank_count_select(s, k)), (n, k)


def test_topk_through_candidate_ids_with_empty_slots():
    rng = np.random.default_rng(4)
    ids = np.sort(rng.choice(5000, size=300, replace=False)).astype(np.int32)
    ids[rng.random(300) < 0.1] = -1
    s = rng.integers(-3, 4, size=300).astype(np.float32)
    got = oracle.topk(s, 40, ids)
    assert np.array_equal(got, rank_count_select(s, 40, ids))


def test_topk_brute_force_over_all_subsets():
    """The chosen set has the best score multiset; among equally good sets it
    is the one made of the lowest positions."""
    rng = np.random.default_rng(5)
    for trial in range(60):
        n = int(rng.integers(1, 13))
        k = int(rng.integers(1, 5))
        s = rng.integers(-2, 3, size=n).astype(np.float32)
        best = None
        for sub in itertools.combinations(range(n), min(k, n)):
            key = (sorted((float(s[i]) for i in sub), reverse=True), [-i for i in sub])
            if best is None or key > best[0]:
                best = (key, sub)
        want = list(best[1]) + [-1] * (k - min(k, n))
        assert np.array_equal(oracle.topk(s, k), np.array(want, np.int32)), (s, k)


def test_topk_k_at_least_n_takes_everything():
    s = np.array([3.0, -1.0, 2.0], np.float32)
    assert np.array_equal(oracle.topk(s, 5), np.array([0, 1, 2, -1, -1], np.int32))


# -------------------------------------------------------------- blockwise

def test_block_scores_are_block_maxima_with_ragged_tail():
    rng = np.random.default_rng(6)
    s = rng.standard_normal(1000).astype(np.float32)
    b = oracle.block_scores(s, 64)
    assert b.size == 16
    for i in range(16):
        assert b[i] == s[i * 64:(i + 1) * 64].max()
