"""Pins of the oracle's verification (S4) and acceptance accounting.

Pins used: brute force over every (draft, target, block length) on V=3, k=3
against the product formula a = sum_i prod_{j<=i} [d_j = t_j][L > j];
invariants (0 <= a <= L <= k, the bonus always emitted, emitted tokens equal the
target's greedy tokens, counts non-increasing); the truncation rule on hand
cases; and the acceptance figures printed on the pages.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import reference as ref

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_brute_force_product_formula_v3_k3():
    V, k = 3, 3
    ds = list(itertools.product(range(V), repeat=k))
    ts = list(itertools.product(range(V), repeat=k + 1))
    D = np.array([d for d in ds for _ in ts for _ in range(k + 1)])
    T = np.array([t for _ in ds for t in ts for _ in range(k + 1)])
    L = np.array([Lb for _ in ds for _ in ts for Lb in range(k + 1)])
    a, bonus, acc, prop = ref.verify_greedy(D, T, L)
    for n in range(D.shape[0]):
        want_a = sum(int(np.prod([(D[n, j] == T[n, j]) and (L[n] > j) for j in range(i + 1)]))
                     for i in range(k))
        assert a[n] == want_a
        assert bonus[n] == T[n, want_a]
    assert np.array_equal(acc, [int(np.sum(a > i)) for i in range(k)])
    assert np.array_equal(prop, [int(np.sum(L > i)) for i in range(k)])


def test_invariants_random():
    g = np.random.default_rng(9)
    B, k, V = 500, 8, 4
    d = g.integers(0, V, (B, k))
    t = g.integers(0, V, (B, k + 1))
    t[:, :k] = np.where(g.random((B, k)) < 0.7, d, t[:, :k])
    L = g.integers(0, k + 1, B)
    a, bonus, acc, prop = ref.verify_greedy(d, t, L)
    assert np.all((0 <= a) & (a <= L) & (L <= k))
    for b in range(B):
        emitted = list(d[b, :a[b]]) + [bonus[b]]
        assert emitted == list(t[b, :a[b] + 1])      # lossless: target's own greedy tokens
        assert 0 <= bonus[b] < V
    assert np.all(np.diff(acc) <= 0) and np.all(np.diff(prop) <= 0)
    assert np.all(acc <= prop)
    assert acc.sum() == a.sum() and prop.sum() == L.sum()


@pytest.mark.parametrize("conf,th,want", [
    ([0.5, 0.2, 0.9], 0.3, 1),     # first position below the threshold cuts the block
    ([0.1, 0.9, 0.9], 0.3, 0),     # L = 0 allowed: only the bonus is emitted
    ([0.5, 0.6, 0.9], 0.3, 3),     # never below: full block
    ([0.3, 0.3, 0.3], 0.3, 3),     # strict comparison: equal is kept
    ([0.9, 0.29, 0.95], 0.3, 1),   # later high scores do not resume the block
    ([0.1, 0.1, 0.1], float("nan"), 3),
])
def test_truncation_rule(conf, th, want):
    L = ref.truncate_by_confidence(np.array([conf], np.float32), th, 1, 3)
    assert L[0] == want


def test_truncation_off_without_scores():
    assert np.array_equal(ref.truncate_by_confidence(None, 0.3, 2, 5), [5, 5])


def test_target_argmax_skips_rows_past_block():
    Y = np.zeros((2, 4, 10), np.float32)
    Y[:, :, 6] = 1.0
    t = ref.target_argmax(Y, "f32", L=np.array([1, 3]))
    assert t.tolist() == [[6, 6, -1, -1], [6, 6, 6, 6]]


def test_target_argmax_bf16_exact_ties():
    Y = np.full((1, 2, 20), 0xBF80, np.uint16)       # -1.0
    Y[0, 0, [4, 17]] = 0x4000                         # 2.0 twice -> 4
    Y[0, 1, 19] = 0x0000                              # +0.0 at the tail
    Y[0, 1, 2] = 0x8000                               # -0.0 ties it at a lower index -> 2
    assert ref.target_argmax(Y, "bf16").tolist() == [[4, 2]]


def test_mean_acceptance_length_matches_page_figures():
    """The k=7 per-position acceptance curve of the model card, fed through
    the accounting, lands inside the mean-acceptance range the same card gives."""
    curve = GOLDEN["k7_per_position_acceptance"]["values"]
    lo, hi = GOLDEN["int4_mean_acceptance_range"]["values"]
    N, k = 100, 7
    # 100 sequences whose accept lengths reproduce the curve: #(a > i) = 100 * curve[i]
    need = [round(N * c) for c in curve]
    a_len = np.zeros(N, np.int64)
    for i in range(k):
        a_len[:need[i]] = i + 1
    d = np.zeros((N, k), np.int64)
    t = np.ones((N, k + 1), np.int64)
    for b in range(N):
        t[b, :a_len[b]] = 0
    a, bonus, acc, prop = ref.verify_greedy(d, t, np.full(N, k))
    assert np.array_equal(acc, need)
    mal = ref.mean_acceptance_length(acc, steps=1, batch=N)
    assert mal == pytest.approx(1 + sum(curve))
    assert lo <= mal <= hi


def test_drafted_token_rate_matches_replication_figure():
    fig = GOLDEN["replication_acceptance"]
    acc = np.array([fig["accepted"]])
    prop = np.array([fig["proposed"]])
    assert round(100 * ref.drafted_token_rate(acc, prop), 1) == fig["rate_percent"]
