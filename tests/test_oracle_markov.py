"""Pins of the oracle's Markov-biased semi-autoregressive argmax (S3).

Pins used: the zero-Markov special case (reduces to numpy's argmax per position),
a planted successor map with a closed-form chain, brute-force enumeration of all
V^k sequences on a tiny vocabulary, crafted exact ties (lowest index wins,
-0.0 ties +0.0), and the top-2 gap definition.
"""
import itertools

import numpy as np
import pytest

from oracle import reference as ref


def _rand(B, k, V, r, seed):
    g = np.random.default_rng(seed)
    Z = g.standard_normal((B, k, V)).astype(np.float32)
    w1 = g.standard_normal((V, r)).astype(np.float32)
    w2 = (g.standard_normal((V, r)) * 0.3).astype(np.float32)
    prev0 = g.integers(0, V, B)
    return Z, w1, w2, prev0


@pytest.mark.parametrize("which", ["none", "w1", "w2", "rank0"])
def test_zero_markov_reduces_to_plain_argmax(which):
    B, k, V, r = 3, 5, 257, 4
    Z, w1, w2, prev0 = _rand(B, k, V, r, 11)
    if which == "none":
        w1 = w2 = None
    elif which == "w1":
        w1 = np.zeros_like(w1)
    elif which == "w2":
        w2 = np.zeros_like(w2)
    else:
        w1 = np.zeros((V, 0), np.float32)
        w2 = np.zeros((V, 0), np.float32)
    d, _ = ref.semi_ar_argmax(Z, w1, w2, prev0, "f32")
    assert np.array_equal(d, np.argmax(Z, axis=-1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_planted_successor_map_closed_form(dtype):
    """Z = 0, w1[p] = e_(p mod r), w2[v, c] = 100 [v = sigma(c)]:
    d_0 = sigma(prev0 mod r) and d_i = sigma(d_(i-1) mod r).

    A chain that used the unbiased argmax as context, ignored prev0, or swapped
    the embedding and projection roles of the two matrices fails this.
    """
    V, r, k, B = 97, 6, 7, 4
    sigma = np.array([13, 40, 2, 77, 61, 30])
    w1 = np.zeros((V, r), np.float32)
    w1[np.arange(V), np.arange(V) % r] = 1.0
    w2 = np.zeros((V, r), np.float32)
    w2[sigma, np.arange(r)] = 100.0
    prev0 = np.array([5, 50, 96, 13])
    Z = np.zeros((B, k, V), np.float32)
    if dtype == "bf16":
        conv = ref.f32_to_bf16_bits
        d, _ = ref.semi_ar_argmax(Z, conv(w1), conv(w2), prev0, dtype)
    else:
        d, _ = ref.semi_ar_argmax(Z, w1, w2, prev0, dtype)
    for b in range(B):
        p = prev0[b]
        for i in range(k):
            p = sigma[p % r]
            assert d[b, i] == p


def test_brute_force_all_sequences_tiny_vocab():
    """Enumerate all V^k token sequences; exactly one is self-consistent
    (each token is the argmax of its logits plus the bigram bias of the token
    before it, the first one conditioned on prev0) and it is the oracle's."""
    V, k, r = 7, 4, 2
    unique = 0
    for seed in range(20):
        g = np.random.default_rng(100 + seed)
        Z = g.standard_normal((1, k, V)).astype(np.float32)
        w1 = g.standard_normal((V, r)).astype(np.float32)
        w2 = g.standard_normal((V, r)).astype(np.float32)
        prev0 = np.array([int(g.integers(0, V))])
        # bigram bias table by explicit sums: bias[p][v] = sum_j w2[v,j] * w1[p,j]
        table = np.zeros((V, V), np.float32)
        for p in range(V):
            for v in range(V):
                table[p, v] = np.float32(sum(float(w2[v, j]) * float(w1[p, j]) for j in range(r)))
        consistent = []
        for seq in itertools.product(range(V), repeat=k):
            ctx, ok = int(prev0[0]), True
            for i in range(k):
                s = Z[0, i] + table[ctx]
                if np.sort(s)[-1] - np.sort(s)[-2] < 1e-6:
                    ok = False  # skip seeds with near-ties
                    break
                if int(np.argmax(s)) != seq[i]:
                    ok = False
                    break
                ctx = seq[i]
            if ok:
                consistent.append(seq)
        d, _ = ref.semi_ar_argmax(Z, w1, w2, prev0, "f32")
        assert len(consistent) <= 1
        if len(consistent) == 1:
            unique += 1
            assert tuple(d[0]) == consistent[0]
    assert unique >= 15


def test_brute_force_differs_from_unbiased_context():
    """The chain must feed the biased prediction forward: on this seed the
    plain-argmax context gives a different block."""
    V, k, r = 7, 4, 2
    g = np.random.default_rng(5)
    Z = g.standard_normal((1, k, V)).astype(np.float32)
    w1 = (g.standard_normal((V, r)) * 2).astype(np.float32)
    w2 = (g.standard_normal((V, r)) * 2).astype(np.float32)
    prev0 = np.array([3])
    d, _ = ref.semi_ar_argmax(Z, w1, w2, prev0, "f32")
    # alternative (wrong) chain: context = unbiased argmax of the previous position
    wrong, ctx = [], 3
    for i in range(k):
        s = Z[0, i] + ref.markov_bias(w1.astype(np.float64), w2.astype(np.float64), ctx)
        wrong.append(int(np.argmax(s)))
        ctx = int(np.argmax(Z[0, i]))
    assert list(d[0]) != wrong


def test_ties_break_to_lowest_index():
    V = 1000
    Z = np.full((1, 3, V), -5.0, np.float32)
    Z[0, 0, [900, 5, 999]] = 2.0          # three-way tie -> 5
    Z[0, 1, [999, 998]] = 1.0             # tie at the vocabulary tail -> 998
    Z[0, 2, 7] = 0.0                      # +0.0 ...
    Z[0, 2, 3] = -0.0                     # ... ties -0.0 at a lower index -> 3
    d, gap = ref.semi_ar_argmax(Z, None, None, np.array([0]), "f32")
    assert list(d[0]) == [5, 998, 3]
    assert np.all(gap[0] == 0.0)


def test_tie_created_by_bias():
    V, r = 64, 1
    Z = np.zeros((1, 1, V), np.float32)
    Z[0, 0, 40] = 1.0
    w1 = np.ones((V, r), np.float32)
    w2 = np.zeros((V, r), np.float32)
    w2[10, 0] = 1.0                       # bias lifts v=10 to exactly 1.0
    d, gap = ref.semi_ar_argmax(Z, w1, w2, np.array([0]), "f32")
    assert d[0, 0] == 10 and gap[0, 0] == 0.0


def test_top2_gap_definition():
    assert ref.top2_gap(np.array([1.0, 3.0, 3.0])) == 0.0
    assert ref.top2_gap(np.array([1.0, 2.0, 5.0])) == 3.0
    assert ref.top2_gap(np.array([-1.0, -4.0])) == 3.0
    assert ref.top2_gap(np.array([2.0])) == float("inf")


def test_first_argmax_rejects_nan():
    with pytest.raises(ValueError):
        ref.first_argmax(np.array([0.0, np.nan]))


def test_prev_token_range_checked():
    Z = np.zeros((1, 1, 10), np.float32)
    w = np.zeros((10, 2), np.float32)
    with pytest.raises(ValueError):
        ref.semi_ar_argmax(Z, w, w, np.array([10]), "f32")
