"""Pins of the oracle's checks of a GIVEN draft or verification outcome.

``score_draft`` / ``score_sampled_draft`` take each position's context from the
given draft (the chain conditions position i on the prediction actually made at
i-1), and ``verify_sample_outcome`` evaluates the rejection-sampling rule along
the path a given (accepted, bonus) outcome takes.  The GPU parity tests use them
to check every position of a GPU draft, including after a near-tie where the
GPU may legitimately have taken the other token.

Pins: the planted successor map (closed-form context, best token and deficit
for an arbitrary given draft), brute force over every draft of a tiny
vocabulary (exactly one draft has zero deficit everywhere, the brute-force
chain), a hand-built near-tie, out-of-range tokens, the vanishing-temperature
limit, and for verification: p = q (every test accepts), a draft token with no
target mass (rejected), and enumeration of every outcome of tiny rows (exactly
one is the rule's, the one ``verify_sample`` returns).
"""
import itertools

import numpy as np

from oracle import reference as ref
from oracle import sampling as S


def _successor_case(V=97, r=6, k=7, B=4):
    sigma = np.array([13, 40, 2, 77, 61, 30])
    w1 = np.zeros((V, r), np.float32)
    w1[np.arange(V), np.arange(V) % r] = 1.0
    w2 = np.zeros((V, r), np.float32)
    w2[sigma, np.arange(r)] = 100.0
    prev0 = np.array([5, 50, 96, 13])
    return sigma, w1, w2, prev0, np.zeros((B, k, V), np.float32)


def test_score_draft_planted_successor_map_any_draft():
    """Z = 0, w1[p] = e_(p mod r), w2[v, c] = 100 [v = sigma(c)]: under context c
    the biased logits are 100 at sigma(c mod r) and 0 elsewhere, so for ANY
    given draft: best = sigma(context mod r), deficit = 0 where the draft token
    is that successor and 100 elsewhere, gap = 100.  A check that took its
    contexts from its own argmax, ignored prev0 or swapped w1/w2 fails here."""
    sigma, w1, w2, prev0, Z = _successor_case()
    B, k, V = Z.shape
    r = w1.shape[1]
    g = np.random.default_rng(3)
    for trial in range(4):
        draft = g.integers(0, V, (B, k))
        if trial == 0:            # the exact chain: zero deficit everywhere
            for b in range(B):
                c = prev0[b]
                for i in range(k):
                    c = draft[b, i] = sigma[c % r]
        best, gap, deficit = ref.score_draft(Z, w1, w2, prev0, draft, "f32")
        for b in range(B):
            c = prev0[b]
            for i in range(k):
                want = sigma[c % r]
                assert best[b, i] == want
                assert gap[b, i] == 100.0
                assert deficit[b, i] == (0.0 if draft[b, i] == want else 100.0)
                c = draft[b, i]
        if trial == 0:
            assert np.all(deficit == 0)


def test_score_draft_brute_force_tiny_vocab():
    """Over every one of the V^k drafts, exactly one has zero deficit at every
    position (on tie-free inputs) and it is the chain found by brute-force
    enumeration of self-consistent sequences."""
    V, k, r = 5, 3, 2
    checked = 0
    for seed in range(12):
        g = np.random.default_rng(500 + seed)
        Z = g.standard_normal((1, k, V)).astype(np.float32)
        w1 = g.standard_normal((V, r)).astype(np.float32)
        w2 = g.standard_normal((V, r)).astype(np.float32)
        prev0 = np.array([int(g.integers(0, V))])
        table = np.zeros((V, V), np.float32)   # bias[p][v] by explicit sums
        for p in range(V):
            for v in range(V):
                table[p, v] = np.float32(sum(float(w2[v, j]) * float(w1[p, j]) for j in range(r)))
        zero, consistent, tie = [], [], False
        for seq in itertools.product(range(V), repeat=k):
            ctx, ok = int(prev0[0]), True
            for i in range(k):
                s = Z[0, i] + table[ctx]
                srt = np.sort(s)
                tie |= bool(srt[-1] - srt[-2] < 1e-6)
                ok &= int(np.argmax(s)) == seq[i]
                ctx = seq[i]
            if ok:
                consistent.append(seq)
            _, _, deficit = ref.score_draft(Z, w1, w2, prev0, np.array([seq]), "f32")
            if np.all(deficit == 0):
                zero.append(seq)
        if tie:
            continue
        checked += 1
        assert len(consistent) == 1 and zero == consistent
    assert checked >= 8


def test_score_draft_near_tie_and_out_of_range():
    V = 50
    Z = np.zeros((1, 3, V), np.float32)
    Z[0, 0, 7] = 1.0
    Z[0, 0, 30] = np.float32(1.0) - np.float32(2.0 ** -10)     # 2^-10 below the max
    Z[0, 1, 4] = 2.0
    draft = np.array([[30, 60, -1]])
    best, gap, deficit = ref.score_draft(Z, None, None, np.array([0]), draft, "f32")
    assert best[0, 0] == 7 and gap[0, 0] == 2.0 ** -10 and deficit[0, 0] == 2.0 ** -10
    assert best[0, 1] == 4 and np.isinf(deficit[0, 1])
    assert np.isinf(deficit[0, 2])


def test_score_draft_agrees_with_the_chain():
    """The chain's own draft scores zero deficit everywhere and best = draft."""
    g = np.random.default_rng(9)
    B, k, V, r = 3, 6, 301, 4
    Z = g.standard_normal((B, k, V)).astype(np.float32)
    w1 = g.standard_normal((V, r)).astype(np.float32)
    w2 = (g.standard_normal((V, r)) * 0.5).astype(np.float32)
    prev0 = g.integers(0, V, B)
    d, gap = ref.semi_ar_argmax(Z, w1, w2, prev0, "f32")
    best, gap2, deficit = ref.score_draft(Z, w1, w2, prev0, d, "f32")
    assert np.array_equal(best, d) and np.all(deficit == 0) and np.array_equal(gap, gap2)


def test_score_sampled_draft_successor_map_and_vanishing_temperature():
    """Successor map at T = 1: the Gumbel noise cannot overcome a logit margin
    of 100, so the draw under any given context is sigma(context mod r) and a
    wrong token's deficit is above 50.  At T -> 0 the draw is the greedy best."""
    sigma, w1, w2, prev0, Z = _successor_case()
    B, k, V = Z.shape
    r = w1.shape[1]
    draft = np.random.default_rng(4).integers(0, V, (B, k))
    best, gap, deficit, x = S.score_sampled_draft(Z, w1, w2, prev0, draft, "f32", 1.0, 77)
    for b in range(B):
        c = prev0[b]
        for i in range(k):
            want = sigma[c % r]
            assert best[b, i] == want
            assert x[b, i, want] == 100.0 and np.count_nonzero(x[b, i]) == 1
            assert deficit[b, i] == 0.0 if draft[b, i] == want else deficit[b, i] > 50.0
            c = draft[b, i]
    g = np.random.default_rng(10)
    Zr = (g.standard_normal((2, 4, 211)) * 3).astype(np.float32)
    w1r = g.standard_normal((211, 3)).astype(np.float32)
    w2r = (g.standard_normal((211, 3)) * 0.5).astype(np.float32)
    p0 = np.array([3, 100])
    dg, _ = ref.semi_ar_argmax(Zr, w1r, w2r, p0, "f32")
    bs, _, ds, _ = S.score_sampled_draft(Zr, w1r, w2r, p0, dg, "f32", 1e-7, 5)
    assert np.array_equal(bs, dg) and np.all(ds == 0)


def test_score_sampled_draft_agrees_with_the_sampler():
    g = np.random.default_rng(11)
    B, k, V, r = 3, 5, 257, 4
    Z = (g.standard_normal((B, k, V)) * 2).astype(np.float32)
    w1 = g.standard_normal((V, r)).astype(np.float32)
    w2 = (g.standard_normal((V, r)) * 0.5).astype(np.float32)
    prev0 = g.integers(0, V, B)
    d, gap, x = S.semi_ar_sample(Z, w1, w2, prev0, "f32", 0.9, 123)
    best, gap2, deficit, x2 = S.score_sampled_draft(Z, w1, w2, prev0, d, "f32", 0.9, 123)
    assert np.array_equal(best, d) and np.all(deficit == 0)
    assert np.array_equal(x, x2) and np.array_equal(gap, gap2)


def _tiny_verify_case(seed, B=4, k=3, V=4, corr=0.6):
    g = np.random.default_rng(seed)
    Z = (g.standard_normal((B, k, V)) * 1.5).astype(np.float32)
    d, _, x = S.semi_ar_sample(Z, None, None, np.zeros(B, np.int64), "f32", 1.0, seed)
    Y = (g.standard_normal((B, k + 1, V)) * 1.5).astype(np.float32)
    Y[:, :k] = corr * x + (1 - corr) * Y[:, :k]
    return d, x, Y


def test_verify_outcome_enumeration_has_one_consistent_outcome():
    """For every row, over all (accepted, bonus) outcomes, exactly one agrees
    with every tested decision and has zero bonus deficit, and it is
    verify_sample's outcome."""
    for seed in range(6):
        d, x, Y = _tiny_verify_case(40 + seed)
        B, k = d.shape
        V = Y.shape[-1]
        L = np.array([k, k, 1, 0])[:B]
        res = S.verify_sample(d, x, Y, "f32", L, 1.0, seed)
        for b in range(B):
            ok = []
            for a in range(int(L[b]) + 1):
                for bonus in range(V):
                    acc = np.zeros(B, np.int64)
                    bon = np.zeros(B, np.int64)
                    acc[:] = res["accepted"]
                    bon[:] = res["bonus"]
                    acc[b], bon[b] = a, bonus
                    o = S.verify_sample_outcome(d, x, Y, "f32", L, 1.0, seed, acc, bon)
                    dec = o["decision"][b]
                    agree = all(dec[n] for n in range(a)) and (a == L[b] or not dec[a])
                    if agree and o["bonus_deficit"][b] == 0 and o["draw"][b] == bonus:
                        ok.append((a, bonus))
            assert ok == [(int(res["accepted"][b]), int(res["bonus"][b]))], (seed, b, ok)


def test_verify_outcome_identical_distributions_and_zero_mass():
    """p = q: every tested position accepts (a full block is the only outcome
    the decisions allow).  A draft token with no target mass is rejected."""
    d, x, _ = _tiny_verify_case(60, B=3, k=4, V=6)
    B, k = d.shape
    Y = np.concatenate([x, x[:, :1]], axis=1)
    L = np.full(B, k)
    o = S.verify_sample_outcome(d, x, Y, "f32", L, 1.0, 8, np.full(B, k), np.zeros(B, np.int64))
    assert np.all(o["decision"][:, :k])
    Y2 = Y.copy()
    Y2[0, 0, d[0, 0]] = -1e4                   # p(d_00) = 0 (underflows)
    o2 = S.verify_sample_outcome(d, x, Y2, "f32", L, 1.0, 8, np.zeros(B, np.int64),
                                 np.zeros(B, np.int64))
    assert not o2["decision"][0, 0]
    # the residual draw after that rejection never picks the rejected token
    assert o2["draw"][0] != d[0, 0] and np.isinf(
        S.verify_sample_outcome(d, x, Y2, "f32", L, 1.0, 8, np.zeros(B, np.int64),
                                np.full(B, d[0, 0]))["bonus_deficit"][0])
    bad = S.verify_sample_outcome(d, x, Y, "f32", L, 1.0, 8, np.full(B, k + 1),
                                  np.zeros(B, np.int64))
    assert not bad["valid"].any()
