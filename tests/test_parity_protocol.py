"""The parity protocol of the GPU tests, exercised on the CPU with planted
mistakes: a draft that takes the other side of a near-tie and continues by the
rule from there passes; a wrong token at a clear position, an inadmissible pick
at a near-tie, or a continuation that ignores the changed context fails.  The
same for sampled drafts and for rejection-sampling outcomes."""
import numpy as np
import pytest

import oracle
from oracle import sampling as S
from gpu_util import NEAR_TIE, check_draft, check_sampled_draft, check_verify_sample


def _case(seed=1, B=3, k=6, V=401, r=4):
    g = np.random.default_rng(seed)
    Z = (g.standard_normal((B, k, V)) * 2).astype(np.float32)
    w1 = g.standard_normal((V, r)).astype(np.float32)
    w2 = (g.standard_normal((V, r)) * 0.5).astype(np.float32)
    prev = g.integers(0, V, B)
    return Z, w1, w2, prev


def _plant_near_tie(Z, w1, w2, prev, b, i):
    """Make position (b, i) of the oracle chain a near-tie (a second token 1e-3
    below the maximum); returns the chain, the runner-up and the new Z."""
    d, _ = oracle.semi_ar_argmax(Z, w1, w2, prev, "f32")
    ctx = prev[b] if i == 0 else d[b, i - 1]
    s = Z[b, i] + oracle.markov_bias(w1.astype(np.float64), w2.astype(np.float64), ctx)
    other = (int(d[b, i]) + 17) % Z.shape[-1]
    Z = Z.copy()
    Z[b, i, other] += np.float32(s[d[b, i]] - s[other] - 1e-3)
    d, gap = oracle.semi_ar_argmax(Z, w1, w2, prev, "f32")
    assert gap[b, i] < NEAR_TIE
    return d, other, Z


def _continue_from(Z, w1, w2, prev, d, b, i, token):
    """The chain's row b with position i forced to ``token`` and the later
    positions following the rule from that context."""
    out = d.copy()
    out[b, i] = token
    for j in range(i + 1, d.shape[1]):
        best, _, _ = oracle.score_draft(Z, w1, w2, prev, out, "f32")
        out[b, j] = best[b, j]
    return out


def test_greedy_protocol_accepts_an_admissible_other_side():
    Z, w1, w2, prev = _case()
    d, other, Z = _plant_near_tie(Z, w1, w2, prev, 1, 2)
    assert check_draft(d, Z, w1, w2, prev, "f32")["other_side"] == 0
    flipped = _continue_from(Z, w1, w2, prev, d, 1, 2, other)
    c = check_draft(flipped, Z, w1, w2, prev, "f32")
    assert c["other_side"] == 1 and c["n"] == d.size


def test_greedy_protocol_rejects_planted_mistakes():
    Z, w1, w2, prev = _case()
    d, other, Z = _plant_near_tie(Z, w1, w2, prev, 1, 2)
    wrong = d.copy()
    wrong[0, 3] = (wrong[0, 3] + 1) % Z.shape[-1]          # clear position
    with pytest.raises(AssertionError):
        check_draft(wrong, Z, w1, w2, prev, "f32")
    far = d.copy()
    far[1, 2] = (d[1, 2] + 5) % Z.shape[-1]                  # near-tie, not admissible
    with pytest.raises(AssertionError):
        check_draft(far, Z, w1, w2, prev, "f32")
    stale = d.copy()
    stale[1, 2] = other                                      # later positions keep the old context
    if not np.array_equal(stale, _continue_from(Z, w1, w2, prev, d, 1, 2, other)):
        with pytest.raises(AssertionError):
            check_draft(stale, Z, w1, w2, prev, "f32")


def test_sampled_protocol():
    Z, w1, w2, prev = _case(seed=3)
    T, seed = 0.8, 77
    d, gap, x = S.semi_ar_sample(Z, w1, w2, prev, "f32", T, seed)
    check_sampled_draft(d, x, Z, w1, w2, prev, "f32", T, seed)
    wrong = d.copy()
    i = int(np.flatnonzero(gap[0] >= NEAR_TIE)[0])
    wrong[0, i] = (wrong[0, i] + 1) % Z.shape[-1]
    with pytest.raises(AssertionError):
        check_sampled_draft(wrong, None, Z, w1, w2, prev, "f32", T, seed)
    xbad = x.copy()
    xbad[2, 1, 5] += 0.01
    with pytest.raises(AssertionError):
        check_sampled_draft(d, xbad, Z, w1, w2, prev, "f32", T, seed)


def test_verify_sample_protocol():
    g = np.random.default_rng(8)
    B, k, V, T, seed = 6, 4, 300, 1.0, 5
    Z = (g.standard_normal((B, k, V)) * 2).astype(np.float32)
    d, _, x = S.semi_ar_sample(Z, None, None, np.zeros(B, np.int64), "f32", T, seed)
    Y = (0.8 * np.concatenate([x, x[:, :1]], axis=1)
         + 0.2 * g.standard_normal((B, k + 1, V))).astype(np.float32)
    L = np.array([k, k, 2, 0, k, 1])
    ref = S.verify_sample(d, x, Y, "f32", L, T, seed)
    check_verify_sample(ref["accepted"], ref["bonus"], d, x, Y, "f32", L, T, seed)
    for b in range(B):
        bad_a = ref["accepted"].copy()
        bad_a[b] = (bad_a[b] + 1) % (L[b] + 1)
        if bad_a[b] == ref["accepted"][b]:
            continue
        # a different accepted length is caught unless the decision it needs is
        # within rounding (these random rows have wide margins)
        o = S.verify_sample_outcome(d, x, Y, "f32", L, T, seed, bad_a, ref["bonus"])
        if np.all(o["margin"][b][np.isfinite(o["margin"][b])] >= 1e-3):
            with pytest.raises(AssertionError):
                check_verify_sample(bad_a, ref["bonus"], d, x, Y, "f32", L, T, seed)
    bad_b = ref["bonus"].copy()
    bad_b[0] = (bad_b[0] + 1) % V
    if ref["draw_gap"][0] >= NEAR_TIE:
        with pytest.raises(AssertionError):
            check_verify_sample(ref["accepted"], bad_b, d, x, Y, "f32", L, T, seed)
