"""Pins of the sampling oracle (oracle.sampling) against what the mathematics
fixes, not against itself:
  * the generator equals rocRAND's Philox4x32-10 (an independent
    implementation, compiled here from the ROCm headers) bit for bit; its
    uniforms are uniform and 23-bit exact, and every counter and key bit
    diffuses over the output;
  * Gumbel-max draws reproduce softmax frequencies;
  * at vanishing temperature probabilistic drafting is the greedy chain;
  * speculative sampling is lossless: the first emitted token is distributed
    as the target p_0, the acceptance rate of position 0 is sum_v min(p, q),
    identical distributions are always accepted, and a draft token the target
    gives no mass to is always rejected and replaced by a draw from p.
Frequencies are checked within 5 binomial standard deviations."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import sampling as S


def _within(count, n, prob, sig=5.0):
    sd = np.sqrt(n * prob * (1 - prob)) + 1e-12
    return abs(count - n * prob) <= sig * sd + 1


def test_uniforms_are_uniform_and_exact():
    u = S.uniforms(20251202, S.STREAM_DRAFT, 7, 3, 1 << 18)
    assert np.all((u > 0) & (u < 1))
    assert np.all(np.float32(u).astype(np.float64) == u)          # exact in float32
    m = u * 2.0 ** 24
    assert np.all(m == np.round(m)) and np.all(np.round(m) % 2 == 1)  # odd multiples of 2^-24
    n = u.size
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / n)
    assert abs(u.var() - 1 / 12) < 0.002
    counts = np.bincount((u * 256).astype(int), minlength=256)
    chi2 = float(np.sum((counts - n / 256) ** 2 / (n / 256)))
    assert chi2 < 255 + 5 * np.sqrt(2 * 255)                       # ~ mean + 5 sd of chi2(255)


def test_philox_counter_and_key_bits_diffuse():
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 1 << 32, size=(2048, 4), dtype=np.uint64).astype(np.uint32)
    key = (0x12345678, 0x9ABCDEF0)
    base = S.philox4x32(ctr, key)

    def flipped_bits(a, b):
        x = (a ^ b).astype(np.uint32)
        return np.unpackbits(x.view(np.uint8), axis=-1).sum(axis=-1)

    for word in range(4):
        for bit in (0, 7, 13, 31):
            c2 = ctr.copy()
            c2[:, word] ^= np.uint32(1 << bit)
            f = flipped_bits(base, S.philox4x32(c2, key)).mean()
            assert 60.0 < f < 68.0, (word, bit, f)                # ~ half of 128 output bits
    for kw in range(2):
        for bit in (0, 16, 31):
            k2 = list(key)
            k2[kw] ^= 1 << bit
            f = flipped_bits(base, S.philox4x32(ctr, tuple(k2))).mean()
            assert 60.0 < f < 68.0, (kw, bit, f)
    # fewer rounds diffuse less (the round count is what the generator relies on)
    c2 = ctr.copy()
    c2[:, 1] ^= np.uint32(1)
    f1 = flipped_bits(S.philox4x32(ctr, key, rounds=1), S.philox4x32(c2, key, rounds=1)).mean()
    assert f1 < 8.0


def _hipcc():
    import shutil
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else shutil.which("hipcc")


def test_philox_matches_rocrand(tmp_path):
    """The oracle's Philox4x32-10 against rocRAND's independent implementation
    (its host-callable engine, built here from the ROCm headers) on random and
    extreme counters and keys."""
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "philox_rocrand")
    src = os.path.join(os.path.dirname(__file__), "philox_rocrand.cpp")
    r = subprocess.run([cc, "-O1", src, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    rng = np.random.default_rng(17)
    ctr = rng.integers(0, 1 << 32, size=(2000, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 1 << 32, size=(2000, 2), dtype=np.uint64).astype(np.uint32)
    ctr[0], key[0] = 0, 0
    ctr[1], key[1] = 0xFFFFFFFF, 0xFFFFFFFF
    ctr[2] = (7, 3, 2, S.STREAM_RESAMPLE)          # a counter of the sampling layout
    lines = "\n".join(" ".join(str(int(v)) for v in (*c, *k)) for c, k in zip(ctr, key))
    out = subprocess.run([exe], input=lines, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(t) for t in l.split()] for l in out.strip().splitlines()], dtype=np.uint64)
    got = np.stack([S.philox4x32(c[None], (int(k[0]), int(k[1])))[0] for c, k in zip(ctr, key)])
    assert ref.shape == (2000, 4)
    assert np.array_equal(got.astype(np.uint64), ref)


def test_streams_rows_and_positions_are_uncorrelated():
    n = 1 << 16
    a = S.uniforms(99, S.STREAM_DRAFT, 0, 0, n)
    for other in (S.uniforms(99, S.STREAM_RESAMPLE, 0, 0, n), S.uniforms(99, S.STREAM_DRAFT, 1, 0, n),
                  S.uniforms(99, S.STREAM_DRAFT, 0, 1, n), S.uniforms(100, S.STREAM_DRAFT, 0, 0, n)):
        assert abs(np.corrcoef(a, other)[0, 1]) < 5 / np.sqrt(n)


def test_gumbel_max_reproduces_softmax():
    logits = np.array([0.3, -1.2, 2.0, 0.0, 1.1])
    p = np.exp(logits - logits.max())
    p /= p.sum()
    n = 40000
    counts = np.zeros(5, dtype=np.int64)
    for t in range(n):
        idx, _ = S.gumbel_max(logits, S.uniforms(3, S.STREAM_DRAFT, t, 0, 5))
        counts[idx] += 1
    for v in range(5):
        assert _within(counts[v], n, p[v]), (v, counts[v] / n, p[v])


def test_gumbel_max_skips_zero_weight_entries():
    logw = np.array([-np.inf, 0.0, -np.inf])
    for t in range(50):
        assert S.gumbel_max(logw, S.uniforms(1, 2, t, 0, 3))[0] == 1


def test_vanishing_temperature_is_the_greedy_chain():
    rng = np.random.default_rng(11)
    B, k, V, r = 3, 4, 40, 4
    Z = (rng.standard_normal((B, k, V)) * 3).astype(np.float32)
    w1 = rng.standard_normal((V, r)).astype(np.float32)
    w2 = rng.standard_normal((V, r)).astype(np.float32)
    prev = rng.integers(0, V, B)
    dg, gap = oracle.semi_ar_argmax(Z, w1, w2, prev, "f32")
    assert gap.min() > 1e-3
    ds, _, x = S.semi_ar_sample(Z, w1, w2, prev, "f32", 1e-5, seed=4)
    assert np.array_equal(dg, ds)
    # the stored distribution logits are the greedy chain's biased logits
    for b in range(B):
        p = prev[b]
        for i in range(k):
            bias = oracle.markov_bias(w1.astype(np.float64), w2.astype(np.float64), p)
            assert np.array_equal(x[b, i], Z[b, i] + bias)
            p = dg[b, i]


def _tiny_case(seed_data=0):
    rng = np.random.default_rng(seed_data)
    k, V = 2, 6
    x = (rng.standard_normal((1, k, V)) * 1.5).astype(np.float32)      # draft logits
    y = (rng.standard_normal((1, k + 1, V)) * 1.5).astype(np.float32)  # target logits
    return x, y


def _softmax(v):
    e = np.exp(v - v.max())
    return e / e.sum()


def test_speculative_sampling_is_lossless():
    x, y = _tiny_case(0)
    k = x.shape[1]
    p0, q0 = _softmax(y[0, 0].astype(np.float64)), _softmax(x[0, 0].astype(np.float64))
    p1 = _softmax(y[0, 1].astype(np.float64))
    n = 20000
    first = np.zeros(6, dtype=np.int64)
    second = np.zeros(6, dtype=np.int64)
    acc0 = 0
    n_second = 0
    L = np.array([k])
    for t in range(n):
        d, _, xs = S.semi_ar_sample(x, None, None, np.array([0]), "f32", 1.0, seed=t)
        out = S.verify_sample(d, xs, y, "f32", L, 1.0, seed=t)
        a = int(out["accepted"][0])
        emitted = list(d[0, :a]) + [int(out["bonus"][0])]
        first[emitted[0]] += 1
        acc0 += a >= 1
        if a >= 1:                 # the second emitted token, given the first was the draft
            second[emitted[1]] += 1
            n_second += 1
    for v in range(6):
        assert _within(first[v], n, p0[v]), (v, first[v] / n, p0[v])
        assert _within(second[v], n_second, p1[v]), (v, second[v] / n_second, p1[v])
    assert _within(acc0, n, float(np.minimum(p0, q0).sum()))


def test_identical_distributions_are_always_accepted():
    x, _ = _tiny_case(1)
    y = np.concatenate([x, x[:, :1]], axis=1)          # p_i == q_i for i < k
    for t in range(200):
        d, _, xs = S.semi_ar_sample(x, None, None, np.array([0]), "f32", 0.7, seed=t)
        out = S.verify_sample(d, xs, y, "f32", np.array([2]), 0.7, seed=t)
        assert out["accepted"][0] == 2


def test_draft_token_without_target_mass_is_replaced_from_p():
    k, V = 1, 4
    x = np.array([[[8.0, -8.0, -8.0, -8.0]]], dtype=np.float32)   # q puts ~all mass on 0
    y = np.array([[[-60.0, 0.0, 1.0, 0.5], [0.0, 0.0, 0.0, 0.0]]], dtype=np.float32)
    p = _softmax(y[0, 0].astype(np.float64))
    n = 6000
    counts = np.zeros(V, dtype=np.int64)
    for t in range(n):
        d, _, xs = S.semi_ar_sample(x, None, None, np.array([0]), "f32", 1.0, seed=t)
        out = S.verify_sample(d, xs, y, "f32", np.array([k]), 1.0, seed=t)
        if d[0, 0] == 0:
            assert out["accepted"][0] == 0 and out["resampled"][0]
        counts[out["bonus"][0] if out["accepted"][0] == 0 else d[0, 0]] += 1
    for v in range(V):
        assert _within(counts[v], n, p[v]), (v, counts[v] / n, p[v])


def test_truncated_blocks_and_counts():
    x, y = _tiny_case(2)
    x = np.repeat(x, 3, axis=0)
    y = np.repeat(y, 3, axis=0)
    L = np.array([0, 1, 2])
    d, _, xs = S.semi_ar_sample(x, None, None, np.array([0, 1, 2]), "f32", 1.0, seed=9)
    out = S.verify_sample(d, xs, y, "f32", L, 1.0, seed=9)
    a = out["accepted"]
    assert np.all(a <= L) and a[0] == 0
    assert np.array_equal(out["proposed_counts"], np.array([2, 1]))
    assert np.array_equal(out["accept_counts"], np.array([(a > 0).sum(), (a > 1).sum()]))
    assert np.all((out["bonus"] >= 0) & (out["bonus"] < x.shape[2]))
