"""Seeded generator checks, and the statistical pin of generator + oracle verify.

With the planted target logits, position i of a sequence is accepted exactly
when every planted match up to i hit, so E[acc[i]] / N = prod_{j<=i} p_j (times
0.7^(i+1) under truncation at 0.3 with U(0,1) confidence).  A verify step that
dropped a term, shifted a position or mis-counted fails these at 4 sigma.
"""
import dataclasses

import numpy as np
import pytest

import workloads
from workloads import synth
from oracle import reference as ref


def _small(w, **kw):
    return dataclasses.replace(w, **kw)


def test_generator_is_deterministic_and_step_dependent():
    w = _small(workloads.get("b16"), hidden=64, vocab=300, batch=3)
    a = synth.make_step(w, 3)
    b = synth.make_step(w, 3)
    c = synth.make_step(w, 4)
    for key in ("draft_hidden", "prev0", "noise"):
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])
    for x, y in zip(a["taps"], b["taps"]):
        assert np.array_equal(x, y)


def test_generator_chunking_independent_of_threads(monkeypatch):
    x = synth.normal_f32((3, synth.CHUNK + 5), (9, 0, 0, 1))
    monkeypatch.setattr(synth, "_threads", lambda: 1)
    y = synth.normal_f32((3, synth.CHUNK + 5), (9, 0, 0, 1))
    assert np.array_equal(x, y)


@pytest.mark.parametrize("name", ["tiny", "qwen27b_b1", "flashnext_b4", "b16", "adaptive_b16"])
def test_shapes_and_dtypes(name):
    w = workloads.get(name)
    if w.hidden > 64:   # shrink the large shapes; the layout logic is the same
        w = _small(w, hidden=64, vocab=512)
    W = synth.make_weights(w)
    dt = np.float32 if w.dtype == "f32" else np.uint16
    assert W["fc_w"].shape == (w.hidden, w.n_taps * w.hidden) and W["fc_w"].dtype == dt
    assert W["lm_w"].shape == (w.vocab, w.hidden)
    assert W["w1"].shape == W["w2"].shape == (w.vocab, w.rank)
    s = synth.make_step(w, 0)
    assert len(s["taps"]) == w.n_taps
    assert all(t.shape == (w.rows, w.hidden) and t.dtype == dt for t in s["taps"])
    assert s["draft_hidden"].shape == (w.batch, w.k, w.hidden)
    assert s["prev0"].shape == (w.batch,) and s["prev0"].dtype == np.int32
    assert np.all((0 <= s["prev0"]) & (s["prev0"] < w.vocab))
    assert s["noise"].shape == (w.batch, w.k + 1, w.vocab)


def test_tiny_taps_are_the_listed_fake_layers():
    w = workloads.get("tiny")
    s = synth.make_step(w, 2)
    layers = synth.normal_f32((w.fake_layers, w.rows, w.hidden), (w.cid, 1, 2, 0))
    for t, l in zip(s["taps"], w.tap_layers):
        assert np.array_equal(t, layers[l])


def test_weight_variances():
    w = _small(workloads.get("qwen27b_b1"), hidden=256, vocab=4096, rank=32)
    W = synth.make_weights(w)
    var = lambda x: float(np.var(ref.widen(x, w.dtype)))
    assert var(W["fc_w"]) == pytest.approx(1.0 / (5 * 256), rel=0.05)
    assert var(W["lm_w"]) == pytest.approx(1.0 / 256, rel=0.05)
    assert var(W["w1"]) == pytest.approx(1.0, rel=0.05)
    assert var(W["w2"]) == pytest.approx(0.1, rel=0.05)


def test_planting_puts_boost_where_stated():
    w = _small(workloads.get("qwen27b_b1"), vocab=2000)
    d = synth.random_drafts(w, 0)
    s = synth.make_step(w, 0)
    p = synth.plant_targets(w, 0, s["noise"], d)
    y = ref.widen(p["target_logits"], w.dtype) - s["noise"]
    tok = p["planted_token"]
    for j in range(w.k + 1):
        assert y[0, j, tok[0, j]] == pytest.approx(8.0, abs=0.07)   # bf16 rounding of noise+8
    hit = p["planted_hit"]
    assert np.array_equal(hit[0], tok[0, :w.k] == d[0])


def _verify_counts(w, steps):
    acc_tot = np.zeros(w.k, np.int64)
    prop_tot = np.zeros(w.k, np.int64)
    for s in range(steps):
        d = synth.random_drafts(w, s)
        noise = synth.make_step(w, s, noise=True)["noise"]
        Y = synth.plant_targets(w, s, noise, d)["target_logits"]
        conf = synth.make_confidence(w, s)
        L = ref.truncate_by_confidence(conf, w.threshold, w.batch, w.k)
        t = ref.target_argmax(Y, w.dtype, L)
        _, _, acc, prop = ref.verify_greedy(d, t, L)
        acc_tot += acc
        prop_tot += prop
    return acc_tot, prop_tot


def test_acceptance_statistics_fixed_curve():
    w = _small(workloads.get("tiny"), batch=4)
    steps = 600
    acc, prop = _verify_counts(w, steps)
    N = steps * w.batch
    q = np.cumprod(w.plant_p)
    sd = np.sqrt(N * q * (1 - q)) + 1e-9
    assert np.all(np.abs(acc - N * q) <= 4 * sd + 1), (acc, N * q)
    assert np.all(prop == N)


def test_acceptance_statistics_mixture_with_truncation():
    w = _small(workloads.get("adaptive_b16"), hidden=64, vocab=1000)
    steps = 150
    acc, prop = _verify_counts(w, steps)
    N = steps * w.batch
    keep = 0.7 ** np.arange(1, w.k + 1)
    q = 0.5 * (np.cumprod(w.plant_hi) + np.cumprod(w.plant_lo)) * keep
    sd = np.sqrt(N * q * (1 - q)) + 1e-9
    assert np.all(np.abs(acc - N * q) <= 4 * sd + 1), (acc, N * q)
    sdp = np.sqrt(N * keep * (1 - keep))
    assert np.all(np.abs(prop - N * keep) <= 4 * sdp + 1)


def test_plant_fast_path_is_identical():
    w = _small(workloads.get("adaptive_b16"), hidden=64, vocab=3000)
    s = synth.make_step(w, 5)
    d = synth.random_drafts(w, 5)
    slow = synth.plant_targets(w, 5, s["noise"], d)
    fast = synth.plant_targets(w, 5, s["noise"], d, noise_stored=synth.store(s["noise"], w.dtype))
    assert np.array_equal(slow["target_logits"], fast["target_logits"])
    assert np.array_equal(slow["planted_token"], fast["planted_token"])
