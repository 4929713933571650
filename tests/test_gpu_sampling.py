"""GPU parity of probabilistic drafting and rejection-sampling verification.

Expected values come only from the CPU oracle (oracle.sampling) on the same
seeded inputs; both sides run their own Philox4x32-10.  Every decision the GPU
takes is checked, following the GPU's own path:
  * draft draws: each position with the GPU's previous draw as its context;
    bit-exact where the oracle's top-2 Gumbel-key gap is >= NEAR_TIE, else the
    GPU's token must have a key within NEAR_TIE of the maximum;
  * acceptance tests along the GPU's outcome: accept below a_b, reject at a_b,
    unless the relative margin |r q - p| / max(p, q) there is below 1e-3
    (then either outcome is admissible);
  * the residual / bonus draw at the end of that path: bit-exact where its key
    gap is >= NEAR_TIE, else a key within NEAR_TIE of the maximum.
Accept counts are then compared with those of the GPU's validated outcomes.
A statistical test checks losslessness on the GPU alone against closed forms.
"""
import numpy as np
import pytest

import oracle
from oracle import sampling as S
from workloads import synth
from gpu_util import check_draft, check_sampled_draft, check_verify_sample, dev, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_readout_amd as bdr
    bdr.lib()


def bdr():
    import block_draft_readout_amd as m
    return m


def _markov(cid, V, r, dtype):
    w1 = synth.store(synth.normal_f32((V, r), (cid, 0, 0, 2), 1.0), dtype)
    w2 = synth.store(synth.normal_f32((V, r), (cid, 0, 0, 3), np.sqrt(0.1)), dtype)
    return w1, w2


def _logits(cid, B, k, V, std):
    return synth.normal_f32((B, k, V), (cid, 1, 0, 1), std)


# ----------------------------------------------------------------------------- generator
@pytest.mark.parametrize("stream", [0, 2])
def test_gumbel_noise_matches_the_generator(stream):
    B, k, V, seed = 3, 4, 1003, 0x0123456789ABCDEF
    log(f"noise B={B} k={k} V={V} stream={stream}")
    got = bdr().dspark_gumbel_noise(B, k, V, seed, stream).cpu().numpy().astype(np.float64)
    ref = np.stack([np.stack([S.gumbel(S.uniforms(seed, stream, b, i, V)) for i in range(k)])
                    for b in range(B)])
    err = np.abs(got - ref)
    log(f"  max abs err {err.max():.3e}")
    assert np.all(err <= 1e-6 + 1e-6 * np.abs(ref))
    # the uniforms recovered from the noise sit on the generator's own grid points
    m_ref = np.round(np.exp(-np.exp(-ref)) * 2.0 ** 23 - 0.5)
    m_got = np.round(np.exp(-np.exp(-got)) * 2.0 ** 23 - 0.5)
    assert np.mean(m_ref == m_got) > 0.95


def test_gumbel_noise_over_a_large_sample_of_the_grid():
    """16.7M variates (most of the 2^23 uniforms of the grid): every one within
    2e-6 of the exact -log(-log u)."""
    k, V, seed = 8, 1 << 21, 99
    got = bdr().dspark_gumbel_noise(1, k, V, seed, 0).cpu().numpy()
    worst = 0.0
    for i in range(k):
        ref = S.gumbel(S.uniforms(seed, 0, 0, i, V))
        worst = max(worst, float(np.max(np.abs(got[0, i].astype(np.float64) - ref))))
    log(f"  max abs err {worst:.3e}")
    assert worst <= 2e-6


def test_gumbel_noise_seeds_and_streams_differ():
    a = bdr().dspark_gumbel_noise(1, 2, 4096, 5, 0)
    b = bdr().dspark_gumbel_noise(1, 2, 4096, 6, 0)
    c = bdr().dspark_gumbel_noise(1, 2, 4096, 5, 2)
    assert not torch.equal(a, b) and not torch.equal(a, c)
    assert torch.equal(a, bdr().dspark_gumbel_noise(1, 2, 4096, 5, 0))


# ----------------------------------------------------------------------------- drafting
DRAFT_CASES = {
    # name: (B, k, V, rank, dtype, logit std, temperature)
    "tiny_f32": (1, 4, 1000, 8, "f32", 2.0, 1.0),
    "f32_ragged": (5, 6, 2053, 12, "f32", 3.0, 0.7),
    "bf16_b5": (5, 7, 5003, 64, "bf16", 2.5, 1.0),
    "bf16_b20": (20, 3, 1031, 8, "bf16", 2.0, 1.3),
    "bf16_b256": (256, 3, 3001, 16, "bf16", 2.0, 1.0),   # the chain's largest batch
    "no_bias": (3, 5, 4099, 0, "bf16", 2.0, 0.8),
    "f32_r128_passes": (2, 3, 3001, 128, "f32", 2.0, 1.0),   # per-position launches
    "qwen_vocab": (1, 7, 151936, 32, "bf16", 3.0, 1.0),
    "b1_bf16_r64": (1, 6, 20011, 64, "bf16", 3.0, 1.0),
    "b1_f32_r48": (1, 6, 20011, 48, "f32", 3.0, 0.8),
    "b16_vocab": (16, 7, 151936, 64, "bf16", 3.0, 0.9),
}


@pytest.mark.parametrize("name", list(DRAFT_CASES))
def test_markov_sample_parity(name):
    B, k, V, r, dtype, std, T = DRAFT_CASES[name]
    cid = 70 + list(DRAFT_CASES).index(name)
    seed = 1000 + cid
    Z = _logits(cid, B, k, V, std)
    w1, w2 = _markov(cid, V, r, dtype) if r else (None, None)
    prev = np.random.default_rng(cid).integers(0, V, B).astype(np.int32)
    log(f"markov sample {name}: B={B} k={k} V={V} r={r} {dtype} T={T}")
    d, x = bdr().dspark_markov_sample(dev(Z), dev(w1) if r else None, dev(w2) if r else None,
                                      dev(prev), T, seed)
    c = check_sampled_draft(d.cpu().numpy(), x.cpu().numpy(), Z, w1, w2, prev, dtype, T, seed)
    log(f"  {c}")


@pytest.mark.parametrize("name", ["bf16_b5", "bf16_b20", "f32_r128_passes", "b1_bf16_r64",
                                  "b16_vocab"])
def test_markov_sample_x_only_where_verified(name):
    """With the block's confidences and threshold, draft_logits is written only
    at the positions j < L_b (the first confidence below the threshold ends the
    block) and elsewhere keeps what it held; the tokens are those of the call
    without them, and x where written is the same, bit for bit."""
    B, k, V, r, dtype, std, T = DRAFT_CASES[name]
    cid = 70 + list(DRAFT_CASES).index(name)
    seed = 1000 + cid
    Z = _logits(cid, B, k, V, std)
    w1, w2 = _markov(cid, V, r, dtype) if r else (None, None)
    prev = np.random.default_rng(cid).integers(0, V, B).astype(np.int32)
    rng = np.random.default_rng(cid + 5)
    conf = rng.random((B, k)).astype(np.float32)
    conf[0] = 1.0                       # one row never truncated
    if B > 1:
        conf[1, 0] = 0.0                # one row truncated at position 0 (no x at all)
    th = 0.3
    L = np.array([next((j for j in range(k) if conf[b, j] < th), k) for b in range(B)])
    args = (dev(Z), dev(w1) if r else None, dev(w2) if r else None, dev(prev), T, seed)
    d_all, x_all = bdr().dspark_markov_sample(*args)
    x_gated = torch.full((B, k, V), float("nan"), dtype=torch.float32, device="cuda")
    d, _ = bdr().dspark_markov_sample(*args, draft_logits=x_gated, confidence=dev(conf),
                                      threshold=th)
    assert np.array_equal(d.cpu().numpy(), d_all.cpu().numpy())
    xa, xg = x_all.cpu().numpy(), x_gated.cpu().numpy()
    live = np.arange(k)[None, :] < L[:, None]
    assert np.array_equal(xg[live].view(np.uint32), xa[live].view(np.uint32))
    assert np.isnan(xg[~live]).all()
    log(f"markov sample {name}, x gated by confidence: {int(live.sum())} of {B * k} positions "
        f"written")


def test_small_temperature_is_the_greedy_chain():
    B, k, V, r = 4, 6, 5003, 64
    Z = _logits(90, B, k, V, 3.0)
    w1, w2 = _markov(90, V, r, "bf16")
    prev = np.arange(B, dtype=np.int32) * 7
    dg = bdr().dspark_markov_argmax(dev(Z), dev(w1), dev(w2), dev(prev)).cpu().numpy()
    ds, _ = bdr().dspark_markov_sample(dev(Z), dev(w1), dev(w2), dev(prev), 1e-6, 3)
    ds = ds.cpu().numpy()
    check_draft(dg, Z, w1, w2, prev, "bf16")
    check_draft(ds, Z, w1, w2, prev, "bf16")      # the greedy rule, position by position


def test_markov_sample_repeat_and_workspace_reuse():
    B, k, V, r = 3, 5, 7001, 32
    Z = dev(_logits(91, B, k, V, 2.0))
    w1, w2 = (dev(t) for t in _markov(91, V, r, "bf16"))
    prev = dev(np.array([1, 2, 3], dtype=np.int32))
    L = bdr().lib()
    ws = torch.zeros(L.dspark_markov_sample_workspace_bytes(B, k, V) + 256, dtype=torch.uint8,
                     device="cuda")
    a = bdr().dspark_markov_sample(Z, w1, w2, prev, 1.0, 11, workspace=ws)
    b = bdr().dspark_markov_sample(Z, w1, w2, prev, 1.0, 11, workspace=ws)
    c = bdr().dspark_markov_sample(Z, w1, w2, prev, 1.0, 12, workspace=ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.equal(a[0], c[0])
    # the error word (first 4 of the last 256 bytes) stays clear
    n = L.dspark_markov_sample_workspace_bytes(B, k, V)
    base = (ws.data_ptr() + 255) // 256 * 256 - ws.data_ptr()
    assert int(ws[base + n - 256: base + n - 252].sum()) == 0


# ----------------------------------------------------------------------------- verification
def _verify_inputs(cid, B, k, V, std, T, dtype, corr):
    """Oracle-drafted block and target logits y = corr * x + noise (acceptance
    rates between the extremes)."""
    Z = _logits(cid, B, k, V, std)
    d, _, x = S.semi_ar_sample(Z, None, None, np.zeros(B, np.int32), "f32", T, cid)
    noise = synth.normal_f32((B, k + 1, V), (cid, 1, 0, 3), std)
    y = noise.copy()
    y[:, :k] = corr * x + (1 - corr) * noise[:, :k]
    return d.astype(np.int32), x, synth.store(y, dtype)


VERIFY_CASES = {
    # name: (B, k, V, dtype, std, T, corr, threshold)
    "tiny_f32": (6, 4, 1000, "f32", 2.0, 1.0, 0.8, None),
    "bf16_ragged": (9, 5, 4099, "bf16", 2.0, 0.8, 0.9, None),     # scalar LSE path
    "bf16_adaptive": (16, 8, 5000, "bf16", 2.0, 1.0, 0.85, 0.3),  # truncated blocks, L = 0 rows
    "f32_low_accept": (7, 6, 2048, "f32", 3.0, 1.2, 0.3, None),
    "bf16_b64": (64, 3, 1536, "bf16", 2.0, 1.0, 0.9, None),
    "qwen_vocab": (1, 7, 151936, "bf16", 3.0, 1.0, 0.95, None),
    "b16_vocab": (16, 7, 151936, "bf16", 3.0, 1.0, 0.9, None),
}


@pytest.mark.parametrize("name", list(VERIFY_CASES))
def test_verify_sample_parity(name):
    B, k, V, dtype, std, T, corr, th = VERIFY_CASES[name]
    cid = 100 + list(VERIFY_CASES).index(name)
    seed = 5000 + cid
    d, x, Y = _verify_inputs(cid, B, k, V, std, T, dtype, corr)
    conf = None
    if th is not None:
        conf = np.random.default_rng(cid).random((B, k), dtype=np.float32)
        conf[0, 0] = 0.0                       # row 0: empty block
    L = oracle.truncate_by_confidence(conf, th, B, k)
    log(f"verify sample {name}: B={B} k={k} V={V} {dtype} T={T}")
    acc = torch.zeros(k, dtype=torch.int64, device="cuda")
    prop = torch.zeros(k, dtype=torch.int64, device="cuda")
    out = bdr().spec_verify_sample(dev(Y), dev(d), dev(x), T, seed,
                                   confidence=dev(conf) if conf is not None else None,
                                   threshold=th if th is not None else float("nan"),
                                   accept_counts=acc, proposed_counts=prop)
    got = {n: t.cpu().numpy() for n, t in out.items()}
    assert np.array_equal(got["block_len"], L)
    c = check_verify_sample(got["accepted"], got["bonus"], d, x, Y, dtype, L, T, seed)
    log(f"  accepted {got['accepted'].tolist()[:16]}; {c}")
    a = got["accepted"]
    assert np.array_equal(acc.cpu().numpy(), [(a > i).sum() for i in range(k)])
    assert np.array_equal(prop.cpu().numpy(), [(L > i).sum() for i in range(k)])


def test_out_of_range_draft_token_is_rejected():
    B, k, V = 2, 3, 1000
    d, x, Y = _verify_inputs(120, B, k, V, 2.0, 1.0, "f32", 1.0)
    d[0, 0] = V + 5
    d[1, 1] = -1
    out = bdr().spec_verify_sample(dev(Y), dev(d), dev(x), 1.0, 9)
    a = out["accepted"].cpu().numpy()
    assert a[0] == 0 and a[1] <= 1


def test_identical_distributions_accept_everything():
    B, k, V = 32, 5, 3000
    d, x, _ = _verify_inputs(121, B, k, V, 2.0, 1.0, "f32", 1.0)
    Y = np.concatenate([x, x[:, :1]], axis=1)
    out = bdr().spec_verify_sample(dev(Y), dev(d), dev(x), 1.0, 4)
    assert np.all(out["accepted"].cpu().numpy() == k)


def test_sampling_is_lossless_on_the_gpu():
    """Many independent rows of one tiny case: the first emitted token follows
    p_0 and position 0 is accepted with probability sum_v min(p_0, q_0)
    (5 standard deviations)."""
    B, k, V, T = 8192, 2, 8, 1.0
    rng = np.random.default_rng(7)
    z = (rng.standard_normal((1, k, V)) * 1.5).astype(np.float32)
    yrow = (rng.standard_normal((1, k + 1, V)) * 1.5).astype(np.float32)
    Z = np.repeat(z, B, axis=0)
    Y = np.repeat(yrow, B, axis=0)
    prev = np.zeros(B, dtype=np.int32)
    d, x = bdr().dspark_markov_sample(dev(Z), None, None, dev(prev), T, 77)
    out = bdr().spec_verify_sample(dev(Y), d, x, T, 78)
    d = d.cpu().numpy()
    a = out["accepted"].cpu().numpy()
    bonus = out["bonus"].cpu().numpy()
    first = np.where(a >= 1, d[:, 0], bonus)
    p0 = np.exp(yrow[0, 0] - yrow[0, 0].max()).astype(np.float64)
    p0 /= p0.sum()
    q0 = np.exp(z[0, 0] - z[0, 0].max()).astype(np.float64)
    q0 /= q0.sum()
    # the draft draws themselves follow q_0
    for v in range(V):
        c = np.sum(d[:, 0] == v)
        assert abs(c - B * q0[v]) <= 5 * np.sqrt(B * q0[v] * (1 - q0[v])) + 1, ("q", v)
        c = np.sum(first == v)
        assert abs(c - B * p0[v]) <= 5 * np.sqrt(B * p0[v] * (1 - p0[v])) + 1, ("p", v)
    pa = float(np.minimum(p0, q0).sum())
    assert abs(np.sum(a >= 1) - B * pa) <= 5 * np.sqrt(B * pa * (1 - pa)) + 1


def test_end_to_end_block_matches_oracle_on_gpu_draft():
    """Drafting and verification chained on the device; the oracle verifies the
    GPU's own draft (tokens and draft logits) with the same seed."""
    B, k, V, r, T = 4, 6, 9001, 32, 1.0
    Z = _logits(130, B, k, V, 2.5)
    w1, w2 = _markov(130, V, r, "bf16")
    prev = np.array([5, 6, 7, 8], dtype=np.int32)
    noise = synth.normal_f32((B, k + 1, V), (130, 1, 0, 3), 2.5)
    d, x = bdr().dspark_markov_sample(dev(Z), dev(w1), dev(w2), dev(prev), T, 131)
    xh = x.cpu().numpy()
    Y = noise.copy()
    Y[:, :k] = 0.9 * xh + 0.1 * noise[:, :k]
    Yb = synth.store(Y, "bf16")
    out = bdr().spec_verify_sample(dev(Yb), d, x, T, 132)
    check_sampled_draft(d.cpu().numpy(), xh, Z, w1, w2, prev, "bf16", T, 131)
    c = check_verify_sample(out["accepted"].cpu().numpy(), out["bonus"].cpu().numpy(),
                            d.cpu().numpy(), xh, Yb, "bf16", np.full(B, k), T, 132)
    log(f"end-to-end sampled block: {c}")


# ----------------------------------------------------------------------------- randomized shapes
def _random_shapes(n, seed):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(g.choice([1, 1, 2, 3, 5, 16, 17, 33]))
        k = int(g.integers(1, 17))
        V = int(g.integers(16, 9000))
        dtype = str(g.choice(["bf16", "f32"]))
        r = int(g.choice([0, 8, 16, 32, 48, 64])) if dtype == "f32" else int(g.choice([0, 8, 32, 64]))
        out.append((B, k, V, r, dtype))
    return out


@pytest.mark.parametrize("shape", _random_shapes(12, 2026))
def test_chain_random_shapes(shape):
    """Greedy and sampled drafts over seeded random shapes (batch 1 to 33, k 1
    to 16, ragged vocabularies, ranks 0 to 64, both dtypes), every position
    checked against the oracle's rule from the GPU's own context."""
    B, k, V, r, dtype = shape
    cid = 300 + B * 7 + k * 13 + V % 97
    Z = _logits(cid, B, k, V, 3.0)
    w1, w2 = _markov(cid, V, r, dtype) if r else (None, None)
    prev = np.random.default_rng(cid).integers(0, V, B).astype(np.int32)
    log(f"random chain B={B} k={k} V={V} r={r} {dtype}")
    d = bdr().dspark_markov_argmax(dev(Z), dev(w1) if r else None, dev(w2) if r else None,
                                   dev(prev)).cpu().numpy()
    check_draft(d, Z, w1, w2, prev, dtype)
    T, seed = 0.9, 4000 + cid
    ds, xs = bdr().dspark_markov_sample(dev(Z), dev(w1) if r else None, dev(w2) if r else None,
                                        dev(prev), T, seed)
    check_sampled_draft(ds.cpu().numpy(), xs.cpu().numpy(), Z, w1, w2, prev, dtype, T, seed)
