"""GPU parity of each stage on small and mid-size seeded inputs that span several
tiles with ragged tails, plus the degenerate cases of the method.

Every call goes through the C ABI (libbdr) via the binding; expected values come
only from the CPU oracle.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
import workloads
from workloads import synth
from gpu_util import REL_TOL, check_draft, dev, host_bits, log, max_rel_err

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


# mid-size shapes: 3 m-tiles with a ragged row tail, ragged vocabulary, K tails
MID = {
    "mid_bf16": dataclasses.replace(workloads.get("b16"), cid=20, name="mid_bf16", batch=3,
                                    hidden=96, n_taps=3, k=5, vocab=4099, rank=16),
    "mid_f32": dataclasses.replace(workloads.get("tiny"), cid=21, name="mid_f32", batch=5,
                                   hidden=48, n_taps=4, fake_layers=0, tap_layers=(0, 1, 2, 3),
                                   k=6, vocab=2053, rank=12,
                                   plant_p=(0.76, 0.45, 0.31, 0.14, 0.10, 0.02)),
    "mid_bf16_b20": dataclasses.replace(workloads.get("b16"), cid=22, name="mid_bf16_b20",
                                        batch=20, hidden=64, n_taps=2, k=3, vocab=1031, rank=8),
    # the chain's [B, k] logits do not fit in LDS: prefetched into registers
    # position by position instead of staged once
    "mid_bf16_b40": dataclasses.replace(workloads.get("b16"), cid=23, name="mid_bf16_b40",
                                        batch=40, hidden=64, n_taps=2, k=7, vocab=3001, rank=24),
}


def _data(w, step=0):
    W = synth.make_weights(w)
    s = synth.make_step(w, step)
    return W, s


@pytest.mark.parametrize("name", list(MID))
def test_fc_parity_mid(name):
    w = MID[name]
    W, s = _data(w)
    log(f"fc parity {w.describe()} rows={w.rows}")
    ref = oracle.fuse_fc(s["taps"], W["fc_w"], w.dtype)
    out = bdr().dflash_fuse_fc([dev(t) for t in s["taps"]], dev(W["fc_w"]))
    got = oracle.widen(host_bits(out), w.dtype)
    err = max_rel_err(got, ref)
    log(f"  max rel err {err:.3e}")
    assert err <= REL_TOL[w.dtype]
    if w.dtype == "bf16":   # rounding of the fp32 sum to bf16 dominates: <= 2^-8 relative
        assert err <= 4e-3


@pytest.mark.parametrize("name", list(MID))
def test_lm_head_parity_mid(name):
    w = MID[name]
    W, s = _data(w)
    log(f"lm head parity {w.describe()}")
    ref = oracle.lm_head(s["draft_hidden"], W["lm_w"], w.dtype)
    got = bdr().dspark_lm_head(dev(s["draft_hidden"]), dev(W["lm_w"])).cpu().numpy()
    err = max_rel_err(got, ref)
    log(f"  max rel err {err:.3e}")
    assert err <= min(REL_TOL[w.dtype], 1e-3)


@pytest.mark.parametrize("name", list(MID))
def test_markov_parity_identical_logits(name):
    w = MID[name]
    W, s = _data(w)
    Z = oracle.lm_head(s["draft_hidden"], W["lm_w"], w.dtype)
    d = bdr().dspark_markov_argmax(dev(Z), dev(W["w1"]), dev(W["w2"]), dev(s["prev0"]))
    c = check_draft(d.cpu().numpy(), Z, W["w1"], W["w2"], s["prev0"], w.dtype)
    log(f"markov {name}: {c}")


@pytest.mark.parametrize("name", list(MID))
def test_draft_block_parity(name):
    w = MID[name]
    W, s = _data(w)
    Z = oracle.lm_head(s["draft_hidden"], W["lm_w"], w.dtype)
    logits = torch.full((w.batch, w.k, w.vocab), float("nan"), device="cuda")
    d = bdr().dspark_draft_block(dev(s["draft_hidden"]), dev(W["lm_w"]), dev(W["w1"]),
                                 dev(W["w2"]), dev(s["prev0"]), logits_out=logits)
    assert max_rel_err(logits.cpu().numpy(), Z) <= 1e-3
    check_draft(d.cpu().numpy(), Z, W["w1"], W["w2"], s["prev0"], w.dtype)
    # logits kept in the workspace gives the same tokens
    d2 = bdr().dspark_draft_block(dev(s["draft_hidden"]), dev(W["lm_w"]), dev(W["w1"]),
                                  dev(W["w2"]), dev(s["prev0"]))
    assert torch.equal(d, d2)


def _verify_both(w, d, Y, conf, acc0=None):
    L = oracle.truncate_by_confidence(conf, w.threshold, w.batch, w.k)
    t = oracle.target_argmax(Y, w.dtype, L)
    a, bonus, acc, prop = oracle.verify_greedy(d, t, L)
    accd = torch.zeros(w.k, dtype=torch.int64, device="cuda") if acc0 is None else acc0
    propd = torch.zeros(w.k, dtype=torch.int64, device="cuda")
    th = math.nan if w.threshold is None else w.threshold
    r = bdr().spec_verify_greedy(dev(Y), dev(d.astype(np.int32)),
                                 None if conf is None else dev(conf), th, accd, propd)
    assert np.array_equal(r["block_len"].cpu().numpy(), L)
    assert np.array_equal(r["target_argmax"].cpu().numpy(), t)
    assert np.array_equal(r["accepted"].cpu().numpy(), a)
    assert np.array_equal(r["bonus"].cpu().numpy(), bonus)
    return accd, propd, acc, prop


@pytest.mark.parametrize("name", list(MID))
@pytest.mark.parametrize("threshold", [None, 0.3])
def test_verify_parity_identical_inputs(name, threshold):
    w = dataclasses.replace(MID[name], threshold=threshold)
    for step in range(3):
        d = synth.random_drafts(w, step)
        s = synth.make_step(w, step)
        Y = synth.plant_targets(w, step, s["noise"], d)["target_logits"]
        conf = synth.make_confidence(w, step)
        accd, propd, acc, prop = _verify_both(w, d, Y, conf)
        assert np.array_equal(accd.cpu().numpy(), acc)
        assert np.array_equal(propd.cpu().numpy(), prop)


def test_verify_counts_accumulate():
    w = MID["mid_bf16"]
    d = synth.random_drafts(w, 0)
    Y = synth.plant_targets(w, 0, synth.make_step(w, 0)["noise"], d)["target_logits"]
    acc0 = torch.full((w.k,), 1000, dtype=torch.int64, device="cuda")
    accd, _, acc, _ = _verify_both(w, d, Y, None, acc0=acc0)
    assert np.array_equal(accd.cpu().numpy(), acc + 1000)


# ----------------------------------------------------------------------------- edge cases

def test_single_row_context():
    """rows = 1: a one-token context through the fc (the short-prompt edge case
    in the replication report of llm-scaler PR #620)."""
    g = np.random.default_rng(1)
    H, T = 128, 5
    taps = [synth.to_bf16_bits(g.standard_normal((1, H)).astype(np.float32)) for _ in range(T)]
    Wf = synth.to_bf16_bits((g.standard_normal((H, T * H)) / np.sqrt(T * H)).astype(np.float32))
    ref = oracle.fuse_fc(taps, Wf, "bf16")
    out = bdr().dflash_fuse_fc([dev(t) for t in taps], dev(Wf))
    assert max_rel_err(oracle.widen(host_bits(out), "bf16"), ref) <= 4e-3


def test_k1_and_vocab_one():
    g = np.random.default_rng(2)
    for V in (1, 17, 64):
        Z = g.standard_normal((2, 1, V)).astype(np.float32)
        w1 = synth.to_bf16_bits(g.standard_normal((V, 8)).astype(np.float32))
        w2 = synth.to_bf16_bits(g.standard_normal((V, 8)).astype(np.float32))
        prev = g.integers(0, V, 2).astype(np.int32)
        d = bdr().dspark_markov_argmax(dev(Z), dev(w1), dev(w2), dev(prev)).cpu().numpy()
        check_draft(d, Z, w1, w2, prev, "bf16")
        if V == 1:
            assert d.tolist() == [[0], [0]]


def test_empty_batch_is_a_noop():
    V, k = 100, 3
    Y = torch.zeros((0, k + 1, V), dtype=torch.bfloat16, device="cuda")
    d = torch.zeros((0, k), dtype=torch.int32, device="cuda")
    acc = torch.full((k,), 7, dtype=torch.int64, device="cuda")
    r = bdr().spec_verify_greedy(Y, d, accept_counts=acc)
    torch.cuda.synchronize()
    assert acc.tolist() == [7, 7, 7] and r["accepted"].numel() == 0
    Z = torch.zeros((0, k, V), dtype=torch.float32, device="cuda")
    out = bdr().dspark_markov_argmax(Z, None, None, torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert out.shape == (0, k)


def test_exact_ties_across_tiles_and_tail():
    """Equal maxima placed in different workgroups / chunks and at V-1: the
    lowest index wins; -0.0 ties +0.0."""
    V, k = 151936, 4
    Z = np.full((3, k, V), -3.0, np.float32)
    Z[0, 0, [150000, 77, 151935]] = 5.0
    Z[0, 1, [151935, 151934]] = 5.0
    Z[0, 2, [40000, 120000]] = 5.0
    Z[0, 3, 3] = -0.0                     # -0.0 at the lower index ...
    Z[0, 3, 9] = 0.0                      # ... ties +0.0: index 3 wins
    Z[0, 3, :3] = -4.0
    Z[1] = Z[0, ::-1]
    Z[2, :, :] = 1.0                      # every entry ties: index 0
    d_ref, _ = oracle.semi_ar_argmax(Z, None, None, np.zeros(3, np.int32), "f32")
    d = bdr().dspark_markov_argmax(dev(Z), None, None, dev(np.zeros(3, np.int32))).cpu().numpy()
    assert np.array_equal(d, d_ref)
    # same rows as bf16 target logits through verification
    Yb = synth.to_bf16_bits(np.concatenate([Z, Z[:, :1]], axis=1))
    t_ref = oracle.target_argmax(Yb, "bf16")
    r = bdr().spec_verify_greedy(dev(Yb), dev(d_ref.astype(np.int32)))
    assert np.array_equal(r["target_argmax"].cpu().numpy(), t_ref)


def test_single_row_chain_ties_and_edges():
    """B = 1 takes its own chain path (the bias product transposed, one
    vocabulary entry per lane): exact ties across workgroups and at V-1,
    -0.0 against +0.0 and all-equal rows, with no Markov head and with zero
    bf16 Markov weights (bias exactly 0 through the MFMAs); k = 1 with tiny
    vocabularies; zero weights against the plain argmax."""
    V, k = 151936, 4
    Z = np.full((3, k, V), -3.0, np.float32)
    Z[0, 0, [150000, 77, 151935]] = 5.0
    Z[0, 1, [151935, 151934]] = 5.0
    Z[0, 2, [40000, 120000]] = 5.0
    Z[0, 3, 3] = -0.0
    Z[0, 3, 9] = 0.0
    Z[0, 3, :3] = -4.0
    Z[1] = Z[0, ::-1]
    Z[2, :, :] = 1.0
    zeros = np.zeros((V, 32), np.uint16)
    for b in range(3):
        Zb = np.ascontiguousarray(Z[b:b + 1])
        prev = np.array([b * 1000 + 5], np.int32)
        d_ref, _ = oracle.semi_ar_argmax(Zb, None, None, prev, "f32")
        d = bdr().dspark_markov_argmax(dev(Zb), None, None, dev(prev)).cpu().numpy()
        assert np.array_equal(d, d_ref), (b, d, d_ref)
        d = bdr().dspark_markov_argmax(dev(Zb), dev(zeros), dev(zeros), dev(prev)).cpu().numpy()
        assert np.array_equal(d, d_ref), (b, d, d_ref)
    g = np.random.default_rng(12)
    for V in (1, 17, 64, 1000):
        Zs = g.standard_normal((1, 1, V)).astype(np.float32)
        w1 = synth.to_bf16_bits(g.standard_normal((V, 8)).astype(np.float32))
        w2 = synth.to_bf16_bits(g.standard_normal((V, 8)).astype(np.float32))
        prev = g.integers(0, V, 1).astype(np.int32)
        d = bdr().dspark_markov_argmax(dev(Zs), dev(w1), dev(w2), dev(prev)).cpu().numpy()
        check_draft(d, Zs, w1, w2, prev, "bf16")
    Z1 = g.standard_normal((1, 6, 3001)).astype(np.float32)
    w = synth.to_bf16_bits(g.standard_normal((3001, 32)).astype(np.float32))
    z32 = np.zeros((3001, 32), np.uint16)
    for w1, w2 in ((z32, w), (w, z32)):
        d = bdr().dspark_markov_argmax(dev(Z1), dev(w1), dev(w2), dev(np.array([7], np.int32)))
        assert np.array_equal(d.cpu().numpy(), np.argmax(Z1, axis=-1))


@pytest.mark.parametrize("dtype,r", [("bf16", 64), ("f32", 24), ("f32", 48), ("f32", 64)])
def test_single_row_chain_ranks(dtype, r):
    """B = 1 chain with two to four operand chunks of the Markov rank (bf16
    r = 64; fp32 r = 24, 48, 64) over a ragged vocabulary."""
    g = np.random.default_rng(r)
    k, V = 6, 20011
    Z = (g.standard_normal((1, k, V)) * 3.0).astype(np.float32)
    w = [(g.standard_normal((V, r)) * 0.4).astype(np.float32) for _ in range(2)]
    w1, w2 = [synth.store(x, dtype) for x in w]
    prev = g.integers(0, V, 1).astype(np.int32)
    d = bdr().dspark_markov_argmax(dev(Z), dev(w1), dev(w2), dev(prev)).cpu().numpy()
    c = check_draft(d, Z, w1, w2, prev, dtype)
    log(f"B=1 chain {dtype} r={r}: {c}")


def test_zero_markov_equals_plain_argmax():
    g = np.random.default_rng(4)
    B, k, V, r = 4, 6, 3001, 32
    Z = g.standard_normal((B, k, V)).astype(np.float32)
    zeros = np.zeros((V, r), np.uint16)
    w = synth.to_bf16_bits(g.standard_normal((V, r)).astype(np.float32))
    prev = g.integers(0, V, B).astype(np.int32)
    want = np.argmax(Z, axis=-1)
    for w1, w2 in ((zeros, w), (w, zeros)):
        d = bdr().dspark_markov_argmax(dev(Z), dev(w1), dev(w2), dev(prev)).cpu().numpy()
        assert np.array_equal(d, want)
    d = bdr().dspark_markov_argmax(dev(Z), None, None, dev(prev)).cpu().numpy()
    assert np.array_equal(d, want)


def test_planted_successor_map_on_gpu():
    V, r, k, B = 4096, 8, 16, 5
    sigma = np.array([13, 4000, 2, 777, 61, 3000, 1, 4095])
    w1 = np.zeros((V, r), np.float32)
    w1[np.arange(V), np.arange(V) % r] = 1.0
    w2 = np.zeros((V, r), np.float32)
    w2[sigma, np.arange(r)] = 100.0
    prev = np.array([5, 50, 96, 13, 4095], np.int32)
    Z = np.zeros((B, k, V), np.float32)
    d = bdr().dspark_markov_argmax(dev(Z), dev(synth.to_bf16_bits(w1)), dev(synth.to_bf16_bits(w2)),
                                   dev(prev)).cpu().numpy()
    for b in range(B):
        p = prev[b]
        for i in range(k):
            p = sigma[p % r]
            assert d[b, i] == p


def test_block_truncated_to_zero_and_max_sizes():
    """L = 0 rows (first confidence below threshold), k = 16, rank = 128, 8 taps."""
    w = dataclasses.replace(MID["mid_bf16"], cid=23, k=16, rank=128, n_taps=8, hidden=64,
                            batch=6, threshold=0.5,
                            plant_hi=tuple(0.9 * 0.85 ** i for i in range(16)),
                            plant_lo=tuple(0.6 * 0.5 ** i for i in range(16)))
    d = synth.random_drafts(w, 0)
    Y = synth.plant_targets(w, 0, synth.make_step(w, 0)["noise"], d)["target_logits"]
    conf = synth.make_confidence(w, 0)
    conf[0, 0] = 0.1                                  # row 0: L = 0
    conf[1, :] = 0.9                                  # row 1: full block
    accd, propd, acc, prop = _verify_both(w, d, Y, conf)
    assert np.array_equal(accd.cpu().numpy(), acc) and np.array_equal(propd.cpu().numpy(), prop)
    W, s = _data(w)
    ref = oracle.fuse_fc(s["taps"], W["fc_w"], w.dtype)
    out = bdr().dflash_fuse_fc([dev(t) for t in s["taps"]], dev(W["fc_w"]))
    assert max_rel_err(oracle.widen(host_bits(out), w.dtype), ref) <= 4e-3
    Z = oracle.lm_head(s["draft_hidden"], W["lm_w"], w.dtype)
    dg = bdr().dspark_markov_argmax(dev(Z), dev(W["w1"]), dev(W["w2"]), dev(s["prev0"]))
    check_draft(dg.cpu().numpy(), Z, W["w1"], W["w2"], s["prev0"], w.dtype)


@pytest.mark.parametrize("B", [17, 256, 257])
def test_markov_row_count_limits(B):
    """Row counts at the chain's limits: a second row group holding one row
    (17); the most rows whose contexts the chain keeps in LDS (256), where some
    workgroups reduce two rows (3001 entries: 188 workgroups); one row more
    (257), which takes one launch per position."""
    g = np.random.default_rng(100 + B)
    k, V, r = 3, 3001, 16
    Z = (g.standard_normal((B, k, V)) * 4.0).astype(np.float32)
    w1 = synth.to_bf16_bits((g.standard_normal((V, r)) * 0.5).astype(np.float32))
    w2 = synth.to_bf16_bits((g.standard_normal((V, r)) * 0.5).astype(np.float32))
    prev = g.integers(0, V, B).astype(np.int32)
    d = bdr().dspark_markov_argmax(dev(Z), dev(w1), dev(w2), dev(prev)).cpu().numpy()
    c = check_draft(d, Z, w1, w2, prev, "bf16")
    log(f"markov B={B}: {c}")


@pytest.mark.parametrize("B", [7, 8, 16, 33])
def test_chain_wave_layouts(B):
    """Both chain layouts against the oracle at the full vocabulary and rank
    64: five waves (a hand-off wave beside four compute waves) below eight
    rows, four waves (wave 0 compares its tiles, then takes the hand-off) from
    eight on; 7 and 8 sit on either side of the switch, 33 takes three row
    groups, the last holding one row."""
    g = np.random.default_rng(900 + B)
    k, V, r = 8, 151936, 64
    Z = (g.standard_normal((B, k, V)) * 3).astype(np.float32)
    w1 = synth.to_bf16_bits(g.standard_normal((V, r)).astype(np.float32))
    w2 = synth.to_bf16_bits((g.standard_normal((V, r)) * 0.3).astype(np.float32))
    prev = g.integers(0, V, B).astype(np.int32)
    d = bdr().dspark_markov_argmax(dev(Z), dev(w1), dev(w2), dev(prev)).cpu().numpy()
    c = check_draft(d, Z, w1, w2, prev, "bf16")
    log(f"chain B={B}: {c}")


def test_sentinel_outputs_all_written_and_deterministic():
    w = MID["mid_bf16"]
    W, s = _data(w)
    outs = []
    for _ in range(2):
        out = torch.full((w.rows, w.hidden), 12345.0, dtype=torch.bfloat16, device="cuda")
        bdr().dflash_fuse_fc([dev(t) for t in s["taps"]], dev(W["fc_w"]), out=out)
        logits = torch.full((w.batch, w.k, w.vocab), float("nan"), device="cuda")
        dd = torch.full((w.batch, w.k), -7, dtype=torch.int32, device="cuda")
        bdr().dspark_draft_block(dev(s["draft_hidden"]), dev(W["lm_w"]), dev(W["w1"]),
                                 dev(W["w2"]), dev(s["prev0"]), draft_tokens=dd, logits_out=logits)
        torch.cuda.synchronize()
        assert not torch.isnan(logits).any()
        assert not (out == 12345.0).any()
        assert (dd >= 0).all() and (dd < w.vocab).all()
        outs.append((out.clone(), logits.clone(), dd.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)          # bitwise identical run to run


def test_workspace_reuse_and_restored_to_zero():
    """One zero-filled workspace per entry point reused across calls with
    different inputs gives the results of fresh workspaces, and is left zeroed."""
    w = MID["mid_bf16"]
    W, _ = _data(w)
    m = bdr()
    ws_fc = torch.zeros(m.workspace_bytes("fc", rows=w.rows, hidden=w.hidden, n_taps=w.n_taps,
                                          dtype=m.BDR_BF16) + 256, dtype=torch.uint8, device="cuda")
    ws_dr = torch.zeros(m.workspace_bytes("draft", batch=w.batch, k=w.k, vocab=w.vocab) + 256,
                        dtype=torch.uint8, device="cuda")
    ws_v = torch.zeros(m.workspace_bytes("verify", batch=w.batch, k=w.k, vocab=w.vocab) + 256,
                       dtype=torch.uint8, device="cuda")
    for step in range(3):
        s = synth.make_step(w, step)
        F1 = m.dflash_fuse_fc([dev(t) for t in s["taps"]], dev(W["fc_w"]), workspace=ws_fc)
        F2 = m.dflash_fuse_fc([dev(t) for t in s["taps"]], dev(W["fc_w"]))
        d1 = m.dspark_draft_block(dev(s["draft_hidden"]), dev(W["lm_w"]), dev(W["w1"]),
                                  dev(W["w2"]), dev(s["prev0"]), workspace=ws_dr)
        d2 = m.dspark_draft_block(dev(s["draft_hidden"]), dev(W["lm_w"]), dev(W["w1"]),
                                  dev(W["w2"]), dev(s["prev0"]))
        Y = synth.plant_targets(w, step, s["noise"], d2.cpu().numpy())["target_logits"]
        r1 = m.spec_verify_greedy(dev(Y), d1, workspace=ws_v)
        r2 = m.spec_verify_greedy(dev(Y), d2)
        torch.cuda.synchronize()
        assert torch.equal(F1, F2) and torch.equal(d1, d2)
        for key in r2:
            assert torch.equal(r1[key], r2[key]), key
    # keys, barrier counter and error word are back at zero; the draft workspace
    # holds the logits first, the verify workspace ends with its counter block
    for t in (ws_fc, ws_dr, ws_v):
        assert t.data_ptr() % 256 == 0
    logits_bytes = (w.batch * w.k * w.vocab * 4 + 255) // 256 * 256
    need_dr = m.workspace_bytes("draft", batch=w.batch, k=w.k, vocab=w.vocab)
    assert int(ws_dr[logits_bytes:need_dr].count_nonzero()) == 0
    need_v = m.workspace_bytes("verify", batch=w.batch, k=w.k, vocab=w.vocab)
    assert int(ws_v[need_v - 256 - 16 * 128:need_v].count_nonzero()) == 0


def test_graph_replay_matches_eager():
    """A HIP graph of the whole step replayed several times, with eager work in
    between, reproduces the eager results every time."""
    w = MID["mid_bf16"]
    W, s = _data(w)
    m = bdr()
    gW = {k: dev(v) for k, v in W.items()}
    taps = [dev(t) for t in s["taps"]]
    hid, prev = dev(s["draft_hidden"]), dev(s["prev0"])
    Yd = dev(synth.plant_targets(w, 0, s["noise"], synth.random_drafts(w, 0))["target_logits"])
    F = torch.empty((w.rows, w.hidden), dtype=torch.bfloat16, device="cuda")
    d = torch.empty((w.batch, w.k), dtype=torch.int32, device="cuda")
    out = {"block_len": torch.empty(w.batch, dtype=torch.int32, device="cuda"),
           "accepted": torch.empty(w.batch, dtype=torch.int32, device="cuda"),
           "bonus": torch.empty(w.batch, dtype=torch.int32, device="cuda"),
           "target_argmax": torch.empty((w.batch, w.k + 1), dtype=torch.int32, device="cuda")}
    acc = torch.zeros(w.k, dtype=torch.int64, device="cuda")
    ws = {k: torch.zeros(m.workspace_bytes(k, **a) + 256, dtype=torch.uint8, device="cuda")
          for k, a in (("fc", dict(rows=w.rows, hidden=w.hidden, n_taps=w.n_taps, dtype=m.BDR_BF16)),
                       ("draft", dict(batch=w.batch, k=w.k, vocab=w.vocab)),
                       ("verify", dict(batch=w.batch, k=w.k, vocab=w.vocab)))}

    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")

    def step():
        m.dflash_fuse_fc(taps, gW["fc_w"], out=F, workspace=ws["fc"])
        m.dspark_draft_block(hid, gW["lm_w"], gW["w1"], gW["w2"], prev, draft_tokens=d,
                             workspace=ws["draft"], status=status, check=False)
        m.spec_verify_greedy(Yd, d, accept_counts=acc, out=out, workspace=ws["verify"])

    step()
    torch.cuda.synchronize()
    eager = [F.clone(), d.clone()] + [out[k].clone() for k in sorted(out)]
    acc_eager = acc.clone()
    g = torch.cuda.CUDAGraph()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_cap):
        step()                                   # warm on the capture stream
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in [F, d] + list(out.values()):
            t.fill_(-3) if t.dtype == torch.int32 else t.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [F, d] + [out[k] for k in sorted(out)]
        for a, b in zip(got, eager):
            assert torch.equal(a, b), f"replay {rep}"
        assert int(status.item()) == 0
        status.fill_(-1)
        # eager work between replays
        step()
        torch.cuda.synchronize()
    # counts: eager once + warm-up + 4 replays + 4 eager = 10 accumulations
    assert torch.equal(acc, acc_eager * 10)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_chain_time_out_is_reported(B):
    """The chain's bounded waits made to give up (the host's error-path hook,
    which has every wait disregard what it reads, with a limit of 0): every
    kernel still runs to completion, every draft token is -1, the status word
    reports the time-out and the binding raises; the error word does not
    outlive the call that reported it, and with the hook off and the default
    limit the same call reports 0 and drafts the oracle's tokens."""
    g = np.random.default_rng(700 + B)
    k, V, r = 8, 151936, 64
    Z = (g.standard_normal((B, k, V)) * 3).astype(np.float32)
    w1 = synth.to_bf16_bits(g.standard_normal((V, r)).astype(np.float32))
    w2 = synth.to_bf16_bits((g.standard_normal((V, r)) * 0.3).astype(np.float32))
    prev = g.integers(0, V, B).astype(np.int32)
    m = bdr()
    Zd, w1d, w2d, pd = dev(Z), dev(w1), dev(w2), dev(prev)
    ws = torch.zeros(m.workspace_bytes("markov", batch=B, k=k) + 256, dtype=torch.uint8,
                     device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    m.set_markov_poll_timeout_us(0.0)
    m.set_markov_forced_time_out(True)
    try:
        log(f"chain time-out B={B}: waits forced to give up, limit 0 us")
        d = m.dspark_markov_argmax(Zd, w1d, w2d, pd, workspace=ws, status=status, check=False)
        torch.cuda.synchronize()
        assert int(status.item()) != 0
        assert bool((d == -1).all())
        with pytest.raises(m.BdrError) as e:
            m.dspark_markov_argmax(Zd, w1d, w2d, pd, workspace=ws)
        assert e.value.code == m.MARKOV_TIMED_OUT
    finally:
        m.set_markov_forced_time_out(False)
        m.set_markov_poll_timeout_us(-1.0)
    torch.cuda.synchronize()
    d = m.dspark_markov_argmax(Zd, w1d, w2d, pd, workspace=ws, status=status, check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_draft(d.cpu().numpy(), Z, w1, w2, prev, "bf16")
    base = (ws.data_ptr() + 255) // 256 * 256 - ws.data_ptr()
    assert int(ws[base:base + m.workspace_bytes("markov", batch=B, k=k)].count_nonzero()) == 0


def _verify_random_shapes(n, seed):
    g = np.random.default_rng(seed)
    return [(int(g.choice([1, 2, 3, 8, 16, 17, 40])), int(g.integers(1, 17)), int(g.integers(8, 20000)),
             str(g.choice(["bf16", "f32"])), bool(g.integers(0, 2))) for _ in range(n)]


@pytest.mark.parametrize("shape", _verify_random_shapes(12, 77))
def test_verify_random_shapes(shape):
    """Greedy verification over seeded random shapes (batch 1 to 40, k 1 to 16,
    ragged vocabularies, bf16 and fp32 targets, with and without confidence
    truncation), drafts planted to match the target on a random prefix:
    block lengths, accepted counts, bonus tokens, target argmaxes and counts
    bit-exact against the oracle."""
    B, k, V, dtype, use_conf = shape
    g = np.random.default_rng(B * 1000 + k * 37 + V)
    Y = synth.store((g.standard_normal((B, k + 1, V)) * 2.0).astype(np.float32), dtype)
    t_all = oracle.target_argmax(Y, dtype, np.full(B, k))
    d = g.integers(0, V, (B, k)).astype(np.int32)
    for b in range(B):
        m = int(g.integers(0, k + 1))
        d[b, :m] = t_all[b, :m]
    conf = g.uniform(0.0, 1.0, (B, k)).astype(np.float32) if use_conf else None
    th = 0.2 if use_conf else None
    L = oracle.truncate_by_confidence(conf, th, B, k)
    t = oracle.target_argmax(Y, dtype, L)
    a, bonus, acc, prop = oracle.verify_greedy(d, t, L)
    accd = torch.zeros(k, dtype=torch.int64, device="cuda")
    propd = torch.zeros(k, dtype=torch.int64, device="cuda")
    r = bdr().spec_verify_greedy(dev(Y), dev(d), None if conf is None else dev(conf),
                                 math.nan if th is None else th, accd, propd)
    log(f"verify B={B} k={k} V={V} {dtype} conf={use_conf}: accepted {int(a.sum())}")
    assert np.array_equal(r["block_len"].cpu().numpy(), L)
    assert np.array_equal(r["target_argmax"].cpu().numpy(), t)
    assert np.array_equal(r["accepted"].cpu().numpy(), a)
    assert np.array_equal(r["bonus"].cpu().numpy(), bonus)
    assert np.array_equal(accd.cpu().numpy(), acc) and np.array_equal(propd.cpu().numpy(), prop)
