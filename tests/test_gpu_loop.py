"""GPU parity of closing the loop between block-steps: the commit of a verified
block, the fc on the accepted rows, and several block-steps chained on the
device (each step's Markov context is the previous step's bonus token, taken
on the device with no host round trip), against the closed-loop oracle.

Near-ties follow the usual protocol: a row whose acceptance was decided at or
after its first near-tie draft position (oracle top-2 gap < 1e-2) may
legitimately diverge; it is reported, and from then on only the rows that did
not diverge are compared (the fc of a step is compared when no row diverged).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads
from oracle import loop
from workloads import synth
from gpu_util import NEAR_TIE, REL_TOL, dev, first_near_tie, host_bits, log, max_rel_err, weights

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


@pytest.mark.parametrize("B,k", [(1, 7), (5, 3), (300, 4), (1000, 16)])
def test_commit_matches_oracle(B, k):
    rng = np.random.default_rng(B * 31 + k)
    d = rng.integers(0, 5000, size=(B, k)).astype(np.int32)
    L = rng.integers(0, k + 1, size=B).astype(np.int32)
    a = np.array([rng.integers(0, l + 1) for l in L], dtype=np.int32)
    bonus = rng.integers(0, 5000, size=B).astype(np.int32)
    ref = loop.commit_step(d, a, bonus, L)
    got = bdr().spec_commit(dev(d), dev(a), dev(bonus), dev(L))
    got = {n: t.cpu().numpy() for n, t in got.items()}
    n = int(got["row_count"][0])
    assert n == ref["row_count"]
    assert np.array_equal(got["row_index"][:n], ref["row_index"])
    for name in ("next_prev", "emitted", "draft_list", "row_offsets"):
        assert np.array_equal(got[name], ref[name]), name


def test_commit_full_blocks_without_block_len():
    d = np.arange(12, dtype=np.int32).reshape(3, 4)
    a = np.array([4, 0, 2], dtype=np.int32)
    bonus = np.array([90, 91, 92], dtype=np.int32)
    got = bdr().spec_commit(dev(d), dev(a), dev(bonus))
    ref = loop.commit_step(d, a, bonus, np.full(3, 4))
    assert np.array_equal(got["draft_list"].cpu().numpy(), ref["draft_list"])
    assert np.array_equal(got["emitted"].cpu().numpy(), ref["emitted"])


@pytest.mark.parametrize("dtype,H,T,rows", [("bf16", 512, 5, 40), ("f32", 64, 5, 20),
                                            ("bf16", 2560, 5, 36)])
def test_fc_on_accepted_rows(dtype, H, T, rows):
    rng = np.random.default_rng(H + rows)
    taps = [synth.store(synth.normal_f32((rows, H), (91, 1, H, t)), dtype) for t in range(T)]
    fc_w = synth.store(synth.normal_f32((H, T * H), (91, 0, H, 0), (1.0 / (T * H)) ** 0.5), dtype)
    idx = np.sort(rng.choice(rows, size=rows // 3, replace=False)).astype(np.int32)
    row_index = np.full(rows, -7, dtype=np.int32)
    row_index[:idx.size] = idx
    count = np.array([idx.size], dtype=np.int32)
    out = bdr().dflash_fuse_fc_rows([dev(t) for t in taps], dev(fc_w), dev(row_index), dev(count))
    got = oracle.widen(host_bits(out), dtype)
    ref = loop.fuse_fc_rows(taps, idx, fc_w, dtype)
    err = max_rel_err(got[:idx.size], ref)
    log(f"fc rows {dtype} H={H}: {idx.size}/{rows} rows, max rel err {err:.3e}")
    assert err <= (4e-3 if dtype == "bf16" else REL_TOL["f32"])
    assert np.all(got[idx.size:] == 0)


LOOP_CASES = {
    "mid_bf16": (dataclasses.replace(workloads.get("b16"), cid=95, name="loop_mid", batch=3,
                                     hidden=96, n_taps=3, k=5, vocab=4099, rank=16), 6),
    "flashnext_b4": (workloads.get("flashnext_b4"), 3),
}


@pytest.mark.parametrize("name", list(LOOP_CASES))
def test_closed_loop_on_device(name):
    w, steps = LOOP_CASES[name]
    W = weights(w.name) if w.name == "flashnext_b4" else synth.make_weights(w)
    inputs = [synth.make_step(w, s) for s in range(steps)]
    planted = {}

    def Y(s, d):
        planted[s] = synth.plant_targets(w, s, inputs[s]["noise"], d)["target_logits"]
        return planted[s]

    log(f"closed loop {w.describe()}, {steps} steps: oracle")
    ref = loop.closed_loop(w.dtype, steps, inputs[0]["prev0"], W["fc_w"], W["lm_w"], W["w1"],
                           W["w2"], lambda s: inputs[s], Y)
    B, k, H, V = w.batch, w.k, w.hidden, w.vocab
    g = {n: dev(W[n]) for n in ("fc_w", "lm_w", "w1", "w2")}
    prev = dev(inputs[0]["prev0"])
    rec = []
    for s in range(steps):   # all on the device: prev is the previous commit's output
        Z = bdr().dspark_lm_head(dev(inputs[s]["draft_hidden"]), g["lm_w"])
        d = bdr().dspark_markov_argmax(Z, g["w1"], g["w2"], prev)
        v = bdr().spec_verify_greedy(dev(planted[s]), d, target_argmax=False)
        c = bdr().spec_commit(d, v["accepted"], v["bonus"], v["block_len"])
        F = bdr().dflash_fuse_fc_rows([dev(t) for t in inputs[s]["taps"]], g["fc_w"],
                                      c["row_index"], c["row_count"])
        rec.append(dict(d=d, accepted=v["accepted"], bonus=v["bonus"], F=F, **c))
        prev = c["next_prev"]
    torch.cuda.synchronize()
    live = np.ones(B, dtype=bool)          # rows whose context chain still agrees
    n_rows_fc = 0
    for s in range(steps):
        o, r = ref[s], {n: host_bits(t) for n, t in rec[s].items()}
        istar = first_near_tie(o["gap"])
        got = oracle.widen(r["F"], w.dtype)
        for b in range(B):
            if not live[b]:
                continue
            m = int(istar[b])
            assert np.array_equal(r["d"][b, :m], o["draft_tokens"][b, :m]), (s, b)
            if m <= min(int(o["accepted"][b]), int(o["block_len"][b]) - 1):
                live[b] = False          # acceptance decided by a near-tie: may diverge
                log(f"  step {s} row {b}: near-tie at {m}, row left out from here")
                continue
            a = int(o["accepted"][b])
            assert r["accepted"][b] == a, (s, b)
            assert r["bonus"][b] == o["bonus"][b], (s, b)
            assert np.array_equal(r["emitted"][b], o["emitted"][b]), (s, b)
            assert r["next_prev"][b] == o["next_prev"][b]
            # this row's accepted rows in each side's gathered fc output
            g0, o0 = int(r["row_offsets"][b]), int(o["row_offsets"][b])
            assert np.array_equal(r["row_index"][g0:g0 + a + 1], o["row_index"][o0:o0 + a + 1])
            err = max_rel_err(got[g0:g0 + a + 1], o["fc_out"][o0:o0 + a + 1])
            assert err <= (4e-3 if w.dtype == "bf16" else REL_TOL["f32"]), (s, b, err)
            n_rows_fc += a + 1
        if live.all():
            assert int(r["row_count"][0]) == o["row_count"]
    log(f"  rows compared to the end: {int(live.sum())}/{B}; fc rows compared: {n_rows_fc}")
    assert live.sum() >= B - 1
