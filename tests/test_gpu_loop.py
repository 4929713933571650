"""GPU parity of closing the loop between block-steps: the commit of a verified
block, the fc on the accepted rows, and several block-steps chained on the
device (each step's Markov context is the previous step's bonus token, taken
on the device with no host round trip), against the closed-loop oracle.

The comparison follows the GPU's own path: at every step each draft position
is checked against the oracle's rule with the GPU's previous token as context
(bit-exact where the oracle's top-2 gap is >= 1e-2, an admissible pick below
it), then the oracle verifies and commits the GPU's draft, and every row's
accepted length, bonus, committed tokens, next context, gathered rows and fc
output are compared -- so a near-tie that the GPU took the other way changes
the path, never the coverage.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads
from oracle import loop
from workloads import synth
from gpu_util import REL_TOL, check_draft, dev, host_bits, log, max_rel_err, weights

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
    prev_g = np.asarray(inputs[0]["prev0"], dtype=np.int64)
    n_near = n_rows_fc = 0
    for s in range(steps):
        o, r = ref[s], {n: host_bits(t) for n, t in rec[s].items()}
        c = check_draft(r["d"], o["logits"], W["w1"], W["w2"], prev_g, w.dtype)
        n_near += c["other_side"]
        L = oracle.truncate_by_confidence(inputs[s].get("confidence"), None, B, k)
        t = oracle.target_argmax(planted[s], w.dtype, L)
        a, bonus, _, _ = oracle.verify_greedy(r["d"], t, L)
        cm = loop.commit_step(r["d"], a, bonus, L)
        assert np.array_equal(r["accepted"], a), s
        assert np.array_equal(r["bonus"], bonus), s
        for n in ("emitted", "next_prev", "draft_list", "row_offsets"):
            assert np.array_equal(r[n], cm[n]), (s, n)
        n = int(r["row_count"][0])
        assert n == cm["row_count"] and np.array_equal(r["row_index"][:n], cm["row_index"]), s
        F_ref = loop.fuse_fc_rows(inputs[s]["taps"], cm["row_index"], W["fc_w"], w.dtype)
        err = max_rel_err(oracle.widen(r["F"], w.dtype)[:n], F_ref)
        assert err <= (4e-3 if w.dtype == "bf16" else REL_TOL["f32"]), (s, err)
        n_rows_fc += n
        prev_g = cm["next_prev"]
    log(f"  every row compared at every step; fc rows compared: {n_rows_fc}; near-tie "
        f"positions where the GPU took the other admissible token: {n_near}")
