"""Pins of the closed-loop oracle (oracle.loop): a hand-worked commit, the
invariants every commit satisfies, the fc on gathered rows against the fc on all
rows, and the loop's step-to-step hand-over (the bonus token becomes the next
Markov context; the committed tokens are the target's own greedy tokens)."""
import numpy as np

import oracle
from oracle import loop
from workloads import synth
import workloads
import dataclasses


def test_commit_hand_example():
    d = np.array([[5, 6, 7], [1, 2, 3]])
    c = loop.commit_step(d, accepted=np.array([2, 0]), bonus=np.array([9, 4]),
                         block_len=np.array([3, 1]))
    assert c["emitted"].tolist() == [[5, 6, 9, -1], [4, -1, -1, -1]]
    assert c["n_emitted"].tolist() == [3, 1]
    assert c["row_index"].tolist() == [0, 1, 2, 4]
    assert c["row_count"] == 4
    assert c["row_offsets"].tolist() == [0, 3, 4]
    assert c["draft_list"].tolist() == [[5, 6, 7], [1, -1, -1]]
    assert c["next_prev"].tolist() == [9, 4]


def test_commit_invariants():
    rng = np.random.default_rng(3)
    for _ in range(200):
        B, k = int(rng.integers(1, 9)), int(rng.integers(1, 8))
        d = rng.integers(0, 50, size=(B, k))
        L = rng.integers(0, k + 1, size=B)
        a = np.array([rng.integers(0, l + 1) for l in L])
        bonus = rng.integers(0, 50, size=B)
        c = loop.commit_step(d, a, bonus, L)
        assert c["row_count"] == int(np.sum(a + 1)) == c["row_index"].size
        assert np.all(np.diff(c["row_index"]) > 0)
        for r in c["row_index"]:
            b, j = divmod(int(r), k + 1)
            assert j <= a[b]
        for b in range(B):
            assert np.array_equal(c["emitted"][b, :a[b]], d[b, :a[b]])
            assert c["emitted"][b, a[b]] == bonus[b]
            assert np.all(c["emitted"][b, a[b] + 1:] == -1)
            assert np.array_equal(c["draft_list"][b, :L[b]], d[b, :L[b]])
            assert np.all(c["draft_list"][b, L[b]:] == -1)
            assert c["row_offsets"][b + 1] - c["row_offsets"][b] == a[b] + 1


def test_fc_on_gathered_rows_is_the_fc_of_those_rows():
    rng = np.random.default_rng(4)
    T, rows, H = 3, 12, 16
    taps = [rng.standard_normal((rows, H)).astype(np.float32) for _ in range(T)]
    fc_w = rng.standard_normal((H, T * H)).astype(np.float32)
    idx = np.array([0, 3, 4, 11])
    F_all = oracle.fuse_fc(taps, fc_w, "f32")
    assert np.array_equal(loop.fuse_fc_rows(taps, idx, fc_w, "f32"), F_all[idx])


def _tiny(steps):
    w = dataclasses.replace(workloads.get("tiny"), cid=30, name="loop_tiny", batch=3)
    W = synth.make_weights(w)
    inputs = [synth.make_step(w, s) for s in range(steps)]
    return w, W, inputs


def test_closed_loop_hands_the_bonus_to_the_next_step():
    steps = 4
    w, W, inputs = _tiny(steps)

    def Y(s, d):
        return synth.plant_targets(w, s, inputs[s]["noise"], d)["target_logits"]

    out = loop.closed_loop(w.dtype, steps, inputs[0]["prev0"], W["fc_w"], W["lm_w"], W["w1"],
                           W["w2"], lambda s: inputs[s], Y)
    assert np.array_equal(out[0]["prev"], inputs[0]["prev0"])
    for s in range(1, steps):
        assert np.array_equal(out[s]["prev"], out[s - 1]["bonus"])
    for s, o in enumerate(out):
        # the committed tokens are the target's own greedy tokens (lossless)
        t = oracle.target_argmax(o["target_logits"], w.dtype, o["block_len"])
        for b in range(w.batch):
            n = int(o["n_emitted"][b])
            assert np.array_equal(o["emitted"][b, :n], t[b, :n])
        # step s equals one plain block-step from the same context
        ref = oracle.block_step(w.dtype, inputs[s]["taps"], W["fc_w"], inputs[s]["draft_hidden"],
                                W["lm_w"], W["w1"], W["w2"], o["prev"],
                                target_logits=o["target_logits"])
        assert np.array_equal(ref["draft_tokens"], o["draft_tokens"])
        assert np.array_equal(ref["accepted"], o["accepted"])
        assert np.array_equal(ref["bonus"], o["bonus"])
        assert np.array_equal(o["fc_out"], ref["fc_out"][o["row_index"]])
