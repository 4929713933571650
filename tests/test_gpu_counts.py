"""Adaptive-block workload: per-position acceptance counts accumulated on the GPU
over 1000 seeded verification steps, bit-exact against the oracle, and within
4 sigma of the planted closed form E[acc_i]/N = E[prod_{j<=i} p_j] * 0.7^(i+1).

Each step's draft tokens, confidence scores and planted target logits come from
the seeded generator (target-logit noise drawn from a pool of 8 steps, planted
afresh every step), so both sides verify identical inputs.
"""
import time

import numpy as np
import pytest

import oracle
import workloads
from workloads import synth
from gpu_util import dev, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.timeout(600)
def test_adaptive_counts_over_1000_steps():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_readout_amd as bdr
    w = workloads.get("adaptive_b16")
    steps = w.count_steps
    pool = [synth.make_step(w, s)["noise"] for s in range(8)]
    pool_st = [synth.store(n, w.dtype) for n in pool]
    acc_g = torch.zeros(w.k, dtype=torch.int64, device="cuda")
    prop_g = torch.zeros(w.k, dtype=torch.int64, device="cuda")
    acc_o = np.zeros(w.k, np.int64)
    prop_o = np.zeros(w.k, np.int64)
    ws = torch.zeros(bdr.workspace_bytes("verify", batch=w.batch, k=w.k, vocab=w.vocab) + 256,
                     dtype=torch.uint8, device="cuda")
    t0 = time.time()
    for step in range(steps):
        d = synth.random_drafts(w, step)
        Y = synth.plant_targets(w, step, pool[step % 8], d, noise_stored=pool_st[step % 8])
        conf = synth.make_confidence(w, step)
        r = bdr.spec_verify_greedy(dev(Y["target_logits"]), dev(d), dev(conf), w.threshold,
                                   acc_g, prop_g, target_argmax=False, workspace=ws)
        L = oracle.truncate_by_confidence(conf, w.threshold, w.batch, w.k)
        t = oracle.target_argmax(Y["target_logits"], w.dtype, L)
        a, bonus, acc, prop = oracle.verify_greedy(d, t, L)
        acc_o += acc
        prop_o += prop
        if step % 50 == 0:
            assert np.array_equal(r["accepted"].cpu().numpy(), a)
            assert np.array_equal(r["bonus"].cpu().numpy(), bonus)
        if step % 100 == 99:
            log(f"  step {step + 1}/{steps}  {time.time() - t0:.0f}s")
    acc_gn = acc_g.cpu().numpy()
    prop_gn = prop_g.cpu().numpy()
    log(f"accept counts {acc_gn.tolist()}  proposed {prop_gn.tolist()}")
    assert np.array_equal(acc_gn, acc_o)
    assert np.array_equal(prop_gn, prop_o)
    N = steps * w.batch
    keep = 0.7 ** np.arange(1, w.k + 1)
    q = 0.5 * (np.cumprod(w.plant_hi) + np.cumprod(w.plant_lo)) * keep
    sd = np.sqrt(N * q * (1 - q))
    assert np.all(np.abs(acc_gn - N * q) <= 4 * sd + 1), (acc_gn, N * q)
    mal = oracle.mean_acceptance_length(acc_gn, steps, w.batch)
    log(f"mean acceptance length {mal:.3f}, drafted-token rate "
        f"{oracle.drafted_token_rate(acc_gn, prop_gn):.3f}")
