"""GPU parity of the whole block-step on the five workloads at their full sizes,
in the same launch configuration the benchmark times (the three ABI calls with
their default plans).

Per workload: fc output and logits within the max-relative-error bar; draft
tokens bit-exact before each row's first oracle near-tie (top-2 gap < 1e-2);
verification bit-exact on identical inputs; end-to-end accept lengths, bonus
tokens and counts bit-exact on every row whose acceptance-deciding positions
were tie-free.
"""
import math

import numpy as np
import pytest

import workloads
from gpu_util import (REL_TOL, compare_drafts, dev, first_near_tie, host_bits, log,
                      max_rel_err, oracle_step, weights)
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAMES = ["tiny", "qwen27b_b1", "flashnext_b4", "b16", "adaptive_b16"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", NAMES)
def test_block_step_parity(name):
    import block_draft_readout_amd as bdr
    w = workloads.get(name)
    log(f"== {w.describe()}")
    ref = oracle_step(name)
    W = weights(name)
    s = ref["step"]
    gW = {k: dev(v) for k, v in W.items()}

    # S1
    F = bdr.dflash_fuse_fc([dev(t) for t in s["taps"]], gW["fc_w"])
    errF = max_rel_err(oracle.widen(host_bits(F), w.dtype), ref["F"])
    # S2 + S3
    logits = torch.empty((w.batch, w.k, w.vocab), dtype=torch.float32, device="cuda")
    d = bdr.dspark_draft_block(dev(s["draft_hidden"]), gW["lm_w"], gW["w1"], gW["w2"],
                               dev(s["prev0"]), logits_out=logits)
    errZ = max_rel_err(logits.cpu().numpy(), ref["Z"])
    n_cmp, n_ex = compare_drafts(d.cpu().numpy(), ref["d"], ref["gap"])
    log(f"   fc rel err {errF:.2e}  logits rel err {errZ:.2e}  draft compared {n_cmp} "
        f"excluded {n_ex}")
    assert errF <= REL_TOL[w.dtype]
    assert errZ <= REL_TOL[w.dtype]
    # S3 on the oracle's logits
    d3 = bdr.dspark_markov_argmax(dev(ref["Z"]), gW["w1"], gW["w2"], dev(s["prev0"]))
    compare_drafts(d3.cpu().numpy(), ref["d"], ref["gap"])

    # S4 on identical inputs (oracle draft)
    th = math.nan if w.threshold is None else w.threshold
    conf = None if ref["conf"] is None else dev(ref["conf"])
    Yd = dev(ref["Y"])
    acc = torch.zeros(w.k, dtype=torch.int64, device="cuda")
    prop = torch.zeros(w.k, dtype=torch.int64, device="cuda")
    r = bdr.spec_verify_greedy(Yd, dev(ref["d"].astype(np.int32)), conf, th, acc, prop)
    assert np.array_equal(r["block_len"].cpu().numpy(), ref["L"])
    assert np.array_equal(r["target_argmax"].cpu().numpy(), ref["t"])
    assert np.array_equal(r["accepted"].cpu().numpy(), ref["a"])
    assert np.array_equal(r["bonus"].cpu().numpy(), ref["bonus"])
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    assert np.array_equal(prop.cpu().numpy(), ref["prop"])

    # end to end: verification of the GPU's own draft
    r2 = bdr.spec_verify_greedy(Yd, d, conf, th)
    istar = first_near_tie(ref["gap"])
    a_ref, L_ref = ref["a"], ref["L"]
    include = istar > np.minimum(a_ref, L_ref - 1)
    a_g = r2["accepted"].cpu().numpy()
    b_g = r2["bonus"].cpu().numpy()
    assert np.array_equal(a_g[include], a_ref[include])
    assert np.array_equal(b_g[include], ref["bonus"][include])
    log(f"   end-to-end rows compared {int(include.sum())}/{w.batch}; accepted "
        f"{a_ref.tolist()} bonus {ref['bonus'].tolist()}")
