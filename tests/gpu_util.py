"""Helpers of the GPU parity tests: device transfer, the error metric, the
position-by-position checks of GPU drafts and sampling outcomes against the
oracle's rule (admissible picks at near-ties), and cached per-workload oracle
results."""
from __future__ import annotations

import functools
import sys
import time

import numpy as np

import oracle
import workloads
from workloads import synth

# max relative error bars for float intermediates: bf16 storage (stated bar) and
# fp32 storage (tiny workload)
REL_TOL = {"bf16": 2e-2, "f32": 1e-4}
NEAR_TIE = 1e-2


# Row-split GEMM: ring depths built by A row-tile count (bf16 and fp8 weights)
# and the accumulator tiles one pass holds
RINGS = {2: (8, 5, 3), 3: (7, 5, 3), 4: (6, 5, 3), 5: (6, 5, 3), 6: (6, 5, 3), 7: (5, 3),
         8: (5, 3), 9: (4, 3), 10: (3,)}
NTW_MAX = {2: 16, 3: 14, 4: 12, 5: 9, 6: 8, 7: 6, 8: 5, 9: 4, 10: 3}
RING_CASES = [(m, r) for m, rs in RINGS.items() for r in rs]


def ring_tiles(mt: int, ring: int) -> int:
    """Tiles of the largest wave for a ring test: more than a pass holds, so
    two passes, the second with groups of slots left empty."""
    return NTW_MAX[mt] // ring * ring + ring + 1


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def dev(x: np.ndarray, device="cuda"):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def host_bits(t) -> np.ndarray:
    """Device tensor -> numpy in storage convention (bf16 -> uint16 bits)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |g - r| / max(|r|, 0.01 * rms(r))."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    floor = 0.01 * np.sqrt(np.mean(ref * ref))
    den = np.maximum(np.abs(ref), max(floor, 1e-30))
    return float(np.max(np.abs(got - ref) / den))


def first_near_tie(gap: np.ndarray, thr: float = NEAR_TIE) -> np.ndarray:
    """i*_b: first position of row b whose oracle top-2 gap is below thr (k if none)."""
    B, k = gap.shape
    out = np.full(B, k, dtype=np.int64)
    for b in range(B):
        idx = np.flatnonzero(gap[b] < thr)
        if idx.size:
            out[b] = idx[0]
    return out


def check_draft(got: np.ndarray, Z, w1, w2, prev0, dtype: str) -> dict:
    """Every position of a GPU greedy draft against the oracle's rule.

    Each position's Markov context is the GPU's own previous token (prev0 at
    position 0), as the chain defines it, so a block that took the other side
    of a near-tie is still checked at every later position.  Where the oracle's
    top-2 gap under that context is >= NEAR_TIE the token must be the oracle's
    argmax bit for bit; below it the GPU's token must be an admissible pick,
    within NEAR_TIE of the maximum of the oracle's biased logits.
    """
    got = np.asarray(got).astype(np.int64)
    best, gap, deficit = oracle.score_draft(Z, w1, w2, prev0, got, dtype)
    clear = gap >= NEAR_TIE
    bad = np.argwhere(clear & (got != best))
    assert bad.size == 0, ("draft token differs at a clear position", bad[:4].tolist(),
                           [(int(got[b, i]), int(best[b, i]), float(gap[b, i])) for b, i in bad[:4]])
    near = ~clear
    assert np.all(deficit[near] <= NEAR_TIE), ("inadmissible pick at a near-tie",
                                                np.argwhere(near & (deficit > NEAR_TIE))[:4].tolist())
    return dict(n=int(got.size), exact=int(clear.sum()), near=int(near.sum()),
                other_side=int(np.sum(near & (got != best))),
                max_near_deficit=float(deficit[near].max()) if near.any() else 0.0)


def check_sampled_draft(got: np.ndarray, x_got, Z, w1, w2, prev0, dtype: str, T: float,
                        seed: int) -> dict:
    """Every position of a GPU sampled draft against the oracle's rule, each
    position's context being the GPU's own previous draw: the draw bit for bit
    where the oracle's top-2 Gumbel-key gap is >= NEAR_TIE, otherwise a key
    within NEAR_TIE of the maximum; the written draft distribution (biased
    logits under those contexts) within 1e-4 (1 + |x|)."""
    from oracle import sampling as S
    got = np.asarray(got).astype(np.int64)
    best, gap, deficit, x = S.score_sampled_draft(Z, w1, w2, prev0, got, dtype, T, seed)
    clear = gap >= NEAR_TIE
    bad = np.argwhere(clear & (got != best))
    assert bad.size == 0, ("sampled token differs at a clear position", bad[:4].tolist())
    near = ~clear
    assert np.all(deficit[near] <= NEAR_TIE), ("inadmissible draw at a near-tie",
                                                np.argwhere(near & (deficit > NEAR_TIE))[:4].tolist())
    if x_got is not None:
        diff = np.abs(np.asarray(x_got, dtype=np.float64) - x)
        assert np.all(diff <= 1e-4 * (1 + np.abs(x))), float(diff.max())
    return dict(n=int(got.size), exact=int(clear.sum()), near=int(near.sum()),
                other_side=int(np.sum(near & (got != best))))


MARGIN_TOL = 1e-3


def check_verify_sample(accepted, bonus, d, x, Y, dtype: str, L, T: float, seed: int) -> dict:
    """A GPU rejection-sampling outcome (accepted, bonus per row) against the
    oracle's rule along the path that outcome takes: every acceptance test
    below a_b must accept and the test at a_b < L_b must reject, unless the
    oracle's margin |r q - p| / max(p, q) there is below MARGIN_TOL (then
    either outcome is admissible); the bonus must be the oracle's draw at the
    end of that path, or within NEAR_TIE of its maximum key where the oracle's
    draw gap is below NEAR_TIE.  Returns counts of the decisions taken at a
    near-tie."""
    from oracle import sampling as S
    accepted = np.asarray(accepted).astype(np.int64)
    bonus = np.asarray(bonus).astype(np.int64)
    o = S.verify_sample_outcome(d, x, Y, dtype, L, T, seed, accepted, bonus)
    assert o["valid"].all(), np.flatnonzero(~o["valid"]).tolist()
    B = accepted.shape[0]
    near_tests = near_draws = 0
    for b in range(B):
        a, Lb = int(accepted[b]), int(L[b])
        for n in range(min(a + 1, Lb)):
            want = n < a
            if bool(o["decision"][b, n]) != want:
                assert o["margin"][b, n] < MARGIN_TOL, ("acceptance decision", b, n,
                                                        float(o["margin"][b, n]))
                near_tests += 1
        if int(o["draw"][b]) != int(bonus[b]):
            assert o["draw_gap"][b] < NEAR_TIE and o["bonus_deficit"][b] <= NEAR_TIE, (
                "bonus draw", b, int(bonus[b]), int(o["draw"][b]), float(o["draw_gap"][b]))
            near_draws += 1
    return dict(rows=B, near_tests=near_tests, near_draws=near_draws)


@functools.lru_cache(maxsize=2)
def weights(name: str):
    w = workloads.get(name)
    t0 = time.time()
    W = synth.make_weights(w)
    log(f"{name}: weights generated in {time.time() - t0:.1f}s")
    return W


@functools.lru_cache(maxsize=2)
def oracle_step(name: str, step: int = 0):
    """Oracle S1..S4 for one step of a workload (target logits planted on the
    oracle's own draft)."""
    w = workloads.get(name)
    W = weights(name)
    s = synth.make_step(w, step)
    t0 = time.time()
    F = oracle.fuse_fc(s["taps"], W["fc_w"], w.dtype)
    Z = oracle.lm_head(s["draft_hidden"], W["lm_w"], w.dtype)
    d, gap = oracle.semi_ar_argmax(Z, W["w1"], W["w2"], s["prev0"], w.dtype)
    plant = synth.plant_targets(w, step, s["noise"], d)
    Y = plant["target_logits"]
    conf = synth.make_confidence(w, step)
    L = oracle.truncate_by_confidence(conf, w.threshold, w.batch, w.k)
    t = oracle.target_argmax(Y, w.dtype, L)
    a, bonus, acc, prop = oracle.verify_greedy(d, t, L)
    log(f"{name}: oracle step {step} in {time.time() - t0:.1f}s")
    return dict(step=s, F=F, Z=Z, d=d, gap=gap, Y=Y, conf=conf, L=L, t=t, a=a, bonus=bonus,
                acc=acc, prop=prop)
