"""Helpers of the GPU parity tests: device transfer, the error metric, the
near-tie exclusion cascade, and cached per-workload oracle results."""
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


def compare_drafts(got: np.ndarray, ref: np.ndarray, gap: np.ndarray):
    """Bit-exact comparison of draft tokens at positions before each row's first
    near-tie; returns (n_compared, n_excluded)."""
    istar = first_near_tie(gap)
    B, k = ref.shape
    n_cmp = 0
    for b in range(B):
        m = int(istar[b])
        assert np.array_equal(got[b, :m], ref[b, :m]), (b, got[b], ref[b], gap[b])
        n_cmp += m
    return n_cmp, B * k - n_cmp


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
