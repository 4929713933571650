"""Seeded synthetic inputs for the block-draft readout workloads.

This module only draws random numbers and stores them; it holds none of the
method's arithmetic.  Both the CPU oracle (tests, CPU baseline) and the HIP path
(tests, benchmark, smoke run) consume its outputs, and nothing else is shared
between the two.

Storage convention: a ``bf16`` tensor is a ``numpy.uint16`` array of bfloat16 bit
patterns (rounded to nearest-even from float32 by torch's CPU conversion); an
``f32`` tensor is a ``numpy.float32`` array.

Seeding: every tensor is filled in fixed chunks of ``CHUNK`` elements, chunk ``c``
of tensor ``t`` drawn from ``PCG64(SeedSequence([workload, stream, step, t, c]))``.
Stream 0 holds the weights, 1 the per-step activations and target-logit noise,
2 the planting decisions, 3 the confidence scores and 4 free-standing draft
tokens.  The result does not depend on the number of threads used.

Value distributions: N(mean, var) with the second argument a variance, so the
weights are N(0, 1/fan_in) (fan_in = T*H for fc, H for the LM head),
markov_w1 ~ N(0, 1), markov_w2 ~ N(0, 0.1), hidden states N(0, 1), target logits
N(0, 1) with +8 planted in float32 before rounding to bf16.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

from .configs import Workload

CHUNK = 1 << 22

# tensor ids inside stream 0 (weights) and stream 1 (per step)
_W_FC, _W_LM, _W_W1, _W_W2 = 0, 1, 2, 3
_S_TAPS, _S_HIDDEN, _S_PREV, _S_NOISE = 0, 1, 2, 3


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def normal_f32(shape, key, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) array, chunk-seeded from ``key`` (a tuple of ints)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK
    s = np.float32(std)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        view = out[lo:hi]
        _rng(*key, c).standard_normal(out=view, dtype=np.float32)
        if std != 1.0:
            np.multiply(view, s, out=view)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (torch CPU)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast a float32 array to the workload's storage dtype."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def make_weights(w: Workload) -> Dict[str, np.ndarray]:
    """fc_w [H, T*H], lm_w [V, H], w1 [V, r], w2 [V, r] in storage dtype."""
    H, V, r, K = w.hidden, w.vocab, w.rank, w.fc_in
    out = {}
    out["fc_w"] = store(normal_f32((H, K), (w.cid, 0, 0, _W_FC), math.sqrt(1.0 / K)), w.dtype)
    out["lm_w"] = store(normal_f32((V, H), (w.cid, 0, 0, _W_LM), math.sqrt(1.0 / H)), w.dtype)
    out["w1"] = store(normal_f32((V, r), (w.cid, 0, 0, _W_W1), 1.0), w.dtype)
    out["w2"] = store(normal_f32((V, r), (w.cid, 0, 0, _W_W2), math.sqrt(0.1)), w.dtype)
    return out


def quantize_e4m3_rows(x: np.ndarray, rows_at_once: int = 8192):
    """float32 [N, K] -> (E4M3 codes uint8 [N, K], float32 scales [N]).

    The synthetic fp8 checkpoint recipe: scale[n] = max_k |x[n, k]| / 448 (1 for
    an all-zero row) and code = x / scale rounded to nearest even by torch's CPU
    float8_e4m3fn conversion, so every row uses the full E4M3 range.  This makes
    inputs for the fp8 weight path; that path only reads codes and scales.
    """
    import torch
    x = np.asarray(x, dtype=np.float32)
    N, K = x.shape
    codes = np.empty((N, K), dtype=np.uint8)
    amax = np.abs(x).max(axis=1) if K else np.zeros(N, dtype=np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    for r0 in range(0, N, rows_at_once):
        r1 = min(N, r0 + rows_at_once)
        t = torch.from_numpy(x[r0:r1]) / torch.from_numpy(scale[r0:r1])[:, None]
        codes[r0:r1] = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def make_weights_fp8(w: Workload) -> Dict[str, np.ndarray]:
    """The weights of make_weights with fc_w and lm_w as E4M3 codes + row scales.

    fc_q [H, T*H] / fc_scale [H] and lm_q [V, H] / lm_scale [V] quantise the
    same float32 draws that make_weights stores; markov_w1 / markov_w2 keep the
    workload's storage dtype.
    """
    H, V, r, K = w.hidden, w.vocab, w.rank, w.fc_in
    out = {}
    out["fc_q"], out["fc_scale"] = quantize_e4m3_rows(
        normal_f32((H, K), (w.cid, 0, 0, _W_FC), math.sqrt(1.0 / K)))
    out["lm_q"], out["lm_scale"] = quantize_e4m3_rows(
        normal_f32((V, H), (w.cid, 0, 0, _W_LM), math.sqrt(1.0 / H)))
    out["w1"] = store(normal_f32((V, r), (w.cid, 0, 0, _W_W1), 1.0), w.dtype)
    out["w2"] = store(normal_f32((V, r), (w.cid, 0, 0, _W_W2), math.sqrt(0.1)), w.dtype)
    return out


def make_step(w: Workload, step: int, noise: bool = True,
              noise_step: Optional[int] = None) -> Dict[str, object]:
    """Per-step activations.

    taps:          list of T arrays [B*(k+1), H] (storage dtype), fc concat order
    draft_hidden:  [B, k, H] (storage dtype) -- stands in for the drafter backbone
    prev0:         [B] int32, the accepted bonus token of the previous step
    noise:         [B, k+1, V] float32 target-logit noise (before planting);
                   drawn from ``noise_step`` (default ``step``)
    """
    B, H, k, V = w.batch, w.hidden, w.k, w.vocab
    rows = w.rows
    if w.fake_layers > 0:
        layers = normal_f32((w.fake_layers, rows, H), (w.cid, 1, step, _S_TAPS))
        taps = [store(layers[l], w.dtype) for l in w.tap_layers]
    else:
        stacked = normal_f32((w.n_taps, rows, H), (w.cid, 1, step, _S_TAPS))
        taps = [store(stacked[t], w.dtype) for t in range(w.n_taps)]
    hidden = store(normal_f32((B, k, H), (w.cid, 1, step, _S_HIDDEN)), w.dtype)
    prev0 = _rng(w.cid, 1, step, _S_PREV, 0).integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    out = {"taps": taps, "draft_hidden": hidden, "prev0": prev0}
    if noise:
        ns = step if noise_step is None else noise_step
        out["noise"] = normal_f32((B, k + 1, V), (w.cid, 1, ns, _S_NOISE))
    return out


def plant_probabilities(w: Workload, step: int) -> np.ndarray:
    """[B, k] per-position match probability used when planting this step."""
    B, k = w.batch, w.k
    for name in (("plant_p",) if w.plant == "fixed" else ("plant_hi", "plant_lo")):
        if len(getattr(w, name)) < k:
            raise ValueError(f"{w.name}: {name} needs {k} probabilities")
    if w.plant == "fixed":
        return np.tile(np.asarray(w.plant_p, dtype=np.float64)[None, :k], (B, 1))
    if w.plant == "mixture":
        cls = _rng(w.cid, 2, step, 0, 0).random(B) < 0.5  # True = acceptance-friendly
        hi = np.asarray(w.plant_hi[:k], dtype=np.float64)
        lo = np.asarray(w.plant_lo[:k], dtype=np.float64)
        return np.where(cls[:, None], hi[None, :], lo[None, :])
    raise ValueError(w.plant)


def plant_targets(w: Workload, step: int, noise: np.ndarray,
                  draft_tokens: np.ndarray,
                  noise_stored: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Target logits [B, k+1, V] in storage dtype.

    For position j < k, +boost goes on the draft token with the position's match
    probability, else on a token drawn uniformly from the other V-1; position k
    (no draft) gets +boost on a uniformly drawn token.  ``draft_tokens`` [B, k] is
    supplied by the caller.

    ``noise_stored`` (optional) is ``store(noise, w.dtype)`` computed once by the
    caller; only the planted entries are then recomputed.  Rounding to the
    storage dtype is elementwise, so the result is identical.
    """
    B, k, V = w.batch, w.k, w.vocab
    d = np.asarray(draft_tokens, dtype=np.int64).reshape(B, k)
    p = plant_probabilities(w, step)
    g = _rng(w.cid, 2, step, 1, 0)
    u = g.random((B, k))
    other = g.integers(0, V - 1, size=(B, k), dtype=np.int64)
    last = g.integers(0, V, size=B, dtype=np.int64)
    hit = u < p
    tok = np.where(hit, d, other + (other >= d))
    all_tok = np.concatenate([tok, last[:, None]], axis=1)          # [B, k+1]
    boost = np.float32(w.plant_boost)
    noise = np.asarray(noise, dtype=np.float32).reshape(B, k + 1, V)
    bi = np.repeat(np.arange(B), k + 1)
    ji = np.tile(np.arange(k + 1), B)
    vi = all_tok.reshape(-1)
    if noise_stored is None:
        y = noise.copy()
        y[bi, ji, vi] += boost
        out = store(y, w.dtype)
    else:
        out = np.array(noise_stored, copy=True).reshape(B, k + 1, V)
        out[bi, ji, vi] = store(noise[bi, ji, vi] + boost, w.dtype)
    return {"target_logits": out, "planted_hit": hit, "planted_token": all_tok}


def make_confidence(w: Workload, step: int) -> Optional[np.ndarray]:
    """[B, k] float32 U(0,1) confidence scores (only for workloads with a threshold)."""
    if w.threshold is None:
        return None
    return _rng(w.cid, 3, step, 0, 0).random((w.batch, w.k), dtype=np.float32)


def random_drafts(w: Workload, step: int) -> np.ndarray:
    """[B, k] int32 free-standing draft tokens (for verification-only workloads)."""
    return _rng(w.cid, 4, step, 0, 0).integers(0, w.vocab, size=(w.batch, w.k),
                                               dtype=np.int64).astype(np.int32)
