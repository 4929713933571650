"""The five synthetic block-step workloads of the block-draft readout hot path.

Each workload fixes the shapes, dtypes and value distributions of one drafting +
verification block-step:

* ``tiny``          -- fp32, H=64, V=1000, r=8, k=4; 8 fake target layers of which
                       layers 1,3,5,6,7 are tapped (5x64 concatenated).
* ``qwen27b_b1``    -- Qwen3.8-27B-shaped single stream: H=5120, 5 taps, V=151936,
                       r=32, k=7, bf16.  The 5x5120 fc input and the tap layers
                       4/16/28/40/52 follow the Qwen3.8-27B-DSpark model card
                       ("Target quantisation", "Limitations").
* ``flashnext_b4``  -- Qwen3.8-Flash-Next-shaped, 4 concurrent streams: H=2560,
                       fc [2560, 12800], taps 5/15/25/35/45 (vllm-backport PR #128,
                       "What was missing", item 1), r=32, k=8, bf16.
* ``b16``           -- 16 concurrent sequences (the model card's max-num-seqs 16
                       serve recipe, "Usage"): H=5120, r=64, k=7, bf16, per-row
                       mixture of acceptance-friendly and natural-text rows.
* ``adaptive_b16``  -- as ``b16`` with k=8 plus per-position confidence scores and
                       truncation threshold 0.3 (the adaptive draft block of the
                       DSpark proposer, llm-scaler PR #620, DSpark port notes).

Vocabulary 151936 and the planted per-position match probabilities are workload
choices; the k=7 probabilities are the per-position acceptance curve printed on the
model card ("Measured results").

Nothing here computes any step of the method.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    cid: int                      # workload id; first component of every seed
    name: str
    batch: int                    # B, concurrent sequences
    hidden: int                   # H
    n_taps: int                   # T, tapped target layers fed to fc
    fake_layers: int              # >0: generate this many fake layers and tap some
    tap_layers: Tuple[int, ...]   # which fake layers are tapped, in fc concat order
    vocab: int                    # V
    rank: int                     # r, markov_rank
    k: int                        # draft block length (num_speculative_tokens)
    dtype: str                    # 'f32' or 'bf16' storage of weights / activations
    plant: str                    # 'fixed' or 'mixture'
    plant_p: Tuple[float, ...]    # per-position match probability ('fixed')
    plant_hi: Tuple[float, ...] = ()   # 'mixture': acceptance-friendly rows
    plant_lo: Tuple[float, ...] = ()   # 'mixture': natural-text rows
    threshold: Optional[float] = None  # confidence truncation threshold, None = off
    count_steps: int = 8          # steps over which acceptance counts are accumulated
    plant_boost: float = 8.0      # logit added to the planted token

    @property
    def rows(self) -> int:
        """Rows fed to the fc: the k+1 verified positions of each sequence."""
        return self.batch * (self.k + 1)

    @property
    def fc_in(self) -> int:
        return self.n_taps * self.hidden

    def describe(self) -> str:
        return (f"{self.name}: B={self.batch} H={self.hidden} T={self.n_taps} "
                f"V={self.vocab} r={self.rank} k={self.k} {self.dtype}")


def _geom(a: float, q: float, n: int) -> Tuple[float, ...]:
    return tuple(a * q ** i for i in range(n))


TINY = Workload(
    cid=0, name="tiny", batch=1, hidden=64, n_taps=5, fake_layers=8,
    tap_layers=(1, 3, 5, 6, 7), vocab=1000, rank=8, k=4, dtype="f32",
    plant="fixed", plant_p=(0.76, 0.45, 0.31, 0.14), count_steps=100)

QWEN27B_B1 = Workload(
    cid=1, name="qwen27b_b1", batch=1, hidden=5120, n_taps=5, fake_layers=0,
    tap_layers=(4, 16, 28, 40, 52), vocab=151936, rank=32, k=7, dtype="bf16",
    plant="fixed", plant_p=(0.76, 0.45, 0.31, 0.14, 0.10, 0.02, 0.00))

FLASHNEXT_B4 = Workload(
    cid=2, name="flashnext_b4", batch=4, hidden=2560, n_taps=5, fake_layers=0,
    tap_layers=(5, 15, 25, 35, 45), vocab=151936, rank=32, k=8, dtype="bf16",
    plant="fixed", plant_p=_geom(0.85, 0.8, 8))

B16 = Workload(
    cid=3, name="b16", batch=16, hidden=5120, n_taps=5, fake_layers=0,
    tap_layers=(4, 16, 28, 40, 52), vocab=151936, rank=64, k=7, dtype="bf16",
    plant="mixture", plant_p=(), plant_hi=_geom(0.9, 0.85, 7),
    plant_lo=_geom(0.6, 0.5, 7))

ADAPTIVE_B16 = Workload(
    cid=4, name="adaptive_b16", batch=16, hidden=5120, n_taps=5, fake_layers=0,
    tap_layers=(4, 16, 28, 40, 52), vocab=151936, rank=64, k=8, dtype="bf16",
    plant="mixture", plant_p=(), plant_hi=_geom(0.9, 0.85, 8),
    plant_lo=_geom(0.6, 0.5, 8), threshold=0.3, count_steps=1000)

WORKLOADS = (TINY, QWEN27B_B1, FLASHNEXT_B4, B16, ADAPTIVE_B16)
BY_NAME = {w.name: w for w in WORKLOADS}


def get(name_or_id) -> Workload:
    if isinstance(name_or_id, int):
        return WORKLOADS[name_or_id]
    return BY_NAME[name_or_id]
