"""Seeded synthetic inputs for the DPO head path.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no softmax, no sums, no loss).  Both the HIP path and the
CPU oracle are fed from here, so the bits each side sees are identical.

Workload shapes follow the problem statement of "DPO Training on GPU, in
depth" (section "What one DPO step computes": a prompt shared by a chosen and a
rejected completion, scores summed over completion tokens only, chosen and
rejected rows concatenated into one batch of 2B rows) and its memory section
("Where the memory goes for an 8B model": 2,048-token sequences, a 128,256-token
vocabulary, micro-batches of four pairs).  The offline-scored reference case
follows "feat(training): add DPO training with offline-scored reference model"
(section "Why the reference is scored offline": sums per row, no beta applied).

Recipe (fixed draw order from one numpy PCG64 stream seeded with the workload
number): prompt lengths -> completion lengths -> targets -> hidden (or logits)
-> W_vocab -> reference-sum noise.  Normal draws are float32
(``Generator.standard_normal(dtype=float32)``), scaled by the standard deviation
in float32, optionally RMS-normalised per position in float32 (no epsilon, no
gain), then rounded to bfloat16 with round-to-nearest-even.  Targets at
positions whose mask is 0 are set to -100 (the ignore index of the torchtune
recipe in "Run Distributed Full-Model DPO with PyTorch FSDP", section "Step 4:
Computing Concatenated Forward Passes"), so no consumer may use them as
indices.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

IGNORE_INDEX = -100
PAIRS_ADJACENT = 0  # rows 2i (chosen), 2i+1 (rejected)
PAIRS_HALVES = 1    # rows i (chosen), B+i (rejected)

_CHUNK = 1 << 24


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even.

    Inputs are finite by construction here, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """The same chunked N(0, std) float32 draws as ``_normal_bf16``, kept in float32."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    pos = 0
    while pos < n:
        m = min(_CHUNK, n - pos)
        x = rng.standard_normal(m, dtype=np.float32)
        x *= np.float32(std)
        out[pos:pos + m] = x
        pos += m
    return out.reshape(shape)


def _normal_bf16(rng: np.random.Generator, shape, std: float,
                 rms_rows: Optional[int] = None) -> np.ndarray:
    """Draw N(0, std) float32 values in fixed-size chunks and round to bf16.

    With ``rms_rows`` = row length, each row of that length is divided by its
    root-mean-square before rounding.  Chunk boundaries fall on row boundaries.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = _CHUNK
    if rms_rows:
        step = max(rms_rows, (_CHUNK // rms_rows) * rms_rows)
    pos = 0
    while pos < n:
        m = min(step, n - pos)
        x = rng.standard_normal(m, dtype=np.float32)
        x *= np.float32(std)
        if rms_rows:
            xr = x.reshape(-1, rms_rows)
            rms = np.sqrt(np.mean(xr * xr, axis=1, dtype=np.float32))
            xr /= rms[:, None]
        out[pos:pos + m] = bf16_rne_bits(x)
        pos += m
    return out.reshape(shape)


def zipf_ids(rng: np.random.Generator, n: int, V: int, s: float = 1.1) -> np.ndarray:
    """Token ids with P(id = k-1) proportional to k^-s for ranks k = 1..V (inverse CDF)."""
    k = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-s))
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int32)


@dataclasses.dataclass
class HeadInputs:
    """One batch of the head path.  Arrays are host numpy arrays.

    hidden  uint16 [R, T, H]  bf16 bits of the final hidden states (None for logits workloads)
    w_vocab uint16 [V, H]     bf16 bits of the LM-head weight (None for logits workloads)
    logits  uint16 [R, T, V]  bf16 bits of given logits (logits workloads only)
    targets int32  [R, T]     aligned: targets[r, t] is the token predicted at (r, t)
    mask    uint8  [R, T]     1 = completion position counted in the row score
    ref_noise float64 [R]     N(0,1) noise added to the policy sums to form reference sums
    """
    name: str
    rows: int
    T: int
    H: int
    V: int
    beta: float
    layout: int
    targets: np.ndarray
    mask: np.ndarray
    ref_noise: np.ndarray
    hidden: Optional[np.ndarray] = None
    w_vocab: Optional[np.ndarray] = None
    logits: Optional[np.ndarray] = None

    @property
    def num_pairs(self) -> int:
        return self.rows // 2

    @property
    def n_completion(self) -> int:
        return int((self.mask != 0).sum())


def _mask_from_spans(R: int, T: int, starts, ends) -> np.ndarray:
    mask = np.zeros((R, T), dtype=np.uint8)
    for r in range(R):
        mask[r, starts[r]:ends[r]] = 1
    return mask


def _rows_of_pairs(num_pairs: int, layout: int):
    """(chosen_row, rejected_row) index arrays for a pair layout."""
    i = np.arange(num_pairs)
    if layout == PAIRS_ADJACENT:
        return 2 * i, 2 * i + 1
    return i, num_pairs + i


def make_head_inputs(*, name: str, seed: int, rows: int, T: int, H: int, V: int,
                     prompt_lo: int, prompt_hi: int, comp_mode: str = "fill",
                     comp_ratio: float = 2.0, hidden_std: float = 1.0,
                     rms_normalise: bool = False, w_std: float = 0.02,
                     targets_dist: str = "uniform", beta: float = 0.1,
                     layout: int = PAIRS_ADJACENT) -> HeadInputs:
    """General head-path generator.

    comp_mode "fill": completion covers [P, T).  comp_mode "independent": each
    row of a pair draws its completion length in 1..T-P independently, redrawn
    until the longer is at most ``comp_ratio`` times the shorter; the rest of
    the row is tail padding (mask 0).
    """
    assert rows % 2 == 0 and rows > 0
    rng = np.random.default_rng(seed)
    B = rows // 2
    chosen, rejected = _rows_of_pairs(B, layout)
    prompt = rng.integers(prompt_lo, prompt_hi + 1, size=B)
    starts = np.zeros(rows, dtype=np.int64)
    ends = np.zeros(rows, dtype=np.int64)
    for i in range(B):
        P = int(prompt[i])
        starts[chosen[i]] = starts[rejected[i]] = P
        if comp_mode == "fill":
            ends[chosen[i]] = ends[rejected[i]] = T
        else:
            while True:
                lc, lr = rng.integers(1, T - P + 1, size=2)
                if max(lc, lr) <= comp_ratio * min(lc, lr):
                    break
            ends[chosen[i]] = P + lc
            ends[rejected[i]] = P + lr
    mask = _mask_from_spans(rows, T, starts, ends)
    if targets_dist == "zipf":
        targets = zipf_ids(rng, rows * T, V).reshape(rows, T)
    else:
        targets = rng.integers(0, V, size=(rows, T), dtype=np.int32)
    targets = np.where(mask != 0, targets, IGNORE_INDEX).astype(np.int32)
    hidden = _normal_bf16(rng, (rows, T, H), hidden_std, rms_rows=H if rms_normalise else None)
    w = _normal_bf16(rng, (V, H), w_std)
    ref_noise = rng.standard_normal(rows)
    return HeadInputs(name=name, rows=rows, T=T, H=H, V=V, beta=beta, layout=layout,
                      targets=targets, mask=mask, ref_noise=ref_noise,
                      hidden=hidden, w_vocab=w)


def make_logits_inputs(*, name: str, seed: int, rows: int, T: int, V: int,
                       comp_start: int, logit_std: float = 3.0, beta: float = 0.1,
                       layout: int = PAIRS_ADJACENT, logits_dtype: str = "bf16") -> HeadInputs:
    """Materialised-logits workload: mask = 1 on [comp_start, T) of every row.

    ``logits_dtype`` "bf16" gives uint16 bf16 bit patterns; "f32" gives the
    same float32 draws unrounded (a float32 array)."""
    assert rows % 2 == 0 and rows > 0
    rng = np.random.default_rng(seed)
    mask = _mask_from_spans(rows, T, [comp_start] * rows, [T] * rows)
    targets = rng.integers(0, V, size=(rows, T), dtype=np.int32)
    targets = np.where(mask != 0, targets, IGNORE_INDEX).astype(np.int32)
    if logits_dtype == "f32":
        logits = _normal_f32(rng, (rows, T, V), logit_std)
    elif logits_dtype == "bf16":
        logits = _normal_bf16(rng, (rows, T, V), logit_std)
    else:
        raise ValueError("logits_dtype is bf16 or f32")
    ref_noise = rng.standard_normal(rows)
    return HeadInputs(name=name, rows=rows, T=T, H=0, V=V, beta=beta, layout=layout,
                      targets=targets, mask=mask, ref_noise=ref_noise, logits=logits)


# The five fixed workloads.  Each entry is (description, generator kwargs).
WORKLOADS = {
    1: ("tiny: 2 pairs adjacent, T=64 (prompt 16), H=256, V=1024",
        dict(kind="head", rows=4, T=64, H=256, V=1024, prompt_lo=16, prompt_hi=16,
             hidden_std=1.0, w_std=0.02, targets_dist="uniform")),
    2: ("8B head: 4 pairs, T=2048, prompt U[128,512], H=4096, V=128256, RMS-normalised hidden, Zipf(1.1) targets",
        dict(kind="head", rows=8, T=2048, H=4096, V=128256, prompt_lo=128, prompt_hi=512,
             hidden_std=1.0, rms_normalise=True, w_std=0.01, targets_dist="zipf")),
    3: ("offline reference scoring: 64 pairs, T=1024, prompt U[64,256], H=4096, V=128256",
        dict(kind="head", rows=128, T=1024, H=4096, V=128256, prompt_lo=64, prompt_hi=256,
             hidden_std=1.0, rms_normalise=True, w_std=0.01, targets_dist="zipf")),
    4: ("30B-A3B-like head: 2 pairs, T=4096, prompt U[256,1024], independent completion lengths (ratio<=2), H=2048, V=151936",
        dict(kind="head", rows=4, T=4096, H=2048, V=151936, prompt_lo=256, prompt_hi=1024,
             comp_mode="independent", hidden_std=1.0, w_std=0.02, targets_dist="zipf")),
    5: ("materialised logits: 8 rows x T=2048 x V=128256 bf16 ~N(0,3), mask on the last 75%",
        dict(kind="logits", rows=8, T=2048, V=128256, comp_start=512, logit_std=3.0)),
}


def make_workload(k: int, seed: Optional[int] = None) -> HeadInputs:
    """Workload ``k`` (1..5) with seed ``k`` unless given."""
    desc, kw = WORKLOADS[k]
    kw = dict(kw)
    kind = kw.pop("kind")
    seed = k if seed is None else seed
    if kind == "logits":
        return make_logits_inputs(name=f"workload{k}", seed=seed, **kw)
    return make_head_inputs(name=f"workload{k}", seed=seed, **kw)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for building device copies only)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def expected_n_completion(k: int) -> Optional[int]:
    """Completion-position count fixed by the recipe (None where it is random)."""
    return {1: 4 * 48, 5: 8 * 1536}.get(k)


__all__ = [
    "IGNORE_INDEX", "PAIRS_ADJACENT", "PAIRS_HALVES", "HeadInputs", "WORKLOADS",
    "bf16_rne_bits", "zipf_ids", "make_head_inputs", "make_logits_inputs",
    "make_workload", "bf16_bits_to_f32", "expected_n_completion",
]
