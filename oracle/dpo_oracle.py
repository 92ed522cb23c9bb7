"""CPU fp64 oracle for the DPO sequence log-probability, loss and LM-head gradient.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP path and imports nothing from it; the only thing both sides share is
the seeded input generator, which holds none of the arithmetic below.

What is computed, and where the pages define it
-----------------------------------------------
"DPO Training on GPU, in depth" (aicassindra.com):
  * section "What one DPO step computes": the loss is minus the log-sigmoid
    of beta times the difference between the chosen and rejected
    policy-minus-reference log-ratios; sequence scores are sums of token
    log-probabilities over completion tokens only; chosen and rejected rows
    are concatenated into one batch of 2B rows.
  * section "A worked example of the numbers": implicit reward = beta times
    the log-ratio, margin = chosen reward minus rejected reward, the
    per-pair gradient is scaled by sigmoid(-margin), and a policy equal to the
    reference gives loss ln 2.
  * section "A training configuration that fits" (the hand-written chunked
    loss): fp32-or-better log-softmax over the whole vocabulary, gather of
    the target token, masked sum per row, mean of the per-pair loss over
    pairs, accuracy = fraction of pairs with margin strictly above zero.
"Run Distributed Full-Model DPO with PyTorch FSDP" (aimastery.page), section
"Step 4: Computing Concatenated Forward Passes": chosen rows first, then
rejected rows, split at half the batch, summed (not averaged) log-probs.
"feat(training): add DPO training with offline-scored reference model",
changelog and section "Why the reference is scored offline": chosen and
rejected rows of a pair sit next to each other; reference scores are plain
per-row sums with no beta.

Readings taken where the pages leave a step open:
targets arrive already shifted (targets[r, t] is the token predicted from
hidden[r, t]); an explicit 0/1 mask selects completion positions and targets
at mask-0 positions are never read; accuracy uses a strict ``>``; the
gradient weight of a row is w = -d loss / d score = +-beta*sigmoid(-m)/B.

Everything is float64.  bf16 inputs are widened exactly (bits << 16).  The
LM-head contraction uses numpy's BLAS matmul in float64 as a library step.
Every function here is pinned by tests in tests/test_oracle_pins.py against
the worked example, closed forms, brute force, finite differences and a
PyTorch-fp64 autograd cross-check.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

PAIRS_ADJACENT = 0
PAIRS_HALVES = 1


# ----------------------------------------------------------------------------
# input decoding
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: the 16 bits are the top half of a float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); returns float64 values.

    Used only to state the expected value of a bf16 output.  Implemented by
    scaling to the bf16 grid of each value's binade: a bf16 number has 8
    significant bits, so the spacing in [2^e, 2^(e+1)) is 2^(e-7).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    e = np.floor(np.log2(np.abs(x[nz])))
    # guard log2 rounding at exact powers of two
    e = np.where(np.abs(x[nz]) < 2.0 ** e, e - 1, e)
    e = np.where(np.abs(x[nz]) >= 2.0 ** (e + 1), e + 1, e)
    ulp = 2.0 ** (e - 7)
    out[nz] = np.round(x[nz] / ulp) * ulp  # numpy rounds half to even
    return out


# ----------------------------------------------------------------------------
# completion positions ("sums run only over completion tokens")
# ----------------------------------------------------------------------------
def completion_positions(mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Flat indices r*T+t of completion positions in row-major order, and per-row counts."""
    m = np.asarray(mask) != 0
    idx = np.flatnonzero(m.reshape(-1)).astype(np.int64)
    n_tokens = m.sum(axis=1).astype(np.int64)
    return idx, n_tokens


def _check_targets(targets_at_idx: np.ndarray, V: int) -> None:
    if targets_at_idx.size and (targets_at_idx.min() < 0 or targets_at_idx.max() >= V):
        raise ValueError("target id out of range at a completion position")


# ----------------------------------------------------------------------------
# per-position log-softmax over the whole vocabulary and target gather
# ----------------------------------------------------------------------------
def logsumexp_rows(Z: np.ndarray) -> np.ndarray:
    """log(sum_v exp(Z[i, v])) per row, shifted by the row max for range safety."""
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def position_logps(Z: np.ndarray, tgt: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(lse, log p(target)) for each row of a logits block Z [n, V]."""
    lse = logsumexp_rows(Z)
    return lse, Z[np.arange(Z.shape[0]), tgt] - lse


def _row_sums(logp_flat: np.ndarray, idx: np.ndarray, R: int, T: int) -> np.ndarray:
    """Exactly rounded per-row sum of the per-position log-probs (math.fsum)."""
    sums = np.zeros(R, dtype=np.float64)
    rows = idx // T
    for r in range(R):
        sums[r] = math.fsum(logp_flat[idx[rows == r]].tolist())
    return sums


def seq_logps_f64(hidden: np.ndarray, w: np.ndarray, targets: np.ndarray, mask: np.ndarray,
                  chunk: int = 256) -> Dict[str, np.ndarray]:
    """Sequence scores from hidden states [R,T,H] (float64) and W_vocab [V,H] (float64).

    Returns logp_sum [R] (exact sums), lse [R,T] and logp [R,T] (0 at mask-0
    positions), n_tokens [R], idx [N_c].
    """
    R, T, H = hidden.shape
    V = w.shape[0]
    idx, n_tokens = completion_positions(mask)
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    _check_targets(tflat[idx], V)
    hflat = hidden.reshape(R * T, H)
    lse = np.zeros(R * T)
    logp = np.zeros(R * T)
    for s in range(0, idx.size, chunk):
        c = idx[s:s + chunk]
        Z = hflat[c] @ w.T
        lse[c], logp[c] = position_logps(Z, tflat[c])
    return dict(logp_sum=_row_sums(logp, idx, R, T), lse=lse.reshape(R, T),
                logp=logp.reshape(R, T), n_tokens=n_tokens, idx=idx)


def seq_logps(hidden_bits, w_bits, targets, mask, chunk: int = 256) -> Dict[str, np.ndarray]:
    """As ``seq_logps_f64`` on bf16 bit-pattern inputs."""
    return seq_logps_f64(bf16_to_f64(hidden_bits), bf16_to_f64(w_bits), targets, mask, chunk)


def logits_seq_logps_f64(logits: np.ndarray, targets: np.ndarray, mask: np.ndarray,
                         chunk: int = 256) -> Dict[str, np.ndarray]:
    """Sequence scores from given logits [R,T,V] (float64)."""
    R, T, V = logits.shape
    idx, n_tokens = completion_positions(mask)
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    _check_targets(tflat[idx], V)
    lflat = logits.reshape(R * T, V)
    lse = np.zeros(R * T)
    logp = np.zeros(R * T)
    for s in range(0, idx.size, chunk):
        c = idx[s:s + chunk]
        lse[c], logp[c] = position_logps(lflat[c], tflat[c])
    return dict(logp_sum=_row_sums(logp, idx, R, T), lse=lse.reshape(R, T),
                logp=logp.reshape(R, T), n_tokens=n_tokens, idx=idx)


def logits_seq_logps(logits_bits, targets, mask, chunk: int = 256) -> Dict[str, np.ndarray]:
    """As ``logits_seq_logps_f64`` on bf16 bit patterns, decoded chunk by chunk."""
    R, T, V = logits_bits.shape
    idx, n_tokens = completion_positions(mask)
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    _check_targets(tflat[idx], V)
    lflat = logits_bits.reshape(R * T, V)
    lse = np.zeros(R * T)
    logp = np.zeros(R * T)
    for s in range(0, idx.size, chunk):
        c = idx[s:s + chunk]
        lse[c], logp[c] = position_logps(bf16_to_f64(lflat[c]), tflat[c])
    return dict(logp_sum=_row_sums(logp, idx, R, T), lse=lse.reshape(R, T),
                logp=logp.reshape(R, T), n_tokens=n_tokens, idx=idx)


def logits_f32_seq_logps(logits_f32, targets, mask, chunk: int = 256) -> Dict[str, np.ndarray]:
    """Sequence scores from float32 logits [R,T,V] ("DPO Training on GPU, in
    depth", "Where the memory goes": fp32 logits of a 2,048-token sequence at
    V = 128,256 take 0.98 GiB).  float32 widens to float64 exactly."""
    return logits_seq_logps_f64(np.asarray(logits_f32, dtype=np.float32).astype(np.float64),
                                targets, mask, chunk)


# ----------------------------------------------------------------------------
# a vocabulary shard's share of the log-sum-exp (tensor parallelism over V:
# the Megatron-Bridge change scores with TP=4 and notes that sums change with
# the shard count; "DPO Training on GPU, in depth", "A training configuration
# that fits": the log-softmax spans the whole vocabulary)
# ----------------------------------------------------------------------------
def shard_partials_f64(hidden: np.ndarray, w_shard: np.ndarray, targets: np.ndarray,
                       mask: np.ndarray, v_begin: int, V_total: int, chunk: int = 256
                       ) -> Dict[str, np.ndarray]:
    """For the logits z[v] = W[v] . h, v in [v_begin, v_begin + V_shard), at
    every completion position: the shard maximum m, the shard sum of
    exp(z - m), and the target logit when the target lies in the shard.

    All outputs are [R, T]; positions outside the mask, and target logits of
    targets held by another shard, are (-inf, 0, -inf).
    """
    R, T, H = hidden.shape
    Vs = w_shard.shape[0]
    idx, _ = completion_positions(mask)
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    _check_targets(tflat[idx], V_total)
    hflat = hidden.reshape(R * T, H)
    pmax = np.full(R * T, -np.inf)
    psum = np.zeros(R * T)
    ptgt = np.full(R * T, -np.inf)
    for s in range(0, idx.size, chunk):
        c = idx[s:s + chunk]
        Z = hflat[c] @ w_shard.T
        m = Z.max(axis=1)
        pmax[c] = m
        psum[c] = np.exp(Z - m[:, None]).sum(axis=1)
        y = tflat[c] - v_begin
        inside = np.flatnonzero((y >= 0) & (y < Vs))
        ptgt[c[inside]] = Z[inside, y[inside]]
    return dict(max=pmax.reshape(R, T), sumexp=psum.reshape(R, T), tgt=ptgt.reshape(R, T))


def combine_shards(part_max: np.ndarray, part_sumexp: np.ndarray, part_tgt: np.ndarray,
                   mask: np.ndarray) -> Dict[str, np.ndarray]:
    """Whole-vocabulary lse and scores from S shards' partials [S, R, T]:
    lse = M + log(sum_s sumexp_s * exp(max_s - M)) with M = max_s max_s; the
    target logit is the one shard's finite value; log p = target - lse."""
    pm = np.asarray(part_max, dtype=np.float64)
    ps = np.asarray(part_sumexp, dtype=np.float64)
    pt = np.asarray(part_tgt, dtype=np.float64)
    S, R, T = pm.shape
    idx, n_tokens = completion_positions(mask)
    pm = pm.reshape(S, R * T)[:, idx]
    ps = ps.reshape(S, R * T)[:, idx]
    pt = pt.reshape(S, R * T)[:, idx]
    M = pm.max(axis=0)
    scaled = np.where(np.isfinite(pm), ps * np.exp(np.where(np.isfinite(pm), pm - M, 0.0)), 0.0)
    lse_c = M + np.log(scaled.sum(axis=0))
    tgt = pt.max(axis=0)
    if idx.size and not np.all(np.isfinite(tgt)):
        raise ValueError("a completion position has no shard holding its target")
    lse = np.zeros(R * T)
    logp = np.zeros(R * T)
    lse[idx] = lse_c
    logp[idx] = tgt - lse_c
    return dict(logp_sum=_row_sums(logp, idx, R, T), lse=lse.reshape(R, T),
                logp=logp.reshape(R, T), n_tokens=n_tokens, idx=idx)


# ----------------------------------------------------------------------------
# forward by-product: logits sums for the logits-mean metrics ("Run
# Distributed Full-Model DPO with PyTorch FSDP", "What to Watch Out For": the loop
# logs the mean chosen and rejected logits, then frees the logits)
# ----------------------------------------------------------------------------
def logit_row_sums_f64(hidden: np.ndarray, w: np.ndarray, mask: np.ndarray,
                       chunk: int = 256) -> np.ndarray:
    """Per row: the sum of all V logits over the row's completion positions."""
    R, T, H = hidden.shape
    idx, _ = completion_positions(mask)
    hflat = hidden.reshape(R * T, H)
    tot = np.zeros(R * T)
    for s in range(0, idx.size, chunk):
        c = idx[s:s + chunk]
        tot[c] = (hflat[c] @ w.T).sum(axis=1)
    rows = idx // T
    return np.array([math.fsum(tot[idx[rows == r]].tolist()) for r in range(R)])


def logits_means(logit_sum: np.ndarray, n_tokens: np.ndarray, V: int,
                 layout: int = PAIRS_ADJACENT) -> Tuple[float, float]:
    """Mean logit over the completion positions and the vocabulary of the
    chosen rows and of the rejected rows (0 for a half without tokens)."""
    ls = np.asarray(logit_sum, dtype=np.float64)
    n = np.asarray(n_tokens, dtype=np.int64)
    c, r = pair_rows(ls.size // 2, layout)
    out = []
    for rows in (c, r):
        cnt = int(n[rows].sum())
        out.append(math.fsum(ls[rows].tolist()) / (cnt * V) if cnt else 0.0)
    return out[0], out[1]


# ----------------------------------------------------------------------------
# the sigmoid DPO loss
# ----------------------------------------------------------------------------
def pair_rows(num_pairs: int, layout: int) -> Tuple[np.ndarray, np.ndarray]:
    """Chosen and rejected row indices of each pair."""
    i = np.arange(num_pairs)
    if layout == PAIRS_ADJACENT:
        return 2 * i, 2 * i + 1
    if layout == PAIRS_HALVES:
        return i, num_pairs + i
    raise ValueError("unknown pair layout")


def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + exp(x)) without overflow: max(x, 0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-x)), evaluated on the side that cannot overflow."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def dpo_loss(policy_sum: np.ndarray, ref_sum: np.ndarray, beta: float,
             layout: int = PAIRS_ADJACENT) -> Dict[str, np.ndarray]:
    """Sigmoid DPO loss over pairs of rows.

    margin_i = beta*((pi_c - ref_c) - (pi_r - ref_r)); loss = mean_i -log sigmoid(margin_i)
    = mean_i softplus(-margin_i).  weight = -d loss / d pi per row:
    +beta*sigmoid(-margin_i)/B on the chosen row, the negative on the rejected row.
    reward = beta*(pi - ref) per row; accuracy = mean(margin_i > 0).
    """
    if not (np.isfinite(beta) and beta > 0):
        raise ValueError("beta must be finite and positive")
    pi = np.asarray(policy_sum, dtype=np.float64)
    ref = np.asarray(ref_sum, dtype=np.float64)
    R = pi.size
    if R % 2 or R == 0:
        raise ValueError("rows must be even and positive")
    B = R // 2
    c, r = pair_rows(B, layout)
    reward = beta * (pi - ref)
    margin = reward[c] - reward[r]
    loss = float(np.mean(softplus(-margin)))
    s = sigmoid(-margin)
    weight = np.zeros(R)
    weight[c] = beta * s / B
    weight[r] = -beta * s / B
    return dict(loss=loss, weight=weight, reward=reward, margin=margin,
                accuracy=float(np.mean(margin > 0)), sig_neg_margin=s)


def dpo_loss_variant(policy_sum: np.ndarray, ref_sum, n_tokens, beta: float,
                     layout: int = PAIRS_ADJACENT, length_normalise: bool = False,
                     reference_free: bool = False, sft_alpha: float = 0.0
                     ) -> Dict[str, np.ndarray]:
    """The sigmoid loss with the variants the pages name, on the same row scores.

    * reference-free ("Run Distributed Full-Model DPO with PyTorch FSDP",
      "Where to Go Next": the loop checks whether the objective is
      reference-free, which drops the reference model): reference scores are 0.
    * length-normalised ("DPO Training on GPU, in depth", "Failure modes you
      will see on real runs": sigmoid_norm against length exploitation; the
      FSDP page, "Step 4", passes sums so that the loss can average): each
      row's policy and reference scores are divided by the row's completion
      token count; a row without completion tokens averages to 0.
    * SFT / NLL term on chosen rows ("Direct Preference Optimization (DPO):
      End-to-End Implementation": total = DPO loss + alpha * NLL on the chosen
      responses, alpha called RPO alpha; "DPO Training on GPU, in depth": the
      sigmoid + sft multi-loss; the Megatron-Bridge change: optional SFT term):
      NLL = mean negative log-probability per chosen completion token of the
      batch = -sum(pi_c) / sum(n_c), 0 when the chosen rows hold no tokens.

    weight = -d loss / d pi per row, as for ``dpo_loss``.
    """
    if not (np.isfinite(beta) and beta > 0):
        raise ValueError("beta must be finite and positive")
    if not (np.isfinite(sft_alpha) and sft_alpha >= 0):
        raise ValueError("sft_alpha must be finite and non-negative")
    pi = np.asarray(policy_sum, dtype=np.float64)
    R = pi.size
    if R % 2 or R == 0:
        raise ValueError("rows must be even and positive")
    B = R // 2
    ref = np.zeros(R) if reference_free else np.asarray(ref_sum, dtype=np.float64)
    n = np.asarray(n_tokens, dtype=np.int64) if n_tokens is not None else None
    if (length_normalise or sft_alpha > 0) and n is None:
        raise ValueError("token counts are needed for length normalisation and the NLL term")
    if length_normalise:
        scale = np.where(n > 0, 1.0 / np.maximum(n, 1), 0.0)
    else:
        scale = np.ones(R)
    c, r = pair_rows(B, layout)
    reward = beta * (pi - ref) * scale
    margin = reward[c] - reward[r]
    pref = float(np.mean(softplus(-margin)))
    s = sigmoid(-margin)
    weight = np.zeros(R)
    weight[c] = beta * s * scale[c] / B
    weight[r] = -beta * s * scale[r] / B
    nll = 0.0
    if sft_alpha > 0 or n is not None:
        n_ch = int(n[c].sum()) if n is not None else 0
        if n_ch > 0:
            nll = -math.fsum(pi[c].tolist()) / n_ch
            if sft_alpha > 0:
                weight[c] += sft_alpha / n_ch
    return dict(loss=pref + sft_alpha * nll, pref_loss=pref, nll=nll, weight=weight, reward=reward,
                margin=margin, accuracy=float(np.mean(margin > 0)), sig_neg_margin=s)


# ----------------------------------------------------------------------------
# backward: dlogits = w * (softmax - onehot), dHidden = D @ W, dW = D^T @ Hc
# ----------------------------------------------------------------------------
def _row_weight(weight: np.ndarray, idx: np.ndarray, T: int) -> np.ndarray:
    return np.asarray(weight, dtype=np.float64)[idx // T]


def head_backward_f64(hidden: np.ndarray, w: np.ndarray, targets: np.ndarray, mask: np.ndarray,
                      lse: np.ndarray, weight: np.ndarray, chunk: int = 256
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Gradient of the loss w.r.t. hidden [R,T,H] and W_vocab [V,H].

    ``weight`` is -d loss / d score per row; ``lse`` the per-position
    log-sum-exp from the forward.  For a completion position t with target y:
    d loss / d z[t, v] = w_r * (softmax(z_t)[v] - [v == y]).  Mask-0 positions
    get an exactly zero hidden gradient.
    """
    R, T, H = hidden.shape
    V = w.shape[0]
    idx, _ = completion_positions(mask)
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    _check_targets(tflat[idx], V)
    hflat = hidden.reshape(R * T, H)
    lse_flat = np.asarray(lse, dtype=np.float64).reshape(-1)
    wrow = _row_weight(weight, idx, T)
    dH = np.zeros((R * T, H))
    dW = np.zeros((V, H))
    for s in range(0, idx.size, chunk):
        c = idx[s:s + chunk]
        Hc = hflat[c]
        Z = Hc @ w.T
        P = np.exp(Z - lse_flat[c][:, None])
        P[np.arange(c.size), tflat[c]] -= 1.0
        D = wrow[s:s + chunk][:, None] * P
        dH[c] = D @ w
        dW += D.T @ Hc
    return dH.reshape(R, T, H), dW


def head_backward(hidden_bits, w_bits, targets, mask, lse, weight, chunk: int = 256):
    """As ``head_backward_f64`` on bf16 bit-pattern inputs."""
    return head_backward_f64(bf16_to_f64(hidden_bits), bf16_to_f64(w_bits), targets, mask,
                             lse, weight, chunk)


def _dlogits_rows(rows_f64, targets, mask, lse, weight, pos, T, V) -> np.ndarray:
    """d loss / d logits at flat positions ``pos`` given the logits of those
    positions as float64 rows [n, V] (``rows_f64(p)`` returns them for a subset
    p of ``pos``): w_r (softmax - onehot) at completion positions, 0 elsewhere.

    The gradient of the page's hand-written loss over given logits ("DPO
    Training on GPU, in depth", "A training configuration that fits": log-softmax
    over the whole vocabulary, gather of the target, masked sum, then the
    sigmoid loss) is, per completion position t of row r with target y,
    d loss / d z[t, v] = (d loss / d pi_r) (d pi_r / d z[t, v])
                       = -w_r ([v == y] - softmax(z_t)[v]).
    """
    m = np.asarray(mask).reshape(-1) != 0
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    lse_flat = np.asarray(lse, dtype=np.float64).reshape(-1)
    out = np.zeros((pos.size, V))
    live = np.flatnonzero(m[pos])
    if live.size:
        p = pos[live]
        _check_targets(tflat[p], V)
        P = np.exp(rows_f64(p) - lse_flat[p][:, None])
        P[np.arange(p.size), tflat[p]] -= 1.0
        out[live] = _row_weight(weight, p, T)[:, None] * P
    return out


def logits_backward_rows_f64(logits, targets, mask, lse, weight, flat_positions) -> np.ndarray:
    """dlogits [n, V] (float64) at the given flat positions of float64 logits [R,T,V]."""
    R, T, V = logits.shape
    lflat = np.asarray(logits, dtype=np.float64).reshape(R * T, V)
    return _dlogits_rows(lambda p: lflat[p], targets, mask, lse, weight,
                         np.asarray(flat_positions, dtype=np.int64), T, V)


def logits_backward_rows(logits_bits, targets, mask, lse, weight, flat_positions) -> np.ndarray:
    """dlogits [n, V] (float64) for the given flat positions of a [R,T,V] bf16 logits input.

    Completion positions get w_r*(softmax - onehot); mask-0 positions get 0.
    Only the requested rows are decoded.
    """
    R, T, V = logits_bits.shape
    lflat = logits_bits.reshape(R * T, V)
    return _dlogits_rows(lambda p: bf16_to_f64(lflat[p]), targets, mask, lse, weight,
                         np.asarray(flat_positions, dtype=np.int64), T, V)


def head_backward_shard_f64(hidden: np.ndarray, w_shard: np.ndarray, targets: np.ndarray,
                            mask: np.ndarray, lse: np.ndarray, weight: np.ndarray, v_begin: int,
                            V_total: int, chunk: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """One vocabulary shard's part of the head gradient: with the whole-vocabulary
    lse, d loss / d z[t, v] = w_r (softmax[v] - [v == y]) for v in the shard;
    returns this shard's dHidden term (the shards' terms add up to dHidden) and
    dW for the shard's rows."""
    R, T, H = hidden.shape
    Vs = w_shard.shape[0]
    idx, _ = completion_positions(mask)
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    _check_targets(tflat[idx], V_total)
    hflat = hidden.reshape(R * T, H)
    lse_flat = np.asarray(lse, dtype=np.float64).reshape(-1)
    wrow = _row_weight(weight, idx, T)
    dH = np.zeros((R * T, H))
    dW = np.zeros((Vs, H))
    for s in range(0, idx.size, chunk):
        c = idx[s:s + chunk]
        Hc = hflat[c]
        P = np.exp(Hc @ w_shard.T - lse_flat[c][:, None])
        y = tflat[c] - v_begin
        inside = np.flatnonzero((y >= 0) & (y < Vs))
        P[inside, y[inside]] -= 1.0
        D = wrow[s:s + chunk][:, None] * P
        dH[c] = D @ w_shard
        dW += D.T @ Hc
    return dH.reshape(R, T, H), dW


# ----------------------------------------------------------------------------
# the same quantities at chosen positions or vocabulary rows only: checks at
# sizes where a whole [N_c, V] or [V, H] float64 array is too large for the host
# ----------------------------------------------------------------------------
def _shard_of(w, v_begin, V_total):
    Vs = w.shape[0]
    return Vs, (Vs if V_total is None else V_total)


def dhidden_rows_f64(hidden: np.ndarray, w: np.ndarray, targets, mask, lse, weight, flat_positions,
                     v_begin: int = 0, V_total=None) -> np.ndarray:
    """dHidden [n, H] at the given flat positions of hidden [R,T,H] (float64):
    sum over the vocabulary rows v of ``w`` (rows [v_begin, v_begin + V_s) of a
    V_total vocabulary; by default the whole vocabulary) of
    w_r (softmax(z_t)[v] - [v == y_t]) W[v], with ``lse`` the whole-vocabulary
    log-sum-exp.  Mask-0 positions get 0.  Per position this is the row of
    ``head_backward_f64`` (or of ``head_backward_shard_f64`` for a shard)."""
    R, T, H = hidden.shape
    Vs, V_total = _shard_of(w, v_begin, V_total)
    pos = np.asarray(flat_positions, dtype=np.int64)
    m = np.asarray(mask).reshape(-1) != 0
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    lse_flat = np.asarray(lse, dtype=np.float64).reshape(-1)
    out = np.zeros((pos.size, H))
    live = np.flatnonzero(m[pos])
    if live.size:
        p = pos[live]
        _check_targets(tflat[p], V_total)
        P = np.exp(hidden.reshape(R * T, H)[p] @ w.T - lse_flat[p][:, None])
        y = tflat[p] - v_begin
        inside = np.flatnonzero((y >= 0) & (y < Vs))
        P[inside, y[inside]] -= 1.0
        out[live] = (_row_weight(weight, p, T)[:, None] * P) @ w
    return out


def dw_rows_f64(hidden: np.ndarray, w: np.ndarray, targets, mask, lse, weight, vocab_rows,
                v_begin: int = 0, V_total=None, chunk: int = 4096) -> np.ndarray:
    """Rows ``vocab_rows`` (indices into ``w``) of dW_vocab [k, H]: the sum
    over completion positions t of w_r (softmax(z_t)[v] - [v == y_t]) h_t, as
    ``head_backward_f64`` (or ``head_backward_shard_f64``) forms it for those rows."""
    R, T, H = hidden.shape
    Vs, V_total = _shard_of(w, v_begin, V_total)
    vs = np.asarray(vocab_rows, dtype=np.int64)
    idx, _ = completion_positions(mask)
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    _check_targets(tflat[idx], V_total)
    hflat = hidden.reshape(R * T, H)
    lse_flat = np.asarray(lse, dtype=np.float64).reshape(-1)
    wrow = _row_weight(weight, idx, T)
    Wv = w[vs]
    out = np.zeros((vs.size, H))
    for s in range(0, idx.size, chunk):
        c = idx[s:s + chunk]
        Hc = hflat[c]
        P = np.exp(Hc @ Wv.T - lse_flat[c][:, None])
        P -= (tflat[c][:, None] - v_begin) == (vs[None, :])
        out += (wrow[s:s + chunk][:, None] * P).T @ Hc
    return out


def shard_partials_rows_f64(hidden: np.ndarray, w_shard: np.ndarray, targets, mask, v_begin: int,
                            V_total: int, flat_positions) -> Dict[str, np.ndarray]:
    """``shard_partials_f64`` at the given flat positions only ([n] arrays)."""
    R, T, H = hidden.shape
    Vs = w_shard.shape[0]
    pos = np.asarray(flat_positions, dtype=np.int64)
    m = np.asarray(mask).reshape(-1) != 0
    tflat = np.asarray(targets).reshape(-1).astype(np.int64)
    pmax = np.full(pos.size, -np.inf)
    psum = np.zeros(pos.size)
    ptgt = np.full(pos.size, -np.inf)
    live = np.flatnonzero(m[pos])
    if live.size:
        p = pos[live]
        _check_targets(tflat[p], V_total)
        Z = hidden.reshape(R * T, H)[p] @ w_shard.T
        mx = Z.max(axis=1)
        pmax[live] = mx
        psum[live] = np.exp(Z - mx[:, None]).sum(axis=1)
        y = tflat[p] - v_begin
        inside = np.flatnonzero((y >= 0) & (y < Vs))
        ptgt[live[inside]] = Z[inside, y[inside]]
    return dict(max=pmax, sumexp=psum, tgt=ptgt)


def logit_row_sums_by_column_sum(hidden: np.ndarray, w: np.ndarray, mask, chunk: int = 8192) -> np.ndarray:
    """The per-row logit sums of ``logit_row_sums_f64`` through the identity
    sum_t sum_v W[v] . h_t = (sum_v W[v]) . (sum_t h_t), which needs no
    [positions x V] contraction (float64; the order of the additions differs)."""
    R, T, H = hidden.shape
    wsum = np.zeros(H)
    for s in range(0, w.shape[0], chunk):
        wsum += np.asarray(w[s:s + chunk], dtype=np.float64).sum(axis=0)
    m = np.asarray(mask) != 0
    return np.array([hidden[r][m[r]].sum(axis=0) @ wsum for r in range(R)])


def logit_abs_sums_f64(hidden: np.ndarray, w: np.ndarray, flat_positions) -> np.ndarray:
    """sum over the vocabulary of |z| at each given flat position: the scale
    of the rounding error of any summation of that position's logits."""
    R, T, H = hidden.shape
    pos = np.asarray(flat_positions, dtype=np.int64)
    return np.abs(hidden.reshape(R * T, H)[pos] @ w.T).sum(axis=1)


def logits_f32_backward_rows(logits_f32, targets, mask, lse, weight, flat_positions) -> np.ndarray:
    """As ``logits_backward_rows`` for float32 logits (widened to float64 exactly)."""
    R, T, V = logits_f32.shape
    lflat = np.asarray(logits_f32, dtype=np.float32).reshape(R * T, V)
    return _dlogits_rows(lambda p: lflat[p].astype(np.float64), targets, mask, lse, weight,
                         np.asarray(flat_positions, dtype=np.int64), T, V)


# ----------------------------------------------------------------------------
# the whole path on one batch
# ----------------------------------------------------------------------------
def head_step(hidden_bits, w_bits, targets, mask, ref_sum, beta, layout=PAIRS_ADJACENT,
              chunk: int = 256) -> Dict[str, np.ndarray]:
    """Forward scores, loss and head gradients for one batch (float64 throughout)."""
    hidden = bf16_to_f64(hidden_bits)
    w = bf16_to_f64(w_bits)
    fwd = seq_logps_f64(hidden, w, targets, mask, chunk)
    loss = dpo_loss(fwd["logp_sum"], ref_sum, beta, layout)
    dH, dW = head_backward_f64(hidden, w, targets, mask, fwd["lse"], loss["weight"], chunk)
    out = dict(fwd)
    out.update(loss)
    out["d_hidden"] = dH
    out["d_w"] = dW
    return out
