"""Pins of the oracle's loss variants, vocabulary shards, fp32-logits path and
logits-mean by-products against things other than themselves: reductions to
the already pinned plain loss, hand-computed decimal values, finite
differences, the unsharded oracle (the shard combine is an exact identity of
the log-sum-exp), and closed forms.  Planted mistakes in copies of the oracle
must fail a pin.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import dpo_oracle as O

getcontext().prec = 60


def _d(x):
    return Decimal(repr(float(x)))


def _dsoftplus(x: Decimal) -> Decimal:
    return (Decimal(1) + x.exp()).ln()


def _dsigmoid(x: Decimal) -> Decimal:
    return Decimal(1) / (Decimal(1) + (-x).exp())


class _Mod:
    """Namespace copying the oracle, with some functions replaced."""

    def __init__(self, **overrides):
        for k in dir(O):
            if not k.startswith("__"):
                setattr(self, k, getattr(O, k))
        for k, v in overrides.items():
            setattr(self, k, v)


def _scores(seed, B):
    rng = np.random.default_rng(seed)
    pi = rng.standard_normal(2 * B) * 30 - 400
    ref = (pi + rng.standard_normal(2 * B) * 2).astype(np.float32)
    n = rng.integers(1, 500, size=2 * B)
    return pi, ref, n


# ----------------------------------------------------------------------------
# loss variants
# ----------------------------------------------------------------------------
def check_variant_defaults(mod):
    for seed, B, layout in [(0, 1, 0), (1, 7, 0), (2, 5, 1)]:
        pi, ref, n = _scores(seed, B)
        a = mod.dpo_loss_variant(pi, ref, n, 0.1, layout)
        b = O.dpo_loss(pi, ref, 0.1, layout)
        for k in ("weight", "reward", "margin"):
            np.testing.assert_allclose(a[k], b[k], rtol=1e-15, atol=0)
        assert abs(a["loss"] - b["loss"]) <= 1e-15 * max(1, abs(b["loss"]))
        assert a["accuracy"] == b["accuracy"]


def check_reference_free(mod):
    pi, ref, n = _scores(3, 6)
    a = mod.dpo_loss_variant(pi, None, n, 0.2, O.PAIRS_HALVES, reference_free=True)
    b = O.dpo_loss(pi, np.zeros_like(pi), 0.2, O.PAIRS_HALVES)
    np.testing.assert_allclose(a["weight"], b["weight"], rtol=1e-15)
    np.testing.assert_allclose(a["reward"], b["reward"], rtol=1e-15)
    assert abs(a["loss"] - b["loss"]) <= 1e-14


def check_length_norm_uniform(mod):
    # n = k everywhere: averaging is the plain loss with beta / k
    pi, ref, _ = _scores(4, 5)
    for k in (1, 3, 250):
        n = np.full(pi.size, k)
        a = mod.dpo_loss_variant(pi, ref, n, 0.1, O.PAIRS_ADJACENT, length_normalise=True)
        b = O.dpo_loss(pi, ref, 0.1 / k, O.PAIRS_ADJACENT)
        np.testing.assert_allclose(a["weight"], b["weight"], rtol=1e-13)
        np.testing.assert_allclose(a["margin"], b["margin"], rtol=1e-13)
        assert abs(a["loss"] - b["loss"]) <= 1e-14


def check_length_norm_decimal(mod):
    # chosen: pi -20 over 4 tokens, ref -22; rejected: pi -30 over 5 tokens, ref -29; beta 0.5
    out = mod.dpo_loss_variant(np.array([-20.0, -30.0]), np.array([-22.0, -29.0], dtype=np.float32),
                               np.array([4, 5]), 0.5, O.PAIRS_ADJACENT, length_normalise=True)
    beta = Decimal("0.5")
    rc = beta * (Decimal(-20) - Decimal(-22)) / 4
    rr = beta * (Decimal(-30) - Decimal(-29)) / 5
    m = rc - rr
    assert m == Decimal("0.35")
    assert abs(_d(out["margin"][0]) - m) < Decimal("1e-15")
    assert abs(_d(out["loss"]) - _dsoftplus(-m)) < Decimal("1e-15")
    s = _dsigmoid(-m)
    assert abs(_d(out["weight"][0]) - beta * s / 4) < Decimal("1e-16")
    assert abs(_d(out["weight"][1]) + beta * s / 5) < Decimal("1e-16")
    assert abs(_d(out["reward"][0]) - rc) < Decimal("1e-16")


def check_nll_decimal(mod):
    # chosen rows hold 5 + 3 tokens scoring -10 and -6: NLL = 16 / 8 = 2
    pi = np.array([-10.0, -12.0, -6.0, -9.0])
    ref = np.array([-11.0, -11.5, -7.0, -8.0], dtype=np.float32)
    n = np.array([5, 6, 3, 4])
    for alpha in (0.0, 1.0, 0.25):
        out = mod.dpo_loss_variant(pi, ref, n, 0.1, O.PAIRS_ADJACENT, sft_alpha=alpha)
        plain = O.dpo_loss(pi, ref, 0.1, O.PAIRS_ADJACENT)
        assert out["nll"] == 2.0
        assert abs(out["loss"] - (plain["loss"] + alpha * 2.0)) <= 1e-15
        np.testing.assert_allclose(out["weight"][[0, 2]], plain["weight"][[0, 2]] + alpha / 8, rtol=1e-15)
        np.testing.assert_allclose(out["weight"][[1, 3]], plain["weight"][[1, 3]], rtol=1e-15)


def check_variant_fd(mod):
    pi, ref, n = _scores(5, 3)
    n[1] = 0   # a row without tokens
    for ln in (False, True):
        for rf in (False, True):
            for alpha in (0.0, 0.7):
                for layout in (O.PAIRS_ADJACENT, O.PAIRS_HALVES):
                    kw = dict(length_normalise=ln, reference_free=rf, sft_alpha=alpha)
                    w = mod.dpo_loss_variant(pi, ref, n, 0.3, layout, **kw)["weight"]
                    for r in range(pi.size):
                        h = 1e-3
                        p1, p2 = pi.copy(), pi.copy()
                        p1[r] += h
                        p2[r] -= h
                        g = (mod.dpo_loss_variant(p1, ref, n, 0.3, layout, **kw)["loss"]
                             - mod.dpo_loss_variant(p2, ref, n, 0.3, layout, **kw)["loss"]) / (2 * h)
                        assert abs(-g - w[r]) <= 1e-8 + 1e-6 * abs(w[r]), (kw, layout, r, g, w[r])


def test_variant_defaults_equal_plain_loss():
    check_variant_defaults(O)


def test_reference_free_is_zero_reference():
    check_reference_free(O)


def test_length_norm_with_uniform_counts_scales_beta():
    check_length_norm_uniform(O)


def test_length_norm_decimal_example():
    check_length_norm_decimal(O)


def test_nll_term_decimal_example():
    check_nll_decimal(O)


def test_variant_weights_are_minus_gradient():
    check_variant_fd(O)


def test_length_norm_empty_row_has_no_weight():
    pi, ref, n = _scores(6, 2)
    n[3] = 0
    out = O.dpo_loss_variant(pi, ref, n, 0.1, O.PAIRS_ADJACENT, length_normalise=True)
    assert out["weight"][3] == 0.0 and out["reward"][3] == 0.0


def test_variant_rejects_bad_arguments():
    pi, ref, n = _scores(7, 2)
    with pytest.raises(ValueError):
        O.dpo_loss_variant(pi, ref, n, 0.0)
    with pytest.raises(ValueError):
        O.dpo_loss_variant(pi, ref, n, 0.1, sft_alpha=-1.0)
    with pytest.raises(ValueError):
        O.dpo_loss_variant(pi, ref, n, 0.1, sft_alpha=float("nan"))
    with pytest.raises(ValueError):
        O.dpo_loss_variant(pi, ref, None, 0.1, length_normalise=True)


def _mut_nll_per_pair(policy_sum, ref_sum, n_tokens, beta, layout=O.PAIRS_ADJACENT, length_normalise=False,
                      reference_free=False, sft_alpha=0.0):
    out = O.dpo_loss_variant(policy_sum, ref_sum, n_tokens, beta, layout, length_normalise, reference_free, 0.0)
    c, _ = O.pair_rows(len(policy_sum) // 2, layout)
    nll = -np.sum(np.asarray(policy_sum)[c]) / c.size   # mean over pairs, not tokens
    out["nll"] = nll
    out["loss"] += sft_alpha * nll
    out["weight"][c] += sft_alpha / c.size
    return out


def _mut_ref_not_normalised(policy_sum, ref_sum, n_tokens, beta, layout=O.PAIRS_ADJACENT, length_normalise=False,
                            reference_free=False, sft_alpha=0.0):
    if not length_normalise:
        return O.dpo_loss_variant(policy_sum, ref_sum, n_tokens, beta, layout, False, reference_free, sft_alpha)
    n = np.asarray(n_tokens, dtype=np.float64)
    pi = np.asarray(policy_sum, dtype=np.float64)
    ref = np.asarray(ref_sum, dtype=np.float64)
    # averages the policy score but not the reference score
    shifted = pi - ref * n + ref
    return O.dpo_loss_variant(shifted, ref, n_tokens, beta, layout, True, reference_free, sft_alpha)


def _mut_weight_ignores_length(policy_sum, ref_sum, n_tokens, beta, layout=O.PAIRS_ADJACENT, length_normalise=False,
                               reference_free=False, sft_alpha=0.0):
    out = O.dpo_loss_variant(policy_sum, ref_sum, n_tokens, beta, layout, length_normalise, reference_free, sft_alpha)
    if length_normalise:
        plain = O.dpo_loss_variant(policy_sum, ref_sum, n_tokens, beta, layout, False, reference_free, sft_alpha)
        out["weight"] = plain["weight"]
    return out


# ----------------------------------------------------------------------------
# vocabulary shards
# ----------------------------------------------------------------------------
def _tiny(seed=0, R=4, T=8, H=16, V=40, wscale=0.8):
    rng = np.random.default_rng(seed)
    hidden = rng.standard_normal((R, T, H))
    w = rng.standard_normal((V, H)) * wscale
    targets = rng.integers(0, V, size=(R, T))
    mask = np.zeros((R, T), dtype=np.uint8)
    for r in range(R):
        mask[r, rng.integers(1, T // 2):] = 1
    mask[2, :] = 0   # an empty row
    return hidden, w, np.where(mask != 0, targets, -100), mask


def _split(V, cuts):
    b = [0] + list(cuts) + [V]
    return [(b[i], b[i + 1]) for i in range(len(b) - 1)]


def check_shard_combine(mod):
    hidden, w, targets, mask = _tiny()
    V = w.shape[0]
    whole = O.seq_logps_f64(hidden, w, targets, mask)
    for cuts in ([], [20], [7, 20, 33], list(range(8, 40, 8))):
        parts = [mod.shard_partials_f64(hidden, w[a:b], targets, mask, a, V) for a, b in _split(V, cuts)]
        comb = mod.combine_shards(np.stack([p["max"] for p in parts]), np.stack([p["sumexp"] for p in parts]),
                                  np.stack([p["tgt"] for p in parts]), mask)
        np.testing.assert_array_equal(comb["n_tokens"], whole["n_tokens"])
        np.testing.assert_array_equal(comb["idx"], whole["idx"])
        np.testing.assert_allclose(comb["lse"], whole["lse"], rtol=1e-14, atol=1e-13)
        np.testing.assert_allclose(comb["logp_sum"], whole["logp_sum"], rtol=1e-13, atol=1e-12)


def check_shard_backward(mod):
    hidden, w, targets, mask = _tiny(1)
    V = w.shape[0]
    fwd = O.seq_logps_f64(hidden, w, targets, mask)
    weight = np.array([0.03, -0.03, 0.01, -0.01])
    dH, dW = O.head_backward_f64(hidden, w, targets, mask, fwd["lse"], weight)
    sH = np.zeros_like(dH)
    sW = []
    for a, b in _split(V, [9, 25]):
        h, g = mod.head_backward_shard_f64(hidden, w[a:b], targets, mask, fwd["lse"], weight, a, V)
        sH += h
        sW.append(g)
    np.testing.assert_allclose(sH, dH, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(np.concatenate(sW), dW, rtol=1e-12, atol=1e-15)


def test_shards_combine_to_whole_vocabulary():
    check_shard_combine(O)


def test_shard_gradients_add_up_to_whole():
    check_shard_backward(O)


def test_shard_partials_outside_mask_and_foreign_targets():
    hidden, w, targets, mask = _tiny(2)
    p = O.shard_partials_f64(hidden, w[10:20], targets, mask, 10, w.shape[0])
    off = mask == 0
    assert np.all(p["max"][off] == -np.inf) and np.all(p["sumexp"][off] == 0) and np.all(p["tgt"][off] == -np.inf)
    on = mask != 0
    inside = on & (targets >= 10) & (targets < 20)
    assert np.all(np.isfinite(p["tgt"][inside])) and np.all(p["tgt"][on & ~inside] == -np.inf)
    # one shard's sum of exp(z - max) lies in [1, V_shard]
    assert np.all(p["sumexp"][on] >= 1.0) and np.all(p["sumexp"][on] <= 10.0)


def test_combine_rejects_missing_target_shard():
    hidden, w, targets, mask = _tiny(3)
    p = O.shard_partials_f64(hidden, w[:20], targets, mask, 0, w.shape[0])
    if np.any((targets >= 20) & (mask != 0)):
        with pytest.raises(ValueError):
            O.combine_shards(p["max"][None], p["sumexp"][None], p["tgt"][None], mask)


def _mut_combine_no_rescale(part_max, part_sumexp, part_tgt, mask):
    pm = np.asarray(part_max)
    out = O.combine_shards(np.zeros_like(pm) + pm.max(axis=0, keepdims=True), part_sumexp, part_tgt, mask)
    return out   # sums exp(z - m_s) of every shard as if all shards had the same max


def _mut_shard_onehot_everywhere(hidden, w_shard, targets, mask, lse, weight, v_begin, V_total, chunk=256):
    t = np.where(np.asarray(mask) != 0, np.asarray(targets) % w_shard.shape[0] + v_begin, targets)
    return O.head_backward_shard_f64(hidden, w_shard, t, mask, lse, weight, v_begin, V_total, chunk)


# ----------------------------------------------------------------------------
# fp32 logits
# ----------------------------------------------------------------------------
def check_f32_logits(mod):
    rng = np.random.default_rng(8)
    R, T, V = 4, 6, 48
    bits = O.f64_to_bf16_rne(rng.standard_normal((R, T, V)) * 3)
    f32 = bits.astype(np.float32)   # bf16 values are exact in float32
    raw = (f32.view(np.uint32) >> 16).astype(np.uint16)
    mask = np.zeros((R, T), dtype=np.uint8)
    mask[:, 2:] = 1
    targets = np.where(mask != 0, rng.integers(0, V, (R, T)), -100)
    a = mod.logits_f32_seq_logps(f32, targets, mask)
    b = O.logits_seq_logps(raw, targets, mask)
    np.testing.assert_array_equal(a["logp_sum"], b["logp_sum"])
    np.testing.assert_array_equal(a["lse"], b["lse"])
    weight = np.array([0.05, -0.05, 0.02, -0.02])
    pos = np.arange(R * T)
    np.testing.assert_array_equal(mod.logits_f32_backward_rows(f32, targets, mask, a["lse"], weight, pos),
                                  O.logits_backward_rows(raw, targets, mask, a["lse"], weight, pos))
    # values off the bf16 grid: an fp32 logit keeps its full value
    f = (rng.standard_normal((R, T, V)) * 3).astype(np.float32)
    c = mod.logits_f32_seq_logps(f, targets, mask)
    z = f.astype(np.float64).reshape(R * T, V)
    t = targets.reshape(-1)
    for p in np.flatnonzero(mask.reshape(-1)):
        lse = math.log(math.fsum(math.exp(x) for x in z[p]))
        assert abs(c["lse"].reshape(-1)[p] - lse) < 1e-12
        assert abs(c["logp"].reshape(-1)[p] - (z[p, t[p]] - lse)) < 1e-12


def test_f32_logits_path():
    check_f32_logits(O)


# ----------------------------------------------------------------------------
# logits-mean by-products
# ----------------------------------------------------------------------------
def check_logit_sums(mod):
    hidden, w, targets, mask = _tiny(4)
    got = mod.logit_row_sums_f64(hidden, w, mask)
    colsum = w.sum(axis=0)   # sum_v z[v] = h . sum_v W[v]
    want = np.array([(hidden[r][mask[r] != 0] @ colsum).sum() for r in range(hidden.shape[0])])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert got[2] == 0.0


def check_logits_means(mod):
    ls = np.array([10.0, -4.0, 6.0, 2.0])
    n = np.array([2, 1, 3, 1])
    assert mod.logits_means(ls, n, 4, O.PAIRS_ADJACENT) == (0.8, -0.25)
    assert mod.logits_means(ls, n, 4, O.PAIRS_HALVES) == (0.5, 0.5)
    assert mod.logits_means(ls, np.array([0, 1, 0, 1]), 4, O.PAIRS_ADJACENT)[0] == 0.0


def test_logit_row_sums_closed_form():
    check_logit_sums(O)


def test_logits_means_hand_values():
    check_logits_means(O)


def _mut_means_without_vocab(logit_sum, n_tokens, V, layout=O.PAIRS_ADJACENT):
    return O.logits_means(logit_sum, n_tokens, 1, layout)


def _mut_logit_sums_all_positions(hidden, w, mask, chunk=256):
    return O.logit_row_sums_f64(hidden, w, np.ones_like(mask), chunk)


# ----------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("mutant,pin", [
    (dict(dpo_loss_variant=_mut_nll_per_pair), check_nll_decimal),
    (dict(dpo_loss_variant=_mut_ref_not_normalised), check_length_norm_uniform),
    (dict(dpo_loss_variant=_mut_weight_ignores_length), check_variant_fd),
    (dict(combine_shards=_mut_combine_no_rescale), check_shard_combine),
    (dict(head_backward_shard_f64=_mut_shard_onehot_everywhere), check_shard_backward),
    (dict(logits_means=_mut_means_without_vocab), check_logits_means),
    (dict(logit_row_sums_f64=_mut_logit_sums_all_positions), check_logit_sums),
])
def test_planted_mistake_is_caught(mutant, pin):
    with pytest.raises(AssertionError):
        pin(_Mod(**mutant))
