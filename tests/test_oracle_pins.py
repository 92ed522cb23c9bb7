"""Pins of the CPU oracle against things other than itself.

Each test ties an oracle function to something the pages or mathematics fix:
the worked example printed on "DPO Training on GPU, in depth" (section "A
worked example of the numbers"), the ln 2 start-of-training invariant from the
same section, closed forms, brute force with high-precision decimals,
finite differences, and a PyTorch float64 autograd cross-check of the page's
hand-written loss (section "A training configuration that fits").  The last
group plants mistakes in a copy of the oracle and checks that a pin fails.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import dpo_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
getcontext().prec = 60


def _dexp(x: float) -> Decimal:
    return Decimal(repr(float(x))).exp()


def _dlog(x: Decimal) -> Decimal:
    return x.ln()


def _worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def _tiny_case(seed=0, R=4, T=8, H=16, V=32, hscale=1.0, wscale=0.3, layout=O.PAIRS_ADJACENT):
    rng = np.random.default_rng(seed)
    hidden = rng.standard_normal((R, T, H)) * hscale
    w = rng.standard_normal((V, H)) * wscale
    targets = rng.integers(0, V, size=(R, T))
    mask = np.zeros((R, T), dtype=np.uint8)
    for r in range(R):
        a = rng.integers(1, T // 2)
        mask[r, a:] = 1
    targets = np.where(mask != 0, targets, -100)
    ref = rng.standard_normal(R) * 2 - 20
    return hidden, w, targets, mask, ref


# ----------------------------------------------------------------------------
# the loss: worked example, ln 2, closed forms
# ----------------------------------------------------------------------------
def check_worked_example(mod):
    g = _worked()
    p = g["printed"]
    d = g["printed_decimals"]
    pi = np.array([g["policy_chosen"], g["policy_rejected"]])
    ref = np.array([g["ref_chosen"], g["ref_rejected"]])
    out = mod.dpo_loss(pi, ref, g["beta"], mod.PAIRS_ADJACENT)
    half = lambda k: 0.5 * 10.0 ** (-d[k]) + 1e-12  # noqa: E731
    assert abs(out["reward"][0] - p["reward_chosen"]) <= half("reward_chosen")
    assert abs(out["reward"][1] - p["reward_rejected"]) <= half("reward_rejected")
    assert abs(out["margin"][0] - p["margin"]) <= half("margin")
    assert abs(out["loss"] - p["loss"]) <= half("loss")
    assert abs(out["sig_neg_margin"][0] - p["gradient_scale_sigmoid_neg_margin"]) <= half(
        "gradient_scale_sigmoid_neg_margin")
    # one pair: the row weights are +-beta*sigmoid(-margin)
    assert abs(out["weight"][0] - g["beta"] * p["gradient_scale_sigmoid_neg_margin"]) <= 1e-4
    assert out["weight"][1] == -out["weight"][0]
    assert out["accuracy"] == 1.0


def test_worked_example_printed_values():
    check_worked_example(O)


def test_worked_example_exact_decimal():
    """Same pair, loss and gradient scale from 60-digit decimals."""
    g = _worked()
    m = Decimal("0.1") * ((Decimal("-42.0") + Decimal("43.0")) - (Decimal("-47.5") + Decimal("46.0")))
    assert m == Decimal("0.25")
    loss = (Decimal(1) + (-m).exp()).ln()
    sig = Decimal(1) / (Decimal(1) + m.exp())
    out = O.dpo_loss(np.array([-42.0, -47.5]), np.array([-43.0, -46.0]), g["beta"])
    assert abs(Decimal(repr(float(out["loss"]))) - loss) < Decimal("1e-15")
    assert abs(Decimal(repr(float(out["sig_neg_margin"][0]))) - sig) < Decimal("1e-15")


def check_ln2(mod):
    rng = np.random.default_rng(3)
    for B in (1, 2, 7):
        pi = rng.standard_normal(2 * B) * 50 - 300
        for layout in (mod.PAIRS_ADJACENT, mod.PAIRS_HALVES):
            out = mod.dpo_loss(pi, pi.copy(), 0.1, layout)
            assert abs(out["loss"] - math.log(2.0)) < 1e-15
            assert abs(round(out["loss"], 3) - _worked()["printed"]["loss_at_policy_equal_reference"]) < 1e-12
            assert out["accuracy"] == 0.0          # strict margin > 0
            np.testing.assert_allclose(np.abs(out["weight"]), 0.1 * 0.5 / B, rtol=1e-15)
            assert abs(out["weight"].sum()) < 1e-15


def test_ln2_when_policy_equals_reference():
    check_ln2(O)


def check_loss_closed_forms(mod):
    # L(m) - L(-m) = -m for the per-pair loss softplus(-m)
    for m in [-800.0, -30.0, -1.5, -1e-9, 0.0, 1e-9, 0.25, 3.0, 40.0, 800.0]:
        lhs = mod.softplus(np.array([-m]))[0] - mod.softplus(np.array([m]))[0]
        assert abs(lhs - (-m)) <= 1e-12 * max(1.0, abs(m))
    # against high-precision decimals in the range where they are cheap
    for x in [-20.0, -3.3, -0.1, 0.0, 0.7, 5.0, 30.0]:
        ref_sp = _dlog(Decimal(1) + _dexp(x))
        assert abs(Decimal(repr(float(mod.softplus(np.array([x]))[0]))) - ref_sp) < Decimal("1e-14")
        ref_sig = Decimal(1) / (Decimal(1) + _dexp(-x))
        assert abs(Decimal(repr(float(mod.sigmoid(np.array([x]))[0]))) - ref_sig) < Decimal("1e-15")


def test_loss_closed_forms():
    check_loss_closed_forms(O)


def test_loss_mean_over_pairs_and_layouts():
    """Mean over pairs; the halves layout is a row permutation of the adjacent layout."""
    rng = np.random.default_rng(5)
    B = 5
    pi = rng.standard_normal(2 * B) * 10 - 100
    ref = pi + rng.standard_normal(2 * B)
    adj = O.dpo_loss(pi, ref, 0.1, O.PAIRS_ADJACENT)
    perm = np.concatenate([np.arange(0, 2 * B, 2), np.arange(1, 2 * B, 2)])
    hv = O.dpo_loss(pi[perm], ref[perm], 0.1, O.PAIRS_HALVES)
    assert abs(adj["loss"] - hv["loss"]) < 1e-15
    np.testing.assert_array_equal(adj["weight"][perm], hv["weight"])
    # a single-pair loss per pair, averaged
    singles = [O.dpo_loss(pi[2 * i:2 * i + 2], ref[2 * i:2 * i + 2], 0.1)["loss"] for i in range(B)]
    assert abs(adj["loss"] - math.fsum(singles) / B) < 1e-15


def test_loss_gradient_is_minus_weight():
    """weight = -d loss / d score, by central differences on the loss."""
    rng = np.random.default_rng(9)
    pi = rng.standard_normal(6) * 3 - 50
    ref = pi + rng.standard_normal(6) * 4
    out = O.dpo_loss(pi, ref, 0.3, O.PAIRS_ADJACENT)
    h = 1e-6
    for r in range(6):
        e = np.zeros(6)
        e[r] = h
        fd = (O.dpo_loss(pi + e, ref, 0.3)["loss"] - O.dpo_loss(pi - e, ref, 0.3)["loss"]) / (2 * h)
        assert abs(-fd - out["weight"][r]) < 1e-9


def test_loss_rejects_bad_beta_and_rows():
    for beta in (0.0, -0.1, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            O.dpo_loss(np.zeros(2), np.zeros(2), beta)
    with pytest.raises(ValueError):
        O.dpo_loss(np.zeros(3), np.zeros(3), 0.1)


# ----------------------------------------------------------------------------
# log-softmax, gather, masked sums
# ----------------------------------------------------------------------------
def check_bruteforce_logsoftmax(mod):
    rng = np.random.default_rng(11)
    for V in (1, 2, 7, 64):
        Z = rng.standard_normal((5, V)) * 4
        tgt = rng.integers(0, V, size=5)
        lse, logp = mod.position_logps(Z, tgt)
        for i in range(5):
            s = sum((_dexp(z) for z in Z[i]), Decimal(0))
            ref_lse = _dlog(s)
            assert abs(Decimal(repr(float(lse[i]))) - ref_lse) < Decimal("1e-13")
            ref_lp = Decimal(repr(float(Z[i, tgt[i]]))) - ref_lse
            assert abs(Decimal(repr(float(logp[i]))) - ref_lp) < Decimal("1e-13")
            assert logp[i] <= 1e-15


def test_logsoftmax_bruteforce_decimal():
    check_bruteforce_logsoftmax(O)


def test_logsoftmax_large_logits_and_shift_invariance():
    rng = np.random.default_rng(12)
    Z = rng.standard_normal((4, 300)) * 3
    tgt = rng.integers(0, 300, size=4)
    _, lp = O.position_logps(Z, tgt)
    for c in (-1e4, 1e4, 700.0):
        _, lp2 = O.position_logps(Z + c, tgt)
        np.testing.assert_allclose(lp2, lp, atol=1e-9)
    # softmax sums to one
    lse = O.logsumexp_rows(Z)
    np.testing.assert_allclose(np.exp(Z - lse[:, None]).sum(1), 1.0, rtol=1e-14)


def check_w_zero_closed_form(mod):
    R, T, H = 4, 16, 8
    for V in (1, 5, 1024, 128256):
        hidden = np.random.default_rng(1).standard_normal((R, T, H))
        w = np.zeros((V, H))
        targets = np.random.default_rng(2).integers(0, V, size=(R, T))
        mask = np.zeros((R, T), np.uint8)
        mask[:, 4:] = 1
        mask[3, :] = 0
        mask[2, 10:] = 0
        out = mod.seq_logps_f64(hidden, w, targets, mask)
        n = mask.astype(np.int64).sum(1)
        np.testing.assert_array_equal(out["n_tokens"], n)
        np.testing.assert_allclose(out["logp_sum"], -n * math.log(V), rtol=1e-14, atol=0)
        np.testing.assert_allclose(out["lse"][mask != 0], math.log(V), rtol=1e-14)


def test_w_zero_gives_minus_n_log_v():
    check_w_zero_closed_form(O)


def test_bf16_decode_known_patterns():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0x4049, 0x7F7F, 0x0080, 0x3F81], np.uint16)
    want = [0.0, -0.0, 1.0, -1.0, 2.0, 3.140625, 3.3895313892515355e38, 2.0 ** -126, 1.0 + 2 ** -7]
    got = O.bf16_to_f64(bits)
    for g_, w_ in zip(got, want):
        assert g_ == w_


def test_bf16_rne_rounding_matches_float32_encoder():
    """The oracle's fp64 -> bf16 rounding agrees with an independent float32 bit-level encoder."""
    from preference_alignment_amd.workloads import bf16_rne_bits
    rng = np.random.default_rng(4)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    # include exact ties
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3 * 2 ** -9, 257.0, 259.0], np.float32)
    x32 = np.concatenate([x32, ties])
    enc = O.bf16_to_f64(bf16_rne_bits(x32))
    np.testing.assert_array_equal(O.f64_to_bf16_rne(x32.astype(np.float64)), enc)
    assert O.f64_to_bf16_rne(np.array([1 + 2 ** -8]))[0] == 1.0
    assert O.f64_to_bf16_rne(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


def test_masked_targets_are_never_read():
    hidden, w, targets, mask, ref = _tiny_case(seed=21)
    a = O.seq_logps_f64(hidden, w, targets, mask)
    t2 = targets.copy()
    t2[mask == 0] = 10 ** 9
    b = O.seq_logps_f64(hidden, w, t2, mask)
    np.testing.assert_array_equal(a["logp_sum"], b["logp_sum"])
    loss = O.dpo_loss(a["logp_sum"], ref, 0.1)
    g1 = O.head_backward_f64(hidden, w, targets, mask, a["lse"], loss["weight"])
    g2 = O.head_backward_f64(hidden, w, t2, mask, b["lse"], loss["weight"])
    np.testing.assert_array_equal(g1[0], g2[0])
    np.testing.assert_array_equal(g1[1], g2[1])
    with pytest.raises(ValueError):
        t3 = targets.copy()
        t3[mask != 0] = w.shape[0]
        O.seq_logps_f64(hidden, w, t3, mask)


def test_empty_row_scores_zero_and_gets_no_gradient():
    hidden, w, targets, mask, ref = _tiny_case(seed=22)
    mask[1, :] = 0
    targets[1, :] = -100
    out = O.seq_logps_f64(hidden, w, targets, mask)
    assert out["logp_sum"][1] == 0.0 and out["n_tokens"][1] == 0
    loss = O.dpo_loss(out["logp_sum"], ref, 0.1)
    dH, _ = O.head_backward_f64(hidden, w, targets, mask, out["lse"], loss["weight"])
    assert np.all(dH[1] == 0)
    assert np.all(dH[mask == 0] == 0)


def test_row_sums_equal_sum_of_positions_and_counts():
    hidden, w, targets, mask, _ = _tiny_case(seed=23, T=40)
    out = O.seq_logps_f64(hidden, w, targets, mask, chunk=7)
    for r in range(hidden.shape[0]):
        cols = np.flatnonzero(mask[r])
        direct = 0.0
        for t in cols:
            z = w @ hidden[r, t]
            direct += z[targets[r, t]] - math.log(sum(math.exp(v) for v in z))
        assert abs(out["logp_sum"][r] - direct) < 1e-10
        assert out["n_tokens"][r] == cols.size
    # chunk size does not change anything
    out2 = O.seq_logps_f64(hidden, w, targets, mask, chunk=1000)
    np.testing.assert_array_equal(out["logp_sum"], out2["logp_sum"])


def test_logits_path_matches_head_path():
    hidden, w, targets, mask, ref = _tiny_case(seed=24)
    a = O.seq_logps_f64(hidden, w, targets, mask)
    logits = hidden @ w.T
    b = O.logits_seq_logps_f64(logits, targets, mask)
    np.testing.assert_allclose(a["logp_sum"], b["logp_sum"], rtol=1e-13)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-13)


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------
def _total_loss(hidden, w, targets, mask, ref, beta, layout=O.PAIRS_ADJACENT):
    out = O.seq_logps_f64(hidden, w, targets, mask)
    return O.dpo_loss(out["logp_sum"], ref, beta, layout)["loss"]


def check_finite_differences(mod, seed=31):
    hidden, w, targets, mask, ref = _tiny_case(seed=seed)
    beta = 0.5
    fwd = mod.seq_logps_f64(hidden, w, targets, mask)
    loss = mod.dpo_loss(fwd["logp_sum"], ref, beta)
    dH, dW = mod.head_backward_f64(hidden, w, targets, mask, fwd["lse"], loss["weight"])
    rng = np.random.default_rng(seed + 1)
    h = 1e-5
    for _ in range(12):
        r, t, k = rng.integers(0, hidden.shape[0]), rng.integers(0, hidden.shape[1]), rng.integers(0, hidden.shape[2])
        hp, hm = hidden.copy(), hidden.copy()
        hp[r, t, k] += h
        hm[r, t, k] -= h
        fd = (_total_loss(hp, w, targets, mask, ref, beta) - _total_loss(hm, w, targets, mask, ref, beta)) / (2 * h)
        assert abs(fd - dH[r, t, k]) < 1e-8 + 1e-5 * abs(fd)
    for _ in range(12):
        v, k = rng.integers(0, w.shape[0]), rng.integers(0, w.shape[1])
        wp, wm = w.copy(), w.copy()
        wp[v, k] += h
        wm[v, k] -= h
        fd = (_total_loss(hidden, wp, targets, mask, ref, beta) - _total_loss(hidden, wm, targets, mask, ref, beta)) / (2 * h)
        assert abs(fd - dW[v, k]) < 1e-8 + 1e-5 * abs(fd)


def test_backward_finite_differences():
    check_finite_differences(O)


def test_backward_torch_fp64_autograd():
    """Library cross-check: torch float64 log_softmax/gather/logsigmoid + autograd."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    for layout in (O.PAIRS_ADJACENT, O.PAIRS_HALVES):
        hidden, w, targets, mask, ref = _tiny_case(seed=41 + layout, R=6, T=12, H=24, V=40)
        beta = 0.1
        fwd = O.seq_logps_f64(hidden, w, targets, mask)
        loss = O.dpo_loss(fwd["logp_sum"], ref, beta, layout)
        dH, dW = O.head_backward_f64(hidden, w, targets, mask, fwd["lse"], loss["weight"])

        th = torch.tensor(hidden, dtype=torch.float64, requires_grad=True)
        tw = torch.tensor(w, dtype=torch.float64, requires_grad=True)
        logits = th @ tw.T
        lbl = torch.tensor(np.where(mask != 0, targets, 0), dtype=torch.int64)
        m = torch.tensor(mask, dtype=torch.float64)
        lp = torch.gather(F.log_softmax(logits, dim=-1), 2, lbl.unsqueeze(-1)).squeeze(-1)
        logps = (lp * m).sum(dim=1)
        B = hidden.shape[0] // 2
        if layout == O.PAIRS_ADJACENT:
            pc, pr = logps[0::2], logps[1::2]
            rc, rr = torch.tensor(ref[0::2]), torch.tensor(ref[1::2])
        else:
            pc, pr = logps[:B], logps[B:]
            rc, rr = torch.tensor(ref[:B]), torch.tensor(ref[B:])
        margin = beta * ((pc - rc) - (pr - rr))
        tl = -F.logsigmoid(margin).mean()
        tl.backward()
        np.testing.assert_allclose(fwd["logp_sum"], logps.detach().numpy(), rtol=1e-13)
        assert abs(loss["loss"] - tl.item()) < 1e-14
        assert abs(loss["accuracy"] - (margin > 0).double().mean().item()) == 0
        np.testing.assert_allclose(dH, th.grad.numpy(), rtol=1e-10, atol=1e-16)
        np.testing.assert_allclose(dW, tw.grad.numpy(), rtol=1e-10, atol=1e-16)


def test_backward_invariants():
    hidden, w, targets, mask, ref = _tiny_case(seed=51, V=50)
    fwd = O.seq_logps_f64(hidden, w, targets, mask)
    loss = O.dpo_loss(fwd["logp_sum"], ref, 0.1)
    dH, dW = O.head_backward_f64(hidden, w, targets, mask, fwd["lse"], loss["weight"])
    # sum over the vocabulary of dlogits is 0 at every position, hence sum_v dW[v, :] = 0
    np.testing.assert_allclose(dW.sum(0), 0.0, atol=1e-13)
    # dH_t = w_r * (E_softmax[W] - W[target])
    for r in range(hidden.shape[0]):
        for t in np.flatnonzero(mask[r]):
            z = w @ hidden[r, t]
            p = np.exp(z - z.max())
            p /= p.sum()
            want = loss["weight"][r] * (p @ w - w[targets[r, t]])
            np.testing.assert_allclose(dH[r, t], want, rtol=1e-10, atol=1e-15)


# ----------------------------------------------------------------------------
# planted mistakes: a copy of the oracle with one error must fail a pin
# ----------------------------------------------------------------------------
class _Mutant:
    """Namespace copying the oracle, with one function replaced."""

    def __init__(self, **overrides):
        for k in dir(O):
            if not k.startswith("__"):
                setattr(self, k, getattr(O, k))
        for k, v in overrides.items():
            setattr(self, k, v)


def _mut_loss_sign(policy_sum, ref_sum, beta, layout=O.PAIRS_ADJACENT):
    out = O.dpo_loss(policy_sum, ref_sum, beta, layout)
    out["loss"] = float(np.mean(O.softplus(out["margin"])))   # sign of the margin flipped
    return out


def _mut_loss_sum_not_mean(policy_sum, ref_sum, beta, layout=O.PAIRS_ADJACENT):
    out = O.dpo_loss(policy_sum, ref_sum, beta, layout)
    out["loss"] = float(np.sum(O.softplus(-out["margin"])))
    return out


def _mut_swapped_pairs(policy_sum, ref_sum, beta, layout=O.PAIRS_ADJACENT):
    return O.dpo_loss(policy_sum, ref_sum, beta, O.PAIRS_HALVES if layout == O.PAIRS_ADJACENT else O.PAIRS_ADJACENT)


def _mut_no_log(Z, tgt):
    m = Z.max(axis=1)
    lse = m + np.exp(Z - m[:, None]).sum(axis=1)   # forgot the log
    return lse, Z[np.arange(Z.shape[0]), tgt] - lse


def _mut_lse_missing_max(Z):
    m = Z.max(axis=1)
    return np.log(np.exp(Z - m[:, None]).sum(axis=1))   # dropped the +m term


def _mut_backward_dw_sign(hidden, w, targets, mask, lse, weight, chunk=256):
    dH, dW = O.head_backward_f64(hidden, w, targets, mask, lse, weight, chunk)
    return dH, -dW   # dW sign flipped


def _mut_seq_shifted_targets(hidden, w, targets, mask, chunk=256):
    return O.seq_logps_f64(hidden, w, np.roll(np.where(mask != 0, targets, 0), 1, axis=1), mask, chunk)


def _mut_backward_no_onehot(hidden, w, targets, mask, lse, weight, chunk=256):
    R, T, H = hidden.shape
    idx, _ = O.completion_positions(mask)
    hflat = hidden.reshape(R * T, H)
    dH = np.zeros((R * T, H))
    dW = np.zeros_like(w)
    wr = np.asarray(weight)[idx // T]
    Z = hflat[idx] @ w.T
    D = wr[:, None] * np.exp(Z - np.asarray(lse).reshape(-1)[idx][:, None])   # onehot term dropped
    dH[idx] = D @ w
    dW += D.T @ hflat[idx]
    return dH.reshape(R, T, H), dW


@pytest.mark.parametrize("mutant,pin", [
    (dict(dpo_loss=_mut_loss_sign), check_worked_example),
    (dict(dpo_loss=_mut_loss_sum_not_mean), check_ln2),
    (dict(dpo_loss=_mut_swapped_pairs), lambda mod: check_finite_differences(mod)),
    (dict(position_logps=_mut_no_log), check_bruteforce_logsoftmax),
    (dict(logsumexp_rows=_mut_lse_missing_max), check_bruteforce_logsoftmax),
    (dict(head_backward_f64=_mut_backward_dw_sign), check_finite_differences),
    (dict(seq_logps_f64=_mut_seq_shifted_targets), check_finite_differences),
    (dict(head_backward_f64=_mut_backward_no_onehot), check_finite_differences),
])
def test_planted_mistake_is_caught(mutant, pin):
    mod = _Mutant(**mutant)
    if "logsumexp_rows" in mutant:
        # position_logps reaches logsumexp_rows through the module; route it to the mutant
        def position_logps(Z, tgt, _f=mutant["logsumexp_rows"]):
            lse = _f(Z)
            return lse, Z[np.arange(Z.shape[0]), tgt] - lse
        mod.position_logps = position_logps
    with pytest.raises(AssertionError):
        pin(mod)
