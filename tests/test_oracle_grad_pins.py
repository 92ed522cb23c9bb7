"""Pins of the oracle's gradient over given logits and of its sampled-output
helpers, against things other than themselves.

The gradient over given logits ("DPO Training on GPU, in depth", "A training
configuration that fits": the hand-written chunked loss takes logits, applies
a full-vocabulary log-softmax, gathers the target, sums over the completion
mask and feeds the sigmoid loss; "Where the memory goes for an 8B model" sizes
those logits) is tied to:

* central finite differences of the oracle's own forward-plus-loss over
  given logits (``logits_seq_logps*`` then ``dpo_loss``, both pinned in
  tests/test_oracle_pins.py), element by element, on float64, bf16 and fp32
  logits; the bf16 and fp32 perturbations are exact in their own format
  (grid values, power-of-two steps) and the bf16 one is extrapolated
  (Richardson) because its step cannot be small;
* the head path: with logits = Hc W^T, dlogits . W must be the pinned
  ``head_backward_f64`` dHidden and dlogits^T . Hc its dW;
* planted mistakes (another row's weight, no weight, one-hot at the wrong id,
  a doubled weight, a softmax without its shift) that must each fail a pin.

The sampled-output helpers (dHidden at chosen positions, dW at chosen rows,
shard partials at chosen positions, logit sums through the column-sum
identity) are tied to the whole-tensor oracle functions they restrict.
"""
import numpy as np
import pytest

from oracle import dpo_oracle as O
from preference_alignment_amd.workloads import bf16_rne_bits


class _Mod:
    """Namespace copying the oracle, with some functions replaced."""

    def __init__(self, **overrides):
        for k in dir(O):
            if not k.startswith("__"):
                setattr(self, k, getattr(O, k))
        for k, v in overrides.items():
            setattr(self, k, v)


def _logits_case(seed, R=4, T=6, V=11, scale=1.5, grid=None):
    """Random logits [R,T,V] with a ragged completion mask (one hole, one row
    without completion positions when R > 2), targets, reference sums."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((R, T, V)) * scale
    if grid is not None:  # values on a grid of the given step, inside (-1, 1)
        z = np.clip(np.round(z / grid), -(1.0 / grid) + 1, (1.0 / grid) - 1) * grid
    mask = np.zeros((R, T), np.uint8)
    for r in range(R):
        mask[r, rng.integers(1, T // 2):] = 1
    mask[0, T - 2] = 0
    if R > 2:
        mask[R - 1, :] = 0
    targets = np.where(mask != 0, rng.integers(0, V, size=(R, T)), -100)
    ref = rng.standard_normal(R) * 2 - 10
    return z, targets, mask, ref


BETA = 0.7


def _loss_f64(z, targets, mask, ref):
    return O.dpo_loss(O.logits_seq_logps_f64(z, targets, mask)["logp_sum"], ref, BETA)["loss"]


def _weights_and_lse(fwd, ref):
    return O.dpo_loss(fwd["logp_sum"], ref, BETA)["weight"], fwd["lse"]


# ----------------------------------------------------------------------------
# finite differences
# ----------------------------------------------------------------------------
def check_dlogits_fd_f64(mod, seed=71):
    z, targets, mask, ref = _logits_case(seed)
    R, T, V = z.shape
    weight, lse = _weights_and_lse(O.logits_seq_logps_f64(z, targets, mask), ref)
    g = mod.logits_backward_rows_f64(z, targets, mask, lse, weight, np.arange(R * T)).reshape(R, T, V)
    h = 1e-6
    gmax = np.abs(g).max()
    assert gmax > 1e-3
    for r in range(R):
        for t in range(T):
            for v in range(V):
                zp, zm = z.copy(), z.copy()
                zp[r, t, v] += h
                zm[r, t, v] -= h
                fd = (_loss_f64(zp, targets, mask, ref) - _loss_f64(zm, targets, mask, ref)) / (2 * h)
                assert abs(fd - g[r, t, v]) <= 1e-9 + 1e-6 * abs(fd), (r, t, v, fd, g[r, t, v])


def test_dlogits_f64_finite_differences():
    check_dlogits_fd_f64(O)


def _bits(values):
    b = bf16_rne_bits(np.asarray(values, dtype=np.float32))
    assert np.array_equal(O.bf16_to_f64(b), np.asarray(values, dtype=np.float64)), "not a bf16 value"
    return b


def check_dlogits_fd_bf16(mod, seed=72):
    """Element-wise derivative of the loss over bf16 logits: the logits sit on
    the 2^-7 grid inside (-1, 1), so z +- 2^-6 and z +- 2^-5 are bf16 values
    (exact perturbations), and the two central differences are combined by
    Richardson extrapolation (error of order h^4)."""
    z, targets, mask, ref = _logits_case(seed, grid=2.0 ** -7, scale=0.5)
    R, T, V = z.shape
    bits = _bits(z)
    fwd = O.logits_seq_logps(bits, targets, mask)
    weight, lse = _weights_and_lse(fwd, ref)
    g = mod.logits_backward_rows(bits, targets, mask, lse, weight, np.arange(R * T)).reshape(R, T, V)
    assert np.abs(g).max() > 1e-3

    def loss_at(r, t, v, dz):
        zz = z.copy()
        zz[r, t, v] += dz
        return O.dpo_loss(O.logits_seq_logps(_bits(zz), targets, mask)["logp_sum"], ref, BETA)["loss"]

    h = 2.0 ** -6
    for r in range(R):
        for t in range(T):
            if mask[r, t] == 0:
                # the loss does not depend on logits outside the mask
                assert np.all(g[r, t] == 0)
                assert loss_at(r, t, 0, h) == loss_at(r, t, 0, -h)
                continue
            for v in range(V):
                d1 = (loss_at(r, t, v, h) - loss_at(r, t, v, -h)) / (2 * h)
                d2 = (loss_at(r, t, v, 2 * h) - loss_at(r, t, v, -2 * h)) / (4 * h)
                fd = (4 * d1 - d2) / 3
                assert abs(fd - g[r, t, v]) <= 2e-7 + 1e-4 * abs(fd), (r, t, v, fd, g[r, t, v])


def test_dlogits_bf16_finite_differences():
    check_dlogits_fd_bf16(O)


def check_dlogits_fd_f32(mod, seed=73):
    """Over fp32 logits on the 2^-16 grid, z +- 2^-12 are fp32 values."""
    z, targets, mask, ref = _logits_case(seed, grid=2.0 ** -16, scale=0.5)
    z32 = z.astype(np.float32)
    assert np.array_equal(z32.astype(np.float64), z)
    R, T, V = z.shape
    fwd = O.logits_f32_seq_logps(z32, targets, mask)
    weight, lse = _weights_and_lse(fwd, ref)
    g = mod.logits_f32_backward_rows(z32, targets, mask, lse, weight, np.arange(R * T)).reshape(R, T, V)
    h = np.float32(2.0 ** -12)
    for r in range(R):
        for t in range(T):
            for v in range(V):
                zp, zm = z32.copy(), z32.copy()
                zp[r, t, v] += h
                zm[r, t, v] -= h
                assert float(zp[r, t, v]) - float(zm[r, t, v]) == 2 * float(h)
                lp = O.dpo_loss(O.logits_f32_seq_logps(zp, targets, mask)["logp_sum"], ref, BETA)["loss"]
                lm = O.dpo_loss(O.logits_f32_seq_logps(zm, targets, mask)["logp_sum"], ref, BETA)["loss"]
                fd = (lp - lm) / (2 * float(h))
                assert abs(fd - g[r, t, v]) <= 1e-8 + 1e-5 * abs(fd), (r, t, v, fd, g[r, t, v])


def test_dlogits_f32_finite_differences():
    check_dlogits_fd_f32(O)


# ----------------------------------------------------------------------------
# agreement with the head path when the logits are Hc W^T
# ----------------------------------------------------------------------------
def check_dlogits_match_head_path(mod, seed=74, layout=O.PAIRS_ADJACENT):
    rng = np.random.default_rng(seed)
    R, T, H, V = 6, 9, 12, 23
    hidden = rng.standard_normal((R, T, H))
    w = rng.standard_normal((V, H)) * 0.4
    mask = np.zeros((R, T), np.uint8)
    for r in range(R):
        mask[r, rng.integers(1, 5):] = 1
    mask[2, 6] = 0
    targets = np.where(mask != 0, rng.integers(0, V, size=(R, T)), -100)
    ref = rng.standard_normal(R) - 30
    fwd = O.seq_logps_f64(hidden, w, targets, mask)
    loss = O.dpo_loss(fwd["logp_sum"], ref, 0.3, layout)
    dH, dW = O.head_backward_f64(hidden, w, targets, mask, fwd["lse"], loss["weight"])
    logits = hidden @ w.T
    rows = mod.logits_backward_rows_f64(logits, targets, mask, fwd["lse"], loss["weight"], np.arange(R * T))
    np.testing.assert_allclose(rows @ w, dH.reshape(R * T, H), rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(rows.T @ hidden.reshape(R * T, H), dW, rtol=1e-11, atol=1e-15)
    # and the scores over those logits are the head path's
    np.testing.assert_allclose(O.logits_seq_logps_f64(logits, targets, mask)["logp_sum"], fwd["logp_sum"],
                               rtol=1e-13)


@pytest.mark.parametrize("layout", [O.PAIRS_ADJACENT, O.PAIRS_HALVES])
def test_dlogits_match_head_path(layout):
    check_dlogits_match_head_path(O, layout=layout)


def test_dlogits_wrappers_decode_then_match_f64():
    """The bf16 and fp32 entry points are the float64 gradient of the decoded values."""
    z, targets, mask, ref = _logits_case(75, V=40, scale=3.0)
    R, T, V = z.shape
    bits = bf16_rne_bits(z.astype(np.float32))
    zb = O.bf16_to_f64(bits)
    fwd = O.logits_seq_logps_f64(zb, targets, mask)
    weight, lse = _weights_and_lse(fwd, ref)
    pos = np.array([0, 3, 5, 7, 11, R * T - 1])
    np.testing.assert_array_equal(O.logits_backward_rows(bits, targets, mask, lse, weight, pos),
                                  O.logits_backward_rows_f64(zb, targets, mask, lse, weight, pos))
    z32 = z.astype(np.float32)
    np.testing.assert_array_equal(O.logits_f32_backward_rows(z32, targets, mask, lse, weight, pos),
                                  O.logits_backward_rows_f64(z32.astype(np.float64), targets, mask, lse, weight,
                                                             pos))


# ----------------------------------------------------------------------------
# planted mistakes in the gradient over given logits
# ----------------------------------------------------------------------------
def _planted(kind):
    def f(logits, targets, mask, lse, weight, flat_positions):
        R, T, V = logits.shape
        w = np.asarray(weight, dtype=np.float64)
        tg = np.asarray(targets).copy()
        if kind == "wrong_row":
            w = np.roll(w, 1)
        elif kind == "no_weight":
            w = np.where(w != 0, 1.0, 0.0)
        elif kind == "double_weight":
            w = 2 * w
        elif kind == "onehot_shift":
            tg = np.where(np.asarray(mask) != 0, (tg + 1) % V, tg)
        if kind == "no_shift":
            out = O.logits_backward_rows_f64(logits, targets, mask, np.zeros_like(lse), w, flat_positions)
            return out
        return O.logits_backward_rows_f64(logits, tg, mask, lse, w, flat_positions)
    return f


def _planted_bits(kind):
    g = _planted(kind)

    def f(logits_bits, targets, mask, lse, weight, flat_positions):
        return g(O.bf16_to_f64(logits_bits), targets, mask, lse, weight, flat_positions)
    return f


def _planted_f32(kind):
    g = _planted(kind)

    def f(logits_f32, targets, mask, lse, weight, flat_positions):
        return g(np.asarray(logits_f32, np.float64), targets, mask, lse, weight, flat_positions)
    return f


KINDS = ["wrong_row", "no_weight", "double_weight", "onehot_shift", "no_shift"]


@pytest.mark.parametrize("kind", KINDS)
def test_planted_dlogits_mistake_fails_finite_differences(kind):
    with pytest.raises(AssertionError):
        check_dlogits_fd_f64(_Mod(logits_backward_rows_f64=_planted(kind)))


@pytest.mark.parametrize("kind", KINDS)
def test_planted_dlogits_mistake_fails_head_path(kind):
    with pytest.raises(AssertionError):
        check_dlogits_match_head_path(_Mod(logits_backward_rows_f64=_planted(kind)))


@pytest.mark.parametrize("kind", ["wrong_row", "onehot_shift", "double_weight"])
def test_planted_dlogits_mistake_fails_bf16_and_f32_pins(kind):
    with pytest.raises(AssertionError):
        check_dlogits_fd_bf16(_Mod(logits_backward_rows=_planted_bits(kind)))
    with pytest.raises(AssertionError):
        check_dlogits_fd_f32(_Mod(logits_f32_backward_rows=_planted_f32(kind)))


# ----------------------------------------------------------------------------
# sampled-output helpers against the whole-tensor oracle
# ----------------------------------------------------------------------------
def _head_case(seed=81, R=4, T=20, H=16, V=40):
    rng = np.random.default_rng(seed)
    hidden = rng.standard_normal((R, T, H))
    w = rng.standard_normal((V, H)) * 0.5
    mask = np.zeros((R, T), np.uint8)
    for r in range(R):
        mask[r, rng.integers(1, T // 2):] = 1
    mask[1, 15] = 0
    targets = np.where(mask != 0, rng.integers(0, V, size=(R, T)), -100)
    targets[0, T - 1] = V - 1
    targets[2, T - 1] = 0
    ref = rng.standard_normal(R) - 20
    fwd = O.seq_logps_f64(hidden, w, targets, mask)
    weight = O.dpo_loss(fwd["logp_sum"], ref, 0.2)["weight"]
    return hidden, w, targets, mask, fwd["lse"], weight


def check_sampled_gradients(mod):
    hidden, w, targets, mask, lse, weight = _head_case()
    R, T, H = hidden.shape
    V = w.shape[0]
    dH, dW = O.head_backward_f64(hidden, w, targets, mask, lse, weight)
    pos = np.array([0, 5, 19, 23, 35, 39, 41, 79])
    np.testing.assert_allclose(mod.dhidden_rows_f64(hidden, w, targets, mask, lse, weight, pos),
                               dH.reshape(R * T, H)[pos], rtol=1e-12, atol=1e-17)
    vs = np.array([0, 1, 7, 30, V - 1])
    np.testing.assert_allclose(mod.dw_rows_f64(hidden, w, targets, mask, lse, weight, vs, chunk=7), dW[vs],
                               rtol=1e-11, atol=1e-16)
    # a shard [a, b): its dHidden term and its dW rows
    a, b = 8, 27
    sH, sW = O.head_backward_shard_f64(hidden, w[a:b], targets, mask, lse, weight, a, V)
    np.testing.assert_allclose(mod.dhidden_rows_f64(hidden, w[a:b], targets, mask, lse, weight, pos, a, V),
                               sH.reshape(R * T, H)[pos], rtol=1e-12, atol=1e-17)
    np.testing.assert_allclose(mod.dw_rows_f64(hidden, w[a:b], targets, mask, lse, weight, [0, 5, b - a - 1], a, V),
                               sW[[0, 5, b - a - 1]], rtol=1e-11, atol=1e-16)
    # shard partials at positions
    full = O.shard_partials_f64(hidden, w[a:b], targets, mask, a, V)
    rows = mod.shard_partials_rows_f64(hidden, w[a:b], targets, mask, a, V, pos)
    for k in ("max", "sumexp", "tgt"):
        np.testing.assert_array_equal(rows[k], full[k].reshape(-1)[pos])


def test_sampled_gradients_match_whole_tensors():
    check_sampled_gradients(O)


def _dw_no_onehot_impl(hidden, w, targets, mask, lse, weight, vocab_rows, v_begin=0, V_total=None, chunk=4096):
    """dW rows with the one-hot term dropped."""
    R, T, H = hidden.shape
    idx, _ = O.completion_positions(mask)
    Z = hidden.reshape(R * T, H)[idx] @ w[vocab_rows].T
    P = np.exp(Z - np.asarray(lse).reshape(-1)[idx][:, None])
    return (np.asarray(weight)[idx // T][:, None] * P).T @ hidden.reshape(R * T, H)[idx]


def _dh_rows_wrong_lse(hidden, w, targets, mask, lse, weight, flat_positions, v_begin=0, V_total=None):
    return O.dhidden_rows_f64(hidden, w, targets, mask, np.asarray(lse) + 0.01, weight, flat_positions, v_begin,
                              V_total)


def test_planted_sampled_mistakes():
    with pytest.raises(AssertionError):
        check_sampled_gradients(_Mod(dw_rows_f64=_dw_no_onehot_impl))
    with pytest.raises(AssertionError):
        check_sampled_gradients(_Mod(dhidden_rows_f64=_dh_rows_wrong_lse))


def test_logit_sums_by_column_sum_and_abs_sums():
    hidden, w, targets, mask, lse, weight = _head_case(seed=82)
    R, T, H = hidden.shape
    want = O.logit_row_sums_f64(hidden, w, mask)
    got = O.logit_row_sums_by_column_sum(hidden, w, mask, chunk=7)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    pos = np.array([3, 17, 44])
    brute = [sum(abs(float(np.dot(w[v], hidden.reshape(R * T, H)[p]))) for v in range(w.shape[0])) for p in pos]
    np.testing.assert_allclose(O.logit_abs_sums_f64(hidden, w, pos), brute, rtol=1e-12)


def test_minus_inf_logits_equal_removed_columns():
    """Logits masked to -inf by a caller drop out of the log-sum-exp: the scores
    and the gradient over the remaining columns equal those of the logits with
    the masked columns removed (and the gradient there is exactly 0)."""
    z, targets, mask, ref = _logits_case(76, V=30)
    R, T, V = z.shape
    keep = np.ones(V, bool)
    keep[:8] = False
    keep[25:] = False
    zi = z.copy()
    zi[:, :, ~keep] = -np.inf
    # targets on kept columns, renumbered for the reduced array
    kept = np.flatnonzero(keep)
    rng = np.random.default_rng(77)
    tk = rng.integers(0, kept.size, size=targets.shape)
    t_full = np.where(mask != 0, kept[tk], -100)
    t_red = np.where(mask != 0, tk, -100)
    a = O.logits_seq_logps_f64(zi, t_full, mask)
    b = O.logits_seq_logps_f64(z[:, :, keep], t_red, mask)
    np.testing.assert_allclose(a["logp_sum"], b["logp_sum"], rtol=1e-14)
    weight = O.dpo_loss(a["logp_sum"], ref, BETA)["weight"]
    ga = O.logits_backward_rows_f64(zi, t_full, mask, a["lse"], weight, np.arange(R * T))
    gb = O.logits_backward_rows_f64(z[:, :, keep], t_red, mask, b["lse"], weight, np.arange(R * T))
    assert np.all(ga[:, ~keep] == 0)
    np.testing.assert_allclose(ga[:, keep], gb, rtol=1e-13, atol=1e-18)
    # the bf16 entry point decodes -inf (0xFF80) to -inf
    bits = bf16_rne_bits(z.astype(np.float32))
    bits[:, :, ~keep] = 0xFF80
    c = O.logits_seq_logps(bits, t_full, mask)
    assert np.all(np.isfinite(c["logp_sum"]))
