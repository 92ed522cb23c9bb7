"""The seeded input generators: shapes, mask structure, determinism, encodings."""
import numpy as np

from preference_alignment_amd import workloads as W


def test_workload1_recipe():
    a = W.make_workload(1)
    b = W.make_workload(1)
    assert a.hidden.shape == (4, 64, 256) and a.w_vocab.shape == (1024, 256)
    assert a.hidden.dtype == np.uint16 and a.targets.dtype == np.int32 and a.mask.dtype == np.uint8
    np.testing.assert_array_equal(a.hidden, b.hidden)
    np.testing.assert_array_equal(a.w_vocab, b.w_vocab)
    assert a.n_completion == W.expected_n_completion(1) == 192
    assert np.all(a.mask[:, :16] == 0) and np.all(a.mask[:, 16:] == 1)
    assert np.all(a.targets[a.mask == 0] == W.IGNORE_INDEX)
    t = a.targets[a.mask != 0]
    assert t.min() >= 0 and t.max() < 1024
    h = W.bf16_bits_to_f32(a.hidden)
    assert 0.9 < h.std() < 1.1
    assert 0.018 < W.bf16_bits_to_f32(a.w_vocab).std() < 0.022


def test_head_generator_structure_small():
    x = W.make_head_inputs(name="t", seed=7, rows=6, T=300, H=64, V=777, prompt_lo=20, prompt_hi=90,
                           comp_mode="independent", rms_normalise=True, targets_dist="zipf")
    for i in range(3):
        rc, rr = x.mask[2 * i], x.mask[2 * i + 1]
        pc, pr = int(np.argmax(rc)), int(np.argmax(rr))
        assert pc == pr and 20 <= pc <= 90          # the pair shares its prompt
        lc, lr = int(rc.sum()), int(rr.sum())
        assert max(lc, lr) <= 2 * min(lc, lr)       # ratio bound
        # contiguous completion span then tail padding
        assert np.all(rc[pc:pc + lc] == 1) and rc.sum() == lc
    h = W.bf16_bits_to_f32(x.hidden).reshape(-1, 64).astype(np.float64)
    rms = np.sqrt((h * h).mean(1))
    assert np.all(np.abs(rms - 1) < 0.01)            # RMS-normalised, then rounded to bf16


def test_halves_layout_pairs_share_prompt():
    x = W.make_head_inputs(name="t", seed=8, rows=8, T=64, H=8, V=16, prompt_lo=5, prompt_hi=30,
                           layout=W.PAIRS_HALVES)
    for i in range(4):
        assert np.argmax(x.mask[i]) == np.argmax(x.mask[4 + i])


def test_zipf_ids_distribution():
    rng = np.random.default_rng(0)
    ids = W.zipf_ids(rng, 200000, 128256)
    assert ids.min() >= 0 and ids.max() < 128256
    c = np.bincount(ids, minlength=4)
    # P(k) ~ k^-1.1: ratio of the first two ranks is 2^1.1
    assert abs(c[0] / c[1] - 2 ** 1.1) < 0.1


def test_logits_generator_small():
    x = W.make_logits_inputs(name="t", seed=5, rows=4, T=40, V=300, comp_start=10)
    assert x.logits.shape == (4, 40, 300)
    assert x.n_completion == 4 * 30
    assert 2.8 < W.bf16_bits_to_f32(x.logits).std() < 3.2


def test_bf16_encoder_round_to_nearest_even():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    bits = W.bf16_rne_bits(vals)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]
