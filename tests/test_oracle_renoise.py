"""Re-noise and its counter-based RNG, pinned to numpy's Philox and to the
invariants of uniform-state diffusion (explainer "DiffusionGemma", section
"Uniform State Diffusion": low-confidence slots get a fresh uniformly random
vocabulary token, the others keep the model's prediction)."""
import numpy as np
import pytest

import oracle


def _numpy_philox_block(ctr, key):
    """numpy.random.Philox is Philox4x64-10; it increments its counter before
    producing a block, so start it one below the block wanted."""
    c = np.array(ctr, dtype=np.uint64)
    c0 = c.copy()
    c0[0] = c[0] - np.uint64(1)   # tests keep ctr[0] >= 1 (no borrow)
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=c0)
    return g.random_raw(4).astype(np.uint64)


def test_philox_matches_numpy():
    rng = np.random.default_rng(5)
    for _ in range(200):
        ctr = rng.integers(0, 2**63, 4, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
        key = rng.integers(0, 2**63, 2, dtype=np.uint64) * np.uint64(2)
        np.testing.assert_array_equal(oracle.philox4x64_10(ctr, key), _numpy_philox_block(ctr, key))
    for ctr, key in [([1, 0, 0, 0], [0, 0]), ([2**64 - 1] * 4, [2**64 - 1] * 2),
                     ([5, 7, 3, 0], [1, 0])]:
        np.testing.assert_array_equal(oracle.philox4x64_10(np.array(ctr, np.uint64), np.array(key, np.uint64)),
                                      _numpy_philox_block(ctr, key))


@pytest.mark.parametrize("V", [1024, 32768, 1 << 20])
def test_noise_token_is_top_bits_of_philox_word0(V):
    """With V = 2^m, floor(r0 * V / 2^64) is the top m bits of word 0 of the
    block for counter (pos, pass_tag, request, 0) and key (seed, 0)."""
    B, N, seed, tag = 3, 40, 123456789, 7
    pos0 = np.array([5, 1000, 77], np.int32)
    req = np.array([4, 9, 2], np.uint32)
    out = oracle.renoise(np.zeros((B, N), np.int32), None, None, 0.5, seed, tag, pos0, V, req_id=req)
    m = V.bit_length() - 1
    for b in range(B):
        for i in range(N):
            r0 = _numpy_philox_block([pos0[b] + i, tag, req[b], 0], [seed, 0])[0]
            assert out[b, i] == int(r0) >> (64 - m)


def test_default_request_id_is_batch_index():
    pos0 = np.array([3, 3], np.int32)
    a = oracle.renoise(np.zeros((2, 8), np.int32), None, None, 0.5, 1, 0, pos0, 1000)
    b = oracle.renoise(np.zeros((2, 8), np.int32), None, None, 0.5, 1, 0, pos0, 1000,
                       req_id=np.array([0, 1], np.uint32))
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a[0], a[1])


def test_noise_tokens_uniform_chi2():
    V, N = 64, 64 * 400
    out = oracle.renoise(np.zeros((1, N), np.int32), None, None, 0.5, 99, 3, np.array([0], np.int32), V)
    counts = np.bincount(out.ravel(), minlength=V)
    exp = N / V
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    # 63 degrees of freedom: mean 63, sd ~11.2; 130 is beyond 6 sd
    assert chi2 < 130, chi2
    assert out.min() >= 0 and out.max() < V


def test_non_power_of_two_vocab_in_range_and_spread():
    V = 1000
    out = oracle.renoise(np.zeros((1, 20000), np.int32), None, None, 0.5, 5, 1, np.array([0], np.int32), V)
    assert out.min() >= 0 and out.max() < V
    assert len(np.unique(out)) > 990


def test_keys_change_the_stream():
    base = dict(canvas=np.zeros((1, 64), np.int32), argmax=None, conf=None, tau=0.5, V=1 << 15)
    a = oracle.renoise(seed=1, pass_tag=1, pos0=np.array([0], np.int32), **base)
    for kw in (dict(seed=2, pass_tag=1, pos0=np.array([0], np.int32)),
               dict(seed=1, pass_tag=2, pos0=np.array([0], np.int32)),
               dict(seed=1, pass_tag=1, pos0=np.array([1], np.int32))):
        b = oracle.renoise(**base, **kw)
        assert (a != b).mean() > 0.9
    # shifting pos0 by one shifts the stream by one slot
    b = oracle.renoise(seed=1, pass_tag=1, pos0=np.array([1], np.int32), **base)
    np.testing.assert_array_equal(a[0, 1:], b[0, :-1])


def test_threshold_invariants():
    rng = np.random.default_rng(3)
    B, N, V = 4, 50, 4096
    canvas = rng.integers(0, V, (B, N)).astype(np.int32)
    am = rng.integers(0, V, (B, N)).astype(np.int32)
    conf = rng.random((B, N)).astype(np.float32)
    conf[0, :5] = [0.5, np.nextafter(np.float32(0.5), np.float32(0)), np.nan, 1.0, 0.0]
    pos0 = np.array([10, 20, 30, 40], np.int32)
    tau = 0.5
    out = oracle.renoise(canvas, am, conf, tau, 11, 4, pos0, V)
    noise = oracle.renoise(canvas, None, None, tau, 11, 4, pos0, V)
    keep = conf >= tau
    np.testing.assert_array_equal(out[keep], am[keep])          # confident slots keep argmax
    np.testing.assert_array_equal(out[~keep], noise[~keep])     # the rest: the RNG token
    assert keep[0, 0] and not keep[0, 1] and not keep[0, 2]     # boundary and NaN
    # tau = 0 keeps every prediction; tau > 1 noises every slot
    np.testing.assert_array_equal(oracle.renoise(canvas, am, conf, 0.0, 11, 4, pos0, V)[~np.isnan(conf)],
                                  am[~np.isnan(conf)])
    np.testing.assert_array_equal(oracle.renoise(canvas, am, conf, 1.5, 11, 4, pos0, V), noise)
    # the old canvas content never matters
    np.testing.assert_array_equal(oracle.renoise(canvas * 0, am, conf, tau, 11, 4, pos0, V), out)


# ---- masked ("absorbing") diffusion: explainer "DiffusionGemma", "First
# attempt: masked diffusion" -- a filled [MASK] slot locks in ----

def _masked_case(seed=3, B=3, N=50, V=100, mask_id=99):
    rng = np.random.default_rng(seed)
    canvas = rng.integers(0, V - 1, (B, N)).astype(np.int32)
    canvas[rng.random((B, N)) < 0.6] = mask_id
    argmax = rng.integers(0, V - 1, (B, N)).astype(np.int32)
    conf = rng.random((B, N)).astype(np.float32)
    return canvas, argmax, conf


def test_unmask_fills_confident_masked_slots_and_locks_the_rest():
    canvas, argmax, conf = _masked_case()
    out, ch, ml = oracle.unmask(canvas, argmax, conf, 0.5, 99)
    masked = canvas == 99
    fill = masked & (conf >= 0.5)
    np.testing.assert_array_equal(out[fill], argmax[fill])
    np.testing.assert_array_equal(out[~masked], canvas[~masked])        # filled slots never change
    assert (out[masked & ~fill] == 99).all()                            # the rest stay masked
    np.testing.assert_array_equal(ch, (out != canvas).sum(1))           # brute-force counts
    np.testing.assert_array_equal(ml, (out == 99).sum(1))


def test_unmask_special_thresholds_and_final_pass():
    canvas, argmax, conf = _masked_case(seed=4)
    masked = canvas == 99
    out, _, ml = oracle.unmask(canvas, argmax, conf, 0.0, 99)           # tau 0: every masked slot fills
    np.testing.assert_array_equal(out[masked], argmax[masked])
    assert (ml == 0).all()
    out, ch, _ = oracle.unmask(canvas, argmax, conf, 1.5, 99)           # tau > 1: none fills
    np.testing.assert_array_equal(out, canvas)
    assert (ch == 0).all()
    out, _, ml = oracle.unmask(canvas, argmax, conf, 1.5, 99, final_pass=True)
    np.testing.assert_array_equal(out[masked], argmax[masked])          # the last pass fills all
    np.testing.assert_array_equal(out[~masked], canvas[~masked])
    assert (ml == 0).all()
    # an argmax equal to the mask token keeps the slot masked (and unchanged)
    am2 = argmax.copy()
    am2[masked] = 99
    out, ch, ml = oracle.unmask(canvas, am2, conf, 0.0, 99)
    np.testing.assert_array_equal(out, canvas)
    assert (ch == 0).all() and (ml == masked.sum(1)).all()


def test_uniform_update_fixed_point():
    """Uniform-state re-noise has converged once every slot is confident and
    already holds its prediction: the update then changes nothing (explainer,
    "Uniform State Diffusion": after several passes the canvas converges)."""
    rng = np.random.default_rng(6)
    canvas = rng.integers(0, 1000, (2, 30)).astype(np.int32)
    conf = (0.6 + 0.4 * rng.random((2, 30))).astype(np.float32)
    out = oracle.renoise(canvas, canvas, conf, 0.6, 9, 3, np.array([0, 100], np.int32), 1000)
    np.testing.assert_array_equal(out, canvas)
    conf[1, 7] = 0.1                                                    # one unsure slot moves
    out = oracle.renoise(canvas, canvas, conf, 0.6, 9, 3, np.array([0, 100], np.int32), 1000)
    assert (out != canvas).sum() <= 1 and (out[0] == canvas[0]).all()
