"""Pins of the oracle's score-magnitude helpers (CPU only).

The GPU parity tests measure each log-sum-exp against the size of the dot products it is made of:
a score is a sum of products, and its rounding error scales with the sum of the magnitudes of its
terms, not with the score itself ("DeepSeek-V3.2-Exp · Attention update", mla-decode: scores are
the latent and rotary dot products times softmax_scale; "Kimi-K2 · value_states", mla-prefill:
the scaled query-key products under the causal mask). These helpers set that size, so a mistake in
them would silently widen every lse bar; the pins below fix them by a hand-computed case, by the
special case where no term is negative (the magnitude is then the largest score itself, which for
one key equals the lse the attention pins already fix), by their scaling and sign symmetries, and
by the causal range of the prefill form."""
import numpy as np
import pytest

from oracle import mla_oracle as O

SCALE = 192 ** -0.5


def _bits(a):
    return O.bf16_encode(np.asarray(a, np.float64))


def _identity_wkv(H):
    """wkv_b whose key half maps latent feature d to content feature d (d < 128) for every head;
    the value half is zero. q_lat is then q_nope in its first 128 features and 0 after."""
    w = np.zeros((H * 256, 512))
    for h in range(H):
        w[h * 256 + np.arange(128), np.arange(128)] = 1.0
    return _bits(w)


def test_decode_magnitude_hand_case():
    """One head, two cached rows, small integers; worked by hand:
      row 0: |1*3| + |-2*1| + |1*2| = 7   -> 0.5 * 7 = 3.5
      row 1: |1*-1| + |-2*-4| + |1*0| = 9 -> 0.5 * 9 = 4.5   (the scores are 0.5 and 3.5)"""
    q = np.zeros((1, 192))
    q[0, 0], q[0, 1], q[0, 128] = 1.0, -2.0, 1.0
    kv = np.zeros((2, 512))
    kv[0, :2] = [3.0, 1.0]
    kv[1, :2] = [-1.0, -4.0]
    pe = np.zeros((2, 64))
    pe[0, 0] = 2.0
    mag = O.decode_score_magnitude(q, _identity_wkv(1), _bits(kv), _bits(pe), 0.5)
    assert mag.shape == (1,)
    assert mag[0] == pytest.approx(4.5, abs=1e-12)


def test_decode_magnitude_is_the_score_when_no_term_is_negative():
    """With q, W_UK, the cached latent and the rotary key all nonnegative every term is
    nonnegative, so the magnitude is the largest score; with one cached row it is that row's score,
    which equals the decode's lse (the log of a single exponential)."""
    rng = np.random.default_rng(7)
    H = 3
    q = np.abs(rng.standard_normal((H, 192)))
    w = _bits(np.abs(rng.standard_normal((H * 256, 512))) / np.sqrt(512))
    kv = _bits(np.abs(rng.standard_normal((1, 512))))
    pe = _bits(np.abs(rng.standard_normal((1, 64))))
    mag = O.decode_score_magnitude(q, w, kv, pe, SCALE)
    _, lse = O.decode_absorbed(q, w, kv, pe, SCALE)
    np.testing.assert_allclose(mag, lse, rtol=1e-12)


def test_decode_magnitude_scaling_sign_and_zero_query():
    rng = np.random.default_rng(8)
    H, L = 4, 9
    q = rng.standard_normal((H, 192))
    w = _bits(rng.standard_normal((H * 256, 512)) / np.sqrt(512))
    kv = _bits(rng.standard_normal((L, 512)))
    pe = _bits(rng.standard_normal((L, 64)))
    m1 = O.decode_score_magnitude(q, w, kv, pe, SCALE)
    assert np.all(m1 > 0)
    # linear in the softmax scale
    np.testing.assert_allclose(O.decode_score_magnitude(q, w, kv, pe, 2 * SCALE), 2 * m1, rtol=1e-14)
    # sizes of terms: flipping the sign of the query or of the cached rows changes nothing
    np.testing.assert_allclose(O.decode_score_magnitude(-q, w, kv, pe, SCALE), m1, rtol=1e-14)
    neg_kv = _bits(-O.bf16_decode(kv))
    neg_pe = _bits(-O.bf16_decode(pe))
    np.testing.assert_allclose(O.decode_score_magnitude(q, w, neg_kv, neg_pe, SCALE), m1, rtol=1e-14)
    # at least the largest |score| (the triangle inequality), which the rotary part alone can reach
    s = np.abs(SCALE * (O.absorb_query(q, w) @ O.bf16_decode(kv).T + q[:, 128:] @ O.bf16_decode(pe).T))
    assert np.all(m1 >= s.max(axis=1) * (1 - 1e-14))
    # no query, no terms
    assert np.all(O.decode_score_magnitude(np.zeros_like(q), w, kv, pe, SCALE) == 0)


def test_prefill_magnitude_hand_case_and_causal_range():
    """One head, three positions; the identity key half makes k_nope the latent's first 128
    features. Key 0 gives 0.5 * (|2*1| + |1*1|) = 1.5, key 1 gives 0.5 * |2*1| = 1 and key 2 gives
    0.5 * |2*-3| = 3. Row 0 sees key 0 (1.5), row 1 keys 0 and 1 (1.5), row 2 all three (3)."""
    q = np.zeros((3, 1, 192))
    q[:, 0, 0] = 2.0
    q[:, 0, 128] = 1.0
    lat = np.zeros((3, 512))
    lat[0, 0], lat[1, 0], lat[2, 0] = 1.0, 1.0, -3.0
    kpe = np.zeros((3, 64))
    kpe[0, 0] = 1.0
    mag = O.prefill_score_magnitude(q, _bits(lat), _bits(kpe), _identity_wkv(1), 0.5)
    assert mag.shape == (1, 3)
    np.testing.assert_allclose(mag[0], [1.5, 1.5, 3.0], atol=1e-12)


def test_prefill_magnitude_is_the_score_when_no_term_is_negative():
    """Nonnegative terms: row 0 sees one key, so its magnitude is its score, which equals its lse."""
    rng = np.random.default_rng(9)
    T, H = 5, 2
    q = np.abs(rng.standard_normal((T, H, 192)))
    w = _bits(np.abs(rng.standard_normal((H * 256, 512))) / np.sqrt(512))
    lat = _bits(np.abs(rng.standard_normal((T, 512))))
    kpe = _bits(np.abs(rng.standard_normal((T, 64))))
    mag = O.prefill_score_magnitude(q, lat, kpe, w, SCALE, rows=[0])
    _, lse = O.prefill_causal(q, lat, kpe, w, SCALE, rows=[0])
    np.testing.assert_allclose(mag[:, 0], lse[:, 0], rtol=1e-12)


def test_prefill_magnitude_scaling_sign_future_rows_and_zero_query():
    rng = np.random.default_rng(11)
    T, H = 6, 2
    q = rng.standard_normal((T, H, 192))
    w = _bits(rng.standard_normal((H * 256, 512)) / np.sqrt(512))
    lat = _bits(rng.standard_normal((T, 512)))
    kpe = _bits(rng.standard_normal((T, 64)))
    m1 = O.prefill_score_magnitude(q, lat, kpe, w, SCALE)
    assert m1.shape == (H, T) and np.all(m1 > 0)
    np.testing.assert_allclose(O.prefill_score_magnitude(q, lat, kpe, w, 3 * SCALE), 3 * m1, rtol=1e-14)
    np.testing.assert_allclose(O.prefill_score_magnitude(-q, lat, kpe, w, SCALE), m1, rtol=1e-14)
    # a running maximum over the keys a row sees: never decreasing along the rows of one query
    # vector (up to the summation order of the product), and unchanged by keys after the row
    qc = np.repeat(q[:1], T, axis=0)
    mc = O.prefill_score_magnitude(qc, lat, kpe, w, SCALE)
    assert np.all(np.diff(mc, axis=1) >= -1e-12 * mc[:, 1:])
    lat2 = lat.copy()
    lat2[3:] = _bits(10 * rng.standard_normal((T - 3, 512)))
    m2 = O.prefill_score_magnitude(q, lat2, kpe, w, SCALE)
    np.testing.assert_array_equal(m2[:, :3], m1[:, :3])
    assert np.all(O.prefill_score_magnitude(np.zeros_like(q), lat, kpe, w, SCALE) == 0)
