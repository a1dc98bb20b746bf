"""Pins of the oracle's query path, absorbed decode, split combine and causal prefill (CPU only).

Nothing here compares the oracle with a retyped copy of itself: the pins are the pages' printed
parameter counts and shapes, algebraic identities between the two attention forms the pages show
(absorbed decode vs. expanded keys/values), special cases with closed-form answers, invariances,
and library routines (torch on the CPU in float64)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from synth import inputs as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = 192 ** -0.5


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(a):
    return O.bf16_encode(np.asarray(a, np.float64))


def _rand_bits(rng, shape, std=1.0):
    return _bits(rng.standard_normal(shape) * std)


# ------------------------------------------------------------------------------ weight shapes
def test_param_counts_match_pages():
    g = _golden("param_counts.json")
    qh = g["query_heads"]
    c = O.param_counts(qh["n_heads"], qh["q_lora_rank"])
    assert c["query_content"] == qh["query_content"] == 1536 * 16384
    assert c["query_rotary"] == qh["query_rotary"] == 1536 * 8192
    assert c["query_total"] == qh["per_instance"] == c["query_content"] + c["query_rotary"]
    assert c["query_total"] * qh["instances"] == qh["across_instances"]
    vs = g["value_states"]
    c = O.param_counts(vs["n_heads"])
    assert c["value_up"] == vs["value_up"]
    assert c["value_up"] * vs["instances"] == vs["across_instances"]
    assert c["key_up"] + c["value_up"] == c["kv_up_total"] == 64 * 256 * 512
    qn = g["query_rmsnorm_gain"]
    assert qn["per_instance"] == qn["width"]


def test_value_half_is_last_rows_of_each_head():
    """The decode excerpt slices wkv_b[:, :nope] as the key half and wkv_b[:, -v:] as the value
    half of each head's 256 rows: zeroing the last 128 rows of every head must zero the output,
    zeroing the first 128 must make the output independent of q_nope."""
    rng = np.random.default_rng(10)
    H, L = 3, 6
    w = rng.standard_normal((H, 256, 512)) / np.sqrt(512)
    kv, pe = _rand_bits(rng, (L, 512)), _rand_bits(rng, (L, 64))
    q = rng.standard_normal((H, 192))
    w_noval = w.copy()
    w_noval[:, 128:, :] = 0
    out, _ = O.decode_absorbed(q, _bits(w_noval.reshape(H * 256, 512)), kv, pe, SCALE, staged=False)
    assert np.all(out == 0)
    w_nokey = w.copy()
    w_nokey[:, :128, :] = 0
    wb = _bits(w_nokey.reshape(H * 256, 512))
    q2 = q.copy()
    q2[:, :128] = rng.standard_normal((H, 128))
    o1, l1 = O.decode_absorbed(q, wb, kv, pe, SCALE, staged=False)
    o2, l2 = O.decode_absorbed(q2, wb, kv, pe, SCALE, staged=False)
    np.testing.assert_allclose(o1, o2, rtol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


# ------------------------------------------------------------------------------ query path
def _query_inputs(rng, n, H):
    return (_rand_bits(rng, (n, 1536)), (1 + 0.1 * rng.standard_normal(1536)).astype(np.float32),
            _rand_bits(rng, (1536, H * 192), 1536 ** -0.5))


def test_query_path_shape_and_head_column_ownership():
    rng = np.random.default_rng(11)
    n, H = 3, 4
    x, g, w = _query_inputs(rng, n, H)
    cs = S.rope_table(np.array([5, 6, 7]))
    q, inv = O.query_path(x, g, w, cs, H, staged=False)
    assert q.shape == (n, H, 192) and inv.shape == (n,)
    # perturb one content column (head 2, feature 37) and one rotary column (head 1, feature 128+9)
    for h, j in [(2, 37), (1, 128 + 9)]:
        w2 = O.bf16_decode(w).copy()
        w2[:, h * 192 + j] += 0.25
        q2, _ = O.query_path(x, g, _bits(w2), cs, H, staged=False)
        changed = np.argwhere(np.any(np.abs(q2 - q) > 1e-9, axis=0))
        if j < 128:
            assert changed.tolist() == [[h, j]]
        else:
            pair = (j - 128) // 2
            assert changed.tolist() == [[h, 128 + 2 * pair], [h, 128 + 2 * pair + 1]]


def test_query_path_scale_invariance_and_position_zero():
    rng = np.random.default_rng(12)
    n, H = 4, 2
    x, g, w = _query_inputs(rng, n, H)
    cs0 = S.rope_table(np.zeros(n, np.int64))
    q, _ = O.query_path(x, g, w, cs0, H, eps=0.0, staged=False)
    x4 = _bits(O.bf16_decode(x) * 4.0)        # exact in bf16
    q4, _ = O.query_path(x4, g, w, cs0, H, eps=0.0, staged=False)
    np.testing.assert_allclose(q4, q, rtol=1e-12, atol=1e-14)
    # at position 0 the rotary part is the plain product
    y = O.bf16_decode(x) / np.sqrt(np.mean(O.bf16_decode(x) ** 2, axis=1, keepdims=True)) * g
    plain = (y @ O.bf16_decode(w)).reshape(n, H, 192)
    np.testing.assert_allclose(q, plain, rtol=1e-11, atol=1e-12)
    # at other positions the rotary pairs keep their norms and the content part is unchanged
    cs = S.rope_table(np.array([1, 99, 1000, 131072]))
    qp, _ = O.query_path(x, g, w, cs, H, eps=0.0, staged=False)
    np.testing.assert_allclose(qp[:, :, :128], plain[:, :, :128], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.hypot(qp[:, :, 128::2], qp[:, :, 129::2]),
                               np.hypot(plain[:, :, 128::2], plain[:, :, 129::2]), rtol=1e-6)


def test_query_path_matches_torch_complex_route():
    rng = np.random.default_rng(13)
    n, H = 5, 3
    x, g, w = _query_inputs(rng, n, H)
    pos = np.array([0, 1, 10, 1000, 4095])
    cs = S.rope_table(pos)
    q, inv = O.query_path(x, g, w, cs, H, staged=False)
    xt = torch.from_numpy(O.bf16_decode(x))
    y = torch.nn.functional.rms_norm(xt, (1536,), torch.from_numpy(g.astype(np.float64)), 1e-6)
    qt = (y @ torch.from_numpy(O.bf16_decode(w))).view(n, H, 192)
    pe = torch.view_as_complex(qt[..., 128:].reshape(n, H, 32, 2).contiguous())
    rot = torch.view_as_complex(torch.from_numpy(cs.astype(np.float64)).contiguous())[:, None, :]
    qt[..., 128:] = torch.view_as_real(pe * rot).reshape(n, H, 64)
    np.testing.assert_allclose(q, qt.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(inv, 1 / np.sqrt(np.mean(O.bf16_decode(x) ** 2, 1) + 1e-6), rtol=1e-13)


def test_query_path_staged_points_are_bf16_and_close_to_exact():
    rng = np.random.default_rng(14)
    x, g, w = _query_inputs(rng, 6, 2)
    cs = S.rope_table(np.arange(6) * 300)
    qs, _ = O.query_path(x, g, w, cs, 2, staged=True)
    qe, _ = O.query_path(x, g, w, cs, 2, staged=False)
    assert np.array_equal(O.bf16_round(qs), qs)
    assert np.max(np.abs(qs - qe)) <= 2e-2 * np.sqrt(np.mean(qe ** 2))
    # before the last rounding: the content features are the exact Linear output (the RMSNorm
    # output rounded first), so they round to the staged values; the rotary features round to them
    # too, and differ from the exact path's only through the rounding of the Linear output
    qu, _ = O.query_path(x, g, w, cs, 2, staged=True, round_output=False)
    assert np.array_equal(O.bf16_round(qu), qs)
    assert not np.array_equal(qu[:, :, :128], qs[:, :, :128])
    lin = (O.bf16_round(O.rms_norm(O.bf16_decode(x), g)[0]) @ O.bf16_decode(w)).reshape(6, 2, 192)
    np.testing.assert_allclose(qu[:, :, :128], lin[:, :, :128], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------------ decode
@pytest.mark.parametrize("H,L", [(1, 1), (2, 3), (2, 7), (4, 5), (128, 3)])
def test_absorbed_equals_expanded(H, L):
    rng = np.random.default_rng(100 + H * 10 + L)
    w = _rand_bits(rng, (H * 256, 512), 512 ** -0.5)
    kv, pe = _rand_bits(rng, (L, 512)), _rand_bits(rng, (L, 64))
    q = O.bf16_round(rng.standard_normal((H, 192)))
    oa, la = O.decode_absorbed(q, w, kv, pe, SCALE, staged=False)
    oe, le = O.decode_expanded(q, w, kv, pe, SCALE)
    np.testing.assert_allclose(oa, oe, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(la, le, rtol=1e-12)


def test_decode_matches_torch_sdpa():
    rng = np.random.default_rng(21)
    H, L = 4, 37
    w = _rand_bits(rng, (H * 256, 512), 512 ** -0.5)
    kv, pe = _rand_bits(rng, (L, 512)), _rand_bits(rng, (L, 64))
    q = O.bf16_round(rng.standard_normal((H, 192)))
    out, lse = O.decode_absorbed(q, w, kv, pe, SCALE, staged=False)
    wv = torch.from_numpy(O.bf16_decode(w)).view(H, 256, 512)
    c = torch.from_numpy(O.bf16_decode(kv))
    k = torch.cat([torch.einsum("tc,hdc->htd", c, wv[:, :128]),
                   torch.from_numpy(O.bf16_decode(pe))[None].expand(H, L, 64)], dim=-1)
    v = torch.einsum("tc,hdc->htd", c, wv[:, 128:])
    qt = torch.from_numpy(q)[:, None, :]
    want = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=SCALE)[:, 0]
    np.testing.assert_allclose(out, want.numpy(), rtol=1e-10, atol=1e-12)
    want_lse = torch.logsumexp(SCALE * (qt @ k.transpose(1, 2))[:, 0], dim=-1)
    np.testing.assert_allclose(lse, want_lse.numpy(), rtol=1e-12)


def test_decode_special_cases():
    rng = np.random.default_rng(22)
    H = 3
    w = _rand_bits(rng, (H * 256, 512), 512 ** -0.5)
    _, uv = O.wkv_b_heads(O.bf16_decode(w), H)
    kv, pe = _rand_bits(rng, (9, 512)), _rand_bits(rng, (9, 64))
    q = O.bf16_round(rng.standard_normal((H, 192)))
    # one cached row: out = W_UV c_0 for any query, lse = its scaled score
    o1, l1 = O.decode_absorbed(q, w, kv[:1], pe[:1], SCALE, staged=False)
    np.testing.assert_allclose(o1, uv @ O.bf16_decode(kv[0]), rtol=1e-12)
    # all rows equal: independent of q; lse = s + ln L
    same_kv, same_pe = np.repeat(kv[:1], 9, 0), np.repeat(pe[:1], 9, 0)
    oa, la = O.decode_absorbed(q, w, same_kv, same_pe, SCALE, staged=False)
    np.testing.assert_allclose(oa, o1, rtol=1e-12)
    np.testing.assert_allclose(la, l1 + np.log(9), rtol=1e-12)
    # zero query: uniform weights, out = W_UV mean_t c_t, lse = ln L
    oz, lz = O.decode_absorbed(np.zeros((H, 192)), w, kv, pe, SCALE, staged=False)
    np.testing.assert_allclose(oz, uv @ O.bf16_decode(kv).mean(0), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lz, np.log(9), rtol=1e-13)
    # zero rows
    o0, l0 = O.decode_batch(q[None], w, kv, pe, np.array([0]), np.array([0]), SCALE)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


def test_decode_invariances():
    rng = np.random.default_rng(23)
    H, L = 2, 11
    w = _rand_bits(rng, (H * 256, 512), 512 ** -0.5)
    kv, pe = _rand_bits(rng, (L, 512)), _rand_bits(rng, (L, 64))
    q = O.bf16_round(rng.standard_normal((H, 192)))
    o, l = O.decode_absorbed(q, w, kv, pe, SCALE, staged=False)
    perm = rng.permutation(L)
    op, lp = O.decode_absorbed(q, w, kv[perm], pe[perm], SCALE, staged=False)
    np.testing.assert_allclose(op, o, rtol=1e-11)
    np.testing.assert_allclose(lp, l, rtol=1e-13)
    # a vector added to every rotary key shifts every score of a head equally: out unchanged,
    # lse shifted by scale * q_pe . v
    v = np.round(rng.standard_normal(64) * 4) / 4
    pe_shift = _bits(O.bf16_decode(pe) + v)
    exact = np.array_equal(O.bf16_decode(pe_shift), O.bf16_decode(pe) + v)
    os_, ls = O.decode_absorbed(q, w, kv, pe_shift, SCALE, staged=False)
    if exact:
        np.testing.assert_allclose(os_, o, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(ls, l + SCALE * q[:, 128:] @ v, rtol=1e-11)


@pytest.mark.parametrize("cuts", [[5], [0, 0, 7], [3, 3, 3, 20], [1, 2, 4, 8, 16], [30, 30]])
def test_split_partition_invariance(cuts):
    rng = np.random.default_rng(24)
    H, L = 3, 30
    w = _rand_bits(rng, (H * 256, 512), 512 ** -0.5)
    kv, pe = _rand_bits(rng, (L, 512)), _rand_bits(rng, (L, 64))
    q = O.bf16_round(rng.standard_normal((H, 192)))
    o, l = O.decode_absorbed(q, w, kv, pe, SCALE, staged=False)
    os_, ls = O.decode_absorbed(q, w, kv, pe, SCALE, staged=False, segments=cuts)
    np.testing.assert_allclose(os_, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ls, l, rtol=1e-13)


def test_combine_all_empty():
    H = 2
    o, l = O.combine_segments([(np.zeros((H, 512)), np.full(H, -np.inf))] * 3)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_decode_staged_close_to_exact_with_spikes():
    """Config-4-like data (some rows scaled by 8): staged within the parity tolerance of exact."""
    case = S.DecodeCase("t", 900, 4, np.array([700]), spike_frac=0.01)
    d = S.decode_inputs(case, seed=3, workers=1)
    q, _ = O.query_path(d["q_latent"], d["gamma"], d["wq_b"], d["rope_cs"], 4)
    os_, ls = O.decode_batch(q, d["wkv_b"], d["kv_cache"], d["pe_cache"], d["row_offset"], d["lengths"],
                             SCALE, staged=True)
    oe, le = O.decode_batch(q, d["wkv_b"], d["kv_cache"], d["pe_cache"], d["row_offset"], d["lengths"],
                            SCALE, staged=False)
    assert np.max(np.abs(os_ - oe)) <= 2e-2 * np.sqrt(np.mean(oe ** 2))
    # rounding q_lat to bf16 moves each score by ~2^-9 of its terms: lse shifts by ~0.1% here
    np.testing.assert_allclose(ls, le, rtol=5e-3)


# ------------------------------------------------------------------------------ prefill
def _prefill_small(rng, T, H):
    q = O.bf16_round(rng.standard_normal((T, H, 192)))
    lat = _rand_bits(rng, (T, 512))
    kpe = _rand_bits(rng, (T, 64))
    w = _rand_bits(rng, (H * 256, 512), 512 ** -0.5)
    return q, lat, kpe, w


def test_prefill_row_equals_decode_over_prefix():
    rng = np.random.default_rng(30)
    T, H = 9, 3
    q, lat, kpe, w = _prefill_small(rng, T, H)
    out, lse = O.prefill_causal(q, lat, kpe, w, SCALE, staged=False)
    assert out.shape == (T, H, 128) and lse.shape == (H, T)
    for t in range(T):
        od, ld = O.decode_absorbed(q[t], w, lat[: t + 1], kpe[: t + 1], SCALE, staged=False)
        np.testing.assert_allclose(out[t], od, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[:, t], ld, rtol=1e-12)


def test_prefill_first_row_future_rows_and_sdpa():
    rng = np.random.default_rng(31)
    T, H = 12, 2
    q, lat, kpe, w = _prefill_small(rng, T, H)
    out, lse = O.prefill_causal(q, lat, kpe, w, SCALE, staged=False)
    _, uv = O.wkv_b_heads(O.bf16_decode(w), H)
    np.testing.assert_allclose(out[0], uv @ O.bf16_decode(lat[0]), rtol=1e-12)
    # rows after t do not change row t
    lat2, kpe2 = lat.copy(), kpe.copy()
    lat2[6:] = _rand_bits(rng, (T - 6, 512))
    kpe2[6:] = _rand_bits(rng, (T - 6, 64))
    out2, _ = O.prefill_causal(q, lat2, kpe2, w, SCALE, staged=False)
    np.testing.assert_array_equal(out2[:6], out[:6])
    # library: causal SDPA over explicitly expanded keys and values
    wv = torch.from_numpy(O.bf16_decode(w)).view(H, 256, 512)
    c = torch.from_numpy(O.bf16_decode(lat))
    k = torch.cat([torch.einsum("tc,hdc->htd", c, wv[:, :128]),
                   torch.from_numpy(O.bf16_decode(kpe))[None].expand(H, T, 64)], dim=-1)
    v = torch.einsum("tc,hdc->htd", c, wv[:, 128:])
    qt = torch.from_numpy(q).permute(1, 0, 2)
    want = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=SCALE)
    np.testing.assert_allclose(out, want.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_prefill_sampled_rows_match_full():
    rng = np.random.default_rng(32)
    T, H = 20, 4
    q, lat, kpe, w = _prefill_small(rng, T, H)
    out, lse = O.prefill_causal(q, lat, kpe, w, SCALE, staged=True)
    rows, heads = [0, 7, 19], [1, 3]
    o2, l2 = O.prefill_causal(q, lat, kpe, w, SCALE, staged=True, heads=heads, rows=rows)
    np.testing.assert_array_equal(o2, out[rows][:, heads])
    np.testing.assert_array_equal(l2, lse[heads][:, rows])


def test_value_states_shape():
    """Kimi-K2 value_states: [B, 1, 512] latent -> [B, 64 heads, 1, 128] values."""
    rng = np.random.default_rng(33)
    lat = _rand_bits(rng, (1, 512))
    w = _rand_bits(rng, (64 * 256, 512), 512 ** -0.5)
    _, v = O.expand_latent(lat, w, 64, staged=False)
    assert v.shape == (1, 64, 128)
