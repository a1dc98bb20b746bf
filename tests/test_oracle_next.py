"""Pins of the oracle's steps next to the hot path (CPU only): the key/value side of new tokens
and the cache write, decode restricted to top-k positions, prefill over a cached prefix, and the
output projection wo.

As for the core path, nothing here retypes the oracle's formulas: the pins are closed forms and
special cases, invariances, agreement between different forms of the same quantity (mask vs.
gathered rows, chunked vs. whole prefill, prefill row vs. decode over the prefix), library
routines (torch on the CPU in float64) and the pages' printed shapes."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from synth import inputs as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = 192 ** -0.5


def _bits(a):
    return O.bf16_encode(np.asarray(a, np.float64))


def _rand_bits(rng, shape, std=1.0):
    return _bits(rng.standard_normal(shape) * std)


# ------------------------------------------------------------------------------ kv side
def _kv_a(rng, n):
    return _rand_bits(rng, (n, 576)), (1 + 0.1 * rng.standard_normal(512)).astype(np.float32)


def test_kv_side_split_order():
    """The latent is the first 512 features, the rotary key the last 64: changing one part leaves
    the other output unchanged bit for bit."""
    rng = np.random.default_rng(40)
    a, g = _kv_a(rng, 5)
    cs = S.rope_table(np.arange(5) * 17)
    lat, pe = O.kv_side(a, g, cs, staged=False)
    assert lat.shape == (5, 512) and pe.shape == (5, 64)
    a2 = a.copy()
    a2[:, 512:] = _rand_bits(rng, (5, 64))
    lat2, pe2 = O.kv_side(a2, g, cs, staged=False)
    np.testing.assert_array_equal(lat2, lat)
    assert np.all(np.abs(pe2 - pe).max(axis=1) > 0)
    a3 = a.copy()
    a3[:, :512] = _rand_bits(rng, (5, 512))
    lat3, pe3 = O.kv_side(a3, g, cs, staged=False)
    np.testing.assert_array_equal(pe3, pe)
    assert np.all(np.abs(lat3 - lat).max(axis=1) > 0)


def test_kv_side_latent_norm_and_library():
    rng = np.random.default_rng(41)
    a, g = _kv_a(rng, 6)
    cs = S.rope_table(np.zeros(6, np.int64))
    lat, _ = O.kv_side(a, np.ones(512, np.float32), cs, eps=0.0, staged=False)
    np.testing.assert_allclose(np.mean(lat ** 2, axis=1), 1.0, rtol=1e-13)
    lat_g, _ = O.kv_side(a, g, cs, staged=False)
    want = torch.nn.functional.rms_norm(torch.from_numpy(O.bf16_decode(a)[:, :512]), (512,),
                                        torch.from_numpy(g.astype(np.float64)), 1e-6)
    np.testing.assert_allclose(lat_g, want.numpy(), rtol=1e-12, atol=1e-14)
    # a constant row normalises to the gain itself
    c = _bits(np.full((1, 576), 2.0))
    lat_c, _ = O.kv_side(c, g, cs[:1], eps=0.0, staged=False)
    np.testing.assert_allclose(lat_c[0], g.astype(np.float64), rtol=1e-15)


def test_kv_side_rotary_key():
    rng = np.random.default_rng(42)
    a, g = _kv_a(rng, 4)
    x = O.bf16_decode(a)[:, 512:]
    _, pe0 = O.kv_side(a, g, S.rope_table(np.zeros(4, np.int64)), staged=False)
    np.testing.assert_array_equal(pe0, x)                       # position 0: identity
    pos = np.array([1, 7, 4096, 131072])
    cs = S.rope_table(pos)
    _, pe = O.kv_side(a, g, cs, staged=False)
    np.testing.assert_allclose(np.hypot(pe[:, 0::2], pe[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]), rtol=1e-6)
    # the complex-multiplication route of torch, pairs (2i, 2i+1)
    z = torch.view_as_complex(torch.from_numpy(x).reshape(4, 32, 2).contiguous())
    r = torch.view_as_complex(torch.from_numpy(cs.astype(np.float64)).contiguous())
    np.testing.assert_allclose(pe, torch.view_as_real(z * r).reshape(4, 64).numpy(), rtol=1e-12, atol=1e-14)


def test_cache_append_rows_and_decode_roundtrip():
    rng = np.random.default_rng(43)
    B, T, Lmax, H = 3, 2, 9, 2
    kv = _rand_bits(rng, (B * Lmax, 512))
    pe = _rand_bits(rng, (B * Lmax, 64))
    off = np.arange(B) * Lmax
    start = np.array([0, 4, 8])                        # the last sequence's second token falls off
    a, g = _kv_a(rng, B * T)
    pos = (start[:, None] + np.arange(T)[None]).reshape(-1)
    lat, kpe = O.kv_side(a, g, S.rope_table(pos), staged=True)
    lat_b, kpe_b = _bits(lat).reshape(B, T, 512), _bits(kpe).reshape(B, T, 64)
    kv2, pe2 = O.cache_append(kv, pe, off, start, lat_b, kpe_b, Lmax)
    written = {int(off[b] + start[b] + t) for b in range(B) for t in range(T) if start[b] + t < Lmax}
    assert written == {0, 1, 13, 14, 26}
    for row in range(B * Lmax):
        if row in written:
            b, t = next((b, t) for b in range(B) for t in range(T) if off[b] + start[b] + t == row)
            np.testing.assert_array_equal(kv2[row], lat_b[b, t])
            np.testing.assert_array_equal(pe2[row], kpe_b[b, t])
        else:
            np.testing.assert_array_equal(kv2[row], kv[row])
            np.testing.assert_array_equal(pe2[row], pe[row])
    # decode over the updated cache = decode over the old prefix followed by the new rows
    w = _rand_bits(rng, (H * 256, 512), 512 ** -0.5)
    q = rng.standard_normal((H, 192))
    b = 1
    L = start[b] + T
    o1, l1 = O.decode_absorbed(q, w, kv2[off[b]:off[b] + L], pe2[off[b]:off[b] + L], SCALE, staged=False)
    o2, l2 = O.decode_absorbed(q, w, np.concatenate([kv[off[b]:off[b] + start[b]], lat_b[b]]),
                               np.concatenate([pe[off[b]:off[b] + start[b]], kpe_b[b]]), SCALE, staged=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ------------------------------------------------------------------------------ top-k decode
def _decode_small(rng, L, H):
    kv = _rand_bits(rng, (L, 512))
    pe = _rand_bits(rng, (L, 64))
    w = _rand_bits(rng, (H * 256, 512), 512 ** -0.5)
    q = O.bf16_round(rng.standard_normal((H, 192)))
    return q, w, kv, pe


def test_topk_all_positions_is_dense_decode():
    rng = np.random.default_rng(50)
    L, H = 11, 3
    q, w, kv, pe = _decode_small(rng, L, H)
    dense = O.decode_absorbed(q, w, kv, pe, SCALE, staged=False)
    sel = O.decode_topk(q, w, kv, pe, rng.permutation(L), SCALE, staged=False)
    np.testing.assert_allclose(sel[0], dense[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sel[1], dense[1], rtol=1e-13)


def test_topk_equals_dense_decode_over_gathered_rows():
    rng = np.random.default_rng(51)
    L, H = 40, 2
    q, w, kv, pe = _decode_small(rng, L, H)
    idx = rng.choice(L, 9, replace=False)
    got = O.decode_topk(q, w, kv, pe, np.concatenate([idx, [-1, -1, L, L + 5]]), SCALE, staged=False)
    want = O.decode_absorbed(q, w, kv[np.sort(idx)], pe[np.sort(idx)], SCALE, staged=False)
    np.testing.assert_allclose(got[0], want[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got[1], want[1], rtol=1e-13)
    # the order of the list and repeated names do not matter (the mask is a set of positions)
    got2 = O.decode_topk(q, w, kv, pe, np.concatenate([idx[::-1], idx[:3]]), SCALE, staged=False)
    np.testing.assert_allclose(got2[0], got[0], rtol=1e-12, atol=1e-14)


def test_topk_special_cases():
    rng = np.random.default_rng(52)
    L, H = 7, 2
    q, w, kv, pe = _decode_small(rng, L, H)
    _, uv = O.wkv_b_heads(O.bf16_decode(w), H)
    out, lse = O.decode_topk(q, w, kv, pe, np.array([4, -1, -1]), SCALE, staged=False)
    np.testing.assert_allclose(out, uv @ O.bf16_decode(kv[4]), rtol=1e-12)   # one position: its value
    out, lse = O.decode_topk(q, w, kv, pe, np.array([-1, 7, 100]), SCALE, staged=False)
    assert np.all(out == 0) and np.all(lse == -np.inf)                       # nothing selected
    # rows not selected do not matter
    kv2, pe2 = kv.copy(), pe.copy()
    kv2[[0, 1, 5]] = _rand_bits(rng, (3, 512))
    pe2[[0, 1, 5]] = _rand_bits(rng, (3, 64))
    sel = np.array([2, 3, 6])
    a = O.decode_topk(q, w, kv, pe, sel, SCALE, staged=False)
    b = O.decode_topk(q, w, kv2, pe2, sel, SCALE, staged=False)
    np.testing.assert_array_equal(a[0], b[0])


# ------------------------------------------------------------------------------ prefix prefill
def _prefill_small(rng, T, H):
    q = O.bf16_round(rng.standard_normal((T, H, 192)))
    lat = _rand_bits(rng, (T, 512))
    kpe = _rand_bits(rng, (T, 64))
    w = _rand_bits(rng, (H * 256, 512), 512 ** -0.5)
    return q, lat, kpe, w


def test_prefix_prefill_equals_tail_of_whole_prefill():
    rng = np.random.default_rng(60)
    S_, H = 14, 3
    q, lat, kpe, w = _prefill_small(rng, S_, H)
    whole, lse_w = O.prefill_causal(q, lat, kpe, w, SCALE, staged=False)
    for Tq in (1, 5, 14):
        part, lse_p = O.prefill_causal(q[S_ - Tq:], lat, kpe, w, SCALE, staged=False)
        np.testing.assert_allclose(part, whole[S_ - Tq:], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse_p, lse_w[:, S_ - Tq:], rtol=1e-13)


def test_prefix_prefill_rows_equal_decode_and_sdpa():
    rng = np.random.default_rng(61)
    S_, Tq, H = 12, 4, 2
    q, lat, kpe, w = _prefill_small(rng, S_, H)
    qn = q[:Tq] * 1.5                                   # new queries, unrelated to the prefix's own
    out, lse = O.prefill_causal(qn, lat, kpe, w, SCALE, staged=False)
    off = S_ - Tq
    for i in range(Tq):
        od, ld = O.decode_absorbed(qn[i], w, lat[: off + i + 1], kpe[: off + i + 1], SCALE, staged=False)
        np.testing.assert_allclose(out[i], od, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[:, i], ld, rtol=1e-12)
    # library: SDPA with the explicit offset mask (query i keeps keys <= off + i)
    wv = torch.from_numpy(O.bf16_decode(w)).view(H, 256, 512)
    c = torch.from_numpy(O.bf16_decode(lat))
    k = torch.cat([torch.einsum("tc,hdc->htd", c, wv[:, :128]),
                   torch.from_numpy(O.bf16_decode(kpe))[None].expand(H, S_, 64)], dim=-1)
    v = torch.einsum("tc,hdc->htd", c, wv[:, 128:])
    mask = torch.arange(S_)[None, :] <= (off + torch.arange(Tq))[:, None]
    want = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(qn).permute(1, 0, 2), k, v,
                                                            attn_mask=mask, scale=SCALE)
    np.testing.assert_allclose(out, want.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    with pytest.raises(ValueError):
        O.prefill_causal(q, lat[:5], kpe[:5], w, SCALE)


# ------------------------------------------------------------------------------ output projection
def test_output_proj_width_flatten_order_and_library():
    with open(os.path.join(GOLDEN, "shapes.json")) as f:
        g = json.load(f)["attention_update"]
    rng = np.random.default_rng(70)
    n, H, dim = 3, 4, 24
    x = _rand_bits(rng, (n, H, 128))
    wo = _rand_bits(rng, (dim, H * 128), (H * 128) ** -0.5)
    y = O.output_proj(x, wo, staged=False)
    assert y.shape == (n, dim)
    # the DeepSeek-V3.2 update is [B, 1, 7168]: wo maps 128 heads x 128 values to that width
    wo_shape = (g["width"], g["n_heads"] * g["v_head_dim"])
    assert wo_shape == (7168, 16384) and wo_shape[0] * wo_shape[1] == g["wo_parameters"]
    # feature h*128 + d of the flattened input is head h, value d
    xs = np.zeros((1, H, 128))
    xs[0, 2, 5] = 1.0
    ys = O.output_proj(_bits(xs), wo, staged=False)
    np.testing.assert_array_equal(ys[0], O.bf16_decode(wo)[:, 2 * 128 + 5])
    want = torch.nn.functional.linear(torch.from_numpy(O.bf16_decode(x)).reshape(n, -1),
                                      torch.from_numpy(O.bf16_decode(wo)))
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=1e-13)
