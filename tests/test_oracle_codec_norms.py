"""Pins of the oracle's bf16 codec, RMSNorm, LayerNorm and rotation (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------ codec
def test_bf16_roundtrip_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_decode(bits)
    back = O.bf16_encode(vals)
    nan = np.isnan(vals)
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(np.isnan(O.bf16_decode(back[nan])))


def test_bf16_decode_known_values():
    assert O.bf16_decode(np.uint16(0x3F80)) == 1.0
    assert O.bf16_decode(np.uint16(0xC000)) == -2.0
    assert O.bf16_decode(np.uint16(0x0001)) == 2.0 ** -133
    assert O.bf16_decode(np.uint16(0x7F7F)) == (2 - 2 ** -7) * 2.0 ** 127


@pytest.mark.parametrize("x,bits", [
    (1 + 2 ** -8, 0x3F80),                  # tie between 1 and 1+2^-7 -> even (1)
    (1 + 3 * 2 ** -8, 0x3F82),              # tie between 1+2^-7 and 1+2^-6 -> even
    (-(1 + 2 ** -8), 0xBF80),
    (1 + 2 ** -8 + 2 ** -30, 0x3F81),       # just above the tie
    (1 + 2 ** -8 - 2 ** -30, 0x3F80),       # just below the tie
    ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80),   # tie between max finite and 2^128 -> inf
    ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),
    (2.0 ** -134, 0x0000),                  # subnormal tie -> even (0)
    (3 * 2.0 ** -134, 0x0002),              # subnormal tie -> even (2)
    (0.0, 0x0000), (-0.0, 0x8000),
    (np.inf, 0x7F80), (-np.inf, 0xFF80),
])
def test_bf16_encode_ties_and_limits(x, bits):
    assert int(O.bf16_encode(np.float64(x))) == bits


def test_bf16_encode_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000), rng.standard_normal(20000) * 1e-38,
                        rng.standard_normal(20000) * 1e30]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_encode(x.astype(np.float64))
    assert np.array_equal(got, want)


# ------------------------------------------------------------------------------------ RMSNorm
def test_rmsnorm_hand_case():
    g = _golden("hand_cases.json")["rmsnorm"]
    y, inv = O.rms_norm(np.array(g["x"]), np.array(g["gamma"]), g["eps"])
    np.testing.assert_allclose(y, g["y"], rtol=1e-14)
    np.testing.assert_allclose(inv, g["inv_rms"], rtol=1e-14)


def test_rmsnorm_unit_rms_and_eps_shrink():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 1536)) * rng.uniform(0.01, 10, (16, 1))
    y, _ = O.rms_norm(x, np.ones(1536), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-12)
    eps = 1e-2
    y, _ = O.rms_norm(x, np.ones(1536), eps)
    m2 = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), m2 / (m2 + eps), rtol=1e-12)


def test_rmsnorm_scale_invariance_gain_and_zero_row():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 64))
    g = 1 + 0.1 * rng.standard_normal(64)
    y1, _ = O.rms_norm(x, g, 0.0)
    y2, _ = O.rms_norm(-7.5 * x, g, 0.0)
    np.testing.assert_allclose(y2, -y1, rtol=1e-12)
    y0, inv0 = O.rms_norm(np.zeros((1, 64)), g, 1e-6)
    assert np.all(y0 == 0) and np.isfinite(inv0).all()
    # the gain multiplies feature j only
    yg, _ = O.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(y1, yg * g, rtol=1e-13)


def test_rmsnorm_matches_torch_fp64():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 1536))
    g = 1 + 0.1 * rng.standard_normal(1536)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (1536,), torch.from_numpy(g), 1e-6).numpy()
    y, _ = O.rms_norm(x, g, 1e-6)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------------------ LayerNorm
def test_layernorm_hand_case():
    g = _golden("hand_cases.json")["layernorm"]
    y = O.layer_norm(np.array(g["x"]), np.array(g["gamma"]), np.array(g["beta"]), g["eps"])
    np.testing.assert_allclose(y, g["y"], rtol=1e-13)


def test_layernorm_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((32, 128)) * 3 + rng.standard_normal((32, 1)) * 5
    y = O.layer_norm(x, np.ones(128), np.zeros(128), 0.0)
    np.testing.assert_allclose(np.mean(y, axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-12)
    eps = 0.5
    y = O.layer_norm(x, np.ones(128), np.zeros(128), eps)
    var = np.var(x, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), var / (var + eps), rtol=1e-12)
    # shift invariance and the bias adds per feature
    beta = rng.standard_normal(128)
    np.testing.assert_allclose(O.layer_norm(x + 11.0, np.ones(128), beta, 1e-6),
                               O.layer_norm(x, np.ones(128), beta, 1e-6), atol=1e-10)


def test_layernorm_matches_torch_fp64_and_param_count():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 128))
    g = 1 + 0.1 * rng.standard_normal(128)
    b = 0.1 * rng.standard_normal(128)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (128,), torch.from_numpy(g),
                                          torch.from_numpy(b), 1e-6).numpy()
    np.testing.assert_allclose(O.layer_norm(x, g, b, 1e-6), want, rtol=1e-12, atol=1e-13)
    pc = _golden("param_counts.json")["indexer_key_layernorm"]
    assert g.size + b.size == pc["per_instance"]
    assert pc["per_instance"] * pc["instances"] == pc["across_instances"]


# ------------------------------------------------------------------------------------ rotation
def test_rope_hand_case():
    g = _golden("hand_cases.json")["rope"]
    cs = np.array([[np.cos(g["angle"]), np.sin(g["angle"])]])
    np.testing.assert_allclose(O.rope_rotate(np.array(g["pair"]), cs), g["rotated"], rtol=1e-13)


def test_rope_identity_norms_relative_position():
    from synth.inputs import rope_table
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 64))
    np.testing.assert_array_equal(O.rope_rotate(x, rope_table([0] * 5)), x)
    pos = np.array([1, 17, 1000, 4096, 131072])
    r = O.rope_rotate(x, rope_table(pos))
    np.testing.assert_allclose(np.hypot(r[:, 0::2], r[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]),
                               rtol=1e-6)
    # <RoPE(q, m), RoPE(k, n)> depends on m - n only (fp64 angles here)
    q, k = rng.standard_normal(64), rng.standard_normal(64)

    def cs64(p):
        ang = p * 10000.0 ** (-2.0 * np.arange(32) / 64)
        return np.stack([np.cos(ang), np.sin(ang)], -1)

    d1 = O.rope_rotate(q, cs64(10)) @ O.rope_rotate(k, cs64(3))
    d2 = O.rope_rotate(q, cs64(1007)) @ O.rope_rotate(k, cs64(1000))
    assert abs(d1 - d2) < 1e-10
    # the complex-number route: (a + ib) e^{i phi}
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * (pos[:, None] * 10000.0 ** (-2.0 * np.arange(32) / 64)))
    np.testing.assert_allclose(r[:, 0::2], z.real, atol=2e-6)
    np.testing.assert_allclose(r[:, 1::2], z.imag, atol=2e-6)


def test_rope_table_frequencies():
    from synth.inputs import rope_table
    t = rope_table(np.array([1, 100]))
    # pair 0 turns by the position itself; pair 16 by position/100 (10000^(-1/2))
    np.testing.assert_allclose(t[0, 0], [np.cos(1.0), np.sin(1.0)], rtol=1e-7)
    np.testing.assert_allclose(t[1, 16], [np.cos(1.0), np.sin(1.0)], rtol=1e-6)
    assert t.shape == (2, 32, 2) and t.dtype == np.float32
