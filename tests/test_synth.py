"""The seeded input module: determinism, regenerable slices, layouts and the workload recipe."""
import numpy as np

from synth import inputs as S


def test_seeded_determinism_and_seed_sensitivity():
    c = S.DecodeCase("t", 50, 4, np.array([5, 0, 33]), layout="padded", max_seqlen=40)
    a = S.decode_inputs(c, seed=1, workers=1)
    b = S.decode_inputs(c, seed=1, workers=3)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=False) or np.array_equal(
            a[k].view(np.uint8), b[k].view(np.uint8)), k
    d = S.decode_inputs(c, seed=2, workers=1)
    assert not np.array_equal(a["kv_cache"][:5], d["kv_cache"][:5])


def test_sequence_regeneration_and_padding_poison():
    c = S.DecodeCase("t", 51, 2, np.array([7, 3, 0, 12]), layout="padded", max_seqlen=16)
    d = S.decode_inputs(c, seed=0, workers=1)
    assert d["kv_cache"].shape == (64, 512) and d["pe_cache"].shape == (64, 64)
    for b in range(4):
        s = S.sequence_cache(c, b, seed=0)
        r0, L = int(d["row_offset"][b]), int(d["lengths"][b])
        assert np.array_equal(d["kv_cache"][r0:r0 + L], s["kv"])
        assert np.array_equal(d["pe_cache"][r0:r0 + L], s["pe"])
        assert np.all(d["kv_cache"][r0 + L:r0 + 16] == 0x7FC0)


def test_packed_layout_offsets():
    c = S.DecodeCase("t", 52, 2, np.array([3, 5, 2]), layout="packed")
    d = S.decode_inputs(c, seed=0, workers=1)
    assert d["row_offset"].tolist() == [0, 3, 8]
    assert d["kv_cache"].shape[0] == 10


def test_spikes_scale_rows_by_eight_exactly():
    base = S.DecodeCase("t", 53, 2, np.array([500]))
    spk = S.DecodeCase("t", 53, 2, np.array([500]), spike_frac=0.01)
    a = S.bf16_bits_to_f32(S.sequence_cache(base, 0, 0)["kv"])
    b = S.bf16_bits_to_f32(S.sequence_cache(spk, 0, 0)["kv"])
    ratio_rows = np.where(np.any(a != b, axis=1))[0]
    assert len(ratio_rows) == 5
    np.testing.assert_array_equal(b[ratio_rows], a[ratio_rows] * 8)


def test_workload_recipe():
    c0 = S.workload(0)
    assert c0.batch == 1 and c0.n_heads == 64 and int(c0.lengths[0]) == 1000 and int(c0.positions[0]) == 1000
    c3 = S.workload(3)
    assert c3.batch == 128 and c3.lengths.min() >= 256 and c3.lengths.max() <= 32768
    assert c3.layout == "packed"
    c4 = S.workload(4)
    assert c4.spike_frac == 0.01 and int(c4.lengths.sum()) == 8 * 131072
    c2 = S.workload(2)
    assert (c2.batch, c2.seqlen, c2.n_heads) == (1, 4096, 128)


def test_weight_and_activation_statistics():
    w = S.query_weights(128, 0, 1)
    x = S.bf16_bits_to_f32(w["wq_b"][:, :4096]).astype(np.float64)
    assert abs(x.std() * np.sqrt(1536) - 1) < 0.01
    assert abs(w["gamma"].mean() - 1) < 0.01 and abs(w["gamma"].std() - 0.1) < 0.01
    kvw = S.bf16_bits_to_f32(S.kv_weights(4, 0, 1)).astype(np.float64)
    assert abs(kvw.std() * np.sqrt(512) - 1) < 0.02


def test_synth_imports_nothing_from_oracle_or_library():
    import inspect
    src = inspect.getsource(S)
    assert "oracle" not in src.replace("the oracle", "")
    assert "head_latent_attention_fp32_amd" not in src
