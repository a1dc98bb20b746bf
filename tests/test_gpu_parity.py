"""GPU parity of libmla (through its C ABI) against the CPU oracle on the same seeded inputs.

Bars (tests/gpu_helpers.py): bf16 outputs within 2e-2 x RMS of each oracle output vector, against
the oracle's staged value before its final bf16 rounding; inv_rms and lse within 1e-4 relative
(lse relative to the magnitude of its score dot products); -inf lse exactly where the oracle has it;
cache rows beyond each length are NaN-poisoned, so reading one fails the check. Full-size workloads are checked on sampled sequences,
rows and heads that the oracle computes one by one."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from synth import inputs as S
from tests.gpu_helpers import (assert_bf16_parity, assert_f32_parity, bits_of, dev, dev_bf16, host_bits, say)

binding = pytest.importorskip("head_latent_attention_fp32_amd.binding")

pytestmark = pytest.mark.gpu
SCALE = 192 ** -0.5


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    binding.lib()   # raises if the HIP library is not built


# ----------------------------------------------------------------------------------- query path
def _query_case(H, n, seed, case_id, positions=None):
    rng = np.random.default_rng(seed * 1000 + case_id)
    x = S.normal_bf16_rows(n, S.Q_LORA, 1.0, (seed, case_id, S.T_Q_LATENT))
    w = S.query_weights(H, seed, case_id)
    pos = rng.integers(0, 131073, size=n) if positions is None else np.asarray(positions)
    return x, w["gamma"], w["wq_b"], S.rope_table(pos)


def _run_query(x, g, w, cs, H, with_inv=True):
    n = x.shape[0]
    inv = torch.empty(n, dtype=torch.float32, device="cuda") if with_inv else None
    q, _ = binding.query_path(dev_bf16(x), dev(g), dev_bf16(w), dev(cs), H, inv_rms=inv)
    torch.cuda.synchronize()
    return host_bits(q), (inv.cpu().numpy() if with_inv else None)


@pytest.mark.parametrize("H,n,with_inv", [(16, 1, True), (64, 1, True), (128, 1, True), (128, 5, False),
                                          (128, 32, True), (64, 32, False), (16, 32, True), (128, 33, True),
                                          (128, 64, True), (64, 67, True), (32, 130, False), (128, 200, True),
                                          (16, 1100, True), (32, 1024, False)])
def test_query_path_parity(H, n, with_inv):
    """Every path of the product: n <= 32 (activation in registers), 33..1023 (mid-size tiles),
    >= 1024 (256 x 256 tiles on wq_b as stored; full tiles through LDS, a partial last tile at
    1100 tokens through direct stores)."""
    say(f"query_path H={H} n={n} inv={with_inv}")
    x, g, w, cs = _query_case(H, n, 0, 200 + H + n)
    qg, inv = _run_query(x, g, w, cs, H, with_inv)
    qo, invo = O.query_path(x, g, w, cs, H, round_output=False)
    assert_bf16_parity(qg, qo, "q_out")
    if with_inv:
        assert_f32_parity(inv, invo, "inv_rms")


@pytest.mark.parametrize("H", [16, 64, 128])
def test_wq_b_pack_is_the_stated_rearrangement(H):
    """mla_wq_b_pack moves bytes only: packed[g, k, j] == wq_b[k, 32 g + j], bit for bit."""
    say(f"wq_b_pack H={H}")
    w = S.query_weights(H, 0, 260 + H)["wq_b"]
    p = binding.wq_b_pack(dev_bf16(w), H)
    torch.cuda.synchronize()
    want = w.reshape(S.Q_LORA, H * 192 // 32, 32).transpose(1, 0, 2)
    assert np.array_equal(host_bits(p), want)


@pytest.mark.parametrize("H,n", [(16, 1), (64, 1), (128, 1), (32, 5), (64, 32), (128, 32), (128, 33),
                                 (64, 67), (128, 200), (64, 1023), (16, 1100), (128, 1024)])
def test_query_path_packed_matches_stored_weights(H, n):
    """mla_query_path_packed on mla_wq_b_pack's copy: bit-identical to mla_query_path on wq_b as
    stored, on every product (n <= 32, 33..1023, >= 1024, and each slice width of the small one),
    and within the bar of the oracle ("DeepSeek-V3.2-Exp · Query heads", query excerpt)."""
    say(f"query_path packed H={H} n={n}")
    x, g, w, cs = _query_case(H, n, 1, 300 + H + n)
    wd = dev_bf16(w)
    packed = binding.wq_b_pack(wd, H)
    inv_p = torch.empty(n, dtype=torch.float32, device="cuda")
    inv_s = torch.empty(n, dtype=torch.float32, device="cuda")
    qp, _ = binding.query_path(dev_bf16(x), dev(g), packed, dev(cs), H, inv_rms=inv_p, packed=True)
    qs, _ = binding.query_path(dev_bf16(x), dev(g), wd, dev(cs), H, inv_rms=inv_s)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qp), host_bits(qs))
    assert np.array_equal(inv_p.cpu().numpy().view(np.uint32), inv_s.cpu().numpy().view(np.uint32))
    qo, invo = O.query_path(x, g, w, cs, H, round_output=False)
    assert_bf16_parity(host_bits(qp), qo, "q_out (packed weights)")
    assert_f32_parity(inv_p.cpu().numpy(), invo, "inv_rms (packed weights)")


@pytest.mark.slow
def test_query_path_past_4gib_of_activations():
    """16 heads over 1,398,200 tokens: the normalised activations span 4.3 GB, so one 256-token
    tile of the product (the first) starts more than 4 GiB of activation rows before the end. Its
    buffer descriptor covers only the rows the tile reads; were it sized to every row left, its
    32-bit byte range would wrap and rows 99.. of the tile would read as zeros ("DeepSeek-V3.2-Exp
    · Query heads", in/out shapes: every token's 1536 latent features become its query heads).
    The inputs are drawn on the device (seeded) and the tile's rows, plus the last tile's, copied
    back for the oracle."""
    H, n = 16, 1_398_200
    say(f"query_path H={H} n={n} (activations past 4 GiB)")
    x = S.device_normal_bf16((n, S.Q_LORA), seed=7, case_id=250)
    w = S.query_weights(H, 7, 250)
    pos = np.arange(n) % 131072
    cs = S.rope_table(pos)
    inv = torch.empty(n, dtype=torch.float32, device="cuda")
    q, _ = binding.query_path(x, dev(w["gamma"]), dev_bf16(w["wq_b"]), dev(cs), H, inv_rms=inv)
    torch.cuda.synchronize()
    rows = np.r_[0:256, n - 300:n]
    xr = host_bits(x[torch.from_numpy(rows).cuda()])
    qg = host_bits(q[torch.from_numpy(rows).cuda()])
    del q, x
    qo, invo = O.query_path(xr, w["gamma"], w["wq_b"], cs[rows], H, round_output=False)
    assert_bf16_parity(qg, qo, "q_out rows of the first and last tiles")
    assert_f32_parity(inv.cpu().numpy()[rows], invo, "inv_rms")


# ----------------------------------------------------------------------------------- decode
def _run_decode(case, q_bits, d, with_lse=True):
    B, H = case.batch, case.n_heads
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda") if with_lse else None
    out, _ = binding.decode(dev_bf16(q_bits), dev_bf16(d["wkv_b"]), dev_bf16(d["kv_cache"]),
                            dev_bf16(d["pe_cache"]), dev(d["lengths"]), int(case.max_seqlen),
                            cache_row_offset=None if case.layout == "padded" else dev(d["row_offset"]),
                            lse=lse)
    torch.cuda.synchronize()
    return host_bits(out), (lse.cpu().numpy() if with_lse else None)


def _decode_magnitude(q_vals, d, lens, ids):
    mags = []
    for b in ids:
        r0, L = int(d["row_offset"][b]), int(lens[b])
        mags.append(O.decode_score_magnitude(q_vals[b], d["wkv_b"], d["kv_cache"][r0:r0 + L],
                                             d["pe_cache"][r0:r0 + L], SCALE))
    return np.stack(mags)


def _check_decode(case, q_bits, d, out_bits, lse, batch_ids=None):
    lens = np.clip(d["lengths"].astype(np.int64), 0, int(case.max_seqlen))
    ids = list(range(case.batch)) if batch_ids is None else list(batch_ids)
    qv = O.bf16_decode(q_bits)
    oo, lo = O.decode_batch(qv, d["wkv_b"], d["kv_cache"], d["pe_cache"], d["row_offset"], lens,
                            SCALE, staged=True, batch_ids=ids, round_output=False)
    assert_bf16_parity(out_bits[ids], oo, "out")
    if lse is not None:
        assert_f32_parity(lse[ids], lo, "lse", magnitude=_decode_magnitude(qv, d, lens, ids))


DECODE_SMALL = [
    (16, [1], "padded"), (64, [31], "padded"), (64, [32], "padded"), (64, [33], "padded"),
    (128, [1000], "padded"), (32, [0, 5, 300], "padded"), (128, [257, 1, 0, 64, 512], "padded"),
    (64, [3, 700, 45, 0, 1, 96], "packed"), (128, [2049, 17], "packed"), (16, [0, 0], "padded"),
    # short caches: runs shorter than 256 tokens, a sequence's runs merged by several thread groups
    (128, [4096], "padded"),
    (128, [(37 * i) % 500 + 1 for i in range(20)], "packed"),
    # 72 sequences over 4 merge blocks per head: a block's second group holds 8 sequences
    (128, [(53 * i) % 300 for i in range(72)], "packed"),
    (64, [(29 * i) % 400 + 33 for i in range(40)], "padded"),
    # one merge group split four ways (at most four sequences) or two ways (5..16), and two groups
    (128, [700, 1, 2049, 33], "packed"), (128, [(61 * i) % 900 + 1 for i in range(16)], "padded"),
    (128, [(67 * i) % 800 for i in range(17)], "packed"),
]


@pytest.mark.parametrize("H,lens,layout", DECODE_SMALL)
def test_decode_parity_small(H, lens, layout):
    say(f"decode H={H} lens={lens} layout={layout}")
    case = S.DecodeCase("t", 300 + H + len(lens), H, np.array(lens, np.int32), layout=layout,
                        max_seqlen=max(max(lens), 1))
    d = S.decode_inputs(case, seed=1, with_q_latent=False)
    q = S.decode_query(case, seed=1)
    out, lse = _run_decode(case, q, d)
    _check_decode(case, q, d, out, lse)


def _many_lengths(B, mod, zero_every):
    return [0 if i % zero_every == 0 else (97 * i + 13) % mod for i in range(B)]


@pytest.mark.parametrize("H,B,layout", [(16, 300, "packed"), (64, 300, "padded"), (16, 1000, "padded"),
                                        (64, 1000, "packed"), (128, 300, "packed")])
def test_decode_parity_many_sequences(H, B, layout):
    """More than 256 sequences: the run plan takes its chunked branch (each plan thread owns a
    contiguous chunk of sequences, prefix sums across the chunks, run start records stepped within
    them). Short ragged caches with every 7th sequence empty, so that runs cross many sequence
    boundaries and some runs start right after empty sequences ("DeepSeek-V3.2-Exp · Attention
    update", mla-decode: each sequence attends exactly its own rows kv_cache[b, :end_pos])."""
    lens = _many_lengths(B, 301 if B == 300 else 257, 7)
    say(f"decode H={H} B={B} layout={layout} sum L={sum(lens)}")
    case = S.DecodeCase("t", 360 + H + B, H, np.array(lens, np.int32), layout=layout, max_seqlen=max(lens))
    d = S.decode_inputs(case, seed=5, with_q_latent=False)
    q = S.decode_query(case, seed=5)
    out, lse = _run_decode(case, q, d)
    _check_decode(case, q, d, out, lse)


@pytest.mark.parametrize("shift", [16, -20])
def test_decode_partials_outside_fp16_range(shift):
    """The split partials are kept as fp16 times a power of two per 128 columns: a cache scaled by
    2^shift, with the query's content part scaled by 2^-shift (the same scores), gives outputs
    2^shift times larger -- for shift 16 past fp16's largest finite value, for -20 inside its
    subnormal range -- which must still meet the bar."""
    say(f"decode with the cache scaled by 2^{shift}")
    case = S.DecodeCase("t", 340 + (shift > 0), 128, np.array([3000, 700, 1], np.int32), layout="packed")
    d = S.decode_inputs(case, seed=4, with_q_latent=False)
    q = S.decode_query(case, seed=4)
    f = 2.0 ** shift
    d["kv_cache"] = bits_of(O.bf16_decode(d["kv_cache"]) * f)
    qv = O.bf16_decode(q)
    qv[..., :128] *= 1.0 / f
    q = bits_of(qv)
    out, lse = _run_decode(case, q, d)
    _check_decode(case, q, d, out, lse)


def test_decode_lengths_are_clamped():
    say("decode clamped lengths")
    case = S.DecodeCase("t", 330, 64, np.array([40, 40, 40], np.int32), max_seqlen=40)
    d = S.decode_inputs(case, seed=2, with_q_latent=False)
    d["lengths"] = np.array([-7, 41000, 13], np.int32)     # clamped to [0, max_seqlen]
    q = S.decode_query(case, seed=2)
    out, lse = _run_decode(case, q, d)
    _check_decode(case, q, d, out, lse)


def test_decode_is_deterministic():
    case = S.DecodeCase("t", 331, 128, np.array([3000, 5, 1200], np.int32), layout="packed")
    d = S.decode_inputs(case, seed=3, with_q_latent=False)
    q = S.decode_query(case, seed=3)
    a, la = _run_decode(case, q, d)
    b, lb = _run_decode(case, q, d)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def _decode_step(cfg, sample):
    case = S.workload(cfg)
    say(f"decode step {case.name}: query path + decode on the GPU, oracle on sequences {sample}")
    d = S.decode_inputs(case, seed=0)
    H = case.n_heads
    inv = torch.empty(case.batch, dtype=torch.float32, device="cuda")
    q, _ = binding.query_path(dev_bf16(d["q_latent"]), dev(d["gamma"]), dev_bf16(d["wq_b"]), dev(d["rope_cs"]), H,
                              inv_rms=inv)
    lse = torch.empty((case.batch, H), dtype=torch.float32, device="cuda")
    out, _ = binding.decode(q, dev_bf16(d["wkv_b"]), dev_bf16(d["kv_cache"]), dev_bf16(d["pe_cache"]),
                            dev(d["lengths"]), int(case.max_seqlen),
                            cache_row_offset=None if case.layout == "padded" else dev(d["row_offset"]), lse=lse)
    torch.cuda.synchronize()
    qg = host_bits(q)
    qo, invo = O.query_path(d["q_latent"][sample], d["gamma"], d["wq_b"], d["rope_cs"][sample], H)
    qu, _ = O.query_path(d["q_latent"][sample], d["gamma"], d["wq_b"], d["rope_cs"][sample], H, round_output=False)
    assert_bf16_parity(qg[sample], qu, "q_out")
    assert_f32_parity(inv.cpu().numpy()[sample], invo, "inv_rms")
    # decode checked on the oracle's own query (no GPU value feeds the oracle)
    qfull = _scatter(qo, sample, case.batch)
    oo, lo = O.decode_batch(qfull, d["wkv_b"], d["kv_cache"], d["pe_cache"], d["row_offset"], d["lengths"], SCALE,
                            staged=True, batch_ids=sample, round_output=False)
    assert_bf16_parity(host_bits(out)[sample], oo, "out")
    assert_f32_parity(lse.cpu().numpy()[sample], lo, "lse",
                      magnitude=_decode_magnitude(qfull, d, d["lengths"], sample))


def _scatter(vals, ids, n):
    full = np.zeros((n,) + vals.shape[1:])
    full[ids] = vals
    return full


def test_decode_step_config0():
    _decode_step(0, [0])


@pytest.mark.slow
def test_decode_step_config1():
    _decode_step(1, [0, 13, 31])


@pytest.mark.slow
def test_decode_step_config3_ragged():
    lens = S.workload(3).lengths
    _decode_step(3, sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 64, 127}))


@pytest.mark.slow
def test_decode_step_config4_long():
    _decode_step(4, [0, 7])


# ----------------------------------------------------------------------------------- prefill
def _run_prefill(q_bits, lat, kpe, w, H):
    B, T = lat.shape[:2]
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    out, _ = binding.prefill(dev_bf16(q_bits), dev_bf16(lat), dev_bf16(kpe), dev_bf16(w), lse=lse)
    torch.cuda.synchronize()
    return host_bits(out), lse.cpu().numpy()


@pytest.mark.parametrize("H,B,T", [(16, 1, 1), (16, 2, 5), (64, 1, 64), (32, 1, 65), (128, 1, 130),
                                   (64, 3, 200), (16, 1, 257), (16, 2, 384), (64, 1, 512), (32, 2, 512)])
def test_prefill_parity_small(H, B, T):
    """(16, 2, 384): expansion tiles of 256 tokens inside one sequence (through LDS) and one across
    the boundary (direct stores); (64, 1, 512) and (32, 2, 512): every tile through LDS, in one and
    in two sequences."""
    say(f"prefill H={H} B={B} T={T}")
    case = S.PrefillCase("t", 400 + H + T + B, H, B, T)
    d = S.prefill_inputs(case, seed=4, with_q_latent=False)
    q = S.prefill_query(case, seed=4)
    out, lse = _run_prefill(q, d["kv_latent"], d["k_pe"], d["wkv_b"], H)
    for b in range(B):
        qv = O.bf16_decode(q[b])
        oo, lo = O.prefill_causal(qv, d["kv_latent"][b], d["k_pe"][b], d["wkv_b"], SCALE, round_output=False)
        assert_bf16_parity(out[b], oo, f"out[b={b}]")
        mag = O.prefill_score_magnitude(qv, d["kv_latent"][b], d["k_pe"][b], d["wkv_b"], SCALE)
        assert_f32_parity(lse[b], lo, f"lse[b={b}]", magnitude=mag)


@pytest.mark.parametrize("shift", [16, -20])
def test_prefill_values_outside_fp16_range(shift):
    """The expanded values are stored as f16 divided by a power of two per head, chosen from a
    bound of what the head can produce: with the value half of wkv_b scaled by 2^shift the scores
    are unchanged and the outputs 2^shift times larger -- for shift 16 past f16's largest finite
    value, for -20 inside its subnormal range -- and must still meet the bar ("Kimi-K2 ·
    value_states", mla-prefill: the values are kv_b_proj's bf16 output, of any size)."""
    H, B, T = 32, 1, 200
    say(f"prefill with the value half of wkv_b scaled by 2^{shift}")
    case = S.PrefillCase("t", 470 + (shift > 0), H, B, T)
    d = S.prefill_inputs(case, seed=6, with_q_latent=False)
    q = S.prefill_query(case, seed=6)
    w = O.bf16_decode(d["wkv_b"]).reshape(H, 256, 512)
    w[:, 128:, :] *= 2.0 ** shift
    wb = bits_of(w.reshape(H * 256, 512))
    out, lse = _run_prefill(q, d["kv_latent"], d["k_pe"], wb, H)
    qv = O.bf16_decode(q[0])
    oo, lo = O.prefill_causal(qv, d["kv_latent"][0], d["k_pe"][0], wb, SCALE, round_output=False)
    assert_bf16_parity(out[0], oo, "out")
    mag = O.prefill_score_magnitude(qv, d["kv_latent"][0], d["k_pe"][0], wb, SCALE)
    assert_f32_parity(lse[0], lo, "lse", magnitude=mag)


@pytest.mark.slow
def test_prefill_expansion_past_4gib_of_latent():
    """1025 sequences of 4096 positions at 16 heads: 4,198,400 latent rows (4.3 GB). The expansion
    tile at row 4096 (sequence 1, positions 0..255) starts exactly 4 GiB of latent rows before the
    end, where a descriptor sized to every row left would wrap to an empty range. Sequence 1 is
    checked on its first 256 rows and on rows near its end ("Kimi-K2 · value_states", mla-prefill:
    kv_b_proj expands every position's latent). Inputs drawn on the device (seeded)."""
    H, B, T = 16, 1025, 4096
    say(f"prefill H={H} B={B} T={T} (latent past 4 GiB)")
    w = S.kv_weights(H, 8, 451)
    lat = S.device_normal_bf16((B, T, S.KV_LORA), seed=8, case_id=451, tensor=S.T_KV_LAT)
    kpe = S.device_normal_bf16((B, T, S.ROPE), seed=8, case_id=451, tensor=S.T_K_PE)
    q = S.device_normal_bf16((B, T, H, S.QK_DIM), seed=8, case_id=451, tensor=S.T_Q)
    out, _ = binding.prefill(q, lat, kpe, dev_bf16(w))
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 100, 200, 255, 256, 4000, 4095]
    heads = [0, 9, 15]
    b = 1
    og = host_bits(out[b])[rows][:, heads]
    del out
    qb = O.bf16_decode(host_bits(q[b]))
    latb, kpeb = host_bits(lat[b]), host_bits(kpe[b])
    oo, _ = O.prefill_causal(qb, latb, kpeb, w, SCALE, heads=heads, rows=rows, round_output=False)
    assert_bf16_parity(og, oo, "out of sequence 1")


@pytest.mark.slow
def test_prefill_config2_sampled():
    case = S.workload(2)
    say(f"prefill {case.name}: query path + prefill on the GPU, oracle on sampled rows and heads")
    d = S.prefill_inputs(case, seed=0)
    H, T = case.n_heads, case.seqlen
    q, _ = binding.query_path(dev_bf16(d["q_latent"][0]), dev(d["gamma"]), dev_bf16(d["wq_b"]), dev(d["rope_cs"]), H)
    out, lse = _run_prefill(host_bits(q)[None], d["kv_latent"], d["k_pe"], d["wkv_b"], H)
    rows = [0, 1, 63, 64, 65, 1000, 2047, 4094, 4095]
    heads = [0, 77, 127]
    qo, _ = O.query_path(d["q_latent"][0][: max(rows) + 1], d["gamma"], d["wq_b"], d["rope_cs"][: max(rows) + 1], H)
    qu, _ = O.query_path(d["q_latent"][0][rows], d["gamma"], d["wq_b"], d["rope_cs"][rows], H, round_output=False)
    assert_bf16_parity(host_bits(q)[rows], qu, "q_out rows")
    oo, lo = O.prefill_causal(qo, d["kv_latent"][0], d["k_pe"][0], d["wkv_b"], SCALE, heads=heads, rows=rows,
                              round_output=False)
    assert_bf16_parity(out[0][rows][:, heads], oo, "out")
    mag = O.prefill_score_magnitude(qo, d["kv_latent"][0], d["k_pe"][0], d["wkv_b"], SCALE, heads=heads, rows=rows)
    assert_f32_parity(lse[0][heads][:, rows], lo, "lse", magnitude=mag)
