"""GPU parity of the steps next to the hot path (through the C ABI) against the CPU oracle:
the key/value side with its cache write, prefill over a cached prefix, and their composition with
decode and prefill on caches the library wrote itself.

Bars as in tests/gpu_helpers.py. Cache rows that no new token owns are compared bit for bit
(they must be untouched); written rows within 2e-2 x RMS of each row."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from synth import inputs as S
from tests.gpu_helpers import (assert_bf16_parity, assert_f32_parity, dev, dev_bf16, host_bits, say)

binding = pytest.importorskip("head_latent_attention_fp32_amd.binding")

pytestmark = pytest.mark.gpu
SCALE = 192 ** -0.5


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    binding.lib()


# ----------------------------------------------------------------------------------- kv side
def _kv_append_case(B, T, max_seqlen, start, packed, seed):
    rng = np.random.default_rng(seed)
    n = B * T
    inp = S.kv_side_inputs(n, seed, 500 + B + T)
    pos = (np.asarray(start)[:, None] + np.arange(T)[None]).reshape(-1)
    cs = S.rope_table(np.maximum(pos, 0)).reshape(B, T, 32, 2)
    if packed:
        offs = np.concatenate([[0], np.cumsum(np.full(B, max_seqlen + 3))[:-1]]).astype(np.int64)
        rows = int(offs[-1]) + max_seqlen + 3
    else:
        offs = np.arange(B, dtype=np.int64) * max_seqlen
        rows = B * max_seqlen
    kv = S.f32_to_bf16_bits(rng.standard_normal((rows, 512)).astype(np.float32))
    pe = S.f32_to_bf16_bits(rng.standard_normal((rows, 64)).astype(np.float32))
    return inp, cs, offs, kv, pe


@pytest.mark.parametrize("B,T,max_seqlen,start,packed", [
    (3, 5, 16, [0, 7, 13], False),          # the last sequence's tokens 3, 4 fall past the cache
    (2, 1, 9, [8, 0], True),
    (32, 1, 4096, list(range(4064, 4096)), False),
    (1, 300, 512, [100], True),
])
def test_kv_append_parity(B, T, max_seqlen, start, packed):
    say(f"kv_append B={B} T={T} max_seqlen={max_seqlen} packed={packed}")
    inp, cs, offs, kv, pe = _kv_append_case(B, T, max_seqlen, start, packed, seed=B * 100 + T)
    kv_d, pe_d = dev_bf16(kv), dev_bf16(pe)
    binding.kv_append(dev_bf16(inp["kv_a"].reshape(B, T, 576)), dev(inp["kv_gamma"]), dev(cs),
                      dev(np.asarray(start, np.int32)), kv_d, pe_d, max_seqlen,
                      cache_row_offset=dev(offs) if packed else None)
    torch.cuda.synchronize()
    kv_g, pe_g = host_bits(kv_d), host_bits(pe_d)
    lat, kpe = O.kv_side(inp["kv_a"], inp["kv_gamma"], cs.reshape(-1, 32, 2), staged=False)
    written = np.zeros(kv.shape[0], bool)
    rows, src = [], []
    for b in range(B):
        for t in range(T):
            p = start[b] + t
            if 0 <= p < max_seqlen:
                rows.append(int(offs[b]) + p)
                src.append(b * T + t)
    written[rows] = True
    np.testing.assert_array_equal(kv_g[~written], kv[~written])
    np.testing.assert_array_equal(pe_g[~written], pe[~written])
    assert_bf16_parity(kv_g[rows], lat[src], "latent rows")
    assert_bf16_parity(pe_g[rows], kpe[src], "rotary key rows")


def test_append_then_decode_on_own_caches():
    """One decode step after appending each sequence's newest token: the library writes the row
    and then attends over it; the oracle does the same with its own rows."""
    B, H, Lmax = 4, 64, 300
    lens_before = np.array([0, 1, 150, 299], np.int32)
    seed = 7
    rng = np.random.default_rng(seed)
    kv = S.f32_to_bf16_bits(rng.standard_normal((B * Lmax, 512)).astype(np.float32))
    pe = S.f32_to_bf16_bits(rng.standard_normal((B * Lmax, 64)).astype(np.float32))
    offs = np.arange(B, dtype=np.int64) * Lmax
    inp = S.kv_side_inputs(B, seed, 601)
    cs = S.rope_table(lens_before).reshape(B, 1, 32, 2)
    w = S.kv_weights(H, seed, 601)
    q = S.normal_bf16_rows(B, H * 192, 1.0, (seed, 601, S.T_Q)).reshape(B, H, 192)
    kv_d, pe_d = dev_bf16(kv), dev_bf16(pe)
    binding.kv_append(dev_bf16(inp["kv_a"].reshape(B, 1, 576)), dev(inp["kv_gamma"]), dev(cs),
                      dev(lens_before), kv_d, pe_d, Lmax)
    lens = lens_before + 1
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out, _ = binding.decode(dev_bf16(q), dev_bf16(w), kv_d, pe_d, dev(lens), Lmax, lse=lse)
    torch.cuda.synchronize()
    lat, kpe = O.kv_side(inp["kv_a"], inp["kv_gamma"], cs.reshape(B, 32, 2), staged=True)
    kv_o, pe_o = O.cache_append(kv, pe, offs, lens_before, O.bf16_encode(lat)[:, None],
                                O.bf16_encode(kpe)[:, None], Lmax)
    oo, lo = O.decode_batch(O.bf16_decode(q), w, kv_o, pe_o, offs, lens, SCALE, round_output=False)
    assert_bf16_parity(host_bits(out), oo, "decode out")
    qv = O.bf16_decode(q)
    mag = np.stack([O.decode_score_magnitude(qv[b], w, kv_o[offs[b]:offs[b] + lens[b]],
                                             pe_o[offs[b]:offs[b] + lens[b]], SCALE) for b in range(B)])
    assert_f32_parity(lse.cpu().numpy(), lo, "decode lse", magnitude=mag)


# ----------------------------------------------------------------------------------- prefix prefill
def _run_prefix(q_bits, lat, kpe, w, H):
    B, Tq = q_bits.shape[:2]
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device="cuda")
    out, _ = binding.prefill_with_prefix(dev_bf16(q_bits), dev_bf16(lat), dev_bf16(kpe), dev_bf16(w), lse=lse)
    torch.cuda.synchronize()
    return host_bits(out), lse.cpu().numpy()


@pytest.mark.parametrize("H,B,Tq,Skv", [(16, 1, 1, 1), (16, 2, 5, 70), (64, 1, 64, 164), (32, 1, 130, 257),
                                        (128, 1, 65, 300), (16, 1, 1, 513), (64, 2, 200, 200)])
def test_prefill_with_prefix_parity(H, B, Tq, Skv):
    say(f"prefill_with_prefix H={H} B={B} q_len={Tq} kv_len={Skv}")
    case = S.PrefillCase("t", 700 + H + Tq + Skv, H, B, Skv)
    d = S.prefill_inputs(case, seed=5, with_q_latent=False)
    q = S.prefill_query(case, seed=5)[:, Skv - Tq:].copy()
    out, lse = _run_prefix(q, d["kv_latent"], d["k_pe"], d["wkv_b"], H)
    for b in range(B):
        qv = O.bf16_decode(q[b])
        oo, lo = O.prefill_causal(qv, d["kv_latent"][b], d["k_pe"][b], d["wkv_b"], SCALE, round_output=False)
        assert_bf16_parity(out[b], oo, f"out[b={b}]")
        mag = O.prefill_score_magnitude(qv, d["kv_latent"][b], d["k_pe"][b], d["wkv_b"], SCALE)
        assert_f32_parity(lse[b], lo, f"lse[b={b}]", magnitude=mag)


@pytest.mark.slow
def test_prefill_with_prefix_chunk_of_4096_sampled():
    """The second half of the 4096-token prefill as a chunk over its 2048-position prefix."""
    H, S_, Tq = 128, 4096, 2048
    case = S.PrefillCase("chunk", 2, H, 1, S_)
    d = S.prefill_inputs(case, seed=0, with_q_latent=False)
    q = S.prefill_query(case, seed=0)[:, S_ - Tq:].copy()
    say(f"prefill_with_prefix H={H} q_len={Tq} kv_len={S_}: oracle on sampled rows and heads")
    out, lse = _run_prefix(q, d["kv_latent"], d["k_pe"], d["wkv_b"], H)
    rows, heads = [0, 1, 63, 64, 1000, 2046, 2047], [0, 50, 127]
    qv = O.bf16_decode(q[0])
    oo, lo = O.prefill_causal(qv, d["kv_latent"][0], d["k_pe"][0], d["wkv_b"], SCALE, heads=heads, rows=rows,
                              round_output=False)
    assert_bf16_parity(out[0][rows][:, heads], oo, "out")
    mag = O.prefill_score_magnitude(qv, d["kv_latent"][0], d["k_pe"][0], d["wkv_b"], SCALE, heads=heads, rows=rows)
    assert_f32_parity(lse[0][heads][:, rows], lo, "lse", magnitude=mag)


def test_chunked_prefill_on_own_cache():
    """Two chunks of one sequence: kv_append writes each chunk's rows into the cache, and each
    chunk's prefill reads the cache's first kv_len rows; both chunks match the oracle's whole
    prefill rows."""
    H, S_, c1 = 32, 200, 120
    seed = 11
    inp = S.kv_side_inputs(S_, seed, 801)
    cs = S.rope_table(np.arange(S_))
    w = S.kv_weights(H, seed, 801)
    q = S.normal_bf16_rows(S_, H * 192, 1.0, (seed, 801, S.T_Q)).reshape(1, S_, H, 192)
    kv_d = torch.zeros((S_, 512), dtype=torch.bfloat16, device="cuda")
    pe_d = torch.zeros((S_, 64), dtype=torch.bfloat16, device="cuda")
    outs = []
    for a, b in [(0, c1), (c1, S_)]:
        binding.kv_append(dev_bf16(inp["kv_a"][a:b].reshape(1, b - a, 576)), dev(inp["kv_gamma"]),
                          dev(cs[a:b].reshape(1, b - a, 32, 2)), dev(np.array([a], np.int32)), kv_d, pe_d, S_)
        o, _ = binding.prefill_with_prefix(dev_bf16(q[:, a:b]), kv_d[:b].reshape(1, b, 512),
                                           pe_d[:b].reshape(1, b, 64), dev_bf16(w))
        outs.append(host_bits(o)[0])
    torch.cuda.synchronize()
    lat, kpe = O.kv_side(inp["kv_a"], inp["kv_gamma"], cs, staged=True)
    oo, _ = O.prefill_causal(O.bf16_decode(q[0]), O.bf16_encode(lat), O.bf16_encode(kpe), w, SCALE,
                             round_output=False)
    assert_bf16_parity(np.concatenate(outs), oo, "chunked prefill out")


# ----------------------------------------------------------------------------------- top-k decode
def _selected(idx, L):
    idx = np.asarray(idx, np.int64)
    return np.unique(idx[(idx >= 0) & (idx < L)])


def _check_sparse(case, q_bits, d, topk, out_bits, lse, ids):
    qv = O.bf16_decode(q_bits)
    lens = np.clip(d["lengths"].astype(np.int64), 0, int(case.max_seqlen))
    oo, lo = O.decode_topk_batch(qv, d["wkv_b"], d["kv_cache"], d["pe_cache"], d["row_offset"], lens, topk, SCALE,
                                 batch_ids=ids, round_output=False)
    assert_bf16_parity(out_bits[ids], oo, "out")
    mags = []
    for b in ids:
        r0 = int(d["row_offset"][b])
        rows = r0 + _selected(topk[b], lens[b])
        mags.append(O.decode_score_magnitude(qv[b], d["wkv_b"], d["kv_cache"][rows], d["pe_cache"][rows], SCALE))
    assert_f32_parity(lse[ids], lo, "lse", magnitude=np.stack(mags))


def _run_sparse(case, q_bits, d, topk):
    B, H = case.batch, case.n_heads
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out, _ = binding.decode_sparse(dev_bf16(q_bits), dev_bf16(d["wkv_b"]), dev_bf16(d["kv_cache"]),
                                   dev_bf16(d["pe_cache"]), dev(d["lengths"]), int(case.max_seqlen),
                                   dev(np.ascontiguousarray(topk, np.int32)),
                                   cache_row_offset=None if case.layout == "padded" else dev(d["row_offset"]), lse=lse)
    torch.cuda.synchronize()
    return host_bits(out), lse.cpu().numpy()


SPARSE_SMALL = [
    (16, [1], 1, "padded"), (64, [100], 33, "padded"), (64, [40, 0, 300], 64, "padded"),
    (128, [1000, 2, 64], 200, "packed"), (32, [500, 37], 37, "packed"), (128, [5000], 2048, "padded"),
]


@pytest.mark.parametrize("H,lens,k,layout", SPARSE_SMALL)
def test_decode_sparse_parity(H, lens, k, layout):
    say(f"decode_sparse H={H} lens={lens} k={k} layout={layout}")
    case = S.DecodeCase("t", 900 + H + len(lens) + k, H, np.array(lens, np.int32), layout=layout,
                        max_seqlen=max(max(lens), 1))
    d = S.decode_inputs(case, seed=9, with_q_latent=False)
    q = S.decode_query(case, seed=9)
    topk = S.topk_indices(case.lengths, k, seed=9, case_id=case.case_id)
    # entries that name no position: past the sequence (the padding rows hold NaN) and negative
    rng = np.random.default_rng(k)
    for b, L in enumerate(lens):
        free = np.flatnonzero(topk[b] == -1)
        bad = np.array([L, L + 1, L + 1000, -5, 2 ** 31 - 1], np.int64)
        topk[b, free[: len(bad)]] = bad[: len(free)]
        rng.shuffle(topk[b])
    out, lse = _run_sparse(case, q, d, topk)
    _check_sparse(case, q, d, topk, out, lse, list(range(case.batch)))


@pytest.mark.parametrize("H,B", [(16, 300), (64, 1000)])
def test_decode_sparse_many_sequences(H, B):
    """More than 256 sequences in top-k mode: the run plan's chunked branch over the compacted
    counts; every 7th sequence is empty and lists are padded with -1 past the sequence."""
    lens = [0 if i % 7 == 0 else (89 * i + 5) % 311 for i in range(B)]
    say(f"decode_sparse H={H} B={B} k=64")
    case = S.DecodeCase("t", 960 + H + B, H, np.array(lens, np.int32), layout="packed")
    d = S.decode_inputs(case, seed=12, with_q_latent=False)
    q = S.decode_query(case, seed=12)
    topk = S.topk_indices(case.lengths, 64, seed=12, case_id=case.case_id)
    out, lse = _run_sparse(case, q, d, topk)
    _check_sparse(case, q, d, topk, out, lse, list(range(B)))


def test_decode_sparse_empty_lists_and_full_lists():
    case = S.DecodeCase("t", 950, 64, np.array([0, 50, 7], np.int32), max_seqlen=50)
    d = S.decode_inputs(case, seed=10, with_q_latent=False)
    q = S.decode_query(case, seed=10)
    # k = 0: nothing selected anywhere
    out, lse = _run_sparse(case, q, d, np.zeros((3, 0), np.int32))
    assert np.all(O.bf16_decode(out) == 0) and np.all(np.isneginf(lse))
    # every position listed: the dense decode
    topk = S.topk_indices(case.lengths, 50, seed=10, case_id=950)
    out_s, lse_s = _run_sparse(case, q, d, topk)
    lse_d = torch.empty((3, 64), dtype=torch.float32, device="cuda")
    out_d, _ = binding.decode(dev_bf16(q), dev_bf16(d["wkv_b"]), dev_bf16(d["kv_cache"]), dev_bf16(d["pe_cache"]),
                              dev(d["lengths"]), 50, lse=lse_d)
    torch.cuda.synchronize()
    _check_sparse(case, q, d, topk, out_s, lse_s, [0, 1, 2])
    np.testing.assert_allclose(O.bf16_decode(out_s), O.bf16_decode(host_bits(out_d)), rtol=0, atol=0.05)


@pytest.mark.parametrize("H,k,max_seqlen", [(16, 64, 300), (128, 300, 300), (64, 3000, 300), (16, 64, 600000),
                                          (64, 3000, 600000)])
def test_decode_sparse_repeated_positions(H, k, max_seqlen):
    """A position listed more than once is attended once ([AU] mla-decode: the index mask is a
    scatter of 0 into -inf). Lists mix distinct positions, repeats of them, -1 and positions past
    the sequence; the result matches the oracle's mask, and is bit-identical to the run on the same
    lists with every repeat after the first replaced by -1 (the compacted lists are the same).
    max_seqlen 300: the positions' bitmap; 600000 (packed caches, the same short sequences): the
    first-entry table, in LDS for k = 64 and in the workspace for k = 3000."""
    lens = [97, 300, 1, 64, 0, 250]
    say(f"decode_sparse repeated positions H={H} k={k} max_seqlen={max_seqlen}")
    case = S.DecodeCase("t", 970 + H + k, H, np.array(lens, np.int32),
                        layout="padded" if max_seqlen == 300 else "packed", max_seqlen=max_seqlen)
    d = S.decode_inputs(case, seed=13, with_q_latent=False)
    q = S.decode_query(case, seed=13)
    rng = np.random.default_rng(97 + k)
    topk = np.full((len(lens), k), -1, np.int32)
    for b, L in enumerate(lens):
        if L == 0:
            topk[b, : k // 2] = rng.integers(0, 5, k // 2)   # names nothing: the sequence is empty
            continue
        n = min(L, k // 3)
        base = rng.choice(L, n, replace=False)
        rep = rng.choice(base, k - n - 4)                      # repeats of listed positions
        row = np.concatenate([base, rep, [-1, L, L + 7, -3]])
        rng.shuffle(row)
        topk[b] = row.astype(np.int32)
    topk[2, :] = 0                                             # one position, listed k times
    out, lse = _run_sparse(case, q, d, topk)
    _check_sparse(case, q, d, topk, out, lse, list(range(case.batch)))
    first = topk.copy()
    for b in range(len(lens)):
        seen = set()
        for j, x in enumerate(first[b]):
            if x in seen:
                first[b, j] = -1
            elif 0 <= x < lens[b]:
                seen.add(int(x))
    out1, lse1 = _run_sparse(case, q, d, first)
    assert np.array_equal(out, out1), "repeats changed the result beyond dropping them"
    assert np.array_equal(lse.view(np.uint32), lse1.view(np.uint32))


@pytest.mark.slow
def test_decode_sparse_config1_top2048_sampled():
    """32 sequences of 4096 cached positions, 2048 of them selected per sequence."""
    case = S.workload(1)
    d = S.decode_inputs(case, seed=0, with_q_latent=False)
    q = S.decode_query(case, seed=0)
    topk = S.topk_indices(case.lengths, 2048, seed=0, case_id=case.case_id)
    say(f"decode_sparse {case.name} k=2048: oracle on sequences 0, 13, 31")
    out, lse = _run_sparse(case, q, d, topk)
    _check_sparse(case, q, d, topk, out, lse, [0, 13, 31])


# ----------------------------------------------------------------------------------- output projection
def _run_out_proj(x_bits, wo_bits):
    y = binding.output_proj(dev_bf16(x_bits), dev_bf16(wo_bits))
    torch.cuda.synchronize()
    return host_bits(y)


@pytest.mark.parametrize("H,n,dim", [(16, 1, 64), (16, 5, 320), (32, 16, 1024), (128, 32, 7168), (64, 33, 512),
                                     (16, 64, 192), (16, 65, 320), (32, 300, 704), (16, 513, 256),
                                     (128, 128, 7168), (64, 100, 1024)])
def test_output_proj_parity(H, n, dim):
    say(f"output_proj H={H} n={n} dim={dim}")
    x = S.head_outputs(n, H, seed=12, case_id=1000 + n)
    wo = S.wo_weights(H, seed=12, case_id=1000 + n, dim=dim, workers=S.default_workers())
    y = _run_out_proj(x, wo)
    assert_bf16_parity(y, O.output_proj(x, wo, staged=False), "y")


@pytest.mark.slow
def test_output_proj_prefill_4096_sampled():
    H, n, dim = 128, 4096, 7168
    say(f"output_proj H={H} n={n} dim={dim}: oracle on sampled tokens")
    x = S.head_outputs(n, H, seed=0, case_id=2, workers=S.default_workers())
    wo = S.wo_weights(H, seed=0, case_id=2, dim=dim, workers=S.default_workers())
    y = _run_out_proj(x, wo)
    rows = [0, 1, 255, 256, 2047, 4000, 4095]
    assert_bf16_parity(y[rows], O.output_proj(x[rows], wo, staged=False), "y rows")


def test_decode_then_output_proj():
    """A decode step's head outputs projected by wo: the composition the attention update is."""
    case = S.DecodeCase("t", 1100, 64, np.array([300, 7], np.int32), max_seqlen=300)
    d = S.decode_inputs(case, seed=13, with_q_latent=False)
    q = S.decode_query(case, seed=13)
    wo = S.wo_weights(64, seed=13, case_id=1100, dim=512)
    out, _ = binding.decode(dev_bf16(q), dev_bf16(d["wkv_b"]), dev_bf16(d["kv_cache"]), dev_bf16(d["pe_cache"]),
                            dev(d["lengths"]), 300)
    y = binding.output_proj(out, dev_bf16(wo))
    torch.cuda.synchronize()
    oo, _ = O.decode_batch(O.bf16_decode(q), d["wkv_b"], d["kv_cache"], d["pe_cache"], d["row_offset"],
                           d["lengths"], SCALE)
    assert_bf16_parity(host_bits(y), O.output_proj(O.bf16_encode(oo), wo, staged=False), "attention update")
