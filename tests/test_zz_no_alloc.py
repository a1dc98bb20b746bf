"""mla_decode_noalloc (decode on the library's fixed device scratch, for callers that cannot
allocate) against mla_decode with a caller workspace, through the C ABI: two calls in a row, the
second on a smaller batch (the scratch keeps the first call's contents), each compared with
mla_decode on the same inputs -- the same kernels, so the outputs must agree bit for bit -- and
with the oracle to the parity bar."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from synth import inputs as S
from tests.gpu_helpers import assert_bf16_parity, assert_f32_parity, dev, dev_bf16, host_bits, say

binding = pytest.importorskip("head_latent_attention_fp32_amd.binding")

pytestmark = pytest.mark.gpu
SCALE = 192 ** -0.5


def _case(H, lens, layout, case_id, seed):
    case = S.DecodeCase("t", case_id, H, np.array(lens, np.int32), layout=layout, max_seqlen=max(max(lens), 1))
    d = S.decode_inputs(case, seed=seed, with_q_latent=False)
    q = S.decode_query(case, seed=seed)
    return case, d, q


def _both(case, d, q):
    B, H = case.batch, case.n_heads
    args = (dev_bf16(q), dev_bf16(d["wkv_b"]), dev_bf16(d["kv_cache"]), dev_bf16(d["pe_cache"]), dev(d["lengths"]),
            int(case.max_seqlen))
    off = None if case.layout == "padded" else dev(d["row_offset"])
    lse_n = torch.full((B, H), 7.0, dtype=torch.float32, device="cuda")
    out_n, _ = binding.decode_noalloc(*args, cache_row_offset=off, lse=lse_n)
    torch.cuda.synchronize()
    lse_w = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out_w, _ = binding.decode(*args, cache_row_offset=off, lse=lse_w)
    torch.cuda.synchronize()
    return host_bits(out_n), lse_n.cpu().numpy(), host_bits(out_w), lse_w.cpu().numpy()


def test_noalloc_decode_matches_workspace_decode_on_two_calls():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    binding.lib()
    calls = [
        (128, [4096, 1, 0, 2500, 700] + [(37 * i) % 900 + 1 for i in range(35)], "packed", 970, 21),
        (64, [300, 0, 45], "padded", 971, 22),   # smaller: fewer sequences, heads and runs
    ]
    for H, lens, layout, cid, seed in calls:
        say(f"decode_noalloc H={H} B={len(lens)} layout={layout}")
        case, d, q = _case(H, lens, layout, cid, seed)
        out_n, lse_n, out_w, lse_w = _both(case, d, q)
        assert np.array_equal(out_n, out_w), "outputs differ from mla_decode with a workspace"
        assert np.array_equal(lse_n, lse_w), "lse differs from mla_decode with a workspace"
        ids = list(range(case.batch))
        lens_c = np.clip(d["lengths"].astype(np.int64), 0, int(case.max_seqlen))
        oo, lo = O.decode_batch(O.bf16_decode(q), d["wkv_b"], d["kv_cache"], d["pe_cache"], d["row_offset"], lens_c,
                                SCALE, staged=True, round_output=False)
        assert_bf16_parity(out_n, oo, "out")
        qv = O.bf16_decode(q)
        mag = np.stack([O.decode_score_magnitude(qv[b], d["wkv_b"], d["kv_cache"][r0:r0 + L], d["pe_cache"][r0:r0 + L],
                                                 SCALE)
                        for b, r0, L in zip(ids, d["row_offset"].astype(np.int64), lens_c)])
        assert_f32_parity(lse_n, lo, "lse", magnitude=mag)


def test_noalloc_decode_rejects_batches_beyond_the_scratch():
    binding.lib()
    H, B, max_seqlen = 128, 4096, 4096
    need = binding.decode_workspace_size(H, B, max_seqlen)
    assert need > binding.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, 192), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((H * 256, 512), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((16, 512), dtype=torch.bfloat16, device="cuda")
    pe = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    off = torch.zeros(B, dtype=torch.int64, device="cuda")
    with pytest.raises(binding.MlaError) as e:
        binding.decode_noalloc(q, w, kv, pe, lens, max_seqlen, cache_row_offset=off)
    assert e.value.status == 5
