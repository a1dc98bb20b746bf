"""A decode step captured in a HIP graph and replayed: the query path on packed weights, then
mla_decode_noalloc (the entry point for callers that cannot allocate, code under graph capture
among them) and mla_decode with a caller workspace. The library enqueues kernels only -- no
allocation, memset or synchronisation -- so the step captures as it is; every replay must give,
bit for bit, what the same calls gave eagerly, also after eager calls on other inputs between the
replays have overwritten the outputs and the no-alloc scratch."""
import numpy as np
import pytest
import torch

from synth import inputs as S
from tests.gpu_helpers import dev, dev_bf16, host_bits, say

binding = pytest.importorskip("head_latent_attention_fp32_amd.binding")

pytestmark = pytest.mark.gpu


def _inputs(H, lens, case_id, seed):
    case = S.DecodeCase("graph", case_id, H, np.array(lens, np.int32), layout="packed", max_seqlen=max(lens))
    d = S.decode_inputs(case, seed=seed)
    t = {"x": dev_bf16(d["q_latent"]), "gamma": dev(d["gamma"]), "wq_b": dev_bf16(d["wq_b"]),
         "cs": dev(d["rope_cs"]), "wkv_b": dev_bf16(d["wkv_b"]), "kv": dev_bf16(d["kv_cache"]),
         "pe": dev_bf16(d["pe_cache"]), "lens": dev(d["lengths"]), "off": dev(d["row_offset"])}
    t["wq_packed"] = binding.wq_b_pack(t["wq_b"], H)
    return case, t


def test_decode_step_replays_from_a_hip_graph():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    binding.lib()
    H, lens = 64, [700, 1, 0, 313, 96]
    B = len(lens)
    say(f"graph capture of a decode step H={H} B={B}")
    case, t = _inputs(H, lens, 980, 31)
    max_seqlen = int(case.max_seqlen)
    q = torch.empty((B, H, 192), dtype=torch.bfloat16, device="cuda")
    out_n = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    out_w = torch.empty_like(out_n)
    lse_n = torch.empty((B, H), dtype=torch.float32, device="cuda")
    lse_w = torch.empty_like(lse_n)
    ws = torch.empty(binding.decode_workspace_size(H, B, max_seqlen), dtype=torch.uint8, device="cuda")

    def step(src, q_, on, ln, ow, lw):
        binding.query_path(src["x"], src["gamma"], src["wq_packed"], src["cs"], H, q_out=q_, packed=True)
        binding.decode_noalloc(q_, src["wkv_b"], src["kv"], src["pe"], src["lens"], max_seqlen,
                               cache_row_offset=src["off"], out=on, lse=ln)
        binding.decode(q_, src["wkv_b"], src["kv"], src["pe"], src["lens"], max_seqlen, cache_row_offset=src["off"],
                       workspace=ws, out=ow, lse=lw)

    # eager reference (the first no-alloc call also looks up the scratch address, outside the capture)
    step(t, q, out_n, lse_n, out_w, lse_w)
    torch.cuda.synchronize()
    want = [host_bits(q), host_bits(out_n), lse_n.cpu().numpy().view(np.uint32), host_bits(out_w),
            lse_w.cpu().numpy().view(np.uint32)]
    assert np.array_equal(want[1], want[3]) and np.array_equal(want[2], want[4])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(t, q, out_n, lse_n, out_w, lse_w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(t, q, out_n, lse_n, out_w, lse_w)
    torch.cuda.synchronize()

    # other inputs for the eager calls between the replays (same shapes, other values)
    _, t2 = _inputs(H, lens, 981, 32)
    q2, o2n, o2w = torch.empty_like(q), torch.empty_like(out_n), torch.empty_like(out_w)
    l2n, l2w = torch.empty_like(lse_n), torch.empty_like(lse_w)
    for rep in range(4):
        for buf in (q, out_n, out_w):
            buf.fill_(0)
        lse_n.fill_(0.0)
        lse_w.fill_(0.0)
        step(t2, q2, o2n, l2n, o2w, l2w)   # eager work that rewrites the scratch and the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host_bits(q), host_bits(out_n), lse_n.cpu().numpy().view(np.uint32), host_bits(out_w),
               lse_w.cpu().numpy().view(np.uint32)]
        for name, a, b in zip(("q", "out (no-alloc)", "lse (no-alloc)", "out (workspace)", "lse (workspace)"),
                              got, want):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs from the eager step"
        say(f"  replay {rep}: bit-identical to the eager step")
    assert not np.array_equal(host_bits(o2n), want[1]), "the eager calls between replays used other inputs"
