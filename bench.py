"""Benchmark of the MLA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads 3,0,1,4] [--no-prefill]
                    [--no-next] [--no-cpu] [--no-peaks] [--query-weights packed|stored]

A step is one pass of the decode hot path over one batch of a decode workload: the query path on
the batch's new tokens, then mla_decode (absorb, split-KV attention, log-sum-exp combine, value
projection). The query path reads wq_b rearranged once by mla_wq_b_pack, as a model would do when
it loads its weights (mla_query_path_packed; --query-weights stored times mla_query_path on wq_b as
stored instead); the rearrangement is not part of a step. Inputs are synthetic (seeded) and resident in HBM before the timed region; workloads
whose inputs fit the 256 MB Infinity Cache rotate copies of every input so that a step never finds
the previous step's data there.

The headline is the first workload of --workloads (default: the ragged batch, 128 sequences of
256..32768 cached tokens at 128 heads, the largest decode configuration); the other decode
workloads (Kimi-K2 B = 1 x 1000 at 64 heads, DeepSeek-V3.2 32 x 4096, 8 x 131072 with spikes) are
measured in the same run and reported under "decode_workloads".

The printed JSON line carries:
  value       whole-job decode throughput of the headline workload, cache-token.heads/s =
              H * sum(L_b) / step time
  roofline    the split-KV attention kernel (the dominant kernel): algorithmic bytes per launch
              (1152 B per cached token: 512 latent + 64 rotary bf16) / its mean duration, timed with
              HIP events recorded on its own stream around that kernel, against 8 TB/s, and against
              the stream-read rate measured in the same process (`peaks`); `traffic` is the HBM
              bytes per launch measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE, scaled by a
              copy-kernel calibration) as committed under profiles/, or null when the kernel source
              has changed since (checked by hash)
  peaks       achievable rates measured in this process: a plain streaming read of 4 GiB and a loop
              of independent bf16 MFMAs on every SIMD
  decode_workloads  the same record (step, stages, attention roofline, oracle baseline) for every
              decode workload
  prefill     the DeepSeek-V3.2-shaped prefill (T = 4096, 128 heads): query path + expansion +
              causal attention, TFLOP/s of algorithmic flops against 2.5 PFLOP/s bf16, with an
              oracle sample
  cpu_baseline the CPU oracle on a bounded sample of the headline workload (whole sequences, one at
              a time), with the host's CPU model, core count and NumPy's BLAS
  next_rows   the steps next to the path, each with its time, roofline fraction and an oracle
              sample: mla_kv_append (32 decode / 4096 prefill tokens), mla_decode_sparse (the
              32 x 4096 workload with 2048 of 4096 positions per sequence), mla_prefill_with_prefix
              (the last 2048 of the 4096 prefill positions over the first 2048), mla_output_proj (wo
              7168 x 16384 after 32 and 4096 tokens)

    python bench.py --copy-calibration MIB   only runs a plain device copy of MIB MiB (for scaling
                                             the rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
BYTES_PER_CACHED_TOKEN = (512 + 64) * 2
METRIC = "MLA decode cache-tokens·heads/s + HBM GB/s; prefill TFLOP/s (% of peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SRC = os.path.join(ROOT, "head_latent_attention_fp32_amd", "csrc", "decode.hip")
PEAKS_LIB = os.path.join(ROOT, "head_latent_attention_fp32_amd", "libmla_peaks.so")


class HipEvents:
    """Raw hipEvent_t handles (created up front, so the library can record them). They are created
    without the system-scope fence on record, which otherwise adds microseconds to every stage."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE)) == 0
            self.ev[i] = h.value

    def ptr(self, i):
        return ctypes.cast(ctypes.byref(self.ev, i * ctypes.sizeof(ctypes.c_void_p)), ctypes.POINTER(ctypes.c_void_p))

    def ms(self, a, b):
        f = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(self.ev[a]), ctypes.c_void_p(self.ev[b])) == 0
        return f.value


def to_dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def decode_bench(args, torch, binding, S, workload):
    case = S.workload(workload)
    B, H = case.batch, case.n_heads
    log(f"[bench] generating {case.name} (B={B}, H={H}, sum L={int(case.lengths.sum())})")
    d = S.decode_inputs(case, seed=0)
    L = binding.lib()
    dims = binding.dims(H)
    # copies rotated so that the inputs of the steps in flight never fit the 256 MB Infinity Cache
    # together: enough copies for about 1 GB, at most --copies (one when a single copy is larger)
    one = sum(int(d[k].nbytes) for k in ("q_latent", "wq_b", "wkv_b", "kv_cache", "pe_cache"))
    n_copies = int(max(1, min(args.copies, -(-(1 << 30) // one))))
    sets = []
    base = {
        "q_latent": to_dev_bf16(torch, d["q_latent"]), "gamma": torch.from_numpy(d["gamma"]).cuda(),
        "wq_b": to_dev_bf16(torch, d["wq_b"]), "rope_cs": torch.from_numpy(d["rope_cs"]).cuda(),
        "wkv_b": to_dev_bf16(torch, d["wkv_b"]), "kv": to_dev_bf16(torch, d["kv_cache"]),
        "pe": to_dev_bf16(torch, d["pe_cache"]), "lens": torch.from_numpy(d["lengths"]).cuda(),
        "off": torch.from_numpy(d["row_offset"]).cuda(),
    }
    for i in range(n_copies):
        sets.append({k: (v if i == 0 else v.clone()) for k, v in base.items()})
    qpath = L.mla_query_path_ex
    if args.query_weights == "packed":
        # the query weights rearranged once, as at model load (mla_wq_b_pack), outside every timed step
        for s_ in sets:
            s_["wq_b"] = binding.wq_b_pack(s_["wq_b"], H)
        qpath = L.mla_query_path_packed_ex
        torch.cuda.synchronize()
    ws_bytes = binding.decode_workspace_size(H, B, int(case.max_seqlen))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    q = torch.empty((B, H, 192), dtype=torch.bfloat16, device="cuda")
    inv = torch.empty(B, dtype=torch.float32, device="cuda")
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    qws_bytes = binding.query_path_workspace_size(H, B)
    qws = torch.empty(max(qws_bytes, 1), dtype=torch.uint8, device="cuda")
    qws_ptr = qws.data_ptr() if qws_bytes else None
    stream = torch.cuda.current_stream().cuda_stream
    packed = case.layout == "packed"
    K, W = args.steps, args.warmup
    evq = HipEvents(3 * K)
    evd = HipEvents(4 * K)
    P = ctypes.POINTER(ctypes.c_void_p)
    # Timed steps record two events, around the attention stage only (each event on the stream costs
    # about 2 us of GPU time); the per-stage breakdown comes from a separate instrumented pass.
    attn_ev = [ctypes.cast((ctypes.c_void_p * 4)(None, evd.ev[4 * k + 1], evd.ev[4 * k + 2], None), P)
               for k in range(K)]

    def step(i, timed, all_stages=False):
        s = sets[i % n_copies]
        eq = evq.ptr(3 * (i - W)) if (timed and all_stages) else None
        ed = (evd.ptr(4 * (i - W)) if all_stages else attn_ev[i - W]) if timed else None
        st = qpath(ctypes.byref(dims), B, s["q_latent"].data_ptr(), s["gamma"].data_ptr(),
                   s["wq_b"].data_ptr(), s["rope_cs"].data_ptr(), q.data_ptr(), inv.data_ptr(),
                   qws_ptr, qws_bytes, stream, eq)
        assert st == 0, st
        st = L.mla_decode_ex(ctypes.byref(dims), B, q.data_ptr(), s["wkv_b"].data_ptr(), s["kv"].data_ptr(),
                             s["pe"].data_ptr(), s["off"].data_ptr() if packed else None, s["lens"].data_ptr(),
                             int(case.max_seqlen), ws.data_ptr(), ws_bytes, out.data_ptr(), lse.data_ptr(),
                             stream, ed)
        assert st == 0, st

    L.mla_query_path_ex.argtypes = list(L.mla_query_path.argtypes) + [ctypes.POINTER(ctypes.c_void_p)]
    L.mla_query_path_packed_ex.argtypes = list(L.mla_query_path.argtypes) + [ctypes.POINTER(ctypes.c_void_p)]
    L.mla_decode_ex.argtypes = list(L.mla_decode.argtypes) + [ctypes.POINTER(ctypes.c_void_p)]
    for i in range(W):
        step(i, False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(W, W + K):
        step(i, True)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms = total_ms / K
    attn_ms = float(np.mean([evd.ms(4 * k + 1, 4 * k + 2) for k in range(K)]))
    # instrumented pass (not timed as a whole): every stage boundary recorded, then two events back to
    # back after the step: the span an event pair itself adds between two kernels
    eve = HipEvents(2 * K)
    for i in range(W, W + K):
        step(i, True, all_stages=True)
        k = i - W
        eve.hip.hipEventRecord(ctypes.c_void_p(eve.ev[2 * k]), ctypes.c_void_p(stream))
        eve.hip.hipEventRecord(ctypes.c_void_p(eve.ev[2 * k + 1]), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    pair_ms = float(np.mean([eve.ms(2 * k, 2 * k + 1) for k in range(K)]))
    stage_q = np.array([[evq.ms(3 * k + j, 3 * k + j + 1) for j in range(2)] for k in range(K)]).mean(0)
    stage_d = np.array([[evd.ms(4 * k + j, 4 * k + j + 1) for j in range(3)] for k in range(K)]).mean(0)
    tokens = int(np.clip(case.lengths, 0, case.max_seqlen).sum())
    alg_cache = tokens * BYTES_PER_CACHED_TOKEN
    alg_decode = alg_cache + 2 * H * 128 * 512 * 2 + B * H * (192 + 128) * 2
    alg_query = 1536 * H * 192 * 2 + B * 1536 * 2 + B * H * 192 * 2
    decode_ms = ms - float(stage_q.sum()) * (ms / float(stage_q.sum() + stage_d.sum()))
    res = {
        "case": case, "ms": ms, "tokens": tokens, "H": H, "B": B, "copies": n_copies,
        "value": H * tokens / (ms * 1e-3),
        "attn_ms": attn_ms,
        "event_pair_ms": pair_ms,
        "stages_ms": {"query_stats": float(stage_q[0]), "query_gemm_rope": float(stage_q[1]),
                      "absorb_plan": float(stage_d[0]), "split_kv_attention": float(stage_d[1]),
                      "lse_combine_value_proj": float(stage_d[2])},
        "attn_gbps": alg_cache / (max(attn_ms - pair_ms, 1e-6) * 1e-3) / 1e9,
        "decode_gbps": alg_decode / (decode_ms * 1e-3) / 1e9,
        "step_gbps": (alg_decode + alg_query) / (ms * 1e-3) / 1e9,
        "alg_cache": alg_cache,
    }
    return res, d


def prefill_bench(args, torch, binding, S, p):
    case = S.workload(2)
    B, T, H = case.batch, case.seqlen, case.n_heads
    L = binding.lib()
    dims = binding.dims(H)
    xs = to_dev_bf16(torch, p["q_latent"])
    g = torch.from_numpy(p["gamma"]).cuda()
    wq = to_dev_bf16(torch, p["wq_b"])
    cs = torch.from_numpy(p["rope_cs"]).cuda()
    wkv = to_dev_bf16(torch, p["wkv_b"])
    lat = to_dev_bf16(torch, p["kv_latent"])
    kpe = to_dev_bf16(torch, p["k_pe"])
    q = torch.empty((B, T, H, 192), dtype=torch.bfloat16, device="cuda")
    inv = torch.empty(B * T, dtype=torch.float32, device="cuda")
    out = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
    qws_bytes = binding.query_path_workspace_size(H, B * T)
    qws = torch.empty(qws_bytes, dtype=torch.uint8, device="cuda")
    ws_bytes = binding.prefill_workspace_size(H, B, T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    L.mla_prefill_ex.argtypes = list(L.mla_prefill.argtypes) + [ctypes.POINTER(ctypes.c_void_p)]
    L.mla_query_path_ex.argtypes = list(L.mla_query_path.argtypes) + [ctypes.POINTER(ctypes.c_void_p)]
    L.mla_query_path_packed_ex.argtypes = list(L.mla_query_path.argtypes) + [ctypes.POINTER(ctypes.c_void_p)]
    qpath = L.mla_query_path_ex
    if args.query_weights == "packed":
        wq = binding.wq_b_pack(wq, H)
        qpath = L.mla_query_path_packed_ex
        torch.cuda.synchronize()
    K, W = max(3, args.steps // 4), 2
    evq, evp = HipEvents(3 * K), HipEvents(3 * K)

    def step(i, timed):
        eq = evq.ptr(3 * (i - W)) if timed else None
        ep = evp.ptr(3 * (i - W)) if timed else None
        assert qpath(ctypes.byref(dims), B * T, xs.data_ptr(), g.data_ptr(), wq.data_ptr(),
                     cs.data_ptr(), q.data_ptr(), inv.data_ptr(), qws.data_ptr(), qws_bytes,
                     stream, eq) == 0
        assert L.mla_prefill_ex(ctypes.byref(dims), B, T, q.data_ptr(), lat.data_ptr(), kpe.data_ptr(),
                                wkv.data_ptr(), ws.data_ptr(), ws_bytes, out.data_ptr(), None, stream, ep) == 0

    for i in range(W):
        step(i, False)
    torch.cuda.synchronize()
    for i in range(W, W + K):
        step(i, True)
    torch.cuda.synchronize()
    sq = np.array([[evq.ms(3 * k + j, 3 * k + j + 1) for j in range(2)] for k in range(K)]).mean(0)
    sp = np.array([[evp.ms(3 * k + j, 3 * k + j + 1) for j in range(2)] for k in range(K)]).mean(0)
    f_query = 2.0 * B * T * 1536 * H * 192
    f_expand = 2.0 * B * T * 512 * 256 * H
    f_attn = 640.0 * B * (T * (T + 1) // 2) * H
    t_q, t_e, t_a = float(sq.sum()), float(sp[0]), float(sp[1])
    tot = t_q + t_e + t_a
    return {
        "workload": case.name, "ms": tot,
        "tflops": (f_query + f_expand + f_attn) / (tot * 1e-3) / 1e12,
        "stages": {
            "query_path": {"ms": t_q, "tflops": f_query / (t_q * 1e-3) / 1e12},
            "expansion": {"ms": t_e, "tflops": f_expand / (t_e * 1e-3) / 1e12},
            "causal_attention": {"ms": t_a, "tflops": f_attn / (t_a * 1e-3) / 1e12},
        },
    }


def _time_calls(torch, fn, n_stages, warmup=3, reps=10):
    """Mean per-stage times (ms) of fn(events) over `reps` calls, each recording n_stages + 1 events
    on the stream the library runs on."""
    ev = HipEvents((n_stages + 1) * reps)
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    for k in range(reps):
        fn(ev.ptr((n_stages + 1) * k))
    torch.cuda.synchronize()
    return np.array([[ev.ms((n_stages + 1) * k + j, (n_stages + 1) * k + j + 1) for j in range(n_stages)]
                     for k in range(reps)]).mean(0)


def _cpu_timed(fn, budget_s, unit_per_call, unit):
    """Oracle calls repeated for about budget_s (at least one): rate in `unit` per second."""
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": n * unit_per_call / dt, "unit": unit, "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "seconds": dt, "calls": n}


def next_rows_bench(args, torch, binding, S, dec_d, pre_inputs):
    """The steps next to the hot path, each on a workload of the benchmark's shapes: the key/value
    side with its cache write, top-k decode, prefill over a cached prefix and the output projection.
    Each reports its time, its algorithmic bytes or flops against the roofline, and the CPU oracle on
    a small sample (about --next-cpu-budget seconds each)."""
    from oracle import mla_oracle as O
    L = binding.lib()
    stream = torch.cuda.current_stream().cuda_stream
    P = ctypes.POINTER(ctypes.c_void_p)
    L.mla_decode_sparse_ex.argtypes = list(L.mla_decode_sparse.argtypes) + [P]
    L.mla_prefill_with_prefix_ex.argtypes = list(L.mla_prefill_with_prefix.argtypes) + [P]
    L.mla_output_proj_ex.argtypes = list(L.mla_output_proj.argtypes) + [P]
    budget = args.next_cpu_budget
    rows = {}

    # N1: key/value side + cache write, 32 decode tokens and 4096 prefill tokens
    kvres = {}
    for name, B, T in (("decode_b32", 32, 1), ("prefill_t4096", 1, 4096)):
        H = 128
        dims = binding.dims(H)
        inp = S.kv_side_inputs(B * T, 0, 30 + T)
        cs = S.rope_table(np.arange(B * T) % 4096).reshape(B, T, 32, 2)
        max_seqlen = T + 64
        kv_a = to_dev_bf16(torch, inp["kv_a"]).view(B, T, 576)
        g = torch.from_numpy(inp["kv_gamma"]).cuda()
        csd = torch.from_numpy(cs).cuda()
        start = torch.full((B,), 64, dtype=torch.int32, device="cuda")
        kvc = torch.zeros((B * max_seqlen, 512), dtype=torch.bfloat16, device="cuda")
        pec = torch.zeros((B * max_seqlen, 64), dtype=torch.bfloat16, device="cuda")
        ev_holder = {}

        def call(evp, B=B, T=T, kv_a=kv_a, g=g, csd=csd, start=start, kvc=kvc, pec=pec, max_seqlen=max_seqlen,
                 dims=dims):
            # no staged variant: events recorded around the call on the same stream
            if evp is not None:
                ev_holder["ev"].hip.hipEventRecord(ctypes.c_void_p(evp[0]), ctypes.c_void_p(stream))
            assert L.mla_kv_append(ctypes.byref(dims), B, T, kv_a.data_ptr(), g.data_ptr(), csd.data_ptr(),
                                   start.data_ptr(), None, max_seqlen, kvc.data_ptr(), pec.data_ptr(), stream) == 0
            if evp is not None:
                ev_holder["ev"].hip.hipEventRecord(ctypes.c_void_p(evp[1]), ctypes.c_void_p(stream))

        reps = 10
        ev = HipEvents(2 * reps)
        ev_holder["ev"] = ev
        for _ in range(3):
            call(None)
        torch.cuda.synchronize()
        for k in range(reps):
            call([ev.ev[2 * k], ev.ev[2 * k + 1]])
        torch.cuda.synchronize()
        ms = float(np.mean([ev.ms(2 * k, 2 * k + 1) for k in range(reps)]))
        n = B * T
        byts = n * (576 * 2 + 256 + 1152) + 512 * 4
        kvres[name] = {"tokens": n, "us": ms * 1e3, "achieved_gbps": byts / (ms * 1e-3) / 1e9,
                       "frac_of_hbm_peak": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "bytes": byts}
    a_cpu = S.kv_side_inputs(4096, 0, 4126)
    cs_cpu = S.rope_table(np.arange(4096))
    kvres["cpu_baseline"] = _cpu_timed(lambda: O.kv_side(a_cpu["kv_a"], a_cpu["kv_gamma"], cs_cpu), budget, 4096,
                                       "tokens/s")
    kvres["cpu_baseline"]["sample"] = "kv_side of 4096 tokens (fp64 NumPy), repeated"
    rows["kv_append"] = {"bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS,
                         "bytes_per_token": 576 * 2 + 256 + 1152, **kvres}

    # N2: top-k decode on the decode workload's caches, 2048 positions per sequence
    case = S.workload(1)
    B, H = case.batch, case.n_heads
    dims = binding.dims(H)
    k = 2048
    topk = S.topk_indices(case.lengths, k, 0, case.case_id)
    q = to_dev_bf16(torch, S.decode_query(case, 0))
    wkv = to_dev_bf16(torch, dec_d["wkv_b"])
    kvd, ped = to_dev_bf16(torch, dec_d["kv_cache"]), to_dev_bf16(torch, dec_d["pe_cache"])
    lens = torch.from_numpy(dec_d["lengths"]).cuda()
    tk = torch.from_numpy(topk).cuda()
    wsb = binding.decode_sparse_workspace_size(H, B, int(case.max_seqlen), k)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    st = _time_calls(torch, lambda e: L.mla_decode_sparse_ex(
        ctypes.byref(dims), B, q.data_ptr(), wkv.data_ptr(), kvd.data_ptr(), ped.data_ptr(), None, lens.data_ptr(),
        int(case.max_seqlen), tk.data_ptr(), k, ws.data_ptr(), wsb, out.data_ptr(), None, stream, e), 3)
    sel = int(np.sum(topk >= 0))
    attn_bytes = sel * BYTES_PER_CACHED_TOKEN
    tot_bytes = attn_bytes + 2 * H * 128 * 512 * 2 + B * H * (192 + 128) * 2 + B * k * 4
    qv = O.bf16_decode(S.decode_query(case, 0))

    def cpu_sparse():
        b = 0
        O.decode_topk(qv[b], dec_d["wkv_b"], dec_d["kv_cache"][:4096], dec_d["pe_cache"][:4096], topk[b], 192 ** -0.5)
    c = _cpu_timed(cpu_sparse, budget, H * k, "selected-token·heads/s")
    c["sample"] = "decode_topk of sequence 0 (2048 of 4096 positions, fp64 NumPy), repeated"
    rows["decode_sparse"] = {
        "workload": f"{case.name}_top{k}", "selected_tokens": sel, "us": float(st.sum()) * 1e3,
        "stages_us": [float(x) * 1e3 for x in st],
        "value": H * sel / (float(st.sum()) * 1e-3), "unit": "selected-token·heads/s",
        "roofline": {"bound": "hbm", "kernel": "gathering split-KV attention",
                     "achieved": attn_bytes / (float(st[1]) * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": attn_bytes / (float(st[1]) * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "bytes_per_launch": attn_bytes},
        "decode_gbps": tot_bytes / (float(st.sum()) * 1e-3) / 1e9, "cpu_baseline": c}

    # N3: the second half of the prefill workload as a chunk over its first half
    p = pre_inputs
    pc = S.workload(2)
    T, H = pc.seqlen, pc.n_heads
    dims = binding.dims(H)
    tq = T // 2
    qfull = to_dev_bf16(torch, S.prefill_query(pc, 0))
    qc = qfull[:, T - tq:].contiguous()
    lat, kpe, wkv2 = to_dev_bf16(torch, p["kv_latent"]), to_dev_bf16(torch, p["k_pe"]), to_dev_bf16(torch, p["wkv_b"])
    wsb = binding.prefill_workspace_size(H, 1, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    outp = torch.empty((1, tq, H, 128), dtype=torch.bfloat16, device="cuda")
    st = _time_calls(torch, lambda e: L.mla_prefill_with_prefix_ex(
        ctypes.byref(dims), 1, tq, T, qc.data_ptr(), lat.data_ptr(), kpe.data_ptr(), wkv2.data_ptr(), ws.data_ptr(),
        wsb, outp.data_ptr(), None, stream, e), 2, reps=5)
    pairs = sum(T - tq + i + 1 for i in range(tq))
    f_exp = 2.0 * T * 512 * 256 * H
    f_att = 640.0 * pairs * H
    qcv = O.bf16_decode(S.prefill_query(pc, 0)[0, T - tq:])
    c = _cpu_timed(lambda: O.prefill_causal(qcv, p["kv_latent"][0], p["k_pe"][0], p["wkv_b"], 192 ** -0.5,
                                            heads=[0], rows=[tq - 1]), budget, 2.0 * T * 512 * 256 + 640.0 * T,
                   "FLOP/s")
    c["sample"] = ("one head's expansion of the 4096 keys and the chunk's last query row over them "
                   "(fp64 NumPy), repeated")
    t_tot = float(st.sum())
    rows["prefill_with_prefix"] = {
        "workload": f"dsv32_prefill_chunk_q{tq}_kv{T}_h{H}", "ms": t_tot,
        "tflops": (f_exp + f_att) / (t_tot * 1e-3) / 1e12,
        "stages": {"expansion": {"ms": float(st[0]), "tflops": f_exp / (float(st[0]) * 1e-3) / 1e12},
                   "causal_attention": {"ms": float(st[1]), "tflops": f_att / (float(st[1]) * 1e-3) / 1e12}},
        "roofline": {"bound": "mfma", "kernel": "causal attention", "achieved": f_att / (float(st[1]) * 1e-3) / 1e12,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": f_att / (float(st[1]) * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "cpu_baseline": c}

    # N4: output projection after a decode step (32 tokens) and after the prefill (4096 tokens)
    dim = S.MODEL_DIM
    wo = to_dev_bf16(torch, S.wo_weights(128, 0, 40, dim, workers=S.default_workers()))
    dims = binding.dims(128)
    opres = {}
    for name, n in (("decode_b32", 32), ("prefill_t4096", 4096)):
        x = to_dev_bf16(torch, S.head_outputs(n, 128, 0, 41, workers=S.default_workers()))
        y = torch.empty((n, dim), dtype=torch.bfloat16, device="cuda")
        wsb = binding.output_proj_workspace_size(128, n, dim)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        st = _time_calls(torch, lambda e: L.mla_output_proj_ex(ctypes.byref(dims), n, dim, x.data_ptr(), wo.data_ptr(),
                                                              ws.data_ptr() if wsb else None, wsb, y.data_ptr(),
                                                              stream, e), 2)
        t = float(st.sum())
        fl = 2.0 * n * 128 * 128 * dim
        by = dim * 128 * 128 * 2 + n * 128 * 128 * 2 + n * dim * 2
        opres[name] = {"tokens": n, "us": t * 1e3, "tflops": fl / (t * 1e-3) / 1e12, "gbps": by / (t * 1e-3) / 1e9,
                       "roofline": ({"bound": "hbm", "achieved": by / (t * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                                     "unit": "GB/s", "frac": by / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS} if n <= 64 else
                                    {"bound": "mfma", "achieved": fl / (t * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "frac": fl / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS})}
    wo_h = S.wo_weights(128, 0, 40, dim, workers=S.default_workers())
    x1 = S.head_outputs(1, 128, 0, 41)
    c = _cpu_timed(lambda: O.output_proj(x1, wo_h), budget, 2.0 * 128 * 128 * dim, "FLOP/s")
    c["sample"] = "one token through the 7168 x 16384 wo (fp64 NumPy), repeated"
    opres["cpu_baseline"] = c
    rows["output_proj"] = {"dim": dim, **opres}
    return rows


def measured_traffic(workload_name):
    """HBM bytes per launch of the attention kernel on this workload, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary profiles/attend_kernel_hbm_traffic_<workload>.txt --
    None when there is none or decode.hip changed since it was taken."""
    import hashlib
    try:
        path = os.path.join(PROFILES, f"attend_kernel_hbm_traffic_{workload_name}.txt")
        fields = dict(l.split(":", 1) for l in open(path).read().splitlines() if ":" in l)
        src = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
        if fields.get("decode_hip_sha256", "").strip() != src:
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def measure_peaks(torch):
    """Achievable rates on this GPU, measured in this process: a plain streaming read of 4 GiB (the
    HBM read rate a kernel can reach) and a loop of independent bf16 16x16x32 MFMAs on every SIMD
    (the matrix rate at the clock the chip holds under it). Each is the median of 7 launches timed
    with events on the stream they run on."""
    lib = ctypes.CDLL(PEAKS_LIB)
    lib.mla_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def timed(launch, reps=7):
        for _ in range(3):
            assert launch() == 0
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            assert launch() == 0
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    ms_read = timed(lambda: lib.mla_peak_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream))
    del buf
    blocks, iters = 1024, 20000
    ms_mfma = timed(lambda: lib.mla_peak_mfma(blocks, iters, sink.data_ptr(), stream))
    flops = blocks * 4 * iters * 8 * 16384
    return {"stream_read_gbps": nbytes / (ms_read * 1e-3) / 1e9, "stream_read_bytes": nbytes,
            "mfma_bf16_tflops": flops / (ms_mfma * 1e-3) / 1e12,
            "note": "plain 4 GiB streaming read (16-byte loads, 2048 blocks) and 8 independent 16x16x32 bf16 "
                    "MFMA chains per wave, 1024 blocks of 4 waves; median of 7 launches"}


def copy_calibration(torch, mib):
    """A plain device copy of known size (bytes read = bytes written = mib MiB), for scaling the
    FETCH_SIZE / WRITE_SIZE counters."""
    n = mib << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def host_description():
    """The host the oracle runs on: CPU model, cores it may use, and NumPy's BLAS build."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    blas = None
    try:
        import threadpoolctl
        for i in threadpoolctl.threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')} threads, " \
                       f"{i.get('architecture')})"
                break
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "numpy_blas": blas}


def cpu_baseline(case, d, budget_s):
    """The oracle (untuned) on the whole batch of the decode step: query path + decode."""
    from oracle import mla_oracle as O
    try:
        import threadpoolctl
        cores = len(os.sched_getaffinity(0))
        ctl = threadpoolctl.threadpool_limits(limits=cores)
        info = threadpoolctl.threadpool_info()
        used = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:  # pragma: no cover
        ctl, used = None, os.cpu_count()
    H = case.n_heads
    # passes over the batch, one sequence at a time, until about half the budget is spent (at least
    # one sequence, at most the budget)
    t0 = time.perf_counter()
    n_seq = 0
    tokens = 0
    passes = 0
    done = False
    while not done:
        for b in range(case.batch):
            qo, _ = O.query_path(d["q_latent"][b:b + 1], d["gamma"], d["wq_b"], d["rope_cs"][b:b + 1], H)
            r0, Lb = int(d["row_offset"][b]), int(d["lengths"][b])
            O.decode_absorbed(qo[0], d["wkv_b"], d["kv_cache"][r0:r0 + Lb], d["pe_cache"][r0:r0 + Lb],
                              192 ** -0.5)
            n_seq += 1
            tokens += Lb
            if time.perf_counter() - t0 > budget_s:
                done = True
                break
        passes += 1
        done = done or time.perf_counter() - t0 > budget_s / 2
    dt = time.perf_counter() - t0
    if ctl is not None:
        ctl.unregister() if hasattr(ctl, "unregister") else None
    return {"value": H * tokens / dt, "unit": "cache-token·heads/s", "cores": int(used), "kind": "oracle",
            "sample": f"{n_seq} sequences ({passes} pass(es) over the {case.batch} of {case.name}; query path + "
                      f"absorbed decode, fp64 NumPy, one sequence at a time), {dt:.1f} s",
            "host": host_description()}


def decode_record(res, cpu, peaks):
    """The per-workload record: step, stages, the attention kernel's roofline and the oracle."""
    case = res["case"]
    achieved = res["attn_gbps"]
    roof = {"bound": "hbm", "kernel": "split-KV attention (mla_decode stage 2)",
            "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic(case.name),
            "bytes_per_launch": res["alg_cache"],
            "attn_us": (res["attn_ms"] - res["event_pair_ms"]) * 1e3,
            "attn_us_between_events": res["attn_ms"] * 1e3,
            "event_pair_us": res["event_pair_ms"] * 1e3,
            "duration_note": "mean span between the events that bracket the kernel in the timed loop, "
                             "less the mean span of two events recorded back to back after a step "
                             "(what a pair of events adds by itself)"}
    if peaks:
        roof["frac_of_measured_read_peak"] = achieved / peaks["stream_read_gbps"]
    return {"workload": case.name, "batch": res["B"], "heads": res["H"], "cached_tokens": res["tokens"],
            "value": res["value"], "unit": "cache-token·heads/s", "ms_per_step": res["ms"],
            "input_copies_rotated": res["copies"],
            "hbm_gbps": res["step_gbps"], "decode_hbm_gbps": res["decode_gbps"],
            "stages_ms": res["stages_ms"], "roofline": roof, "cpu_baseline": cpu}


def prefill_cpu_baseline(p, budget):
    """The oracle on a sample of the prefill workload: one head's expansion of the 4096 keys and
    the causal attention of that head's last query row over them."""
    from oracle import mla_oracle as O
    T = p["kv_latent"].shape[1]
    qh = np.random.default_rng(0).standard_normal((T, 1, 192))
    c = _cpu_timed(lambda: O.prefill_causal(qh, p["kv_latent"][0], p["k_pe"][0], p["wkv_b"][:256], 192 ** -0.5,
                                            heads=[0], rows=[T - 1]), budget,
                   2.0 * T * 512 * 256 + 640.0 * T, "FLOP/s")
    c["sample"] = ("one head's expansion of the 4096 latent rows (k_nope and values) and its last query row's "
                   "causal attention over them (fp64 NumPy), repeated")
    c["host"] = host_description()
    return c


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first (the clock settles from ~1.9 to ~2.3 GHz over ~0.2 s of work)")
    ap.add_argument("--workloads", default="3,0,1,4",
                    help="decode workloads, the first one the headline (0, 1, 3 and/or 4)")
    ap.add_argument("--copies", type=int, default=64, help="most input copies rotated (defeat the Infinity Cache)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="oracle seconds for the headline workload")
    ap.add_argument("--sub-cpu-budget", type=float, default=3.0, help="oracle seconds for each other workload")
    ap.add_argument("--no-next", action="store_true", help="skip the steps next to the path")
    ap.add_argument("--next-cpu-budget", type=float, default=2.0, help="oracle seconds per next-row baseline")
    ap.add_argument("--query-weights", choices=("packed", "stored"), default="packed",
                    help="wq_b layout the query path reads: rearranged once by mla_wq_b_pack (default), or as stored")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    workloads = [int(w) for w in args.workloads.split(",") if w.strip()]
    if not workloads or any(w not in (0, 1, 3, 4) for w in workloads):
        sys.exit("--workloads takes decode workloads 0, 1, 3 and 4")

    import torch
    from head_latent_attention_fp32_amd import binding
    from synth import inputs as S
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    binding.lib()

    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks(torch)
        log(f"[bench] peaks: stream read {peaks['stream_read_gbps']:.0f} GB/s, "
            f"MFMA bf16 {peaks['mfma_bf16_tflops']:.0f} TFLOP/s")

    records, head_res, head_d, dec1 = [], None, None, None
    for k, w in enumerate(workloads):
        res, d = decode_bench(args, torch, binding, S, w)
        log(f"[bench] {res['case'].name}: step {res['ms'] * 1e3:.1f} us; attention "
            f"{(res['attn_ms'] - res['event_pair_ms']) * 1e3:.1f} us; stages (ms) {json.dumps(res['stages_ms'])}")
        cpu = None
        if not args.no_cpu:
            log(f"[bench] timing the CPU oracle on {res['case'].name}")
            cpu = cpu_baseline(res["case"], d, args.cpu_budget if k == 0 else args.sub_cpu_budget)
        records.append(decode_record(res, cpu, peaks))
        if k == 0:
            head_res, head_d = res, d
        if w == 1:
            dec1 = d
        if k > 0 and w != 1:
            del d
        torch.cuda.empty_cache()
    head = records[0]

    p_in = None
    if not (args.no_prefill and args.no_next):
        log(f"[bench] generating {S.workload(2).name}")
        p_in = S.prefill_inputs(S.workload(2), seed=0)
    pre = None if args.no_prefill else prefill_bench(args, torch, binding, S, p_in)
    if pre:
        log(f"[bench] prefill {pre['ms']:.3f} ms, {pre['tflops']:.1f} TFLOP/s")
        if not args.no_cpu:
            pre["cpu_baseline"] = prefill_cpu_baseline(p_in, args.sub_cpu_budget)
    nxt = None
    if not args.no_next:
        dec_d = dec1 if dec1 is not None else S.decode_inputs(S.workload(1), seed=0)
        log("[bench] steps next to the path (kv append, top-k decode, prefix prefill, output projection)")
        nxt = next_rows_bench(args, torch, binding, S, dec_d, p_in)
        log(f"[bench] next rows: {json.dumps({k: v.get('us', v.get('ms')) for k, v in nxt.items()})}")
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "cache-token·heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "batch": head["batch"], "heads": head["heads"],
                   "cached_tokens": head["cached_tokens"],
                   "step": ("mla_query_path_packed" if args.query_weights == "packed" else "mla_query_path")
                           + " + mla_decode",
                   "query_weights": args.query_weights,
                   "input_copies_rotated": head["input_copies_rotated"]},
        "hbm_gbps": head["hbm_gbps"],
        "decode_hbm_gbps": head["decode_hbm_gbps"],
        "stages_ms": head["stages_ms"],
        "stages_note": "stages_ms from a separate pass with an event at every stage boundary (each event adds about "
                       "2 us); ms_per_step and the roofline come from the timed pass, whose only events bracket the "
                       "attention kernel",
        "roofline": head["roofline"],
        "peaks": peaks,
        "cpu_baseline": head["cpu_baseline"],
        "decode_workloads": {r["workload"]: r for r in records},
        "prefill": None if pre is None else {
            "workload": pre["workload"], "ms": pre["ms"], "tflops": pre["tflops"],
            "frac_of_bf16_peak": pre["tflops"] / BF16_PEAK_TFLOPS,
            "frac_of_measured_mfma_peak": (pre["tflops"] / peaks["mfma_bf16_tflops"]) if peaks else None,
            "stages": pre["stages"], "cpu_baseline": pre.get("cpu_baseline")},
        "next_rows": nxt,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
