"""Benchmark of the MLA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N] [--no-prefill] [--no-cpu]

A step is one pass of the decode hot path over one batch of the DeepSeek-V3.2-shaped decode
workload (32 sequences x 4096 cached tokens, 128 heads): mla_query_path on the 32 new tokens, then
mla_decode (absorb, split-KV attention, log-sum-exp combine, value projection). Inputs are
synthetic (seeded) and resident in HBM before the timed region; four copies of every input are
rotated so that the 256 MB Infinity Cache cannot hold the working set between steps.

The printed JSON line carries:
  value       whole-job decode throughput, cache-token.heads/s = H * sum(L_b) / step time
  roofline    the split-KV attention kernel (the dominant kernel): algorithmic bytes per launch
              (1152 B per cached token: 512 latent + 64 rotary bf16) / its mean duration, timed with
              HIP events recorded on its own stream around that kernel, against 8 TB/s; `traffic`
              is the HBM bytes per launch measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE, scaled by a
              copy-kernel calibration) as committed under profiles/, or null when the kernel source
              has changed since (checked by hash) or for another workload
  prefill     the DeepSeek-V3.2-shaped prefill (T = 4096, 128 heads): query path + expansion +
              causal attention, TFLOP/s of algorithmic flops against 2.5 PFLOP/s bf16
  cpu_baseline the CPU oracle on a bounded sample of the same workload (whole sequences, one at a
              time, for about half of --cpu-budget seconds)

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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_kernel_hbm_traffic_dsv32_b32_l4096.txt")
DECODE_SRC = os.path.join(ROOT, "head_latent_attention_fp32_amd", "csrc", "decode.hip")


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


def decode_bench(args, torch, binding, S):
    case = S.workload(args.workload)
    B, H = case.batch, case.n_heads
    log(f"[bench] generating {case.name} (B={B}, H={H}, sum L={int(case.lengths.sum())})")
    d = S.decode_inputs(case, seed=0)
    L = binding.lib()
    dims = binding.dims(H)
    n_copies = args.copies
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
    evd = HipEvents(5 * K)

    def step(i, timed):
        s = sets[i % n_copies]
        eq = evq.ptr(3 * (i - W)) if timed else None
        ed = evd.ptr(5 * (i - W)) if timed else None
        st = L.mla_query_path_ex(ctypes.byref(dims), B, s["q_latent"].data_ptr(), s["gamma"].data_ptr(),
                                 s["wq_b"].data_ptr(), s["rope_cs"].data_ptr(), q.data_ptr(), inv.data_ptr(),
                                 qws_ptr, qws_bytes, stream, eq)
        assert st == 0, st
        st = L.mla_decode_ex(ctypes.byref(dims), B, q.data_ptr(), s["wkv_b"].data_ptr(), s["kv"].data_ptr(),
                             s["pe"].data_ptr(), s["off"].data_ptr() if packed else None, s["lens"].data_ptr(),
                             int(case.max_seqlen), ws.data_ptr(), ws_bytes, out.data_ptr(), lse.data_ptr(),
                             stream, ed)
        assert st == 0, st

    L.mla_query_path_ex.argtypes = list(L.mla_query_path.argtypes) + [ctypes.POINTER(ctypes.c_void_p)]
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
    stage_q = np.array([[evq.ms(3 * k + j, 3 * k + j + 1) for j in range(2)] for k in range(K)]).mean(0)
    stage_d = np.array([[evd.ms(5 * k + j, 5 * k + j + 1) for j in range(4)] for k in range(K)]).mean(0)
    tokens = int(np.clip(case.lengths, 0, case.max_seqlen).sum())
    alg_cache = tokens * BYTES_PER_CACHED_TOKEN
    alg_decode = alg_cache + 2 * H * 128 * 512 * 2 + B * H * (192 + 128) * 2
    alg_query = 1536 * H * 192 * 2 + B * 1536 * 2 + B * H * 192 * 2
    attn_ms = float(stage_d[1])
    decode_ms = float(stage_d.sum())
    res = {
        "case": case, "ms": ms, "tokens": tokens, "H": H, "B": B,
        "value": H * tokens / (ms * 1e-3),
        "stages_ms": {"query_stats": float(stage_q[0]), "query_gemm_rope": float(stage_q[1]),
                      "absorb_plan": float(stage_d[0]), "split_kv_attention": attn_ms,
                      "lse_combine": float(stage_d[2]), "value_proj": float(stage_d[3])},
        "attn_gbps": alg_cache / (attn_ms * 1e-3) / 1e9,
        "decode_gbps": alg_decode / (decode_ms * 1e-3) / 1e9,
        "step_gbps": (alg_decode + alg_query) / (ms * 1e-3) / 1e9,
        "alg_cache": alg_cache,
    }
    return res, d


def prefill_bench(args, torch, binding, S):
    case = S.workload(2)
    B, T, H = case.batch, case.seqlen, case.n_heads
    log(f"[bench] generating {case.name}")
    p = S.prefill_inputs(case, seed=0)
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
    K, W = max(3, args.steps // 4), 2
    evq, evp = HipEvents(3 * K), HipEvents(3 * K)

    def step(i, timed):
        eq = evq.ptr(3 * (i - W)) if timed else None
        ep = evp.ptr(3 * (i - W)) if timed else None
        assert L.mla_query_path_ex(ctypes.byref(dims), B * T, xs.data_ptr(), g.data_ptr(), wq.data_ptr(),
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


def measured_traffic():
    """HBM bytes per launch of the attention kernel on this workload, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary -- None when decode.hip changed since it was taken."""
    import hashlib
    try:
        fields = dict(l.split(":", 1) for l in open(TRAFFIC_FILE).read().splitlines() if ":" in l)
        src = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
        if fields.get("decode_hip_sha256", "").strip() != src:
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


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
                      f"absorbed decode, fp64 NumPy, one sequence at a time), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, help="decode workload: 0, 1 (default), 3 or 4")
    ap.add_argument("--copies", type=int, default=4, help="rotated input copies (defeat the Infinity Cache)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if args.workload not in (0, 1, 3, 4):
        sys.exit("--workload must be a decode workload (0, 1, 3 or 4)")

    import torch
    from head_latent_attention_fp32_amd import binding
    from synth import inputs as S
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    binding.lib()

    res, d = decode_bench(args, torch, binding, S)
    case = res["case"]
    log(f"[bench] decode step {res['ms'] * 1e3:.1f} us; stages (ms) {json.dumps(res['stages_ms'])}")
    pre = None if args.no_prefill else prefill_bench(args, torch, binding, S)
    if pre:
        log(f"[bench] prefill {pre['ms']:.3f} ms, {pre['tflops']:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(case, d, args.cpu_budget)
    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "cache-token·heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": res["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, "batch": res["B"], "heads": res["H"],
                   "cached_tokens": res["tokens"], "step": "mla_query_path + mla_decode",
                   "input_copies_rotated": args.copies},
        "hbm_gbps": res["step_gbps"],
        "decode_hbm_gbps": res["decode_gbps"],
        "stages_ms": res["stages_ms"],
        "roofline": {"bound": "hbm", "kernel": "split-KV attention (mla_decode stage 2)",
                     "achieved": res["attn_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": res["attn_gbps"] / HBM_PEAK_GBPS,
                     "traffic": measured_traffic() if case.name == "dsv32_decode_b32_l4096_h128" else None,
                     "bytes_per_launch": res["alg_cache"], "attn_us": res["stages_ms"]["split_kv_attention"] * 1e3},
        "prefill": None if pre is None else {
            "workload": pre["workload"], "ms": pre["ms"], "tflops": pre["tflops"],
            "frac_of_bf16_peak": pre["tflops"] / BF16_PEAK_TFLOPS, "stages": pre["stages"]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
