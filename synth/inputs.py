"""Seeded synthetic inputs for the MLA query path, absorbed decode and causal prefill.

This module only draws numbers, stores them the way the pages store tensors (bf16 weights,
caches and activations; an fp32 RMSNorm gain) and lays them out. It holds none of the method's
arithmetic. The one table it builds is R, the per-position (cos, sin) rows that the
"DeepSeek-V3.2-Exp · Query heads" page lists as an input of the query heads ("R [T positions,
32 pairs]"); it is built in fp64 and stored in fp32 so that every consumer sees identical values.

Recipe (identical for the GPU path, the oracle, the tests and the benchmark):
  * every tensor draws from its own PCG64 stream keyed by (seed, case id, tensor id[, sequence,
    chunk]), so any slice (one sequence of a ragged cache, one chunk of rows) can be regenerated
    without drawing the rest;
  * activations and caches are N(0, 1); weights are N(0, 1/fan_in) with fan_in = 1536 for wq_b and
    512 for wkv_b; the RMSNorm gain is 1 + 0.1 N(0, 1) in fp32;
  * draws are made in fp32 and rounded to bf16 with round-to-nearest-even;
  * rotary frequencies follow theta = 10000 over 64 rotary features (32 pairs).
Steps next to the path draw in the same way: the joint down-projection output kv_a [n, 576] is
N(0, 1) (an N(0,1) token through N(0, 1/fan_in) weights), the kv_norm gain 1 + 0.1 N(0, 1), wo
[7168, H*128] N(0, 1/(H*128)), head outputs N(0, 1); a top-k list of sequence b holds
min(k, L_b) distinct positions drawn uniformly from [0, L_b) in random order, padded with -1.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

# Model widths shared by every workload (DeepSeek-V3.2-Exp and Kimi-K2 attention).
Q_LORA = 1536
KV_LORA = 512
NOPE = 128
ROPE = 64
V_DIM = 128
QK_DIM = NOPE + ROPE           # 192 features per query head
KV_ROW = NOPE + V_DIM          # 256 rows of wkv_b per head
ROPE_THETA = 10000.0
RMS_EPS = 1e-6
SOFTMAX_SCALE = QK_DIM ** -0.5

# Tensor ids of the PCG64 key.
T_Q_LATENT, T_GAMMA, T_WQ_B, T_WKV_B, T_KV, T_PE, T_LENGTHS, T_SPIKES, T_KV_LAT, T_K_PE, T_Q = range(11)
T_KV_A, T_KV_GAMMA, T_WO, T_TOPK, T_HEAD_OUT = range(11, 16)

MODEL_DIM = 7168               # DeepSeek-V3.2 model width (the attention update is [B, 1, 7168])

_ROWS_PER_CHUNK = 16384


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 patterns to float32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_block(n: int, std: float, key: Sequence[int]) -> np.ndarray:
    x = _rng(*key).standard_normal(n, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def normal_bf16_rows(n_rows: int, width: int, std: float, key: Sequence[int],
                     workers: int = 1) -> np.ndarray:
    """[n_rows, width] bf16 draws; chunk c of rows comes from the stream key + (c,)."""
    out = np.empty((n_rows, width), dtype=np.uint16)
    n_chunks = (n_rows + _ROWS_PER_CHUNK - 1) // _ROWS_PER_CHUNK

    def fill(c: int) -> None:
        r0 = c * _ROWS_PER_CHUNK
        r1 = min(n_rows, r0 + _ROWS_PER_CHUNK)
        out[r0:r1] = _normal_block((r1 - r0) * width, std, tuple(key) + (c,)).reshape(r1 - r0, width)

    if workers > 1 and n_chunks > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(n_chunks)))
    else:
        for c in range(n_chunks):
            fill(c)
    return out


def rope_table(positions: np.ndarray, rope_dim: int = ROPE, theta: float = ROPE_THETA) -> np.ndarray:
    """R rows: float32 [n, rope_dim/2, 2] holding (cos, sin) of pos * theta^(-2i/rope_dim)."""
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    i = np.arange(rope_dim // 2, dtype=np.float64).reshape(1, -1)
    ang = pos * theta ** (-2.0 * i / rope_dim)
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


# --------------------------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeCase:
    """One decode batch: B sequences, one new query token each, over cached latents."""
    name: str
    case_id: int
    n_heads: int
    lengths: np.ndarray            # int32 [B]
    layout: str = "padded"         # "padded": row b*max_seqlen + t; "packed": back to back
    max_seqlen: Optional[int] = None
    positions: Optional[np.ndarray] = None   # query RoPE positions; default = lengths
    spike_frac: float = 0.0        # fraction of cached rows (kv and pe) scaled by spike_gain
    spike_gain: float = 8.0
    poison_padding: bool = True    # fill rows that no sequence owns with NaN

    @property
    def batch(self) -> int:
        return int(len(self.lengths))

    def __post_init__(self) -> None:
        self.lengths = np.asarray(self.lengths, dtype=np.int32)
        if self.max_seqlen is None:
            self.max_seqlen = int(self.lengths.max()) if len(self.lengths) else 0
        if self.positions is None:
            self.positions = self.lengths.astype(np.int64)
        self.positions = np.asarray(self.positions, dtype=np.int64)


@dataclasses.dataclass
class PrefillCase:
    """B sequences of T new tokens each, attending causally to themselves (start position 0)."""
    name: str
    case_id: int
    n_heads: int
    batch: int
    seqlen: int


def ragged_lengths(batch: int, lo: int, hi: int, seed: int, case_id: int) -> np.ndarray:
    """Lengths drawn uniformly from the integers lo..hi inclusive."""
    return _rng(seed, case_id, T_LENGTHS).integers(lo, hi + 1, size=batch).astype(np.int32)


def workload(cfg: int, seed: int = 0):
    """The five benchmark workloads (their index is the stream's case id)."""
    if cfg == 0:
        return DecodeCase("kimi_k2_decode_b1_l1000_h64", 0, 64, np.array([1000], np.int32),
                          positions=np.array([1000]))
    if cfg == 1:
        return DecodeCase("dsv32_decode_b32_l4096_h128", 1, 128, np.full(32, 4096, np.int32))
    if cfg == 2:
        return PrefillCase("dsv32_prefill_b1_t4096_h128", 2, 128, 1, 4096)
    if cfg == 3:
        lens = ragged_lengths(128, 256, 32768, seed, 3)
        return DecodeCase("ragged_decode_b128_l256to32768_h128", 3, 128, lens, layout="packed",
                          max_seqlen=32768)
    if cfg == 4:
        return DecodeCase("long_decode_b8_l131072_h128", 4, 128, np.full(8, 131072, np.int32),
                          spike_frac=0.01)
    raise ValueError(f"unknown workload {cfg}")


# --------------------------------------------------------------------------------------------
# Tensor builders
# --------------------------------------------------------------------------------------------
def query_weights(n_heads: int, seed: int, case_id: int, workers: int = 1) -> Dict[str, np.ndarray]:
    g = _rng(seed, case_id, T_GAMMA).standard_normal(Q_LORA, dtype=np.float32)
    gamma = (np.float32(1.0) + np.float32(0.1) * g).astype(np.float32)
    wq_b = normal_bf16_rows(Q_LORA, n_heads * QK_DIM, Q_LORA ** -0.5, (seed, case_id, T_WQ_B), workers)
    return {"gamma": gamma, "wq_b": wq_b}


def kv_weights(n_heads: int, seed: int, case_id: int, workers: int = 1) -> np.ndarray:
    return normal_bf16_rows(n_heads * KV_ROW, KV_LORA, KV_LORA ** -0.5, (seed, case_id, T_WKV_B), workers)


def decode_row_offsets(case: DecodeCase) -> np.ndarray:
    if case.layout == "padded":
        return np.arange(case.batch, dtype=np.int64) * int(case.max_seqlen)
    if case.layout == "packed":
        return np.concatenate([[0], np.cumsum(case.lengths.astype(np.int64))[:-1]]).astype(np.int64)
    raise ValueError(case.layout)


def decode_cache_rows(case: DecodeCase) -> int:
    if case.layout == "padded":
        return case.batch * int(case.max_seqlen)
    return int(case.lengths.astype(np.int64).sum())


def sequence_cache(case: DecodeCase, b: int, seed: int) -> Dict[str, np.ndarray]:
    """kv [L_b, 512] and pe [L_b, 64] bf16 rows of sequence b (regenerable on its own)."""
    L = int(case.lengths[b])
    kv = normal_bf16_rows(L, KV_LORA, 1.0, (seed, case.case_id, T_KV, b))
    pe = normal_bf16_rows(L, ROPE, 1.0, (seed, case.case_id, T_PE, b))
    if case.spike_frac > 0 and L > 0:
        k = int(round(case.spike_frac * L))
        rows = _rng(seed, case.case_id, T_SPIKES, b).choice(L, size=k, replace=False)
        gain = np.float32(case.spike_gain)
        kv[rows] = f32_to_bf16_bits(bf16_bits_to_f32(kv[rows]) * gain)
        pe[rows] = f32_to_bf16_bits(bf16_bits_to_f32(pe[rows]) * gain)
    return {"kv": kv, "pe": pe}


def decode_inputs(case: DecodeCase, seed: int = 0, workers: Optional[int] = None,
                  with_q_latent: bool = True) -> Dict[str, np.ndarray]:
    """All host tensors of one decode batch.

    Returns bf16 tensors as uint16 arrays: q_latent [B,1536], wq_b [1536,H*192],
    wkv_b [H*256,512], kv_cache [rows,512], pe_cache [rows,64]; fp32 gamma [1536] and
    rope_cs [B,32,2]; int64 row_offset [B]; int32 lengths [B].
    """
    workers = default_workers() if workers is None else workers
    H = case.n_heads
    out: Dict[str, np.ndarray] = {}
    if with_q_latent:
        out["q_latent"] = normal_bf16_rows(case.batch, Q_LORA, 1.0, (seed, case.case_id, T_Q_LATENT))
        out.update(query_weights(H, seed, case.case_id, workers))
        out["rope_cs"] = rope_table(case.positions)
    out["wkv_b"] = kv_weights(H, seed, case.case_id, workers)
    rows = decode_cache_rows(case)
    offs = decode_row_offsets(case)
    kv = np.empty((rows, KV_LORA), dtype=np.uint16)
    pe = np.empty((rows, ROPE), dtype=np.uint16)
    if case.layout == "padded" and case.poison_padding:
        owned = np.zeros(rows, dtype=bool)
        for b in range(case.batch):
            owned[offs[b]:offs[b] + case.lengths[b]] = True
        kv[~owned] = 0x7FC0   # bf16 quiet NaN: never to be read
        pe[~owned] = 0x7FC0

    def fill(b: int) -> None:
        L = int(case.lengths[b])
        if L == 0:
            return
        s = sequence_cache(case, b, seed)
        kv[offs[b]:offs[b] + L] = s["kv"]
        pe[offs[b]:offs[b] + L] = s["pe"]

    if workers > 1 and case.batch > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(case.batch)))
    else:
        for b in range(case.batch):
            fill(b)
    out["kv_cache"] = kv
    out["pe_cache"] = pe
    out["row_offset"] = offs
    out["lengths"] = case.lengths.copy()
    out["max_seqlen"] = np.int64(case.max_seqlen)
    return out


def decode_query(case: DecodeCase, seed: int = 0) -> np.ndarray:
    """A directly drawn decode query [B, H, 192] ~ N(0,1) bf16 (for decode-only tests)."""
    return normal_bf16_rows(case.batch, case.n_heads * QK_DIM, 1.0,
                            (seed, case.case_id, T_Q)).reshape(case.batch, case.n_heads, QK_DIM)


def prefill_inputs(case: PrefillCase, seed: int = 0, workers: Optional[int] = None,
                   with_q_latent: bool = True) -> Dict[str, np.ndarray]:
    """Host tensors of one prefill batch: q_latent [B,T,1536], kv_latent [B,T,512],
    k_pe [B,T,64] (bf16), wq_b, gamma, wkv_b and rope_cs [T,32,2] for positions 0..T-1."""
    workers = default_workers() if workers is None else workers
    B, T, H = case.batch, case.seqlen, case.n_heads
    out: Dict[str, np.ndarray] = {}
    if with_q_latent:
        out["q_latent"] = normal_bf16_rows(B * T, Q_LORA, 1.0, (seed, case.case_id, T_Q_LATENT),
                                           workers).reshape(B, T, Q_LORA)
        out.update(query_weights(H, seed, case.case_id, workers))
        out["rope_cs"] = rope_table(np.arange(T))
    out["wkv_b"] = kv_weights(H, seed, case.case_id, workers)
    out["kv_latent"] = normal_bf16_rows(B * T, KV_LORA, 1.0, (seed, case.case_id, T_KV_LAT),
                                        workers).reshape(B, T, KV_LORA)
    out["k_pe"] = normal_bf16_rows(B * T, ROPE, 1.0, (seed, case.case_id, T_K_PE),
                                   workers).reshape(B, T, ROPE)
    return out


def prefill_query(case: PrefillCase, seed: int = 0, workers: Optional[int] = None) -> np.ndarray:
    """A directly drawn prefill query [B, T, H, 192] ~ N(0,1) bf16 (for prefill-only tests)."""
    workers = default_workers() if workers is None else workers
    return normal_bf16_rows(case.batch * case.seqlen, case.n_heads * QK_DIM, 1.0,
                            (seed, case.case_id, T_Q), workers).reshape(
        case.batch, case.seqlen, case.n_heads, QK_DIM)


# --------------------------------------------------------------------------------------------
# Inputs of the steps next to the path
# --------------------------------------------------------------------------------------------
def kv_side_inputs(n_tokens: int, seed: int, case_id: int, workers: int = 1) -> Dict[str, np.ndarray]:
    """kv_a bf16 [n, 576] (the joint down-projection output) and the kv_norm gain fp32 [512]."""
    g = _rng(seed, case_id, T_KV_GAMMA).standard_normal(KV_LORA, dtype=np.float32)
    return {"kv_a": normal_bf16_rows(n_tokens, KV_LORA + ROPE, 1.0, (seed, case_id, T_KV_A), workers),
            "kv_gamma": (np.float32(1.0) + np.float32(0.1) * g).astype(np.float32)}


def wo_weights(n_heads: int, seed: int, case_id: int, dim: int = MODEL_DIM, workers: int = 1) -> np.ndarray:
    """wo bf16 [dim, H*128] (output x input) ~ N(0, 1/(H*128))."""
    return normal_bf16_rows(dim, n_heads * V_DIM, (n_heads * V_DIM) ** -0.5, (seed, case_id, T_WO), workers)


def head_outputs(n_tokens: int, n_heads: int, seed: int, case_id: int, workers: int = 1) -> np.ndarray:
    """Attention head outputs bf16 [n, H, 128] ~ N(0, 1) (input of wo for wo-only tests)."""
    return normal_bf16_rows(n_tokens, n_heads * V_DIM, 1.0, (seed, case_id, T_HEAD_OUT), workers).reshape(
        n_tokens, n_heads, V_DIM)


def topk_indices(lengths: np.ndarray, k: int, seed: int, case_id: int) -> np.ndarray:
    """int32 [B, k]: for sequence b, min(k, L_b) distinct positions of [0, L_b) in random order,
    then -1 padding."""
    lengths = np.asarray(lengths)
    out = np.full((lengths.shape[0], k), -1, dtype=np.int32)
    for b, L in enumerate(lengths):
        L = int(L)
        n = min(k, L)
        if n > 0:
            out[b, :n] = _rng(seed, case_id, T_TOPK, b).choice(L, size=n, replace=False)
    return out


def device_normal_bf16(shape, seed: int, case_id: int, tensor: int = T_Q_LATENT, std: float = 1.0):
    """N(0, std^2) bf16 drawn directly on the GPU (torch's seeded Philox generator on cuda:0), for
    inputs too large to draw on the host (several GB). Rows needed by a CPU check are copied back
    from the returned tensor; the stream is keyed by (seed, case id, tensor id) like the host ones."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed((int(seed) * 1_000_003 + int(case_id)) * 101 + int(tensor))
    x = torch.randn(tuple(shape), generator=g, device="cuda", dtype=torch.float32)
    if std != 1.0:
        x *= std
    return x.to(torch.bfloat16)
