"""Plain CPU oracle for multi-head latent attention (MLA): query path, absorbed decode, causal prefill.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg do. It shares no code with
the GPU library and imports nothing from it.

Everything is NumPy in float64, one sequence (decode) or one sequence and head (prefill) at a
time, with no blocking, fusion or reordering beyond what the definitions state. bf16 appears
only as the storage format the pages' code uses; the codec below converts it.

Two modes:
  * exact  (staged=False): fp64 from the bf16 inputs to the end;
  * staged (staged=True):  fp64 between the points where the pages' code stores bf16 tensors --
      the RMSNorm output (".to(dtype)" in the RMSNorm excerpts), the wq_b Linear output, q_pe after
      its rotation, the absorbed query latent (output of the first einsum of the V3.2 MQA-decode
      excerpt), the expanded k_nope / value states of the Kimi-K2 prefill, and each final output.
    Scores, softmax, the latent weighted sum and the log-sum-exp stay unrounded (the softmax is
    taken in fp32-or-better, as the Kimi-K2 prefill excerpt upcasts it).

Sources (page title -- section):
  [QN]  "DeepSeek V4.1 · Query RMSNorm" -- equation, RMSNorm code excerpt
  [LN]  "DeepSeek-V3.2-Exp · Indexer key LayerNorm" -- equation, LayerNorm code excerpt
  [QH]  "DeepSeek-V3.2-Exp · Query heads" -- equations (all 6 steps), in/out shapes, Parameters,
        MLA __init__ and query code excerpts
  [AU]  "DeepSeek-V3.2-Exp · Attention update" -- RMSNorm excerpt, mla-decode (MQA decode) excerpt
  [VS]  "Kimi-K2 · value_states" -- shapes, Parameters, mla-init and mla-prefill excerpts
  The same pages also fix the steps next to the path: the key/value side of new tokens (wkv_a
  split, kv_norm, rotary key) and the cache rows they fill ([QH], [VS], [AU]); the top-k index mask
  of V3.2 decode ([AU] mla-decode); prefill of new queries over cached keys ([VS] mla-prefill);
  the output projection wo ([AU] mla-output, attention-update shape).

Readings taken where the pages are silent (each also listed in the design notes):
  * RoPE pairs are adjacent, interleaved features (2i, 2i+1) of the 64 rotary features: the V3.2
    indexer passes an explicit "not interleaved" flag as the exception ([LN], Indexer forward),
    while the MLA query call passes none ([QH], query excerpt). The rotation is multiplication by
    e^{+i phi}. The (cos, sin) rows are inputs (R in [QH], in/out shapes).
  * eps = 1e-6 (the code default in [QN] and [AU]; the 1e-20 of the [QN] equation is not used).
  * softmax scale = 192^-0.5 ([QH], MLA __init__), without the long-context mscale correction.
  * decode attends exactly the L_b cached rows it is given; L_b = 0 gives out = 0, lse = -inf.
  * lse is the natural log of the sum over attended positions of exp(scaled score).
  * prefill keeps key t' for query t iff t' <= t; with a cached prefix of S - Tq keys, query i is
    position S - Tq + i.
  * wkv_a's 576 outputs are [latent 512 | rotary key 64] in that order (the order of the sum in its
    width); the rotary key is rotated like q_pe.
  * a top-k entry outside [0, L) names no position; an empty selection gives out = 0, lse = -inf.
  * wo is stored [dim, H*128] (torch Linear orientation) and y = x W^T.

Parity unpinned: the RoPE pairing/sign convention itself (the pages never show the rotation's body);
the oracle's rotation is pinned only to its own reading (identity at position 0, norm preservation,
relative-position property, a hand case).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

NOPE = 128
ROPE = 64
V_DIM = 128
KV_LORA = 512
Q_LORA = 1536
QK = NOPE + ROPE


# ---------------------------------------------------------------------------------------------
# bf16 storage codec
# ---------------------------------------------------------------------------------------------
def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: a bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_encode(x) -> np.ndarray:
    """float64 -> bf16 bit patterns by one direct round-to-nearest-even onto the bf16 grid.

    A bf16 has 8 significant bits, so a normal value with frexp exponent e (x = m 2^e, 0.5<=|m|<1)
    is quantised to multiples of 2^(e-8); below 2^-126 the grid is fixed at 2^-133. Values that
    round past the largest finite bf16 become +-inf; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    o = out.reshape(-1)
    nan = np.isnan(flat)
    fin = np.isfinite(flat)
    _, e = np.frexp(flat[fin])
    q = np.maximum(e - 8, -133).astype(np.float64)
    r = np.rint(flat[fin] * np.exp2(-q)) * np.exp2(q)        # rint: ties to even
    r32 = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r).astype(np.float32)
    o[fin] = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    inf = ~fin & ~nan
    o[inf] = np.where(flat[inf] > 0, 0x7F80, 0xFF80)
    o[nan] = 0x7FC0
    return out


def bf16_round(x) -> np.ndarray:
    return bf16_decode(bf16_encode(x))


def _maybe_round(x: np.ndarray, staged: bool) -> np.ndarray:
    return bf16_round(x) if staged else x


# ---------------------------------------------------------------------------------------------
# Normalisations
# ---------------------------------------------------------------------------------------------
def rms_norm(x, gamma, eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray]:
    """[QN] equation: m2 = mean_j x_j^2; y = gamma * x / sqrt(m2 + eps). Rows are the last axis.

    Returns (y, inv_rms) with inv_rms = 1/sqrt(m2 + eps) per row, both fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    m2 = np.mean(x * x, axis=-1, keepdims=True)
    inv = 1.0 / np.sqrt(m2 + eps)
    y = np.asarray(gamma, dtype=np.float64) * (x * inv)
    return y, inv[..., 0]


def layer_norm(x, gamma, beta, eps: float = 1e-6) -> np.ndarray:
    """[LN] equation: y = gamma * (x - mu) / sqrt(sigma^2 + eps) + beta, sigma^2 the biased (1/d)
    variance over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return np.asarray(gamma, np.float64) * (x - mu) / np.sqrt(var + eps) + np.asarray(beta, np.float64)


# ---------------------------------------------------------------------------------------------
# Rotary embedding on the rotary features
# ---------------------------------------------------------------------------------------------
def rope_rotate(x, cs) -> np.ndarray:
    """Rotate pairs (x[2i], x[2i+1]) by the angle whose (cos, sin) is cs[..., i, :].

    x: [..., 2P]; cs: broadcastable to [..., P, 2]. (a, b) -> (a cos - b sin, a sin + b cos).
    """
    x = np.asarray(x, dtype=np.float64)
    cs = np.asarray(cs, dtype=np.float64)
    a = x[..., 0::2]
    b = x[..., 1::2]
    c = cs[..., 0]
    s = cs[..., 1]
    ra = a * c - b * s
    rb = a * s + b * c
    return np.stack([ra, rb], axis=-1).reshape(ra.shape[:-1] + (2 * ra.shape[-1],))


# ---------------------------------------------------------------------------------------------
# Weight views
# ---------------------------------------------------------------------------------------------
def wq_b_heads(wq_b, n_heads: int) -> Tuple[np.ndarray, np.ndarray]:
    """[QH] one matrix wq_b [1536, H*192] (input x output) holds both parts: head h owns output
    columns h*192 .. h*192+191, the first 128 content (W_UQ), the last 64 rotary (W_QR).

    Returns (W_UQ [1536, H, 128], W_QR [1536, H, 64]) as views of the input array.
    """
    w = np.asarray(wq_b).reshape(-1, n_heads, QK)
    return w[:, :, :NOPE], w[:, :, NOPE:]


def wkv_b_heads(wkv_b, n_heads: int) -> Tuple[np.ndarray, np.ndarray]:
    """[AU] mla-decode: wkv_b [H*256, 512] (output x input) viewed [H, 256, 512]; rows :128 of each
    head are the key-content half W_UK, the last 128 the value half W_UV ([VS] value_states).

    Returns (W_UK [H, 128, 512], W_UV [H, 128, 512]).
    """
    w = np.asarray(wkv_b).reshape(n_heads, NOPE + V_DIM, KV_LORA)
    return w[:, :NOPE, :], w[:, NOPE:, :]


def param_counts(n_heads: int, q_lora: int = Q_LORA) -> dict:
    """Parameter counts of the oracle's weight views, counted element by element."""
    wq = np.empty((q_lora, n_heads * QK), dtype=np.uint8)
    wkv = np.empty((n_heads * (NOPE + V_DIM), KV_LORA), dtype=np.uint8)
    uq, qr = wq_b_heads(wq, n_heads)
    uk, uv = wkv_b_heads(wkv, n_heads)
    return {"query_content": uq.size, "query_rotary": qr.size, "query_total": wq.size,
            "key_up": uk.size, "value_up": uv.size, "kv_up_total": wkv.size}


# ---------------------------------------------------------------------------------------------
# Query path: RMSNorm -> wq_b -> split -> RoPE on the rotary part
# ---------------------------------------------------------------------------------------------
def query_path(q_latent_bits, gamma, wq_b_bits, rope_cs, n_heads: int, eps: float = 1e-6,
               staged: bool = True, round_output: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """[QH] q^C = c^Q W_UQ, q^pe = c^Q W_QR, Q^R_t = RoPE(Q^pe_t, R_t), Q = [Q^C; Q^R], with
    c^Q = q_norm(q latent) ([QN], [AU] RMSNorm; [QH] query excerpt: qr = q_norm(.), q = wq_b(qr)).

    q_latent_bits: bf16 [n, 1536]; gamma fp32 [1536]; wq_b_bits bf16 [1536, H*192];
    rope_cs fp32 [n, 32, 2]. Returns (q [n, H, 192] fp64 -- bf16-valued when staged and
    round_output, inv_rms [n]). Token-major layout [n, H, 192] as the query code's view.
    staged and not round_output: every feature before its last rounding -- the content features
    are the Linear output before its bf16 rounding (their last), the rotary features the rotation
    of the bf16 Linear output before the rotated values are rounded.
    """
    x = bf16_decode(q_latent_bits)
    y, inv_rms = rms_norm(x, gamma, eps)
    y = _maybe_round(y, staged)                         # RMSNorm output stored in the input dtype
    w = bf16_decode(wq_b_bits)
    lin = y @ w
    q = _maybe_round(lin, staged)                       # bf16 Linear output
    q = q.reshape(q.shape[0], n_heads, QK)
    rot = rope_rotate(q[:, :, NOPE:], np.asarray(rope_cs, np.float64)[:, None, :, :])
    if staged and not round_output:
        q = lin.reshape(q.shape).copy()
        q[:, :, NOPE:] = rot
        return q, inv_rms
    q[:, :, NOPE:] = _maybe_round(rot, staged)          # rotated q_pe stored in bf16
    return q, inv_rms


# ---------------------------------------------------------------------------------------------
# Decode (one new query token per sequence)
# ---------------------------------------------------------------------------------------------
def _logsumexp_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True)))[..., 0]


def decode_expanded(q, wkv_b_bits, kv_bits, pe_bits, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """The non-absorbed definition for one sequence, in exact fp64: each cached latent c_t is
    expanded to per-head keys k_t,h = [W_UK[h] c_t ; pe_t] and values v_t,h = W_UV[h] c_t ([VS]
    mla-prefill excerpt, applied to one query); s = scale q.k; p = softmax_t(s); out = sum_t p v.

    q [H, 192] fp64 values; kv_bits [L, 512]; pe_bits [L, 64]. Returns (out [H,128], lse [H]).
    """
    q = np.asarray(q, np.float64)
    H = q.shape[0]
    uk, uv = wkv_b_heads(bf16_decode(wkv_b_bits), H)
    c = bf16_decode(kv_bits)
    pe = bf16_decode(pe_bits)
    L = c.shape[0]
    if L == 0:
        return np.zeros((H, V_DIM)), np.full(H, -np.inf)
    out = np.empty((H, V_DIM))
    lse = np.empty(H)
    for h in range(H):
        k_nope = c @ uk[h].T                 # [L, 128]
        v = c @ uv[h].T                      # [L, 128]
        s = scale * (k_nope @ q[h, :NOPE] + pe @ q[h, NOPE:])
        m = s.max()
        p = np.exp(s - m)
        out[h] = (p @ v) / p.sum()
        lse[h] = m + np.log(p.sum())
    return out, lse


def absorb_query(q, wkv_b_bits, staged: bool = True) -> np.ndarray:
    """[AU] mla-decode first einsum: q_lat[h, c] = sum_d q_nope[h, d] W_UK[h, d, c]. [H, 512]."""
    q = np.asarray(q, np.float64)
    uk, _ = wkv_b_heads(bf16_decode(wkv_b_bits), q.shape[0])
    q_lat = np.einsum("hd,hdc->hc", q[:, :NOPE], uk)
    return _maybe_round(q_lat, staged)


def attend_latent(q_lat, q_pe, kv_bits, pe_bits, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """[AU] mla-decode scores and weighted sum over one run of cached rows:
    s[h, t] = scale (q_lat[h].c_t + q_pe[h].pe_t); returns the normalised latent sum
    o[h] = sum_t softmax_t(s)[h, t] c_t  ([H, 512]) and lse[h] = ln sum_t exp(s[h, t]).
    An empty run gives o = 0, lse = -inf."""
    q_lat = np.asarray(q_lat, np.float64)
    H = q_lat.shape[0]
    c = bf16_decode(kv_bits)
    pe = bf16_decode(pe_bits)
    if c.shape[0] == 0:
        return np.zeros((H, KV_LORA)), np.full(H, -np.inf)
    s = scale * (q_lat @ c.T + np.asarray(q_pe, np.float64) @ pe.T)     # [H, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ c) / l, (m + np.log(l))[:, 0]


def combine_segments(parts: Sequence[Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Merge softmax-normalised results over disjoint runs of rows into the result over their
    union: with M = max_s lse_s and w_s = exp(lse_s - M), o = sum_s w_s o_s / sum_s w_s and
    lse = M + ln sum_s w_s. Empty runs (lse = -inf) carry zero weight; all empty gives o = 0,
    lse = -inf."""
    os_ = np.stack([np.asarray(p[0], np.float64) for p in parts])     # [S, H, D]
    ls = np.stack([np.asarray(p[1], np.float64) for p in parts])      # [S, H]
    M = ls.max(axis=0)                                               # [H]
    safe_M = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(ls), np.exp(ls - safe_M), 0.0)          # [S, H]
    tot = w.sum(axis=0)
    o = np.where(tot[:, None] > 0, np.einsum("sh,shd->hd", w, os_) / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
    lse = np.where(tot > 0, safe_M + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    return o, lse


def decode_absorbed(q, wkv_b_bits, kv_bits, pe_bits, scale: float, staged: bool = True,
                    segments: Optional[Sequence[int]] = None, round_output: bool = True
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """[AU] mla-decode for one sequence: absorb q_nope through W_UK, attend the cached latent and
    rotary key, project the latent sum out through W_UV:
      out[h, d] = sum_c o_lat[h, c] W_UV[h, d, c].
    `segments` optionally gives cut points inside [0, L] at which the rows are attended
    separately and merged with combine_segments (the split form; identical by algebra).
    q [H,192] fp64 values. Returns (out [H,128] -- bf16-valued when staged and round_output,
    lse [H])."""
    q = np.asarray(q, np.float64)
    H = q.shape[0]
    _, uv = wkv_b_heads(bf16_decode(wkv_b_bits), H)
    q_lat = absorb_query(q, wkv_b_bits, staged)
    L = np.asarray(kv_bits).shape[0]
    cuts = [0] + sorted(segments or []) + [L]
    parts = [attend_latent(q_lat, q[:, NOPE:], kv_bits[a:b], pe_bits[a:b], scale)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o_lat, lse = parts[0] if len(parts) == 1 else combine_segments(parts)
    out = np.einsum("hc,hdc->hd", o_lat, uv)
    return _maybe_round(out, staged and round_output), lse


def decode_batch(q, wkv_b_bits, kv_cache_bits, pe_cache_bits, row_offset, lengths, scale: float,
                 staged: bool = True, batch_ids: Optional[Sequence[int]] = None, round_output: bool = True
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Absorbed decode of every (or each listed) sequence b over cache rows
    [row_offset[b], row_offset[b] + lengths[b]). q [B, H, 192]. Returns (out [n, H, 128], lse [n, H])."""
    q = np.asarray(q, np.float64)
    ids = range(q.shape[0]) if batch_ids is None else list(batch_ids)
    outs, lses = [], []
    for b in ids:
        r0 = int(row_offset[b])
        L = int(lengths[b])
        if L == 0:
            outs.append(np.zeros((q.shape[1], V_DIM)))
            lses.append(np.full(q.shape[1], -np.inf))
            continue
        o, l = decode_absorbed(q[b], wkv_b_bits, kv_cache_bits[r0:r0 + L], pe_cache_bits[r0:r0 + L],
                               scale, staged, round_output=round_output)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------------------------
# Prefill (non-absorbed, causal)
# ---------------------------------------------------------------------------------------------
def expand_latent(kv_latent_bits, wkv_b_bits, n_heads: int, staged: bool = True,
                  heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """[VS] kv_b_proj applied to the latent: k_nope[t, h] = W_UK[h] c_t, v[t, h] = W_UV[h] c_t.
    kv_latent_bits [T, 512]. Returns (k_nope [T, n, 128], v [T, n, 128]) for the listed heads
    (all heads by default)."""
    c = bf16_decode(kv_latent_bits)
    uk, uv = wkv_b_heads(bf16_decode(wkv_b_bits), n_heads)
    heads = list(range(n_heads)) if heads is None else list(heads)
    k = np.stack([c @ uk[h].T for h in heads], axis=1)
    v = np.stack([c @ uv[h].T for h in heads], axis=1)
    return _maybe_round(k, staged), _maybe_round(v, staged)


def prefill_head(q_h, k_nope_h, v_h, k_pe, scale: float, rows: Optional[Sequence[int]] = None,
                 q_offset: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """[VS] mla-prefill for one head: key_states = [k_nope ; k_pe] (k_pe shared by all heads),
    S = scale Q K^T, add the causal mask (0 where t' <= t, -inf after), softmax in float64,
    O = P V. Query row i sits at position t = q_offset + i (q_offset > 0: the queries are the
    last rows of a longer sequence whose earlier keys are cached). q_h [Tq, 192],
    k_nope_h / v_h [>= t+1, 128], k_pe [>= t+1, 64] (fp64 values).
    Returns (O [n, 128], lse [n]) for the listed query rows (all rows by default)."""
    Tq = q_h.shape[0]
    rows = list(range(Tq)) if rows is None else list(rows)
    k = np.concatenate([k_nope_h, k_pe], axis=1)                      # [S, 192]
    O = np.empty((len(rows), V_DIM))
    lse = np.empty(len(rows))
    for i, r in enumerate(rows):
        t = q_offset + r
        s = scale * (k[: t + 1] @ q_h[r])                              # keys 0..t only
        m = s.max()
        p = np.exp(s - m)
        O[i] = (p @ v_h[: t + 1]) / p.sum()
        lse[i] = m + np.log(p.sum())
    return O, lse


def prefill_causal(q, kv_latent_bits, k_pe_bits, wkv_b_bits, scale: float, staged: bool = True,
                   heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None,
                   round_output: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Causal non-absorbed prefill of one sequence. q [Tq, H, 192] fp64 values; the latent and
    rotary key cover S >= Tq positions (S = Tq: the plain prefill from position 0; S > Tq: the
    queries are the last Tq positions, the first S - Tq keys a cached prefix -- [VS] mla-prefill,
    whose weights and mask are sized (q_len, kv_seq_len) once past keys join the new ones).
    Returns (out [n_rows, n_heads_sel, 128] -- bf16-valued when staged and round_output,
    lse [n_heads_sel, n_rows])."""
    q = np.asarray(q, np.float64)
    Tq, H, _ = q.shape
    S = np.asarray(kv_latent_bits).shape[0]
    if S < Tq:
        raise ValueError("fewer key positions than queries")
    off = S - Tq
    heads = list(range(H)) if heads is None else list(heads)
    rows = list(range(Tq)) if rows is None else list(rows)
    need = off + max(rows) + 1 if rows else 0
    pe = bf16_decode(k_pe_bits[:need])
    out = np.empty((len(rows), len(heads), V_DIM))
    lse = np.empty((len(heads), len(rows)))
    for j, h in enumerate(heads):
        k_h, v_h = expand_latent(kv_latent_bits[:need], wkv_b_bits, H, staged, heads=[h])
        o, l = prefill_head(q[:, h, :], k_h[:, 0, :], v_h[:, 0, :], pe, scale, rows, q_offset=off)
        out[:, j, :] = o
        lse[j] = l
    return _maybe_round(out, staged and round_output), lse


# ---------------------------------------------------------------------------------------------
# Key/value side of new tokens and the cache write
# ---------------------------------------------------------------------------------------------
def kv_side(kv_a_bits, kv_gamma, rope_cs, eps: float = 1e-6, staged: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """[QH] MLA __init__ / [VS] mla-init: the joint down-projection wkv_a gives each token
    kv_lora + rope = 576 features. The first 512 are the latent, normalised by kv_norm (an RMSNorm
    of width 512 with its own gain, [QN] equation); the last 64 are the rotary key shared by every
    head, rotated at the token's position with the same pairing as q_pe ([VS] mla-prefill rotates
    q_pe and k_pe together).
    kv_a_bits bf16 [n, 576]; kv_gamma fp32 [512]; rope_cs fp32 [n, 32, 2].
    Returns (latent [n, 512], k_pe [n, 64]) -- bf16-valued when staged: what the caches hold."""
    a = bf16_decode(kv_a_bits)
    lat, _ = rms_norm(a[:, :KV_LORA], kv_gamma, eps)
    pe = rope_rotate(a[:, KV_LORA:], np.asarray(rope_cs, np.float64))
    return _maybe_round(lat, staged), _maybe_round(pe, staged)


def cache_append(kv_cache_bits, pe_cache_bits, row_offset, start_pos, latent_bits, k_pe_bits,
                 max_seqlen: int) -> Tuple[np.ndarray, np.ndarray]:
    """[AU] mla-decode reads kv_cache[:bsz, :end_pos] and pe_cache[:bsz, :end_pos]: the cache rows
    of a sequence are its positions in order. New token t of sequence b (latent_bits [B, T, 512],
    k_pe_bits [B, T, 64]) is position start_pos[b] + t, stored at cache row
    row_offset[b] + start_pos[b] + t; positions outside [0, max_seqlen) are not stored.
    Returns updated copies of both caches (rows of 512 and of 64 bf16 bit patterns)."""
    kv = np.array(kv_cache_bits, copy=True)
    pe = np.array(pe_cache_bits, copy=True)
    lat = np.asarray(latent_bits)
    kpe = np.asarray(k_pe_bits)
    B, T = lat.shape[:2]
    for b in range(B):
        for t in range(T):
            pos = int(start_pos[b]) + t
            if 0 <= pos < max_seqlen:
                row = int(row_offset[b]) + pos
                kv[row] = lat[b, t]
                pe[row] = kpe[b, t]
    return kv, pe


# ---------------------------------------------------------------------------------------------
# Decode restricted to the indexer's top-k positions
# ---------------------------------------------------------------------------------------------
def decode_topk(q, wkv_b_bits, kv_bits, pe_bits, topk, scale: float, staged: bool = True,
                round_output: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """[AU] mla-decode with its index mask: a mask of -inf over the L cached positions gets 0 at
    every position the top-k list names (a scatter, so a position named twice is still one
    position) and is added to the scores before the softmax. Entries outside [0, L) name no
    position (reading: padding of a list longer than the sequence). No named position gives
    out = 0, lse = -inf. q [H, 192] fp64 values; topk int [K].
    Returns (out [H, 128] -- bf16-valued when staged and round_output, lse [H])."""
    q = np.asarray(q, np.float64)
    H = q.shape[0]
    c = bf16_decode(kv_bits)
    pe = bf16_decode(pe_bits)
    L = c.shape[0]
    idx = np.asarray(topk, np.int64)
    mask = np.full(L, -np.inf)
    mask[idx[(idx >= 0) & (idx < L)]] = 0.0
    if not np.isfinite(mask).any():
        return np.zeros((H, V_DIM)), np.full(H, -np.inf)
    _, uv = wkv_b_heads(bf16_decode(wkv_b_bits), H)
    q_lat = absorb_query(q, wkv_b_bits, staged)
    s = scale * (q_lat @ c.T + q[:, NOPE:] @ pe.T) + mask[None, :]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o_lat = (p @ c) / l
    out = np.einsum("hc,hdc->hd", o_lat, uv)
    return _maybe_round(out, staged and round_output), (m + np.log(l))[:, 0]


def decode_topk_batch(q, wkv_b_bits, kv_cache_bits, pe_cache_bits, row_offset, lengths, topk, scale: float,
                      staged: bool = True, batch_ids: Optional[Sequence[int]] = None, round_output: bool = True
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """decode_topk of every (or each listed) sequence b over its rows [row_offset[b],
    row_offset[b] + lengths[b]) with top-k list topk[b]. Returns (out [n, H, 128], lse [n, H])."""
    q = np.asarray(q, np.float64)
    ids = range(q.shape[0]) if batch_ids is None else list(batch_ids)
    outs, lses = [], []
    for b in ids:
        r0, L = int(row_offset[b]), int(lengths[b])
        o, l = decode_topk(q[b], wkv_b_bits, kv_cache_bits[r0:r0 + L], pe_cache_bits[r0:r0 + L], topk[b],
                           scale, staged, round_output)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------------------------
# Output projection
# ---------------------------------------------------------------------------------------------
def output_proj(x_bits, wo_bits, staged: bool = True) -> np.ndarray:
    """[AU] mla-output: the head outputs [.., H, 128] are flattened (head-major, feature h*128 + d)
    and projected by wo, a Linear from H*128 features to the model width ([QH] MLA __init__;
    [AU] shape of the attention update: 7168 for DeepSeek-V3.2). The weight is stored as a torch
    Linear stores it, [out = dim, in = H*128], and y = x W^T, a bf16 Linear output.
    x_bits bf16 [n, H, 128]; wo_bits bf16 [dim, H*128]. Returns y [n, dim]."""
    x = bf16_decode(x_bits)
    x = x.reshape(x.shape[0], -1)
    w = bf16_decode(wo_bits)
    return _maybe_round(x @ w.T, staged)


# ---------------------------------------------------------------------------------------------
# Magnitude of the score dot products (the scale against which their rounding error is measured)
# ---------------------------------------------------------------------------------------------
def decode_score_magnitude(q, wkv_b_bits, kv_bits, pe_bits, scale: float, staged: bool = True) -> np.ndarray:
    """Per head, max_t of scale * sum_i |q_i k_t,i| over the terms of the absorbed score
    (|q_lat|.|c_t| + |q_pe|.|pe_t|): the size of the sum whose rounding a score inherits. [H]."""
    q = np.asarray(q, np.float64)
    q_lat = absorb_query(q, wkv_b_bits, staged)
    c = np.abs(bf16_decode(kv_bits))
    pe = np.abs(bf16_decode(pe_bits))
    if c.shape[0] == 0:
        return np.zeros(q.shape[0])
    return scale * np.max(np.abs(q_lat) @ c.T + np.abs(q[:, NOPE:]) @ pe.T, axis=1)


def prefill_score_magnitude(q, kv_latent_bits, k_pe_bits, wkv_b_bits, scale: float, staged: bool = True,
                            heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None
                            ) -> np.ndarray:
    """For each listed head and query row t, max_{t' <= t} scale * sum_i |q_t,i k_t',i|. [n_heads_sel, n_rows]."""
    q = np.asarray(q, np.float64)
    Tq, H, _ = q.shape
    off = np.asarray(kv_latent_bits).shape[0] - Tq
    heads = list(range(H)) if heads is None else list(heads)
    rows = list(range(Tq)) if rows is None else list(rows)
    need = off + max(rows) + 1 if rows else 0
    pe = np.abs(bf16_decode(k_pe_bits[:need]))
    mag = np.empty((len(heads), len(rows)))
    for j, h in enumerate(heads):
        k_h, _ = expand_latent(kv_latent_bits[:need], wkv_b_bits, H, staged, heads=[h])
        k = np.concatenate([np.abs(k_h[:, 0, :]), pe], axis=1)
        for i, r in enumerate(rows):
            mag[j, i] = scale * np.max(k[: off + r + 1] @ np.abs(q[r, h]))
    return mag
