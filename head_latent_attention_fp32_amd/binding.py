"""Python binding of libmla (ctypes): argument marshalling only.

Each function checks tensor dtypes, shapes, devices and contiguity, passes raw device pointers and
the current HIP stream to the C ABI of include/mla.h, and raises on a non-zero status. Every step of
the computation runs in the library's HIP kernels; there is no other code path. Importing this
module raises if libmla.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK = 0
STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_SHAPE",
                4: "MLA_ERR_ALIGNMENT", 5: "MLA_ERR_WORKSPACE", 6: "MLA_ERR_HIP"}

Q_LORA, KV_LORA, NOPE, ROPE, V_DIM = 1536, 512, 128, 64, 128
QK = NOPE + ROPE


class MlaDims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("q_lora_rank", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_nope_dim", ctypes.c_int32), ("qk_rope_dim", ctypes.c_int32), ("v_head_dim", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib().mla_status_string(status).decode()}")


_LIB = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmla.so is not built ({LIB_PATH}); run python -m head_latent_attention_fp32_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(MlaDims)
        lib.mla_dims_default.argtypes = [_I32, dp]
        lib.mla_query_path_workspace_size.argtypes = [dp, _I64, ctypes.POINTER(_SZ)]
        lib.mla_query_path.argtypes = [dp, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
        lib.mla_query_path_packed.argtypes = [dp, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
        lib.mla_wq_b_pack.argtypes = [dp, _P, _P, _P]
        lib.mla_decode_workspace_size.argtypes = [dp, _I32, _I64, ctypes.POINTER(_SZ)]
        lib.mla_decode.argtypes = [dp, _I32, _P, _P, _P, _P, _P, _P, _I64, _P, _SZ, _P, _P, _P]
        lib.mla_prefill_workspace_size.argtypes = [dp, _I32, _I32, ctypes.POINTER(_SZ)]
        lib.mla_prefill.argtypes = [dp, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P, _P, _P]
        lib.mla_decode_sparse_workspace_size.argtypes = [dp, _I32, _I64, _I32, ctypes.POINTER(_SZ)]
        lib.mla_decode_sparse.argtypes = [dp, _I32, _P, _P, _P, _P, _P, _P, _I64, _P, _I32, _P, _SZ, _P, _P, _P]
        lib.mla_output_proj_workspace_size.argtypes = [dp, _I64, _I32, ctypes.POINTER(_SZ)]
        lib.mla_output_proj.argtypes = [dp, _I64, _I32, _P, _P, _P, _SZ, _P, _P]
        lib.mla_prefill_with_prefix.argtypes = [dp, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P, _P, _P]
        lib.mla_kv_append.argtypes = [dp, _I32, _I32, _P, _P, _P, _P, _P, _I64, _P, _P, _P]
        lib.mla_decode_noalloc.argtypes = [dp, _I32, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _P]
        for f in ("mla_dims_default", "mla_query_path_workspace_size", "mla_query_path", "mla_decode_workspace_size",
                  "mla_decode", "mla_prefill_workspace_size", "mla_prefill", "mla_prefill_with_prefix",
                  "mla_kv_append", "mla_decode_sparse_workspace_size", "mla_decode_sparse",
                  "mla_output_proj_workspace_size", "mla_output_proj", "mla_decode_noalloc", "mla_wq_b_pack",
                  "mla_query_path_packed"):
            getattr(lib, f).restype = ctypes.c_int
        lib.mla_status_string.argtypes = [ctypes.c_int]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_version.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _lib()


def dims(n_heads: int, softmax_scale: Optional[float] = None, rms_eps: Optional[float] = None) -> MlaDims:
    d = MlaDims()
    st = _lib().mla_dims_default(n_heads, ctypes.byref(d))
    if st != MLA_OK:
        raise MlaError(st, "mla_dims_default")
    if softmax_scale is not None:
        d.softmax_scale = softmax_scale
    if rms_eps is not None:
        d.rms_eps = rms_eps
    return d


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check(status: int, what: str) -> None:
    if status != MLA_OK:
        raise MlaError(status, what)


def query_path_workspace_size(n_heads: int, n_tokens: int, d: Optional[MlaDims] = None) -> int:
    d = d or dims(n_heads)
    n = _SZ(0)
    _check(_lib().mla_query_path_workspace_size(ctypes.byref(d), n_tokens, ctypes.byref(n)),
           "mla_query_path_workspace_size")
    return n.value


def wq_b_pack(wq_b: torch.Tensor, n_heads: int, out: Optional[torch.Tensor] = None,
              d: Optional[MlaDims] = None) -> torch.Tensor:
    """wq_b bf16 [1536, H*192] -> the packed copy bf16 [H*192/32, 1536, 32] that query_path(...,
    packed=True) reads (out[g, k, j] = wq_b[k, 32 g + j])."""
    d = d or dims(n_heads)
    _need(wq_b, "wq_b", torch.bfloat16, (Q_LORA, n_heads * QK))
    shape = (n_heads * QK // 32, Q_LORA, 32)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=wq_b.device)
    _need(out, "out", torch.bfloat16, shape)
    _check(_lib().mla_wq_b_pack(ctypes.byref(d), _ptr(wq_b), _ptr(out), _stream()), "mla_wq_b_pack")
    return out


def query_path(q_latent: torch.Tensor, q_norm_w: torch.Tensor, wq_b: torch.Tensor, rope_cs: torch.Tensor,
               n_heads: int, q_out: Optional[torch.Tensor] = None, inv_rms: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, d: Optional[MlaDims] = None, packed: bool = False
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q_latent bf16 [n, 1536] (or [..., 1536]), q_norm_w fp32 [1536], wq_b bf16 [1536, H*192]
    (packed=True: the [H*192/32, 1536, 32] copy from wq_b_pack, through mla_query_path_packed),
    rope_cs fp32 [n, 32, 2] -> q_out bf16 [n, H, 192] (and inv_rms fp32 [n] if given). The workspace
    (uint8, needed above 32 tokens) is allocated when not given."""
    d = d or dims(n_heads)
    lead = tuple(q_latent.shape[:-1])
    n = 1
    for s in lead:
        n *= s
    _need(q_latent, "q_latent", torch.bfloat16)
    if q_latent.shape[-1] != Q_LORA:
        raise ValueError("q_latent last dim must be 1536")
    _need(q_norm_w, "q_norm_w", torch.float32, (Q_LORA,))
    _need(wq_b, "wq_b", torch.bfloat16, (n_heads * QK // 32, Q_LORA, 32) if packed else (Q_LORA, n_heads * QK))
    _need(rope_cs, "rope_cs", torch.float32)
    if rope_cs.numel() != n * (ROPE // 2) * 2:
        raise ValueError("rope_cs must hold one (cos, sin) row of 32 pairs per token")
    if q_out is None:
        q_out = torch.empty(lead + (n_heads, QK), dtype=torch.bfloat16, device=q_latent.device)
    _need(q_out, "q_out", torch.bfloat16, lead + (n_heads, QK))
    if inv_rms is not None:
        _need(inv_rms, "inv_rms", torch.float32)
        if inv_rms.numel() != n:
            raise ValueError("inv_rms must hold one value per token")
    ws_bytes = query_path_workspace_size(n_heads, n, d)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q_latent.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    fn = _lib().mla_query_path_packed if packed else _lib().mla_query_path
    _check(fn(ctypes.byref(d), n, _ptr(q_latent), _ptr(q_norm_w), _ptr(wq_b), _ptr(rope_cs), _ptr(q_out),
              _ptr(inv_rms), _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream()),
           "mla_query_path_packed" if packed else "mla_query_path")
    return q_out, inv_rms


def decode_workspace_size(n_heads: int, batch: int, max_seqlen: int, d: Optional[MlaDims] = None) -> int:
    d = d or dims(n_heads)
    n = _SZ(0)
    _check(_lib().mla_decode_workspace_size(ctypes.byref(d), batch, max_seqlen, ctypes.byref(n)),
           "mla_decode_workspace_size")
    return n.value


def decode(q: torch.Tensor, wkv_b: torch.Tensor, kv_cache: torch.Tensor, pe_cache: torch.Tensor,
           cache_seqlens: torch.Tensor, max_seqlen: int, cache_row_offset: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, d: Optional[MlaDims] = None
           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q bf16 [B, H, 192]; wkv_b bf16 [H*256, 512]; kv_cache bf16 [rows, 512]; pe_cache bf16 [rows, 64];
    cache_seqlens int32 [B]; cache_row_offset int64 [B] or None (row b*max_seqlen) -> out bf16 [B, H, 128]."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != QK:
        raise ValueError("q must be [B, H, 192]")
    B, H = int(q.shape[0]), int(q.shape[1])
    d = d or dims(H)
    _need(wkv_b, "wkv_b", torch.bfloat16, (H * (NOPE + V_DIM), KV_LORA))
    _need(kv_cache, "kv_cache", torch.bfloat16)
    _need(pe_cache, "pe_cache", torch.bfloat16)
    if kv_cache.shape[-1] != KV_LORA or pe_cache.shape[-1] != ROPE:
        raise ValueError("kv_cache rows must be 512 wide and pe_cache rows 64 wide")
    if kv_cache.numel() // KV_LORA != pe_cache.numel() // ROPE:
        raise ValueError("kv_cache and pe_cache must hold the same number of rows")
    _need(cache_seqlens, "cache_seqlens", torch.int32, (B,))
    if cache_row_offset is not None:
        _need(cache_row_offset, "cache_row_offset", torch.int64, (B,))
    elif kv_cache.numel() // KV_LORA < B * max_seqlen:
        raise ValueError("padded caches (no row offsets) need batch * max_seqlen rows")
    need = decode_workspace_size(H, B, max_seqlen, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((B, H, V_DIM), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, H, V_DIM))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H))
    _check(_lib().mla_decode(ctypes.byref(d), B, _ptr(q), _ptr(wkv_b), _ptr(kv_cache), _ptr(pe_cache),
                             _ptr(cache_row_offset), _ptr(cache_seqlens), int(max_seqlen), _ptr(workspace),
                             workspace.numel(), _ptr(out), _ptr(lse), _stream()), "mla_decode")
    return out, lse


DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_noalloc(q: torch.Tensor, wkv_b: torch.Tensor, kv_cache: torch.Tensor, pe_cache: torch.Tensor,
                   cache_seqlens: torch.Tensor, max_seqlen: int, cache_row_offset: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   d: Optional[MlaDims] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """mla_decode_noalloc: decode as decode() does, with the library's fixed device scratch in place of
    a workspace (at most DECODE_NOALLOC_SCRATCH_BYTES of it; larger batches raise). The library
    allocates nothing; `out` is allocated here only when not given."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != QK:
        raise ValueError("q must be [B, H, 192]")
    B, H = int(q.shape[0]), int(q.shape[1])
    d = d or dims(H)
    _need(wkv_b, "wkv_b", torch.bfloat16, (H * (NOPE + V_DIM), KV_LORA))
    _need(kv_cache, "kv_cache", torch.bfloat16)
    _need(pe_cache, "pe_cache", torch.bfloat16)
    if kv_cache.shape[-1] != KV_LORA or pe_cache.shape[-1] != ROPE:
        raise ValueError("kv_cache rows must be 512 wide and pe_cache rows 64 wide")
    if kv_cache.numel() // KV_LORA != pe_cache.numel() // ROPE:
        raise ValueError("kv_cache and pe_cache must hold the same number of rows")
    _need(cache_seqlens, "cache_seqlens", torch.int32, (B,))
    if cache_row_offset is not None:
        _need(cache_row_offset, "cache_row_offset", torch.int64, (B,))
    elif kv_cache.numel() // KV_LORA < B * max_seqlen:
        raise ValueError("padded caches (no row offsets) need batch * max_seqlen rows")
    if out is None:
        out = torch.empty((B, H, V_DIM), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, H, V_DIM))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H))
    _check(_lib().mla_decode_noalloc(ctypes.byref(d), B, _ptr(q), _ptr(wkv_b), _ptr(kv_cache), _ptr(pe_cache),
                                     _ptr(cache_row_offset), _ptr(cache_seqlens), int(max_seqlen), _ptr(out),
                                     _ptr(lse), _stream()), "mla_decode_noalloc")
    return out, lse


def prefill_workspace_size(n_heads: int, batch: int, seqlen: int, d: Optional[MlaDims] = None) -> int:
    d = d or dims(n_heads)
    n = _SZ(0)
    _check(_lib().mla_prefill_workspace_size(ctypes.byref(d), batch, seqlen, ctypes.byref(n)),
           "mla_prefill_workspace_size")
    return n.value


def prefill(q: torch.Tensor, kv_latent: torch.Tensor, k_pe: torch.Tensor, wkv_b: torch.Tensor,
            workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, d: Optional[MlaDims] = None
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q bf16 [B, T, H, 192]; kv_latent bf16 [B, T, 512]; k_pe bf16 [B, T, 64]; wkv_b bf16 [H*256, 512]
    -> out bf16 [B, T, H, 128] (and lse fp32 [B, H, T] if given)."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 4 or q.shape[3] != QK:
        raise ValueError("q must be [B, T, H, 192]")
    B, T, H = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    d = d or dims(H)
    _need(kv_latent, "kv_latent", torch.bfloat16, (B, T, KV_LORA))
    _need(k_pe, "k_pe", torch.bfloat16, (B, T, ROPE))
    _need(wkv_b, "wkv_b", torch.bfloat16, (H * (NOPE + V_DIM), KV_LORA))
    need = prefill_workspace_size(H, B, T, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((B, T, H, V_DIM), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, T, H, V_DIM))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H, T))
    _check(_lib().mla_prefill(ctypes.byref(d), B, T, _ptr(q), _ptr(kv_latent), _ptr(k_pe), _ptr(wkv_b),
                              _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream()), "mla_prefill")
    return out, lse


def prefill_with_prefix(q: torch.Tensor, kv_latent: torch.Tensor, k_pe: torch.Tensor, wkv_b: torch.Tensor,
                        workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, d: Optional[MlaDims] = None
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q bf16 [B, Tq, H, 192] for the last Tq of S positions; kv_latent bf16 [B, S, 512]; k_pe bf16
    [B, S, 64]; wkv_b bf16 [H*256, 512] -> out bf16 [B, Tq, H, 128] (and lse fp32 [B, H, Tq] if given)."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 4 or q.shape[3] != QK:
        raise ValueError("q must be [B, Tq, H, 192]")
    B, Tq, H = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    d = d or dims(H)
    _need(kv_latent, "kv_latent", torch.bfloat16)
    if kv_latent.dim() != 3 or kv_latent.shape[0] != B or kv_latent.shape[2] != KV_LORA:
        raise ValueError("kv_latent must be [B, S, 512]")
    S = int(kv_latent.shape[1])
    _need(k_pe, "k_pe", torch.bfloat16, (B, S, ROPE))
    _need(wkv_b, "wkv_b", torch.bfloat16, (H * (NOPE + V_DIM), KV_LORA))
    need = prefill_workspace_size(H, B, S, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((B, Tq, H, V_DIM), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, Tq, H, V_DIM))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H, Tq))
    _check(_lib().mla_prefill_with_prefix(ctypes.byref(d), B, Tq, S, _ptr(q), _ptr(kv_latent), _ptr(k_pe),
                                          _ptr(wkv_b), _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
                                          _stream()), "mla_prefill_with_prefix")
    return out, lse


def kv_append(kv_a: torch.Tensor, kv_norm_w: torch.Tensor, rope_cs: torch.Tensor, start_pos: torch.Tensor,
              kv_cache: torch.Tensor, pe_cache: torch.Tensor, max_seqlen: int,
              cache_row_offset: Optional[torch.Tensor] = None, d: Optional[MlaDims] = None,
              n_heads: int = 128) -> None:
    """kv_a bf16 [B, T, 576]; kv_norm_w fp32 [512]; rope_cs fp32 [B, T, 32, 2]; start_pos int32 [B];
    kv_cache bf16 [rows, 512] and pe_cache bf16 [rows, 64], written in place at rows
    cache_row_offset[b] (or b*max_seqlen) + start_pos[b] + t."""
    d = d or dims(n_heads)
    _need(kv_a, "kv_a", torch.bfloat16)
    if kv_a.dim() != 3 or kv_a.shape[2] != KV_LORA + ROPE:
        raise ValueError("kv_a must be [B, T, 576]")
    B, T = int(kv_a.shape[0]), int(kv_a.shape[1])
    _need(kv_norm_w, "kv_norm_w", torch.float32, (KV_LORA,))
    _need(rope_cs, "rope_cs", torch.float32, (B, T, ROPE // 2, 2))
    _need(start_pos, "start_pos", torch.int32, (B,))
    _need(kv_cache, "kv_cache", torch.bfloat16)
    _need(pe_cache, "pe_cache", torch.bfloat16)
    if kv_cache.shape[-1] != KV_LORA or pe_cache.shape[-1] != ROPE:
        raise ValueError("kv_cache rows must be 512 wide and pe_cache rows 64 wide")
    if kv_cache.numel() // KV_LORA != pe_cache.numel() // ROPE:
        raise ValueError("kv_cache and pe_cache must hold the same number of rows")
    if cache_row_offset is not None:
        _need(cache_row_offset, "cache_row_offset", torch.int64, (B,))
    elif kv_cache.numel() // KV_LORA < B * max_seqlen:
        raise ValueError("padded caches (no row offsets) need batch * max_seqlen rows")
    _check(_lib().mla_kv_append(ctypes.byref(d), B, T, _ptr(kv_a), _ptr(kv_norm_w), _ptr(rope_cs), _ptr(start_pos),
                                _ptr(cache_row_offset), int(max_seqlen), _ptr(kv_cache), _ptr(pe_cache), _stream()),
           "mla_kv_append")


def decode_sparse_workspace_size(n_heads: int, batch: int, max_seqlen: int, topk: int,
                                 d: Optional[MlaDims] = None) -> int:
    d = d or dims(n_heads)
    n = _SZ(0)
    _check(_lib().mla_decode_sparse_workspace_size(ctypes.byref(d), batch, max_seqlen, topk, ctypes.byref(n)),
           "mla_decode_sparse_workspace_size")
    return n.value


def decode_sparse(q: torch.Tensor, wkv_b: torch.Tensor, kv_cache: torch.Tensor, pe_cache: torch.Tensor,
                  cache_seqlens: torch.Tensor, max_seqlen: int, topk_indices: torch.Tensor,
                  cache_row_offset: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  d: Optional[MlaDims] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """decode() restricted to the positions topk_indices (int32 [B, k]) names for each sequence."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != QK:
        raise ValueError("q must be [B, H, 192]")
    B, H = int(q.shape[0]), int(q.shape[1])
    d = d or dims(H)
    _need(wkv_b, "wkv_b", torch.bfloat16, (H * (NOPE + V_DIM), KV_LORA))
    _need(kv_cache, "kv_cache", torch.bfloat16)
    _need(pe_cache, "pe_cache", torch.bfloat16)
    if kv_cache.shape[-1] != KV_LORA or pe_cache.shape[-1] != ROPE:
        raise ValueError("kv_cache rows must be 512 wide and pe_cache rows 64 wide")
    if kv_cache.numel() // KV_LORA != pe_cache.numel() // ROPE:
        raise ValueError("kv_cache and pe_cache must hold the same number of rows")
    _need(cache_seqlens, "cache_seqlens", torch.int32, (B,))
    _need(topk_indices, "topk_indices", torch.int32)
    if topk_indices.dim() != 2 or topk_indices.shape[0] != B:
        raise ValueError("topk_indices must be [B, k]")
    k = int(topk_indices.shape[1])
    if cache_row_offset is not None:
        _need(cache_row_offset, "cache_row_offset", torch.int64, (B,))
    elif kv_cache.numel() // KV_LORA < B * max_seqlen:
        raise ValueError("padded caches (no row offsets) need batch * max_seqlen rows")
    need = decode_sparse_workspace_size(H, B, max_seqlen, k, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((B, H, V_DIM), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, H, V_DIM))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H))
    _check(_lib().mla_decode_sparse(ctypes.byref(d), B, _ptr(q), _ptr(wkv_b), _ptr(kv_cache), _ptr(pe_cache),
                                    _ptr(cache_row_offset), _ptr(cache_seqlens), int(max_seqlen),
                                    _ptr(topk_indices) if k else None, k, _ptr(workspace), workspace.numel(),
                                    _ptr(out), _ptr(lse), _stream()), "mla_decode_sparse")
    return out, lse


def output_proj_workspace_size(n_heads: int, n_tokens: int, dim: int, d: Optional[MlaDims] = None) -> int:
    d = d or dims(n_heads)
    n = _SZ(0)
    _check(_lib().mla_output_proj_workspace_size(ctypes.byref(d), n_tokens, dim, ctypes.byref(n)),
           "mla_output_proj_workspace_size")
    return n.value


def output_proj(x: torch.Tensor, wo: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                y: Optional[torch.Tensor] = None, d: Optional[MlaDims] = None) -> torch.Tensor:
    """x bf16 [..., H, 128] or [..., H*128]; wo bf16 [dim, H*128] -> y bf16 [..., dim]."""
    _need(x, "x", torch.bfloat16)
    _need(wo, "wo", torch.bfloat16)
    if wo.dim() != 2 or wo.shape[1] % V_DIM:
        raise ValueError("wo must be [dim, H*128]")
    dim, K = int(wo.shape[0]), int(wo.shape[1])
    H = K // V_DIM
    d = d or dims(H)
    if x.numel() % K:
        raise ValueError("x must hold H*128 features per token")
    n = x.numel() // K
    lead = tuple(x.shape[:-2]) if x.shape[-1] == V_DIM and x.dim() >= 2 and x.shape[-2] == H else tuple(x.shape[:-1])
    need = output_proj_workspace_size(H, n, dim, d)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    if y is None:
        y = torch.empty(lead + (dim,), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16)
    if y.numel() != n * dim:
        raise ValueError("y must be [n_tokens, dim]")
    _check(_lib().mla_output_proj(ctypes.byref(d), n, dim, _ptr(x), _ptr(wo), _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _ptr(y), _stream()),
           "mla_output_proj")
    return y
