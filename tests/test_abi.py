"""C ABI checks that need no GPU: the library loads, exports every function include/mla.h declares,
and host-side validation rejects bad arguments before any HIP call (fake pointers are never used)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

binding = pytest.importorskip("head_latent_attention_fp32_amd.binding")


def _lib():
    try:
        return binding.lib()
    except ImportError as e:  # pragma: no cover - build() runs before the suite
        pytest.skip(str(e))


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for f in ("mla_query_path", "mla_query_path_workspace_size", "mla_decode", "mla_prefill",
              "mla_decode_workspace_size",
              "mla_prefill_workspace_size", "mla_status_string", "mla_prefill_with_prefix", "mla_kv_append",
              "mla_decode_sparse", "mla_decode_sparse_workspace_size", "mla_output_proj",
              "mla_output_proj_workspace_size"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def _dims(h=128):
    d = binding.MlaDims()
    assert _lib().mla_dims_default(h, ctypes.byref(d)) == 0
    return d


def test_dims_default_values():
    d = _dims(64)
    assert (d.n_heads, d.q_lora_rank, d.kv_lora_rank, d.qk_nope_dim, d.qk_rope_dim, d.v_head_dim) == (
        64, 1536, 512, 128, 64, 128)
    assert abs(d.softmax_scale - 192 ** -0.5) < 1e-8 and abs(d.rms_eps - 1e-6) < 1e-12
    bad = binding.MlaDims()
    assert _lib().mla_dims_default(48, ctypes.byref(bad)) == 2


FAKE = 0x10000          # 16-byte aligned, never dereferenced
MIS = 0x10002           # misaligned


def test_query_path_workspace_size():
    lib = _lib()
    d = _dims()
    n = ctypes.c_size_t(7)
    assert lib.mla_query_path_workspace_size(ctypes.byref(d), 32, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.mla_query_path_workspace_size(ctypes.byref(d), 33, ctypes.byref(n)) == 0
    assert n.value >= 33 * (1536 * 2 + 4) and n.value % 256 == 0
    assert lib.mla_query_path_workspace_size(ctypes.byref(d), -1, ctypes.byref(n)) == 3
    assert lib.mla_query_path_workspace_size(ctypes.byref(d), 65535 * 128 + 1, ctypes.byref(n)) == 3
    assert lib.mla_query_path_workspace_size(ctypes.byref(d), 4, None) == 1


def test_query_path_validation():
    lib = _lib()
    d = _dims()
    q = lib.mla_query_path
    assert q(None, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    assert q(ctypes.byref(d), -1, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 3
    assert q(ctypes.byref(d), 0, None, None, None, None, None, None, None, 0, None) == 0       # nothing to do
    assert q(ctypes.byref(d), 4, None, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    assert q(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, MIS, None, None, 0, None) == 4
    assert q(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, FAKE, MIS, None, 0, None) == 4
    d2 = _dims()
    d2.q_lora_rank = 1024
    assert q(ctypes.byref(d2), 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 2
    d3 = _dims()
    d3.softmax_scale = float("nan")
    assert q(ctypes.byref(d3), 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    # above 32 tokens a workspace is required and checked
    n = ctypes.c_size_t(0)
    assert lib.mla_query_path_workspace_size(ctypes.byref(d), 100, ctypes.byref(n)) == 0
    assert q(ctypes.byref(d), 100, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    assert q(ctypes.byref(d), 100, FAKE, FAKE, FAKE, FAKE, FAKE, None, MIS, n.value, None) == 4
    assert q(ctypes.byref(d), 100, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, n.value - 1, None) == 5


def test_packed_query_weights_validation():
    lib = _lib()
    d = _dims()
    pk = lib.mla_wq_b_pack
    assert pk(None, FAKE, FAKE, None) == 1
    assert pk(ctypes.byref(d), None, FAKE, None) == 1
    assert pk(ctypes.byref(d), FAKE, None, None) == 1
    assert pk(ctypes.byref(d), MIS, FAKE, None) == 4
    assert pk(ctypes.byref(d), FAKE, MIS, None) == 4
    # not in place: overlapping byte ranges are rejected before any launch
    size = 1536 * d.n_heads * 192 * 2
    assert pk(ctypes.byref(d), FAKE, FAKE, None) == 1
    assert pk(ctypes.byref(d), FAKE, FAKE + size - 16, None) == 1
    assert pk(ctypes.byref(d), FAKE + size - 16, FAKE, None) == 1
    bad = _dims()
    bad.n_heads = 48
    assert pk(ctypes.byref(bad), FAKE, FAKE, None) == 2
    # the packed query path validates as mla_query_path does
    q = lib.mla_query_path_packed
    assert q(None, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    assert q(ctypes.byref(d), -1, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 3
    assert q(ctypes.byref(d), 0, None, None, None, None, None, None, None, 0, None) == 0
    assert q(ctypes.byref(d), 4, FAKE, FAKE, None, FAKE, FAKE, None, None, 0, None) == 1
    assert q(ctypes.byref(d), 4, FAKE, FAKE, MIS, FAKE, FAKE, None, None, 0, None) == 4
    n = ctypes.c_size_t(0)
    assert lib.mla_query_path_workspace_size(ctypes.byref(d), 100, ctypes.byref(n)) == 0
    assert q(ctypes.byref(d), 100, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, n.value - 1, None) == 5


def test_decode_validation_and_workspace():
    lib = _lib()
    d = _dims()
    n = ctypes.c_size_t(0)
    assert lib.mla_decode_workspace_size(ctypes.byref(d), 32, 4096, ctypes.byref(n)) == 0
    need = n.value
    assert need > 32 * 128 * 512 * 2 * 2          # at least q_lat and o_lat
    assert lib.mla_decode_workspace_size(ctypes.byref(d), -1, 4096, ctypes.byref(n)) == 3
    assert lib.mla_decode_workspace_size(ctypes.byref(d), 1, -5, ctypes.byref(n)) == 3
    assert lib.mla_decode_workspace_size(ctypes.byref(d), 1, (1 << 21) + 1, ctypes.byref(n)) == 3
    assert lib.mla_decode_workspace_size(ctypes.byref(d), 0, 10, ctypes.byref(n)) == 0 and n.value == 0
    dec = lib.mla_decode
    args = lambda **kw: [kw.get(k, v) for k, v in [
        ("dims", ctypes.byref(d)), ("batch", 32), ("q", FAKE), ("w", FAKE), ("kv", FAKE), ("pe", FAKE),
        ("off", None), ("lens", FAKE), ("maxl", 4096), ("ws", FAKE), ("wsb", need), ("out", FAKE),
        ("lse", None), ("stream", None)]]
    assert dec(*args(batch=0, q=None)) == 0
    assert dec(*args(batch=-2)) == 3
    assert dec(*args(maxl=-1)) == 3
    assert dec(*args(kv=None)) == 1
    assert dec(*args(lens=None)) == 1
    assert dec(*args(ws=None)) == 1
    assert dec(*args(pe=MIS)) == 4
    assert dec(*args(off=MIS)) == 4
    assert dec(*args(lse=MIS)) == 4
    assert dec(*args(wsb=need - 1)) == 5
    d2 = _dims()
    d2.n_heads = 96
    assert dec(*args(dims=ctypes.byref(d2))) == 2


def test_prefill_validation_and_workspace():
    lib = _lib()
    d = _dims()
    n = ctypes.c_size_t(0)
    assert lib.mla_prefill_workspace_size(ctypes.byref(d), 1, 4096, ctypes.byref(n)) == 0
    assert n.value >= 1 * 128 * 4096 * 256 * 2      # expanded k_nope and values
    need = n.value
    pf = lib.mla_prefill
    assert pf(ctypes.byref(d), 1, 0, None, None, None, None, None, 0, None, None, None) == 0
    assert pf(ctypes.byref(d), 1, -3, FAKE, FAKE, FAKE, FAKE, FAKE, need, FAKE, None, None) == 3
    assert pf(ctypes.byref(d), 1, 4096, FAKE, None, FAKE, FAKE, FAKE, need, FAKE, None, None) == 1
    assert pf(ctypes.byref(d), 1, 4096, FAKE, FAKE, MIS, FAKE, FAKE, need, FAKE, None, None) == 4
    assert pf(ctypes.byref(d), 1, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, need - 256, FAKE, None, None) == 5
    # at most 2^23 key positions over the batch, at most 65535 sequences (the 32-bit grids and byte
    # ranges of the expansion and attention stay far from wrapping)
    big = 1 << 23
    assert lib.mla_prefill_workspace_size(ctypes.byref(d), 1, big, ctypes.byref(n)) == 0
    assert lib.mla_prefill_workspace_size(ctypes.byref(d), 1, big + 1, ctypes.byref(n)) == 3
    assert lib.mla_prefill_workspace_size(ctypes.byref(d), 2, big // 2 + 1, ctypes.byref(n)) == 3
    assert lib.mla_prefill_workspace_size(ctypes.byref(d), 65536, 1, ctypes.byref(n)) == 3
    assert pf(ctypes.byref(d), 1, big + 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 62, FAKE, None, None) == 3
    assert pf(ctypes.byref(d), 4, big // 4 + 64, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 62, FAKE, None, None) == 3


def test_prefill_with_prefix_validation():
    lib = _lib()
    d = _dims()
    n = ctypes.c_size_t(0)
    assert lib.mla_prefill_workspace_size(ctypes.byref(d), 1, 4096, ctypes.byref(n)) == 0
    need = n.value
    pf = lib.mla_prefill_with_prefix
    args = lambda **kw: [kw.get(k, v) for k, v in [
        ("dims", ctypes.byref(d)), ("batch", 1), ("q_len", 1024), ("kv_len", 4096), ("q", FAKE), ("lat", FAKE),
        ("pe", FAKE), ("w", FAKE), ("ws", FAKE), ("wsb", need), ("out", FAKE), ("lse", None), ("stream", None)]]
    assert pf(*args(q_len=0, q=None)) == 0
    assert pf(*args(kv_len=1023)) == 3                 # fewer keys than queries
    assert pf(*args(q_len=-1)) == 3
    assert pf(*args(lat=None)) == 1
    assert pf(*args(lse=MIS)) == 4
    assert pf(*args(wsb=need - 1)) == 5
    assert pf(*args(kv_len=(1 << 23) + 1, wsb=1 << 62)) == 3   # more than 2^23 key positions
    assert pf(*args(batch=3, kv_len=(1 << 23) // 3 + 1, wsb=1 << 62)) == 3


def test_kv_append_validation():
    lib = _lib()
    d = _dims()
    ap = lib.mla_kv_append
    args = lambda **kw: [kw.get(k, v) for k, v in [
        ("dims", ctypes.byref(d)), ("batch", 4), ("seqlen", 1), ("kv_a", FAKE), ("g", FAKE), ("cs", FAKE),
        ("start", FAKE), ("off", None), ("maxl", 4096), ("kv", FAKE), ("pe", FAKE), ("stream", None)]]
    assert ap(*args(batch=0, kv_a=None)) == 0
    assert ap(*args(seqlen=-1)) == 3
    assert ap(*args(maxl=(1 << 21) + 1)) == 3
    assert ap(*args(start=None)) == 1
    assert ap(*args(pe=None)) == 1
    assert ap(*args(off=MIS)) == 4
    assert ap(*args(kv_a=MIS)) == 4
    d2 = _dims()
    d2.kv_lora_rank = 256
    assert ap(*args(dims=ctypes.byref(d2))) == 2


def test_decode_noalloc_validation():
    """mla_decode_noalloc validates like mla_decode and rejects, before any HIP call, a batch whose
    scratch (mla_decode_workspace_size) exceeds the library's fixed array."""
    lib = _lib()
    d = _dims()
    f = lib.mla_decode_noalloc
    args = lambda **kw: [kw.get(k, v) for k, v in [
        ("dims", ctypes.byref(d)), ("batch", 4096), ("q", FAKE), ("w", FAKE), ("kv", FAKE), ("pe", FAKE),
        ("off", None), ("lens", FAKE), ("max_seqlen", 4096), ("out", FAKE), ("lse", None), ("stream", None)]]
    n = ctypes.c_size_t(0)
    assert lib.mla_decode_workspace_size(ctypes.byref(d), 4096, 4096, ctypes.byref(n)) == 0
    assert n.value > binding.DECODE_NOALLOC_SCRATCH_BYTES
    assert f(*args()) == 5                                   # scratch too small for this batch
    assert f(*args(batch=0, q=None)) == 0                    # nothing to do
    assert f(*args(batch=-1)) == 3
    assert f(*args(max_seqlen=(1 << 21) + 1)) == 3
    assert f(*args(out=None)) == 1
    assert f(*args(lens=MIS)) == 4
    d2 = _dims()
    d2.n_heads = 96
    assert f(*args(dims=ctypes.byref(d2))) == 2


def test_decode_sparse_validation():
    lib = _lib()
    d = _dims()
    n = ctypes.c_size_t(0)
    assert lib.mla_decode_sparse_workspace_size(ctypes.byref(d), 32, 4096, 2048, ctypes.byref(n)) == 0
    need = n.value
    m = ctypes.c_size_t(0)
    assert lib.mla_decode_workspace_size(ctypes.byref(d), 32, 4096, ctypes.byref(m)) == 0
    assert need > 32 * 2048 * 4                        # holds the compacted lists
    assert lib.mla_decode_sparse_workspace_size(ctypes.byref(d), 32, 4096, -1, ctypes.byref(n)) == 3
    assert lib.mla_decode_sparse_workspace_size(ctypes.byref(d), 32, 4096, (1 << 21) + 1, ctypes.byref(n)) == 3
    sp = lib.mla_decode_sparse
    args = lambda **kw: [kw.get(k, v) for k, v in [
        ("dims", ctypes.byref(d)), ("batch", 32), ("q", FAKE), ("w", FAKE), ("kv", FAKE), ("pe", FAKE),
        ("off", None), ("lens", FAKE), ("maxl", 4096), ("idx", FAKE), ("k", 2048), ("ws", FAKE), ("wsb", need),
        ("out", FAKE), ("lse", None), ("stream", None)]]
    assert sp(*args(batch=0, q=None)) == 0
    assert sp(*args(idx=None)) == 1
    assert sp(*args(k=-3)) == 3
    assert sp(*args(idx=MIS)) == 4
    assert sp(*args(wsb=need - 1)) == 5


def test_output_proj_validation():
    lib = _lib()
    d = _dims()
    n = ctypes.c_size_t(7)
    assert lib.mla_output_proj_workspace_size(ctypes.byref(d), 32, 7168, ctypes.byref(n)) == 0
    need = n.value
    assert need >= 2 * 32 * 7168 * 4                    # fp32 partials of the K-slices
    assert lib.mla_output_proj_workspace_size(ctypes.byref(d), 4096, 7168, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.mla_output_proj_workspace_size(ctypes.byref(d), 128, 7168, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.mla_output_proj_workspace_size(ctypes.byref(d), 32, 7000, ctypes.byref(n)) == 3   # not x64
    assert lib.mla_output_proj_workspace_size(ctypes.byref(d), 1 << 20, 7168, ctypes.byref(n)) == 3
    op = lib.mla_output_proj
    assert op(ctypes.byref(d), 0, 7168, None, None, None, 0, None, None) == 0
    assert op(ctypes.byref(d), 32, 7168, FAKE, FAKE, None, 0, FAKE, None) == 1      # workspace needed
    assert op(ctypes.byref(d), 32, 7168, FAKE, None, FAKE, need, FAKE, None) == 1
    assert op(ctypes.byref(d), 32, 7168, MIS, FAKE, FAKE, need, FAKE, None) == 4
    assert op(ctypes.byref(d), 32, 7168, FAKE, FAKE, FAKE, need - 1, FAKE, None) == 5
    assert op(ctypes.byref(d), 32, 0, FAKE, FAKE, FAKE, need, FAKE, None) == 3


def test_status_strings():
    lib = _lib()
    for s in range(7):
        assert lib.mla_status_string(s).decode().startswith(binding.STATUS_NAMES[s])
    assert lib.mla_version().decode().count(".") == 2


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(binding, "_LIB", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libmla.so")
    with pytest.raises(ImportError):
        binding.lib()


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "head_latent_attention_fp32_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "mla_oracle" not in src, f
