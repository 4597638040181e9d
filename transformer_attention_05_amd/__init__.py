"""Python binding of libmi_attn, the MI355X (gfx950) attention library.

Argument marshalling only: every function here checks that tensors are on
the GPU, takes their device pointers, sizes and the current HIP stream, and
calls the C ABI of the same name (declared in include/mi_attn.h).  There is
no CPU or PyTorch fallback; if the shared library is missing, every call
raises.  PyTorch supplies device memory and streams.

With the environment variable MI_ATTN_DEBUG=1 the debug library
(libmi_attn_debug.so: the same kernels, which also record malformed
device-side inputs for attn_debug_flags) is loaded instead of the release
one; `debug_library()` switches to it for a block of code.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np
import torch

__all__ = [
    "AttnError",
    "Pool",
    "attn_copy_blocks",
    "attn_decode_paged",
    "attn_decode_paged_auto_partition",
    "attn_decode_paged_partition_for",
    "attn_decode_paged_noalloc",
    "attn_decode_paged_rope",
    "attn_decode_paged_plan",
    "attn_decode_paged_workspace_size",
    "attn_debug_flags",
    "attn_kv_cache_write_rope",
    "attn_last_error",
    "attn_prefill",
    "attn_prefill_masked",
    "attn_residual_rms_norm",
    "attn_prefill_paged",
    "attn_prefill_paged_masked",
    "attn_prefill_paged_workspace_size",
    "attn_prefill_workspace_size",
    "debug_library",
    "lib_path",
    "load",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmi_attn.so"
LIB_DEBUG_NAME = "libmi_attn_debug.so"
BLOCK_SIZE = 16

ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_NOMEM, ATTN_E_STATE, ATTN_E_DEVICE = 0, -1, -2, -3, -4, -5
ATTN_F32, ATTN_BF16 = 0, 1
ATTN_PREFILL_SHARE_CU = 1  # attn_prefill_paged_ex flag

_c_i32 = ctypes.c_int32
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_c_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p

class _PrefillPart(ctypes.Structure):
    """attn_paged_prefill_part (mi_attn.h)."""
    _fields_ = [("q", _vp), ("block_table", _vp), ("max_blocks_per_seq", _c_i32), ("cu_seqlens_q", _vp),
                ("context_lens", _vp), ("o", _vp), ("num_seqs", _c_i32), ("total_q", _c_i32),
                ("max_seqlen_q", _c_i32), ("max_context_len", _c_i32), ("causal", _c_i32)]


class _DecodePart(ctypes.Structure):
    """attn_paged_decode_part (mi_attn.h)."""
    _fields_ = [("q", _vp), ("block_table", _vp), ("max_blocks_per_seq", _c_i32), ("context_lens", _vp),
                ("o", _vp), ("num_seqs", _c_i32), ("max_context_len", _c_i32), ("partition_size", _c_i32),
                ("plan", _vp), ("plan_items", _c_i32), ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("k_new", _vp), ("v_new", _vp), ("positions", _vp), ("slot_mapping", _vp), ("q_rot_out", _vp),
                ("rope_base", ctypes.c_float)]


_SIGNATURES = {
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_prefill_workspace_size": (ctypes.c_size_t, [_c_i32] * 6 + [ctypes.c_int]),
    "attn_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                    _c_i64p, _c_i64p, _c_i64p, _c_i64p, ctypes.c_float, _c_i32, ctypes.c_int,
                                    _vp, ctypes.c_size_t, _vp]),
    "attn_prefill_masked": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64p, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_i32, _c_i32, _c_i64p, _c_i64p, _c_i64p, _c_i64p, ctypes.c_float, _c_i32,
                                           ctypes.c_int, _vp]),
    "attn_prefill_paged_workspace_size": (ctypes.c_size_t, [_c_i32] * 7),
    "attn_prefill_paged": (ctypes.c_int, [_vp, _vp, _vp, _vp, _c_i32, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                          _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_float,
                                          _c_i32, ctypes.c_int, _vp, ctypes.c_size_t, _vp]),
    "attn_prefill_paged_ex": (ctypes.c_int, [_vp, _vp, _vp, _vp, _c_i32, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                             _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_float,
                                             _c_i32, ctypes.c_int, _c_i32, _vp, ctypes.c_size_t, _vp]),
    "attn_prefill_paged_masked": (ctypes.c_int, [_vp, _vp, _vp, _vp, _c_i32, _vp, _vp, _vp, _c_i64p, _c_i32, _vp,
                                                 _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                 _c_i32, ctypes.c_float, _c_i32, ctypes.c_int, _vp]),
    "attn_decode_paged_workspace_size": (ctypes.c_size_t, [_c_i32] * 6),
    "attn_decode_paged_auto_partition": (_c_i32, [_c_i32] * 3),
    "attn_decode_paged_partition_for": (_c_i32, [_c_i32p, _c_i32, _c_i32, _c_i32, _c_i32]),
    "attn_decode_paged": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                         _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_float, ctypes.c_int, _vp, _c_i32,
                                         _vp, ctypes.c_size_t, _vp]),
    "attn_decode_paged_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                                 _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_float,
                                                 ctypes.c_int, _vp, _c_i32, _vp]),
    "attn_decode_paged_rope": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp,
                                              _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                              _c_i32, ctypes.c_float, ctypes.c_int, _vp, _c_i32, _vp,
                                              ctypes.c_size_t, _vp]),
    "attn_decode_paged_plan": (ctypes.c_int64, [_c_i32p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32p, ctypes.c_int64]),
    "attn_prefill_decode_paged": (ctypes.c_int, [ctypes.POINTER(_PrefillPart), ctypes.POINTER(_DecodePart), _vp,
                                                 _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_float,
                                                 ctypes.c_int, _vp]),
    "attn_kv_cache_write_rope": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                                _c_i32, _c_i32, ctypes.c_float, ctypes.c_int, _vp]),
    "attn_pool_create": (ctypes.c_int, [_c_i32, _c_i32, ctypes.POINTER(_vp)]),
    "attn_pool_destroy": (None, [_vp]),
    "attn_pool_alloc": (ctypes.c_int, [_vp, _c_i32, _c_i32p]),
    "attn_pool_free": (ctypes.c_int, [_vp, _c_i32p, _c_i32]),
    "attn_pool_retain": (ctypes.c_int, [_vp, _c_i32p, _c_i32]),
    "attn_pool_num_free": (_c_i32, [_vp]),
    "attn_pool_num_blocks": (_c_i32, [_vp]),
    "attn_pool_refcount": (ctypes.c_int, [_vp, _c_i32]),
    "attn_seq_reserve": (ctypes.c_int, [_vp, _c_i32p, _c_i32, _c_i32, _c_i32, _c_i32p]),
    "attn_residual_rms_norm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, ctypes.c_float, ctypes.c_int,
                                              _vp]),
    "attn_seq_fork": (ctypes.c_int, [_vp, _c_i32p, _c_i32, _c_i32p, _c_i32]),
    "attn_seq_reserve_cow": (ctypes.c_int, [_vp, _c_i32p, _c_i32, _c_i32, _c_i32, _c_i32p, _c_i32p]),
    "attn_copy_blocks": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_int, _vp]),
    "attn_debug_flags": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]),
}
ATTN_DEBUG_BLOCK_ID, ATTN_DEBUG_SLOT, ATTN_DEBUG_CONTEXT, ATTN_DEBUG_COPY_PAIR, ATTN_DEBUG_SEQLENS = 1, 2, 4, 8, 16

_libs: dict = {}
_debug_override = None  # set by debug_library()


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


def _debug_selected() -> bool:
    if _debug_override is not None:
        return _debug_override
    return os.environ.get("MI_ATTN_DEBUG", "0") == "1"


def lib_path(debug: bool | None = None) -> str:
    """Path of the library calls go to: the debug one when `debug` (default:
    the MI_ATTN_DEBUG setting) is true."""
    debug = _debug_selected() if debug is None else debug
    return os.path.join(_HERE, LIB_DEBUG_NAME if debug else LIB_NAME)


def load(debug: bool | None = None) -> ctypes.CDLL:
    """Load the in-tree shared library (built by transformer_attention_05_amd.build)."""
    path = lib_path(debug)
    lib = _libs.get(path)
    if lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m transformer_attention_05_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _libs[path] = lib
    return lib


@contextlib.contextmanager
def debug_library(on: bool = True):
    """Within the block, calls go to the debug library (on=True) or the
    release one (on=False), whatever MI_ATTN_DEBUG says.  Pools keep the
    library they were created with."""
    global _debug_override
    prev = _debug_override
    _debug_override = bool(on)
    try:
        yield load()
    finally:
        _debug_override = prev


def attn_last_error() -> str:
    return load().attn_last_error().decode()


def attn_debug_flags(clear: bool = True) -> int:
    """Debug library: wait for the current device and return the ATTN_DEBUG_*
    bits its kernels recorded (forgetting them when `clear`).  The release
    library raises AttnError (ATTN_E_UNSUPPORTED)."""
    out = ctypes.c_uint32(0)
    _check(load().attn_debug_flags(ctypes.byref(out), int(bool(clear))))
    return int(out.value)


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    return 99  # rejected by the library as unsupported


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    return t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


# --- argument checks.  They run before any pointer is taken, so a malformed
# call raises ValueError/TypeError here (CPU tensors included) instead of
# reaching the kernels: an int64 block table or a token-major value cache
# would otherwise be read with the wrong layout.

def _tensor(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    return t


def _int32(t, name, shape=None):
    """A contiguous int32 tensor, optionally of an exact shape."""
    _tensor(t, name)
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32 (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _like(t, name, shape, dtype):
    """A contiguous tensor of an exact shape and dtype."""
    _tensor(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} like q (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _caches(k_cache, v_cache, dtype, head_dim, num_kv_heads=None):
    """k_cache [nb, hkv, 16, D] and v_cache [nb, hkv, D, 16] (value blocks
    token-minor), contiguous, in the queries' dtype.  Returns (nb, hkv, bs)."""
    _tensor(k_cache, "k_cache")
    _tensor(v_cache, "v_cache")
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, hkv, bs, d = k_cache.shape
    if d != head_dim or (num_kv_heads is not None and hkv != num_kv_heads):
        raise ValueError(f"k_cache shape {tuple(k_cache.shape)} does not match the queries' heads / head_dim")
    _like(k_cache, "k_cache", (nb, hkv, bs, d), dtype)
    _like(v_cache, "v_cache [num_blocks, num_kv_heads, head_dim, block_size]", (nb, hkv, d, bs), dtype)
    return nb, hkv, bs


def _workspace_bytes(ws, name="workspace"):
    _tensor(ws, name)
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ws.numel() * ws.element_size()


def _i64x3(vals):
    return (ctypes.c_int64 * 3)(*[int(x) for x in vals])


def _bth_strides(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [batch, tokens, heads, head_dim]")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: head_dim must be contiguous")
    return _i64x3(t.stride()[:3])


# ----------------------------------------------------------------------------- kernels

def _workspace(ws, need, device):
    """(pointer, bytes) of a split-KV workspace: None allocates one of `need`
    bytes, False passes none (one pass per query tile)."""
    if ws is False or need == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    nbytes = _workspace_bytes(ws)
    return _dev(ws, "workspace"), nbytes


def _check_bthd(q, k, v, o, lse):
    """q [B, Tq, Hq, D]; k, v [B, Tk, Hkv, D] (any strides, D contiguous);
    o like q; lse float32 [B, Hq, Tq] contiguous."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _tensor(t, name)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [batch, tokens, heads, head_dim]")
    b, tq, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[3] != d:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must be [batch, seqlen_k, num_kv_heads, head_dim]"
                         f" matching q {tuple(q.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    if o is not None:
        _tensor(o, "o")
        if o.shape != q.shape or o.dtype != q.dtype:
            raise ValueError("o must have q's shape and dtype")
    if lse is not None:
        _like(lse, "lse", (b, hq, tq), torch.float32)
    return b, tq, hq, d, k.shape[1], k.shape[2]


def attn_prefill_workspace_size(batch, seqlen_q, seqlen_k, num_q_heads, num_kv_heads, head_dim,
                                dtype=torch.bfloat16) -> int:
    code = ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32
    return int(load().attn_prefill_workspace_size(batch, seqlen_q, seqlen_k, num_q_heads, num_kv_heads,
                                                  head_dim, code))


def attn_prefill(q, k, v, o=None, lse=None, causal=True, scale=0.0, workspace=None):
    """Contiguous attention on [B, T, H, D] tensors (any batch/token/head strides).

    ``workspace``: a uint8 GPU tensor of at least
    attn_prefill_workspace_size(...) bytes, None to allocate one here, or
    False to run without split-KV."""
    b, tq, hq, d, tk, hkv = _check_bthd(q, k, v, o, lse)
    if o is None:
        o = torch.empty_like(q)
    need = attn_prefill_workspace_size(b, tq, tk, hq, hkv, d, q.dtype)
    ws_ptr, ws_bytes = _workspace(workspace, need, q.device)
    st = load().attn_prefill(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(lse, "lse") if lse is not None else None,
        b, tq, tk, hq, hkv, d,
        _bth_strides(q, "q"), _bth_strides(k, "k"), _bth_strides(v, "v"), _bth_strides(o, "o"),
        float(scale), 1 if causal else 0, _dtype_code(q), ws_ptr, ws_bytes, _stream(q))
    _check(st)
    return o


def attn_prefill_masked(q, k, v, mask, o=None, lse=None, causal=False, scale=0.0):
    """Contiguous attention with an additive fp32 mask: ``mask`` is a GPU
    float32 tensor broadcastable to [B, Hq, Tq, Tk] (a [Tq, Tk] mask serves
    every batch and head) with contiguous keys; `causal` applies on top."""
    b, tq, hq, d, tk, hkv = _check_bthd(q, k, v, o, lse)
    if o is None:
        o = torch.empty_like(q)
    _tensor(mask, "mask")
    if mask.dtype != torch.float32:
        raise ValueError("mask must be float32")
    m = mask
    while m.dim() < 4:
        m = m.unsqueeze(0)
    m = m.expand(b, hq, tq, tk)
    if m.stride(3) != 1:
        raise ValueError("mask: keys must be contiguous")
    st = load().attn_prefill_masked(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(lse, "lse") if lse is not None else None,
        _dev(m, "mask"), _i64x3(m.stride()[:3]), b, tq, tk, hq, hkv, d,
        _bth_strides(q, "q"), _bth_strides(k, "k"), _bth_strides(v, "v"), _bth_strides(o, "o"),
        float(scale), 1 if causal else 0, _dtype_code(q), _stream(q))
    _check(st)
    return o


def attn_prefill_paged_workspace_size(num_seqs, total_q, max_seqlen_q, max_context_len, num_q_heads,
                                      num_kv_heads, head_dim) -> int:
    return int(load().attn_prefill_paged_workspace_size(num_seqs, total_q, max_seqlen_q, max_context_len,
                                                        num_q_heads, num_kv_heads, head_dim))


def attn_prefill_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, context_lens, max_seqlen_q,
                       o=None, causal=True, scale=0.0, max_context_len=0, workspace=None, share_cu=False):
    """Chunked prefill of packed queries q [total_q, Hq, D] over the paged caches.

    ``max_context_len``: the longest context (0: what the block table holds),
    used to plan split-KV; ``workspace`` as for attn_prefill.  ``share_cu``:
    the launch runs beside a decode on another stream (attn_prefill_paged_ex
    with ATTN_PREFILL_SHARE_CU; same results, a tile that leaves the decode
    room on every CU)."""
    total_q, hq, d, nb, hkv, bs, s = _check_paged(q, o, k_cache, v_cache, block_table, context_lens)
    _int32(cu_seqlens_q, "cu_seqlens_q", (s + 1,))
    if o is None:
        o = torch.empty_like(q)
    bound = int(max_context_len) if max_context_len else block_table.shape[1] * bs
    # (the fp32 kernel runs one pass and takes no workspace)
    need = 0 if q.dtype == torch.float32 else attn_prefill_paged_workspace_size(s, total_q, int(max_seqlen_q), bound,
                                                                                  hq, hkv, d)
    ws_ptr, ws_bytes = _workspace(workspace, need, q.device)
    args = (_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
            block_table.shape[1], _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(context_lens, "context_lens"),
            _dev(o, "o"), s, total_q, int(max_seqlen_q), int(max_context_len), hq, hkv, d, bs, nb,
            float(scale), 1 if causal else 0, _dtype_code(q))
    if share_cu:
        st = load().attn_prefill_paged_ex(*args, ATTN_PREFILL_SHARE_CU, ws_ptr, ws_bytes, _stream(q))
    else:
        st = load().attn_prefill_paged(*args, ws_ptr, ws_bytes, _stream(q))
    _check(st)
    return o


def _check_paged(q, o, k_cache, v_cache, block_table, context_lens):
    """Queries [rows, Hq, D] contiguous, o like q, the two caches, an int32
    block table [S, max_blocks] and int32 context lengths [S]."""
    _tensor(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [rows, num_q_heads, head_dim]")
    rows, hq, d = q.shape
    _like(q, "q", (rows, hq, d), q.dtype)
    if o is not None:
        _like(o, "o", (rows, hq, d), q.dtype)
    nb, hkv, bs = _caches(k_cache, v_cache, q.dtype, d)
    _int32(block_table, "block_table")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    s = block_table.shape[0]
    _int32(context_lens, "context_lens", (s,))
    return rows, hq, d, nb, hkv, bs, s


def attn_prefill_paged_masked(q, k_cache, v_cache, block_table, cu_seqlens_q, context_lens, max_seqlen_q, mask,
                              o=None, causal=True, scale=0.0, max_context_len=0):
    """attn_prefill_paged with an additive fp32 mask: ``mask`` is a GPU
    float32 tensor [total_q, Hq, K] or [total_q, K] (one row for every head;
    it broadcasts over heads) whose row for packed query r holds one entry
    per key position of r's sequence, K >= the longest context.  Keys
    contiguous; row and head strides multiples of 4 elements."""
    total_q, hq, d, nb, hkv, bs, s = _check_paged(q, o, k_cache, v_cache, block_table, context_lens)
    _int32(cu_seqlens_q, "cu_seqlens_q", (s + 1,))
    _tensor(mask, "mask")
    if mask.dtype != torch.float32:
        raise ValueError("mask must be float32")
    m = mask if mask.dim() == 3 else mask.unsqueeze(1)
    if m.dim() != 3 or m.shape[0] != total_q:
        raise ValueError("mask must be [total_q, num_q_heads, keys] or [total_q, keys]")
    m = m.expand(total_q, hq, m.shape[2])
    if m.stride(2) != 1:
        raise ValueError("mask: keys must be contiguous")
    if o is None:
        o = torch.empty_like(q)
    st = load().attn_prefill_paged_masked(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        block_table.shape[1], _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(context_lens, "context_lens"),
        _dev(m, "mask"), (ctypes.c_int64 * 2)(int(m.stride(0)), int(m.stride(1))), int(m.shape[2]),
        _dev(o, "o"), s, total_q, int(max_seqlen_q), int(max_context_len), hq, hkv, d, bs, nb,
        float(scale), 1 if causal else 0, _dtype_code(q), _stream(q))
    _check(st)
    return o


def attn_decode_paged_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                     partition_size=0) -> int:
    return int(load().attn_decode_paged_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                       max_context_len, partition_size))


def attn_decode_paged_auto_partition(num_seqs, num_kv_heads, max_context_len) -> int:
    return int(load().attn_decode_paged_auto_partition(num_seqs, num_kv_heads, max_context_len))


def attn_decode_paged_partition_for(context_lens, num_q_heads, num_kv_heads, head_dim=128) -> int:
    """Partition size for these (host) context lengths: the shortest multiple
    of 128 up to 1024 whose workgroups all fit on the GPU at once."""
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    r = int(load().attn_decode_paged_partition_for(cl.ctypes.data_as(_c_i32p), cl.shape[0], int(num_q_heads),
                                                    int(num_kv_heads), int(head_dim)))
    if r < 0:
        raise AttnError(r, attn_last_error())
    return r


def attn_decode_paged_plan(context_lens, num_kv_heads, max_context_len, partition_size=0):
    """Host-side plan: int32 numpy array [n, 2] of (sequence, partition)
    pairs, longest sequences first; move it to the GPU for attn_decode_paged."""
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    lib = load()
    ptr = cl.ctypes.data_as(_c_i32p)
    n = int(lib.attn_decode_paged_plan(ptr, cl.shape[0], num_kv_heads, int(max_context_len), int(partition_size),
                                       None, 0))
    if n < 0:
        raise AttnError(n, attn_last_error())
    items = np.zeros((max(n, 1), 2), dtype=np.int32)
    m = int(lib.attn_decode_paged_plan(ptr, cl.shape[0], num_kv_heads, int(max_context_len), int(partition_size),
                                       items.ctypes.data_as(_c_i32p), n))
    _check(0 if m == n else ATTN_E_INVALID)
    return items[:n]


def attn_decode_paged(q, k_cache, v_cache, block_table, context_lens, max_context_len, o=None,
                      partition_size=0, scale=0.0, workspace=None, plan=None):
    """Decode: q [S, Hq, D], one query per sequence, over the paged caches.

    ``workspace`` is a uint8 GPU tensor of at least
    attn_decode_paged_workspace_size(...) bytes, zero-filled before its first
    use (every completed call leaves its counters zero again); allocated here,
    zeroed, if None.
    ``plan``: optional int32 GPU tensor [n, 2] from attn_decode_paged_plan
    (same lengths and arguments)."""
    s, hq, d, nb, hkv, bs, s_bt = _check_paged(q, o, k_cache, v_cache, block_table, context_lens)
    if s_bt != s:
        raise ValueError(f"block_table has {s_bt} rows for {s} queries")
    if plan is not None:
        _int32(plan, "plan")
        if plan.dim() != 2 or plan.shape[1] != 2:
            raise ValueError("plan must be [n, 2] (sequence, partition)")
    if o is None:
        o = torch.empty_like(q)
    need = attn_decode_paged_workspace_size(s, hq, hkv, d, int(max_context_len), int(partition_size))
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = _workspace_bytes(workspace) if workspace is not None else 0
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    st = load().attn_decode_paged(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        _dev(context_lens, "context_lens"), _dev(o, "o"), s, hq, hkv, d, bs, nb, block_table.shape[1],
        int(max_context_len), int(partition_size), float(scale), _dtype_code(q),
        _dev(plan, "plan") if plan is not None else None, int(plan.shape[0]) if plan is not None else 0,
        ws_ptr, ws_bytes, _stream(q))
    _check(st)
    return o


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, context_lens, max_context_len, o,
                              partition_size=0, scale=0.0, plan=None):
    """attn_decode_paged with the library's fixed device scratch instead of
    a workspace: nothing is allocated, here or in the library (``o`` is
    required).  Calls that overlap on one GPU race."""
    s, hq, d, nb, hkv, bs, s_bt = _check_paged(q, o, k_cache, v_cache, block_table, context_lens)
    if s_bt != s:
        raise ValueError(f"block_table has {s_bt} rows for {s} queries")
    if o is None:
        raise ValueError("o is required (the no-allocation call allocates nothing)")
    if plan is not None:
        _int32(plan, "plan")
        if plan.dim() != 2 or plan.shape[1] != 2:
            raise ValueError("plan must be [n, 2] (sequence, partition)")
    st = load().attn_decode_paged_noalloc(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        _dev(context_lens, "context_lens"), _dev(o, "o"), s, hq, hkv, d, bs, nb, block_table.shape[1],
        int(max_context_len), int(partition_size), float(scale), _dtype_code(q),
        _dev(plan, "plan") if plan is not None else None, int(plan.shape[0]) if plan is not None else 0,
        _stream(q))
    _check(st)
    return o


def attn_decode_paged_rope(q, k_new, v_new, positions, slot_mapping, k_cache, v_cache, block_table, context_lens,
                           max_context_len, o=None, q_rot_out=None, rope_base=10000.0, partition_size=0, scale=0.0,
                           workspace=None, plan=None):
    """Decode with the new token of each sequence rotated and written into
    the cache by the same launch: q [S, Hq, D] (not rotated, left unchanged),
    k_new / v_new [S, Hkv, D], positions / slot_mapping [S] int32.  The
    rotated queries go to ``q_rot_out`` when given.  ``workspace`` and
    ``plan`` as for attn_decode_paged."""
    s, hq, d, nb, hkv, bs, s_bt = _check_paged(q, o, k_cache, v_cache, block_table, context_lens)
    if s_bt != s:
        raise ValueError(f"block_table has {s_bt} rows for {s} queries")
    _like(k_new, "k_new", (s, hkv, d), q.dtype)
    _like(v_new, "v_new", (s, hkv, d), q.dtype)
    _int32(positions, "positions", (s,))
    _int32(slot_mapping, "slot_mapping", (s,))
    if q_rot_out is not None:
        _like(q_rot_out, "q_rot_out", (s, hq, d), q.dtype)
    if plan is not None:
        _int32(plan, "plan")
        if plan.dim() != 2 or plan.shape[1] != 2:
            raise ValueError("plan must be [n, 2] (sequence, partition)")
    if o is None:
        o = torch.empty_like(q)
    need = attn_decode_paged_workspace_size(s, hq, hkv, d, int(max_context_len), int(partition_size))
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = _workspace_bytes(workspace) if workspace is not None else 0
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    st = load().attn_decode_paged_rope(
        _dev(q_rot_out, "q_rot_out") if q_rot_out is not None else None, _dev(q, "q"), _dev(k_new, "k_new"),
        _dev(v_new, "v_new"), _dev(positions, "positions"), _dev(slot_mapping, "slot_mapping"), float(rope_base),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_table, "block_table"),
        _dev(context_lens, "context_lens"), _dev(o, "o"), s, hq, hkv, d, bs, nb, block_table.shape[1],
        int(max_context_len), int(partition_size), float(scale), _dtype_code(q),
        _dev(plan, "plan") if plan is not None else None, int(plan.shape[0]) if plan is not None else 0,
        ws_ptr, ws_bytes, _stream(q))
    _check(st)
    return o


def attn_prefill_decode_paged(k_cache, v_cache, prefill=None, decode=None, scale=0.0):
    """A chunked prefill and a decode over the same paged caches in one
    launch (attn_prefill_decode_paged); bit-identical to attn_prefill_paged
    and attn_decode_paged (or attn_decode_paged_rope) called one after the
    other.

    ``prefill``: dict with q, block_table, cu_seqlens_q, context_lens,
    max_seqlen_q, and optional o, causal (True), max_context_len (0) -- the
    arguments of attn_prefill_paged (no split-KV workspace, no mask).
    ``decode``: dict with q, block_table, context_lens, max_context_len, and
    optional o, partition_size, workspace, plan -- those of attn_decode_paged
    -- plus, for the fused write of each sequence's new token, k_new, v_new,
    positions, slot_mapping and optional q_rot_out, rope_base (10000).
    Either may be None.  Returns (prefill output, decode output)."""
    _tensor(k_cache, "k_cache")
    pp, dp = _PrefillPart(), _DecodePart()
    ref = None
    o_pre = o_dec = None
    if prefill is not None:
        q = prefill["q"]
        total_q, hq, d, nb, hkv, bs, s = _check_paged(q, prefill.get("o"), k_cache, v_cache, prefill["block_table"],
                                                      prefill["context_lens"])
        _int32(prefill["cu_seqlens_q"], "cu_seqlens_q", (s + 1,))
        o_pre = prefill.get("o")
        if o_pre is None:
            o_pre = torch.empty_like(q)
        pp.q, pp.block_table = _dev(q, "q"), _dev(prefill["block_table"], "block_table")
        pp.max_blocks_per_seq = prefill["block_table"].shape[1]
        pp.cu_seqlens_q, pp.context_lens = _dev(prefill["cu_seqlens_q"], "cu_seqlens_q"), _dev(
            prefill["context_lens"], "context_lens")
        pp.o, pp.num_seqs, pp.total_q = _dev(o_pre, "o"), s, total_q
        pp.max_seqlen_q, pp.max_context_len = int(prefill["max_seqlen_q"]), int(prefill.get("max_context_len", 0))
        pp.causal = 1 if prefill.get("causal", True) else 0
        ref = q
    if decode is not None:
        q = decode["q"]
        s, hq, d, nb, hkv, bs, s_bt = _check_paged(q, decode.get("o"), k_cache, v_cache, decode["block_table"],
                                                   decode["context_lens"])
        if s_bt != s:
            raise ValueError(f"block_table has {s_bt} rows for {s} queries")
        if ref is not None and (ref.dtype != q.dtype or ref.shape[1:] != q.shape[1:]):
            raise ValueError("the prefill and decode queries must share dtype, heads and head_dim")
        plan = decode.get("plan")
        if plan is not None:
            _int32(plan, "plan")
            if plan.dim() != 2 or plan.shape[1] != 2:
                raise ValueError("plan must be [n, 2] (sequence, partition)")
        o_dec = decode.get("o")
        if o_dec is None:
            o_dec = torch.empty_like(q)
        part, mx = int(decode.get("partition_size", 0)), int(decode["max_context_len"])
        need = attn_decode_paged_workspace_size(s, hq, hkv, d, mx, part)
        ws = decode.get("workspace")
        if ws is None and need > 0:
            ws = torch.zeros(need, dtype=torch.uint8, device=q.device)
        dp.q, dp.block_table = _dev(q, "q"), _dev(decode["block_table"], "block_table")
        dp.max_blocks_per_seq = decode["block_table"].shape[1]
        dp.context_lens, dp.o = _dev(decode["context_lens"], "context_lens"), _dev(o_dec, "o")
        dp.num_seqs, dp.max_context_len, dp.partition_size = s, mx, part
        dp.plan = _dev(plan, "plan") if plan is not None else None
        dp.plan_items = int(plan.shape[0]) if plan is not None else 0
        dp.workspace = _dev(ws, "workspace") if ws is not None else None
        dp.workspace_bytes = _workspace_bytes(ws) if ws is not None else 0
        if decode.get("k_new") is not None:
            _like(decode["k_new"], "k_new", (s, hkv, d), q.dtype)
            _like(decode["v_new"], "v_new", (s, hkv, d), q.dtype)
            _int32(decode["positions"], "positions", (s,))
            _int32(decode["slot_mapping"], "slot_mapping", (s,))
            dp.k_new, dp.v_new = _dev(decode["k_new"], "k_new"), _dev(decode["v_new"], "v_new")
            dp.positions = _dev(decode["positions"], "positions")
            dp.slot_mapping = _dev(decode["slot_mapping"], "slot_mapping")
            dp.rope_base = float(decode.get("rope_base", 10000.0))
        qr = decode.get("q_rot_out")
        if qr is not None:  # (without the token write the library refuses it)
            _like(qr, "q_rot_out", (s, hq, d), q.dtype)
            dp.q_rot_out = _dev(qr, "q_rot_out")
        ref = q if ref is None else ref
    if ref is None:
        return None, None
    nb, hkv, bs = _caches(k_cache, v_cache, ref.dtype, ref.shape[2])
    st = load().attn_prefill_decode_paged(ctypes.byref(pp), ctypes.byref(dp), _dev(k_cache, "k_cache"),
                                          _dev(v_cache, "v_cache"), ref.shape[1], hkv, ref.shape[2], bs, nb,
                                          float(scale), _dtype_code(ref), _stream(ref))
    _check(st)
    return o_pre, o_dec


def attn_residual_rms_norm(x, residual, weight, eps=1e-6, y=None, residual_out=None):
    """Fused residual add + RMSNorm over the last dimension of [rows, hidden]
    tensors: returns (y, h) with h = x + residual (written to residual_out,
    which may be residual itself) and y = h / rms(h) * weight."""
    _tensor(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [rows, hidden]")
    for name, t in (("residual", residual), ("weight", weight)):
        _tensor(t, name)
        if t.dtype != x.dtype:
            raise ValueError(f"{name} must have x's dtype")
    if y is None:
        y = torch.empty_like(x)
    if residual_out is None:
        residual_out = torch.empty_like(x)
    rows, hidden = x.shape
    for name, t in (("residual", residual), ("y", y), ("residual_out", residual_out)):
        _tensor(t, name)
        if t.shape != x.shape or not t.is_contiguous() or t.dtype != x.dtype:
            raise ValueError(f"{name} must be a contiguous [rows, hidden] tensor like x")
    if not x.is_contiguous() or weight.shape != (hidden,) or not weight.is_contiguous():
        raise ValueError("x must be contiguous and weight a contiguous [hidden] tensor")
    _check(load().attn_residual_rms_norm(_dev(x, "x"), _dev(residual, "residual"), _dev(weight, "weight"),
                                         _dev(y, "y"), _dev(residual_out, "residual_out"), rows, hidden,
                                         float(eps), _dtype_code(x), _stream(x)))
    return y, residual_out


def attn_copy_blocks(k_cache, v_cache, pairs):
    """Copy whole blocks of both caches: ``pairs`` is an int32 GPU tensor
    [n, 2] of (src, dst) block ids."""
    _tensor(k_cache, "k_cache")
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, hkv, bs, d = k_cache.shape
    _caches(k_cache, v_cache, k_cache.dtype, d)
    _int32(pairs, "pairs")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2] (src, dst)")
    _check(load().attn_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(pairs, "pairs"),
                                   int(pairs.shape[0]), hkv, d, bs, nb, _dtype_code(k_cache), _stream(k_cache)))


def attn_kv_cache_write_rope(q, k, v, positions, slot_mapping, k_cache, v_cache, rope_base=10000.0):
    """Rotate q (in place, may be None) and k; write rotated k and v into their slots."""
    _tensor(k, "k")
    if k.dim() != 3:
        raise ValueError("k must be [num_tokens, num_kv_heads, head_dim]")
    n, hkv, d = k.shape
    _like(k, "k", (n, hkv, d), k.dtype)
    _like(v, "v", (n, hkv, d), k.dtype)
    if q is not None:
        _tensor(q, "q")
        if q.dim() != 3 or q.shape[0] != n or q.shape[2] != d:
            raise ValueError("q must be [num_tokens, num_q_heads, head_dim] like k")
        _like(q, "q", tuple(q.shape), k.dtype)
    hq = q.shape[1] if q is not None else hkv
    nb, _, bs = _caches(k_cache, v_cache, k.dtype, d, hkv)
    _int32(positions, "positions", (n,))
    _int32(slot_mapping, "slot_mapping", (n,))
    st = load().attn_kv_cache_write_rope(
        _dev(q, "q") if q is not None else None, _dev(k, "k"), _dev(v, "v"), _dev(positions, "positions"),
        _dev(slot_mapping, "slot_mapping"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        n, hq, hkv, d, bs, nb, float(rope_base), _dtype_code(k), _stream(k))
    _check(st)


# ----------------------------------------------------------------------------- host pool

def _i32_array(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(_c_i32p)


class Pool:
    """Host block pool (LIFO free list with reference counts)."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        self._lib = load()
        h = _vp()
        self._ok(self._lib.attn_pool_create(int(num_blocks), int(block_size), ctypes.byref(h)))
        self._h = h
        self.block_size = block_size

    def _ok(self, status: int):
        if status != ATTN_OK:
            raise AttnError(status, self._lib.attn_last_error().decode())

    def close(self):
        if getattr(self, "_h", None):
            self._lib.attn_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def alloc(self, n: int) -> np.ndarray:
        out = np.zeros(max(int(n), 0), dtype=np.int32)
        self._ok(self._lib.attn_pool_alloc(self._h, int(n), out.ctypes.data_as(_c_i32p)))
        return out

    def free(self, ids):
        a, p = _i32_array(ids)
        self._ok(self._lib.attn_pool_free(self._h, p, a.size))

    def retain(self, ids):
        a, p = _i32_array(ids)
        self._ok(self._lib.attn_pool_retain(self._h, p, a.size))

    @property
    def num_free(self) -> int:
        return int(self._lib.attn_pool_num_free(self._h))

    @property
    def num_blocks(self) -> int:
        return int(self._lib.attn_pool_num_blocks(self._h))

    def refcount(self, block_id: int) -> int:
        r = self._lib.attn_pool_refcount(self._h, int(block_id))
        if r < 0:
            _check(r)
        return int(r)

    def seq_fork(self, parent_row: np.ndarray, length: int, child_row: np.ndarray):
        """Share the blocks holding the first ``length`` tokens of the parent
        with the child (child_row updated in place)."""
        for name, r in (("parent_row", parent_row), ("child_row", child_row)):
            if r.dtype != np.int32 or not r.flags["C_CONTIGUOUS"]:
                raise ValueError(f"{name} must be a contiguous int32 array")
        self._ok(self._lib.attn_seq_fork(self._h, parent_row.ctypes.data_as(_c_i32p), int(length),
                                       child_row.ctypes.data_as(_c_i32p), child_row.size))

    def seq_reserve_cow(self, row: np.ndarray, cur_len: int, n_new: int):
        """seq_reserve that first gives the sequence its own copy of a shared,
        partly filled last block: returns (slots, (src, dst) or None), the
        block pair attn_copy_blocks must copy before the new tokens are
        written."""
        if row.dtype != np.int32 or not row.flags["C_CONTIGUOUS"]:
            raise ValueError("row must be a contiguous int32 array (it is updated in place)")
        slots = np.zeros(max(int(n_new), 0), dtype=np.int32)
        pair = np.full(2, -1, dtype=np.int32)
        self._ok(self._lib.attn_seq_reserve_cow(self._h, row.ctypes.data_as(_c_i32p), row.size, int(cur_len),
                                              int(n_new), slots.ctypes.data_as(_c_i32p),
                                              pair.ctypes.data_as(_c_i32p)))
        return slots, (None if pair[0] < 0 else (int(pair[0]), int(pair[1])))

    def seq_reserve(self, row: np.ndarray, cur_len: int, n_new: int) -> np.ndarray:
        """Grow a sequence in place: ``row`` is its int32 block-table row."""
        if row.dtype != np.int32 or not row.flags["C_CONTIGUOUS"]:
            raise ValueError("row must be a contiguous int32 array (it is updated in place)")
        slots = np.zeros(max(int(n_new), 0), dtype=np.int32)
        self._ok(self._lib.attn_seq_reserve(self._h, row.ctypes.data_as(_c_i32p), row.size, int(cur_len), int(n_new),
                                          slots.ctypes.data_as(_c_i32p)))
        return slots
