"""Python binding of libpagedattn — decode-phase paged attention on MI355X.

Argument marshalling only: every step of the path runs in the library's
gfx950 kernels (device work) or its C++ block allocator (host work).  torch
supplies device memory and streams.  The names mirror the C ABI declared in
``include/pagedattn.h`` without the ``pa_`` prefix.

Loading fails loudly (``ImportError``) when the shared library has not been
built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3, PA_INT8 = 0, 1, 2, 3, 4
DTYPE_CODES = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16, "fp8_e4m3": PA_FP8_E4M3,
               "int8": PA_INT8}
STATUS = {0: "PA_OK", -1: "PA_ERR_INVALID_ARG", -2: "PA_ERR_UNSUPPORTED",
          -3: "PA_ERR_OUT_OF_BLOCKS", -4: "PA_ERR_INDEX", -5: "PA_ERR_UNKNOWN_SEQ",
          -6: "PA_ERR_REFCOUNT", -7: "PA_ERR_HIP", -8: "PA_ERR_WORKSPACE", -9: "PA_ERR_EXISTS"}

_c_int32_p = ctypes.POINTER(ctypes.c_int32)
_c_int64_p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p

# (name, restype, argtypes) for every exported function of include/pagedattn.h
_SIGNATURES = [
    ("pa_status_string", ctypes.c_char_p, [ctypes.c_int32]),
    ("pa_version", ctypes.c_char_p, []),
    ("pa_last_error", ctypes.c_char_p, []),
    ("pa_kv_bytes_per_token", ctypes.c_int64, [ctypes.c_int32] * 4),
    ("pa_kv_cache_write", ctypes.c_int32,
     [_vp, _vp, ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_float, ctypes.c_float, _vp]),
    ("pa_kv_cache_write_int8", ctypes.c_int32,
     [_vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp]),
    ("pa_paged_attention_workspace_size", ctypes.c_size_t, [ctypes.c_int32] * 6),
    ("pa_paged_attention_decode_int8", ctypes.c_int32,
     [_vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32, _vp, ctypes.c_size_t, _vp]),
    ("pa_paged_attention_decode", ctypes.c_int32,
     [_vp, _vp, ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp, ctypes.c_int32, _vp,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_float,
      ctypes.c_int32, _vp, ctypes.c_size_t, _vp]),
    ("pa_paged_attention_decode_noalloc", ctypes.c_int32,
     [_vp, _vp, ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp, ctypes.c_int32, _vp,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_float,
      ctypes.c_int32, _vp]),
    ("pa_paged_attention_prefill", ctypes.c_int32,
     [_vp, _vp, ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp, ctypes.c_int32, _vp, _vp,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _vp]),
    ("pa_copy_blocks", ctypes.c_int32,
     [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int32, _vp]),
    ("pa_stream_read", ctypes.c_int32, [_vp, ctypes.c_size_t, _vp, _vp]),
    ("pa_swap_blocks", ctypes.c_int32,
     [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
      ctypes.c_int32, _vp, ctypes.c_int32, _vp]),
    ("pa_alloc_swap_out", ctypes.c_int32,
     [_vp, _vp, ctypes.c_int64, _c_int32_p, ctypes.c_int32, _c_int32_p]),
    ("pa_alloc_swap_in", ctypes.c_int32,
     [_vp, _vp, ctypes.c_int64, _c_int32_p, ctypes.c_int32, _c_int32_p]),
    ("pa_alloc_create", ctypes.c_int32,
     [ctypes.c_int32, ctypes.c_int32, _c_int32_p, ctypes.POINTER(_vp)]),
    ("pa_alloc_destroy", None, [_vp]),
    ("pa_alloc_add_seq", ctypes.c_int32, [_vp, ctypes.c_int64, ctypes.c_int32]),
    ("pa_alloc_fork", ctypes.c_int32, [_vp, ctypes.c_int64, ctypes.c_int64]),
    ("pa_alloc_append_slots", ctypes.c_int32,
     [_vp, _c_int64_p, ctypes.c_int32, _c_int64_p, _c_int32_p, _c_int32_p]),
    ("pa_alloc_add_seq_tokens", ctypes.c_int32,
     [_vp, ctypes.c_int64, _c_int32_p, ctypes.c_int32, _c_int32_p]),
    ("pa_alloc_append_tokens", ctypes.c_int32,
     [_vp, _c_int64_p, _c_int32_p, ctypes.c_int32, _c_int64_p, _c_int32_p, _c_int32_p]),
    ("pa_alloc_stats", ctypes.c_int32, [_vp, ctypes.c_void_p]),
    ("pa_alloc_num_evictable", ctypes.c_int32, [_vp]),
    ("pa_alloc_free_seq", ctypes.c_int32, [_vp, ctypes.c_int64]),
    ("pa_alloc_export", ctypes.c_int32,
     [_vp, _c_int64_p, ctypes.c_int32, _c_int32_p, ctypes.c_int32, _c_int32_p]),
    ("pa_alloc_physical_block", ctypes.c_int32, [_vp, ctypes.c_int64, ctypes.c_int32, _c_int32_p]),
    ("pa_alloc_num_free", ctypes.c_int32, [_vp]),
    ("pa_alloc_refcount", ctypes.c_int32, [_vp, ctypes.c_int32]),
    ("pa_alloc_seq_len", ctypes.c_int32, [_vp, ctypes.c_int64]),
    ("pa_alloc_num_seqs", ctypes.c_int32, [_vp]),
]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
                          f"g.build()'` (or python paged_kv_cache_129_amd/build.py)")
    # torch ships its own HIP runtime (same soname, libamdhip64.so.7).  Import
    # it first so that this library binds to the runtime torch already loaded:
    # two HIP runtimes in one process do not share devices or memory.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    for name, res, args in _SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.pa_status_string(status).decode()
        if status == -7:
            msg += f": {lib.pa_last_error().decode()}"
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PagedAttnError(status, where)


def version() -> str:
    return lib.pa_version().decode()


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, num_layers: int, dtype: str) -> int:
    return int(lib.pa_kv_bytes_per_token(num_kv_heads, head_dim, num_layers, DTYPE_CODES[dtype]))


# ------------------------------------------------------------------ torch plumbing
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
         torch.uint8: PA_FP8_E4M3, torch.int8: PA_INT8}
    fp8 = getattr(torch, "float8_e4m3fn", None)
    if fp8 is not None:
        m[fp8] = PA_FP8_E4M3
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _same_dtype(a, b, na: str, nb: str):
    """K and V operands are read with one element type: a narrower one would be
    read past its end."""
    if a.dtype != b.dtype:
        raise ValueError(f"{na} and {nb} differ in dtype ({a.dtype} vs {b.dtype})")


def _one_device(*tensors):
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ device calls
def kv_cache_write(k_new, v_new, k_pool, v_pool, slot_mapping, *, k_scale: float = 1.0,
                   v_scale: float = 1.0, stream=None) -> None:
    """Store new tokens' K/V ([T, Hkv, D]) at their slots of [NB, Hkv, bs, D] pools."""
    T, Hkv, D = k_new.shape
    NB, Hkv2, bs, D2 = k_pool.shape
    if (Hkv, D) != (Hkv2, D2) or v_new.shape != k_new.shape or v_pool.shape != k_pool.shape:
        raise ValueError("shape mismatch")
    if slot_mapping.dtype != _torch().int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    _same_dtype(k_new, v_new, "k_new", "v_new")
    _same_dtype(k_pool, v_pool, "k_pool", "v_pool")
    _one_device(k_new, v_new, k_pool, v_pool, slot_mapping)
    _check(lib.pa_kv_cache_write(_dev(k_new, "k_new"), _dev(v_new, "v_new"), dtype_code(k_new),
                                 _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                 dtype_code(k_pool), _dev(slot_mapping, "slot_mapping"), T, Hkv, D,
                                 bs, NB, k_scale, v_scale, _stream(stream, k_pool.device)),
           "kv_cache_write")


def kv_cache_write_int8(k_new, v_new, k_pool, v_pool, k_scales, v_scales, slot_mapping, *,
                        stream=None) -> None:
    """Quantise new tokens' K/V ([T, Hkv, D]) into int8 [NB, Hkv, bs, D] pools, one
    float32 scale per (token, KV head) into [NB, Hkv, bs] scale pools."""
    torch = _torch()
    T, Hkv, D = k_new.shape
    NB, Hkv2, bs, D2 = k_pool.shape
    if (Hkv, D) != (Hkv2, D2) or v_new.shape != k_new.shape or v_pool.shape != k_pool.shape:
        raise ValueError("shape mismatch")
    if k_pool.dtype != torch.int8 or v_pool.dtype != torch.int8:
        raise ValueError("int8 pools expected")
    for sc in (k_scales, v_scales):
        if sc.dtype != torch.float32 or tuple(sc.shape) != (NB, Hkv, bs):
            raise ValueError("scale pools must be float32 [NB, Hkv, bs]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    _same_dtype(k_new, v_new, "k_new", "v_new")
    _one_device(k_new, v_new, k_pool, v_pool, k_scales, v_scales, slot_mapping)
    _check(lib.pa_kv_cache_write_int8(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), dtype_code(k_new), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"), _dev(k_scales, "k_scales"), _dev(v_scales, "v_scales"),
        _dev(slot_mapping, "slot_mapping"), T, Hkv, D, bs, NB, _stream(stream, k_pool.device)),
        "kv_cache_write_int8")


PARTITION_BALANCED = -1


def paged_attention_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int,
                                   head_dim: int, max_context_len: int,
                                   partition_size: int) -> int:
    return int(lib.pa_paged_attention_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                     max_context_len, partition_size))


def new_workspace(nbytes: int, device):
    """Device workspace of at least ``nbytes`` (never empty; no initial contents needed)."""
    return _torch().empty(max(int(nbytes), 256), dtype=_torch().uint8, device=device)


def paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens, *,
                           max_context_len: int, scale: float, k_scale: float = 1.0,
                           v_scale: float = 1.0, partition_size: int = 0, workspace=None,
                           stream=None) -> None:
    """out[S, H, D] = decode attention of q[S, H, D] over paged [NB, Hkv, bs, D] pools."""
    torch = _torch()
    S, H, D = q.shape
    NB, Hkv, bs, D2 = k_pool.shape
    if D2 != D or out.shape != q.shape or out.dtype != q.dtype or v_pool.shape != k_pool.shape:
        raise ValueError("shape mismatch")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [S]")
    _same_dtype(k_pool, v_pool, "k_pool", "v_pool")
    _one_device(out, q, k_pool, v_pool, block_tables, context_lens,
                *([workspace] if workspace is not None else []))
    need = paged_attention_workspace_size(S, H, Hkv, D, max_context_len, partition_size)
    if need and workspace is None:
        # allocated in the order of the stream the kernels run on, so that the
        # caching allocator reuses it only after they are done
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream(q.device)):
            workspace = new_workspace(need, q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_paged_attention_decode(
        _dev(out, "out"), _dev(q, "q"), dtype_code(q), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"), dtype_code(k_pool), _dev(block_tables, "block_tables"),
        block_tables.shape[1], _dev(context_lens, "context_lens"), int(max_context_len), S, H,
        Hkv, D, bs, NB, float(scale), float(k_scale), float(v_scale), int(partition_size),
        ws_ptr, ws_bytes, _stream(stream, q.device)), "paged_attention_decode")


def paged_attention_decode_int8(out, q, k_pool, v_pool, k_scales, v_scales, block_tables,
                                context_lens, *, max_context_len: int, scale: float,
                                partition_size: int = 0, workspace=None, stream=None) -> None:
    """paged_attention_decode over int8 [NB, Hkv, bs, D] pools with float32
    [NB, Hkv, bs] scale pools (as written by kv_cache_write_int8)."""
    torch = _torch()
    S, H, D = q.shape
    NB, Hkv, bs, D2 = k_pool.shape
    if D2 != D or out.shape != q.shape or out.dtype != q.dtype or v_pool.shape != k_pool.shape:
        raise ValueError("shape mismatch")
    if k_pool.dtype != torch.int8 or v_pool.dtype != torch.int8:
        raise ValueError("int8 pools expected")
    for sc in (k_scales, v_scales):
        if sc.dtype != torch.float32 or tuple(sc.shape) != (NB, Hkv, bs):
            raise ValueError("scale pools must be float32 [NB, Hkv, bs]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [S]")
    _one_device(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens,
                *([workspace] if workspace is not None else []))
    need = paged_attention_workspace_size(S, H, Hkv, D, max_context_len, partition_size)
    if need and workspace is None:
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream(q.device)):
            workspace = new_workspace(need, q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_paged_attention_decode_int8(
        _dev(out, "out"), _dev(q, "q"), dtype_code(q), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"), _dev(k_scales, "k_scales"), _dev(v_scales, "v_scales"),
        _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(context_lens, "context_lens"), int(max_context_len), S, H, Hkv, D, bs, NB,
        float(scale), int(partition_size), ws_ptr, ws_bytes, _stream(stream, q.device)),
        "paged_attention_decode_int8")


def paged_attention_prefill(out, q, k_pool, v_pool, block_tables, context_lens, query_start, *,
                            max_query_len: int, scale: float, stream=None) -> None:
    """out[T, H, D] = causal multi-token attention of q[T, H, D] (rows of sequence s
    at query_start[s]:query_start[s+1], the last rows of its context) over paged
    [NB, Hkv, bs, D] pools."""
    torch = _torch()
    T, H, D = q.shape
    NB, Hkv, bs, D2 = k_pool.shape
    S = context_lens.shape[0]
    if D2 != D or out.shape != q.shape or out.dtype != q.dtype or v_pool.shape != k_pool.shape:
        raise ValueError("shape mismatch")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.dim() != 1:
        raise ValueError("context_lens must be int32 [S]")
    if query_start.dtype != torch.int32 or query_start.shape != (S + 1,):
        raise ValueError("query_start must be int32 [S + 1]")
    _same_dtype(k_pool, v_pool, "k_pool", "v_pool")
    _one_device(out, q, k_pool, v_pool, block_tables, context_lens, query_start)
    _check(lib.pa_paged_attention_prefill(
        _dev(out, "out"), _dev(q, "q"), dtype_code(q), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"), dtype_code(k_pool), _dev(block_tables, "block_tables"),
        block_tables.shape[1], _dev(context_lens, "context_lens"), _dev(query_start, "query_start"),
        S, T, int(max_query_len), H, Hkv, D, bs, NB, float(scale), _stream(stream, q.device)),
        "paged_attention_prefill")


NOALLOC_SCRATCH_BYTES = 64 << 20


def paged_attention_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens, *,
                                   max_context_len: int, scale: float, k_scale: float = 1.0,
                                   v_scale: float = 1.0, partition_size: int = 0,
                                   stream=None) -> None:
    """paged_attention_decode without a workspace: the split modes use the
    library's static per-GPU scratch (nothing is allocated; calls that overlap
    on one GPU race)."""
    torch = _torch()
    S, H, D = q.shape
    NB, Hkv, bs, D2 = k_pool.shape
    if D2 != D or out.shape != q.shape or out.dtype != q.dtype or v_pool.shape != k_pool.shape:
        raise ValueError("shape mismatch")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [S]")
    _same_dtype(k_pool, v_pool, "k_pool", "v_pool")
    _one_device(out, q, k_pool, v_pool, block_tables, context_lens)
    _check(lib.pa_paged_attention_decode_noalloc(
        _dev(out, "out"), _dev(q, "q"), dtype_code(q), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"), dtype_code(k_pool), _dev(block_tables, "block_tables"),
        block_tables.shape[1], _dev(context_lens, "context_lens"), int(max_context_len), S, H,
        Hkv, D, bs, NB, float(scale), float(k_scale), float(v_scale), int(partition_size),
        _stream(stream, q.device)), "paged_attention_decode_noalloc")


def copy_blocks(k_pools: Sequence, v_pools: Sequence, pairs, *, stream=None) -> None:
    """Copy block src -> dst for every (src, dst) in ``pairs`` in every layer's K and V pool.

    ``pairs`` is a device int32 tensor [N, 2] (read by the kernel when it
    runs: a captured launch replays with whatever the buffer holds; rows with
    an id outside the pool, e.g. -1 padding, are skipped), or host pairs
    (a sequence or array), which are copied to the device on the call's stream
    first.  Pools are [NB, Hkv, bs, D], or the [NB, Hkv, bs] float32 scale pools
    of an int8 cache."""
    torch = _torch()
    L = len(k_pools)
    if L != len(v_pools):
        raise ValueError("k_pools and v_pools differ in length")
    if L == 0:
        return
    if k_pools[0].dim() == 3:               # int8 scale pools [NB, Hkv, bs]: head_dim 1
        (NB, Hkv, bs), D = k_pools[0].shape, 1
    else:
        NB, Hkv, bs, D = k_pools[0].shape
    for p in list(k_pools) + list(v_pools):
        if p.shape != k_pools[0].shape or p.dtype != k_pools[0].dtype:
            raise ValueError("all pools must share shape and dtype")
    _one_device(*k_pools, *v_pools)
    dev = k_pools[0].device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    if isinstance(pairs, torch.Tensor) and pairs.is_cuda:
        if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
            raise ValueError("device pairs must be int32 [N, 2]")
        _one_device(k_pools[0], pairs)
        dpairs = pairs
    else:
        host = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        if len(host) == 0:
            return
        if torch.cuda.is_current_stream_capturing():
            raise ValueError("copy_blocks under graph capture needs device pairs (a host "
                             "array would be read at capture time only)")
        with torch.cuda.stream(s):          # allocated and filled in the call's stream order
            dpairs = torch.from_numpy(host).to(dev)
    if dpairs.shape[0] == 0:
        return
    kp = (ctypes.c_void_p * L)(*[_dev(p, "k_pool").value for p in k_pools])
    vp = (ctypes.c_void_p * L)(*[_dev(p, "v_pool").value for p in v_pools])
    _check(lib.pa_copy_blocks(kp, vp, L, dtype_code(k_pools[0]), Hkv, D, bs, NB,
                              _dev(dpairs, "pairs"), dpairs.shape[0],
                              ctypes.c_void_p(s.cuda_stream)), "copy_blocks")


def swap_blocks(dst_pools: Sequence, src_pools: Sequence, pairs, *, stream=None) -> None:
    """Move block s of every source pool to block d of the matching destination pool
    for every (s, d) in ``pairs``: device pools and pools in pinned host memory
    (``pin_memory=True``), in either direction.  ``pairs`` is a device int32 tensor
    [N, 2] or host pairs (copied to the device on the call's stream)."""
    torch = _torch()
    L = len(dst_pools)
    if L != len(src_pools):
        raise ValueError("dst_pools and src_pools differ in length")
    if L == 0:
        return
    shape, dt = dst_pools[0].shape[1:], dst_pools[0].dtype
    for p in list(dst_pools) + list(src_pools):
        if p.shape[1:] != shape or p.dtype != dt or not p.is_contiguous():
            raise ValueError("pools must be contiguous and share block shape and dtype")
    if any(p.shape[0] != dst_pools[0].shape[0] for p in dst_pools) or \
            any(p.shape[0] != src_pools[0].shape[0] for p in src_pools):
        raise ValueError("destination pools (and source pools) must hold the same number of blocks")
    for p in list(dst_pools) + list(src_pools):
        if not (p.is_cuda or p.is_pinned()):
            raise ValueError("pools must be device tensors or pinned host tensors")
    dev = next((p.device for p in list(dst_pools) + list(src_pools) if p.is_cuda), None)
    if dev is None:
        raise ValueError("one side must be on the device")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    if isinstance(pairs, torch.Tensor) and pairs.is_cuda:
        if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
            raise ValueError("device pairs must be int32 [N, 2]")
        dpairs = pairs
    else:
        host = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        if len(host) == 0:
            return
        if torch.cuda.is_current_stream_capturing():
            raise ValueError("swap_blocks under graph capture needs device pairs")
        with torch.cuda.stream(s):
            dpairs = torch.from_numpy(host).to(dev)
    if dpairs.shape[0] == 0:
        return
    block_bytes = dst_pools[0][0].numel() * dst_pools[0].element_size()
    dp = (ctypes.c_void_p * L)(*[p.data_ptr() for p in dst_pools])
    sp = (ctypes.c_void_p * L)(*[p.data_ptr() for p in src_pools])
    _check(lib.pa_swap_blocks(dp, sp, L, block_bytes, dst_pools[0].shape[0], src_pools[0].shape[0],
                              _dev(dpairs, "pairs"), dpairs.shape[0], ctypes.c_void_p(s.cuda_stream)),
           "swap_blocks")


STREAM_READ_SINK_WORDS = 4096


def stream_read(buf, sink, *, stream=None) -> None:
    """One pass of the decode kernels' 16-byte streaming loads over the contiguous
    device tensor ``buf`` (a multiple of 16 bytes); ``sink`` is a device int32 or
    uint32 tensor of STREAM_READ_SINK_WORDS words that receives the XOR of buf's
    32-bit words, folded per workgroup.  A measurement aid: the read rate the HBM
    rooflines are compared with."""
    torch = _torch()
    if not buf.is_contiguous() or not sink.is_contiguous():
        raise ValueError("buf and sink must be contiguous")
    if sink.numel() * sink.element_size() < 4 * STREAM_READ_SINK_WORDS:
        raise ValueError(f"sink must hold {STREAM_READ_SINK_WORDS} 32-bit words")
    _one_device(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(buf.device)
    _check(lib.pa_stream_read(_dev(buf, "buf"), nbytes, _dev(sink, "sink"),
                              ctypes.c_void_p(s.cuda_stream)), "stream_read")


# ------------------------------------------------------------------ host allocator
class AllocCounts(ctypes.Structure):
    """pa_alloc_counts of include/pagedattn.h."""
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_blocks", "free_blocks", "evictable_blocks", "used_blocks", "cached_blocks",
        "filled_slots", "prefix_hit_blocks", "evictions")]


class BlockAllocator:
    """Host block allocator (free list, reference counts, copy-on-write) in C++."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self._h = ctypes.c_void_p()
        fo = None
        if free_order is not None:
            self._fo = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            fo = self._fo.ctypes.data_as(_c_int32_p)
        _check(lib.pa_alloc_create(num_blocks, block_size, fo, ctypes.byref(self._h)),
               "alloc_create")
        # kept on the instance: at interpreter exit module globals may be gone
        # before the last allocator is collected
        self._destroy = lib.pa_alloc_destroy
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self._h = None

    def add_seq(self, seq_id: int, num_tokens: int) -> None:
        _check(lib.pa_alloc_add_seq(self._h, seq_id, num_tokens), "alloc_add_seq")

    def fork(self, parent_id: int, child_id: int) -> None:
        _check(lib.pa_alloc_fork(self._h, parent_id, child_id), "alloc_fork")

    def add_seq_tokens(self, seq_id: int, tokens: Sequence[int]) -> int:
        """Admit a sequence with known token ids; returns the tokens already cached."""
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        cached = ctypes.c_int32(0)
        _check(lib.pa_alloc_add_seq_tokens(self._h, seq_id, toks.ctypes.data_as(_c_int32_p),
                                           len(toks), ctypes.byref(cached)), "alloc_add_seq_tokens")
        return cached.value

    def append_slots(self, seq_ids: Sequence[int],
                     token_ids: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = len(ids)
        slots = np.empty(n, dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        npairs = ctypes.c_int32(0)
        if token_ids is None:
            _check(lib.pa_alloc_append_slots(self._h, ids.ctypes.data_as(_c_int64_p), n,
                                             slots.ctypes.data_as(_c_int64_p),
                                             pairs.ctypes.data_as(_c_int32_p), ctypes.byref(npairs)),
                   "alloc_append_slots")
        else:
            toks = np.ascontiguousarray(np.asarray(token_ids, dtype=np.int32))
            if len(toks) != n:
                raise ValueError("one token id per sequence")
            _check(lib.pa_alloc_append_tokens(self._h, ids.ctypes.data_as(_c_int64_p),
                                              toks.ctypes.data_as(_c_int32_p), n,
                                              slots.ctypes.data_as(_c_int64_p),
                                              pairs.ctypes.data_as(_c_int32_p), ctypes.byref(npairs)),
                   "alloc_append_tokens")
        return slots, pairs[:npairs.value].copy()

    def _swap(self, fn, host: "BlockAllocator", seq_id: int, where: str) -> np.ndarray:
        cap = max(1, len(self._table_len_hint(seq_id, host)))
        pairs = np.empty((cap, 2), dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(fn(self._h, host._h, seq_id, pairs.ctypes.data_as(_c_int32_p), cap, ctypes.byref(n)),
               where)
        return pairs[:n.value].copy()

    def _table_len_hint(self, seq_id, host):
        n = max(self.seq_len(seq_id), host.seq_len(seq_id), 0)
        return range((n + self.block_size - 1) // self.block_size)

    def swap_out(self, seq_id: int, host: "BlockAllocator") -> np.ndarray:
        """Move a sequence to ``host`` (an allocator over host blocks); returns the
        (device block, host block) pairs to copy before the device blocks are reused."""
        return self._swap(lib.pa_alloc_swap_out, host, seq_id, "alloc_swap_out")

    def swap_in(self, seq_id: int, host: "BlockAllocator") -> np.ndarray:
        """Bring a sequence back from ``host``; returns the (host block, device block)
        pairs to copy before the sequence is read."""
        return self._swap(lib.pa_alloc_swap_in, host, seq_id, "alloc_swap_in")

    def stats(self) -> dict:
        c = AllocCounts()
        _check(lib.pa_alloc_stats(self._h, ctypes.byref(c)), "alloc_stats")
        return {n: int(getattr(c, n)) for n, _ in AllocCounts._fields_}

    def utilisation(self) -> float:
        st = self.stats()
        return st["filled_slots"] / (st["used_blocks"] * self.block_size) if st["used_blocks"] else 1.0

    def num_evictable(self) -> int:
        return int(lib.pa_alloc_num_evictable(self._h))

    def free_seq(self, seq_id: int) -> None:
        _check(lib.pa_alloc_free_seq(self._h, seq_id), "alloc_free_seq")

    def export(self, seq_ids: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        tables = np.empty((len(ids), max_blocks), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        _check(lib.pa_alloc_export(self._h, ids.ctypes.data_as(_c_int64_p), len(ids),
                                   tables.ctypes.data_as(_c_int32_p), max_blocks,
                                   lens.ctypes.data_as(_c_int32_p)), "alloc_export")
        return tables, lens

    def physical_block(self, seq_id: int, logical_idx: int) -> int:
        out = ctypes.c_int32(0)
        _check(lib.pa_alloc_physical_block(self._h, seq_id, logical_idx, ctypes.byref(out)),
               "alloc_physical_block")
        return out.value

    def num_free(self) -> int:
        return int(lib.pa_alloc_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(lib.pa_alloc_refcount(self._h, block))

    def seq_len(self, seq_id: int) -> int:
        return int(lib.pa_alloc_seq_len(self._h, seq_id))

    def num_seqs(self) -> int:
        return int(lib.pa_alloc_num_seqs(self._h))
