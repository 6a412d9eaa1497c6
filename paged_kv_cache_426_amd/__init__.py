"""Paged-attention decode on MI355X (gfx950): Python face of libpa.

A thin ctypes binding over the C ABI declared in ``include/pa.h``. It only
checks and marshals arguments (device pointers, sizes, element-type codes and
the current HIP stream); every step of the computation runs in libpa's HIP
kernels. PyTorch provides device memory and streams.

There is no CPU fallback: calling any operation with tensors that are not on
a GPU, or without the built library, raises.
"""

import ctypes
import os
from typing import Optional, Tuple

import torch

from . import checks
from .checks import ContractError, set_debug_checks

__all__ = [
    "ContractError", "set_debug_checks",
    "PA_F32", "PA_F16", "PA_BF16", "PA_FP8_E4M3FN", "PA_INT8",
    "PaError", "lib", "library_path", "dtype_code",
    "prefill", "decode", "decode_noalloc", "decode_noalloc_scratch_bytes", "decode_append", "decode_partials", "decode_reduce", "decode_workspace_size",
    "decode_shared_prefix", "decode_shared_prefix_workspace_size",
    "num_partitions", "decode_balanced_splits", "reshape_and_cache", "copy_blocks",
    "decode_scaled", "reshape_and_cache_scaled", "copy_blocks_scaled",
    "PA_SCALE_PER_HEAD", "PA_SCALE_PER_BLOCK", "PA_SCALE_PER_BLOCK_HEAD",
    "PARTITION_AUTO",
]

# partition_size of the balanced split with the automatic share count
PARTITION_AUTO = -1

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3FN, PA_INT8 = 0, 1, 2, 3, 4

# layouts of the scale tables of an 8-bit cache (pa.h pa_scale_layout)
PA_SCALE_PER_HEAD, PA_SCALE_PER_BLOCK, PA_SCALE_PER_BLOCK_HEAD = 1, 2, 3

_DTYPES = {
    torch.float32: PA_F32,
    torch.float16: PA_F16,
    torch.bfloat16: PA_BF16,
    torch.float8_e4m3fn: PA_FP8_E4M3FN,
    torch.uint8: PA_FP8_E4M3FN,  # raw E4M3FN codes
    torch.int8: PA_INT8,         # symmetric int8 codes
}
_TORCH_OF = {PA_F32: torch.float32, PA_F16: torch.float16, PA_BF16: torch.bfloat16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class PaError(RuntimeError):
    """A libpa call returned a non-zero status."""


def library_path() -> str:
    return os.path.join(_HERE, "libpa.so")


def lib() -> ctypes.CDLL:
    """The loaded libpa. Built from source first if no built library exists."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            from .build import build

            build()
        L = ctypes.CDLL(path)
        vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_size_t)
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_status_string.argtypes = [i32]
        L.pa_version.restype = i32
        L.pa_num_partitions.restype = i32
        L.pa_num_partitions.argtypes = [i32, i32, i32]
        L.pa_decode_balanced_splits.restype = i32
        L.pa_decode_balanced_splits.argtypes = [i32] * 5
        L.pa_decode_workspace_size.restype = sz
        L.pa_decode_workspace_size.argtypes = [i32] * 6
        L.pa_decode.restype = i32
        L.pa_decode.argtypes = [vp] * 6 + [i32] * 7 + [f32, i32, i32, f32, f32, i32, vp, sz, vp]
        L.pa_decode_noalloc.restype = i32
        L.pa_decode_noalloc.argtypes = ([vp] * 6 + [i32] * 7 +
                                        [f32, i32, i32, f32, f32, i32, vp])
        L.pa_decode_noalloc_scratch_bytes.restype = sz
        L.pa_decode_noalloc_scratch_bytes.argtypes = []
        L.pa_decode_append.restype = i32
        L.pa_decode_append.argtypes = ([vp] * 8 + [i32] * 7 +
                                       [f32, i32, i32, f32, f32, i32, vp, sz, vp])
        L.pa_decode_partials.restype = i32
        L.pa_decode_partials.argtypes = ([vp] * 3 + [i32] + [vp] * 5 + [i32] * 7 +
                                         [f32, i32, i32, f32, f32, i32, vp])
        L.pa_decode_reduce.restype = i32
        L.pa_decode_reduce.argtypes = [vp] * 5 + [i32] * 6 + [vp]
        L.pa_reshape_and_cache.restype = i32
        L.pa_reshape_and_cache.argtypes = [vp] * 5 + [i32] * 7 + [f32, f32, vp]
        L.pa_copy_blocks.restype = i32
        L.pa_copy_blocks.argtypes = [vp] * 3 + [i32] * 6 + [vp]
        L.pa_decode_scaled.restype = i32
        L.pa_decode_scaled.argtypes = ([vp] * 6 + [i32] * 7 + [f32, i32, i32, vp, vp, i32, i32,
                                                              vp, sz, vp])
        L.pa_reshape_and_cache_scaled.restype = i32
        L.pa_reshape_and_cache_scaled.argtypes = [vp] * 5 + [i32] * 7 + [vp, vp, i32, vp]
        L.pa_copy_blocks_scaled.restype = i32
        L.pa_copy_blocks_scaled.argtypes = [vp] * 5 + [i32] * 7 + [vp]
        L.pa_prefill.restype = i32
        L.pa_prefill.argtypes = [vp] * 7 + [i32] * 9 + [f32, i32, i32, f32, f32, vp]
        L.pa_decode_shared_prefix_workspace_size.restype = sz
        L.pa_decode_shared_prefix_workspace_size.argtypes = [i32] * 7
        L.pa_decode_shared_prefix.restype = i32
        L.pa_decode_shared_prefix.argtypes = ([vp] * 8 + [i32] * 9 +
                                              [f32, i32, i32, f32, f32, vp, sz, vp])
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != 0:
        raise PaError(f"libpa: {lib().pa_status_string(status).decode()} (status {status})")


def dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise PaError(f"unsupported element type {t.dtype}") from None


def _dev(*tensors) -> torch.device:
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise PaError("libpa operations take GPU tensors only (no CPU path)")
        if not t.is_contiguous():
            raise PaError("libpa operations take contiguous tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise PaError("all tensors must be on the same GPU")
    return dev


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _i32(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.int32:
        raise PaError(f"{name} must be int32")


def _i64(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.int64:
        raise PaError(f"{name} must be int64")


def _scale_arg(scale: Optional[float]) -> float:
    """The softmax scale as passed to the C ABI: None becomes a NaN, which the
    library resolves to its default 1/sqrt(head_dim)."""
    return float("nan") if scale is None else float(scale)


def num_partitions(max_blocks_per_seq: int, block_size: int, partition_size: int) -> int:
    return lib().pa_num_partitions(max_blocks_per_seq, block_size, partition_size)


def decode_balanced_splits(num_q_heads: int, num_kv_heads: int, head_dim: int,
                           q_dtype: torch.dtype, kv_dtype: torch.dtype) -> int:
    """Share count of the automatic balanced split on the current device
    (C: pa_decode_balanced_splits); 0 for an unsupported configuration."""
    return lib().pa_decode_balanced_splits(num_q_heads, num_kv_heads, head_dim,
                                           _DTYPES[q_dtype], _DTYPES[kv_dtype])


def decode_workspace_size(num_seqs: int, num_q_heads: int, head_dim: int,
                          max_blocks_per_seq: int, block_size: int, partition_size: int) -> int:
    return lib().pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                                          block_size, partition_size)


def _decode_shapes(q, k_cache, v_cache, block_tables, context_lens):
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise PaError("expected q [B, Hq, d] and caches [num_blocks, block_size, Hkv, d]")
    B, Hq, d = q.shape
    NB, bs, Hkv, d2 = k_cache.shape
    if d2 != d or block_tables.dim() != 2 or block_tables.shape[0] != B or \
            context_lens.shape != (B,):
        raise PaError("inconsistent shapes among q, caches, block_tables, context_lens")
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    return B, Hq, d, NB, bs, Hkv, block_tables.shape[1]


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: Optional[float] = None,
           k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 0,
           out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged-attention decode (C: pa_decode). Returns out [B, Hq, d] in q's type."""
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens, out, workspace)
    B, Hq, d, NB, bs, Hkv, MBS = _decode_shapes(q, k_cache, v_cache, block_tables, context_lens)
    if checks.debug_checks_enabled():
        checks.check_decode(block_tables, context_lens, NB, bs)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise PaError("out must match q in shape and type")
    need = decode_workspace_size(B, Hq, d, MBS, bs, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                           _ptr(context_lens), B, Hq, Hkv, d, bs, NB, MBS, _scale_arg(scale),
                           dtype_code(q), dtype_code(k_cache), float(k_scale), float(v_scale),
                           int(partition_size), _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor,
                   scale: Optional[float] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                   partition_size: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode() with the split partials in the library's fixed per-device
    scratch instead of a workspace (C: pa_decode_noalloc). Pass ``out`` to
    allocate nothing at all. Calls that overlap on one GPU race on the
    scratch."""
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens, out)
    B, Hq, d, NB, bs, Hkv, MBS = _decode_shapes(q, k_cache, v_cache, block_tables, context_lens)
    if checks.debug_checks_enabled():
        checks.check_decode(block_tables, context_lens, NB, bs)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise PaError("out must match q in shape and type")
    _check(lib().pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, d, bs,
                                   NB, MBS, _scale_arg(scale), dtype_code(q),
                                   dtype_code(k_cache), float(k_scale), float(v_scale),
                                   int(partition_size), _stream(dev)))
    return out


def decode_noalloc_scratch_bytes() -> int:
    return lib().pa_decode_noalloc_scratch_bytes()


def prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
            block_tables: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor,
            max_query_len: Optional[int] = None, scale: Optional[float] = None,
            k_scale: float = 1.0, v_scale: float = 1.0,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged (chunked) prefill (C: pa_prefill): rows query_start[b] ..
    query_start[b + 1] - 1 of q [T, Hq, d] are the last tokens of sequence b's
    context_lens[b] cached tokens and attend causally over them. Returns out
    [T, Hq, d] in q's type. Without max_query_len the longest chunk is read
    from a host copy of query_start (a synchronisation)."""
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens, query_start, out)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise PaError("expected q [T, Hq, d] and caches [num_blocks, block_size, Hkv, d]")
    T, Hq, d = q.shape
    NB, bs, Hkv, d2 = k_cache.shape
    B = context_lens.shape[0]
    if d2 != d or block_tables.dim() != 2 or block_tables.shape[0] != B or \
            query_start.shape != (B + 1,):
        raise PaError("inconsistent shapes among q, caches, block_tables, context_lens, "
                      "query_start")
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    _i32(query_start, "query_start")
    if checks.debug_checks_enabled():
        checks.check_decode(block_tables, context_lens, NB, bs)
        checks.check_query_start(query_start, context_lens, T)
    if max_query_len is None:
        qs = query_start.to("cpu")
        max_query_len = int((qs[1:] - qs[:-1]).max()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise PaError("out must match q in shape and type")
    _check(lib().pa_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                            _ptr(context_lens), _ptr(query_start), B, T, int(max_query_len), Hq,
                            Hkv, d, bs, NB, block_tables.shape[1], _scale_arg(scale),
                            dtype_code(q), dtype_code(k_cache), float(k_scale), float(v_scale),
                            _stream(dev)))
    return out


def decode_shared_prefix_workspace_size(num_seqs: int, num_groups: int, group_size: int,
                                        num_q_heads: int, head_dim: int,
                                        max_blocks_per_seq: int, q_dtype: torch.dtype) -> int:
    return lib().pa_decode_shared_prefix_workspace_size(
        num_seqs, num_groups, group_size, num_q_heads, head_dim, max_blocks_per_seq,
        _DTYPES[q_dtype])


def decode_shared_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor,
                         group_members: torch.Tensor, prefix_lens: torch.Tensor,
                         scale: Optional[float] = None, k_scale: float = 1.0,
                         v_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode for groups of sequences sharing a prompt prefix, each shared
    block read once per group (C: pa_decode_shared_prefix). group_members
    [G, M] int32 (sequence ids, -1 for an empty slot), prefix_lens [G] int32
    (tokens). Returns out [B, Hq, d] in q's type: the same attention as
    decode()."""
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens, group_members, prefix_lens, out,
               workspace)
    B, Hq, d, NB, bs, Hkv, MBS = _decode_shapes(q, k_cache, v_cache, block_tables, context_lens)
    if checks.debug_checks_enabled():
        checks.check_decode(block_tables, context_lens, NB, bs)
    if group_members.dim() != 2 or prefix_lens.shape != (group_members.shape[0],):
        raise PaError("group_members must be [G, M] and prefix_lens [G]")
    _i32(group_members, "group_members")
    _i32(prefix_lens, "prefix_lens")
    if checks.debug_checks_enabled():
        checks.check_shared_prefix(block_tables, context_lens, group_members, prefix_lens, bs)
    G, M = group_members.shape
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise PaError("out must match q in shape and type")
    if workspace is None:
        need = decode_shared_prefix_workspace_size(B, G, M, Hq, d, MBS, q.dtype)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_shared_prefix(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(group_members), _ptr(prefix_lens), B, G, M, Hq, Hkv, d, bs, NB, MBS, _scale_arg(scale),
        dtype_code(q), dtype_code(k_cache), float(k_scale), float(v_scale), _ptr(workspace),
        ws_bytes, _stream(dev)))
    return out


def decode_append(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, scale: Optional[float] = None,
                  k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 0,
                  out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step with the new token appended (C: pa_decode_append): key
    and value [B, Hkv, d] (q's type) are written to each sequence's last
    position, then out = decode over the caches. Returns out [B, Hq, d]."""
    dev = _dev(q, key, value, k_cache, v_cache, block_tables, context_lens, out, workspace)
    B, Hq, d, NB, bs, Hkv, MBS = _decode_shapes(q, k_cache, v_cache, block_tables, context_lens)
    if checks.debug_checks_enabled():
        checks.check_decode(block_tables, context_lens, NB, bs)
    if key.shape != (B, Hkv, d) or value.shape != key.shape or key.dtype != q.dtype or \
            value.dtype != q.dtype:
        raise PaError("key and value must be [B, Hkv, d] in q's type")
    if checks.debug_checks_enabled():
        checks.check_append(block_tables, context_lens, bs)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise PaError("out must match q in shape and type")
    need = decode_workspace_size(B, Hq, d, MBS, bs, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_append(_ptr(out), _ptr(q), _ptr(key.contiguous()),
                                  _ptr(value.contiguous()), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, d, bs, NB,
                                  MBS, _scale_arg(scale), dtype_code(q), dtype_code(k_cache),
                                  float(k_scale), float(v_scale), int(partition_size),
                                  _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def decode_partials(q, k_cache, v_cache, block_tables, context_lens, partition_size: int,
                    scale: Optional[float] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                    tmp_out=None, max_logits=None, exp_sums=None
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Split-context partials (C: pa_decode_partials), float32.

    Fixed split (partition_size > 0): tmp_out [B, Hq, NP, d], max_logits and
    exp_sums [B, Hq, NP]. Balanced split (partition_size = -S, S >= 2):
    tmp_out [Hq, S + B, d], max_logits and exp_sums [Hq, S + B]."""
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens, tmp_out, max_logits, exp_sums)
    B, Hq, d, NB, bs, Hkv, MBS = _decode_shapes(q, k_cache, v_cache, block_tables, context_lens)
    if checks.debug_checks_enabled():
        checks.check_decode(block_tables, context_lens, NB, bs)
    lead = (B, Hq) if partition_size > 0 else (Hq,)
    if tmp_out is None:
        NP = num_partitions(MBS, bs, partition_size) if partition_size > 0 \
            else -partition_size + B
        tmp_out = torch.empty(lead + (NP, d), dtype=torch.float32, device=dev)
        max_logits = torch.empty(lead + (NP,), dtype=torch.float32, device=dev)
        exp_sums = torch.empty(lead + (NP,), dtype=torch.float32, device=dev)
    for t in (tmp_out, max_logits, exp_sums):
        if t.dtype != torch.float32:
            raise PaError("partials are float32")
    n = len(lead)
    if tmp_out.dim() != n + 2 or tuple(tmp_out.shape[:n]) != lead or tmp_out.shape[-1] != d or \
            max_logits.shape != tmp_out.shape[:-1] or exp_sums.shape != tmp_out.shape[:-1]:
        raise PaError("partials have the wrong shape")
    _check(lib().pa_decode_partials(_ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums),
                                    tmp_out.shape[n], _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, d, bs,
                                    NB, MBS, _scale_arg(scale), dtype_code(q), dtype_code(k_cache),
                                    float(k_scale), float(v_scale), int(partition_size),
                                    _stream(dev)))
    return tmp_out, max_logits, exp_sums


def decode_reduce(tmp_out, max_logits, exp_sums, context_lens, partition_size: int,
                  out_dtype: torch.dtype = torch.bfloat16,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Merge split partials (C: pa_decode_reduce). Returns out [B, Hq, d]; the
    partial layout follows partition_size as in decode_partials."""
    dev = _dev(tmp_out, max_logits, exp_sums, context_lens, out)
    _i32(context_lens, "context_lens")
    B = context_lens.shape[0]
    if partition_size > 0:
        _, Hq, NP, d = tmp_out.shape
    else:
        Hq, NP, d = tmp_out.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=dev)
    if out.dtype not in _TORCH_OF.values() or out.shape != (B, Hq, d):
        raise PaError("out must be [B, Hq, d] float32, float16 or bfloat16")
    _check(lib().pa_decode_reduce(_ptr(out), _ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums),
                                  _ptr(context_lens), B, Hq, d, NP, int(partition_size),
                                  dtype_code(out), _stream(dev)))
    return out


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float = 1.0,
                      v_scale: float = 1.0) -> None:
    """Write new tokens' K/V rows into their slots (C: pa_reshape_and_cache)."""
    dev = _dev(key, value, k_cache, v_cache, slot_mapping)
    _i64(slot_mapping, "slot_mapping")
    if key.dim() != 3 or value.shape != key.shape or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape or key.shape[1:] != k_cache.shape[2:] or \
            slot_mapping.shape != (key.shape[0],) or value.dtype != key.dtype or \
            v_cache.dtype != k_cache.dtype:
        raise PaError("expected key/value [N, Hkv, d], caches [num_blocks, bs, Hkv, d], slots [N]")
    N, Hkv, d = key.shape
    NB, bs = k_cache.shape[:2]
    if checks.debug_checks_enabled():
        checks.check_slot_mapping(slot_mapping, NB, bs)
    _check(lib().pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(slot_mapping), N, Hkv, d, bs, NB, dtype_code(key),
                                      dtype_code(k_cache), float(k_scale), float(v_scale),
                                      _stream(dev)))


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_mapping: torch.Tensor) -> None:
    """Copy-on-write block copies (C: pa_copy_blocks); block_mapping [P, 2] int64 (src, dst)."""
    dev = _dev(k_cache, v_cache, block_mapping)
    _i64(block_mapping, "block_mapping")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2 or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise PaError("expected caches [num_blocks, bs, Hkv, d] and block_mapping [P, 2]")
    NB, bs, Hkv, d = k_cache.shape
    if checks.debug_checks_enabled():
        checks.check_block_mapping(block_mapping, NB)
    _check(lib().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_mapping),
                                block_mapping.shape[0], Hkv, d, bs, NB, dtype_code(k_cache),
                                _stream(dev)))


def _scale_tables(k_scales: torch.Tensor, v_scales: torch.Tensor, layout: int, num_blocks: int,
                  num_kv_heads: int) -> None:
    """Checks that the two scale tables are float32 and shaped for ``layout``."""
    want = {PA_SCALE_PER_HEAD: (num_kv_heads,), PA_SCALE_PER_BLOCK: (num_blocks,),
            PA_SCALE_PER_BLOCK_HEAD: (num_blocks, num_kv_heads)}.get(int(layout))
    if want is None:
        raise PaError(f"unknown scale layout {layout}")
    for t, name in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if t.dtype != torch.float32 or tuple(t.shape) != want:
            raise PaError(f"{name} must be float32 {list(want)} for layout {layout}")


def decode_scaled(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  block_tables: torch.Tensor, context_lens: torch.Tensor,
                  k_scales: torch.Tensor, v_scales: torch.Tensor, scale_layout: int,
                  scale: Optional[float] = None, partition_size: int = 0,
                  out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode over an 8-bit cache with scale tables per KV head, per block or
    per (block, KV head) (C: pa_decode_scaled). Returns out [B, Hq, d]."""
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens, k_scales, v_scales, out,
               workspace)
    B, Hq, d, NB, bs, Hkv, MBS = _decode_shapes(q, k_cache, v_cache, block_tables, context_lens)
    _scale_tables(k_scales, v_scales, scale_layout, NB, Hkv)
    if checks.debug_checks_enabled():
        checks.check_decode(block_tables, context_lens, NB, bs)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise PaError("out must match q in shape and type")
    need = decode_workspace_size(B, Hq, d, MBS, bs, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_scaled(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, d, bs, NB,
                                  MBS, _scale_arg(scale), dtype_code(q), dtype_code(k_cache),
                                  _ptr(k_scales), _ptr(v_scales), int(scale_layout),
                                  int(partition_size), _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def reshape_and_cache_scaled(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                             v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                             k_scales: torch.Tensor, v_scales: torch.Tensor,
                             scale_layout: int) -> None:
    """Slot write into an 8-bit cache, each row quantised with its block's
    (and head's) scale (C: pa_reshape_and_cache_scaled)."""
    dev = _dev(key, value, k_cache, v_cache, slot_mapping, k_scales, v_scales)
    _i64(slot_mapping, "slot_mapping")
    if key.dim() != 3 or value.shape != key.shape or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape or key.shape[1:] != k_cache.shape[2:] or \
            slot_mapping.shape != (key.shape[0],) or value.dtype != key.dtype or \
            v_cache.dtype != k_cache.dtype:
        raise PaError("expected key/value [N, Hkv, d], caches [num_blocks, bs, Hkv, d], slots [N]")
    N, Hkv, d = key.shape
    NB, bs = k_cache.shape[:2]
    _scale_tables(k_scales, v_scales, scale_layout, NB, Hkv)
    if checks.debug_checks_enabled():
        checks.check_slot_mapping(slot_mapping, NB, bs)
    _check(lib().pa_reshape_and_cache_scaled(_ptr(key), _ptr(value), _ptr(k_cache),
                                             _ptr(v_cache), _ptr(slot_mapping), N, Hkv, d, bs, NB,
                                             dtype_code(key), dtype_code(k_cache),
                                             _ptr(k_scales), _ptr(v_scales), int(scale_layout),
                                             _stream(dev)))


def copy_blocks_scaled(k_cache: torch.Tensor, v_cache: torch.Tensor, k_scales: torch.Tensor,
                       v_scales: torch.Tensor, scale_layout: int,
                       block_mapping: torch.Tensor) -> None:
    """Copy-on-write copies of blocks and their scales (C: pa_copy_blocks_scaled)."""
    dev = _dev(k_cache, v_cache, k_scales, v_scales, block_mapping)
    _i64(block_mapping, "block_mapping")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2 or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise PaError("expected caches [num_blocks, bs, Hkv, d] and block_mapping [P, 2]")
    NB, bs, Hkv, d = k_cache.shape
    _scale_tables(k_scales, v_scales, scale_layout, NB, Hkv)
    if checks.debug_checks_enabled():
        checks.check_block_mapping(block_mapping, NB)
    _check(lib().pa_copy_blocks_scaled(_ptr(k_cache), _ptr(v_cache), _ptr(k_scales),
                                       _ptr(v_scales), _ptr(block_mapping),
                                       block_mapping.shape[0], Hkv, d, bs, NB,
                                       dtype_code(k_cache), int(scale_layout), _stream(dev)))
