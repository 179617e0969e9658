"""Thin Python binding of the C ABI in include/pkv.h (ctypes).

Argument marshalling only: shapes are read off the tensors, pointers and the
current HIP stream are passed through, the C status code is turned into an
exception.  Every step of the computation runs in the library's kernels; if
``libpkv.so`` is missing, loading fails loudly (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_ELAUNCH, PKV_EVALIDATE = 0, -1, -2, -3, -4, -5
BLOCK_SIZE = 16

_c_int, _c_size, _vp, _f = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

SIGNATURES = {
    "pkv_slot_mapping": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp]),
    "pkv_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "pkv_decode_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "pkv_decode_num_splits": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "pkv_attn_decode": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _c_int, _c_int, _f, _vp, _c_size, _vp]),
    "pkv_attn_decode_append": (_c_int, [_vp] * 8 + [_c_int] * 8 + [_f, _vp, _c_size, _vp]),
    "pkv_attn_decode_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                         _c_int, _c_int, _c_int, _c_int, _c_int, _f, _vp]),
    "pkv_prefill_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "pkv_attn_prefill_chunk": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                        _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                        _f, _vp, _c_size, _vp]),
    "pkv_attn_prefill_decode": (_c_int, [_vp] * 5 + [_c_int] * 4 + [_vp] * 4 + [_c_int] * 2 +
                                [_vp] * 2 + [_c_int] * 6 +
                                [_f, _vp, _c_size, _vp, _c_size, _vp]),
    "pkv_attn_prefill_decode_int8": (_c_int, [_vp] * 5 + [_c_int] * 4 + [_vp] * 4 + [_c_int] * 2 +
                                     [_vp] * 4 + [_c_int] * 6 +
                                     [_f, _vp, _c_size, _vp, _c_size, _vp]),
    "pkv_attn_prefill_decode_append": (_c_int, [_vp] * 5 + [_c_int] * 4 + [_vp] * 4 +
                                       [_c_int] * 2 + [_vp] * 5 + [_c_int] * 6 +
                                       [_f, _vp, _c_size, _vp, _c_size, _vp]),
    "pkv_append_int8": (_c_int, [_vp] * 7 + [_c_int] * 5 + [_vp]),
    "pkv_attn_decode_int8": (_c_int, [_vp] * 8 + [_c_int] * 8 + [_f, _vp, _c_size, _vp]),
    "pkv_attn_decode_append_int8": (_c_int, [_vp] * 10 + [_c_int] * 8 + [_f, _vp, _c_size, _vp]),
    "pkv_copy_blocks": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, ctypes.c_int64, _c_int,
                                 ctypes.c_int64, _vp]),
    "pkv_slot_mapping_ring": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _vp]),
    "pkv_attn_decode_ring": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                      _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _f, _vp,
                                      _c_size, _vp]),
    "pkv_attn_prefill_chunk_ring": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _f, _vp, _c_size, _vp]),
    "pkv_attn_prefill_chunk_int8": (_c_int, [_vp] * 9 + [_c_int] * 10 + [_f, _vp, _c_size, _vp]),
    "pkv_qk_norm_rope_append": (_c_int, [_vp] * 8 + [_c_int] + [_vp] * 6 +
                                [_c_int] * 8 + [_f, _vp]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
}


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pkv error {code}: {msg}")
        self.code = code


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv.so (built in-tree by ``python -m paged_kv_gqa_pkv_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m paged_kv_gqa_pkv_amd.build` "
                           "(the library has no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != PKV_OK:
        msg = load().pkv_last_error()
        raise PkvError(rc, msg.decode() if msg else "")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, dtype, name: str, ndim: Optional[int] = None) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def pkv_slot_mapping(slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                     cu_new_lens: torch.Tensor, context_lens: torch.Tensor, stream=None) -> None:
    """slot_mapping[int32 T] <- slots of the appended tokens (see include/pkv.h)."""
    for t, n in ((slot_mapping, "slot_mapping"), (block_tables, "block_tables"),
                 (cu_new_lens, "cu_new_lens"), (context_lens, "context_lens")):
        _need(t, torch.int32, n)
    B, mb = block_tables.shape
    _check(load().pkv_slot_mapping(_p(slot_mapping), _p(block_tables), _p(cu_new_lens),
                                   _p(context_lens), B, mb, slot_mapping.numel(), BLOCK_SIZE,
                                   _stream(stream)))


def pkv_append(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
               k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Scatter k_new/v_new [T, Hkv, D] into the pools [num_blocks, 16, Hkv, D]."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, torch.bfloat16, n, 3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    _need(slot_mapping, torch.int32, "slot_mapping", 1)
    T, Hkv, D = k_new.shape
    nb = k_cache.shape[0]
    if v_new.shape != k_new.shape or v_cache.shape != k_cache.shape or \
            k_cache.shape[2] != Hkv or k_cache.shape[3] != D or slot_mapping.numel() != T:
        raise ValueError("inconsistent shapes")
    _check(load().pkv_append(_p(k_new), _p(v_new), _p(slot_mapping), _p(k_cache), _p(v_cache),
                             T, nb, Hkv, D, k_cache.shape[1], _stream(stream)))


def pkv_decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, max_context_len: int) -> int:
    return int(load().pkv_decode_workspace_bytes(B, Hq, Hkv, D, max_context_len))


def pkv_decode_num_splits(B: int, Hq: int, Hkv: int, D: int, max_context_len: int) -> int:
    return int(load().pkv_decode_num_splits(B, Hq, Hkv, D, max_context_len))


def pkv_prefill_workspace_bytes(B: int, max_q_len: int, Hq: int, Hkv: int, D: int,
                                max_context_len: int) -> int:
    return int(load().pkv_prefill_workspace_bytes(B, max_q_len, Hq, Hkv, D, max_context_len))


def _ws(workspace):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return _p(workspace), workspace.numel() * workspace.element_size()


def pkv_attn_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                    v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                    max_context_len: int, scale: float, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> None:
    """out[B, Hq, D] <- decode attention of q[B, Hq, D] over the paged pools.
    ``workspace``: zero-filled before first use (the library keeps it so)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(out, torch.bfloat16, "out", 3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, Hq, D = q.shape
    nb, bs, Hkv, D2 = k_cache.shape            # [num_blocks, 16, Hkv, D] pages
    if out.shape != q.shape or D2 != D or v_cache.shape != k_cache.shape or \
            block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent shapes")
    ws_ptr, ws_bytes = _ws(workspace)
    _check(load().pkv_attn_decode(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                                  _p(context_lens), B, Hq, Hkv, D, bs, nb, block_tables.shape[1],
                                  int(max_context_len), float(scale), ws_ptr, ws_bytes,
                                  _stream(stream)))


def pkv_attn_decode_append(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                           v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, scale: float,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Append k_new/v_new [B, Hkv, D] (one token per sequence, at position
    context_lens[b] - 1) and run decode attention, in one launch."""
    _need(q, torch.bfloat16, "q", 3)
    _need(out, torch.bfloat16, "out", 3)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, torch.bfloat16, n, 3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, Hq, D = q.shape
    nb, bs, Hkv, D2 = k_cache.shape
    if out.shape != q.shape or D2 != D or v_cache.shape != k_cache.shape or \
            k_new.shape != (B, Hkv, D) or v_new.shape != k_new.shape or \
            block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent shapes")
    ws_ptr, ws_bytes = _ws(workspace)
    _check(load().pkv_attn_decode_append(_p(out), _p(q), _p(k_new), _p(v_new), _p(k_cache),
                                         _p(v_cache), _p(block_tables), _p(context_lens), B, Hq,
                                         Hkv, D, bs, nb, block_tables.shape[1],
                                         int(max_context_len), float(scale), ws_ptr, ws_bytes,
                                         _stream(stream)))


def pkv_attn_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, max_context_len: int, scale: float,
                            stream=None) -> None:
    """pkv_attn_decode with the split buffers in the library's per-GPU array
    (nothing allocated; calls that overlap in time on one GPU race)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(out, torch.bfloat16, "out", 3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, Hq, D = q.shape
    nb, bs, Hkv, D2 = k_cache.shape            # [num_blocks, 16, Hkv, D] pages
    if out.shape != q.shape or D2 != D or v_cache.shape != k_cache.shape or \
            block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent shapes")
    _check(load().pkv_attn_decode_noalloc(_p(out), _p(q), _p(k_cache), _p(v_cache),
                                          _p(block_tables), _p(context_lens), B, Hq, Hkv, D, bs,
                                          nb, block_tables.shape[1], int(max_context_len),
                                          float(scale), _stream(stream)))


def pkv_attn_prefill_chunk(out: torch.Tensor, q: torch.Tensor, cu_q_lens: torch.Tensor,
                           k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_q_len: int, max_context_len: int, scale: float,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """out[total_q, Hq, D] <- causal attention of the chunk rows q[total_q, Hq, D].
    ``workspace``: zero-filled before first use (the library keeps it so)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(out, torch.bfloat16, "out", 3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    for t, n in ((cu_q_lens, "cu_q_lens"), (context_lens, "context_lens")):
        _need(t, torch.int32, n, 1)
    _need(block_tables, torch.int32, "block_tables", 2)
    total_q, Hq, D = q.shape
    nb, bs, Hkv, D2 = k_cache.shape            # [num_blocks, 16, Hkv, D] pages
    B = context_lens.numel()
    if out.shape != q.shape or D2 != D or v_cache.shape != k_cache.shape or \
            block_tables.shape[0] != B or cu_q_lens.numel() != B + 1:
        raise ValueError("inconsistent shapes")
    _check(load().pkv_attn_prefill_chunk(_p(out), _p(q), _p(cu_q_lens), _p(k_cache), _p(v_cache),
                                         _p(block_tables), _p(context_lens), B, total_q,
                                         int(max_q_len), Hq, Hkv, D, bs, nb,
                                         block_tables.shape[1], int(max_context_len),
                                         float(scale), *_ws(workspace), _stream(stream)))


def pkv_attn_prefill_decode(out_prefill: torch.Tensor, q_prefill: torch.Tensor,
                            cu_q_lens: torch.Tensor, block_tables_prefill: torch.Tensor,
                            context_lens_prefill: torch.Tensor, max_q_len: int,
                            max_context_len_prefill: int, out_decode: torch.Tensor,
                            q_decode: torch.Tensor, block_tables_decode: torch.Tensor,
                            context_lens_decode: torch.Tensor, max_context_len_decode: int,
                            k_cache: torch.Tensor, v_cache: torch.Tensor, scale: float,
                            prefill_workspace: Optional[torch.Tensor] = None,
                            decode_workspace: Optional[torch.Tensor] = None,
                            stream=None) -> None:
    """A mixed step's attention in one call: the chunk rows q_prefill
    [total_q, Hq, D] and the decode rows q_decode [B_decode, Hq, D], as
    pkv_attn_prefill_chunk and pkv_attn_decode give them.  Both block tables
    share their row width; workspaces as for the two calls."""
    for t, n in ((q_prefill, "q_prefill"), (out_prefill, "out_prefill"),
                 (q_decode, "q_decode"), (out_decode, "out_decode")):
        _need(t, torch.bfloat16, n, 3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    for t, n in ((cu_q_lens, "cu_q_lens"), (context_lens_prefill, "context_lens_prefill"),
                 (context_lens_decode, "context_lens_decode")):
        _need(t, torch.int32, n, 1)
    for t, n in ((block_tables_prefill, "block_tables_prefill"),
                 (block_tables_decode, "block_tables_decode")):
        _need(t, torch.int32, n, 2)
    total_q, Hq, D = q_prefill.shape
    B_d = q_decode.shape[0]
    nb, bs, Hkv, D2 = k_cache.shape            # [num_blocks, 16, Hkv, D] pages
    B_p = context_lens_prefill.numel()
    width = block_tables_prefill.shape[1]
    if out_prefill.shape != q_prefill.shape or out_decode.shape != q_decode.shape or \
            q_decode.shape[1:] != (Hq, D) or D2 != D or v_cache.shape != k_cache.shape or \
            block_tables_prefill.shape[0] != B_p or cu_q_lens.numel() != B_p + 1 or \
            block_tables_decode.shape != (B_d, width) or context_lens_decode.numel() != B_d:
        raise ValueError("inconsistent shapes")
    pw, pwb = _ws(prefill_workspace)
    dw, dwb = _ws(decode_workspace)
    _check(load().pkv_attn_prefill_decode(
        _p(out_prefill), _p(q_prefill), _p(cu_q_lens), _p(block_tables_prefill),
        _p(context_lens_prefill), B_p, total_q, int(max_q_len), int(max_context_len_prefill),
        _p(out_decode), _p(q_decode), _p(block_tables_decode), _p(context_lens_decode), B_d,
        int(max_context_len_decode), _p(k_cache), _p(v_cache), Hq, Hkv, D, bs, nb, width,
        float(scale), pw, pwb, dw, dwb, _stream(stream)))


def pkv_attn_prefill_decode_append(out_prefill: torch.Tensor, q_prefill: torch.Tensor,
                                   cu_q_lens: torch.Tensor, block_tables_prefill: torch.Tensor,
                                   context_lens_prefill: torch.Tensor, max_q_len: int,
                                   max_context_len_prefill: int, out_decode: torch.Tensor,
                                   q_decode: torch.Tensor, block_tables_decode: torch.Tensor,
                                   context_lens_decode: torch.Tensor,
                                   max_context_len_decode: int, k_new: torch.Tensor,
                                   v_new: torch.Tensor, slot_mapping: torch.Tensor,
                                   k_cache: torch.Tensor, v_cache: torch.Tensor, scale: float,
                                   prefill_workspace: Optional[torch.Tensor] = None,
                                   decode_workspace: Optional[torch.Tensor] = None,
                                   stream=None) -> None:
    """A mixed step's append and attention in one call: k_new/v_new
    [total_q + B_decode, Hkv, D] (the chunk rows, then one row per decode
    sequence) go into their slots (slot_mapping, the step's) and both halves'
    attention runs as in pkv_attn_prefill_decode."""
    for t, n in ((q_prefill, "q_prefill"), (out_prefill, "out_prefill"),
                 (q_decode, "q_decode"), (out_decode, "out_decode"), (k_new, "k_new"),
                 (v_new, "v_new")):
        _need(t, torch.bfloat16, n, 3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    for t, n in ((cu_q_lens, "cu_q_lens"), (context_lens_prefill, "context_lens_prefill"),
                 (context_lens_decode, "context_lens_decode"), (slot_mapping, "slot_mapping")):
        _need(t, torch.int32, n, 1)
    for t, n in ((block_tables_prefill, "block_tables_prefill"),
                 (block_tables_decode, "block_tables_decode")):
        _need(t, torch.int32, n, 2)
    total_q, Hq, D = q_prefill.shape
    B_d = q_decode.shape[0]
    nb, bs, Hkv, D2 = k_cache.shape            # [num_blocks, 16, Hkv, D] pages
    B_p = context_lens_prefill.numel()
    width = block_tables_prefill.shape[1]
    if out_prefill.shape != q_prefill.shape or out_decode.shape != q_decode.shape or \
            q_decode.shape[1:] != (Hq, D) or D2 != D or v_cache.shape != k_cache.shape or \
            block_tables_prefill.shape[0] != B_p or cu_q_lens.numel() != B_p + 1 or \
            block_tables_decode.shape != (B_d, width) or context_lens_decode.numel() != B_d or \
            k_new.shape != (total_q + B_d, Hkv, D) or v_new.shape != k_new.shape or \
            slot_mapping.numel() != total_q + B_d:
        raise ValueError("inconsistent shapes")
    pw, pwb = _ws(prefill_workspace)
    dw, dwb = _ws(decode_workspace)
    _check(load().pkv_attn_prefill_decode_append(
        _p(out_prefill), _p(q_prefill), _p(cu_q_lens), _p(block_tables_prefill),
        _p(context_lens_prefill), B_p, total_q, int(max_q_len), int(max_context_len_prefill),
        _p(out_decode), _p(q_decode), _p(block_tables_decode), _p(context_lens_decode), B_d,
        int(max_context_len_decode), _p(k_new), _p(v_new), _p(slot_mapping), _p(k_cache),
        _p(v_cache), Hq, Hkv, D, bs, nb, width, float(scale), pw, pwb, dw, dwb,
        _stream(stream)))


def _need_scales(k_scales: torch.Tensor, v_scales: torch.Tensor, codes: torch.Tensor) -> None:
    for t, n in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        _need(t, torch.float32, n, 3)
    want = (codes.shape[0], codes.shape[2], codes.shape[1])
    if tuple(k_scales.shape) != want or tuple(v_scales.shape) != want:
        raise ValueError("scales must be [num_blocks, Hkv, 16] (a page's scales head-major)")


def pkv_append_int8(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                    k_codes: torch.Tensor, v_codes: torch.Tensor, k_scales: torch.Tensor,
                    v_scales: torch.Tensor, stream=None) -> None:
    """Quantise k_new/v_new [T, Hkv, D] into int8 pools: codes [num_blocks, 16, Hkv, D],
    scales [num_blocks, Hkv, 16] for K and for V."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, torch.bfloat16, n, 3)
    for t, n in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _need(t, torch.int8, n, 4)
    _need_scales(k_scales, v_scales, k_codes)
    _need(slot_mapping, torch.int32, "slot_mapping", 1)
    T, Hkv, D = k_new.shape
    nb = k_codes.shape[0]
    if v_new.shape != k_new.shape or v_codes.shape != k_codes.shape or \
            k_codes.shape[2] != Hkv or k_codes.shape[3] != D or slot_mapping.numel() != T:
        raise ValueError("inconsistent shapes")
    _check(load().pkv_append_int8(_p(k_new), _p(v_new), _p(slot_mapping), _p(k_codes),
                                  _p(v_codes), _p(k_scales), _p(v_scales), T, nb, Hkv, D,
                                  k_codes.shape[1], _stream(stream)))


def pkv_attn_decode_append_int8(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                                v_new: torch.Tensor, k_codes: torch.Tensor, v_codes: torch.Tensor,
                                k_scales: torch.Tensor, v_scales: torch.Tensor,
                                block_tables: torch.Tensor, context_lens: torch.Tensor,
                                max_context_len: int, scale: float,
                                workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Quantise and append k_new/v_new [B, Hkv, D] (one token per sequence, at
    position context_lens[b] - 1) into int8 pools and run decode attention,
    in one launch (same workspace as pkv_attn_decode)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(out, torch.bfloat16, "out", 3)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, torch.bfloat16, n, 3)
    for t, n in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _need(t, torch.int8, n, 4)
    _need_scales(k_scales, v_scales, k_codes)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, Hq, D = q.shape
    nb, bs, Hkv, D2 = k_codes.shape
    if out.shape != q.shape or D2 != D or v_codes.shape != k_codes.shape or \
            k_new.shape != (B, Hkv, D) or v_new.shape != k_new.shape or \
            block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent shapes")
    ws_ptr, ws_bytes = _ws(workspace)
    _check(load().pkv_attn_decode_append_int8(_p(out), _p(q), _p(k_new), _p(v_new), _p(k_codes),
                                              _p(v_codes), _p(k_scales), _p(v_scales),
                                              _p(block_tables), _p(context_lens), B, Hq, Hkv, D,
                                              bs, nb, block_tables.shape[1], int(max_context_len),
                                              float(scale), ws_ptr, ws_bytes, _stream(stream)))


def pkv_attn_decode_int8(out: torch.Tensor, q: torch.Tensor, k_codes: torch.Tensor,
                         v_codes: torch.Tensor, k_scales: torch.Tensor, v_scales: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor,
                         max_context_len: int, scale: float,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """out[B, Hq, D] <- decode attention of q[B, Hq, D] over int8 pools (same
    workspace as pkv_attn_decode)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(out, torch.bfloat16, "out", 3)
    for t, n in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _need(t, torch.int8, n, 4)
    _need_scales(k_scales, v_scales, k_codes)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, Hq, D = q.shape
    nb, bs, Hkv, D2 = k_codes.shape
    if out.shape != q.shape or D2 != D or v_codes.shape != k_codes.shape or \
            block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent shapes")
    ws_ptr, ws_bytes = _ws(workspace)
    _check(load().pkv_attn_decode_int8(_p(out), _p(q), _p(k_codes), _p(v_codes), _p(k_scales),
                                       _p(v_scales), _p(block_tables), _p(context_lens), B, Hq,
                                       Hkv, D, bs, nb, block_tables.shape[1],
                                       int(max_context_len), float(scale), ws_ptr, ws_bytes,
                                       _stream(stream)))


def pkv_attn_prefill_decode_int8(out_prefill: torch.Tensor, q_prefill: torch.Tensor,
                                 cu_q_lens: torch.Tensor, block_tables_prefill: torch.Tensor,
                                 context_lens_prefill: torch.Tensor, max_q_len: int,
                                 max_context_len_prefill: int, out_decode: torch.Tensor,
                                 q_decode: torch.Tensor, block_tables_decode: torch.Tensor,
                                 context_lens_decode: torch.Tensor, max_context_len_decode: int,
                                 k_codes: torch.Tensor, v_codes: torch.Tensor,
                                 k_scales: torch.Tensor, v_scales: torch.Tensor, scale: float,
                                 prefill_workspace: Optional[torch.Tensor] = None,
                                 decode_workspace: Optional[torch.Tensor] = None,
                                 stream=None) -> None:
    """pkv_attn_prefill_decode over int8 pools (codes [num_blocks, 16, Hkv, D],
    scales [num_blocks, Hkv, 16]): the outputs of pkv_attn_prefill_chunk_int8
    and pkv_attn_decode_int8 from one call."""
    for t, n in ((q_prefill, "q_prefill"), (out_prefill, "out_prefill"),
                 (q_decode, "q_decode"), (out_decode, "out_decode")):
        _need(t, torch.bfloat16, n, 3)
    for t, n in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _need(t, torch.int8, n, 4)
    _need_scales(k_scales, v_scales, k_codes)
    for t, n in ((cu_q_lens, "cu_q_lens"), (context_lens_prefill, "context_lens_prefill"),
                 (context_lens_decode, "context_lens_decode")):
        _need(t, torch.int32, n, 1)
    for t, n in ((block_tables_prefill, "block_tables_prefill"),
                 (block_tables_decode, "block_tables_decode")):
        _need(t, torch.int32, n, 2)
    total_q, Hq, D = q_prefill.shape
    B_d = q_decode.shape[0]
    nb, bs, Hkv, D2 = k_codes.shape
    B_p = context_lens_prefill.numel()
    width = block_tables_prefill.shape[1]
    if out_prefill.shape != q_prefill.shape or out_decode.shape != q_decode.shape or \
            q_decode.shape[1:] != (Hq, D) or D2 != D or v_codes.shape != k_codes.shape or \
            block_tables_prefill.shape[0] != B_p or cu_q_lens.numel() != B_p + 1 or \
            block_tables_decode.shape != (B_d, width) or context_lens_decode.numel() != B_d:
        raise ValueError("inconsistent shapes")
    pw, pwb = _ws(prefill_workspace)
    dw, dwb = _ws(decode_workspace)
    _check(load().pkv_attn_prefill_decode_int8(
        _p(out_prefill), _p(q_prefill), _p(cu_q_lens), _p(block_tables_prefill),
        _p(context_lens_prefill), B_p, total_q, int(max_q_len), int(max_context_len_prefill),
        _p(out_decode), _p(q_decode), _p(block_tables_decode), _p(context_lens_decode), B_d,
        int(max_context_len_decode), _p(k_codes), _p(v_codes), _p(k_scales), _p(v_scales), Hq,
        Hkv, D, bs, nb, width, float(scale), pw, pwb, dw, dwb, _stream(stream)))


def pkv_attn_prefill_chunk_int8(out: torch.Tensor, q: torch.Tensor, cu_q_lens: torch.Tensor,
                                k_codes: torch.Tensor, v_codes: torch.Tensor,
                                k_scales: torch.Tensor, v_scales: torch.Tensor,
                                block_tables: torch.Tensor, context_lens: torch.Tensor,
                                max_q_len: int, max_context_len: int, scale: float,
                                workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """out[total_q, Hq, D] <- causal attention of the chunk rows over int8 pools
    (same workspace as pkv_attn_prefill_chunk)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(out, torch.bfloat16, "out", 3)
    for t, n in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _need(t, torch.int8, n, 4)
    _need_scales(k_scales, v_scales, k_codes)
    for t, n in ((cu_q_lens, "cu_q_lens"), (context_lens, "context_lens")):
        _need(t, torch.int32, n, 1)
    _need(block_tables, torch.int32, "block_tables", 2)
    total_q, Hq, D = q.shape
    nb, bs, Hkv, D2 = k_codes.shape
    B = context_lens.numel()
    if out.shape != q.shape or D2 != D or v_codes.shape != k_codes.shape or \
            block_tables.shape[0] != B or cu_q_lens.numel() != B + 1:
        raise ValueError("inconsistent shapes")
    _check(load().pkv_attn_prefill_chunk_int8(
        _p(out), _p(q), _p(cu_q_lens), _p(k_codes), _p(v_codes), _p(k_scales), _p(v_scales),
        _p(block_tables), _p(context_lens), B, total_q, int(max_q_len), Hq, Hkv, D, bs, nb,
        block_tables.shape[1], int(max_context_len), float(scale), *_ws(workspace),
        _stream(stream)))


def pkv_copy_blocks(src_blocks: torch.Tensor, dst_blocks: torch.Tensor, k_pool: torch.Tensor,
                    v_pool: Optional[torch.Tensor] = None, layered: bool = False,
                    stream=None) -> None:
    """Copy block src -> dst in every layer of the pools (copy-on-write / fork).
    layered=False: a pool is one layer, [num_blocks, ...], contiguous.
    layered=True: a pool is [n_layers, num_blocks, ...]; each layer contiguous,
    layers any 16-byte multiple apart."""
    _need(src_blocks, torch.int32, "src_blocks", 1)
    _need(dst_blocks, torch.int32, "dst_blocks", 1)
    if src_blocks.numel() != dst_blocks.numel():
        raise ValueError("src_blocks and dst_blocks differ in length")
    pools = [k_pool] + ([v_pool] if v_pool is not None else [])
    if len({tuple(p.shape) for p in pools}) != 1 or len({p.dtype for p in pools}) != 1 or \
            len({p.stride() for p in pools}) != 1:
        raise ValueError("k_pool and v_pool differ in shape, dtype or strides")
    if not all(p.is_cuda for p in pools):
        raise TypeError("pools must be device tensors")
    if layered:
        if k_pool.dim() < 3:
            raise ValueError("a layered pool is [n_layers, num_blocks, ...]")
        if not all(p[0].is_contiguous() for p in pools):
            raise ValueError("each layer of a pool must be contiguous")
        n_layers, num_blocks = k_pool.shape[0], k_pool.shape[1]
        stride = k_pool.stride(0) * k_pool.element_size()
    else:
        if k_pool.dim() < 2 or not all(p.is_contiguous() for p in pools):
            raise ValueError("a pool is a contiguous [num_blocks, ...] tensor")
        n_layers, num_blocks, stride = 1, k_pool.shape[0], 0
    block_bytes = (k_pool[0, 0] if layered else k_pool[0]).numel() * k_pool.element_size()
    _check(load().pkv_copy_blocks(_p(k_pool), _p(v_pool), _p(src_blocks), _p(dst_blocks),
                                  src_blocks.numel(), num_blocks, block_bytes, n_layers, stride,
                                  _stream(stream)))


def pkv_slot_mapping_ring(slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                          cu_new_lens: torch.Tensor, context_lens: torch.Tensor, window: int,
                          stream=None) -> None:
    """slot_mapping <- ring slots (position p at ring index p % window)."""
    for t, n in ((slot_mapping, "slot_mapping"), (block_tables, "block_tables"),
                 (cu_new_lens, "cu_new_lens"), (context_lens, "context_lens")):
        _need(t, torch.int32, n)
    B, mb = block_tables.shape
    _check(load().pkv_slot_mapping_ring(_p(slot_mapping), _p(block_tables), _p(cu_new_lens),
                                        _p(context_lens), B, mb, slot_mapping.numel(),
                                        BLOCK_SIZE, int(window), _stream(stream)))


def pkv_attn_decode_ring(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                         v_cache: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, max_context_len: int, window: int,
                         scale: float, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> None:
    """Decode over rings of `window` tokens (a sliding window)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(out, torch.bfloat16, "out", 3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, Hq, D = q.shape
    nb, bs, Hkv, D2 = k_cache.shape
    if out.shape != q.shape or D2 != D or v_cache.shape != k_cache.shape or \
            block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent shapes")
    ws_ptr, ws_bytes = _ws(workspace)
    _check(load().pkv_attn_decode_ring(_p(out), _p(q), _p(k_cache), _p(v_cache),
                                       _p(block_tables), _p(context_lens), B, Hq, Hkv, D, bs, nb,
                                       block_tables.shape[1], int(max_context_len), int(window),
                                       float(scale), ws_ptr, ws_bytes, _stream(stream)))


def pkv_attn_prefill_chunk_ring(out: torch.Tensor, q: torch.Tensor, cu_q_lens: torch.Tensor,
                                k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_tables: torch.Tensor, context_lens: torch.Tensor,
                                max_q_len: int, max_context_len: int, window: int, scale: float,
                                workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Causal chunk over rings of `window` tokens."""
    _need(q, torch.bfloat16, "q", 3)
    _need(out, torch.bfloat16, "out", 3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    for t, n in ((cu_q_lens, "cu_q_lens"), (context_lens, "context_lens")):
        _need(t, torch.int32, n, 1)
    _need(block_tables, torch.int32, "block_tables", 2)
    total_q, Hq, D = q.shape
    nb, bs, Hkv, D2 = k_cache.shape
    B = context_lens.numel()
    if out.shape != q.shape or D2 != D or v_cache.shape != k_cache.shape or \
            block_tables.shape[0] != B or cu_q_lens.numel() != B + 1:
        raise ValueError("inconsistent shapes")
    _check(load().pkv_attn_prefill_chunk_ring(
        _p(out), _p(q), _p(cu_q_lens), _p(k_cache), _p(v_cache), _p(block_tables),
        _p(context_lens), B, total_q, int(max_q_len), Hq, Hkv, D, bs, nb,
        block_tables.shape[1], int(max_context_len), int(window), float(scale),
        *_ws(workspace), _stream(stream)))


def pkv_qk_norm_rope_append(q_out: torch.Tensor, q_in: torch.Tensor, k_in: torch.Tensor,
                            v_in: torch.Tensor, q_norm_w: torch.Tensor, k_norm_w: torch.Tensor,
                            cos_table: torch.Tensor, sin_table: torch.Tensor,
                            block_tables: torch.Tensor, cu_new_lens: torch.Tensor,
                            context_lens: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, eps: float,
                            slot_mapping: Optional[torch.Tensor] = None, stream=None) -> None:
    """q/k RMSNorm + RoPE; rotated q to q_out, rotated k and v into their page slots."""
    for t, n in ((q_out, "q_out"), (q_in, "q_in"), (k_in, "k_in"), (v_in, "v_in")):
        _need(t, torch.bfloat16, n, 3)
    for t, n in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        _need(t, torch.bfloat16, n, 1)
    for t, n in ((cos_table, "cos_table"), (sin_table, "sin_table")):
        _need(t, torch.bfloat16, n, 2)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n, 4)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(cu_new_lens, torch.int32, "cu_new_lens", 1)
    _need(context_lens, torch.int32, "context_lens", 1)
    T, Hq, D = q_in.shape
    nb, bs, Hkv, D2 = k_cache.shape
    B = context_lens.numel()
    if q_out.shape != q_in.shape or k_in.shape != (T, Hkv, D) or v_in.shape != k_in.shape or \
            D2 != D or v_cache.shape != k_cache.shape or q_norm_w.numel() != D or \
            k_norm_w.numel() != D or cos_table.shape != sin_table.shape or \
            cos_table.shape[1] != D or block_tables.shape[0] != B or cu_new_lens.numel() != B + 1:
        raise ValueError("inconsistent shapes")
    if slot_mapping is not None:
        _need(slot_mapping, torch.int32, "slot_mapping", 1)
        if slot_mapping.numel() != T:
            raise ValueError("slot_mapping must hold T entries")
    _check(load().pkv_qk_norm_rope_append(
        _p(q_out), _p(q_in), _p(k_in), _p(v_in), _p(q_norm_w), _p(k_norm_w), _p(cos_table),
        _p(sin_table), cos_table.shape[0], _p(block_tables), _p(cu_new_lens), _p(context_lens),
        _p(slot_mapping), _p(k_cache), _p(v_cache), B, block_tables.shape[1], T, nb, Hq, Hkv, D,
        bs, float(eps), _stream(stream)))
