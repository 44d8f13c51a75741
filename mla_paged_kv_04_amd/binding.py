"""ctypes binding of libmla_decode.so (include/mla_decode.h).

Argument marshalling only: every step of the decode runs in the HIP kernels.
torch supplies device memory (outputs, metadata, workspace) and the current
HIP stream.  If the library is missing this module raises; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmla_decode.so")

MLA_OK = 0
BLOCK_SIZE = 64
D_K = 576
D_V = 512
TILE_META_INTS = 8
FP8_PAGE_BYTES = 41216     # codes [64][512] | bf16 rope [64][64] | fp32 scale [64]

_c_int = ctypes.c_int
_c_ptr = ctypes.c_void_p
_c_i64 = ctypes.c_int64
_c_size = ctypes.c_size_t
_c_float = ctypes.c_float

_SIGNATURES = {
    "mla_decode_num_parts": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int,
                                      ctypes.POINTER(_c_int)]),
    "mla_decode_workspace_bytes": (_c_int, [_c_int, _c_int, _c_int, _c_int,
                                            ctypes.POINTER(_c_size)]),
    "mla_decode_metadata": (_c_int, [_c_ptr, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_ptr, _c_ptr, _c_ptr]),
    "mla_decode_splitkv": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr,
                                    _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                    _c_ptr, _c_ptr, _c_int, _c_ptr, _c_size, _c_ptr, _c_ptr,
                                    _c_ptr]),
    "mla_decode_splitkv_timed": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr,
                                          _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                          _c_ptr, _c_ptr, _c_int, _c_ptr, _c_size, _c_ptr,
                                          _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "mla_decode_combine": (_c_int, [_c_ptr, _c_int, _c_int, _c_int, _c_ptr, _c_int, _c_ptr,
                                    _c_size, _c_ptr, _c_ptr, _c_ptr]),
    "mla_decode_fwd": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr, _c_int,
                                _c_int, _c_int, _c_int, _c_float, _c_int, _c_ptr, _c_ptr,
                                _c_int, _c_ptr, _c_size, _c_ptr, _c_ptr, _c_ptr]),
    "mla_kv_append": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr, _c_int, _c_int,
                               _c_ptr]),
    "mla_decode_splitkv_fp8": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr,
                                        _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                        _c_ptr, _c_ptr, _c_int, _c_ptr, _c_size, _c_ptr,
                                        _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "mla_decode_fwd_fp8": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr, _c_int,
                                    _c_int, _c_int, _c_int, _c_float, _c_int, _c_ptr, _c_ptr,
                                    _c_int, _c_ptr, _c_size, _c_ptr, _c_ptr, _c_ptr]),
    "mla_kv_append_fp8": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr, _c_int,
                                   _c_int, _c_ptr]),
    "mla_decode_sparse_workspace_bytes": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int,
                                                   ctypes.POINTER(_c_size)]),
    "mla_decode_sparse_metadata": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_ptr,
                                            _c_ptr, _c_ptr]),
    "mla_decode_sparse_fwd": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr, _c_int,
                                       _c_int, _c_int, _c_int, _c_float, _c_int, _c_ptr, _c_int,
                                       _c_ptr, _c_ptr, _c_int, _c_ptr, _c_size, _c_ptr, _c_ptr,
                                       _c_ptr, _c_ptr, _c_ptr]),
    "mla_decode_sparse_fwd_fp8": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr,
                                           _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                           _c_ptr, _c_int, _c_ptr, _c_ptr, _c_int, _c_ptr,
                                           _c_size, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "mla_decode_fwd_inline_plan": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr,
                                            _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                            _c_ptr, _c_ptr, _c_int, _c_ptr, _c_size, _c_ptr,
                                            _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "mla_decode_fwd_inline_plan_fp8": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int,
                                                _c_ptr, _c_int, _c_int, _c_int, _c_int,
                                                _c_float, _c_int, _c_ptr, _c_ptr, _c_int,
                                                _c_ptr, _c_size, _c_ptr, _c_ptr, _c_ptr,
                                                _c_ptr, _c_ptr]),
    "mla_decode_fwd_noalloc": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_int, _c_ptr,
                                        _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                        _c_ptr, _c_ptr, _c_ptr]),
    "mla_status_string": (ctypes.c_char_p, [_c_int]),
    "mla_last_hip_error": (ctypes.c_char_p, []),
    "mla_device_num_cus": (_c_int, [_c_int, ctypes.POINTER(_c_int)]),
}

_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        text = lib().mla_status_string(status).decode()
        hip = lib().mla_last_hip_error().decode() if status == -4 else ""
        super().__init__(f"{where}: {text}" + (f" ({hip})" if hip else ""))
        self.status = status


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mla_paged_kv_04_amd.build_lib` (there is no fallback path)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().mla_status_string(status).decode()


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MLAError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def device_num_cus(device=None) -> int:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    out = _c_int(0)
    _check(lib().mla_device_num_cus(dev.index or 0, ctypes.byref(out)), "mla_device_num_cus")
    return out.value


def num_parts(batch: int, s_q: int, h_q: int, h_kv: int = 1, num_cus: int = 256) -> int:
    out = _c_int(0)
    _check(lib().mla_decode_num_parts(batch, s_q, h_q, h_kv, num_cus, ctypes.byref(out)),
           "mla_decode_num_parts")
    return out.value


def workspace_bytes(batch: int, s_q: int, h_q: int, parts: int) -> int:
    out = _c_size(0)
    _check(lib().mla_decode_workspace_bytes(batch, s_q, h_q, parts, ctypes.byref(out)),
           "mla_decode_workspace_bytes")
    return out.value


@dataclass
class Metadata:
    tile_meta: torch.Tensor       # int32 [num_parts, 8]
    split_offsets: torch.Tensor   # int32 [batch + 1]
    num_parts: int
    s_q: int
    h_q: int


def _require(t: torch.Tensor, dtype, name: str, ndim: int | None = None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def metadata(seqlens: torch.Tensor, s_q: int, h_q: int, h_kv: int = 1,
             parts: int | None = None) -> Metadata:
    """Enqueue the split-KV scheduler for these lengths (no host sync)."""
    _require(seqlens, torch.int32, "seqlens", 1)
    batch = seqlens.shape[0]
    if parts is None:
        parts = num_parts(batch, s_q, h_q, h_kv, device_num_cus(seqlens.device))
    tm = torch.empty((parts, TILE_META_INTS), dtype=torch.int32, device=seqlens.device)
    so = torch.empty((batch + 1,), dtype=torch.int32, device=seqlens.device)
    _check(lib().mla_decode_metadata(_ptr(seqlens), batch, s_q, h_q, h_kv, BLOCK_SIZE, parts,
                                     _ptr(tm), _ptr(so), _stream(seqlens.device)),
           "mla_decode_metadata")
    return Metadata(tm, so, parts, s_q, h_q)


def _alloc_workspace(batch, s_q, h_q, parts, device, workspace):
    need = workspace_bytes(batch, s_q, h_q, parts)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=device)
    return workspace


def _decode_args(q, kcache, block_table, seqlens, fp8: bool = False):
    _require(q, torch.bfloat16, "q", 4)
    if fp8:
        _require(kcache, torch.uint8, "kcache (FP8 pages)", 2)
    else:
        _require(kcache, torch.bfloat16, "kcache", 4)
    _require(block_table, torch.int32, "block_table", 2)
    _require(seqlens, torch.int32, "seqlens", 1)
    batch, s_q, h_q, dk = q.shape
    if fp8:
        if dk != D_K or kcache.shape[1] != FP8_PAGE_BYTES:
            raise ValueError(f"shape mismatch: q {tuple(q.shape)}, FP8 kcache "
                             f"{tuple(kcache.shape)} (pages of {FP8_PAGE_BYTES} bytes)")
        return batch, s_q, h_q, 1
    if dk != D_K or kcache.shape[1] != BLOCK_SIZE or kcache.shape[3] != D_K:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, kcache {tuple(kcache.shape)}")
    h_kv = kcache.shape[2]
    return batch, s_q, h_q, h_kv


def _outputs(q, out, lse):
    batch, s_q, h_q, _ = q.shape
    if out is None:
        out = torch.empty((batch, s_q, h_q, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=q.device)
    _require(out, torch.bfloat16, "out", 4)
    _require(lse, torch.float32, "lse", 3)
    return out, lse


def _check_batch_shapes(q, block_table, seqlens, out=None, lse=None, meta=None,
                        items=None, workspace=None):
    """Host-side shape agreement of everything a launch will index, so that a
    mismatched tensor raises here instead of reaching a kernel (which trusts
    these shapes and would read or write out of bounds).  ``items`` is the
    number of split-plan entries the metadata must cover (batch, or
    batch * s_q in the sparse mode)."""
    batch, s_q, h_q, _ = q.shape
    dev = q.device
    for name, t in (("block_table", block_table), ("seqlens", seqlens), ("out", out),
                    ("lse", lse), ("workspace", workspace)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
    if tuple(seqlens.shape) != (batch,):
        raise ValueError(f"seqlens {tuple(seqlens.shape)} does not match batch {batch}")
    if block_table.shape[0] != batch:
        raise ValueError(f"block_table {tuple(block_table.shape)} does not match batch {batch}")
    if out is not None and tuple(out.shape) != (batch, s_q, h_q, D_V):
        raise ValueError(f"out {tuple(out.shape)} must be {(batch, s_q, h_q, D_V)}")
    if lse is not None and tuple(lse.shape) != (batch, s_q, h_q):
        raise ValueError(f"lse {tuple(lse.shape)} must be {(batch, s_q, h_q)}")
    if meta is not None:
        _check_meta(meta, s_q, h_q, batch if items is None else items, dev)


def _check_meta(meta, s_q, h_q, items, dev):
    if (meta.s_q, meta.h_q) != (s_q, h_q):
        raise ValueError(f"metadata was built for s_q={meta.s_q}, h_q={meta.h_q}, "
                         f"not s_q={s_q}, h_q={h_q}")
    _require(meta.tile_meta, torch.int32, "meta.tile_meta", 2)
    _require(meta.split_offsets, torch.int32, "meta.split_offsets", 1)
    if tuple(meta.tile_meta.shape) != (meta.num_parts, TILE_META_INTS):
        raise ValueError(f"meta.tile_meta {tuple(meta.tile_meta.shape)} must be "
                         f"{(meta.num_parts, TILE_META_INTS)}")
    if meta.split_offsets.numel() != items + 1:
        raise ValueError(f"meta.split_offsets has {meta.split_offsets.numel()} entries, "
                         f"{items + 1} expected")
    if meta.tile_meta.device != dev or meta.split_offsets.device != dev:
        raise ValueError("metadata is on another device")


def _event_handle(ev):
    """Raw hipEvent_t of a torch.cuda.Event (None -> NULL).  torch creates the
    event on its first record, so an unrecorded event is recorded once here."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()
    return ev.cuda_event


def splitkv(q, kcache, block_table, seqlens, scale: float, causal: bool, meta: Metadata,
            workspace: torch.Tensor, out=None, lse=None, start_event=None, stop_event=None):
    """Enqueue only the split-KV decode kernel (partials left in workspace).

    With start_event / stop_event (torch.cuda.Event(enable_timing=True)), the
    events are recorded at the kernel's own start and end
    (mla_decode_splitkv_timed)."""
    batch, s_q, h_q, h_kv = _decode_args(q, kcache, block_table, seqlens)
    out, lse = _outputs(q, out, lse)
    _require_workspace(workspace, q.device)
    _check_batch_shapes(q, block_table, seqlens, out, lse, meta, workspace=workspace)
    args = (_ptr(q), _ptr(kcache), kcache.shape[0], _ptr(block_table), block_table.shape[1],
            _ptr(seqlens), batch, s_q, h_q, h_kv, float(scale), int(bool(causal)),
            _ptr(meta.tile_meta), _ptr(meta.split_offsets), meta.num_parts, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse))
    if start_event is None and stop_event is None:
        _check(lib().mla_decode_splitkv(*args, _stream(q.device)), "mla_decode_splitkv")
    else:
        _check(lib().mla_decode_splitkv_timed(*args, _event_handle(start_event),
                                              _event_handle(stop_event), _stream(q.device)),
               "mla_decode_splitkv_timed")
    return out, lse


def combine(seqlens, s_q: int, h_q: int, meta: Metadata, workspace: torch.Tensor, out, lse):
    """Enqueue only the log-sum-exp merge of the split partials."""
    _require(seqlens, torch.int32, "seqlens", 1)
    batch = seqlens.shape[0]
    _require(out, torch.bfloat16, "out", 4)
    _require(lse, torch.float32, "lse", 3)
    _require_workspace(workspace, seqlens.device)
    if tuple(out.shape) != (batch, s_q, h_q, D_V) or tuple(lse.shape) != (batch, s_q, h_q):
        raise ValueError(f"out {tuple(out.shape)} / lse {tuple(lse.shape)} do not match "
                         f"batch {batch}, s_q {s_q}, h_q {h_q}")
    if out.device != seqlens.device or lse.device != seqlens.device:
        raise ValueError("out / lse are on another device than seqlens")
    _require(meta.split_offsets, torch.int32, "meta.split_offsets", 1)
    if meta.split_offsets.numel() != batch + 1 or meta.split_offsets.device != seqlens.device:
        raise ValueError(f"meta.split_offsets has {meta.split_offsets.numel()} entries, "
                         f"{batch + 1} expected")
    _check(lib().mla_decode_combine(
        _ptr(seqlens), batch, s_q, h_q, _ptr(meta.split_offsets), meta.num_parts,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        _stream(seqlens.device)), "mla_decode_combine")
    return out, lse


def fwd(q, kcache, block_table, seqlens, scale: float, causal: bool | None = None,
        meta: Metadata | None = None, parts: int | None = None, workspace=None,
        out=None, lse=None):
    """Paged MLA decode: returns (O bf16 [B, s_q, h_q, 512], LSE fp32 [B, s_q, h_q])."""
    batch, s_q, h_q, h_kv = _decode_args(q, kcache, block_table, seqlens)
    if causal is None:
        causal = s_q > 1
    _check_batch_shapes(q, block_table, seqlens)
    if meta is None:
        meta = metadata(seqlens, s_q, h_q, h_kv, parts)
    workspace = _alloc_workspace(batch, s_q, h_q, meta.num_parts, q.device, workspace)
    out, lse = _outputs(q, out, lse)
    _check_batch_shapes(q, block_table, seqlens, out, lse, meta, workspace=workspace)
    _check(lib().mla_decode_fwd(
        _ptr(q), _ptr(kcache), kcache.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), batch, s_q, h_q, h_kv, float(scale), int(bool(causal)),
        _ptr(meta.tile_meta), _ptr(meta.split_offsets), meta.num_parts, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(q.device)),
        "mla_decode_fwd")
    return out, lse


def _check_append_shapes(new_kv, kcache, block_table, seqlens):
    batch = new_kv.shape[0]
    if tuple(seqlens.shape) != (batch,) or block_table.shape[0] != batch:
        raise ValueError(f"seqlens {tuple(seqlens.shape)} / block_table "
                         f"{tuple(block_table.shape)} do not match new_kv batch {batch}")
    for name, t in (("kcache", kcache), ("block_table", block_table), ("seqlens", seqlens)):
        if t.device != new_kv.device:
            raise ValueError(f"{name} is on {t.device}, new_kv on {new_kv.device}")


def _require_workspace(ws, dev):
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != dev:
        raise ValueError("workspace must be a device tensor on the inputs' device")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")


def fwd_noalloc(q, kcache, block_table, seqlens, scale: float, causal: bool | None = None,
                out=None, lse=None):
    """The decode through mla_decode_fwd_noalloc: plan and partials in the
    library's own device array (nothing allocated by the call itself; out /
    lse are allocated here only when not given)."""
    batch, s_q, h_q, h_kv = _decode_args(q, kcache, block_table, seqlens)
    if causal is None:
        causal = s_q > 1
    out, lse = _outputs(q, out, lse)
    _check_batch_shapes(q, block_table, seqlens, out, lse)
    _check(lib().mla_decode_fwd_noalloc(
        _ptr(q), _ptr(kcache), kcache.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), batch, s_q, h_q, h_kv, float(scale), int(bool(causal)), _ptr(out),
        _ptr(lse), _stream(q.device)), "mla_decode_fwd_noalloc")
    return out, lse


def kv_append(new_kv: torch.Tensor, kcache: torch.Tensor, block_table: torch.Tensor,
              seqlens: torch.Tensor) -> torch.Tensor:
    """Enqueue the write of new_kv [B, s_q, 576] (bf16) into the paged cache
    (mla_kv_append); the lengths already count the new tokens.  Returns kcache."""
    _require(new_kv, torch.bfloat16, "new_kv", 3)
    _require(kcache, torch.bfloat16, "kcache", 4)
    _require(block_table, torch.int32, "block_table", 2)
    _require(seqlens, torch.int32, "seqlens", 1)
    batch, s_q, dk = new_kv.shape
    if dk != D_K or kcache.shape[1] != BLOCK_SIZE or kcache.shape[3] != D_K:
        raise ValueError(f"shape mismatch: new_kv {tuple(new_kv.shape)}, "
                         f"kcache {tuple(kcache.shape)}")
    _check_append_shapes(new_kv, kcache, block_table, seqlens)
    _check(lib().mla_kv_append(_ptr(new_kv), _ptr(kcache), kcache.shape[0], _ptr(block_table),
                               block_table.shape[1], _ptr(seqlens), batch, s_q,
                               _stream(new_kv.device)), "mla_kv_append")
    return kcache


def splitkv_fp8(q, kcache, block_table, seqlens, scale: float, causal: bool, meta: Metadata,
                workspace: torch.Tensor, out=None, lse=None, start_event=None, stop_event=None):
    """splitkv over an FP8 cache: kcache uint8 [num_blocks, 41216]
    (mla_decode_splitkv_fp8; the events as in splitkv)."""
    batch, s_q, h_q, h_kv = _decode_args(q, kcache, block_table, seqlens, fp8=True)
    out, lse = _outputs(q, out, lse)
    _require_workspace(workspace, q.device)
    _check_batch_shapes(q, block_table, seqlens, out, lse, meta, workspace=workspace)
    _check(lib().mla_decode_splitkv_fp8(
        _ptr(q), _ptr(kcache), kcache.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), batch, s_q, h_q, h_kv, float(scale), int(bool(causal)),
        _ptr(meta.tile_meta), _ptr(meta.split_offsets), meta.num_parts, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        _event_handle(start_event), _event_handle(stop_event), _stream(q.device)),
        "mla_decode_splitkv_fp8")
    return out, lse


def fwd_fp8(q, kcache, block_table, seqlens, scale: float, causal: bool | None = None,
            meta: Metadata | None = None, parts: int | None = None, workspace=None,
            out=None, lse=None):
    """Paged MLA decode over an FP8 cache (kcache uint8 [num_blocks, 41216]):
    returns (O bf16 [B, s_q, h_q, 512], LSE fp32 [B, s_q, h_q])."""
    batch, s_q, h_q, h_kv = _decode_args(q, kcache, block_table, seqlens, fp8=True)
    if causal is None:
        causal = s_q > 1
    _check_batch_shapes(q, block_table, seqlens)
    if meta is None:
        meta = metadata(seqlens, s_q, h_q, h_kv, parts)
    workspace = _alloc_workspace(batch, s_q, h_q, meta.num_parts, q.device, workspace)
    out, lse = _outputs(q, out, lse)
    _check_batch_shapes(q, block_table, seqlens, out, lse, meta, workspace=workspace)
    _check(lib().mla_decode_fwd_fp8(
        _ptr(q), _ptr(kcache), kcache.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), batch, s_q, h_q, h_kv, float(scale), int(bool(causal)),
        _ptr(meta.tile_meta), _ptr(meta.split_offsets), meta.num_parts, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(q.device)),
        "mla_decode_fwd_fp8")
    return out, lse


def fwd_inline_plan(q, kcache, block_table, seqlens, scale: float, causal: bool | None = None,
                    parts: int | None = None, workspace=None, out=None, lse=None,
                    meta: Metadata | None = None, start_event=None, stop_event=None,
                    fp8: bool = False):
    """The decode in two launches: the decode kernel derives the split plan
    itself (mla_decode_fwd_inline_plan[_fp8]).  ``meta`` (optional) receives
    the plan the kernel wrote; returns (O, LSE) like fwd."""
    batch, s_q, h_q, h_kv = _decode_args(q, kcache, block_table, seqlens, fp8=fp8)
    if causal is None:
        causal = s_q > 1
    if meta is None:
        p = parts or num_parts(batch, s_q, h_q, h_kv, device_num_cus(q.device))
        meta = Metadata(torch.empty((p, TILE_META_INTS), dtype=torch.int32, device=q.device),
                        torch.empty((batch + 1,), dtype=torch.int32, device=q.device), p,
                        s_q, h_q)
    workspace = _alloc_workspace(batch, s_q, h_q, meta.num_parts, q.device, workspace)
    out, lse = _outputs(q, out, lse)
    _check_batch_shapes(q, block_table, seqlens, out, lse, meta, workspace=workspace)
    name = "mla_decode_fwd_inline_plan_fp8" if fp8 else "mla_decode_fwd_inline_plan"
    _check(getattr(lib(), name)(
        _ptr(q), _ptr(kcache), kcache.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), batch, s_q, h_q, h_kv, float(scale), int(bool(causal)),
        _ptr(meta.tile_meta), _ptr(meta.split_offsets), meta.num_parts, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        _event_handle(start_event), _event_handle(stop_event), _stream(q.device)), name)
    return out, lse


def kv_append_fp8(new_kv: torch.Tensor, kcache: torch.Tensor, block_table: torch.Tensor,
                  seqlens: torch.Tensor) -> torch.Tensor:
    """Enqueue the quantising write of new_kv [B, s_q, 576] (bf16) into an FP8
    cache, uint8 [num_blocks, 41216] (mla_kv_append_fp8).  Returns kcache."""
    _require(new_kv, torch.bfloat16, "new_kv", 3)
    _require(kcache, torch.uint8, "kcache (FP8 pages)", 2)
    _require(block_table, torch.int32, "block_table", 2)
    _require(seqlens, torch.int32, "seqlens", 1)
    batch, s_q, dk = new_kv.shape
    if dk != D_K or kcache.shape[1] != FP8_PAGE_BYTES:
        raise ValueError(f"shape mismatch: new_kv {tuple(new_kv.shape)}, "
                         f"FP8 kcache {tuple(kcache.shape)}")
    _check_append_shapes(new_kv, kcache, block_table, seqlens)
    _check(lib().mla_kv_append_fp8(_ptr(new_kv), _ptr(kcache), kcache.shape[0],
                                   _ptr(block_table), block_table.shape[1], _ptr(seqlens),
                                   batch, s_q, _stream(new_kv.device)), "mla_kv_append_fp8")
    return kcache


def sparse_workspace_bytes(batch: int, s_q: int, h_q: int, topk: int, parts: int) -> int:
    out = _c_size(0)
    _check(lib().mla_decode_sparse_workspace_bytes(batch, s_q, h_q, topk, parts,
                                                   ctypes.byref(out)),
           "mla_decode_sparse_workspace_bytes")
    return out.value


def sparse_metadata(batch: int, s_q: int, h_q: int, topk: int, device,
                    parts: int | None = None) -> Metadata:
    """Enqueue the split plan of the sparse mode: batch*s_q items of topk
    entries each (mla_decode_sparse_metadata)."""
    device = torch.device(device)
    if parts is None:
        parts = num_parts(batch * s_q, 1, h_q, 1, device_num_cus(device))
    tm = torch.empty((parts, TILE_META_INTS), dtype=torch.int32, device=device)
    so = torch.empty((batch * s_q + 1,), dtype=torch.int32, device=device)
    _check(lib().mla_decode_sparse_metadata(batch, s_q, h_q, topk, parts, _ptr(tm), _ptr(so),
                                            _stream(device)), "mla_decode_sparse_metadata")
    return Metadata(tm, so, parts, s_q, h_q)


def sparse_fwd(q, kcache, block_table, seqlens, indices, scale: float,
               causal: bool | None = None, meta: Metadata | None = None,
               parts: int | None = None, workspace=None, out=None, lse=None,
               start_event=None, stop_event=None):
    """Sparse-mode decode over a bf16 cache: every head of query token t of
    request b attends over the cache positions indices[b, t, :] (int32
    [B, s_q, topk], -1 = padding) that are visible.  Returns (O, LSE) like fwd."""
    return _sparse_fwd(q, kcache, block_table, seqlens, indices, scale, causal, meta, parts,
                       workspace, out, lse, start_event, stop_event, fp8=False)


def sparse_fwd_fp8(q, kcache, block_table, seqlens, indices, scale: float,
                   causal: bool | None = None, meta: Metadata | None = None,
                   parts: int | None = None, workspace=None, out=None, lse=None,
                   start_event=None, stop_event=None):
    """sparse_fwd over an FP8 cache, kcache uint8 [num_blocks, 41216]
    (mla_decode_sparse_fwd_fp8)."""
    return _sparse_fwd(q, kcache, block_table, seqlens, indices, scale, causal, meta, parts,
                       workspace, out, lse, start_event, stop_event, fp8=True)


def _sparse_fwd(q, kcache, block_table, seqlens, indices, scale, causal, meta, parts,
                workspace, out, lse, start_event, stop_event, fp8: bool):
    batch, s_q, h_q, h_kv = _decode_args(q, kcache, block_table, seqlens, fp8=fp8)
    _require(indices, torch.int32, "indices", 3)
    if tuple(indices.shape[:2]) != (batch, s_q):
        raise ValueError(f"indices {tuple(indices.shape)} do not match q {tuple(q.shape)}")
    topk = indices.shape[2]
    if indices.device != q.device:
        raise ValueError(f"indices is on {indices.device}, q on {q.device}")
    _check_batch_shapes(q, block_table, seqlens)
    if causal is None:
        causal = s_q > 1
    if meta is None:
        meta = sparse_metadata(batch, s_q, h_q, topk, q.device, parts)
    need = sparse_workspace_bytes(batch, s_q, h_q, topk, meta.num_parts)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    out, lse = _outputs(q, out, lse)
    _require_workspace(workspace, q.device)
    _check_batch_shapes(q, block_table, seqlens, out, lse, meta, items=batch * s_q,
                        workspace=workspace)
    name = "mla_decode_sparse_fwd_fp8" if fp8 else "mla_decode_sparse_fwd"
    _check(getattr(lib(), name)(
        _ptr(q), _ptr(kcache), kcache.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), batch, s_q, h_q, h_kv, float(scale), int(bool(causal)), _ptr(indices),
        topk, _ptr(meta.tile_meta), _ptr(meta.split_offsets), meta.num_parts, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        _event_handle(start_event), _event_handle(stop_event), _stream(q.device)), name)
    return out, lse
