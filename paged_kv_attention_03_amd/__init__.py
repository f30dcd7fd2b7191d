"""Paged-KV attention for one continuous-batching step on MI355X.

Thin ctypes binding over ``libpkv.so`` (C ABI in ``include/pkv.h``).  The
functions carry the C names; this layer only checks tensors and marshals
pointers, sizes and the current HIP stream.  Every step of the computation runs
in the library's HIP kernels: there is no fallback, and a missing library
raises at the first call.

    pkv_append(k_new, v_new, k_pool, v_pool, slot_mapping)
    out = pkv_attention(q, k_pool, v_pool, block_tables, seq_lens,
                        query_start_loc, scale, max_seqlen_q=..., max_seqlen_k=...)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PKV_F32", "PKV_BF16", "PkvError", "pkv_append", "pkv_attention",
    "pkv_attention_workspace_size", "pkv_check_metadata", "pkv_check_slots", "pkv_last_error",
    "library_path", "load_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_F32 = 0
PKV_BF16 = 1
PKV_OK = 0
PKV_E_ARG = -1
PKV_E_UNSUPPORTED = -2
PKV_E_WORKSPACE = -3
PKV_E_HIP = -4
PKV_E_METADATA = -5

_lib = None


class PkvError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"pkv error {code}: {message}")
        self.code = code
        self.message = message


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libpkv.so and bind the C signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m paged_kv_attention_03_amd.build` "
            "or __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.pkv_append.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, i32, vp]
    lib.pkv_append.restype = i32
    lib.pkv_attention_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32, i32]
    lib.pkv_attention_workspace_size.restype = sz
    lib.pkv_attention.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                  i32, i32, i32, i64, ctypes.c_float, i32, vp, sz, vp]
    lib.pkv_attention.restype = i32
    lib.pkv_check_metadata.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, i64]
    lib.pkv_check_metadata.restype = i32
    lib.pkv_check_slots.argtypes = [vp, i64, i32, i64]
    lib.pkv_check_slots.restype = i32
    lib.pkv_last_error.argtypes = []
    lib.pkv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def pkv_last_error() -> str:
    return load_library().pkv_last_error().decode()


def _raise(rc: int):
    if rc != PKV_OK:
        raise PkvError(rc, pkv_last_error())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return PKV_BF16
    if dt == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {dt} (bfloat16 or float32)")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(getattr(stream, "cuda_stream", stream))


def pkv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
               v_pool: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Write new K/V rows [T, Hkv, D] into pools [num_blocks, Hkv, bs, D] at
    ``slot_mapping`` [T] (int64; negative = skip)."""
    lib = load_library()
    dt = _dtype_code(k_pool.dtype)
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("pools must be [num_blocks, Hkv, block_size, D] and equal")
    nb, hkv, bs, d = k_pool.shape
    if k_new.dim() != 3 or k_new.shape[1:] != (hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [T, Hkv, D] matching the pool")
    t = k_new.shape[0]
    if slot_mapping.shape != (t,):
        raise ValueError("slot_mapping must be [T]")
    args = (_dev(k_new, "k_new", k_pool.dtype), _dev(v_new, "v_new", k_pool.dtype),
            _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
            _dev(slot_mapping, "slot_mapping", torch.int64))
    if os.environ.get("PKV_CHECK") == "1":
        pkv_check_slots(slot_mapping, bs, nb)
    _raise(lib.pkv_append(*args, t, hkv, d, bs, nb, dt, _stream(k_pool.device, stream)))


def pkv_attention_workspace_size(num_seqs: int, total_q: int, max_seqlen_q: int,
                                 max_seqlen_k: int, num_q_heads: int, num_kv_heads: int,
                                 head_dim: int, block_size: int = 16,
                                 dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load_library().pkv_attention_workspace_size(
        num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_q_heads, num_kv_heads, head_dim,
        block_size, _dtype_code(dtype)))


def pkv_attention(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                  block_tables: torch.Tensor, seq_lens: torch.Tensor,
                  query_start_loc: torch.Tensor, scale: float, *, max_seqlen_q: int,
                  max_seqlen_k: int, kv_start: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Attention for one packed step.  q [total_q, Hq, D]; pools
    [num_blocks, Hkv, bs, D]; block_tables [S, max_blocks] int32; seq_lens [S]
    int32 (keys incl. this step's tokens); query_start_loc [S+1] int32;
    kv_start [S] int32 or None.  ``max_seqlen_q``/``max_seqlen_k`` are host
    upper bounds.  Returns ``out`` [total_q, Hq, D] (allocated if None)."""
    lib = load_library()
    dt = _dtype_code(q.dtype)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("q must be [total_q, Hq, D] and pools [num_blocks, Hkv, bs, D]")
    total_q, hq, d = q.shape
    nb, hkv, bs, d2 = k_pool.shape
    if d2 != d:
        raise ValueError("head_dim of q and pools differ")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    ns, max_blocks = block_tables.shape
    if seq_lens.shape != (ns,) or query_start_loc.shape != (ns + 1,):
        raise ValueError("seq_lens must be [num_seqs] and query_start_loc [num_seqs + 1]")
    if kv_start is not None and kv_start.shape != (ns,):
        raise ValueError("kv_start must be [num_seqs]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = pkv_attention_workspace_size(ns, total_q, max_seqlen_q, max_seqlen_k, hq, hkv, d, bs,
                                        q.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = 0 if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ptrs = (_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool", q.dtype),
            _dev(v_pool, "v_pool", q.dtype), _dev(block_tables, "block_tables", torch.int32),
            _dev(seq_lens, "seq_lens", torch.int32),
            _dev(query_start_loc, "query_start_loc", torch.int32),
            None if kv_start is None else _dev(kv_start, "kv_start", torch.int32))
    if os.environ.get("PKV_CHECK") == "1":
        pkv_check_metadata(block_tables, seq_lens, query_start_loc, kv_start, total_q, bs, nb)
    _raise(lib.pkv_attention(*ptrs, ns, total_q, max_blocks, int(max_seqlen_q), int(max_seqlen_k),
                             hq, hkv, d, bs, nb, float(scale), dt, ws_ptr, ws_bytes,
                             _stream(q.device, stream)))
    return out


def _host_i32(x):
    import numpy as np
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def pkv_check_metadata(block_tables, seq_lens, query_start_loc, kv_start, total_q: int,
                       block_size: int, num_blocks: int) -> None:
    """Validate host copies of the step metadata; raises PkvError."""
    bt = _host_i32(block_tables)
    sl = _host_i32(seq_lens)
    qsl = _host_i32(query_start_loc)
    ks = None if kv_start is None else _host_i32(kv_start)
    ns = sl.shape[0]
    if bt.ndim != 2 or bt.shape[0] != ns or qsl.shape != (ns + 1,):
        raise ValueError("metadata shapes disagree")
    _raise(load_library().pkv_check_metadata(bt.ctypes.data, sl.ctypes.data, qsl.ctypes.data,
                                             None if ks is None else ks.ctypes.data, ns,
                                             int(total_q), bt.shape[1], block_size, num_blocks))


def pkv_check_slots(slot_mapping, block_size: int, num_blocks: int) -> None:
    """Validate a host copy of a slot mapping; raises PkvError."""
    import numpy as np
    if isinstance(slot_mapping, torch.Tensor):
        slot_mapping = slot_mapping.detach().cpu().numpy()
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    _raise(load_library().pkv_check_slots(sm.ctypes.data, sm.shape[0], block_size, num_blocks))
