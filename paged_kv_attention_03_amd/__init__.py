"""Paged-KV attention for one continuous-batching step on MI355X.

Thin ctypes binding over ``libpkv.so`` (C ABI in ``include/pkv.h``).  The
functions carry the C names; this layer only checks tensors and marshals
pointers, sizes and the current HIP stream.  Every step of the computation runs
in the library's HIP kernels: there is no fallback, and a missing library
raises at the first call.

    pkv_append(k_new, v_new, k_pool, v_pool, slot_mapping)
    out = pkv_attention(q, k_pool, v_pool, block_tables, seq_lens,
                        query_start_loc, scale, max_seqlen_q=..., max_seqlen_k=...)
    out = pkv_attention_shared_prefix(q, k_pool, v_pool, block_tables, seq_lens,
                                      query_start_loc, scale, prefix_group, prefix_len,
                                      max_group_size=..., max_prefix_len=..., ...)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PKV_F32", "PKV_BF16", "PkvError", "pkv_append", "pkv_attention",
    "pkv_attention_workspace_size", "pkv_attention_noalloc", "pkv_attention_shared_prefix",
    "pkv_attention_shared_prefix_workspace_size", "pkv_check_shared_prefix",
    "pkv_check_metadata", "pkv_check_slots", "pkv_last_error",
    "pkv_copy_blocks", "PagePool", "library_path", "load_library", "PreparedCall",
    "prepare_append", "prepare_attention",
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
PKV_E_NOMEM = -6
PKV_PREFIX_PASS_AUTO = 0
PKV_PREFIX_PASS_ALWAYS = 1
_PREFIX_PASS = {"auto": PKV_PREFIX_PASS_AUTO, "always": PKV_PREFIX_PASS_ALWAYS}

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
    lib.pkv_attention_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                          i32, i32, i32, i32, i64, ctypes.c_float, i32, vp]
    lib.pkv_attention_noalloc.restype = i32
    lib.pkv_attention_shared_prefix_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32,
                                                               i32, i32, i32, i32, i32]
    lib.pkv_attention_shared_prefix_workspace_size.restype = sz
    lib.pkv_attention_shared_prefix.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                                i32, i64, i32, i32, i32, i32, i32, i32, i32,
                                                i64, ctypes.c_float, i32, i32, vp, sz, vp]
    lib.pkv_attention_shared_prefix.restype = i32
    lib.pkv_check_shared_prefix.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32]
    lib.pkv_check_shared_prefix.restype = i32
    lib.pkv_check_metadata.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i64]
    lib.pkv_check_metadata.restype = i32
    lib.pkv_check_slots.argtypes = [vp, i64, i32, i64]
    lib.pkv_check_slots.restype = i32
    lib.pkv_last_error.argtypes = []
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_pool_create.argtypes = [i64, i32, i32, i32]
    lib.pkv_pool_create.restype = vp
    lib.pkv_pool_destroy.argtypes = [vp]
    lib.pkv_pool_destroy.restype = None
    lib.pkv_pool_free_blocks.argtypes = [vp]
    lib.pkv_pool_free_blocks.restype = i64
    lib.pkv_pool_set_free_order.argtypes = [vp, vp, i64]
    lib.pkv_pool_set_free_order.restype = i32
    lib.pkv_pool_can_admit.argtypes = [vp, i64]
    lib.pkv_pool_can_admit.restype = i32
    lib.pkv_pool_add_seq.argtypes = [vp, i32]
    lib.pkv_pool_add_seq.restype = i32
    lib.pkv_pool_fork.argtypes = [vp, i32, i32, i64]
    lib.pkv_pool_fork.restype = i32
    lib.pkv_pool_append.argtypes = [vp, i32, i64, vp, vp, vp, vp]
    lib.pkv_pool_append.restype = i32
    lib.pkv_pool_append_batch.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp]
    lib.pkv_pool_append_batch.restype = i32
    lib.pkv_pool_truncate.argtypes = [vp, i32, i64]
    lib.pkv_pool_truncate.restype = i32
    lib.pkv_pool_free_seq.argtypes = [vp, i32]
    lib.pkv_pool_free_seq.restype = i32
    lib.pkv_pool_seq_len.argtypes = [vp, i32]
    lib.pkv_pool_seq_len.restype = i64
    lib.pkv_pool_block_tables.argtypes = [vp, vp, i32, vp, i32, vp]
    lib.pkv_pool_block_tables.restype = i32
    lib.pkv_copy_blocks.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i64, i32, vp]
    lib.pkv_copy_blocks.restype = i32
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


class PreparedCall:
    """One library call whose arguments were checked and converted once.
    Calling the object issues the same C call again: the same device
    pointers, sizes and stream, so the tensors it was prepared with must stay
    alive and keep their storage (the object holds references to them); their
    contents may change between calls.  The host-side metadata checks that
    ``PKV_CHECK=1`` turns on for the plain calls do not run here."""

    __slots__ = ("_fn", "_args", "_keep", "out")

    def __init__(self, fn, args, keep, out=None):
        self._fn = fn
        self._args = tuple(a if a is None else t(a) for t, a in zip(fn.argtypes, args))
        self._keep = keep
        self.out = out

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != PKV_OK:
            raise PkvError(rc, pkv_last_error())


def _append_args(k_new, v_new, k_pool, v_pool, slot_mapping, stream):
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
    return args + (t, hkv, d, bs, nb, dt, _stream(k_pool.device, stream))


def pkv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
               v_pool: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Write new K/V rows [T, Hkv, D] into pools [num_blocks, Hkv, bs, D] at
    ``slot_mapping`` [T] (int64; negative = skip)."""
    lib = load_library()
    args = _append_args(k_new, v_new, k_pool, v_pool, slot_mapping, stream)
    if os.environ.get("PKV_CHECK") == "1":
        pkv_check_slots(slot_mapping, k_pool.shape[2], k_pool.shape[0])
    _raise(lib.pkv_append(*args))


def prepare_append(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
                   v_pool: torch.Tensor, slot_mapping: torch.Tensor,
                   stream=None) -> PreparedCall:
    """``pkv_append`` on these tensors, checked once; each call of the result
    re-issues it (on ``stream``, else the current stream at preparation)."""
    lib = load_library()
    return PreparedCall(lib.pkv_append,
                        _append_args(k_new, v_new, k_pool, v_pool, slot_mapping, stream),
                        (k_new, v_new, k_pool, v_pool, slot_mapping))


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
    args, out, workspace = _attention_args(q, k_pool, v_pool, block_tables, seq_lens,
                                           query_start_loc, scale, max_seqlen_q, max_seqlen_k,
                                           kv_start, out, workspace, stream)
    if os.environ.get("PKV_CHECK") == "1":
        pkv_check_metadata(block_tables, seq_lens, query_start_loc, kv_start, q.shape[0],
                           k_pool.shape[2], k_pool.shape[0], max_seqlen_q=max_seqlen_q,
                           max_seqlen_k=max_seqlen_k)
    _raise(lib.pkv_attention(*args))
    return out


def _attention_args(q, k_pool, v_pool, block_tables, seq_lens, query_start_loc, scale,
                    max_seqlen_q, max_seqlen_k, kv_start, out, workspace, stream):
    """Checks the tensors of an attention call and returns (C arguments, out,
    workspace), allocating ``out`` and the workspace when not given."""
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
    args = ptrs + (ns, total_q, max_blocks, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, bs,
                   nb, float(scale), dt, ws_ptr, ws_bytes, _stream(q.device, stream))
    return args, out, workspace


def prepare_attention(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      block_tables: torch.Tensor, seq_lens: torch.Tensor,
                      query_start_loc: torch.Tensor, scale: float, *, max_seqlen_q: int,
                      max_seqlen_k: int, kv_start: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> PreparedCall:
    """``pkv_attention`` on these tensors, checked once (``out`` and the
    workspace are allocated here when not given; ``.out`` of the result is
    the output tensor); each call of the result re-issues it with the current
    contents of the metadata tensors, which must stay within the same host
    bounds (``max_seqlen_q``, ``max_seqlen_k``)."""
    lib = load_library()
    args, out, workspace = _attention_args(q, k_pool, v_pool, block_tables, seq_lens,
                                           query_start_loc, scale, max_seqlen_q, max_seqlen_k,
                                           kv_start, out, workspace, stream)
    return PreparedCall(lib.pkv_attention, args, (q, k_pool, v_pool, block_tables, seq_lens,
                                                  query_start_loc, kv_start, out, workspace),
                        out=out)


def pkv_attention_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                          block_tables: torch.Tensor, seq_lens: torch.Tensor,
                          query_start_loc: torch.Tensor, scale: float, *, max_seqlen_q: int,
                          max_seqlen_k: int, out: torch.Tensor,
                          kv_start: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pkv_attention whose workspace is the library's static device scratch
    (``PKV_NOALLOC_SCRATCH_BYTES``): neither the call nor this binding
    allocates; ``out`` is the caller's.  Calls that may overlap on one GPU
    share the scratch and race."""
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
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    ptrs = (_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool", q.dtype),
            _dev(v_pool, "v_pool", q.dtype), _dev(block_tables, "block_tables", torch.int32),
            _dev(seq_lens, "seq_lens", torch.int32),
            _dev(query_start_loc, "query_start_loc", torch.int32),
            None if kv_start is None else _dev(kv_start, "kv_start", torch.int32))
    if os.environ.get("PKV_CHECK") == "1":
        pkv_check_metadata(block_tables, seq_lens, query_start_loc, kv_start, total_q, bs, nb,
                           max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k)
    _raise(lib.pkv_attention_noalloc(*ptrs, ns, total_q, max_blocks, int(max_seqlen_q),
                                     int(max_seqlen_k), hq, hkv, d, bs, nb, float(scale), dt,
                                     _stream(q.device, stream)))
    return out


def pkv_attention_shared_prefix_workspace_size(num_seqs: int, total_q: int, max_seqlen_q: int,
                                               max_seqlen_k: int, num_q_heads: int,
                                               num_kv_heads: int, head_dim: int,
                                               block_size: int = 16,
                                               dtype: torch.dtype = torch.bfloat16, *,
                                               num_groups: int, max_group_size: int,
                                               max_prefix_len: int) -> int:
    return int(load_library().pkv_attention_shared_prefix_workspace_size(
        num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_q_heads, num_kv_heads, head_dim,
        block_size, _dtype_code(dtype), num_groups, max_group_size, max_prefix_len))


def pkv_attention_shared_prefix(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                block_tables: torch.Tensor, seq_lens: torch.Tensor,
                                query_start_loc: torch.Tensor, scale: float,
                                prefix_group: torch.Tensor, prefix_len: torch.Tensor, *,
                                max_group_size: int, max_prefix_len: int, max_seqlen_q: int,
                                max_seqlen_k: int, out: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None,
                                prefix_pass: str = "auto", stream=None) -> torch.Tensor:
    """pkv_attention for a step whose decode sequences share prefixes in groups:
    prefix_group [S] int32 (group or -1), prefix_len [num_groups] int32 (shared
    keys, multiples of the page size).  Same result as pkv_attention; with the
    prefix pass each group's shared pages are read once per kv head.
    ``prefix_pass``: "auto" (the library runs the pass only when the re-reads it
    avoids are large) or "always"."""
    lib = load_library()
    if prefix_pass not in _PREFIX_PASS:
        raise ValueError(f"prefix_pass must be one of {sorted(_PREFIX_PASS)}")
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
    if prefix_group.shape != (ns,) or prefix_len.dim() != 1:
        raise ValueError("prefix_group must be [num_seqs] and prefix_len [num_groups]")
    ng = prefix_len.shape[0]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = pkv_attention_shared_prefix_workspace_size(
        ns, total_q, max_seqlen_q, max_seqlen_k, hq, hkv, d, bs, q.dtype, num_groups=ng,
        max_group_size=max_group_size, max_prefix_len=max_prefix_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = 0 if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ptrs = (_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool", q.dtype),
            _dev(v_pool, "v_pool", q.dtype), _dev(block_tables, "block_tables", torch.int32),
            _dev(seq_lens, "seq_lens", torch.int32),
            _dev(query_start_loc, "query_start_loc", torch.int32),
            _dev(prefix_group, "prefix_group", torch.int32),
            _dev(prefix_len, "prefix_len", torch.int32))
    if os.environ.get("PKV_CHECK") == "1":
        pkv_check_metadata(block_tables, seq_lens, query_start_loc, None, total_q, bs, nb,
                           max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k)
        pkv_check_shared_prefix(block_tables, seq_lens, query_start_loc, prefix_group,
                                prefix_len, bs, max_prefix_len)
    _raise(lib.pkv_attention_shared_prefix(
        *ptrs, ng, int(max_group_size), int(max_prefix_len), ns, total_q, max_blocks,
        int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, bs, nb, float(scale), dt,
        _PREFIX_PASS[prefix_pass], ws_ptr, ws_bytes, _stream(q.device, stream)))
    return out


def pkv_check_shared_prefix(block_tables, seq_lens, query_start_loc, prefix_group, prefix_len,
                            block_size: int, max_prefix_len: int) -> None:
    """Validate host copies of a shared-prefix step's groups; raises PkvError."""
    bt = _host_i32(block_tables)
    sl = _host_i32(seq_lens)
    qsl = _host_i32(query_start_loc)
    pg = _host_i32(prefix_group)
    pl = _host_i32(prefix_len)
    ns = sl.shape[0]
    if bt.ndim != 2 or bt.shape[0] != ns or qsl.shape != (ns + 1,) or pg.shape != (ns,):
        raise ValueError("metadata shapes disagree")
    _raise(load_library().pkv_check_shared_prefix(
        bt.ctypes.data, sl.ctypes.data, qsl.ctypes.data, pg.ctypes.data, pl.ctypes.data, ns,
        pl.shape[0], bt.shape[1], block_size, max_prefix_len))


def _host_i32(x):
    import numpy as np
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def pkv_check_metadata(block_tables, seq_lens, query_start_loc, kv_start, total_q: int,
                       block_size: int, num_blocks: int, *, max_seqlen_q: Optional[int] = None,
                       max_seqlen_k: Optional[int] = None) -> None:
    """Validate host copies of the step metadata against the host bounds that
    pkv_attention will receive (``None``: the step's own maxima, i.e. only the
    other rules are checked); raises PkvError."""
    import numpy as np
    bt = _host_i32(block_tables)
    sl = _host_i32(seq_lens)
    qsl = _host_i32(query_start_loc)
    ks = None if kv_start is None else _host_i32(kv_start)
    ns = sl.shape[0]
    if bt.ndim != 2 or bt.shape[0] != ns or qsl.shape != (ns + 1,):
        raise ValueError("metadata shapes disagree")
    if max_seqlen_q is None:
        max_seqlen_q = int(np.max(np.diff(qsl), initial=0)) if ns else 0
    if max_seqlen_k is None:
        max_seqlen_k = int(np.max(sl, initial=0)) if ns else 0
    _raise(load_library().pkv_check_metadata(bt.ctypes.data, sl.ctypes.data, qsl.ctypes.data,
                                             None if ks is None else ks.ctypes.data, ns,
                                             int(total_q), bt.shape[1], max(int(max_seqlen_q), 0),
                                             max(int(max_seqlen_k), 0), block_size, num_blocks))


def pkv_check_slots(slot_mapping, block_size: int, num_blocks: int) -> None:
    """Validate a host copy of a slot mapping; raises PkvError."""
    import numpy as np
    if isinstance(slot_mapping, torch.Tensor):
        slot_mapping = slot_mapping.detach().cpu().numpy()
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    _raise(load_library().pkv_check_slots(sm.ctypes.data, sm.shape[0], block_size, num_blocks))


def pkv_copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, src: torch.Tensor,
                    dst: torch.Tensor, stream=None) -> None:
    """Copy whole pages src[i] -> dst[i] (K and V) inside pools
    [num_blocks, Hkv, bs, D]; src/dst are device int32 [n]."""
    lib = load_library()
    dt = _dtype_code(k_pool.dtype)
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("pools must be [num_blocks, Hkv, block_size, D] and equal")
    nb, hkv, bs, d = k_pool.shape
    if src.dim() != 1 or dst.shape != src.shape:
        raise ValueError("src and dst must be [n]")
    n = src.shape[0]
    _raise(lib.pkv_copy_blocks(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
                               _dev(src, "src", torch.int32), _dev(dst, "dst", torch.int32),
                               n, hkv, d, bs, nb, dt, _stream(k_pool.device, stream)))


class PagePool:
    """Host-side manager of a KV pool of ``num_blocks`` pages reserved once
    (the ``pkv_pool_*`` C calls): slots for new rows, block tables, shared
    prefixes by reference count with copy-on-write, admission against the
    free pages.  Host arrays only; device page copies are the caller's
    (``pkv_copy_blocks``)."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int,
                 max_blocks_per_seq: int):
        self._lib = load_library()
        h = self._lib.pkv_pool_create(num_blocks, block_size, max_seqs, max_blocks_per_seq)
        if not h:
            raise PkvError(PKV_E_ARG, pkv_last_error())
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pkv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def free_blocks(self) -> int:
        return int(self._lib.pkv_pool_free_blocks(self._h))

    def set_free_order(self, order) -> None:
        """Hand out the free pages in this order (a permutation of them)."""
        import numpy as np
        o = np.ascontiguousarray(np.asarray(order, dtype=np.int32))
        _raise(self._lib.pkv_pool_set_free_order(self._h, o.ctypes.data, o.shape[0]))

    def can_admit(self, num_tokens: int) -> bool:
        return self._lib.pkv_pool_can_admit(self._h, num_tokens) == 1

    def add_seq(self, seq: int) -> None:
        _raise(self._lib.pkv_pool_add_seq(self._h, seq))

    def fork(self, parent: int, child: int, shared_tokens: int) -> None:
        _raise(self._lib.pkv_pool_fork(self._h, parent, child, shared_tokens))

    def append(self, seq: int, num_tokens: int):
        """Reserve num_tokens slots; returns (slots int64 [n], copies) where
        copies is a list of (src_page, dst_page) to copy before appending."""
        import numpy as np
        slots = np.empty(max(num_tokens, 1), dtype=np.int64)
        cs = np.zeros(1, dtype=np.int32)
        cd = np.zeros(1, dtype=np.int32)
        nc = ctypes.c_int(0)
        _raise(self._lib.pkv_pool_append(self._h, seq, num_tokens, slots.ctypes.data,
                                         cs.ctypes.data, cd.ctypes.data, ctypes.byref(nc)))
        return slots[:num_tokens], [(int(cs[0]), int(cd[0]))] if nc.value else []

    def append_batch(self, seqs, counts):
        """append() for distinct sequences in one call; returns (slots int64
        [sum(counts)] in the order given, copies [(src, dst)])."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        cnt = np.ascontiguousarray(np.asarray(counts, dtype=np.int64))
        slots = np.empty(max(int(cnt.sum()), 1), dtype=np.int64)
        cs = np.zeros(max(len(ids), 1), dtype=np.int32)
        cd = np.zeros(max(len(ids), 1), dtype=np.int32)
        nc = ctypes.c_int(0)
        _raise(self._lib.pkv_pool_append_batch(self._h, ids.ctypes.data, cnt.ctypes.data,
                                               len(ids), slots.ctypes.data, cs.ctypes.data,
                                               cd.ctypes.data, ctypes.byref(nc)))
        return slots[:int(cnt.sum())], [(int(cs[i]), int(cd[i])) for i in range(nc.value)]

    def truncate(self, seq: int, new_len: int) -> None:
        _raise(self._lib.pkv_pool_truncate(self._h, seq, new_len))

    def free_seq(self, seq: int) -> None:
        _raise(self._lib.pkv_pool_free_seq(self._h, seq))

    def seq_len(self, seq: int) -> int:
        return int(self._lib.pkv_pool_seq_len(self._h, seq))

    def block_tables(self, seqs, width: int):
        """(table int32 [len(seqs), width] with -1 padding, seq_lens int32)."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        table = np.empty((len(ids), width), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        _raise(self._lib.pkv_pool_block_tables(self._h, ids.ctypes.data, len(ids),
                                               table.ctypes.data, width, lens.ctypes.data))
        return table, lens
