"""Float64 CPU oracle for paged-KV attention and the slot-mapped KV append.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
it shares no code with them.

The arithmetic lives in ``pkv_oracle.c`` (plain C, float64, OpenMP over
(sequence, kv head) units).  This module only marshals arrays through ctypes.
What the functions compute, with the passages they follow, is written at the
top of ``pkv_oracle.c``.

Inputs may be torch CPU tensors or numpy arrays.  bfloat16 data is passed as
its raw 16-bit patterns; float32 as float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc -O2 (OpenMP, no fast-math) of one oracle source into a shared object."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, src, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle library next to its source."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """ctypes handle with the oracle's signatures bound (used for the built
    oracle, and by tests for copies of the source with a planted mistake)."""
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_append.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, i32]
    lib.oracle_append.restype = i32
    lib.oracle_attention.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                     i32, i64, ctypes.c_double, i32, i32]
    lib.oracle_attention.restype = i32
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = load_library(_LIB_PATH)
    return _lib


def _as_raw(x):
    """Return (contiguous numpy array holding the raw element bits, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                raise ValueError("oracle inputs must be host tensors")
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                return np.ascontiguousarray(x.view(torch.int16).numpy()), BF16
            if x.dtype == torch.float32:
                return np.ascontiguousarray(x.numpy()), F32
            raise TypeError(f"unsupported dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype in (np.int16, np.uint16):
        return x, BF16
    raise TypeError(f"unsupported dtype {x.dtype}")


def _i32(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _i64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def oracle_append(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Return copies of the pools with each new row written to its slot.

    Pools are [num_blocks, Hkv, bs, D]; new rows [T, Hkv, D]; slot < 0 skips.
    The result is returned in the same raw representation as the inputs
    (numpy; bfloat16 as int16 bit patterns).
    """
    kp, dt = _as_raw(k_pool)
    vp, dt2 = _as_raw(v_pool)
    kn, dt3 = _as_raw(k_new)
    vn, dt4 = _as_raw(v_new)
    if len({dt, dt2, dt3, dt4}) != 1:
        raise TypeError("pool and new rows must share one dtype")
    kp = kp.copy()
    vp = vp.copy()
    nb, hkv, bs, d = kp.shape
    slots = _i64(slot_mapping)
    t = kn.shape[0]
    if kn.shape != (t, hkv, d) or vn.shape != (t, hkv, d) or slots.shape != (t,):
        raise ValueError("shape mismatch")
    rc = _load().oracle_append(kp.ctypes.data, vp.ctypes.data, kn.ctypes.data, vn.ctypes.data,
                               slots.ctypes.data, t, hkv, d, bs, nb, dt)
    if rc != 0:
        raise ValueError(f"oracle_append failed ({rc})")
    return kp, vp


def oracle_attention(q, k_pool, v_pool, block_tables, seq_lens, query_start_loc, scale,
                     kv_start=None, threads: int = 0, lib=None):
    """Float64 softmax attention of each query over its visible keys.

    q [total_q, Hq, D]; pools [num_blocks, Hkv, bs, D]; block_tables
    [num_seqs, max_blocks]; seq_lens [num_seqs] (keys including this step's
    tokens); query_start_loc [num_seqs + 1]; kv_start [num_seqs] or None.
    ``scale`` is used as the double value of the given float (pass the same
    float32 value the device path receives).  Returns float64 [total_q, Hq, D].
    """
    qr, dt = _as_raw(q)
    kp, dt2 = _as_raw(k_pool)
    vp, dt3 = _as_raw(v_pool)
    if len({dt, dt2, dt3}) != 1:
        raise TypeError("q and pools must share one dtype")
    total_q, hq, d = qr.shape
    nb, hkv, bs, d2 = kp.shape
    if d2 != d or vp.shape != kp.shape:
        raise ValueError("shape mismatch")
    bt = _i32(block_tables)
    sl = _i32(seq_lens)
    qsl = _i32(query_start_loc)
    ns = sl.shape[0]
    if bt.ndim != 2 or bt.shape[0] != ns or qsl.shape != (ns + 1,):
        raise ValueError("metadata shape mismatch")
    if ns > 0 and int(qsl[-1]) != total_q:
        raise ValueError("query_start_loc[-1] != total_q")
    ks = None
    if kv_start is not None:
        ks = _i32(kv_start)
        if ks.shape != (ns,):
            raise ValueError("kv_start shape mismatch")
    out = np.zeros((total_q, hq, d), dtype=np.float64)
    rc = (lib or _load()).oracle_attention(out.ctypes.data, qr.ctypes.data, kp.ctypes.data, vp.ctypes.data,
                                  bt.ctypes.data, sl.ctypes.data, qsl.ctypes.data,
                                  None if ks is None else ks.ctypes.data, ns, bt.shape[1], hq,
                                  hkv, d, bs, nb, float(np.float32(scale)), dt, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attention rejected the metadata ({rc})")
    return out
