"""Helpers for the GPU parity tests: run a generated step through the C ABI
(via the Python binding) and compare with the float64 oracle.  Test code."""
import math

import os

import numpy as np
import torch

import oracle
import paged_kv_attention_03_amd as pkv
from tests.helpers import close

# elementwise |gpu - oracle| <= atol + rtol * |oracle|
TOL = {torch.bfloat16: (1e-2, 1e-2), torch.float32: (1e-5, 1e-5)}


def log(msg):
    print(msg, flush=True)


def gpu_pools(st, gen_device="cpu", poison=None):
    """Device pools filled through pkv_append: the rows before the step, then
    the step's own rows."""
    kp, vp = st.new_pool("cuda", poison)
    for which in ("fill", "step"):
        k, v, sl = st.rows(which, "cuda", gen_device=gen_device)
        if k.shape[0]:
            pkv.pkv_append(k, v, kp, vp, sl)
        del k, v, sl
    return kp, vp


def gpu_attention(st, q, kp, vp, **kw):
    md = st.metadata("cuda")
    out = pkv.pkv_attention(q, kp, vp, md["block_tables"], md["seq_lens"],
                            md["query_start_loc"], st.scale, max_seqlen_q=st.max_seqlen_q,
                            max_seqlen_k=st.max_seqlen_k, kv_start=md["kv_start"], **kw)
    torch.cuda.synchronize()
    return out


def oracle_seq_outputs(st, q_host, seqs, gen_device="cpu", tokens=None):
    """Oracle outputs of the listed sequences, from their real rows (drawn on
    ``gen_device`` and copied to the host) laid out in a contiguous pool with an
    identity block table, i.e. the ragged form of the sequence.  ``tokens``
    optionally restricts sequence s to some of its query tokens (each computed
    as the decode it is equivalent to).  Returns {s: float64 [n, Hq, D]}."""
    qsl = st.query_start_loc()
    res = {}
    for s in seqs:
        k, v = st.seq_kv(s, gen_device)
        k, v = k.cpu(), v.cpu()
        L = k.shape[0]
        bs = 16
        nb = max(1, (L + bs - 1) // bs)
        kp = torch.full((nb, st.num_kv_heads, bs, st.head_dim), float("nan"), dtype=st.dtype)
        vp = kp.clone()
        kp, vp = oracle.oracle_append(kp, vp, k, v, np.arange(L, dtype=np.int64))
        bt = np.arange(nb, dtype=np.int32)[None]
        qrows = q_host[qsl[s]:qsl[s + 1]]
        n = qrows.shape[0]
        if tokens is None or s not in tokens:
            res[s] = oracle.oracle_attention(qrows, kp, vp, bt, [L], [0, n], st.scale)
        else:
            outs = []
            for i in tokens[s]:
                outs.append(oracle.oracle_attention(qrows[i:i + 1], kp, vp, bt, [L - n + i + 1],
                                                    [0, 1], st.scale))
            res[s] = np.concatenate(outs)
    return res


def oracle_seq_blocks(st, q_host, s, block=500, gen_device="cpu"):
    """Oracle outputs of every query token of sequence ``s``, computed in
    blocks of ``block`` tokens on a thread pool: tokens [i0, i1) of an n-token
    chunk over L keys are exactly the (i1 - i0)-token chunk at the end of the
    first L - n + i1 keys, so each block is one oracle call of its own (the
    oracle's own threads split a call by (sequence, kv head) only, which
    leaves most cores idle on one long sequence).  Returns float64 [n, Hq, D]."""
    from concurrent.futures import ThreadPoolExecutor
    qsl = st.query_start_loc()
    k, v = st.seq_kv(s, gen_device)
    k, v = k.cpu(), v.cpu()
    L = k.shape[0]
    bs = 16
    nb = max(1, (L + bs - 1) // bs)
    kp = torch.full((nb, st.num_kv_heads, bs, st.head_dim), float("nan"), dtype=st.dtype)
    vp = kp.clone()
    kp, vp = oracle.oracle_append(kp, vp, k, v, np.arange(L, dtype=np.int64))
    bt = np.arange(nb, dtype=np.int32)[None]
    qrows = q_host[qsl[s]:qsl[s + 1]]
    n = qrows.shape[0]
    cuts = list(range(0, n, block)) + [n]

    def run(j):
        i0, i1 = cuts[j], cuts[j + 1]
        return oracle.oracle_attention(qrows[i0:i1], kp, vp, bt, [L - n + i1], [0, i1 - i0],
                                       st.scale, threads=1)

    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        parts = list(pool.map(run, range(len(cuts) - 1)))
    return np.concatenate(parts)


def contiguous_pool(rows, num_kv_heads, head_dim, dtype, bs=16):
    """Oracle-side layout of whole sequences: sequence i's rows ``rows[i] =
    (k, v)`` fill pages base_i, base_i + 1, ... of a pool written by the
    oracle's append (unwritten bytes NaN); returns (k_pool, v_pool, block
    tables) with -1 past each sequence's pages.  Built from the generator's
    rows alone."""
    npg = [max(1, (k.shape[0] + bs - 1) // bs) for k, _ in rows]
    base = np.concatenate([[0], np.cumsum(npg)]).astype(np.int64)
    shape = (int(base[-1]), num_kv_heads, bs, head_dim)
    kp = torch.full(shape, float("nan"), dtype=dtype)
    vp = kp.clone()
    ks = torch.cat([k for k, _ in rows])
    vs = torch.cat([v for _, v in rows])
    slots = np.concatenate([base[i] * bs + np.arange(k.shape[0], dtype=np.int64)
                            for i, (k, _) in enumerate(rows)])
    kp, vp = oracle.oracle_append(kp, vp, ks, vs, slots)
    bt = np.full((len(rows), max(npg)), -1, dtype=np.int32)
    for i, n in enumerate(npg):
        bt[i, :n] = np.arange(base[i], base[i] + n, dtype=np.int32)
    return kp, vp, bt


def oracle_batches(st, q_host, gen_device="cpu", batch=16):
    """Oracle outputs of every sequence of a step, ``batch`` sequences per
    oracle call, each from its real rows (drawn on ``gen_device``) in a
    contiguous pool: yields (first query row, last query row + 1, float64
    [rows, Hq, D])."""
    qsl = st.query_start_loc()
    for s0 in range(0, st.num_seqs, batch):
        seqs = list(range(s0, min(s0 + batch, st.num_seqs)))
        rows = []
        for s in seqs:
            k, v = st.seq_kv(s, gen_device)
            rows.append((k.cpu(), v.cpu()))
        kp, vp, bt = contiguous_pool(rows, st.num_kv_heads, st.head_dim, st.dtype)
        lens = [k.shape[0] for k, _ in rows]
        q0, q1 = int(qsl[seqs[0]]), int(qsl[seqs[-1] + 1])
        sub_qsl = (qsl[seqs[0]:seqs[-1] + 2] - q0).astype(np.int32)
        ref = oracle.oracle_attention(q_host[q0:q1], kp, vp, bt, lens, sub_qsl, st.scale)
        del kp, vp, rows
        yield q0, q1, ref


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(got, ref, dtype, what, quiet=False, tol_scale=1.0):
    atol, rtol = (t * tol_scale for t in TOL[dtype])
    g = to_f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ok, maxerr = close(g, ref, atol, rtol)
    denom = float(np.linalg.norm(ref)) or 1.0
    rel = float(np.linalg.norm(np.nan_to_num(g - ref, nan=1e30))) / denom
    if not quiet or not ok:
        log(f"  {what}: max|err| {maxerr:.3e}  rel-L2 {rel:.3e}  "
            f"finite {bool(np.isfinite(g).all())}")
    assert ok, f"{what}: outside atol={atol} rtol={rtol} (max err {maxerr:.3e})"
    return maxerr, rel


def raw_bits(t: torch.Tensor) -> np.ndarray:
    iv = torch.int16 if t.dtype == torch.bfloat16 else torch.int32
    return t.detach().cpu().contiguous().view(iv).numpy()
