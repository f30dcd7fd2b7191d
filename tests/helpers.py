"""Shared test helpers: build an oracle-side pool from the generator's rows and
run the oracle on a step.  Test code only."""
import numpy as np
import torch

import oracle


def oracle_pools(st, seqs=None):
    """Host pools holding every row of the step (fill rows, then the step's
    own rows), written by the oracle's append."""
    kp, vp = st.new_pool(device="cpu")
    kf, vf, sf = st.rows("fill", device="cpu", seqs=seqs)
    kp, vp = oracle.oracle_append(kp, vp, kf, vf, sf)
    ks, vs, ss = st.rows("step", device="cpu", seqs=seqs)
    kp, vp = oracle.oracle_append(kp, vp, ks, vs, ss)
    return kp, vp


def raw_to_torch(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.view(torch.bfloat16) if dtype == torch.bfloat16 else t


def oracle_step(st, q=None, pools=None, threads=0, lib=None):
    q = st.make_q("cpu") if q is None else q
    kp, vp = oracle_pools(st) if pools is None else pools
    md = st.metadata("cpu")
    return oracle.oracle_attention(q, kp, vp, md["block_tables"], md["seq_lens"],
                                   md["query_start_loc"], st.scale, kv_start=md["kv_start"],
                                   threads=threads, lib=lib)


def close(got, ref, atol, rtol):
    """Elementwise |got - ref| <= atol + rtol * |ref| (ref = oracle)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    ok = err <= atol + rtol * np.abs(ref)
    return bool(np.all(ok)) and bool(np.all(np.isfinite(got))), float(np.nanmax(err) if err.size else 0.0)
