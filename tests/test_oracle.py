"""Pins for the float64 oracle, on the CPU.

Each pin ties the oracle to something other than itself: independent dense
formulations (numpy matrix products; torch's CPU scaled_dot_product_attention
with an explicit mask), closed forms, invariances the pages imply (page
placement, page size, chunking, batch mates, left padding, shared prefix), and
byte-exact agreement of the append with numpy's own scatter.  A last group
plants plausible mistakes in a copy of the oracle source and checks that some
pin fails for each.
"""
import json
import math
import os
import re
import tempfile

import numpy as np
import pytest
import torch

import oracle
from paged_kv_attention_03_amd import workloads as W
from tests.dense_ref import dense_numpy, dense_torch_sdpa, to_f64
from tests.helpers import oracle_pools, oracle_step

HERE = os.path.dirname(os.path.abspath(__file__))

SMALL_CASES = [
    # name, ctx lens, q lens, Hq, Hkv, D, dtype, padded
    ("decode-g2", [17, 33, 64, 100], [1, 1, 1, 1], 4, 2, 64, torch.float32, False),
    ("mixed-g4", [40, 23, 16, 1, 57], [1, 7, 16, 1, 3], 8, 2, 32, torch.bfloat16, False),
    ("chunk-g5", [70, 31], [20, 31], 10, 2, 16, torch.bfloat16, False),
    ("mha", [9, 48], [4, 1], 3, 3, 8, torch.float32, False),
    ("padded-g8", [5, 40, 33, 16], [1, 2, 1, 16], 16, 2, 16, torch.float32, True),
    ("tail-edges", [1, 15, 16, 17, 31, 32, 33], [1] * 7, 2, 1, 8, torch.float32, False),
]


def _step(case, seed=11, **kw):
    name, lens, ql, hq, hkv, d, dt, padded = case
    return W.build_step(name, lens, ql, hq, hkv, d, dt, seed, padded=padded, **kw)


def _per_seq_dense(st, q, fn):
    out = np.zeros((st.total_q, st.num_q_heads, st.head_dim))
    qsl = st.query_start_loc()
    G = st.num_q_heads // st.num_kv_heads
    for s in range(st.num_seqs):
        k, v = st.seq_kv(s, "cpu")
        lo, hi = qsl[s], qsl[s + 1]
        if hi == lo:
            continue
        out[lo:hi] = fn(to_f64(q[lo:hi]), to_f64(k), to_f64(v), np.float64(np.float32(st.scale)),
                        G)
    return out


# ---------------------------------------------------------------- append pins

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_append_matches_numpy_scatter(dtype, oracle_lib):
    rng = np.random.default_rng(5)
    nb, hkv, bs, d, t = 9, 3, 16, 8, 40
    pool_k = W.randn((nb, hkv, bs, d), 1, "cpu", dtype)
    pool_v = W.randn((nb, hkv, bs, d), 2, "cpu", dtype)
    kn = W.randn((t, hkv, d), 3, "cpu", dtype)
    vn = W.randn((t, hkv, d), 4, "cpu", dtype)
    slots = rng.choice(nb * bs, size=t, replace=False).astype(np.int64)
    slots[::7] = -1  # padding tokens are skipped
    kp, vp = oracle.oracle_append(pool_k, pool_v, kn, vn, slots)
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    ek = pool_k.view(iv).numpy().copy()
    ev = pool_v.view(iv).numpy().copy()
    m = slots >= 0
    ek[slots[m] // bs, :, slots[m] % bs, :] = kn.view(iv).numpy()[m]
    ev[slots[m] // bs, :, slots[m] % bs, :] = vn.view(iv).numpy()[m]
    assert np.array_equal(kp.view(ek.dtype), ek)
    assert np.array_equal(vp.view(ev.dtype), ev)


# ---------------------------------------------------------- dense equivalence

@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_oracle_equals_dense_numpy_and_sdpa(case, oracle_lib):
    st = _step(case)
    q = st.make_q("cpu")
    got = oracle_step(st, q)
    ref_np = _per_seq_dense(st, q, dense_numpy)
    ref_sdpa = _per_seq_dense(st, q, dense_torch_sdpa)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref_np, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, ref_sdpa, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- closed forms

def _single(q, k, v, scale=1.0, n=1, a=None):
    """One sequence, contiguous pages; k/v [L, 1, D] float32."""
    L, _, d = k.shape
    bs = 4
    nb = (L + bs - 1) // bs
    kp = np.full((nb, 1, bs, d), np.nan, np.float32)
    vp = np.full((nb, 1, bs, d), np.nan, np.float32)
    for j in range(L):
        kp[j // bs, 0, j % bs] = k[j, 0]
        vp[j // bs, 0, j % bs] = v[j, 0]
    bt = np.arange(nb, dtype=np.int32)[None]
    return oracle.oracle_attention(q.astype(np.float32), kp, vp, bt, [L], [0, n], scale,
                                   kv_start=None if a is None else [a])


def test_single_key_returns_its_value_exactly(oracle_lib):
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, 8)).astype(np.float32)
    k = rng.standard_normal((1, 1, 8)).astype(np.float32)
    v = rng.standard_normal((1, 1, 8)).astype(np.float32)
    out = _single(q, k, v, 0.3)
    assert np.array_equal(out[0, 0], v[0, 0].astype(np.float64))


def test_constant_keys_give_mean_of_visible_values(oracle_lib):
    rng = np.random.default_rng(1)
    L, n = 13, 4
    q = rng.standard_normal((n, 1, 8)).astype(np.float32)
    k = np.repeat(rng.standard_normal((1, 1, 8)).astype(np.float32), L, 0)
    v = rng.standard_normal((L, 1, 8)).astype(np.float32)
    out = _single(q, k, v, 0.7, n=n)
    for i in range(n):
        p = L - n + i
        np.testing.assert_allclose(out[i, 0], v[:p + 1, 0].astype(np.float64).mean(0),
                                   rtol=1e-14, atol=1e-14)


def test_dominant_key_selects_its_value(oracle_lib):
    rng = np.random.default_rng(2)
    L = 9
    k = rng.standard_normal((L, 1, 8)).astype(np.float32) * 0.01
    k[5, 0] = 0.0
    k[5, 0, 3] = 1000.0
    q = np.zeros((1, 1, 8), np.float32)
    q[0, 0, 3] = 1.0
    v = rng.standard_normal((L, 1, 8)).astype(np.float32)
    out = _single(q, k, v, 1.0)
    assert np.array_equal(out[0, 0], v[5, 0].astype(np.float64))


def test_two_keys_follow_the_logistic_weight(oracle_lib):
    # two visible keys with logit gap delta: weight of the second is 1/(1+e^-delta)
    k = np.zeros((2, 1, 4), np.float32)
    k[1, 0, 0] = 2.0
    q = np.zeros((1, 1, 4), np.float32)
    q[0, 0, 0] = 0.75
    v = np.array([[[1, 0, 0, 0]], [[0, 1, 0, 0]]], np.float32)
    delta = 0.5 * 2.0 * 0.75
    w1 = 1.0 / (1.0 + math.exp(-delta))
    out = _single(q, k, v, 0.5)
    np.testing.assert_allclose(out[0, 0], [1 - w1, w1, 0, 0], rtol=0, atol=1e-15)


def test_golden_hand_worked_cases(oracle_lib):
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], np.float32)[:, None, :]
        k = np.array(c["k"], np.float32)[:, None, :]
        v = np.array(c["v"], np.float32)[:, None, :]
        out = _single(q, k, v, c["scale"], n=q.shape[0], a=c.get("kv_start"))
        np.testing.assert_allclose(out[:, 0, :], np.array(c["out"]), rtol=0, atol=c["atol"],
                                   err_msg=c["name"])


# -------------------------------------------------------------- invariances

def test_page_permutation_invariance_bitwise(oracle_lib):
    case = SMALL_CASES[1]
    a = _step(case, perm_seed=101)
    b = _step(case, perm_seed=202)
    assert not np.array_equal(a.block_tables, b.block_tables)
    q = a.make_q("cpu")
    assert np.array_equal(oracle_step(a, q), oracle_step(b, q))


def test_page_size_invariance_bitwise(oracle_lib):
    case = SMALL_CASES[2]
    outs = []
    for bs in (1, 16, 32):
        st = _step(case, block_size=bs)
        outs.append(oracle_step(st, st.make_q("cpu")))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def test_chunking_invariance_bitwise(oracle_lib):
    """One 8-token chunk == two 4-token chunks == eight decode steps."""
    st = W.build_step("chunk", [37], [8], 4, 2, 16, torch.float32, 21)
    kp, vp = oracle_pools(st)
    q = st.make_q("cpu")
    bt = st.block_tables
    L = 37
    one = oracle.oracle_attention(q, kp, vp, bt, [L], [0, 8], st.scale)
    two = np.concatenate([
        oracle.oracle_attention(q[:4], kp, vp, bt, [L - 4], [0, 4], st.scale),
        oracle.oracle_attention(q[4:], kp, vp, bt, [L], [0, 4], st.scale)])
    dec = np.concatenate([oracle.oracle_attention(q[i:i + 1], kp, vp, bt, [L - 7 + i], [0, 1],
                                                  st.scale) for i in range(8)])
    assert np.array_equal(one, two) and np.array_equal(one, dec)


def test_batch_independence_bitwise(oracle_lib):
    st = _step(SMALL_CASES[1])
    q = st.make_q("cpu")
    kp, vp = oracle_pools(st)
    full = oracle_step(st, q, pools=(kp, vp))
    qsl = st.query_start_loc()
    for s in range(st.num_seqs):
        lo, hi = qsl[s], qsl[s + 1]
        one = oracle.oracle_attention(q[lo:hi], kp, vp, st.block_tables[s:s + 1],
                                      [st.seq_lens[s]], [0, hi - lo], st.scale)
        assert np.array_equal(one, full[lo:hi])


def test_gqa_equals_mha_on_repeated_heads_bitwise(oracle_lib):
    st = _step(SMALL_CASES[1])
    q = st.make_q("cpu")
    kp, vp = oracle_pools(st)
    G = st.num_q_heads // st.num_kv_heads
    gqa = oracle_step(st, q, pools=(kp, vp))
    kr = np.repeat(kp, G, axis=1)
    vr = np.repeat(vp, G, axis=1)
    md = st.metadata("cpu")
    mha = oracle.oracle_attention(q, kr, vr, md["block_tables"], md["seq_lens"],
                                  md["query_start_loc"], st.scale)
    assert np.array_equal(gqa, mha)


def test_thread_count_invariance_bitwise(oracle_lib):
    st = _step(SMALL_CASES[2])
    q = st.make_q("cpu")
    pools = oracle_pools(st)
    before = oracle.max_threads()
    assert np.array_equal(oracle_step(st, q, pools, threads=1), oracle_step(st, q, pools, threads=8))
    assert oracle.max_threads() == before  # a thread limit applies to its own call only


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_left_padded_equals_ragged_bitwise(dtype, oracle_lib):
    lens, ql = [5, 40, 33, 16, 70], [1, 2, 1, 16, 1]
    rag = W.build_step("rag", lens, ql, 8, 2, 16, dtype, 31)
    pad = W.build_step("pad", lens, ql, 8, 2, 16, dtype, 31, padded=True)
    assert pad.kv_start is not None and max(pad.kv_start) > 16
    q = rag.make_q("cpu")
    a = oracle_step(rag, q)
    b = oracle_step(pad, q)
    assert np.all(np.isfinite(b))  # padding pages are NaN and must stay unread
    assert np.array_equal(a, b)


def _agent_layout(run, share, seed):
    """Block tables and slots of an agent run laid out in a shuffled pool of
    the test's own: with ``share`` the prefix pages are listed by every
    sequence, else each sequence holds its own copy of the prefix."""
    rng = np.random.default_rng(seed)
    S, P = run.num_seqs, run.shared_prefix
    npg = [(n + 15) // 16 for n in run.final_lens]
    nb = sum(npg) + 8
    free = list(rng.permutation(nb))
    shared = [int(free.pop()) for _ in range(P // 16)] if share else []
    bt = np.full((S, max(npg)), -1, np.int32)
    slots = []
    for s in range(S):
        for p in range(npg[s]):
            bt[s, p] = shared[p] if p < len(shared) else int(free.pop())
        j = np.arange(run.final_lens[s], dtype=np.int64)
        slots.append(bt[s, j // 16].astype(np.int64) * 16 + j % 16)
    return bt, slots, nb


def test_shared_prefix_equals_duplicated_prefix_bitwise(oracle_lib):
    run = W.AgentRun(steps=3, num_q_heads=4, num_kv_heads=2, head_dim=16,
                     prompt_lens=[40, 57, 33, 64], shared_prefix=32)
    rows = [run.seq_kv(s, "cpu") for s in range(run.num_seqs)]
    outs = []
    for share in (True, False):
        bt, slots, nb = _agent_layout(run, share, 5)
        if share:
            assert all((bt[s, :2] == bt[0, :2]).all() for s in range(4))
        else:
            assert len(set(bt[:, 0].tolist())) == 4
        kp = torch.full((nb, 2, 16, 16), float("nan"), dtype=run.dtype)
        vp = kp.clone()
        for s, (k, v) in enumerate(rows):  # a shared page is written with identical rows
            kp, vp = oracle.oracle_append(kp, vp, k, v, slots[s])
        res = []
        for i in range(run.steps):
            res.append(oracle.oracle_attention(run.step_q(i, "cpu"), kp, vp, bt,
                                               run.seq_lens_at(i), np.arange(5, dtype=np.int32),
                                               run.scale))
        outs.append(res)
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_poisoned_pool_never_reaches_the_result(oracle_lib):
    st = _step(SMALL_CASES[5])  # contexts at page edges, pool NaN elsewhere
    out = oracle_step(st)
    assert np.all(np.isfinite(out))


def test_metadata_out_of_range_is_rejected(oracle_lib):
    st = _step(SMALL_CASES[0])
    q = st.make_q("cpu")
    kp, vp = oracle_pools(st)
    bt = st.block_tables.copy()
    bt[0, 0] = st.num_blocks
    with pytest.raises(ValueError):
        oracle.oracle_attention(q, kp, vp, bt, st.seq_lens, st.query_start_loc(), st.scale)
    with pytest.raises(ValueError):  # more query tokens than keys
        oracle.oracle_attention(q, kp, vp, st.block_tables, [1, 33, 64, 100],
                                [0, 2, 3, 4], st.scale)


# ------------------------------------------------- planted mistakes (CPU)

MUTATIONS = {
    "top-left causal": ("const int64_t p = L - n + i;", "const int64_t p = i;"),
    "interleaved GQA": ("const int h = g * G + hh;", "const int h = hh * num_kv_heads + g;"),
    "exclusive last key": ("const int64_t last = p;", "const int64_t last = p - 1;"),
    "wrong page offset": ("+ j % block_size) * D;", "+ ((j % block_size) ^ 1)) * D;"),
    "dropped scale": ("w[j - a] = scale * acc;", "w[j - a] = acc;"),
    "no normalisation": ("o[d] /= Z;", "o[d] /= 1.0;"),
    "ignored kv_start": ("const int64_t a = kv_start ? kv_start[s] : 0;", "const int64_t a = 0;"),
    "flipped exponent": ("w[j - a] = exp(w[j - a] - m);", "w[j - a] = exp(m - w[j - a]);"),
    # (every planted mistake keeps its reads inside the arrays it indexes)
    "pages in reverse order": (
        "int64_t blk = block_tables[(int64_t)s * max_blocks_per_seq + j / block_size];",
        "int64_t blk = block_tables[(int64_t)s * max_blocks_per_seq + (L - 1) / block_size"
        " - j / block_size];"),
}


def _pin_battery(lib):
    """Returns the names of the pins a build fails."""
    failed = []
    for case in SMALL_CASES:
        st = _step(case)
        q = st.make_q("cpu")
        try:
            got = oracle_step(st, q, lib=lib)
        except ValueError:
            failed.append(case[0] + ":rejected")
            continue
        ref = _per_seq_dense(st, q, dense_numpy)
        if not np.allclose(got, ref, rtol=1e-12, atol=1e-12) or not np.all(np.isfinite(got)):
            failed.append(case[0])
    return failed


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_planted_mistake(name, oracle_lib, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "pkv_oracle.c")).read()
    before, after = MUTATIONS[name]
    assert src.count(before) == 1, f"mutation anchor not found: {before}"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(before, after))
    so = oracle.compile_source(str(path), str(tmp_path / "libmut.so"))
    lib = oracle.load_library(so)
    assert _pin_battery(lib), f"no pin caught '{name}'"


def test_unmutated_oracle_passes_battery(oracle_lib):
    assert _pin_battery(None) == []
