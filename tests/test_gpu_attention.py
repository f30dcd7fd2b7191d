"""pkv_attention on the GPU against the float64 oracle over a sweep of shapes:
group sizes 1-16, head_dim 64/128, float32 and bfloat16, decode contexts at
page edges and across several splits, speculative-verify windows of up to
16 / G tokens, prefill chunks of 2 to 1000 tokens with and without cached
context, mixed steps, left-padded steps; plus bitwise
properties of the GPU path itself (physical page placement, run-to-run
determinism, shared versus duplicated prefix pages) and a large packed step
(30,000 + 5,000 + 10 tokens) checked on every output; a step with 8x and 16x queries (sharp softmax rows)
pins the logit precision; sequences with no query token in the step.  Pools are NaN outside the valid rows."""
import numpy as np
import pytest
import torch

import paged_kv_attention_03_amd as pkv
from paged_kv_attention_03_amd import workloads as W
from tests.gpu_helpers import (check_close, gpu_attention, gpu_pools, log, oracle_seq_blocks,
                               raw_bits)
from tests.helpers import oracle_pools, oracle_step

DTYPES = [torch.float32, torch.bfloat16]
EDGE_LENS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 257, 1000]


def _run_full(st, what, q_mul=1.0, tol_scale=1.0):
    """GPU step vs the oracle on the whole step; also the pool bytes.  ``q_mul``
    (a power of two, so exact in both dtypes) scales the queries, ``tol_scale``
    the tolerance."""
    q = st.make_q("cpu") * q_mul
    kp, vp = gpu_pools(st, "cpu")
    okp, ovp = oracle_pools(st)
    assert np.array_equal(raw_bits(kp), okp.view(raw_bits(kp).dtype)), "K pool bytes differ"
    assert np.array_equal(raw_bits(vp), ovp.view(raw_bits(vp).dtype)), "V pool bytes differ"
    out = gpu_attention(st, q.cuda(), kp, vp)
    ref = oracle_step(st, q, pools=(okp, ovp))
    check_close(out, ref, st.dtype, what, tol_scale=tol_scale)
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 5, 8, 16])
def test_decode_sweep(G, D, dtype):
    log(f"decode G={G} D={D} {dtype}")
    st = W.build_step("decode-sweep", EDGE_LENS, [1] * len(EDGE_LENS), 2 * G, 2, D, dtype,
                      100 + G * 7 + D)
    _run_full(st, f"decode G={G} D={D}")


PREFILL_SHAPES = [(2, 2), (3, 10), (17, 17), (64, 100), (200, 213), (33, 1000), (1, 50),
                  (1, 300)]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 5, 8])
def test_prefill_and_mixed_sweep(G, D, dtype):
    log(f"prefill G={G} D={D} {dtype}")
    ql = [a for a, _ in PREFILL_SHAPES]
    lens = [b for _, b in PREFILL_SHAPES]
    st = W.build_step("prefill-sweep", lens, ql, 2 * G, 2, D, dtype, 200 + G * 7 + D)
    _run_full(st, f"prefill G={G} D={D}")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("q_mul", [8.0, 16.0])
def test_sharp_softmax_step(q_mul, dtype):
    """Queries 8x and 16x larger than N(0, 1): logits of tens, so most rows put
    nearly all their weight on a few keys and an error in a logit shows in the
    output almost undamped.  A kernel that rounded the scaled queries (or the
    logits) to bfloat16 before the exponential fails the bfloat16 case (max
    error ~0.09 at 8x against ~0.015 for exact logits), while ordinary inputs
    hide it.  Decodes, verify windows and chunks with cached context, G 4,
    D 128.

    The bfloat16 bound is the usual 1e-2.  The float32 bound of 1e-5 holds for
    logits of order one: a float32 logit carries a rounding error in proportion
    to its magnitude, and the softmax passes it on as a relative error of the
    weights, so the float32 bound is scaled by the query factor (a plain
    float32 softmax attention on the host misses 1e-5 on these inputs by
    2.8x at 8x and 4.4x at 16x, the GPU path by 2.5x and 4.0x)."""
    log(f"sharp softmax q x{q_mul} {dtype}")
    lens = [900, 300, 2000, 77, 1500, 1640, 33, 4097]
    ql = [1, 3, 128, 1, 4, 700, 2, 1000]
    st = W.build_step("sharp-softmax", lens, ql, 16, 4, 128, dtype, 260 + int(q_mul))
    _run_full(st, f"sharp softmax q x{q_mul}", q_mul=q_mul,
              tol_scale=q_mul if dtype == torch.float32 else 1.0)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_whole_segment_decode(G, dtype, monkeypatch):
    """Decode steps run with one wave per (sequence, kv head) segment (no
    segment cut, no merge launch; the library picks it for steps whose
    segments are all short), forced here on longer ones too: page-edge
    contexts, verify windows and a left-padded step against the oracle."""
    monkeypatch.setenv("PKV_DECODE_SEGMENTS", "whole")
    log(f"whole-segment decode G={G} {dtype}")
    st = W.build_step("whole-decode", EDGE_LENS, [1] * len(EDGE_LENS), 2 * G, 2, 128, dtype,
                      310 + G)
    _run_full(st, f"whole-segment decode G={G}")
    W_ = max(1, 16 // G)
    ql = [min(W_, L, 1 + i % W_) for i, L in enumerate(WINDOW_LENS)]
    st = W.build_step("whole-windows", WINDOW_LENS, ql, 2 * G, 2, 64, dtype, 320 + G)
    _run_full(st, f"whole-segment windows G={G}")
    st = W.build_step("whole-padded", [300, 2000, 1000, 17], [1, 1, 1, 1], 2 * G, 2, 128, dtype,
                      330 + G, padded=True)
    _run_full(st, f"whole-segment left-padded G={G}")


WINDOW_LENS = [2, 15, 16, 17, 31, 33, 64, 65, 100, 257, 1000, 1600]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 5, 8, 16])
def test_verify_window_sweep(G, D, dtype):
    """Speculative-verify windows: sequences with 1..W query tokens (W = 16 // G)
    take the decode path with a causal cap per window token; one sequence with
    W + 1 tokens and one long chunk take the prefill path in the same step."""
    wmax = 16 // G
    ql = [1 + i % wmax for i in range(len(WINDOW_LENS))]
    ql = [min(n, L) for n, L in zip(ql, WINDOW_LENS)]
    lens = WINDOW_LENS + [40, 700]
    ql = ql + [min(wmax + 1, 40), 90]
    log(f"windows G={G} D={D} {dtype} q_lens={ql}")
    st = W.build_step("window-sweep", lens, ql, 2 * G, 2, D, dtype, 700 + G * 7 + D)
    _run_full(st, f"windows G={G} D={D}")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("max_q", [2, 3, 4])
def test_windows_only_step(max_q, dtype):
    """A step of decodes and verify windows only (max_seqlen_q <= 16 // G): no
    prefill launch; the window sizes the decode workspace."""
    lens = [3000, 1, 4, 17, 512, 2049, 33, 5000]
    ql = [max_q, 1, min(max_q, 4), 2, max_q, 1, max_q, 2]
    st = W.build_step("windows-only", lens, ql, 16, 4, 128, dtype, 800 + max_q)
    assert st.max_seqlen_q == max_q
    _run_full(st, f"windows-only max_q={max_q}")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("mixed", ["fused", "split"])
def test_sequences_without_query_tokens(mixed, dtype, monkeypatch):
    """Sequences that contribute no query token to the step (query_start_loc
    repeats a value: the first, the last and runs in between) sit among
    decodes, verify windows and prefill chunks; they own no output row, and
    the tokens around them keep their rows and keys.  Both launch forms of a
    mixed step, then a decode-only step in both decode forms."""
    monkeypatch.setenv("PKV_MIXED_STEP", mixed)
    lens = [40, 300, 17, 900, 64, 64, 2000, 33, 1500, 5]
    ql = [0, 1, 0, 3, 0, 0, 700, 0, 40, 0]
    log(f"zero-token sequences {mixed} {dtype} q_lens={ql}")
    st = W.build_step("zero-q-mixed", lens, ql, 8, 2, 128, dtype, 910)
    qsl = st.query_start_loc()
    assert list(qsl).count(0) == 2 and qsl[-1] == st.total_q
    _run_full(st, f"zero-token sequences, mixed step ({mixed})")
    if mixed == "split":
        for form in ("whole", "split"):
            monkeypatch.setenv("PKV_DECODE_SEGMENTS", form)
            st = W.build_step("zero-q-decode", [100, 17, 250, 64, 1, 200], [0, 1, 0, 1, 1, 0],
                              16, 2, 64, dtype, 920)
            _run_full(st, f"zero-token sequences, decode step ({form} segments)")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
def test_left_padded_step_matches_oracle(dtype):
    lens = [5, 40, 33, 16, 700, 1300, 260]
    ql = [1, 2, 1, 16, 1, 100, 1]
    st = W.build_step("padded", lens, ql, 8, 2, 128, dtype, 300, padded=True)
    log(f"padded kv_start={st.kv_start}")
    assert max(st.kv_start) > 1000
    _run_full(st, "left-padded")


@pytest.mark.gpu
def test_page_placement_does_not_change_a_bit():
    outs = []
    for perm in (1, 2, 3):
        st = W.build_step("perm", [5, 700, 33, 300], [1, 1, 20, 1], 8, 2, 128, torch.bfloat16,
                          400, perm_seed=perm)
        q = st.make_q("cpu").cuda()
        kp, vp = gpu_pools(st)
        outs.append(raw_bits(gpu_attention(st, q, kp, vp)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.gpu
def test_runs_are_bitwise_deterministic():
    st = W.config_step(3)
    q = st.make_q("cpu").cuda()
    kp, vp = gpu_pools(st)
    a = raw_bits(gpu_attention(st, q, kp, vp))
    b = raw_bits(gpu_attention(st, q, kp, vp))
    assert np.array_equal(a, b)


@pytest.mark.gpu
def test_shared_prefix_equals_duplicated_prefix_bitwise():
    # the pool manager forks the prefix (pages held in common) in one loop and
    # gives every sequence its own copy in the other
    from paged_kv_attention_03_amd.engine import AgentLoop, AgentPlanner
    run = W.AgentRun(steps=5, num_q_heads=16, num_kv_heads=2, head_dim=128,
                     prompt_lens=[600, 517, 1000, 530], shared_prefix=512)
    loops = []
    for share in (True, False):
        planner = AgentPlanner(run, share_prefix=share)
        loops.append(AgentLoop(run, planner, poison=True, gen_device="cpu"))
    assert len(loops[0].plan.shared_pages) == 32 and not loops[1].plan.shared_pages
    for i in range(run.steps):
        outs = [raw_bits(lp.step(i)).copy() for lp in loops]
        torch.cuda.synchronize()
        assert np.array_equal(outs[0], outs[1]), f"step {i}"
    for lp in loops:
        lp.plan.close()


@pytest.mark.gpu
def test_packed_30000_5000_10_step():
    """A packed prefill step of 30,000 + 5,000 + 10 tokens (the padded-versus-
    packed illustration of the vllm-metal post; ~1,900 prefill tiles, several
    waves of workgroups), every output against the oracle."""
    lens = [30000, 5000, 10]
    st = W.build_step("30k-5k-10", lens, lens, 8, 2, 128, torch.bfloat16, 500)
    q = st.make_q("cpu")
    kp, vp = gpu_pools(st, "cpu")
    out = gpu_attention(st, q.cuda(), kp, vp)
    qsl = st.query_start_loc()
    for s in range(3):
        log(f"30k-5k-10: oracle for sequence {s} ({lens[s]} tokens)")
        ref = oracle_seq_blocks(st, q, s)
        check_close(out[qsl[s]:qsl[s + 1]], ref, st.dtype, f"seq {s}")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("num_seqs", [512, 513, 1500])
def test_many_sequences(num_seqs, dtype):
    """Batches at and past the size where the decode waves stop planning their
    own pieces and a plan kernel does it: ragged short contexts, decodes and
    2-token windows, one prefill chunk."""
    rng = np.random.default_rng(num_seqs)
    lens = rng.integers(1, 300, size=num_seqs).tolist()
    ql = [2 if (i % 7 == 3 and L >= 2) else 1 for i, L in enumerate(lens)]
    lens[5], ql[5] = 400, 37
    log(f"many sequences: {num_seqs} {dtype}")
    st = W.build_step("many-seqs", lens, ql, 16, 4, 64, dtype, 950 + num_seqs)
    _run_full(st, f"{num_seqs} sequences")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
def test_most_sequences_a_step_takes(dtype):
    """16384 sequences, the most a step may hold (the plan kernel keeps one
    count per sequence in LDS): short ragged contexts, decodes, 2-token
    windows and sequences with no query token, against the oracle on every
    output.  The pools are filled directly -- one seeded draw over every slot,
    NaN wherever no sequence has a key -- rather than row by row through the
    append kernel, which would take minutes of host time at this count."""
    n = 16384
    rng = np.random.default_rng(n)
    lens = rng.integers(1, 48, size=n)
    ql = [0 if i % 97 == 13 else (2 if (i % 11 == 4 and L >= 2) else 1)
          for i, L in enumerate(lens.tolist())]
    log(f"{n} sequences {dtype}")
    st = W.build_step("max-seqs", lens.tolist(), ql, 8, 2, 64, dtype, 960)
    assert st.num_seqs == n
    md = st.metadata("cpu")
    bt = md["block_tables"].numpy()
    npg = (lens + 15) // 16
    s_idx = np.repeat(np.arange(n), npg)
    j_idx = np.concatenate([np.arange(k) for k in npg])
    pages = bt[s_idx, j_idx]
    assert np.unique(pages).size == pages.size
    used = np.minimum(16, lens[s_idx] - 16 * j_idx)
    valid = np.zeros((st.num_blocks, 16), dtype=bool)
    valid[pages] = np.arange(16)[None, :] < used[:, None]
    shape = (st.num_blocks, st.num_kv_heads, 16, st.head_dim)
    hole = torch.from_numpy(~valid)[:, None, :, None].expand(shape)
    kp = W.randn(shape, 961, "cpu", dtype).masked_fill(hole, float("nan"))
    vp = W.randn(shape, 962, "cpu", dtype).masked_fill(hole, float("nan"))
    q = st.make_q("cpu")
    out = gpu_attention(st, q.cuda(), kp.cuda(), vp.cuda())
    ref = oracle_step(st, q, pools=(kp, vp))
    check_close(out, ref, st.dtype, f"{n} sequences")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
def test_long_context_prefill_chunk(dtype):
    """A 40-token chunk at the end of a 100,000-key context and a decode over
    70,001 keys in one step: contexts far past 65,536 keys on both paths."""
    st = W.build_step("long-context", [100000, 70001], [40, 1], 4, 1, 64, dtype, 900)
    assert st.max_seqlen_k > 65536
    _run_full(st, "long context")


@pytest.mark.gpu
def test_prepared_calls_match_the_plain_calls():
    """prepare_append / prepare_attention re-issue the same C calls: pools and
    outputs bitwise equal to pkv_append / pkv_attention on the mixed step, also
    after the tensors' contents change in place between calls."""
    st = W.config_step(3)
    log("prepared calls on the mixed step")
    q = st.make_q("cpu").cuda()
    # the step's rows into NaN pools, by the plain and the prepared call
    k_new, v_new, slots = st.rows("step", "cuda", gen_device="cpu")
    ka, va = st.new_pool("cuda", poison=True)
    kb, vb = ka.clone(), va.clone()
    before = raw_bits(kb).copy()
    pkv.pkv_append(k_new, v_new, ka, va, slots)
    app = pkv.prepare_append(k_new, v_new, kb, vb, slots)
    app()
    torch.cuda.synchronize()
    assert not np.array_equal(raw_bits(kb), before), "the prepared append wrote nothing"
    assert np.array_equal(raw_bits(kb), raw_bits(ka)) and np.array_equal(raw_bits(vb), raw_bits(va))
    del ka, va, kb, vb
    kp, vp = gpu_pools(st, "cpu")
    md = st.metadata("cuda")
    att = pkv.prepare_attention(q, kp, vp, md["block_tables"], md["seq_lens"],
                                md["query_start_loc"], st.scale, max_seqlen_q=st.max_seqlen_q,
                                max_seqlen_k=st.max_seqlen_k, kv_start=md["kv_start"])
    for rep in range(2):
        if rep:
            q.mul_(0.5)  # new contents, same storage
        want = raw_bits(gpu_attention(st, q, kp, vp)).copy()
        att()
        torch.cuda.synchronize()
        assert np.array_equal(raw_bits(att.out), want), f"rep {rep}"


@pytest.mark.gpu
def test_workspace_reuse_and_explicit_out():
    st = W.config_step(2)
    q = st.make_q("cpu").cuda()
    kp, vp = gpu_pools(st)
    need = pkv.pkv_attention_workspace_size(st.num_seqs, st.total_q, st.max_seqlen_q,
                                            st.max_seqlen_k, st.num_q_heads, st.num_kv_heads,
                                            st.head_dim, 16, st.dtype)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    out = torch.full_like(q, float("nan"))
    a = raw_bits(gpu_attention(st, q, kp, vp, workspace=ws, out=out))
    b = raw_bits(gpu_attention(st, q, kp, vp, workspace=ws))
    assert np.array_equal(a, b)


@pytest.mark.gpu
def test_unsupported_group_size_raises():
    q = torch.zeros(1, 34, 128, dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros(4, 2, 16, 128, dtype=torch.bfloat16, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError):
        pkv.pkv_attention(q, kp, kp, torch.zeros(1, 4, **i32), torch.ones(1, **i32),
                          torch.tensor([0, 1], **i32), 0.1, max_seqlen_q=1, max_seqlen_k=1)
