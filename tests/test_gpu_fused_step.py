"""The single-launch mixed step (decode waves and prefill tiles in one grid)
against the separate launches and the float64 oracle.

PKV_MIXED_STEP selects the path per call (fused: one launch for decode and
prefill, then the merge; split: decode, merge, prefill), PKV_STEP_TILE_FIRST
how many of every 4 workgroups of the one launch compute their tile before
their decode waves.  Each decode wave and each prefill tile does the same work
in every form, so outputs must be bitwise equal (the fused launch is checked
with the default order, every workgroup decode-first and every workgroup
tile-first); the fused output is also checked against the oracle.  Cases: the
mixed chunked-prefill workload in bf16 and its fp32 shadow, decodes with
verify windows and chunks at several group sizes and head dims, a step past
512 sequences (the plan kernel feeds the decode waves), contexts past 65,536
keys (the prefill variant that reads block ids through the scalar cache), a
prefill-only step, and a HIP graph replay of the fused step."""
import os

import numpy as np
import pytest
import torch

from paged_kv_attention_03_amd import workloads as W
from tests.gpu_helpers import check_close, gpu_attention, gpu_pools, log, raw_bits
from tests.helpers import oracle_pools, oracle_step


def _with_env(name, value, fn):
    old = os.environ.get(name)
    os.environ[name] = value
    try:
        return fn()
    finally:
        if old is None:
            del os.environ[name]
        else:
            os.environ[name] = old


def _with_mode(mode, fn):
    return _with_env("PKV_MIXED_STEP", mode, fn)


def _check(st, what):
    log(f"fused step: {what}: seqs={st.num_seqs} total_q={st.total_q} max_q={st.max_seqlen_q} "
        f"max_k={st.max_seqlen_k} G={st.num_q_heads // st.num_kv_heads} D={st.head_dim} {st.dtype}")
    q = st.make_q("cpu")
    kp, vp = gpu_pools(st, "cpu")
    qd = q.cuda()
    split = _with_mode("split", lambda: gpu_attention(st, qd, kp, vp))
    fused = _with_mode("fused", lambda: gpu_attention(st, qd, kp, vp))
    assert np.array_equal(raw_bits(fused), raw_bits(split)), f"{what}: fused != split"
    for order in ("0", "4"):
        other = _with_env("PKV_STEP_TILE_FIRST", order,
                          lambda: _with_mode("fused", lambda: gpu_attention(st, qd, kp, vp)))
        assert np.array_equal(raw_bits(other), raw_bits(split)), \
            f"{what}: fused with PKV_STEP_TILE_FIRST={order} != split"
    ref = oracle_step(st, q, pools=oracle_pools(st))
    check_close(fused, ref, st.dtype, f"{what} fused vs oracle")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32-shadow"])
def test_mixed_workload(dtype):
    _check(W.config_step(3, dtype=dtype), "mixed chunked-prefill workload")


CASES = [
    # (name, lens, q_lens, Hq, Hkv, D, dtype)
    ("g4-windows-chunks", [900, 300, 2000, 77, 1500, 1640, 33], [1, 3, 128, 1, 4, 700, 2], 16, 4,
     128, torch.bfloat16),
    ("g8-d64", [5000, 17, 4100, 260], [1, 1, 300, 2], 32, 4, 64, torch.bfloat16),
    ("g1-f32-d64", [400, 1000, 31, 150], [1, 60, 1, 149], 4, 4, 64, torch.float32),
    ("g5-f32-d128", [700, 2048, 64], [1, 512, 3], 40, 8, 128, torch.float32),
    # equal chunks: the host bounds rule out decodes, so the prefill launch runs alone
    ("prefill-only", [3000, 1024], [1024, 1024], 32, 8, 128, torch.bfloat16),
    # chunks whose bounds leave room for decodes that are not there: the one
    # launch's decode waves find nothing
    ("prefill-only-loose", [3000, 1024, 300], [1024, 6, 6], 32, 8, 128, torch.bfloat16),
    ("g16-chunk", [1200, 90, 3000], [1, 1, 33], 16, 1, 128, torch.bfloat16),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_split(case):
    name, lens, ql, hq, hkv, D, dtype = case
    _check(W.build_step(name, lens, ql, hq, hkv, D, dtype, 7000 + len(name)), name)


@pytest.mark.gpu
def test_plan_kernel_and_long_context():
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 300, size=600).tolist()
    ql = [2 if (i % 5 == 1 and L >= 2) else 1 for i, L in enumerate(lens)]
    lens[9], ql[9] = 500, 130
    _check(W.build_step("600-seqs", lens, ql, 16, 4, 64, torch.bfloat16, 7101), "600 sequences")
    _check(W.build_step("long-context", [100000, 70001], [40, 1], 4, 1, 64, torch.bfloat16, 7102),
           "contexts past 65,536 keys")


@pytest.mark.gpu
def test_fused_step_graph_replays_bitwise(monkeypatch):
    monkeypatch.delenv("PKV_CHECK", raising=False)  # host checks would synchronise
    import paged_kv_attention_03_amd as pkv
    st = W.config_step(3)
    q = st.make_q("cpu").cuda()
    kp, vp = gpu_pools(st, "cpu")
    md = st.metadata("cuda")
    need = pkv.pkv_attention_workspace_size(st.num_seqs, st.total_q, st.max_seqlen_q,
                                            st.max_seqlen_k, st.num_q_heads, st.num_kv_heads,
                                            st.head_dim, 16, st.dtype)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call(out):
        pkv.pkv_attention(q, kp, vp, md["block_tables"], md["seq_lens"], md["query_start_loc"],
                          st.scale, max_seqlen_q=st.max_seqlen_q, max_seqlen_k=st.max_seqlen_k,
                          out=out, workspace=ws)

    def run():
        eager = torch.empty_like(q)
        call(eager)
        torch.cuda.synchronize()
        out = torch.zeros_like(q)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(out)  # warm-up on a side stream, as torch asks before a capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call(out)
        torch.cuda.synchronize()
        noise = torch.randn(512, 512, device="cuda")
        for rep in range(4):
            out.zero_()
            noise = noise @ noise.T / 512.0  # unrelated eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(raw_bits(out), raw_bits(eager)), f"replay {rep}"
        return eager

    fused = _with_mode("fused", run)
    split = _with_mode("split", lambda: gpu_attention(st, q, kp, vp))
    assert np.array_equal(raw_bits(fused), raw_bits(split))
