"""pkv_append + pkv_attention captured in a HIP graph (torch.cuda.CUDAGraph on
ROCm) and replayed: the calls only enqueue kernels on the caller's stream and
allocate nothing, so a captured step replays with the same results.  Every
replay is checked bit for bit against the eager call, with eager work and
synchronisations between the replays; the eager result itself is checked
against the float64 oracle."""
import numpy as np
import pytest
import torch

import paged_kv_attention_03_amd as pkv
from paged_kv_attention_03_amd import workloads as W
from tests.gpu_helpers import check_close, gpu_pools, log, raw_bits
from tests.helpers import oracle_pools, oracle_step

CASES = [
    # decodes, a verify window and two prefill chunks (decode and prefill kernels)
    ("graph-mixed", [100, 40, 300, 2000, 1500, 700], [1, 24, 1, 3, 200, 1], 32, 8),
    # 600 decode sequences: the plan kernel takes the work split
    ("graph-600seq", [17 + 3 * (i % 50) for i in range(600)], [1] * 600, 16, 8),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_step_replays_from_a_graph(case, monkeypatch):
    monkeypatch.delenv("PKV_CHECK", raising=False)  # host checks would synchronise
    name, lens, ql, hq, hkv = case
    log(f"graph replay: {name}, {len(lens)} sequences")
    st = W.build_step(name, lens, ql, hq, hkv, 128, torch.bfloat16, 515)
    q = st.make_q("cuda")
    kp, vp = gpu_pools(st)
    k, v, slots = st.rows("step", "cuda", gen_device="cpu")  # the rows gpu_pools wrote
    md = st.metadata("cuda")
    need = pkv.pkv_attention_workspace_size(st.num_seqs, st.total_q, st.max_seqlen_q,
                                            st.max_seqlen_k, hq, hkv, 128, 16, torch.bfloat16)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step(out):
        pkv.pkv_append(k, v, kp, vp, slots)
        pkv.pkv_attention(q, kp, vp, md["block_tables"], md["seq_lens"], md["query_start_loc"],
                          st.scale, max_seqlen_q=st.max_seqlen_q, max_seqlen_k=st.max_seqlen_k,
                          kv_start=md["kv_start"], out=out, workspace=ws)

    eager = torch.empty_like(q)
    step(eager)
    torch.cuda.synchronize()
    okp, ovp = oracle_pools(st)
    ref = oracle_step(st, q.cpu(), pools=(okp, ovp))
    check_close(eager, ref, torch.bfloat16, f"{name} eager")

    out = torch.zeros_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)  # warm-up on the capture stream's side, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out)
    torch.cuda.synchronize()

    noise = torch.randn(512, 512, device="cuda")
    want = raw_bits(eager)
    for rep in range(4):
        out.zero_()
        noise = noise @ noise.T / 512.0  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(raw_bits(out), want), f"{name}: replay {rep} differs from eager"
    assert np.array_equal(raw_bits(kp), okp.view(raw_bits(kp).dtype)), "pool bytes changed"
    log(f"graph replay: {name} ok (4 replays bitwise equal to eager)")


@pytest.mark.gpu
def test_shared_prefix_step_replays_from_a_graph(monkeypatch):
    # the setup kernel hands out member slots by atomics, so replays may place
    # members in other rows of the prefix tiles; the output must not change
    monkeypatch.delenv("PKV_CHECK", raising=False)
    from tests.test_gpu_shared_prefix import build
    st = build([(512, [513 + 37 * i for i in range(16)]), (64, [65, 300])], [(200, 1), (90, 24)],
               40, 8, 128, torch.bfloat16, 31)
    log("graph replay: shared-prefix step")
    q = st["q"].cuda()
    kp, vp = st["kp"].cuda(), st["vp"].cuda()
    bt, lens, qsl = (torch.from_numpy(st[k]).cuda() for k in ("bt", "lens", "qsl"))
    grp, plen = torch.from_numpy(st["group"]).cuda(), torch.from_numpy(st["plen"]).cuda()
    mq, mk = max(st["qlens"]), int(st["lens"].max())
    need = pkv.pkv_attention_shared_prefix_workspace_size(
        len(st["lens"]), q.shape[0], mq, mk, 40, 8, 128, 16, torch.bfloat16, num_groups=2,
        max_group_size=16, max_prefix_len=512)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call(out):
        pkv.pkv_attention_shared_prefix(q, kp, vp, bt, lens, qsl, st["scale"], grp, plen,
                                        max_group_size=16, max_prefix_len=512, max_seqlen_q=mq,
                                        max_seqlen_k=mk, out=out, workspace=ws,
                                        prefix_pass="always")

    eager = torch.empty_like(q)
    call(eager)
    torch.cuda.synchronize()
    out = torch.zeros_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    torch.cuda.synchronize()
    want = raw_bits(eager)
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(raw_bits(out), want), f"replay {rep} differs from eager"
    log("graph replay: shared-prefix step ok")
