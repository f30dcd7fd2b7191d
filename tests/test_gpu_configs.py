"""The five workloads at full size on the GPU, against the float64 oracle.

1 tiny decode (fp32), 2 decode-only step, 3 mixed chunked-prefill step,
4 the 70-step agent loop over a shared 512-token prefix, 5 the 128-sequence
large decode (ragged and left-padded to a common offset).  The bf16 runs use
atol = rtol = 1e-2; float32 "shadow" runs of the same shapes use 1e-5, which a
single leaked or dropped key would break.  Configs 1-4 are checked on every
output; config 5 on sampled sequences (all heads), the longest and shortest
among them, plus the left-padded run against the ragged one everywhere."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_03_amd as pkv
from paged_kv_attention_03_amd import workloads as W
from tests.gpu_helpers import (TOL, check_close, gpu_attention, gpu_pools, log, oracle_seq_outputs,
                               raw_bits)
from tests.helpers import close, oracle_pools, oracle_step


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.gpu
@pytest.mark.parametrize("k,dtype", [(1, None), (2, None), (3, None), (2, torch.float32),
                                     (3, torch.float32)],
                         ids=["c1-f32", "c2-bf16", "c3-bf16", "c2-f32-shadow", "c3-f32-shadow"])
def test_config_full(k, dtype):
    st = W.config_step(k, dtype=dtype)
    log(f"config {k} {st.name} dtype={st.dtype} seqs={st.num_seqs} total_q={st.total_q} "
        f"keys={sum(st.seq_lens)}")
    q = st.make_q("cpu")
    kp, vp = gpu_pools(st, "cpu")
    okp, ovp = oracle_pools(st)
    assert np.array_equal(raw_bits(kp), okp.view(raw_bits(kp).dtype))
    assert np.array_equal(raw_bits(vp), ovp.view(raw_bits(vp).dtype))
    out = gpu_attention(st, q.cuda(), kp, vp)
    ref = oracle_step(st, q, pools=(okp, ovp))
    check_close(out, ref, st.dtype, f"config {k}")
    del kp, vp, out
    _free()


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32-shadow"])
def test_config4_agent_loop(dtype):
    run = W.AgentRun(dtype=dtype)
    b = run.base
    log(f"config 4 agent loop dtype={dtype} prompts={run.prompt} pages={b.num_blocks}")
    kp, vp = b.new_pool("cuda")
    k, v, s = run.prefill_rows("cpu")
    pkv.pkv_append(k.cuda(), v.cuda(), kp, vp, s.cuda())
    okp, ovp = oracle.oracle_append(*b.new_pool("cpu"), k, v, s)
    shared = torch.tensor(run.shared_pages, device="cuda")
    shared_before = (raw_bits(kp[shared]).copy(), raw_bits(vp[shared]).copy())
    qsl = torch.arange(b.num_seqs + 1, dtype=torch.int32, device="cuda")
    check_steps = {0, 1, 2, 17, 34, 51, 68, 69} if dtype == torch.bfloat16 else {0, 33, 69}
    ws = None
    for i in range(run.steps):
        pos, slots, bt, sl = run.step(i)
        assert not set(slots // 16) & set(run.shared_pages)
        kn, vn = run.step_rows(i, "cpu")
        pkv.pkv_append(kn.cuda(), vn.cuda(), kp, vp, torch.from_numpy(slots).cuda())
        okp, ovp = oracle.oracle_append(okp, ovp, kn, vn, slots)
        q = run.step_q(i, "cpu")
        if ws is None:
            need = pkv.pkv_attention_workspace_size(b.num_seqs, b.num_seqs, 1, max(run.prompt) + 70,
                                                    b.num_q_heads, b.num_kv_heads, b.head_dim,
                                                    16, dtype)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        out = pkv.pkv_attention(q.cuda(), kp, vp, torch.from_numpy(bt).cuda(),
                                torch.tensor(sl, dtype=torch.int32, device="cuda"), qsl, b.scale,
                                max_seqlen_q=1, max_seqlen_k=max(run.prompt) + 70, workspace=ws)
        if i in check_steps:
            torch.cuda.synchronize()
            ref = oracle.oracle_attention(q, okp, ovp, bt, sl, np.arange(b.num_seqs + 1), b.scale)
            check_close(out, ref, dtype, f"step {i}")
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(kp), okp.view(raw_bits(kp).dtype)), "pool bytes after 70 steps"
    assert np.array_equal(raw_bits(vp), ovp.view(raw_bits(vp).dtype))
    assert np.array_equal(raw_bits(kp[shared]), shared_before[0]), "shared prefix pages changed"
    assert np.array_equal(raw_bits(vp[shared]), shared_before[1])
    del kp, vp
    _free()


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32-shadow"])
def test_config5_large_decode_ragged_and_padded(dtype):
    rag = W.config_step(5, dtype=dtype)
    pad = W.config_step(5, dtype=dtype, padded=True)
    lens = rag.seq_lens
    log(f"config 5 dtype={dtype} keys={sum(lens)} pages={rag.num_blocks} "
        f"max={max(lens)} min={min(lens)}")
    q = rag.make_q("cuda")
    kp, vp = gpu_pools(rag, "cuda")
    out_rag = gpu_attention(rag, q, kp, vp)
    log("  ragged step done")
    del kp, vp
    _free()
    kp, vp = gpu_pools(pad, "cuda")
    out_pad = gpu_attention(pad, q, kp, vp)
    log(f"  padded step done (kv_start up to {max(pad.kv_start)})")
    del kp, vp
    _free()
    sample = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 0, 77})
    ref = oracle_seq_outputs(rag, q.cpu(), sample, "cuda")
    for s in sample:
        check_close(out_rag[s:s + 1], ref[s], dtype, f"ragged seq {s} (L={lens[s]})")
        check_close(out_pad[s:s + 1], ref[s], dtype, f"padded seq {s}")
    # padded == ragged on every output, to the same tolerance
    atol, rtol = TOL[dtype]
    ok, err = close(out_pad.float().cpu().numpy(), out_rag.float().cpu().numpy().astype(np.float64),
                    atol, rtol)
    log(f"  padded vs ragged, all 128 sequences: max|diff| {err:.3e}")
    assert ok
