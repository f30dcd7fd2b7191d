"""pkv_attention_shared_prefix against the float64 oracle and against
pkv_attention on the same step.

Steps are built here with several prefix groups: each group's prefix pages are
shared (same physical ids in every member's block table), each member is a
decode with its own keys after the prefix; steps also carry plain decodes,
verify windows and prefill chunks, and members that break the group contract
(computed as plain sequences).  Pools are NaN outside the written rows."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_03_amd as pkv
from paged_kv_attention_03_amd import workloads as W
from tests.gpu_helpers import check_close, log, raw_bits

BS = 16


def build(groups, plain, hq, hkv, D, dtype, seed):
    """groups: [(prefix_len, [member keys, or (keys, query tokens)])]; plain:
    [(keys, query tokens)].  Returns host tensors of the step and its group
    arrays."""
    rng = np.random.default_rng(seed)
    seqs = []  # (keys, q_len, group, prefix_len)
    for g, (P, lens) in enumerate(groups):
        for L in lens:
            L, n = (L, 1) if isinstance(L, int) else L
            seqs.append((L, n, g, P))
    for L, n in plain:
        seqs.append((L, n, -1, 0))
    order = rng.permutation(len(seqs))  # members interleaved with other sequences
    seqs = [seqs[i] for i in order]
    need = sum(P // BS for P, _ in groups)
    need += sum((L - P + BS - 1) // BS for L, _, g, P in seqs)
    nb = int(math.ceil(1.25 * need)) + 2
    free = list(rng.permutation(nb))
    gpages = [[int(free.pop()) for _ in range(P // BS)] for P, _ in groups]
    maxb = max((L + BS - 1) // BS for L, _, _, _ in seqs)
    S = len(seqs)
    bt = np.full((S, maxb), -1, np.int32)
    kp = torch.full((nb, hkv, BS, D), float("nan"), dtype=dtype)
    vp = kp.clone()
    shp = (hkv, D)
    gk = [W.randn((P,) + shp, seed + 7 + 2 * g, "cpu", dtype) for g, (P, _) in enumerate(groups)]
    gv = [W.randn((P,) + shp, seed + 8 + 2 * g, "cpu", dtype) for g, (P, _) in enumerate(groups)]
    for g, (P, _) in enumerate(groups):
        slots = np.array([gpages[g][j // BS] * BS + j % BS for j in range(P)], np.int64)
        if P:
            kp, vp = oracle.oracle_append(kp, vp, gk[g], gv[g], slots)
    for s, (L, n, g, P) in enumerate(seqs):
        for pg in range(P // BS):
            bt[s, pg] = gpages[g][pg]
        for pg in range(P // BS, (L + BS - 1) // BS):
            bt[s, pg] = int(free.pop())
        own = L - P
        if own == 0:
            continue
        k = W.randn((own,) + shp, seed + 1000 + s, "cpu", dtype)
        v = W.randn((own,) + shp, seed + 2000 + s, "cpu", dtype)
        j = np.arange(P, L)
        slots = (bt[s, j // BS].astype(np.int64) * BS + j % BS)
        kp, vp = oracle.oracle_append(kp, vp, k, v, slots)
    # the oracle's append returns raw numpy arrays (bfloat16 as int16 bits)
    kp, vp = (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a)).view(dtype)
              for a in (kp, vp))
    qlens = [n for _, n, _, _ in seqs]
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = W.randn((int(qsl[-1]), hq, D), seed + 5, "cpu", dtype)
    return dict(q=q, kp=kp, vp=vp, bt=bt, lens=np.array([L for L, _, _, _ in seqs], np.int32),
                qsl=qsl, group=np.array([g for _, _, g, _ in seqs], np.int32),
                plen=np.array([P for P, _ in groups], np.int32), qlens=qlens,
                scale=float(np.float32(1.0 / math.sqrt(D))))


def run_both(st, max_group_size, max_prefix_len, repeat=1, prefix_pass="always"):
    dev = "cuda"
    q = st["q"].to(dev)
    kp, vp = st["kp"].to(dev), st["vp"].to(dev)
    bt = torch.from_numpy(st["bt"]).to(dev)
    lens = torch.from_numpy(st["lens"]).to(dev)
    qsl = torch.from_numpy(st["qsl"]).to(dev)
    grp = torch.from_numpy(st["group"]).to(dev)
    plen = torch.from_numpy(st["plen"]).to(dev)
    mq, mk = max(st["qlens"]), int(st["lens"].max())
    outs = []
    for _ in range(repeat):
        outs.append(pkv.pkv_attention_shared_prefix(
            q, kp, vp, bt, lens, qsl, st["scale"], grp, plen, max_group_size=max_group_size,
            max_prefix_len=max_prefix_len, max_seqlen_q=mq, max_seqlen_k=mk,
            prefix_pass=prefix_pass))
    plain = pkv.pkv_attention(q, kp, vp, bt, lens, qsl, st["scale"], max_seqlen_q=mq,
                              max_seqlen_k=mk)
    torch.cuda.synchronize()
    ref = oracle.oracle_attention(st["q"], st["kp"], st["vp"], st["bt"], st["lens"], st["qsl"],
                                  st["scale"])
    return outs, plain, ref


CASES = [
    # (name, groups, plain sequences, Hq, Hkv, D, dtype, max_group_size)
    ("agent-16x512", [(512, [512 + 1 + 37 * i for i in range(16)])], [], 40, 8, 128,
     torch.bfloat16, 16),
    ("two-groups-mixed", [(64, [65, 100, 300]), (4096, [4097 + 61 * i for i in range(12)])],
     [(700, 1), (33, 1), (900, 3), (600, 40)], 32, 8, 128, torch.bfloat16, 12),
    ("long-prefix-many-chunks", [(8192, [8192 + 16 * i + 5 for i in range(8)])], [(300, 1)],
     64, 8, 128, torch.bfloat16, 8),
    ("fp32-d64-g2", [(128, [129, 200, 1000]), (32, [40, 33])], [(50, 1), (77, 2)], 4, 2, 64,
     torch.float32, 3),
    ("cap-and-singletons", [(256, [300, 400, 500, 600, 700]), (16, [17])], [(64, 1)], 8, 8, 128,
     torch.bfloat16, 3),
    ("g16-bf16-d64", [(1024, [1025 + 100 * i for i in range(5)])], [], 16, 1, 64, torch.bfloat16,
     8),
    # 600 sequences: the plan kernel splits the decode pass
    ("600-seqs-plan-kernel", [(256, [257 + 7 * (i % 40) for i in range(120)]),
                              (64, [65 + 11 * (i % 30) for i in range(100)]),
                              (1024, [1025 + 13 * (i % 20) for i in range(80)])],
     [(40 + 9 * (i % 50), 1) for i in range(300)], 16, 8, 128, torch.bfloat16, 120),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shared_prefix_step_matches_the_oracle(case):
    name, groups, plain, hq, hkv, D, dtype, mgs = case
    log(f"shared prefix: {name}, groups {[(P, len(m)) for P, m in groups]}, plain {plain}")
    st = build(groups, plain, hq, hkv, D, dtype, 900 + len(name))
    maxp = max(P for P, _ in groups)
    pkv.pkv_check_shared_prefix(st["bt"], st["lens"], st["qsl"], st["group"], st["plen"], BS,
                                maxp)
    outs, plain_out, ref = run_both(st, mgs, maxp, repeat=2)
    check_close(outs[0], ref, dtype, f"{name} shared-prefix")
    check_close(plain_out, ref, dtype, f"{name} plain")
    assert np.array_equal(raw_bits(outs[0]), raw_bits(outs[1])), "runs differ"


@pytest.mark.gpu
def test_members_breaking_the_contract_run_as_plain_sequences():
    # in group 0: a 2-token window and a sequence with no keys past the prefix;
    # pkv_check_shared_prefix rejects the step; the kernels compute both as plain sequences
    st = build([(128, [129, (300, 2), 128, 200]), (32, [33, 90])], [(500, 1)], 16, 4, 128,
               torch.bfloat16, 77)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_check_shared_prefix(st["bt"], st["lens"], st["qsl"], st["group"], st["plen"],
                                    BS, 128)
    outs, plain, ref = run_both(st, 4, 128)
    check_close(outs[0], ref, torch.bfloat16, "contract breakers")
    check_close(plain, ref, torch.bfloat16, "contract breakers, plain")


@pytest.mark.gpu
def test_no_groups_is_plain_attention_bitwise():
    st = build([(64, [65, 80])], [(300, 1), (200, 30)], 32, 8, 128, torch.bfloat16, 5)
    st = dict(st, group=np.full_like(st["group"], -1))
    outs, plain, ref = run_both(st, 2, 64)
    assert np.array_equal(raw_bits(outs[0]), raw_bits(plain))
    check_close(outs[0], ref, torch.bfloat16, "no members")


@pytest.mark.gpu
@pytest.mark.parametrize("prefix,members,expect_pass", [(512, 16, False), (8192, 16, True)],
                         ids=["agent-512x16-plain", "long-8192x16-pass"])
def test_auto_routing_picks_a_path_bitwise(prefix, members, expect_pass):
    # "auto" runs the prefix pass only when the re-reads it avoids reach
    # 256 MiB: 15 x 512 keys x 4 KiB = 31 MB -> the plain path, bitwise equal
    # to pkv_attention; 15 x 8192 keys x 4 KiB = 503 MB -> the prefix pass,
    # bitwise equal to prefix_pass="always"
    st = build([(prefix, [prefix + 1 + 37 * i for i in range(members)])], [], 40, 8, 128,
               torch.bfloat16, 4242 + prefix)
    auto, plain, ref = run_both(st, members, prefix, prefix_pass="auto")
    always, _, _ = run_both(st, members, prefix, prefix_pass="always")
    check_close(auto[0], ref, torch.bfloat16, f"auto {prefix}x{members}")
    same = raw_bits(always[0]) if expect_pass else raw_bits(plain)
    assert np.array_equal(raw_bits(auto[0]), same)
