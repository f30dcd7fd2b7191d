"""pkv_append on the GPU: bit-exact against the oracle's append, including
skipped (negative) slots, untouched bytes, arbitrary bit patterns (NaN and
infinity included) and every supported head_dim / dtype / page size."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_03_amd as pkv
from tests.gpu_helpers import log, raw_bits

CASES = [(dt, d, bs, t) for dt in (torch.float32, torch.bfloat16) for d in (64, 128)
         for bs in (1, 16, 32) for t in (1, 37, 1000)]


def _bits(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    if dtype == torch.bfloat16:
        return torch.randint(-32768, 32767, shape, generator=g, dtype=torch.int16).view(dtype)
    return torch.randint(-2**31, 2**31 - 1, shape, generator=g, dtype=torch.int32).view(dtype)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,bs,T", CASES)
def test_append_bit_exact(dtype, D, bs, T):
    log(f"append dtype={dtype} D={D} bs={bs} T={T}")
    hkv = 4
    nb = max(4, (2 * T + bs - 1) // bs)
    rng = np.random.default_rng(T * 7 + D + bs)
    kp = _bits((nb, hkv, bs, D), dtype, 1)
    vp = _bits((nb, hkv, bs, D), dtype, 2)
    kn = _bits((T, hkv, D), dtype, 3)
    vn = _bits((T, hkv, D), dtype, 4)
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[rng.random(T) < 0.2] = -1
    ek, ev = oracle.oracle_append(kp, vp, kn, vn, slots)
    dkp, dvp = kp.cuda(), vp.cuda()
    pkv.pkv_append(kn.cuda(), vn.cuda(), dkp, dvp, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(dkp), ek.view(raw_bits(dkp).dtype))
    assert np.array_equal(raw_bits(dvp), ev.view(raw_bits(dvp).dtype))


@pytest.mark.gpu
def test_append_of_nothing_is_a_no_op():
    kp = torch.zeros(4, 2, 16, 128, dtype=torch.bfloat16, device="cuda")
    vp = kp.clone()
    e = torch.empty(0, 2, 128, dtype=torch.bfloat16, device="cuda")
    pkv.pkv_append(e, e, kp, vp, torch.empty(0, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert int(kp.abs().sum()) == 0 and int(vp.abs().sum()) == 0


@pytest.mark.gpu
def test_append_skips_slots_outside_the_pool():
    # a slot past the pool is skipped by the kernel (memory-safe), never written
    kp = torch.zeros(2, 1, 16, 64, dtype=torch.float32, device="cuda")
    vp = kp.clone()
    kn = torch.ones(3, 1, 64, device="cuda")
    slots = torch.tensor([0, 32, 31], dtype=torch.int64, device="cuda")
    pkv.pkv_append(kn, kn, kp, vp, slots)
    torch.cuda.synchronize()
    flat = kp.view(32, 64).cpu()
    assert flat[0].eq(1).all() and flat[31].eq(1).all() and flat[1:31].eq(0).all()
