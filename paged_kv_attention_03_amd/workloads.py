"""Seeded synthetic inputs for one packed engine step over a paged KV pool.

This module builds inputs only: lengths, per-sequence key/value rows drawn
from N(0, 1), shuffled physical pages, block tables, slot mappings and the
optional left-padded (uniform-offset) layout.  It holds none of the attention
arithmetic and is shared by the tests, the benchmark and the smoke check; both
the HIP path and the float64 oracle consume what it returns.

Shapes follow the workloads the pages describe (an agent split averaging 4.6K
input tokens, 70 output tokens, a 512-token shared prefix, 16 concurrent
requests; chunked prefill sharing a step with decodes).  Concrete draws:

* lengths come from ``numpy.random.default_rng(seed)``;
* every tensor comes from its own ``torch.Generator`` seeded with
  ``seed + stream`` (q: +1, shared prefix K/V: +3/+4, sequence s K/V:
  +10000+s / +20000+s), drawn in float32 and rounded to the working dtype,
  on the device the caller names;
* physical pages are a seeded permutation of the pool;
* pool bytes that hold no valid row are NaN in correctness runs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

BLOCK_SIZE = 16

CONFIG_NAMES = {
    1: "tiny-decode",
    2: "decode-16seq",
    3: "mixed-chunked-prefill",
    4: "agent-shared-prefix",
    5: "large-decode-128seq",
}


def _gen(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev.type if dev.type != "cuda" else dev)
    g.manual_seed(int(seed))
    return g


def randn(shape, seed: int, device, dtype) -> torch.Tensor:
    """N(0,1) drawn in float32 from a generator seeded with ``seed``, rounded
    to ``dtype`` (round to nearest even for bfloat16)."""
    g = _gen(seed, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


@dataclass
class StepInputs:
    """Everything one step needs, plus the recipe to regenerate any sequence."""
    name: str
    seed: int
    device: str
    dtype: torch.dtype
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    seq_lens: List[int]            # keys per sequence, this step's tokens included
    q_lens: List[int]              # query tokens per sequence in this step
    kv_start: Optional[List[int]]  # leading masked keys (left-padded layout) or None
    block_tables: np.ndarray       # [S, max_blocks] int32 (host copy)
    # token index (within the sequence's own rows) -> slot, per sequence; a
    # left-padded layout stores the same rows, shifted by the padding
    token_slots: List[np.ndarray] = field(default_factory=list)
    shared_prefix: int = 0
    poison: bool = True
    shared_pages: List[int] = field(default_factory=list)

    # ---- derived metadata ----
    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def real_lens(self) -> List[int]:
        ks = self.kv_start or [0] * self.num_seqs
        return [L - a for L, a in zip(self.seq_lens, ks)]

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))

    @property
    def max_seqlen_q(self) -> int:
        return int(max(self.q_lens)) if self.q_lens else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(max(self.seq_lens)) if self.seq_lens else 0

    def query_start_loc(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    def metadata(self, device=None):
        dev = device or self.device
        ks = None
        if self.kv_start is not None:
            ks = torch.tensor(self.kv_start, dtype=torch.int32, device=dev)
        return dict(
            block_tables=torch.from_numpy(self.block_tables).to(dev),
            seq_lens=torch.tensor(self.seq_lens, dtype=torch.int32, device=dev),
            query_start_loc=torch.from_numpy(self.query_start_loc()).to(dev),
            kv_start=ks,
        )

    # ---- per-sequence rows ----
    def seq_kv(self, s: int, device=None):
        """Real key/value rows of sequence s, [real_len, Hkv, D] each."""
        dev = device or self.device
        n = self.real_lens[s]
        shp = (self.num_kv_heads, self.head_dim)
        P = min(self.shared_prefix, n)
        parts_k, parts_v = [], []
        if P > 0:
            parts_k.append(randn((self.shared_prefix,) + shp, self.seed + 3, dev, self.dtype)[:P])
            parts_v.append(randn((self.shared_prefix,) + shp, self.seed + 4, dev, self.dtype)[:P])
        rest = n - P
        if rest > 0:
            parts_k.append(randn((rest,) + shp, self.seed + 10000 + s, dev, self.dtype))
            parts_v.append(randn((rest,) + shp, self.seed + 20000 + s, dev, self.dtype))
        if not parts_k:
            z = torch.empty((0,) + shp, dtype=self.dtype, device=dev)
            return z, z.clone()
        return torch.cat(parts_k, 0), torch.cat(parts_v, 0)

    def new_pool(self, device=None, poison: Optional[bool] = None):
        dev = device or self.device
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        fill = float("nan") if (self.poison if poison is None else poison) else 0.0
        return (torch.full(shape, fill, dtype=self.dtype, device=dev),
                torch.full(shape, fill, dtype=self.dtype, device=dev))

    def rows(self, which: str, device=None, seqs: Optional[Sequence[int]] = None,
             gen_device=None):
        """Concatenated (k, v, slot_mapping) of the rows written before the step
        (``which='fill'``) or by the step itself (``which='step'``).  Shared
        prefix rows are written once, by the first sequence that holds them.
        Rows are drawn on ``gen_device`` (default: ``device``) and placed on
        ``device``."""
        dev = device or self.device
        gdev = gen_device or dev
        ks, vs, sl = [], [], []
        written_prefix = False
        for s in (range(self.num_seqs) if seqs is None else seqs):
            n = self.real_lens[s]
            qn = self.q_lens[s]
            lo, hi = (0, n - qn) if which == "fill" else (n - qn, n)
            if hi <= lo:
                continue
            k, v = self.seq_kv(s, gdev)
            idx = np.arange(lo, hi)
            if self.shared_prefix > 0:
                if written_prefix:
                    idx = idx[idx >= self.shared_prefix]
                if lo < self.shared_prefix:
                    written_prefix = True
            if idx.size == 0:
                continue
            sel = torch.from_numpy(idx).to(gdev)
            ks.append(k.index_select(0, sel).to(dev))
            vs.append(v.index_select(0, sel).to(dev))
            sl.append(self.token_slots[s][idx])
        shp = (0, self.num_kv_heads, self.head_dim)
        if not ks:
            e = torch.empty(shp, dtype=self.dtype, device=dev)
            return e, e.clone(), torch.empty((0,), dtype=torch.int64, device=dev)
        slots = torch.from_numpy(np.concatenate(sl).astype(np.int64)).to(dev)
        return torch.cat(ks, 0), torch.cat(vs, 0), slots

    def make_q(self, device=None, gen_device=None):
        dev = device or self.device
        return randn((self.total_q, self.num_q_heads, self.head_dim), self.seed + 1,
                     gen_device or dev, self.dtype).to(dev)


def _assign_pages(real_lens, kv_pad, block_size, free, shared_prefix, max_blocks):
    """Block tables and per-token slots.  ``free`` is the shuffled free list
    (consumed from the front).  With ``kv_pad`` (left padding) sequence s's
    token j sits at padded position kv_pad[s] + j and pages that hold only
    padding all point to ``poison_page``."""
    S = len(real_lens)
    bt = np.full((S, max_blocks), -1, dtype=np.int32)
    token_slots = []
    shared_pages = []
    pos = 0
    if shared_prefix > 0:
        npg = (shared_prefix + block_size - 1) // block_size
        if shared_prefix % block_size != 0:
            raise ValueError("shared prefix must fill whole pages")
        shared_pages = [int(x) for x in free[pos:pos + npg]]
        pos += npg
    poison_page = None
    for s in range(S):
        pad = kv_pad[s] if kv_pad is not None else 0
        n = real_lens[s]
        total = pad + n
        npages = (total + block_size - 1) // block_size
        for p in range(npages):
            if (p + 1) * block_size <= pad:
                if poison_page is None:
                    poison_page = int(free[pos])
                    pos += 1
                bt[s, p] = poison_page
            elif shared_prefix > 0 and p < len(shared_pages) and pad == 0:
                bt[s, p] = shared_pages[p]
            else:
                bt[s, p] = int(free[pos])
                pos += 1
        j = np.arange(n, dtype=np.int64) + pad
        token_slots.append(bt[s, j // block_size].astype(np.int64) * block_size + j % block_size)
    return bt, token_slots, shared_pages, pos


def build_step(name: str, ctx_lens: Sequence[int], q_lens: Sequence[int], num_q_heads: int,
               num_kv_heads: int, head_dim: int, dtype, seed: int, *, device="cpu",
               block_size: int = BLOCK_SIZE, num_blocks: Optional[int] = None,
               pool_factor: float = 1.25, shared_prefix: int = 0, padded: bool = False,
               scale: Optional[float] = None, poison: bool = True, spare_pages: int = 0,
               extra_blocks_per_seq: int = 0, perm_seed: Optional[int] = None) -> StepInputs:
    """One packed step: sequence s has ``ctx_lens[s]`` keys (this step's
    ``q_lens[s]`` tokens included).  With ``padded`` the batch is laid out
    left-padded to the longest sequence (``kv_start`` = padding).
    ``perm_seed`` reshuffles the physical pages without changing any row."""
    real = [int(x) for x in ctx_lens]
    ql = [int(x) for x in q_lens]
    if len(real) != len(ql) or any(q > L for q, L in zip(ql, real)):
        raise ValueError("bad lengths")
    S = len(real)
    rng = np.random.default_rng(seed)
    kv_pad = None
    if padded:
        lmax = max(real) if real else 0
        kv_pad = [lmax - L for L in real]
    tot = [(kv_pad[s] if kv_pad else 0) + real[s] for s in range(S)]
    need = 0
    for s in range(S):
        lo = (kv_pad[s] // block_size) if kv_pad else 0
        need += (tot[s] + block_size - 1) // block_size - lo
    if shared_prefix:
        need -= (S - 1) * (shared_prefix // block_size)
    need += 1 + spare_pages  # a poison page for padded layouts, spares for growth
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * need))
    if num_blocks < need:
        raise ValueError(f"pool of {num_blocks} pages cannot hold {need}")
    free = (rng if perm_seed is None else np.random.default_rng(perm_seed)).permutation(num_blocks)
    max_blocks = max([(t + block_size - 1) // block_size for t in tot] + [1]) + extra_blocks_per_seq
    bt, token_slots, shared_pages, _ = _assign_pages(real, kv_pad, block_size, free,
                                                     shared_prefix, max_blocks)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    st = StepInputs(name=name, seed=seed, device=str(device), dtype=dtype,
                    num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    block_size=block_size, num_blocks=num_blocks, scale=scale,
                    seq_lens=[t for t in tot], q_lens=ql,
                    kv_start=(kv_pad if padded else None), block_tables=bt,
                    token_slots=token_slots, shared_prefix=shared_prefix, poison=poison,
                    shared_pages=shared_pages)
    return st


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def config_step(k: int, *, device="cpu", padded: bool = False, dtype=None,
                poison: bool = True) -> StepInputs:
    """Configs 1, 2, 3 and 5 as one step (config 4 is the multi-step
    :class:`AgentRun`).  ``dtype`` overrides the working dtype (float32
    shadow runs of the bf16 configs)."""
    seed = 1000 * k
    rng = np.random.default_rng(seed)
    if k == 1:
        dt = dtype or torch.float32
        lens = [17, 33, 64, 100]
        return build_step(CONFIG_NAMES[1], lens, [1] * 4, 4, 2, 64, dt, seed, device=device,
                          num_blocks=64, scale=0.125, padded=padded, poison=poison)
    if k == 2:
        dt = dtype or torch.bfloat16
        lens = rng.integers(1024, 4096, size=16, endpoint=True).tolist()
        return build_step(CONFIG_NAMES[2], lens, [1] * 16, 16, 8, 128, dt, seed,
                          device=device, padded=padded, poison=poison)
    if k == 3:
        dt = dtype or torch.bfloat16
        lens = rng.integers(3072, 6144, size=16, endpoint=True).tolist()
        ql = [1] * 16
        # two 512-token prefill chunks whose first token sits at position
        # 4608 (page aligned) and 4601 (mid page)
        for idx, off in ((3, 4608), (10, 4601)):
            lens[idx] = off + 512
            ql[idx] = 512
        return build_step(CONFIG_NAMES[3], lens, ql, 32, 8, 128, dt, seed, device=device,
                          padded=padded, poison=poison)
    if k == 5:
        dt = dtype or torch.bfloat16
        lens = rng.integers(4096, 32768, size=128, endpoint=True).tolist()
        return build_step(CONFIG_NAMES[5], lens, [1] * 128, 64, 8, 128, dt, seed,
                          device=device, padded=padded, poison=poison)
    raise ValueError(f"no single-step config {k}")


def agent_lengths(seed: int = 4000, n: int = 16) -> List[int]:
    """Prompt lengths of the agent workload: lognormal with mean 4600 tokens,
    sigma 0.3, clipped to [528, 8704] (the longest agent prompt is 8.7K)."""
    rng = np.random.default_rng(seed)
    sigma = 0.3
    mu = math.log(4600.0) - sigma * sigma / 2
    t = np.round(rng.lognormal(mu, sigma, size=n)).astype(np.int64)
    return np.clip(t, 528, 8704).tolist()


class AgentRun:
    """Config 4's inputs: 16 sequences whose prompts share a 512-token prefix,
    each growing by one decode token per step for 70 steps (40 q / 8 kv heads,
    head_dim 128, bf16).  Rows, lengths and queries only: which pages hold
    the rows is decided by whoever lays out the pool (the host pool manager in
    the engine loop, or a test's own layout)."""

    def __init__(self, *, steps: int = 70, dtype=None, num_q_heads: int = 40,
                 num_kv_heads: int = 8, head_dim: int = 128,
                 prompt_lens: Optional[Sequence[int]] = None, shared_prefix: int = 512,
                 seed: int = 4000):
        if shared_prefix % BLOCK_SIZE:
            raise ValueError("the shared prefix must fill whole pages")
        self.name = CONFIG_NAMES[4]
        self.steps = steps
        self.dtype = dtype or torch.bfloat16
        self.num_q_heads = num_q_heads
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.prompt = list(prompt_lens) if prompt_lens is not None else agent_lengths(seed)
        if min(self.prompt) < shared_prefix:
            raise ValueError("every prompt must hold the shared prefix")
        self.shared_prefix = shared_prefix
        self.seed = seed
        self.scale = float(np.float32(1.0 / math.sqrt(head_dim)))

    @property
    def num_seqs(self) -> int:
        return len(self.prompt)

    @property
    def final_lens(self) -> List[int]:
        return [p + self.steps for p in self.prompt]

    @property
    def max_seqlen_k(self) -> int:
        return max(self.final_lens)

    def seq_lens_at(self, i: int) -> List[int]:
        """Keys of every sequence in decode step i (0-based), its new token included."""
        return [p + i + 1 for p in self.prompt]

    def seq_kv(self, s: int, device="cpu"):
        """All rows sequence s will hold, [prompt + steps, Hkv, D] each: the
        shared prefix rows first (the same for every sequence), then its own."""
        shp = (self.num_kv_heads, self.head_dim)
        P = self.shared_prefix
        n = self.prompt[s] + self.steps
        k = [randn((P,) + shp, self.seed + 3, device, self.dtype)] if P else []
        v = [randn((P,) + shp, self.seed + 4, device, self.dtype)] if P else []
        k.append(randn((n - P,) + shp, self.seed + 10000 + s, device, self.dtype))
        v.append(randn((n - P,) + shp, self.seed + 20000 + s, device, self.dtype))
        return torch.cat(k, 0), torch.cat(v, 0)

    def step_q(self, i: int, device="cpu"):
        return randn((self.num_seqs, self.num_q_heads, self.head_dim),
                     self.seed + 1 + 7919 * (i + 1), device, self.dtype)

    def free_order(self, num_blocks: int) -> np.ndarray:
        """The order in which a pool of num_blocks pages hands out its free
        pages: a seeded shuffle (a pool that has served for a while hands out
        pages in no particular order)."""
        return np.random.default_rng(self.seed + 17).permutation(num_blocks).astype(np.int32)
