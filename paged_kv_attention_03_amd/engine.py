"""A decode loop over a pool reserved once: the host pool manager hands out
pages, the device calls write and read them.

This is the host side of an engine step as the pages describe it: the KV pool
is sized once at startup and every request draws its pages from it (vllm-metal
v0.4.0 release post, "Set a predictable memory budget"); requests that share a
prompt prefix hold it in common pages ("Prefix caching on hybrid models"); each
step the scheduler hands the runner slots for the new rows and block tables
("How vllm-metal fits into vLLM"), and the step appends its rows and runs
attention through the tables ("Replacing attention, reusing the rest").

``AgentPlanner`` is host only (the ``pkv_pool_*`` manager: fork for the shared
prefix, one ``append_batch`` per step, block-table export).  ``AgentLoop``
owns the device pools and runs each step: metadata upload, any copy-on-write
page copies (``pkv_copy_blocks``), ``pkv_append`` of the step's rows, then
``pkv_attention``.  With ``graphs`` the device part of every step (metadata
upload, append, attention) is captured once in a HIP graph and replayed
after the step's planning on the host, as an engine captures its decode
step: the launches then cost one graph launch of host time instead of one
binding call each.  Neither holds any attention arithmetic.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np
import torch

from . import PagePool, pkv_append, pkv_attention, pkv_attention_shared_prefix, \
    pkv_attention_shared_prefix_workspace_size, pkv_attention_workspace_size, pkv_copy_blocks, \
    prepare_append, prepare_attention

BLOCK_SIZE = 16


@dataclass
class StepPlan:
    """Host metadata of one decode step."""
    slots: np.ndarray                 # [S] int64, the new token's slot per sequence
    copies: List[Tuple[int, int]]     # copy-on-write page copies to run first
    table: np.ndarray                 # [S, width] int32 block tables (-1 past the pages)
    lens: np.ndarray                  # [S] int32 keys per sequence, new token included


class AgentPlanner:
    """Pool-manager bookkeeping of the agent workload (``workloads.AgentRun``).

    With ``share_prefix`` the first sequence's prompt prefix is written once
    and every other sequence is forked from it (its prefix pages held in
    common); otherwise every sequence holds its own copy.  The pool holds
    ``pool_factor`` x the pages the whole run needs and hands out its free
    pages in the run's seeded order."""

    def __init__(self, run, share_prefix: bool = True, pool_factor: float = 1.25):
        self.run = run
        self.share = share_prefix and run.shared_prefix > 0
        S = run.num_seqs
        bs = BLOCK_SIZE
        need = sum((n + bs - 1) // bs for n in run.final_lens)
        if self.share:
            need -= (S - 1) * (run.shared_prefix // bs)
        self.num_blocks = int(math.ceil(pool_factor * need))
        self.width = (run.max_seqlen_k + bs - 1) // bs
        self.pool = PagePool(self.num_blocks, bs, S, self.width)
        self.pool.set_free_order(run.free_order(self.num_blocks))
        self.seqs = list(range(S))
        self.shared_pages: List[int] = []

    def prefill(self):
        """Pages for every prompt.  Returns [(seq, lo, hi, slots)]: rows lo..hi
        of sequence seq go to ``slots`` (the shared prefix is listed once)."""
        run, pool = self.run, self.pool
        P = run.shared_prefix if self.share else 0
        segs = []
        if self.share:
            pool.add_seq(0)
            slots, _ = pool.append(0, P)
            segs.append((0, 0, P, slots))
            for s in self.seqs[1:]:
                pool.fork(0, s, P)
            table, _ = pool.block_tables([0], self.width)
            self.shared_pages = [int(b) for b in table[0][:P // BLOCK_SIZE]]
        else:
            for s in self.seqs:
                pool.add_seq(s)
        counts = [run.prompt[s] - P for s in self.seqs]
        slots, copies = pool.append_batch(self.seqs, counts)
        assert not copies  # the prefix fills whole pages
        at = 0
        for s, c in zip(self.seqs, counts):
            segs.append((s, P, P + c, slots[at:at + c]))
            at += c
        return segs

    def step(self, i: int) -> StepPlan:
        """Decode step i: one new token per sequence."""
        slots, copies = self.pool.append_batch(self.seqs, [1] * len(self.seqs))
        table, lens = self.pool.block_tables(self.seqs, self.width)
        return StepPlan(slots=slots, copies=copies, table=table, lens=lens)

    def close(self):
        self.pool.close()


class AgentLoop:
    """The agent workload on the device, driven by an :class:`AgentPlanner`.

    Every row the run will append is generated on ``gen_device`` up front (the
    model's projections would produce them; they are inputs), so a step's
    device work is the upload of its metadata, the append and attention.
    Pool bytes no row was written to hold NaN when ``poison``.

    ``lookahead`` K: the host plans K steps at a time and uploads their
    metadata with one copy (a decode step appends one token per sequence
    whatever the token is, so its slots and block tables are known before the
    steps ahead of it run); each step then launches its own append and
    attention.  ``graphs`` (with K = 1): each step's upload, append and
    attention are one captured HIP graph, replayed after its planning."""

    def __init__(self, run, planner: AgentPlanner, *, poison: bool = True, gen_device="cuda",
                 prefix_pass: Optional[str] = None, graphs: bool = False, lookahead: int = 1):
        if lookahead < 1 or (graphs and lookahead != 1):
            raise ValueError("lookahead must be >= 1, and 1 with graphs")
        self.run, self.plan = run, planner
        self.K = lookahead
        dev = torch.device("cuda")
        shape = (planner.num_blocks, run.num_kv_heads, BLOCK_SIZE, run.head_dim)
        fill = float("nan") if poison else 0.0
        self.kp = torch.full(shape, fill, dtype=run.dtype, device=dev)
        self.vp = torch.full(shape, fill, dtype=run.dtype, device=dev)
        S = run.num_seqs
        self.rows = [run.seq_kv(s, gen_device) for s in range(S)]
        # prefill rows through pkv_append
        ks, vs, sl = [], [], []
        for s, lo, hi, slots in planner.prefill():
            k, v = self.rows[s]
            ks.append(k[lo:hi].to(dev))
            vs.append(v[lo:hi].to(dev))
            sl.append(slots)
        pkv_append(torch.cat(ks), torch.cat(vs), self.kp, self.vp,
                   torch.from_numpy(np.concatenate(sl).astype(np.int64)).to(dev))
        # the step's rows and queries, resident on the device
        self.step_k, self.step_v, self.step_q = [], [], []
        for i in range(run.steps):
            pos = [p + i for p in run.prompt]
            self.step_k.append(torch.stack([self.rows[s][0][pos[s]] for s in range(S)]).to(dev))
            self.step_v.append(torch.stack([self.rows[s][1][pos[s]] for s in range(S)]).to(dev))
            self.step_q.append(run.step_q(i, gen_device).to(dev))
        self.qsl = torch.arange(S + 1, dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.step_q[0])
        self.prefix_pass = prefix_pass
        if prefix_pass is not None:
            self.group = torch.zeros(S, dtype=torch.int32, device=dev)
            self.plen = torch.tensor([run.shared_prefix], dtype=torch.int32, device=dev)
            need = pkv_attention_shared_prefix_workspace_size(
                S, S, 1, run.max_seqlen_k, run.num_q_heads, run.num_kv_heads, run.head_dim,
                BLOCK_SIZE, run.dtype, num_groups=1, max_group_size=S,
                max_prefix_len=run.shared_prefix)
        else:
            need = pkv_attention_workspace_size(S, S, 1, run.max_seqlen_k, run.num_q_heads,
                                                run.num_kv_heads, run.head_dim, BLOCK_SIZE,
                                                run.dtype)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        # step metadata, one set per step (slots int64 [S] | lens int32 [S] |
        # table int32 [S, W] | copy-on-write pairs int32 [2, S]); two halves of
        # K sets, each a pinned host buffer and a device buffer uploaded with
        # one copy, used by alternate groups of K steps (a half is refilled
        # only after the copy that read it two groups ago ended)
        W = planner.width
        nbytes = 8 * S + 4 * S + 4 * S * W + 8 * S
        nbytes = (nbytes + 255) // 256 * 256
        self._raw = [(torch.empty(self.K * nbytes, dtype=torch.uint8).pin_memory(),
                      torch.empty(self.K * nbytes, dtype=torch.uint8, device=dev))
                     for _ in range(2)]

        def views(buf, k):
            b = buf[k * nbytes:(k + 1) * nbytes]
            o1, o2, o3 = 8 * S, 12 * S, 12 * S + 4 * S * W
            return dict(slots=b[:o1].view(torch.int64), lens=b[o1:o2].view(torch.int32),
                        table=b[o2:o3].view(torch.int32).view(S, W),
                        cow=b[o3:o3 + 8 * S].view(torch.int32).view(2, S))

        self._h = [[views(h, k) for k in range(self.K)] for h, _ in self._raw]
        self._d = [[views(d, k) for k in range(self.K)] for _, d in self._raw]
        self._ev = [None, None]
        self._ev_obj = [torch.cuda.Event(), torch.cuda.Event()]
        self._chunk = []
        self._graphs = None
        # each step's append and attention, checked once, on its metadata set
        self._app, self._att = [], []
        for i in range(run.steps):
            d = self._set(self._d, i)
            self._app.append(prepare_append(self.step_k[i], self.step_v[i], self.kp, self.vp,
                                            d["slots"]))
            if prefix_pass is None:
                self._att.append(prepare_attention(
                    self.step_q[i], self.kp, self.vp, d["table"], d["lens"], self.qsl,
                    run.scale, max_seqlen_q=1, max_seqlen_k=run.max_seqlen_k, out=self.out,
                    workspace=self.ws))
        torch.cuda.synchronize()
        if graphs:
            self._capture()

    def _set(self, sets, i: int):
        """Metadata set of step i: half (i // K) % 2, entry i % K."""
        c, k = divmod(i, self.K)
        return sets[c % 2][k]

    def _upload(self, h: int):
        self._raw[h][1].copy_(self._raw[h][0], non_blocking=True)

    def _fill(self, hs, plan: StepPlan):
        hs["slots"].numpy()[:] = plan.slots
        hs["table"].numpy()[:] = plan.table
        hs["lens"].numpy()[:] = plan.lens
        n = len(plan.copies)
        if n:
            hs["cow"].numpy()[:, :n] = np.array(plan.copies, dtype=np.int32).T

    def _compute(self, i: int, ev=None, prepared: bool = True):
        """Append of step i's rows and attention, on its metadata set."""
        run, d = self.run, self._set(self._d, i)
        if prepared:
            self._app[i]()
        else:
            pkv_append(self.step_k[i], self.step_v[i], self.kp, self.vp, d["slots"])
        if ev is not None:
            ev[0].record()
        if prepared and self._att:
            self._att[i]()
        elif self.prefix_pass is not None:
            pkv_attention_shared_prefix(
                self.step_q[i], self.kp, self.vp, d["table"], d["lens"], self.qsl, run.scale,
                self.group, self.plen, max_group_size=run.num_seqs,
                max_prefix_len=run.shared_prefix, max_seqlen_q=1, max_seqlen_k=run.max_seqlen_k,
                out=self.out, workspace=self.ws, prefix_pass=self.prefix_pass)
        else:
            pkv_attention(self.step_q[i], self.kp, self.vp, d["table"], d["lens"], self.qsl,
                          run.scale, max_seqlen_q=1, max_seqlen_k=run.max_seqlen_k, out=self.out,
                          workspace=self.ws)
        if ev is not None:
            ev[1].record()

    def _capture(self):
        """One graph per step index: upload of the step's metadata half (K is
        1: the host fills its pinned half before the replay), append and
        attention, all on the capturing stream (plain calls: prepared ones
        hold the stream they were prepared on).  A warm-up per half first, on
        metadata that is valid as it stands: every slot -1 (the append writes
        nothing) and the block tables and lengths the pool holds after the
        prompts."""
        run, S = self.run, self.run.num_seqs
        table, lens = self.plan.pool.block_tables(list(range(S)), self.plan.width)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for h in range(2):
                hs = self._h[h][0]
                hs["slots"].numpy()[:] = -1
                hs["table"].numpy()[:] = table
                hs["lens"].numpy()[:] = lens
                self._upload(h)
                self._compute(h, prepared=False)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self._graphs = []
        for i in range(run.steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._upload(i % 2)
                self._compute(i, prepared=False)
            self._graphs.append(g)
        torch.cuda.synchronize()

    def step(self, i: int, ev=None) -> torch.Tensor:
        """Runs decode step i (host planning, upload, copies, append,
        attention) and returns ``out`` [S, Hq, D] (overwritten by the next
        step).  ``ev``: optional (start, end) CUDA events around attention.
        Steps run in order from 0."""
        c, k = divmod(i, self.K)
        h = c % 2
        if k == 0:
            # plan this group of steps and upload its metadata
            if self._ev[h] is not None:
                self._ev[h].synchronize()
            last = min(i + self.K, self.run.steps)
            self._chunk = [self.plan.step(j) for j in range(i, last)]
            for kk, plan in enumerate(self._chunk):
                self._fill(self._h[h][kk], plan)
            if self._graphs is not None and not self._chunk[0].copies:
                if ev is not None:
                    raise ValueError("per-call events are not available in graph mode")
                self._graphs[i].replay()
                e = self._ev_obj[h]
                e.record()
                self._ev[h] = e
                return self.out
            self._upload(h)
            e = self._ev_obj[h]
            e.record()
            self._ev[h] = e
        plan = self._chunk[k]
        n = len(plan.copies)
        if n:  # (in graph mode such a step runs eagerly: the copies land before the append)
            d = self._d[h][k]
            pkv_copy_blocks(self.kp, self.vp, d["cow"][0, :n].contiguous(),
                            d["cow"][1, :n].contiguous())
        self._compute(i, ev)
        return self.out
