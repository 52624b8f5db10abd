"""Three-tier decode step of hierarchical speculative decoding, composed from
the library's C-ABI calls: Force 1 (a small drafter on a sink + window ring)
drafts, Force 2 (the target on the retrieval-sparse cache) keeps or rejects
each round of drafts, and once gamma2 candidates are collected Force 3 (the
target on the full cache) verifies them in one pass (TriForce blog, "1. The
Three Forces of TriForce"; "2. Dual Rejection Sampling" for both levels of
acceptance).

Every step of the computation runs in the library's kernels; this module only
sequences the calls and keeps the host-side counts.  It drives one sequence
(B = 1): how many Force 2 rounds a step needs depends on how many drafts each
round keeps, so after each round the kept count is read back (8 bytes) and
the host decides whether another round is needed and how many rows each cache
gains or loses.  With graphs=True the call sequences between those reads (the
retrieval, a round, Force 3) are HIP graphs captured before the first step
and replayed.

The models' outputs -- new K/V rows, queries and logits -- are synthetic
device tensors given by the caller (there are no weights here); the control
flow, the cache contents and the lengths are those of the method:

  round (until >= gamma2 candidates): the drafter consumes the committed
    tokens it has not seen and the current token, then its own drafts (one
    ring row per token, streaming attention per drafter layer, sampling from
    its logits with tf_accept at gamma = 0); the target appends the current
    token and the gamma1 drafts to its full cache and attends them over the
    retrieved chunks below a causal tail (tf_sparse_verify_attn); level 1
    tests the drafts against q (tf_accept); tf_collect_candidates appends the
    emitted tokens with their q rows; rejected drafts leave both caches;
  then the full cache is cut (or extended by the last drawn token) to the
    current token plus exactly gamma2 candidates, Force 3 attends them over
    the full cache (tf_verify_attn), level 2 tests them against p
    (tf_accept), the rejected candidates leave both caches, and the chunk
    keys the new rows fell into are refreshed for the next step's retrieval.

Host-side counts, per step (n = committed rows before the current token):
  a round keeps 1 + n1 rows of the target's gamma1 + 1 and 1 + min(n1,
  gamma1 - 1) of the drafter's gamma1 new ones; a kept last draft is one the
  drafter has not consumed (it becomes pending).  After the rounds the target
  holds the current token and the first total - 1 emitted tokens (the chain,
  whose device count stops at gamma2, keeps the first gamma2 of them).
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

from . import _lib as tf


@dataclasses.dataclass
class TargetLayer:
    K: torch.Tensor
    V: torch.Tensor
    kv: "tf.KVDesc"     # seq_len: the step's shared length array; max_len: the rows allocated
    ck: torch.Tensor
    ckd: "tf.KVDesc"    # seq_len: the shared chunk-count array


@dataclasses.dataclass
class DrafterLayer:
    Ks: torch.Tensor
    Vs: torch.Tensor
    sd: "tf.KVDesc"     # seq_len: the drafter's shared logical length array


@dataclasses.dataclass
class Synthetic:
    """The models' outputs: fixed device tensors, reused by every round."""
    draft_q: torch.Tensor          # [1][Hq][d] drafter query (also the retrieval query)
    draft_rows: List[torch.Tensor]  # draft_rows[R - 1]: [1][H][R][d] new drafter K/V rows, R = 1, 2, 3
    r_rows: torch.Tensor           # [1][gamma1][V] drafter logits, one row per draft position
    f2_q: torch.Tensor             # [1][Hq][gamma1 + 1][d]
    f2_rows: torch.Tensor          # [1][H][gamma1 + 1][d]
    q_rows: torch.Tensor           # [1][gamma1 + 1][V] Force 2 logits
    f3_q: torch.Tensor             # [1][Hq][gamma2 + 1][d]
    one_row: torch.Tensor          # [1][H][1][d]
    p_rows: torch.Tensor           # [1][gamma2 + 1][V] Force 3 logits
    uniforms: torch.Tensor         # [U] fp64 in (0, 1), consumed in order (wrapping around)


def drafter_reserve(gamma1: int, gamma2: int) -> int:
    """Rows a step may roll back from the drafter's ring (its slack must be at
    least this): everything it consumed since the step began."""
    return gamma1 + gamma2 + 3


def check_ring(slots_after_sinks: int, window: int, gamma1: int, gamma2: int, layer: int = 0) -> None:
    """Raise unless a drafter ring can take a step's appends: an append to a
    ring with fewer than window + reserve slots after the sinks writes nothing
    (it only sets its status), so the drafter would attend stale rows."""
    need = window + drafter_reserve(gamma1, gamma2)
    if slots_after_sinks < need:
        raise ValueError(f"drafter layer {layer}: ring has {slots_after_sinks} slots after the sinks, needs "
                         f"window + reserve = {need} (gamma1 = {gamma1}, gamma2 = {gamma2})")


def check_room(n: int, gamma1: int, gamma2: int, cap: int) -> None:
    """Raise unless the full cache has room for every row a step starting
    from n committed rows may write.  A round starts at a length below
    n + gamma2 and appends gamma1 + 1 rows, so the deepest row is
    n + gamma1 + gamma2 - 1; an append without room writes nothing."""
    if n + gamma1 + gamma2 > cap:
        raise ValueError(f"full cache: a step from {n} committed rows may write up to row "
                         f"{n + gamma1 + gamma2 - 1}, but only {cap} rows are allocated")


class ThreeTierStep:
    def __init__(self, target: List[TargetLayer], drafter: List[DrafterLayer], syn: Synthetic, *, Hq: int,
                 chunk_size: int, k: int, tail: int, gamma1: int, gamma2: int, n_sink: int, window: int,
                 temperature: float = 1.0, stream: Optional[torch.cuda.Stream] = None, record: bool = False,
                 graphs: bool = False):
        self.t, self.dr, self.syn = target, drafter, syn
        self.record = record      # keep each round's and step's decisions (tests)
        # graphs: the fixed call sequences (retrieval, a round for each count of
        # unseen tokens and chain-count parity, Force 3) are captured once as HIP
        # graphs and replayed; the host still decides the rounds between them
        self.graphs = graphs
        if graphs and stream is None:
            stream = torch.cuda.Stream(target[0].K.device)   # graphs are captured on a side stream
        self._g = {}
        self.log: list = []
        self.Hq, self.cs, self.k, self.tail = Hq, chunk_size, k, tail
        self.g1, self.g2, self.S, self.W = gamma1, gamma2, n_sink, window
        self.T, self.s = temperature, stream
        kv0 = target[0].kv
        dev = target[0].K.device
        V = syn.q_rows.shape[-1]
        self.seq_len = kv0.seq_len                 # shared by every target layer's descriptor
        self.ck_len = target[0].ckd.seq_len        # shared by every chunk-key descriptor
        self.d_len = drafter[0].sd.seq_len         # shared by every drafter layer's descriptor
        self.c_max = target[0].ckd.max_len
        i32 = dict(dtype=torch.int32, device=dev)
        self.scores = torch.empty((1, kv0.H, self.c_max), dtype=torch.float32, device=dev)
        self.idx = [torch.empty((1, kv0.H, k), **i32) for _ in target]
        self.o_d = torch.empty((1, Hq, 128), dtype=torch.float32, device=dev)
        self.o2 = torch.empty((1, Hq, gamma1 + 1, 128), dtype=torch.float32, device=dev)
        self.o3 = torch.empty((1, Hq, gamma2 + 1, 128), dtype=torch.float32, device=dev)
        self.drafts = torch.empty((gamma1, 1), **i32)    # row j: draft j (a contiguous [1] per call)
        self.drafts_row = torch.empty((1, gamma1), **i32)
        self.na_d = torch.empty(1, **i32)
        self.n1, self.y = torch.empty(1, **i32), torch.empty(1, **i32)
        self.n2, self.nxt = torch.empty(1, **i32), torch.empty(1, **i32)
        self.cnt = [torch.zeros(1, **i32), torch.zeros(1, **i32)]
        self.cand = torch.empty((1, gamma2), **i32)
        self.cand_q = torch.empty((1, gamma2, V), dtype=torch.float32, device=dev)
        self.zero = torch.zeros(1, **i32)
        # append status: never read; step() checks on the host, before it
        # enqueues anything, that every append of the step has room
        self.status = torch.empty(1, **i32)
        self.chunk_begin = torch.empty(1, **i32)
        self.host = torch.empty(4, dtype=torch.int32).pin_memory()
        self.ws2 = tf.workspace(tf.sparse_verify_attn_workspace_size(1, Hq, kv0.H, gamma1 + 1, k, chunk_size, tail),
                                dev)
        self.ws3 = tf.workspace(tf.verify_attn_workspace_size(1, Hq, kv0.H, gamma2 + 1, kv0.max_len), dev)
        self.wsa = tf.workspace(tf.accept_workspace_size(1, max(gamma1, gamma2), V), dev)
        self.wst = tf.workspace(tf.select_topk_workspace_size(1, kv0.H, self.c_max, k), dev)
        # uniforms of a round (gamma1 drafter draws, then gamma1 + 1 for level 1) and of
        # Force 3 (gamma2 + 1), staged in fixed buffers so that graphs can replay them
        self.u_round = torch.empty((1, 2 * gamma1 + 1), dtype=torch.float64, device=dev)
        self.u_f3 = torch.empty((1, gamma2 + 1), dtype=torch.float64, device=dev)
        self.u_pos = 0
        # capacities, read once: an append without room only sets its status and
        # writes nothing, so a step that would overrun must be refused up front
        self.cap = min(int(L.kv.seq_cap[0].item()) for L in target)
        for i, L in enumerate(drafter):
            check_ring(int(L.sd.seq_cap[0].item()) - n_sink, window, gamma1, gamma2, i)
        self.n = int(kv0.seq_len[0].item())            # committed rows before the current token
        self.pending = self.n - int(drafter[0].sd.seq_len[0].item())  # committed tokens the drafter has not consumed
        assert 0 <= self.pending <= 2
        self.steps = self.rounds = self.emitted = 0

    # -- helpers ---------------------------------------------------------------
    def _sync(self):
        (self.s or torch.cuda.current_stream()).synchronize()

    def _u(self, n):
        if self.u_pos + n > self.syn.uniforms.numel():
            self.u_pos = 0
        u = self.syn.uniforms[self.u_pos:self.u_pos + n]
        self.u_pos += n
        return u.view(1, n)

    def _drop(self, seq_len, rows):
        """seq_len -= rows on the device (a commit of `rows` rejected drafts)."""
        if rows > 0:
            tf.commit_length(seq_len, 0, rows, self.zero, stream=self.s)

    def _drafter_consume(self, R):
        """The drafter consumes R tokens: R rows on every layer's ring, then a
        streaming attention of the last one's query per layer."""
        rows = self.syn.draft_rows[R - 1]
        for L in self.dr:
            tf.append_kv(rows, rows, L.Ks, L.Vs, L.sd, ring=True, n_sink=self.S, window=self.W,
                         reserve=drafter_reserve(self.g1, self.g2), status=self.status, stream=self.s)
        tf.commit_length(self.d_len, R, stream=self.s)
        for L in self.dr:
            tf.stream_attn(self.syn.draft_q, L.Ks, L.Vs, L.sd, self.S, self.W, out=self.o_d, stream=self.s)

    def _capture(self):
        """Capture every graph a step can need before the first step: the
        retrieval, a round for each count of unseen tokens (0-2) and parity
        of the chain count, the one-row extension and Force 3.  Capturing
        records the launches without running them, so no state changes."""
        s = self.s
        s.synchronize()
        bodies = {"retrieval": self._retrieval, "extend": self._extend_one, "force3": self._force3}
        for pend in range(3):
            for cin in range(2):
                bodies[("round", pend, cin)] = (lambda p=pend, c=cin: self._round(p, c))
        for key, body in bodies.items():
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                body()
            self._g[key] = g

    def _run(self, key, body):
        """body() now, eagerly, or as the replay of its graph."""
        if not self.graphs:
            body()
            return
        if not self._g:
            self._capture()
        self._g[key].replay()

    # -- the bodies --------------------------------------------------------------
    def _retrieval(self):
        for L, idx in zip(self.t, self.idx):
            tf.score_chunks(self.syn.draft_q, self.Hq, L.ck, L.ckd, self.c_max, scores=self.scores, stream=self.s)
            tf.select_topk(self.scores, self.ck_len, self.k, idx=idx, ws=self.wst, stream=self.s)

    def _round(self, pend, cin):
        """Force 1 drafts gamma1 tokens (after consuming 1 + pend tokens), Force 2
        verifies them, level 1 tests them and the chain collects what they emit."""
        s, g1 = self.s, self.g1
        self._drafter_consume(1 + pend)
        for j in range(g1):
            if j > 0:
                self._drafter_consume(1)
            tf.accept(self.syn.r_rows[:, j:j + 1], None, None, self.u_round[:, j:j + 1], self.T,
                      n_accepted=self.na_d, next_token=self.drafts[j], ws=self.wsa, stream=s)
        self.drafts_row.copy_(self.drafts.view(1, g1))
        for L in self.t:
            tf.append_kv(self.syn.f2_rows, self.syn.f2_rows, L.K, L.V, L.kv, status=self.status, stream=s)
        tf.commit_length(self.seq_len, g1 + 1, stream=s)
        for L, idx in zip(self.t, self.idx):
            tf.sparse_verify_attn(self.syn.f2_q, L.K, L.V, L.kv, idx, self.cs, self.tail, out=self.o2,
                                  ws=self.ws2, stream=s)
        tf.accept(self.syn.q_rows, self.syn.r_rows, self.drafts_row, self.u_round[:, g1:], self.T,
                  n_accepted=self.n1, next_token=self.y, ws=self.wsa, stream=s)
        tf.collect_candidates(self.drafts_row, self.n1, self.y, self.syn.q_rows, self.cnt[cin], self.cnt[1 - cin],
                              self.cand, self.cand_q, stream=s)
        tf.commit_length(self.seq_len, 0, g1, self.n1, stream=s)   # rejected drafts leave the full cache
        # the drafter consumed the current token and drafts 1 .. g1 - 1: the
        # g1 - 1 - min(n1, g1 - 1) of those after the first rejection leave its ring
        tf.commit_length(self.d_len, 0, g1 - 1, self.n1, stream=s)

    def _extend_one(self):
        for L in self.t:
            tf.append_kv(self.syn.one_row, self.syn.one_row, L.K, L.V, L.kv, status=self.status, stream=self.s)
        tf.commit_length(self.seq_len, 1, stream=self.s)

    def _force3(self):
        """Force 3 on the full cache, level 2, the rejected candidates' rollback and
        the refresh of the chunk keys the step's rows fell into."""
        s, g2 = self.s, self.g2
        for L in self.t:
            tf.verify_attn(self.syn.f3_q, L.K, L.V, L.kv, out=self.o3, ws=self.ws3, stream=s)
        tf.accept(self.syn.p_rows, self.cand_q, self.cand, self.u_f3, self.T, n_accepted=self.n2,
                  next_token=self.nxt, ws=self.wsa, stream=s)
        tf.commit_length(self.seq_len, 0, g2, self.n2, stream=s)
        for L in self.t:
            tf.build_chunk_keys(L.K, L.kv, self.cs, L.ck, L.ckd, chunk_begin=self.chunk_begin,
                                max_chunks=(g2 + 1) // self.cs + 2, stream=s)

    def _stage_uniforms(self, dst, counts):
        """Copy the next uniforms (taken as _u(c) for each c in counts, in order)
        into dst: one copy when they are consecutive (no wrap in between)."""
        start = self.u_pos
        parts = [self._u(c) for c in counts]
        if self.u_pos - start == dst.shape[1]:
            dst.copy_(self.syn.uniforms[start:self.u_pos].view(1, -1))
        else:
            dst.copy_(torch.cat(parts, 1))

    # -- one step --------------------------------------------------------------
    def step(self) -> int:
        """One three-tier step; returns the number of tokens it emits."""
        g1, g2 = self.g1, self.g2
        n_start = self.n
        check_room(n_start, g1, g2, self.cap)
        d_start = self.n - self.pending       # drafter's consumed length
        with torch.cuda.stream(self.s) if self.s is not None else _nullcontext():
            # retrieval for this step, from the committed rows
            self.ck_len.fill_(-(-n_start // self.cs))
            self._run("retrieval", self._retrieval)
            self.cnt[0].zero_()
            cin, total, rounds = 0, 0, 0      # total: tokens the rounds emitted (the chain keeps the first gamma2)
            d_len = d_start                    # host copy of the drafter's length
            while total < g2:
                rounds += 1
                n_round = self.n
                self._stage_uniforms(self.u_round, [1] * g1 + [g1 + 1])
                pend = self.pending
                self._run(("round", pend, cin), lambda: self._round(pend, cin))
                self.host[0:1].copy_(self.n1, non_blocking=True)   # the kept count (outside any graph)
                d_len += g1 + pend            # the current token, the unseen ones, drafts 1 .. g1 - 1
                self.pending = 0
                self._sync()
                n1 = int(self.host[0])
                total += n1 + 1
                cin = 1 - cin
                if self.record:
                    self.log.append(("round", self.drafts_row.cpu().numpy()[0].tolist(), n1, int(self.y.item()),
                                     self.u_round.cpu().numpy()[0, g1:]))
                self.n = n_round + 1 + n1
                # the drafter consumed the current token and drafts 1 .. g1 - 1
                # (the device length was cut inside the round)
                d_len -= (g1 - 1) - min(n1, g1 - 1)
                self.pending = self.n - d_len
            # the full cache holds the current token and the first total - 1
            # emitted tokens: keep the current token and exactly gamma2 candidates
            if total == g2:
                self._run("extend", self._extend_one)
            else:
                self._drop(self.seq_len, total - 1 - g2)
            self._stage_uniforms(self.u_f3, [g2 + 1])
            self.chunk_begin.fill_(n_start // self.cs)
            self._run("force3", self._force3)
            self.host[2:3].copy_(self.n2, non_blocking=True)
            self._sync()
            n2 = int(self.host[2])
            if self.record:
                self.log.append(("step", self.cand.cpu().numpy()[0].tolist(), n2, int(self.nxt.item()),
                                 self.u_f3.cpu().numpy()[0], self.cand_q.cpu().numpy()[0]))
            self.n = n_start + 1 + n2
            # the drafter keeps what it consumed of the committed tokens
            keep = min(d_len, self.n)
            self._drop(self.d_len, d_len - keep)
        self.pending = self.n - keep
        self.steps += 1
        self.rounds += rounds
        self.emitted += n2 + 1
        return n2 + 1


class _nullcontext:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False
