"""fp64 CPU oracle for TriForce's decode-step attention path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package's smoke check and
the benchmark's CPU-baseline leg may import or run this module.  The product
path never does: it shares no code with the HIP kernels and imports nothing
from them, and this module imports nothing from the product package.

Everything is plain numpy in float64, one (sequence, head) at a time.  16-bit
inputs arrive as raw uint16 bit patterns and are widened exactly here.

Sources (web pages, cited by title and section):
  [blog]  aifetchly, "TriForce: Hierarchical Speculative Decoding for LLMs":
          "1. The Three Forces of TriForce" (Force 1 streaming drafter with
          sinks + W = 256 recent tokens; Force 2 retrieval of the top-k KV
          blocks by key-query similarity under a token budget; Force 3 full
          cache verification) and "2. Dual Rejection Sampling: Mathematical
          Losslessness" (acceptance alpha = min(1, p/q) >= u, residual
          max(0, p - q) / sum max(0, p - q)).
  [abs]   mlsanity / fugumt pages for arXiv 2404.11912, "Abstract": the whole
          KV cache is loaded for every generated token; a dynamic sparse KV
          cache via retrieval serves as draft; robustness across temperatures.

Readings where the pages are silent (each one repeated at its function):
  chunk keys are the arithmetic mean of a chunk's keys; scores are unscaled
  dot products summed over the query heads of a KV group; selection is per
  (sequence, KV head) with ties to the lowest chunk index, output ascending,
  -1 padded; a row with no visible key yields o = 0 and lse = -inf; verify
  rows are bottom-right aligned (row i of Q sees keys j <= n - Q + i); the
  accept test is alpha = min(1, p/q) >= u with p(x) = 0 always rejecting,
  residual or bonus drawn by inverse CDF with one extra uniform; T = 0 is
  greedy (one-hot at the lowest-index argmax).
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# Widening of stored values
# ---------------------------------------------------------------------------

def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 bit patterns of fp16 / bf16 -> exact float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp32":
        return np.asarray(bits).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_f64_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once, to nearest with ties to even, to fp16 / bf16
    and return the uint16 bit patterns.  States what a stored chunk key must
    be.  bf16: keep 8 significant bits of the frexp mantissa with np.rint
    (round half to even); values stay in the normal range here."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)  # numpy rounds f64 -> f16 directly
    if dtype == "bf16":
        m, e = np.frexp(x)
        r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # exactly a bf16 value
        return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# a1  Chunk-mean keys
# ---------------------------------------------------------------------------

def chunk_keys(K: np.ndarray, n: int, chunk_size: int) -> np.ndarray:
    """Per-chunk mean of the keys: one summary key per block of `chunk_size`
    consecutive positions, the last block averaged over the positions present.

    [blog] "1. The Three Forces of TriForce", Force 2: retrieval works on KV
    blocks matched by key-query similarity.  Reading: a block is summarised by
    the arithmetic mean of its keys.
    K: float64 [>= n][d].  Returns float64 [ceil(n / chunk_size)][d]."""
    C = -(-n // chunk_size) if n > 0 else 0
    out = np.zeros((C, K.shape[1]), np.float64)
    for c in range(C):
        lo, hi = c * chunk_size, min(n, (c + 1) * chunk_size)
        out[c] = K[lo:hi].sum(axis=0) / (hi - lo)
    return out


# ---------------------------------------------------------------------------
# a2  Query-to-chunk scores
# ---------------------------------------------------------------------------

def chunk_scores(q_group: np.ndarray, ck: np.ndarray) -> np.ndarray:
    """s_c = sum over the query heads h of the group of q_h . kbar_c.

    [blog] Force 2: "Key-Query similarity matching".  Reading: the plain dot
    product, unscaled (no 1/sqrt(d): it would only rescale the ranking), summed
    over the query heads that share the KV head (with one head per KV head this
    is just q . kbar).  q_group: float64 [G][d]; ck: float64 [C][d]."""
    C = ck.shape[0]
    s = np.zeros(C, np.float64)
    for h in range(q_group.shape[0]):
        s += ck @ q_group[h]
    return s


# ---------------------------------------------------------------------------
# a3  Top-k chunk selection under a token budget
# ---------------------------------------------------------------------------

def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """The k highest-scoring chunks of one (sequence, KV head) row.

    [blog] Force 2: a small subset of the most critical KV blocks is chosen
    ("top k = 2,048 tokens out of 128k").  Readings: k = budget // chunk_size
    chunks; ties go to the lower chunk index; NaN counts as -inf and -0.0 as
    +0.0; the result is sorted ascending and padded with -1 when the row has
    fewer than k chunks.  Returns int64 [k]."""
    s = np.array(scores, dtype=np.float64)
    s[np.isnan(s)] = NEG_INF
    s = s + 0.0  # -0.0 -> +0.0
    C = s.shape[0]
    order = np.lexsort((np.arange(C), -s))  # by score descending, then index
    take = np.sort(order[:min(k, C)])
    out = np.full(k, -1, np.int64)
    out[:take.shape[0]] = take
    return out


# ---------------------------------------------------------------------------
# Attention over a set of keys: the plain definition
# ---------------------------------------------------------------------------

def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> Tuple[np.ndarray, float]:
    """o = sum_t softmax_t(q . K_t / sqrt(d)) V_t and lse = log sum_t exp(q . K_t / sqrt(d)).

    Scaled dot-product attention of one query over the given key/value rows.
    Reading: with no keys, o = 0 and lse = -inf.  q: [d]; K, V: [m][d]."""
    d = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros(d, np.float64), NEG_INF
    logits = (K @ q) / math.sqrt(d)
    m = logits.max()
    w = np.exp(logits - m)
    z = w.sum()
    return (w @ V) / z, float(m + math.log(z))


# ---------------------------------------------------------------------------
# a4  Attention over the gathered chunks
# ---------------------------------------------------------------------------

def sparse_token_positions(idx: Sequence[int], chunk_size: int, n: int) -> np.ndarray:
    """Positions covered by the selected chunks (index -1 skipped, positions
    at or beyond n dropped)."""
    pos: List[int] = []
    for c in idx:
        c = int(c)
        if c < 0:
            continue
        pos.extend(t for t in range(c * chunk_size, (c + 1) * chunk_size) if t < n)
    return np.asarray(pos, np.int64)


def sparse_attn(q: np.ndarray, K: np.ndarray, V: np.ndarray, n: int,
                idx: Sequence[int], chunk_size: int) -> Tuple[np.ndarray, float]:
    """Attention of the draft query over the retrieved blocks only.

    [blog] Force 2: the target model runs on a retrieval-sparse KV cache made
    of the selected blocks; [abs]: dynamic sparse KV cache via retrieval as a
    draft.  Reading: only the gathered positions are attended (no extra
    recent-token tail)."""
    pos = sparse_token_positions(idx, chunk_size, n)
    return attention(q, K[pos], V[pos])


def sparse_verify_positions(n: int, Q: int, i: int, idx: Sequence[int], chunk_size: int,
                            tail: int) -> np.ndarray:
    """Rows seen by query row i when the retrieval-sparse cache verifies Q
    drafted rows: the rows of the selected chunks that lie below the tail,
    then the tail [t0, n - Q + i] with t0 = max(0, n - tail)."""
    t0 = max(0, n - tail)
    chunk_rows = [int(p) for p in sparse_token_positions(idx, chunk_size, n) if p < t0]
    return np.asarray(chunk_rows + list(range(t0, max(t0, n - Q + i + 1))), np.int64)


def sparse_verify_attn(qs: np.ndarray, K: np.ndarray, V: np.ndarray, n: int, idx: Sequence[int],
                       chunk_size: int, tail: int) -> Tuple[np.ndarray, np.ndarray]:
    """Force 2 verifying the small drafter's tokens on the sparse cache.

    [blog] "1. The Three Forces of TriForce", Force 2 evaluates the candidates
    from Force 1 on a retrieval-sparse KV cache; "2. Dual Rejection Sampling"
    then tests them r -> q.  Readings: the Q drafted rows are the last Q cache
    rows (as for the full verification); each query row attends the retrieved
    chunks below a causal tail of the most recent `tail` rows (tail >= Q) and
    the tail up to its own position.  qs: [Q][d].  Returns o [Q][d], lse [Q]."""
    Q, d = qs.shape
    o = np.zeros((Q, d), np.float64)
    lse = np.zeros(Q, np.float64)
    for i in range(Q):
        pos = sparse_verify_positions(n, Q, i, idx, chunk_size, tail)
        o[i], lse[i] = attention(qs[i], K[pos], V[pos])
    return o, lse


# ---------------------------------------------------------------------------
# a5  Sink + window streaming attention
# ---------------------------------------------------------------------------

def stream_positions(n: int, n_sink: int, window: int) -> np.ndarray:
    """Visible positions of a streaming cache after n tokens: the first
    n_sink positions and the most recent `window` ones (which include n - 1).

    [blog] Force 1: the drafter keeps the initial prompt sinks plus the most
    recent W tokens (W = 256), as in StreamingLLM."""
    sinks = list(range(min(n_sink, n)))
    recent = list(range(max(n_sink, n - window), n))
    return np.asarray(sinks + recent, np.int64)


def stream_attn_masked(q: np.ndarray, K_log: np.ndarray, V_log: np.ndarray, n: int,
                       n_sink: int, window: int) -> Tuple[np.ndarray, float]:
    """Streaming attention as full attention over the logical sequence with a
    sink/window mask."""
    pos = stream_positions(n, n_sink, window)
    return attention(q, K_log[pos], V_log[pos])


def stream_attn_ring(q: np.ndarray, K_log: np.ndarray, V_log: np.ndarray, n: int,
                     n_sink: int, window: int) -> Tuple[np.ndarray, float]:
    """The same quantity computed the other way: replay the n appends into a
    cache of n_sink sink slots plus a window of `window` slots that evicts
    its oldest entry, then attend over whatever the cache holds."""
    sink_rows: List[int] = []
    ring: List[int] = []
    for p in range(n):
        if len(sink_rows) < n_sink:
            sink_rows.append(p)
        else:
            ring.append(p)
            if len(ring) > window:
                ring.pop(0)
    held = np.asarray(sink_rows + ring, np.int64)
    return attention(q, K_log[held], V_log[held])


# ---------------------------------------------------------------------------
# a6  Full-cache multi-query verification
# ---------------------------------------------------------------------------

def verify_attn(qs: np.ndarray, K: np.ndarray, V: np.ndarray, n: int) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of the Q = gamma + 1 verification queries over the full cache.

    [blog] Force 3: the target with the complete cache checks all candidates
    in one parallel pass; [abs]: the whole KV cache is loaded for every
    generated token.  Reading (chain form): the last Q cache rows are the
    draft positions themselves, so query row i sees keys j <= n - Q + i.
    qs: [Q][d]; K, V: [>= n][d].  Returns o [Q][d], lse [Q]."""
    Q, d = qs.shape
    o = np.zeros((Q, d), np.float64)
    lse = np.zeros(Q, np.float64)
    for i in range(Q):
        vis = n - Q + i + 1
        vis = max(0, min(vis, n))
        o[i], lse[i] = attention(qs[i], K[:vis], V[:vis])
    return o, lse


def tree_masks(parent: Sequence[int]) -> List[int]:
    """Visibility masks of a candidate tree of Q nodes given by parent
    pointers: bit m of mask i is set when node m is node i or one of its
    ancestors.  [blog] Force 3 evaluates the candidate tree from Force 2 in
    one pass with tree attention; a node is conditioned on exactly its path
    from the committed prefix.  Reading: parent[i] = -1 hangs node i off the
    prefix; a parent outside [0, i) is read as -1 (nodes come in topological
    order, so a valid parent always precedes its child)."""
    Q = len(parent)
    out = []
    for i in range(Q):
        m, x = 0, i
        while x >= 0:
            m |= 1 << x
            p = int(parent[x])
            x = p if 0 <= p < x else -1
        out.append(m)
    return out


def verify_tree_attn(qs: np.ndarray, K: np.ndarray, V: np.ndarray, n: int,
                     masks: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Force 3 over a candidate tree.  The last Q cache rows hold the tree's
    nodes in order (node m at row n - Q + m); query row i sees every row
    before them and node m when bit m of masks[i] is set.  With chain masks
    (node i sees nodes 0..i) this is verify_attn.  qs: [Q][d]."""
    Q, d = qs.shape
    base = n - Q
    o = np.zeros((Q, d), np.float64)
    lse = np.zeros(Q, np.float64)
    for i in range(Q):
        vis = [t for t in range(max(0, n)) if t < base or (int(masks[i]) >> (t - base)) & 1]
        o[i], lse[i] = attention(qs[i], K[vis], V[vis])
    return o, lse


# ---------------------------------------------------------------------------
# a7  Lossless accept / reject
# ---------------------------------------------------------------------------

def distribution(logits: np.ndarray, temperature: float, probs: bool = False) -> np.ndarray:
    """Token distribution of one row: softmax(logits / T) for T > 0; for T = 0
    a one-hot at the lowest-index argmax (greedy).  With probs=True the row
    already holds probabilities and is used as given.

    [abs]: speedups hold across sampling temperatures.  Reading: temperature
    divides the logits before the softmax."""
    x = np.asarray(logits, dtype=np.float64)
    if probs:
        return x.copy()
    if temperature == 0.0:
        out = np.zeros_like(x)
        out[int(np.argmax(x))] = 1.0  # np.argmax returns the first maximum
        return out
    z = x / float(temperature)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def inverse_cdf(r: np.ndarray, u: float) -> int:
    """Draw from the (unnormalised, non-negative) weights r with one uniform:
    the smallest t whose running sum exceeds u * sum(r), strictly; clamped to
    the last t with r_t > 0 (guards the rounding of the running sum)."""
    total = float(r.sum())
    target = u * total
    run = 0.0
    last_pos = -1
    for t in range(r.shape[0]):
        if r[t] > 0.0:
            last_pos = t
        run += r[t]
        if run > target:
            return t
    return last_pos


def accept(target: np.ndarray, draft: np.ndarray, tokens: Sequence[int], uniforms: Sequence[float],
           temperature: float, probs: bool = False) -> Tuple[int, int, float]:
    """One sequence's speculative accept/reject over gamma drafted tokens.

    [blog] "2. Dual Rejection Sampling": a drafted token x is kept when
    alpha = min(1, p(x) / q(x)) >= u, u ~ U(0, 1); at the first rejection the
    next token is drawn from max(0, p - q) / sum_v max(0, p(v) - q(v)).
    Readings: p(x) = 0 always rejects (and q(x) = 0 < p(x) accepts, alpha = 1);
    a drafted token outside the vocabulary [0, V) has no probability under p
    and is rejected the same way (the residual draw then proceeds as for any
    rejection at that position);
    if every draft is kept a bonus token is drawn from the target row gamma;
    the draw is by inverse CDF with the extra uniform u[gamma]; a residual
    that sums to 0 (only through rounding) falls back to p.

    target: [gamma+1][V] logits (or probabilities), draft: [gamma][V],
    tokens: [gamma], uniforms: [gamma+1].  Returns (n_accepted, next_token,
    margin) where margin is the smallest distance of any decision taken to its
    threshold (used by tests to skip rounding-level ties)."""
    gamma = len(tokens)
    margin = math.inf
    j = gamma
    for i in range(gamma):
        p = distribution(target[i], temperature, probs)
        q = distribution(draft[i], temperature, probs)
        x = int(tokens[i])
        if not 0 <= x < p.shape[0]:
            j = i
            break
        px, qx = float(p[x]), float(q[x])
        if px > 0.0:
            alpha = 1.0 if qx == 0.0 else min(1.0, px / qx)
            margin = min(margin, abs(alpha - float(uniforms[i])))
            if alpha >= float(uniforms[i]):
                continue
        j = i
        break
    if j < gamma:
        p = distribution(target[j], temperature, probs)
        q = distribution(draft[j], temperature, probs)
        r = np.maximum(0.0, p - q)
        if r.sum() == 0.0:
            r = p
    else:
        r = distribution(target[gamma], temperature, probs)
    u = float(uniforms[gamma])
    nxt = inverse_cdf(r, u)
    # Margin of the inverse-CDF decision: distance of u*Z to the running sums
    # that bracket the chosen token.
    cs = np.cumsum(r)
    tgt = u * float(r.sum())
    if nxt >= 0:
        lo = cs[nxt - 1] if nxt > 0 else 0.0
        margin = min(margin, abs(cs[nxt] - tgt), abs(tgt - lo))
    return j, nxt, margin


def tree_accept(target: np.ndarray, draft: np.ndarray, tokens: Sequence[int], parent: Sequence[int],
                uniforms: Sequence[float], temperature: float, probs: bool = False
                ) -> Tuple[List[int], int, float]:
    """Accept / reject over a candidate tree of Q nodes (Force 3 verifying
    the tree Force 2 assembled, [blog] "1. The Three Forces of TriForce";
    the acceptance rule and the residual of "2. Dual Rejection Sampling").

    Node 0 is the last committed token; nodes 1 .. Q-1 are candidates with
    parent[c] in [0, c) (anything else hangs c off node 0).  target[v] is the
    target's distribution for the children of node v (Q rows); draft[v] the
    distribution they were drafted from (Q rows; rows of leaves unused).
    Reading (the pages give the single-candidate rule only): at node v the
    children are tried in index order; child c with token x is kept when
    p'(x) > 0 and u_c * q_v(x) <= p'(x), where p' starts as p_v and after
    each rejected sibling becomes max(0, p' - q_v) renormalised (p_v again if
    that vanishes through rounding); a kept child becomes v; when no child is
    kept -- or v has none -- the next token is drawn from p' by inverse CDF.
    With siblings drafted independently from q_v this keeps the target's
    distribution; a chain tree is exactly `accept`.  uniforms[c - 1] tests
    node c, uniforms[Q - 1] draws.  Returns (kept nodes in order, next token,
    margin)."""
    Q = len(parent)
    children = [[] for _ in range(Q)]
    for c in range(1, Q):
        pc = int(parent[c])
        children[pc if 0 <= pc < c else 0].append(c)
    margin = math.inf
    path: List[int] = []
    v = 0
    while True:
        p = distribution(target[v], temperature, probs)
        pr = p
        kept = -1
        if children[v]:
            q = distribution(draft[v], temperature, probs)
            for c in children[v]:
                x = int(tokens[c])
                if 0 <= x < p.shape[0] and pr[x] > 0.0:
                    lhs = float(uniforms[c - 1]) * float(q[x])
                    margin = min(margin, abs(lhs - float(pr[x])))
                    if lhs <= pr[x]:
                        kept = c
                        break
                r = np.maximum(0.0, pr - q)
                z = float(r.sum())
                pr = r / z if z > 0.0 else p
        if kept < 0:
            nxt = inverse_cdf(pr, float(uniforms[Q - 1]))
            cs = np.cumsum(pr)
            tgt = float(uniforms[Q - 1]) * float(pr.sum())
            lo = cs[nxt - 1] if nxt > 0 else 0.0
            margin = min(margin, abs(cs[nxt] - tgt), abs(tgt - lo))
            return path, nxt, margin
        path.append(kept)
        v = kept


# ---------------------------------------------------------------------------
# Two-level (dual) rejection sampling across the three tiers
# ---------------------------------------------------------------------------

def two_level_accept(p_rows: np.ndarray, q_rows: np.ndarray, r_rows: np.ndarray, w: Sequence[float],
                     u1: Sequence[float], v1: Sequence[float], u2: Sequence[float], gamma1: int, gamma2: int,
                     temperature: float, probs: bool = False, with_margin: bool = False):
    """One step of the hierarchy's sampling, r -> q -> p.

    [blog] "2. Dual Rejection Sampling": a candidate x proposed by the
    streaming drafter (distribution r) is kept by the sparse-cache target
    (distribution q) when min(1, q(x)/r(x)) >= u1; the candidates that Force 2
    passes on are then tested against the full-cache target p with
    min(1, p(x)/q(x)) >= u2, and a rejection there draws from
    max(0, p - q) / sum max(0, p - q).  "1. The Three Forces of TriForce":
    Force 1 drafts, Force 2 evaluates the drafts, Force 3 verifies what Force
    2 passes on in one pass.

    Readings where the page is silent: rows are indexed by absolute position
    t (row t is the distribution of token t given the tokens before it);
    Force 2 runs rounds of `gamma1` drafts until `gamma2` candidates are
    collected (each round emits its kept drafts plus the token it draws,
    exactly one level of `accept`), the surplus of the last round is dropped,
    and the level-2 draft distribution of a collected token is q at its
    position (the distribution level 1 makes it follow).  The drafter samples
    position t by inverse CDF of r_t with w[t]; a round starting at t0 tests
    its drafts with u1[t0 ..] and draws with v1[t0]; level 2 uses u2.  No
    uniform is ever consulted twice.

    p_rows: [gamma2 + 1][V]; q_rows: [gamma2 + gamma1][V];
    r_rows: [gamma2 + gamma1 - 1][V]; w, u1: gamma2 + gamma1 - 1 values;
    v1: gamma2 values; u2: gamma2 + 1 values.
    Returns (candidates, n_accepted, next_token, rounds): the step emits
    candidates[:n_accepted] followed by next_token.  With with_margin, a
    fifth value is the smallest distance of any decision taken to its
    threshold (tests use it to skip rounding-level ties)."""
    cand: List[int] = []
    rounds = 0
    margin = math.inf
    while len(cand) < gamma2:
        t0 = len(cand)
        drafts = []
        for j in range(gamma1):
            rr = distribution(r_rows[t0 + j], temperature, probs)
            x = inverse_cdf(rr, float(w[t0 + j]))
            cs = np.cumsum(rr)
            tgt = float(w[t0 + j]) * float(rr.sum())
            margin = min(margin, abs(cs[x] - tgt), abs(tgt - (cs[x - 1] if x > 0 else 0.0)))
            drafts.append(x)
        uni = [float(x) for x in u1[t0:t0 + gamma1]] + [float(v1[t0])]
        n1, y, m = accept(q_rows[t0:t0 + gamma1 + 1], r_rows[t0:t0 + gamma1], drafts, uni, temperature, probs)
        margin = min(margin, m)
        cand += drafts[:n1] + [y]
        rounds += 1
    cand = cand[:gamma2]
    n2, nxt, m = accept(p_rows[:gamma2 + 1], q_rows[:gamma2], cand, u2, temperature, probs)
    margin = min(margin, m)
    if with_margin:
        return cand, n2, nxt, rounds, margin
    return cand, n2, nxt, rounds


# ---------------------------------------------------------------------------
# Cache maintenance around the path: drafted rows enter the caches before
# they are verified, rejected ones leave them.
# ---------------------------------------------------------------------------

APPEND_OK, APPEND_NO_ROOM, APPEND_RING_TOO_SMALL, APPEND_BAD_LENGTH = 0, 1, 2, 3


def append_full(rows: np.ndarray, n: int, new: np.ndarray) -> Tuple[np.ndarray, int]:
    """Full cache of one (sequence, head): rows [cap][d], n valid.  The R new
    rows go to positions n .. n + R - 1; a sequence without room for all of
    them is left as it is.  [blog] Force 3 reads the complete cache, which by
    the verification reading already holds the drafted rows.  Returns the
    updated copy and a status."""
    cap, R = rows.shape[0], new.shape[0]
    out = rows.copy()
    if n < 0:
        return out, APPEND_BAD_LENGTH
    if n + R > cap:
        return out, APPEND_NO_ROOM
    out[n:n + R] = new
    return out, APPEND_OK


def ring_slot_of(p: int, n_sink: int, cap: int) -> int:
    """Slot of logical position p in a streaming cache of cap slots: the
    first n_sink positions keep their own slot, later ones cycle through the
    remaining cap - n_sink slots."""
    if p < n_sink:
        return p
    return n_sink + (p - n_sink) % (cap - n_sink)


def append_ring(slots: np.ndarray, n: int, n_sink: int, window: int,
                new: np.ndarray, reserve: Optional[int] = None) -> Tuple[np.ndarray, int]:
    """Streaming cache of one (sequence, head) after n logical positions:
    the R new rows become positions n .. n + R - 1.  [blog] Force 1 keeps the
    sinks and a rolling window of the W most recent tokens.  Reading:
    `reserve` (default R) bounds the rows appended since the last length that
    can no longer be rolled back; the ring keeps window + reserve slots after
    the sinks, so a rollback to any later length never exposes a visible
    position whose slot a newer row took.  A ring without that room is left
    as it is."""
    cap, R = slots.shape[0], new.shape[0]
    reserve = R if reserve is None else reserve
    out = slots.copy()
    if n < 0:
        return out, APPEND_BAD_LENGTH
    if cap - n_sink < window + reserve:
        return out, APPEND_RING_TOO_SMALL
    for r in range(R):
        out[ring_slot_of(n + r, n_sink, cap)] = new[r]
    return out, APPEND_OK


def ring_visible(slots: np.ndarray, n: int, n_sink: int, window: int) -> Tuple[np.ndarray, np.ndarray]:
    """The positions a5 attends after n logical positions, and the rows the
    ring holds for them (in position order)."""
    pos = stream_positions(n, n_sink, window)
    cap = slots.shape[0]
    return pos, slots[[ring_slot_of(int(p), n_sink, cap) for p in pos]]


def commit_length(n: int, add: int, gamma: int = 0, n_accepted: Optional[int] = None) -> int:
    """Length after a decode step: `add` appended rows become valid, and with
    an accept result the gamma - n_accepted rejected drafts leave again
    ([blog] "2. Dual Rejection Sampling": the tokens after the first
    rejection are discarded).  n_accepted is clamped into [0, gamma]; the
    length never goes below 0."""
    drop = 0 if n_accepted is None else gamma - min(max(int(n_accepted), 0), gamma)
    return max(0, n + add - drop)
