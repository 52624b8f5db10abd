"""Pins of the fp64 oracle against things other than itself: closed forms,
library routines (torch / scipy on the CPU), brute force on tiny inputs,
hand-worked examples from the pages, and statistics of the sampling claim.
Runs without a GPU."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa(q, K, V, mask=None):
    """torch's scaled_dot_product_attention on the CPU in float64 (library
    routine; one query row)."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).view(1, 1, 1, -1)
    Kt = torch.from_numpy(np.asarray(K, np.float64)).view(1, 1, K.shape[0], -1)
    Vt = torch.from_numpy(np.asarray(V, np.float64)).view(1, 1, V.shape[0], -1)
    m = None if mask is None else torch.from_numpy(np.asarray(mask, bool)).view(1, 1, 1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m).view(-1).numpy()


# ---------------------------------------------------------------------------
# widening / rounding
# ---------------------------------------------------------------------------

def test_widen_known_bit_patterns():
    assert oracle.widen(np.array([0x3F80], np.uint16), "bf16")[0] == 1.0
    assert oracle.widen(np.array([0xC040], np.uint16), "bf16")[0] == -3.0
    assert oracle.widen(np.array([0x3C00], np.uint16), "fp16")[0] == 1.0
    assert oracle.widen(np.array([0x7BFF], np.uint16), "fp16")[0] == 65504.0


def test_round_to_bf16_ties_and_library():
    one = 1.0
    cases = {one: 0x3F80,
             one + 2.0 ** -8: 0x3F80,            # tie -> even (mantissa 0)
             one + 3 * 2.0 ** -8: 0x3F82,        # tie -> even (mantissa 2)
             one + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # just above the tie
             -2.5: 0xC020}
    for x, bits in cases.items():
        assert int(oracle.round_f64_to_bits(np.array([x]), "bf16")[0]) == bits, x
    # float32-representable inputs: torch's fp32 -> bf16 cast rounds to nearest even
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_f64_to_bits(x.astype(np.float64), "bf16")
    assert np.array_equal(ref, got)


def test_round_to_fp16_ties_subnormals_and_library():
    one = 1.0
    cases = {one: 0x3C00,
             one + 2.0 ** -11: 0x3C00,            # tie -> even (mantissa 0)
             one + 3 * 2.0 ** -11: 0x3C02,        # tie -> even (mantissa 2)
             one + 2.0 ** -11 + 2.0 ** -30: 0x3C01,  # just above the tie: one rounding, not two via fp32
             -2.5: 0xC100,
             2.0 ** -24: 0x0001,                  # smallest subnormal
             3 * 2.0 ** -25: 0x0002,              # subnormal tie -> even
             2.0 ** -26: 0x0000,                  # below half the smallest subnormal
             65504.0: 0x7BFF,                     # largest finite
             65520.0: 0x7C00}                     # tie between 65504 and 2^16 -> even -> overflow to inf
    with np.errstate(over="ignore"):        # 65520 overflows to inf by design
        for x, bits in cases.items():
            assert int(oracle.round_f64_to_bits(np.array([x]), "fp16")[0]) == bits, x
    # float32-representable inputs across the normal and subnormal fp16 range:
    # torch's fp32 -> fp16 cast rounds to nearest even
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-26, 15, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_f64_to_bits(x.astype(np.float64), "fp16")
    assert np.array_equal(ref, got)


# ---------------------------------------------------------------------------
# a1 chunk keys: closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,cs", [(64, 8), (67, 8), (5, 8), (48, 16), (1, 1), (9, 3)])
def test_chunk_keys_ramp_closed_form(n, cs):
    # K_t = (t + 1) * a  =>  mean over [lo, hi) = ((lo + 1) + hi) / 2 * a
    a = np.random.default_rng(n * 31 + cs).standard_normal(8)
    K = np.arange(1, n + 1, dtype=np.float64)[:, None] * a[None, :]
    ck = oracle.chunk_keys(K, n, cs)
    assert ck.shape == (-(-n // cs), 8)
    for c in range(ck.shape[0]):
        lo, hi = c * cs, min(n, (c + 1) * cs)
        np.testing.assert_allclose(ck[c], (lo + 1 + hi) / 2.0 * a, rtol=1e-14, atol=1e-14)


def test_chunk_keys_constant_and_rows_beyond_n_ignored():
    K = np.full((40, 4), 7.0)
    K[30:] = 1e9  # rows past n must not be read
    ck = oracle.chunk_keys(K, 30, 8)
    assert ck.shape == (4, 4)
    assert np.all(ck == 7.0)
    assert oracle.chunk_keys(K, 0, 8).shape == (0, 4)


# ---------------------------------------------------------------------------
# a2 scores: library matrix-vector product, linearity over the group
# ---------------------------------------------------------------------------

def test_scores_match_library_gemv_and_group_linearity():
    rng = np.random.default_rng(5)
    ck = rng.standard_normal((300, 128))
    qs = rng.standard_normal((4, 128))
    s1 = oracle.chunk_scores(qs[:1], ck)
    ref = torch.mv(torch.from_numpy(ck), torch.from_numpy(qs[0])).numpy()
    np.testing.assert_allclose(s1, ref, rtol=1e-12, atol=1e-12)
    # a group of heads scores like one query equal to the heads' sum
    s4 = oracle.chunk_scores(qs, ck)
    ref4 = torch.mv(torch.from_numpy(ck), torch.from_numpy(qs.sum(axis=0))).numpy()
    np.testing.assert_allclose(s4, ref4, rtol=1e-11, atol=1e-11)
    # unscaled: doubling the query doubles the score exactly
    assert np.array_equal(oracle.chunk_scores(2.0 * qs[:1], ck), 2.0 * s1)


# ---------------------------------------------------------------------------
# a3 top-k: brute force on every tie pattern of tiny rows
# ---------------------------------------------------------------------------

def brute_topk(s, k):
    """Chunk c is kept iff fewer than k chunks beat it, where c' beats c when
    its score is larger, or equal with a smaller index."""
    C = len(s)
    keep = []
    for c in range(C):
        beaten = sum(1 for c2 in range(C) if s[c2] > s[c] or (s[c2] == s[c] and c2 < c))
        if beaten < k:
            keep.append(c)
    return keep + [-1] * (k - len(keep))


def test_topk_exhaustive_tie_patterns():
    vals = [-1.0, 0.0, 2.5]
    for C in range(1, 7):
        for row in itertools.product(vals, repeat=C):
            for k in range(1, C + 2):
                got = oracle.select_topk(np.array(row), k).tolist()
                assert got == brute_topk(list(row), k), (row, k)


def test_topk_invariants_random_and_special_values():
    rng = np.random.default_rng(11)
    for C, k in [(1000, 37), (64, 64), (65, 64), (10, 20), (512, 1)]:
        s = np.round(rng.standard_normal(C) * 3) / 2  # many exact ties
        idx = oracle.select_topk(s, k)
        sel = idx[idx >= 0]
        assert len(sel) == min(k, C)
        assert np.all(np.diff(sel) > 0)  # ascending, distinct
        rest = np.setdiff1d(np.arange(C), sel)
        if len(rest) and len(sel):
            assert s[sel].min() >= s[rest].max()
            # among ties at the boundary the kept ones have the lower indices
            t = s[sel].min()
            kept_t, left_t = sel[s[sel] == t], rest[s[rest] == t]
            if len(left_t):
                assert kept_t.max() < left_t.min()
    s = np.array([np.nan, -0.0, 0.0, -np.inf, np.inf, 1.0])
    assert oracle.select_topk(s, 3).tolist() == [1, 4, 5]      # +inf, 1.0, then -0.0 (== +0.0, lower index)
    assert oracle.select_topk(s, 5).tolist() == [0, 1, 2, 4, 5]  # NaN ranks with -inf, lower index first
    assert oracle.select_topk(np.array([np.nan, -np.inf]), 1).tolist() == [0]


# ---------------------------------------------------------------------------
# attention definition: library SDPA, scipy logsumexp, closed forms
# ---------------------------------------------------------------------------

def test_attention_matches_library_sdpa_and_logsumexp():
    rng = np.random.default_rng(17)
    for m in [1, 7, 300]:
        q, K, V = rng.standard_normal(128), rng.standard_normal((m, 128)), rng.standard_normal((m, 128))
        o, lse = oracle.attention(q, K, V)
        np.testing.assert_allclose(o, sdpa(q, K, V), rtol=1e-12, atol=1e-13)
        assert abs(lse - scipy.special.logsumexp(K @ q / math.sqrt(128))) < 1e-12


def test_attention_closed_forms():
    rng = np.random.default_rng(19)
    q, K = rng.standard_normal(16), rng.standard_normal((50, 16))
    c = rng.standard_normal(16)
    o, _ = oracle.attention(q, K, np.tile(c, (50, 1)))          # constant V -> that constant
    np.testing.assert_allclose(o, c, rtol=1e-13, atol=1e-13)
    V = rng.standard_normal((50, 16))
    o, lse = oracle.attention(q, np.zeros((50, 16)), V)          # K = 0 -> mean of V, lse = ln m
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=1e-13, atol=1e-13)
    assert abs(lse - math.log(50)) < 1e-13
    o, lse = oracle.attention(q, np.zeros((0, 16)), np.zeros((0, 16)))
    assert np.all(o == 0) and lse == -math.inf


# ---------------------------------------------------------------------------
# a6 verify: prefix attention per row (bottom-right alignment)
# ---------------------------------------------------------------------------

def test_verify_rows_are_prefix_attention():
    rng = np.random.default_rng(23)
    n, Q = 200, 7
    qs, K, V = rng.standard_normal((Q, 128)), rng.standard_normal((n, 128)), rng.standard_normal((n, 128))
    o, lse = oracle.verify_attn(qs, K, V, n)
    for i in range(Q):
        vis = n - Q + i + 1
        np.testing.assert_allclose(o[i], sdpa(qs[i], K[:vis], V[:vis]), rtol=1e-12, atol=1e-13)
        assert abs(lse[i] - scipy.special.logsumexp(K[:vis] @ qs[i] / math.sqrt(128))) < 1e-12
    # Q = 1 is ordinary decode attention over the whole cache
    o1, _ = oracle.verify_attn(qs[:1], K, V, n)
    np.testing.assert_allclose(o1[0], sdpa(qs[0], K, V), rtol=1e-12, atol=1e-13)


def test_tree_masks_hand_table():
    # node 0 off the prefix; 1 and 2 children of 0; 3 child of 1; 4 a second root
    assert oracle.tree_masks([-1, 0, 0, 1, -1]) == [0b1, 0b11, 0b101, 0b1011, 0b10000]
    # a chain: node i sees nodes 0..i
    assert oracle.tree_masks([-1, 0, 1, 2]) == [0b1, 0b11, 0b111, 0b1111]
    # parents outside [0, i) hang the node off the prefix
    assert oracle.tree_masks([5, 0, 2, -9, 3]) == [0b1, 0b11, 0b100, 0b1000, 0b11000]


def test_verify_tree_chain_is_verify_and_rows_match_masked_sdpa():
    rng = np.random.default_rng(29)
    n, Q = 150, 7
    qs, K, V = rng.standard_normal((Q, 128)), rng.standard_normal((n, 128)), rng.standard_normal((n, 128))
    chain = oracle.tree_masks([-1] + list(range(Q - 1)))
    o_t, l_t = oracle.verify_tree_attn(qs, K, V, n, chain)
    o_v, l_v = oracle.verify_attn(qs, K, V, n)
    assert np.array_equal(o_t, o_v) and np.array_equal(l_t, l_v)
    parent = [-1, 0, 0, 1, 2, -1, 5]
    masks = oracle.tree_masks(parent)
    o, lse = oracle.verify_tree_attn(qs, K, V, n, masks)
    for i in range(Q):
        vis = np.ones(n, bool)
        vis[n - Q:] = False
        x = i
        while x >= 0:                      # the node and its ancestors, walked independently
            vis[n - Q + x] = True
            x = parent[x]
        np.testing.assert_allclose(o[i], sdpa(qs[i], K, V, vis), rtol=1e-12, atol=1e-13)
        assert abs(lse[i] - scipy.special.logsumexp((K @ qs[i] / math.sqrt(128))[vis])) < 1e-12
    # a star (every node off the prefix) sees the prefix and itself only
    star = oracle.tree_masks([-1] * Q)
    o, _ = oracle.verify_tree_attn(qs, K, V, n, star)
    for i in range(Q):
        rows = list(range(n - Q)) + [n - Q + i]
        np.testing.assert_allclose(o[i], sdpa(qs[i], K[rows], V[rows]), rtol=1e-12, atol=1e-13)
    # fewer cache rows than nodes: missing nodes are simply absent
    o, lse = oracle.verify_tree_attn(qs, K, V, 3, masks)
    for i in range(Q):
        vis = [t for t in range(3) if (masks[i] >> (t + Q - 3)) & 1]
        if vis:
            np.testing.assert_allclose(o[i], sdpa(qs[i], K[vis], V[vis]), rtol=1e-12, atol=1e-13)
        else:
            assert np.all(o[i] == 0) and lse[i] == -math.inf


def test_verify_alignment_closed_form():
    # K = 0: row i averages V over its visible prefix [0, n - Q + i].
    n, Q = 5, 3
    V = np.arange(n, dtype=np.float64)[:, None] * np.ones((1, 4))
    o, _ = oracle.verify_attn(np.ones((Q, 4)), np.zeros((n, 4)), V, n)
    assert np.allclose(o[:, 0], [1.0, 1.5, 2.0])   # means of 0..2, 0..3, 0..4
    # fewer cache rows than queries: leading rows see nothing
    o, lse = oracle.verify_attn(np.ones((Q, 4)), np.zeros((2, 4)), V[:2], 2)
    assert np.all(o[0] == 0) and lse[0] == -math.inf
    assert np.allclose(o[1:, 0], [0.0, 0.5])


# ---------------------------------------------------------------------------
# a4 sparse attention
# ---------------------------------------------------------------------------

def test_sparse_full_budget_equals_full_attention():
    rng = np.random.default_rng(29)
    n, cs = 203, 8
    q, K, V = rng.standard_normal(128), rng.standard_normal((n, 128)), rng.standard_normal((n, 128))
    C = -(-n // cs)
    o, lse = oracle.sparse_attn(q, K, V, n, list(range(C)), cs)
    np.testing.assert_allclose(o, sdpa(q, K, V), rtol=1e-12, atol=1e-13)
    o2, lse2 = oracle.verify_attn(q[None], K, V, n)
    np.testing.assert_allclose(o, o2[0], rtol=1e-12, atol=1e-13)
    assert abs(lse - lse2[0]) < 1e-12


def test_sparse_gather_equals_masked_library_attention():
    rng = np.random.default_rng(31)
    n, cs = 100, 8
    q, K, V = rng.standard_normal(128), rng.standard_normal((n, 128)), rng.standard_normal((n, 128))
    idx = [1, 5, 12, -1]   # chunk 12 is the partial last chunk (rows 96..99)
    o, _ = oracle.sparse_attn(q, K, V, n, idx, cs)
    mask = np.zeros(n, bool)
    for c in (1, 5):
        mask[c * cs:(c + 1) * cs] = True
    mask[96:100] = True
    np.testing.assert_allclose(o, sdpa(q, K, V, mask), rtol=1e-12, atol=1e-13)


def test_sparse_single_token_is_that_value_row():
    rng = np.random.default_rng(37)
    q, K, V = rng.standard_normal(128), rng.standard_normal((50, 128)), rng.standard_normal((50, 128))
    o, lse = oracle.sparse_attn(q, K, V, 50, [17], 1)
    assert np.array_equal(o, V[17])
    assert abs(lse - K[17] @ q / math.sqrt(128)) < 1e-12
    o, lse = oracle.sparse_attn(q, K, V, 50, [-1, -1], 8)
    assert np.all(o == 0) and lse == -math.inf


# ---------------------------------------------------------------------------
# a5 streaming attention: two formulations, masks, closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,S,W", [(1000, 4, 252), (256, 4, 252), (100, 4, 252), (3, 4, 252),
                                   (1000, 0, 1), (50, 2, 7), (300, 4, 300)])
def test_stream_ring_equals_mask_and_library(n, S, W):
    rng = np.random.default_rng(n + S + W)
    q, K, V = rng.standard_normal(128), rng.standard_normal((n, 128)), rng.standard_normal((n, 128))
    om, lm = oracle.stream_attn_masked(q, K, V, n, S, W)
    orr, lr = oracle.stream_attn_ring(q, K, V, n, S, W)
    np.testing.assert_allclose(om, orr, rtol=1e-13, atol=1e-14)
    assert abs(lm - lr) < 1e-12
    mask = np.zeros(n, bool)
    mask[:S] = True
    mask[max(0, n - W):] = True
    np.testing.assert_allclose(om, sdpa(q, K, V, mask), rtol=1e-12, atol=1e-13)
    if n <= S + W:
        np.testing.assert_allclose(om, sdpa(q, K, V), rtol=1e-12, atol=1e-13)
    if S == 0 and W == 1:
        assert np.array_equal(om, V[n - 1])


# ---------------------------------------------------------------------------
# a7 accept: hand-worked examples from the pages' formulas, greedy, statistics
# ---------------------------------------------------------------------------

def load_golden():
    with open(os.path.join(GOLDEN, "accept_hand_examples.json")) as f:
        return json.load(f)


def test_accept_hand_examples():
    g = load_golden()
    for case in g["cases"]:
        t = np.array(case["target"], np.float32)
        d = np.array(case["draft"], np.float32)
        n_acc, nxt, _ = oracle.accept(t, d, case["tokens"], case["uniforms"], 1.0, probs=True)
        assert (n_acc, nxt) == (case["n_accepted"], case["next_token"]), case["name"]
    gr = g["greedy"]
    n_acc, nxt, _ = oracle.accept(np.array(gr["target"], np.float32), np.array(gr["draft"], np.float32),
                                  gr["tokens"], gr["uniforms"], 0.0)
    assert (n_acc, nxt) == (gr["n_accepted"], gr["next_token"])


def test_accept_identical_and_disjoint_distributions():
    rng = np.random.default_rng(41)
    gamma, V = 5, 50
    t = rng.normal(0, 2, (gamma + 1, V)).astype(np.float32)
    toks = rng.integers(0, V, gamma)
    for _ in range(20):
        u = rng.random(gamma + 1)
        n_acc, nxt, _ = oracle.accept(t, t[:gamma].copy(), toks, u, 0.8)
        assert n_acc == gamma                       # p = q keeps every draft
    # disjoint supports: the draft's tokens are impossible under the target
    p = np.zeros((gamma + 1, V), np.float32)
    p[:, :10] = 0.1
    q = np.zeros((gamma, V), np.float32)
    q[:, 10:] = 1.0 / 40
    for _ in range(20):
        n_acc, nxt, _ = oracle.accept(p, q, rng.integers(10, V, gamma), rng.random(gamma + 1), 1.0, probs=True)
        assert n_acc == 0 and 0 <= nxt < 10


def test_greedy_is_longest_matching_prefix():
    rng = np.random.default_rng(43)
    gamma, V = 6, 30
    for _ in range(50):
        t = rng.normal(0, 1, (gamma + 1, V)).astype(np.float32)
        d = rng.normal(0, 1, (gamma, V)).astype(np.float32)
        am_t = t.argmax(axis=1)
        toks = d.argmax(axis=1)
        match = rng.random(gamma) < 0.7
        toks[match] = am_t[:gamma][match]
        n_acc, nxt, _ = oracle.accept(t, d, toks, rng.random(gamma + 1) * 0.98 + 0.01, 0.0)
        expect = 0
        while expect < gamma and toks[expect] == am_t[expect]:
            expect += 1
        assert n_acc == expect
        assert nxt == am_t[expect]


def chi2_ok(counts, probs, alpha=1e-3):
    exp = probs * counts.sum()
    keep = exp > 0
    assert np.all(counts[~keep] == 0)
    stat = float(((counts[keep] - exp[keep]) ** 2 / exp[keep]).sum())
    crit = scipy.stats.chi2.ppf(1 - alpha, keep.sum() - 1)
    return stat < crit, stat, crit


def test_accept_is_lossless_statistically():
    """The emitted first token is distributed as p_0, and given that the
    first draft was kept the second emitted token is distributed as p_1
    (blog, '2. Dual Rejection Sampling': the accepted distribution equals the
    target's)."""
    rng = np.random.default_rng(47)
    V, gamma, trials = 8, 3, 60000
    p = rng.dirichlet(np.ones(V) * 0.7, gamma + 1)
    q = rng.dirichlet(np.ones(V) * 0.7, gamma)
    p[0, 5] = 0.0
    p[0] /= p[0].sum()          # a token the target never emits
    first = np.zeros(V, np.int64)
    second = np.zeros(V, np.int64)
    for _ in range(trials):
        toks = [rng.choice(V, p=q[i]) for i in range(gamma)]
        u = 1.0 - rng.random(gamma + 1)   # (0, 1]
        u = np.minimum(u, 1.0 - 1e-16)
        n_acc, nxt, _ = oracle.accept(p, q, toks, u, 1.0, probs=True)
        emitted = list(toks[:n_acc]) + [nxt]
        first[emitted[0]] += 1
        if n_acc >= 1:
            second[emitted[1]] += 1
    ok, stat, crit = chi2_ok(first, p[0])
    assert ok, (stat, crit)
    ok, stat, crit = chi2_ok(second, p[1])
    assert ok, (stat, crit)


def test_accept_with_temperature_is_lossless_statistically():
    rng = np.random.default_rng(53)
    V, gamma, T, trials = 6, 2, 0.7, 20000
    t = rng.normal(0, 1, (gamma + 1, V))
    d = rng.normal(0, 1, (gamma, V))
    p0 = scipy.special.softmax(t[0] / T)
    qd = scipy.special.softmax(d / T, axis=1)
    first = np.zeros(V, np.int64)
    for _ in range(trials):
        toks = [rng.choice(V, p=qd[i]) for i in range(gamma)]
        n_acc, nxt, _ = oracle.accept(t, d, toks, 1.0 - rng.random(gamma + 1) * 0.999999, T)
        first[(list(toks[:n_acc]) + [nxt])[0]] += 1
    ok, stat, crit = chi2_ok(first, p0)
    assert ok, (stat, crit)


# ---------------------------------------------------------------------------
# accept over a candidate tree
# ---------------------------------------------------------------------------

def test_tree_accept_hand_examples():
    with open(os.path.join(GOLDEN, "tree_accept_hand_examples.json")) as f:
        g = json.load(f)
    t, d = np.array(g["target"]), np.array(g["draft"])
    for case in g["cases"]:
        path, nxt, _ = oracle.tree_accept(t, d, case["tokens"], g["parent"], case["uniforms"], 1.0, probs=True)
        assert (path, nxt) == (case["path"], case["next_token"]), case["name"]


def test_tree_accept_chain_is_accept():
    rng = np.random.default_rng(83)
    for trial in range(300):
        g, V = int(rng.integers(1, 7)), 30
        T = [1.0, 0.6, 0.0][trial % 3]
        t = rng.normal(0, 1.5, (g + 1, V))
        d = t + rng.normal(0, 0.7, (g + 1, V))
        tok = [0] + [int(rng.choice(V, p=oracle.distribution(d[i], T if T > 0 else 1.0))) for i in range(g)]
        u = rng.random(g + 1)
        n, x, _ = oracle.accept(t, d[:g], tok[1:], u, T)
        path, y, _ = oracle.tree_accept(t, d, tok, [-1] + list(range(g)), u, T)
        assert path == list(range(1, n + 1)) and y == x


def _tree_lossless_setup(rng, V=6):
    # root 0 -> nodes 1, 2, 3 (drafted i.i.d. from q0); node c in 1..3 ->
    # two children drafted i.i.d. from q1; every depth-1 node has target p1
    p = rng.dirichlet(np.ones(V) * 0.8, 3)
    q = rng.dirichlet(np.ones(V) * 0.8, 2)
    parent = [-1, 0, 0, 0, 1, 1, 2, 2, 3, 3]
    target = np.stack([p[0], p[1], p[1], p[1]] + [p[2]] * 6)
    draft = np.stack([q[0], q[1], q[1], q[1]] + [q[1]] * 6)
    return p, q, parent, target, draft


def test_tree_accept_is_lossless_statistically():
    """Siblings drafted independently from their parent's q: the first emitted
    token follows p_0 and, when a depth-1 node is kept, the second follows
    p_1 (blog, '2. Dual Rejection Sampling')."""
    rng = np.random.default_rng(89)
    V, trials = 6, 20000
    p, q, parent, target, draft = _tree_lossless_setup(rng, V)
    first = np.zeros(V, np.int64)
    second = np.zeros(V, np.int64)
    for _ in range(trials):
        tok = [0] + list(rng.choice(V, 3, p=q[0])) + list(rng.choice(V, 6, p=q[1]))
        path, nxt, _ = oracle.tree_accept(target, draft, tok, parent, rng.random(10), 1.0, probs=True)
        emitted = [tok[c] for c in path] + [nxt]
        first[emitted[0]] += 1
        if path:
            second[emitted[1]] += 1
    for counts, ref in ((first, p[0]), (second, p[1])):
        ok, stat, crit = chi2_ok(counts, ref)
        assert ok, (stat, crit)


# ---------------------------------------------------------------------------
# two-level accept r -> q -> p (dual rejection sampling)
# ---------------------------------------------------------------------------

def test_two_level_hand_examples():
    with open(os.path.join(GOLDEN, "two_level_hand_examples.json")) as f:
        g = json.load(f)
    P, Qr, R = (np.array(g[k], np.float64) for k in ("p_rows", "q_rows", "r_rows"))
    for case in g["cases"]:
        cand, n2, nxt, rounds = oracle.two_level_accept(P, Qr, R, case["w"], case["u1"], case["v1"], case["u2"],
                                                        g["gamma1"], g["gamma2"], 1.0, probs=True)
        assert (cand, n2, nxt, rounds) == (case["candidates"], case["n_accepted"], case["next_token"],
                                           case["rounds"]), case["name"]


def _two_level_inputs(rng, V, g1, g2):
    T = g2 + g1
    return (rng.random(T - 1), rng.random(T - 1), rng.random(g2), rng.random(g2 + 1))


def test_two_level_special_cases():
    rng = np.random.default_rng(61)
    V, g1, g2 = 7, 3, 5
    for _ in range(50):
        P = rng.dirichlet(np.ones(V), g2 + 1)
        Qr = rng.dirichlet(np.ones(V), g2 + g1)
        w, u1, v1, u2 = _two_level_inputs(rng, V, g1, g2)
        # r = q: every level-1 round keeps all gamma1 drafts, so the chain is
        # drafts and bonus tokens in rounds of gamma1 + 1
        cand, n2, nxt, rounds = oracle.two_level_accept(P, Qr, Qr[:-1], w, u1, v1, u2, g1, g2, 1.0, probs=True)
        assert rounds == -(-g2 // (g1 + 1))
        for t in range(g2):
            if t % (g1 + 1) < g1:     # a draft position: the drafter's own sample, kept
                assert cand[t] == oracle.inverse_cdf(Qr[t], w[t])
        # q = p on the candidate positions: level 2 keeps every candidate
        cand, n2, nxt, rounds = oracle.two_level_accept(Qr[:g2 + 1], Qr, rng.dirichlet(np.ones(V), g2 + g1 - 1),
                                                        w, u1, v1, u2, g1, g2, 1.0, probs=True)
        assert n2 == g2 and len(cand) == g2
        assert nxt == oracle.inverse_cdf(Qr[g2], u2[g2])


def test_two_level_is_lossless_statistically():
    """The first candidate Force 2 passes on is distributed as q_0, and the
    first token the step emits as p_0; given the first candidate is kept by
    Force 3, the second emitted token is distributed as p_1 (blog, '2. Dual
    Rejection Sampling': the intermediate approximations cancel)."""
    rng = np.random.default_rng(67)
    V, g1, g2, trials = 6, 2, 3, 25000
    P = rng.dirichlet(np.ones(V) * 0.8, g2 + 1)
    Qr = rng.dirichlet(np.ones(V) * 0.8, g2 + g1)
    R = rng.dirichlet(np.ones(V) * 0.8, g2 + g1 - 1)
    Qr[0, 2] = 0.0
    Qr[0] /= Qr[0].sum()       # a token Force 2 never passes on at position 0
    cand0 = np.zeros(V, np.int64)
    first = np.zeros(V, np.int64)
    second = np.zeros(V, np.int64)
    for _ in range(trials):
        w, u1, v1, u2 = _two_level_inputs(rng, V, g1, g2)
        cand, n2, nxt, _ = oracle.two_level_accept(P, Qr, R, w, u1, v1, u2, g1, g2, 1.0, probs=True)
        emitted = cand[:n2] + [nxt]
        cand0[cand[0]] += 1
        first[emitted[0]] += 1
        if n2 >= 1:
            second[emitted[1]] += 1
    for counts, ref in ((cand0, Qr[0]), (first, P[0]), (second, P[1])):
        ok, stat, crit = chi2_ok(counts, ref)
        assert ok, (stat, crit)


def test_inverse_cdf_never_draws_zero_weight():
    r = np.array([0.0, 0.3, 0.0, 0.0, 0.7, 0.0])
    for u in np.linspace(1e-9, 1 - 1e-9, 2001):
        assert oracle.inverse_cdf(r, u) in (1, 4)
    assert oracle.inverse_cdf(r, 0.3 / 1.0) == 4   # u*Z on a running sum -> strictly past it


# ---------------------------------------------------------------------------
# multi-query sparse verification with a causal tail
# ---------------------------------------------------------------------------

def test_sparse_verify_full_selection_and_tail_is_full_verify():
    rng = np.random.default_rng(59)
    n, Q, cs = 203, 5, 8
    qs, K, V = rng.standard_normal((Q, 128)), rng.standard_normal((n, 128)), rng.standard_normal((n, 128))
    C = -(-n // cs)
    o, lse = oracle.sparse_verify_attn(qs, K, V, n, list(range(C)), cs, tail=Q)
    o2, lse2 = oracle.verify_attn(qs, K, V, n)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)
    o, lse = oracle.sparse_verify_attn(qs, K, V, n, [-1] * 4, cs, tail=n)  # tail covers everything
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)


def test_sparse_verify_rows_match_masked_library_attention():
    rng = np.random.default_rng(61)
    n, Q, cs, tail = 100, 3, 8, 10
    qs, K, V = rng.standard_normal((Q, 128)), rng.standard_normal((n, 128)), rng.standard_normal((n, 128))
    idx = [2, 7, 11, 12, -1]   # chunk 11 straddles the tail start 90, chunk 12 lies inside it
    o, _ = oracle.sparse_verify_attn(qs, K, V, n, idx, cs, tail)
    for i in range(Q):
        mask = np.zeros(n, bool)
        mask[16:24] = True      # chunk 2
        mask[56:64] = True      # chunk 7
        mask[88:90] = True      # chunk 11 below the tail
        mask[90:n - Q + i + 1] = True
        np.testing.assert_allclose(o[i], sdpa(qs[i], K, V, mask), rtol=1e-12, atol=1e-13)
    # no chunk selected: the tail alone, i.e. verification of the last `tail` rows
    o, _ = oracle.sparse_verify_attn(qs, K, V, n, [-1], cs, tail)
    o2, _ = oracle.verify_attn(qs, K[n - tail:], V[n - tail:], tail)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# cache maintenance: a decode loop against a plain list model
# ---------------------------------------------------------------------------

def test_commit_length_closed_forms():
    assert oracle.commit_length(10, 7) == 17
    assert oracle.commit_length(17, 0, gamma=6, n_accepted=2) == 13     # 4 rejected drafts leave
    assert oracle.commit_length(17, 0, gamma=6, n_accepted=6) == 17     # all kept
    assert oracle.commit_length(17, 0, gamma=6, n_accepted=9) == 17     # clamped to gamma
    assert oracle.commit_length(17, 0, gamma=6, n_accepted=-3) == 11    # clamped to 0
    assert oracle.commit_length(2, 0, gamma=6, n_accepted=0) == 0       # never below 0


def test_full_cache_decode_loop_matches_list_model():
    rng = np.random.default_rng(71)
    cap, d = 120, 4
    rows = np.full((cap, d), 1000.0)
    model = [rng.standard_normal(d) for _ in range(20)]
    rows[:20] = np.array(model)
    n = 20
    no_room = 0
    for step in range(60):
        gamma = int(rng.integers(1, 7))
        new = rng.standard_normal((gamma + 1, d))
        rows2, st = oracle.append_full(rows, n, new)
        if n + gamma + 1 > cap:
            assert st == oracle.APPEND_NO_ROOM and np.array_equal(rows2, rows)
            no_room += 1
            n = oracle.commit_length(n, 0, gamma, 0) if n > 60 else n   # free some room
            model = model[:n]
            continue
        assert st == oracle.APPEND_OK
        rows = rows2
        n = oracle.commit_length(n, gamma + 1)
        model += list(new)
        n_acc = int(rng.integers(0, gamma + 1))
        n = oracle.commit_length(n, 0, gamma, n_acc)
        model = model[:len(model) - (gamma - n_acc)]
        assert n == len(model)
        np.testing.assert_array_equal(rows[:n], np.array(model))
    assert no_room > 0
    assert oracle.append_full(rows, -1, new)[1] == oracle.APPEND_BAD_LENGTH


@pytest.mark.parametrize("n_sink,window,slack", [(4, 10, 6), (0, 7, 3), (2, 1, 5)])
def test_ring_decode_loop_matches_list_model(n_sink, window, slack):
    # Force 1 drafts one row at a time (gamma1 appends of R = 1 with
    # reserve = gamma1), then Force 2's result rolls the rejected ones back.
    rng = np.random.default_rng(73 + window)
    d, cap = 3, n_sink + window + slack
    slots = np.full((cap, d), 1000.0)
    model = []
    n = 0
    for step in range(150):
        g1 = int(rng.integers(1, slack + 1))
        for r in range(g1):
            row = rng.standard_normal((1, d))
            slots, st = oracle.append_ring(slots, n, n_sink, window, row, reserve=g1)
            assert st == oracle.APPEND_OK
            n = oracle.commit_length(n, 1)
            model.append(row[0])
            # every intermediate length is readable
            pos, held = oracle.ring_visible(slots, n, n_sink, window)
            np.testing.assert_array_equal(held, np.array(model)[pos])
        n_acc = int(rng.integers(0, g1 + 1))
        n = oracle.commit_length(n, 0, g1, n_acc)
        model = model[:n]
        pos, held = oracle.ring_visible(slots, n, n_sink, window)
        np.testing.assert_array_equal(held, np.array(model)[pos] if n else np.zeros((0, d)))
    # the ring's attention equals streaming attention over the logical sequence
    q = rng.standard_normal(d)
    pos, held = oracle.ring_visible(slots, n, n_sink, window)
    o_ring, l_ring = oracle.attention(q, held, held[:, ::-1])
    L = np.array(model)
    o_log, l_log = oracle.stream_attn_masked(q, L, L[:, ::-1], n, n_sink, window)
    np.testing.assert_allclose(o_ring, o_log, rtol=1e-13, atol=1e-14)
    assert abs(l_ring - l_log) < 1e-12


def test_ring_without_slack_refuses_and_would_corrupt():
    n_sink, window, d = 2, 5, 2
    cap = n_sink + window + 2
    slots = np.arange(cap * d, dtype=np.float64).reshape(cap, d)
    new = np.ones((3, d))
    out, st = oracle.append_ring(slots, 30, n_sink, window, new)       # reserve 3 > slack 2
    assert st == oracle.APPEND_RING_TOO_SMALL and np.array_equal(out, slots)
    # what the check prevents: writing anyway overwrites a position that is
    # visible again after rolling the three rows back
    forced = slots.copy()
    for r in range(3):
        forced[oracle.ring_slot_of(30 + r, n_sink, cap)] = new[r]
    vis_slots = {oracle.ring_slot_of(int(p), n_sink, cap) for p in oracle.stream_positions(30, n_sink, window)}
    assert any(oracle.ring_slot_of(30 + r, n_sink, cap) in vis_slots for r in range(3))
    out, st = oracle.append_ring(slots, 30, n_sink, window, new[:2])  # reserve 2 fits
    assert st == oracle.APPEND_OK


def test_ring_slot_hand_table():
    # 2 sinks, 7 slots: positions 0 and 1 keep slots 0 and 1, later positions
    # cycle through slots 2..6
    assert [oracle.ring_slot_of(p, 2, 7) for p in range(13)] == [0, 1, 2, 3, 4, 5, 6, 2, 3, 4, 5, 6, 2]
    assert [oracle.ring_slot_of(p, 0, 3) for p in range(7)] == [0, 1, 2, 0, 1, 2, 0]
