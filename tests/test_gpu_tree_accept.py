"""GPU parity of the accept walk over candidate trees (tf_tree_accept):
bit-exact against the oracle's tree_accept given the same uniforms, equal to
tf_accept on chains, and statistically lossless with siblings drafted
independently from their parent's distribution."""

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
from hierarchical_speculative_attention_amd import synth
import hierarchical_speculative_attention_amd as tf

pytestmark = pytest.mark.gpu


def d(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def random_tree(rng, Q):
    par = [-1]
    for c in range(1, Q):
        par.append(int(rng.integers(max(0, c - 3), c)) if rng.random() > 0.1 else int(rng.choice([-1, c, -4])))
    return par


def draft_tokens(rng, draft, parent, T, V):
    tok = [0]
    for c in range(1, len(parent)):
        pc = parent[c] if 0 <= parent[c] < c else 0
        q = oracle.distribution(draft[pc], T if T > 0 else 1.0)
        tok.append(int(rng.choice(V, p=q / q.sum())) if rng.random() > 0.05 else int(rng.choice([-1, V + 2])))
    return tok


@pytest.mark.parametrize("T,probs,V", [(1.0, False, 32000), (float(np.float32(0.6)), False, 5000), (0.0, False, 777),
                                       (1.0, True, 50), (1.0, False, 65536)])
def test_tree_accept_matches_oracle(T, probs, V):
    rng = np.random.default_rng(121 + V)
    B, Q = 24, 9
    if probs:
        target = rng.dirichlet(np.ones(V) * 0.5, (B, Q)).astype(np.float32)
        draft = rng.dirichlet(np.ones(V) * 0.5, (B, Q)).astype(np.float32)
    else:
        target = rng.normal(0, 2, (B, Q, V)).astype(np.float32)
        draft = (target + rng.normal(0, 0.8, (B, Q, V))).astype(np.float32)   # close: long kept paths
    parents = [random_tree(rng, Q) for _ in range(B)]
    tokens = np.array([draft_tokens(rng, draft[b], parents[b], T, V) for b in range(B)], np.int32)
    u = synth.open_uniforms(rng, (B, Q))
    n, path, nxt = tf.tree_accept(d(target), d(draft), d(tokens), d(np.array(parents, np.int32)), d(u), T, probs=probs)
    torch.cuda.synchronize()
    n, path, nxt = n.cpu().numpy(), path.cpu().numpy(), nxt.cpu().numpy()
    checked = 0
    for b in range(B):
        rp, rx, margin = oracle.tree_accept(target[b], draft[b], tokens[b], parents[b], u[b], T, probs=probs)
        if margin < 1e-12:
            continue
        checked += 1
        assert int(n[b]) == len(rp) and list(path[b, :n[b]]) == rp and int(nxt[b]) == rx, b
        assert np.all(path[b, n[b]:] == -1)
    assert checked >= B - 2
    assert n.max() >= 2


def test_chain_tree_equals_accept():
    rng = np.random.default_rng(122)
    B, g, V = 64, 6, 32000
    a = synth.make_accept_inputs(B=B, gamma=g, vocab=V, correlated=True, seed=123)
    draft = np.concatenate([a.draft, a.draft[:, -1:]], 1)        # a leaf row (not read)
    tokens = np.concatenate([np.zeros((B, 1), np.int32), a.tokens], 1)
    parent = np.tile(np.arange(-1, g, dtype=np.int32), (B, 1))
    for T in (1.0, 0.0):
        n1, x1 = tf.accept(d(a.target), d(a.draft), d(a.tokens), d(a.uniforms), T)
        n2, path, x2 = tf.tree_accept(d(a.target), d(draft), d(tokens), d(parent), d(a.uniforms), T)
        torch.cuda.synchronize()
        assert torch.equal(n1, n2) and torch.equal(x1, x2)
        p = path.cpu().numpy()
        for b in range(B):
            k = int(n2[b])
            assert list(p[b, :k]) == list(range(1, k + 1))


def test_tree_accept_is_lossless_on_gpu():
    """100,000 sequences at once; root -> 3 children drafted from q0, each ->
    2 children drafted from q1: the first emitted token follows p_0 and, when
    a depth-1 node is kept, the second follows p_1."""
    rng = np.random.default_rng(124)
    B, V = 100000, 6
    p = rng.dirichlet(np.ones(V) * 0.8, 3)
    q = rng.dirichlet(np.ones(V) * 0.8, 2)
    parent = np.tile(np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3], np.int32), (B, 1))
    target = np.broadcast_to(np.stack([p[0], p[1], p[1], p[1]] + [p[2]] * 6).astype(np.float32), (B, 10, V))
    draft = np.broadcast_to(np.stack([q[0], q[1], q[1], q[1]] + [q[1]] * 6).astype(np.float32), (B, 10, V))
    tokens = np.concatenate([np.zeros((B, 1), np.int64), rng.choice(V, (B, 3), p=q[0]), rng.choice(V, (B, 6), p=q[1])],
                            1).astype(np.int32)
    u = synth.open_uniforms(rng, (B, 10))
    n, path, nxt = tf.tree_accept(d(target), d(draft), d(tokens), d(parent), d(u), 1.0, probs=True)
    torch.cuda.synchronize()
    n, path, nxt = n.cpu().numpy(), path.cpu().numpy(), nxt.cpu().numpy()
    first = np.where(n >= 1, tokens[np.arange(B), np.maximum(path[:, 0], 0)], nxt)
    kept = n >= 1
    second = np.where(n[kept] >= 2, tokens[np.arange(B)[kept], np.maximum(path[kept, 1], 0)], nxt[kept])
    for samples, ref in ((first, p[0]), (second, p[1])):
        ref = ref.astype(np.float32).astype(np.float64)
        counts = np.bincount(samples, minlength=V)
        exp = ref / ref.sum() * counts.sum()
        nz = exp > 0
        stat = ((counts[nz] - exp[nz]) ** 2 / exp[nz]).sum()
        assert stat < scipy.stats.chi2.ppf(1 - 1e-3, nz.sum() - 1), stat


@pytest.mark.parametrize("V", [1, 63, 64, 65, 1025, 2049, 4097])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_tree_accept_edge_shapes(V, T):
    """Vocabularies at the draw's segment and the statistics' slice
    boundaries, a single node (a pure draw from p_0), two nodes, and greedy
    rows full of tied maxima (ties go to the lowest index)."""
    rng = np.random.default_rng(125 + V + int(T))
    B = 6
    for Q in (1, 2, 5):
        if T == 0.0:
            target = rng.integers(0, 3, (B, Q, V)).astype(np.float32)   # many tied maxima
            draft = rng.integers(0, 3, (B, Q, V)).astype(np.float32)
        else:
            target = rng.normal(0, 2, (B, Q, V)).astype(np.float32)
            draft = (target + rng.normal(0, 0.8, (B, Q, V))).astype(np.float32)
        parents = [random_tree(rng, Q) for _ in range(B)]
        tokens = np.array([draft_tokens(rng, draft[b], parents[b], T, V) for b in range(B)], np.int32)
        u = synth.open_uniforms(rng, (B, Q))
        n, path, nxt = tf.tree_accept(d(target), d(draft), d(tokens), d(np.array(parents, np.int32)), d(u), T)
        torch.cuda.synchronize()
        n, path, nxt = n.cpu().numpy(), path.cpu().numpy(), nxt.cpu().numpy()
        checked = 0
        for b in range(B):
            rp, rx, margin = oracle.tree_accept(target[b], draft[b], tokens[b], parents[b], u[b], T)
            if margin < 1e-12:
                continue
            checked += 1
            assert int(n[b]) == len(rp) and int(nxt[b]) == rx, (Q, b)
            if Q > 1:
                assert list(path[b, :n[b]]) == rp and np.all(path[b, n[b]:] == -1), (Q, b)
        assert checked >= B - 2, (Q, checked)


@pytest.mark.parametrize("Q", [2, 3, 4, 9])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_tree_accept_many_siblings(Q, T):
    """A root with Q - 1 children drafted independently of the target: most
    are rejected, so the walk uses the precomputed normalisers for the first
    two rejections at a node, and the in-walk passes (and its own draw) from
    the third on; bit-exact against the oracle."""
    rng = np.random.default_rng(126 + Q + int(T))
    B, V = 32, 32000
    target = rng.normal(0, 2, (B, Q, V)).astype(np.float32)
    draft = rng.normal(0, 2, (B, Q, V)).astype(np.float32)
    parents = [[-1] + [0] * (Q - 1) for _ in range(B)]
    tokens = np.array([draft_tokens(rng, draft[b], parents[b], T, V) for b in range(B)], np.int32)
    u = synth.open_uniforms(rng, (B, Q))
    n, path, nxt = tf.tree_accept(d(target), d(draft), d(tokens), d(np.array(parents, np.int32)), d(u), T)
    torch.cuda.synchronize()
    n, path, nxt = n.cpu().numpy(), path.cpu().numpy(), nxt.cpu().numpy()
    checked = 0
    for b in range(B):
        rp, rx, margin = oracle.tree_accept(target[b], draft[b], tokens[b], parents[b], u[b], T)
        if margin < 1e-12:
            continue
        checked += 1
        assert int(n[b]) == len(rp) and list(path[b, :n[b]]) == rp and int(nxt[b]) == rx, b
    assert checked >= B - 2
