"""GPU parity of verification over a candidate tree (tf_verify_tree_attn) and
of its masks (tf_tree_masks) against the oracle, through the C ABI; chain
masks must reproduce tf_verify_attn bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from hierarchical_speculative_attention_amd import synth
import hierarchical_speculative_attention_amd as tf
from tests.gpu_util import compare_attn, desc, dev, host_bits

pytestmark = pytest.mark.gpu


def random_parents(rng, B, Q, p_root=0.15, p_bad=0.05):
    par = np.empty((B, Q), np.int32)
    for b in range(B):
        for i in range(Q):
            r = rng.random()
            if i == 0 or r < p_root:
                par[b, i] = -1
            elif r < p_root + p_bad:
                par[b, i] = rng.choice([i, i + 3, -5])          # out of range: read as -1
            else:
                par[b, i] = rng.integers(max(0, i - 4), i)     # a recent node
    return par


def oracle_tree(inp, Q, masks):
    lay, dt = inp.layout, inp.dtype
    G = inp.Hq // lay.H
    o = np.zeros((lay.B, inp.Hq, Q, lay.d))
    lse = np.zeros((lay.B, inp.Hq, Q))
    for b in range(lay.B):
        n = int(lay.seq_len[b])
        for g in range(lay.H):
            K = oracle.widen(lay.head(inp.K, b, g), dt)
            V = oracle.widen(lay.head(inp.V, b, g), dt)
            for j in range(G):
                h = g * G + j
                o[b, h], lse[b, h] = oracle.verify_tree_attn(oracle.widen(inp.q_verify[b, h], dt), K, V, n, masks[b])
    return o, lse


def test_tree_masks_match_oracle():
    rng = np.random.default_rng(111)
    for Q in (1, 7, 33, 64):
        par = random_parents(rng, 40, Q)
        got = tf.tree_masks(torch.from_numpy(par).cuda()).cpu().numpy()
        for b in range(40):
            assert got[b].view(np.uint64).tolist() == oracle.tree_masks(par[b].tolist()), (Q, b)


@pytest.mark.parametrize("dtype,Hq,Hkv,Q", [("bf16", 8, 2, 5), ("fp16", 8, 2, 9), ("bf16", 32, 8, 16),
                                            ("bf16", 4, 4, 64)])
def test_verify_tree_matches_oracle(dtype, Hq, Hkv, Q):
    # ragged lengths, some shorter than the tree (missing nodes), poison past n
    lens = [1, Q - 1 if Q > 1 else 1, Q, 37, 1000, 5003]
    rng = np.random.default_rng(112 + Q)
    inp = synth.make_attn_inputs(lens=lens, Hq=Hq, Hkv=Hkv, dtype=dtype, Q=Q, seed=113, cap_extra=11)
    par = random_parents(rng, len(lens), Q)
    masks = [oracle.tree_masks(p.tolist()) for p in par]
    tm = tf.tree_masks(torch.from_numpy(par).cuda())
    kv = desc(inp.layout, dtype)
    out, lse = tf.verify_tree_attn(dev(inp.q_verify, dtype), dev(inp.K, dtype), dev(inp.V, dtype), kv, tm)
    torch.cuda.synchronize()
    compare_attn(out, lse, *oracle_tree(inp, Q, masks))


def test_chain_tree_is_verify_bitwise():
    # long sequences: several splits per head, so the split merge is covered too
    Q = 7
    inp = synth.make_attn_inputs(lens=[70000, 12345, 6, 3], Hq=8, Hkv=4, dtype="bf16", Q=Q, seed=114)
    kv = desc(inp.layout, "bf16")
    q, K, V = dev(inp.q_verify, "bf16"), dev(inp.K, "bf16"), dev(inp.V, "bf16")
    chain = torch.tensor([[-1] + list(range(Q - 1))] * 4, dtype=torch.int32, device="cuda")
    o_t, l_t = tf.verify_tree_attn(q, K, V, kv, tf.tree_masks(chain))
    o_v, l_v = tf.verify_attn(q, K, V, kv)
    torch.cuda.synchronize()
    assert torch.equal(o_t, o_v) and torch.equal(l_t, l_v)


def test_verify_tree_llama2_7b_128k_layer():
    """The full Llama2-7B-128K layer (32 heads, n = 131072, bf16) with a
    7-node tree, in the benchmark's launch configuration; the oracle checks
    sampled heads."""
    W = synth.WORKLOADS["llama2-7b-128k-1layer"]
    Q = 7
    K, V, qv, qd, lay, planted = synth.make_layer_torch(
        lens=W["lens"], Hq=32, Hkv=32, d=128, dtype="bf16", Q=Q, chunk_size=8, plant="fraction", seed=0, layer=0,
        device=torch.device("cuda:0"), plant_fraction=0.01, plant_count=0, zipf_s=1.1)
    par = np.array([[-1, 0, 0, 1, 1, 2, -1]], np.int32)
    masks = oracle.tree_masks(par[0].tolist())
    kv = desc(lay, "bf16")
    o, lse = tf.verify_tree_attn(qv, K, V, kv, tf.tree_masks(torch.from_numpy(par).cuda()))
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    qb = host_bits(qv)
    n = int(lay.seq_len[0])
    for g in (0, 13, 31):
        off = int(lay.seq_base[0]) + g * int(lay.seq_cap[0]) * 128
        Kh = oracle.widen(host_bits(K[off:off + n * 128]).reshape(n, 128), "bf16")
        Vh = oracle.widen(host_bits(V[off:off + n * 128]).reshape(n, 128), "bf16")
        ro, rl = oracle.verify_tree_attn(oracle.widen(qb[0, g], "bf16"), Kh, Vh, n, masks)
        assert np.abs(o[0, g] - ro).max() <= 2e-3 and np.abs(lse[0, g] - rl).max() <= 2e-3
