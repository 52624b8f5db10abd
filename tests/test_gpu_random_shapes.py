"""GPU parity of the attention calls on seeded random shapes.

Each case draws a call (verification, sparse attention, sparse verification
with a causal tail, streaming attention), a dtype, a batch of ragged lengths
(empty and one-row sequences, lengths below the query count, a sequence past
several splits), query heads per KV head and query rows up to the 64 rows a
KV head takes, and, for the sparse calls, a chunk size and a selection with
padding, repeats of the last chunk and chunks past the end.  Every output
row is compared with the oracle.  The shapes fall in every split-plan and
kernel-path regime the fixed tests pick one by one: one or several splits,
one to four query tiles, sparse items with and without a slot table, split
merges in groups of 4 to 32."""

import numpy as np
import pytest
import torch

import oracle
from hierarchical_speculative_attention_amd import synth
import hierarchical_speculative_attention_amd as tf
from tests.gpu_util import compare_attn, desc, dev, oracle_sparse, oracle_verify
from tests.test_gpu_attn import oracle_sparse_verify, run_sparse, run_sparse_verify, run_verify

pytestmark = pytest.mark.gpu

CASES = 48


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    mode = ["verify", "sparse", "sparse_verify", "stream"][i % 4]
    dtype = "fp16" if rng.random() < 0.3 else "bf16"
    B = int(rng.integers(1, 7))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    Q = 1 if mode in ("sparse", "stream") else int(rng.integers(1, 10))
    G = int(rng.choice([g for g in (1, 2, 3, 4, 8, 16, 32, 64) if g * Q <= 64 and g * Hkv <= 64]))
    lens = [int(x) for x in rng.integers(0, 2500, B)]
    if B > 1:
        lens[int(rng.integers(0, B))] = int(rng.choice([0, 1, Q - 1 if Q > 1 else 2]))
    if rng.random() < 0.3:
        lens[int(rng.integers(0, B))] = int(rng.integers(5000, 12000))
    return rng, mode, dtype, lens, Hkv, G, Q


def random_idx(rng, lens, Hkv, cs, k):
    idx = np.full((len(lens), Hkv, k), -1, np.int64)
    for b, n in enumerate(lens):
        C = -(-n // cs)
        for g in range(Hkv):
            m = min(int(rng.integers(0, k + 1)), C)
            if m:
                idx[b, g, :m] = np.sort(rng.choice(C, size=m, replace=False))
            extra = [C - 1 if C else -1, C + int(rng.integers(0, 5)), -1]
            for j, v in enumerate(extra):
                if m + j < k:
                    idx[b, g, m + j] = v
    return idx


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape_matches_oracle(i):
    rng, mode, dtype, lens, Hkv, G, Q = draw_case(i)
    Hq = G * Hkv
    if mode == "stream":
        S = int(rng.integers(0, 9))
        W = int(rng.integers(1, 700))
        print(f"case {i}: stream {dtype} lens={lens} Hkv={Hkv} G={G} S={S} W={W}", flush=True)
        s = synth.make_stream_inputs(lens=lens, Hq=Hq, Hkv=Hkv, dtype=dtype, n_sink=S, window=W, seed=2000 + i)
        out, lse = tf.stream_attn(dev(s.q, dtype).view(len(lens), Hq, 128), dev(s.Ks, dtype), dev(s.Vs, dtype),
                                  desc(s.layout, dtype), S, W)
        torch.cuda.synchronize()
        o_ref = np.zeros((len(lens), Hq, 128))
        l_ref = np.zeros((len(lens), Hq))
        for b, n in enumerate(lens):
            for h in range(Hq):
                g = h // G
                o_ref[b, h], l_ref[b, h] = oracle.stream_attn_masked(
                    oracle.widen(s.q[b, h, 0], dtype), oracle.widen(s.K_logical[b][g], dtype),
                    oracle.widen(s.V_logical[b][g], dtype), n, S, W)
        compare_attn(out, lse, o_ref, l_ref)
        return
    cs = int(rng.choice([1, 3, 8, 16, 33]))
    # short selections, and long ones (mostly padding past short sequences)
    # whose workgroups take more than 256 gathered tokens
    k = int(rng.integers(1, 400 // cs + 60)) if rng.random() < 0.5 else int(rng.integers(3000, 20000)) // cs
    tail = int(rng.integers(1, 200))
    print(f"case {i}: {mode} {dtype} lens={lens} Hkv={Hkv} G={G} Q={Q} cs={cs} k={k} tail={tail}", flush=True)
    inp = synth.make_attn_inputs(lens=lens, Hq=Hq, Hkv=Hkv, dtype=dtype, Q=Q, seed=3000 + i,
                                 cap_extra=int(rng.integers(0, 9)))
    if mode == "verify":
        out, lse = run_verify(inp, Q)
        compare_attn(out, lse, *oracle_verify(inp, Q))
        return
    idx = random_idx(rng, lens, Hkv, cs, k)
    if mode == "sparse":
        out, lse = run_sparse(inp, idx, cs)
        compare_attn(out, lse, *oracle_sparse(inp, idx, cs))
    else:
        out, lse = run_sparse_verify(inp, idx, cs, tail)
        compare_attn(out, lse, *oracle_sparse_verify(inp, idx, cs, tail, Q))
