"""The seeded generators: determinism, layout, planting and ring placement."""

import numpy as np
import torch

from hierarchical_speculative_attention_amd import synth
import oracle


def test_to_bits_matches_torch_rounding():
    x = np.random.default_rng(1).standard_normal(50000).astype(np.float32) * 10
    bf = synth.to_bits(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, ref)
    h = synth.to_bits(x, "fp16")
    assert np.array_equal(h, x.astype(np.float16).view(np.uint16))


def test_attn_inputs_deterministic_and_planted():
    a = synth.make_attn_inputs(lens=[1000, 37], Hq=4, Hkv=2, dtype="bf16", Q=3, seed=0,
                               chunk_size=8, plant="count", plant_count=5, cap_extra=9)
    b = synth.make_attn_inputs(lens=[1000, 37], Hq=4, Hkv=2, dtype="bf16", Q=3, seed=0,
                               chunk_size=8, plant="count", plant_count=5, cap_extra=9)
    assert np.array_equal(a.K, b.K) and np.array_equal(a.q_verify, b.q_verify)
    assert np.array_equal(a.q_verify[:, :, 0], a.q_draft[:, :, 0])
    lay = a.layout
    assert lay.seq_cap.tolist() == [1009, 46]
    for bi in range(2):
        assert len(a.planted[bi]) == 5
        for g in range(2):
            tail = lay.head(a.K, bi, g, rows=int(lay.seq_cap[bi]))[int(lay.seq_len[bi]):]
            assert np.all(oracle.widen(tail, "bf16") == synth.POISON)
    # planted rows correlate with the group's mean draft query
    K0 = oracle.widen(lay.head(a.K, 0, 0), "bf16")
    qbar = oracle.widen(a.q_draft[0, 0:2, 0], "bf16").mean(axis=0)
    c = int(a.planted[0][0])
    planted_dot = (K0[c * 8:(c + 1) * 8] @ qbar).mean()
    assert planted_dot > 0.25 * (qbar @ qbar)


def test_stream_ring_placement():
    s = synth.make_stream_inputs(lens=[1000, 100, 3], Hq=2, Hkv=2, dtype="fp16", n_sink=4, window=20, slack=5)
    cap = 4 + 20 + 5
    for b, n in enumerate([1000, 100, 3]):
        vis = oracle.stream_positions(n, 4, 20)
        for g in range(2):
            slots = s.layout.head(s.Ks, b, g, rows=cap)
            owned = set()
            for p in vis:
                sl = synth.ring_slot(int(p), 4, cap)
                owned.add(sl)
                assert np.array_equal(slots[sl], s.K_logical[b][g, p])
            for sl in range(cap):
                if sl not in owned:
                    assert np.all(oracle.widen(slots[sl], "fp16") == synth.POISON)


def test_accept_inputs_open_interval():
    a = synth.make_accept_inputs(B=3, gamma=4, vocab=100, seed=0)
    assert a.target.shape == (3, 5, 100) and a.draft.shape == (3, 4, 100)
    assert np.all((a.uniforms > 0) & (a.uniforms < 1))
    assert a.tokens.dtype == np.int32 and a.tokens.max() < 100
