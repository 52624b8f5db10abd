"""A decode step captured as a HIP graph replays to exactly the eager
results, replay after replay, with unrelated eager work in between (the
benchmark times such replays)."""

import numpy as np
import pytest
import torch

from hierarchical_speculative_attention_amd import synth, KVDesc
import hierarchical_speculative_attention_amd as tf
from tests.gpu_util import desc, dev

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    cs, k, S, W, gamma = 8, 64, 4, 252, 4
    Q = gamma + 1
    inp = synth.make_attn_inputs(lens=[5000, 3001], Hq=8, Hkv=4, dtype="bf16", Q=Q, seed=30,
                                 chunk_size=cs, plant="count", plant_count=4)
    lay = inp.layout
    B = lay.B
    kv = desc(lay, "bf16")
    K, V = dev(inp.K, "bf16"), dev(inp.V, "bf16")
    qv, qd = dev(inp.q_verify, "bf16"), dev(inp.q_draft, "bf16").view(B, 8, 128)
    C = [-(-int(n) // cs) for n in lay.seq_len]
    ckl = synth.KVLayout.build(C, 4, 128, caps=C)
    ckd = KVDesc.from_layout(ckl, torch.bfloat16, "cuda")
    ck = torch.zeros(ckl.total_elems, dtype=torch.bfloat16, device="cuda")
    tf.build_chunk_keys(K, kv, cs, ck, ckd)
    st = synth.make_stream_inputs(lens=[5000, 3001], Hq=8, Hkv=4, dtype="bf16", seed=31)
    sd = desc(st.layout, "bf16")
    Ks, Vs = dev(st.Ks, "bf16"), dev(st.Vs, "bf16")
    a = synth.make_accept_inputs(B=B, gamma=gamma, vocab=32000, seed=32)
    tg, dr = torch.from_numpy(a.target).cuda(), torch.from_numpy(a.draft).cuda()
    tk, un = torch.from_numpy(a.tokens).cuda(), torch.from_numpy(a.uniforms).cuda()
    c_max = max(C)
    n_ch = torch.tensor(C, dtype=torch.int32, device="cuda")
    tail = torch.tensor([max(0, (int(n) - Q) // cs) for n in lay.seq_len], dtype=torch.int32, device="cuda")
    outs = dict(scores=torch.empty((B, 4, c_max), device="cuda"),
                idx=torch.empty((B, 4, k), dtype=torch.int32, device="cuda"),
                o_sp=torch.empty((B, 8, 128), device="cuda"), l_sp=torch.empty((B, 8), device="cuda"),
                o_st=torch.empty((B, 8, 128), device="cuda"), l_st=torch.empty((B, 8), device="cuda"),
                o_v=torch.empty((B, 8, Q, 128), device="cuda"), l_v=torch.empty((B, 8, Q), device="cuda"),
                n_acc=torch.empty(B, dtype=torch.int32, device="cuda"),
                nxt=torch.empty(B, dtype=torch.int32, device="cuda"))
    ws_v = tf.workspace(tf.verify_attn_workspace_size(B, 8, 4, Q, kv.max_len), "cuda")
    ws_s = tf.workspace(tf.sparse_attn_workspace_size(B, 8, 4, k, cs), "cuda")
    ws_a = tf.workspace(tf.accept_workspace_size(B, gamma, 32000), "cuda")
    s = torch.cuda.Stream()

    def step():
        tf.build_chunk_keys(K, kv, cs, ck, ckd, chunk_begin=tail, max_chunks=2, stream=s)
        tf.score_chunks(qd, 8, ck, ckd, c_max, scores=outs["scores"], stream=s)
        tf.select_topk(outs["scores"], n_ch, k, idx=outs["idx"], stream=s)
        tf.sparse_attn(qd, K, V, kv, outs["idx"], cs, out=outs["o_sp"], lse=outs["l_sp"], ws=ws_s, stream=s)
        tf.stream_attn(qd, Ks, Vs, sd, S, W, out=outs["o_st"], lse=outs["l_st"], stream=s)
        tf.verify_attn(qv, K, V, kv, out=outs["o_v"], lse=outs["l_v"], ws=ws_v, stream=s)
        tf.accept(tg, dr, tk, un, 1.0, n_accepted=outs["n_acc"], next_token=outs["nxt"], ws=ws_a, stream=s)

    with torch.cuda.stream(s):
        step()
    s.synchronize()
    ref = {n: t.clone() for n, t in outs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    other_q = torch.flip(qv, dims=[2]).contiguous()
    for rep in range(4):
        for t in outs.values():
            t.zero_()
        with torch.cuda.stream(s):
            # unrelated eager work that overwrites the shared workspace
            tf.verify_attn(other_q, K, V, kv, ws=ws_v, stream=s)
        g.replay()
        s.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, ref[n]), (rep, n)


def test_sliced_topk_graph_replays():
    """Few long rows (8 rows of 32768 chunks) take the slice-and-merge top-k;
    a graph of it replays to the eager result and to the oracle for new
    scores written into the captured buffer between replays, with eager
    calls on other scores overwriting the shared workspace in between."""
    import oracle
    B, rows, C, k = 1, 8, 32768, 512
    ws = tf.workspace(tf.select_topk_workspace_size(B, rows, C, k), "cuda")
    assert ws is not None
    n = torch.tensor([C - 7], dtype=torch.int32, device="cuda")
    scores = torch.empty((B, rows, C), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, rows, k), dtype=torch.int32, device="cuda")
    other = torch.randn((B, rows, C), device="cuda")
    other_idx = torch.empty_like(idx)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        scores.normal_()
        tf.select_topk(scores, n, k, idx=idx, ws=ws, stream=s)  # warm-up before capture
    s.synchronize()
    with torch.cuda.graph(g, stream=s):
        tf.select_topk(scores, n, k, idx=idx, ws=ws, stream=s)
    rng = np.random.default_rng(31)
    for rep in range(3):
        host = (rng.standard_normal((B, rows, C)) * 2).astype(np.float32)
        host[:, :, rng.choice(C, 300)] = 4.5           # ties near the threshold
        with torch.cuda.stream(s):
            scores.copy_(torch.from_numpy(host).to("cuda"))
            tf.select_topk(other, n, k, idx=other_idx, ws=ws, stream=s)
            idx.fill_(-2)
        g.replay()
        s.synchronize()
        got = idx.cpu().numpy()
        eager = tf.select_topk(scores, n, k).cpu().numpy()
        assert np.array_equal(got, eager), rep
        for r in range(rows):
            assert np.array_equal(got[0, r], oracle.select_topk(host[0, r, :C - 7].astype(np.float64), k)), (rep, r)
