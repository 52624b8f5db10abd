"""Parity at the full workload sizes, in the launch configuration the
benchmark uses: every entry point runs over the whole layer on the GPU, and
the oracle recomputes sampled (sequence, head) slices on the host from the
same inputs (generated on the device and copied back)."""

import numpy as np
import pytest
import torch

import oracle
from hierarchical_speculative_attention_amd import synth, KVDesc
import hierarchical_speculative_attention_amd as tf
from tests.gpu_util import ATOL, host_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def layer(name, Q, layer_id=0):
    W = synth.WORKLOADS[name]
    K, V, qv, qd, lay, planted = synth.make_layer_torch(
        lens=W["lens"], Hq=W["Hq"], Hkv=W["Hkv"], d=128, dtype=W["dtype"], Q=Q, chunk_size=W["chunk_size"],
        plant=W["plant"], seed=0, layer=layer_id, device=DEV, plant_fraction=W.get("plant_fraction", 0.01),
        plant_count=W.get("plant_count", 0), zipf_s=W.get("zipf_s", 1.1))
    return W, K, V, qv, qd, lay, planted


def head_rows(flat_bits, lay, b, g):
    n = int(lay.seq_len[b])
    off = int(lay.seq_base[b]) + g * int(lay.seq_cap[b]) * 128
    return oracle.widen(flat_bits[off:off + n * 128].reshape(n, 128), "bf16")


def head_bits_gpu(t, lay, b, g):
    n = int(lay.seq_len[b])
    off = int(lay.seq_base[b]) + g * int(lay.seq_cap[b]) * 128
    return host_bits(t[off:off + n * 128])


def retrieval(W, K, qd, lay, budget):
    cs = W["chunk_size"]
    kv = KVDesc.from_layout(lay, torch.bfloat16, DEV)
    C = [-(-int(n) // cs) for n in lay.seq_len]
    ckl = synth.KVLayout.build(C, W["Hkv"], 128, caps=C)
    ckd = KVDesc.from_layout(ckl, torch.bfloat16, DEV)
    ck = torch.empty(ckl.total_elems, dtype=torch.bfloat16, device=DEV)
    tf.build_chunk_keys(K, kv, cs, ck, ckd)
    q = qd.view(lay.B, W["Hq"], 128)
    scores = tf.score_chunks(q, W["Hq"], ck, ckd, max(C))
    idx = tf.select_topk(scores, torch.tensor(C, dtype=torch.int32, device=DEV), budget // cs)
    torch.cuda.synchronize()
    return kv, ck, ckl, scores, idx


def errs(o_gpu, o_ref, l_gpu, l_ref, acc):
    """Fold the errors of one head's rows into acc (max abs / max relative of
    o, relative to the largest |o| of the row, and of lse)."""
    do = np.abs(o_gpu - o_ref).max()
    acc["o_abs"] = max(acc["o_abs"], float(do))
    acc["o_rel"] = max(acc["o_rel"], float(do / max(np.abs(o_ref).max(), 1e-30)))
    acc["o_max"] = max(acc["o_max"], float(np.abs(o_ref).max()))
    dl = np.abs(np.asarray(l_gpu) - np.asarray(l_ref)).max()
    acc["lse_abs"] = max(acc["lse_abs"], float(dl))
    acc["lse_rel"] = max(acc["lse_rel"], float(dl / max(np.abs(np.asarray(l_ref)).max(), 1e-30)))
    return do, dl


def new_acc():
    return {"o_abs": 0.0, "o_rel": 0.0, "o_max": 0.0, "lse_abs": 0.0, "lse_rel": 0.0}


# A check of the arithmetic tighter than the 2e-3 bar, which at 128K context
# is loose (|o| is 1e-2 to 3e-1 here): the kernels keep each probability to
# about 16 significant bits (a 16-bit high part and a 16-bit remainder) and
# accumulate in fp32, so on these inputs, whose rounding errors are
# independent, an output is off by about 2^-16 |v| sqrt(sum p^2), some 1e-7
# (observed 2e-8 to 7e-7).  The guards sit 60x (lse) and 300x (o, relative)
# above what is seen.
O_REL_GUARD = 1e-3   # max |do| / max |o| over the checked rows
LSE_GUARD = 1e-4     # max |dlse|


def report(name, errs_by_kind):
    """Print the observed error margins under the 2e-3 bar (shown with -s / -rP)
    and hold them to the tighter guards above."""
    for kind, a in errs_by_kind.items():
        print(f"{name} {kind}: max|do| {a['o_abs']:.2e} (rel {a['o_rel']:.2e}, max|o| {a['o_max']:.2e}), "
              f"max|dlse| {a['lse_abs']:.2e} (rel {a['lse_rel']:.2e}); bar {ATOL:.0e}")
        assert a["o_rel"] <= O_REL_GUARD, (name, kind, a)
        assert a["lse_abs"] <= LSE_GUARD, (name, kind, a)


def check_head(W, lay, b, g, Kh, Vh, ck_h, scores_h, idx_h, qd_h, qv_h, o_sp, l_sp, o_v, l_v, Q, budget, acc):
    """Kh, Vh: fp64 rows of this head; *_h: GPU results of this (b, g);
    acc: {"sparse": ..., "verify": ...} error records (updated)."""
    cs = W["chunk_size"]
    G = W["Hq"] // W["Hkv"]
    n = Kh.shape[0]
    k = budget // cs
    # a1: sampled chunks (first, last partial/full, random) against the mean
    C = -(-n // cs)
    rng = np.random.default_rng(b * 1000 + g)
    for c in set([0, C - 1] + rng.integers(0, C, 64).tolist()):
        mean = Kh[c * cs:min(n, (c + 1) * cs)].mean(axis=0)
        exact = oracle.widen(oracle.round_f64_to_bits(mean, "bf16"), "bf16")
        mism = ck_h[c] != exact
        assert np.all(np.abs(ck_h[c] - mean)[mism] <= np.abs(exact[mism]) * 2.0 ** -8 * (1 + 1e-5) + 1e-7)
    # a2: scores given the GPU chunk keys
    qg = qd_h  # [G][128] fp64
    ref = oracle.chunk_scores(qg, ck_h[:C])
    scale = np.linalg.norm(qg.sum(0)) * np.linalg.norm(ck_h[:C], axis=1) + 1e-6
    assert np.all(np.abs(scores_h[:C] - ref) <= 1e-5 * scale)
    # a3: bit-exact given the GPU scores
    assert np.array_equal(idx_h, oracle.select_topk(scores_h[:C].astype(np.float64), k))
    # a4: given the GPU indices
    for j in range(G):
        o, l = oracle.sparse_attn(qg[j], Kh, Vh, n, idx_h, cs)
        do, dl = errs(o_sp[j], o, l_sp[j], l, acc["sparse"])
        assert do <= ATOL and dl <= ATOL
    # a6
    for j in range(G):
        o, l = oracle.verify_attn(qv_h[j], Kh, Vh, n)
        do, dl = errs(o_v[j], o, l_v[j], l, acc["verify"])
        assert do <= ATOL and dl <= ATOL


def run_full(name, Q, budget, samples):
    W, K, V, qv, qd, lay, planted = layer(name, Q)
    kv, ck, ckl, scores, idx = retrieval(W, K, qd, lay, budget)
    cs = W["chunk_size"]
    B, Hq, Hkv = lay.B, W["Hq"], W["Hkv"]
    G = Hq // Hkv
    q = qd.view(B, Hq, 128)
    o_sp, l_sp = tf.sparse_attn(q, K, V, kv, idx, cs)
    o_v, l_v = tf.verify_attn(qv, K, V, kv)
    torch.cuda.synchronize()
    ck_all = oracle.widen(host_bits(ck), "bf16")
    sc, ix = scores.cpu().numpy(), idx.cpu().numpy()
    qd_b, qv_b = host_bits(qd), host_bits(qv)
    osp, lsp, ov, lv = (t.cpu().double().numpy() for t in (o_sp, l_sp, o_v, l_v))
    acc = {"sparse": new_acc(), "verify": new_acc()}
    for b, g in samples:
        Kh = oracle.widen(head_bits_gpu(K, lay, b, g).reshape(-1, 128), "bf16")
        Vh = oracle.widen(head_bits_gpu(V, lay, b, g).reshape(-1, 128), "bf16")
        C = -(-int(lay.seq_len[b]) // cs)
        ck_h = ckl.head(ck_all, b, g, rows=C)
        hs = slice(g * G, (g + 1) * G)
        check_head(W, lay, b, g, Kh, Vh, ck_h, sc[b, g], ix[b, g],
                   oracle.widen(qd_b[b, hs, 0], "bf16"), oracle.widen(qv_b[b, hs], "bf16"),
                   osp[b, hs], lsp[b, hs], ov[b, hs], lv[b, hs], Q, budget, acc)
        if W["plant"] == "fraction":
            # retrieval works: every planted chunk of the row is selected
            assert set(planted[b].tolist()) <= set(ix[b, g].tolist())
        elif W["plant"] == "zipf":
            # the most relevant chunk of the power law is selected
            assert int(planted[b][g][0]) in set(ix[b, g].tolist())
    report(f"{name} Q={Q} budget={budget} samples={samples}", acc)
    return W, lay, ix


def test_llama2_7b_128k_layer():
    run_full("llama2-7b-128k-1layer", Q=7, budget=4096, samples=[(0, 0), (0, 17), (0, 31)])


@pytest.mark.parametrize("budget,gamma", [(2048, 4), (2048, 6), (2048, 8), (4096, 4), (4096, 6), (4096, 8)])
def test_ragged_batch(budget, gamma):
    run_full("ragged-b8-16k-128k", Q=gamma + 1, budget=budget, samples=[(0, 3), (3, 30), (7, 12), (5, 0), (7, 31)])


def test_gqa_512k_layer():
    # the first and last KV heads (each with its 4 query heads x 9 rows) and one between
    W, lay, ix = run_full("gqa-hq32-hkv8-512k-16layers", Q=9, budget=8192, samples=[(0, 0), (0, 5), (0, 7)])
    assert ix.shape == (1, 8, 512)


def test_stream_full_logical_length():
    # logical length 131072, 32 heads, 4 sinks + 252 window in a 272-slot ring
    n, H, S, Wn = 131072, 32, 4, 252
    cap = S + Wn + synth.STREAM_SLACK
    lay = synth.KVLayout.build([n], H, 128, caps=[cap])
    g = torch.Generator(device=DEV).manual_seed(5)
    Ks = torch.randn(lay.total_elems, generator=g, device=DEV).to(torch.bfloat16)
    Vs = torch.randn(lay.total_elems, generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randn((1, H, 128), generator=g, device=DEV).to(torch.bfloat16)
    sd = KVDesc.from_layout(lay, torch.bfloat16, DEV)
    out, lse = tf.stream_attn(q, Ks, Vs, sd, S, Wn)
    torch.cuda.synchronize()
    Kb, Vb, qb = host_bits(Ks), host_bits(Vs), host_bits(q)
    o_h, l_h = out.cpu().double().numpy(), lse.cpu().double().numpy()
    vis = oracle.stream_positions(n, S, Wn)
    acc = new_acc()
    for h in [0, 9, 31]:
        slots = lay.head(Kb, 0, h, rows=cap)
        vslots = lay.head(Vb, 0, h, rows=cap)
        K_log = np.zeros((n, 128))
        V_log = np.zeros((n, 128))
        for p in vis:
            K_log[p] = oracle.widen(slots[synth.ring_slot(int(p), S, cap)], "bf16")
            V_log[p] = oracle.widen(vslots[synth.ring_slot(int(p), S, cap)], "bf16")
        o, l = oracle.stream_attn_masked(oracle.widen(qb[0, h], "bf16"), K_log, V_log, n, S, Wn)
        do, dl = errs(o_h[0, h], o, l_h[0, h], l, acc)
        assert do <= ATOL and dl <= ATOL
    report("stream 131072 logical", {"stream": acc})


def test_llama2_7b_128k_sparse_verify_with_tail():
    # Force 2 verifying gamma1 = 4 drafted rows over the retrieved 4096 tokens + a 64-row tail
    Q, tail = 5, 64
    W, K, V, qv, qd, lay, planted = layer("llama2-7b-128k-1layer", Q)
    kv, ck, ckl, scores, idx = retrieval(W, K, qd, lay, W["budget"])
    out, lse = tf.sparse_verify_attn(qv, K, V, kv, idx, W["chunk_size"], tail)
    torch.cuda.synchronize()
    ix, qv_b = idx.cpu().numpy(), host_bits(qv)
    o_h, l_h = out.cpu().double().numpy(), lse.cpu().double().numpy()
    acc = new_acc()
    for g in [0, 21]:
        Kh = oracle.widen(head_bits_gpu(K, lay, 0, g).reshape(-1, 128), "bf16")
        Vh = oracle.widen(head_bits_gpu(V, lay, 0, g).reshape(-1, 128), "bf16")
        o, l = oracle.sparse_verify_attn(oracle.widen(qv_b[0, g], "bf16"), Kh, Vh, Kh.shape[0], ix[0, g],
                                         W["chunk_size"], tail)
        do, dl = errs(o_h[0, g], o, l_h[0, g], l, acc)
        assert do <= ATOL and dl <= ATOL
    report("llama2-7b-128k sparse verification, tail 64", {"sparse_verify": acc})


def test_llama2_7b_128k_verify_in_a_larger_allocation():
    # 512 rows allocated past the sequence (the three-tier loop's cache): the
    # split plan takes one round of 16 splits of 8192 rows and a short 17th
    # split per head, dispatched after all the others (a 1-D grid); parity on
    # heads of the first and last XCD groups
    Q = 7
    W = synth.WORKLOADS["llama2-7b-128k-1layer"]
    K, V, qv, qd, lay, _ = synth.make_layer_torch(
        lens=W["lens"], Hq=W["Hq"], Hkv=W["Hkv"], d=128, dtype="bf16", Q=Q, chunk_size=W["chunk_size"],
        plant=None, seed=3, layer=0, device=DEV, extra_rows=512)
    n = int(lay.seq_len[0])
    kv = KVDesc.from_layout(lay, torch.bfloat16, DEV, max_len=n + 512)
    o_v, l_v = tf.verify_attn(qv, K, V, kv)
    torch.cuda.synchronize()
    qv_b = host_bits(qv)
    ov, lv = o_v.cpu().double().numpy(), l_v.cpu().double().numpy()
    acc = new_acc()
    for g in (0, 13, 31):
        Kh = oracle.widen(head_bits_gpu(K, lay, 0, g).reshape(-1, 128), "bf16")
        Vh = oracle.widen(head_bits_gpu(V, lay, 0, g).reshape(-1, 128), "bf16")
        o, l = oracle.verify_attn(oracle.widen(qv_b[0, g], "bf16"), Kh, Vh, n)
        do, dl = errs(ov[0, g], o, lv[0, g], l, acc)
        assert do <= ATOL and dl <= ATOL
    report("llama2-7b-128k verify, 512 rows allocated past n", {"verify": acc})


def test_gqa_512k_verify_in_a_larger_allocation():
    # GQA 512K (36 rows per KV head: query rows split over the waves) in a
    # cache allocated 512 rows past the sequence: one round of 64 splits of
    # 8192 rows per KV head and a short 65th, dispatched after all the others
    # (a 1-D grid); parity on the first and last KV heads
    Q = 9
    W = synth.WORKLOADS["gqa-hq32-hkv8-512k-16layers"]
    K, V, qv, qd, lay, _ = synth.make_layer_torch(
        lens=W["lens"], Hq=W["Hq"], Hkv=W["Hkv"], d=128, dtype="bf16", Q=Q, chunk_size=W["chunk_size"],
        plant=None, seed=4, layer=0, device=DEV, extra_rows=512)
    n = int(lay.seq_len[0])
    G = W["Hq"] // W["Hkv"]
    kv = KVDesc.from_layout(lay, torch.bfloat16, DEV, max_len=n + 512)
    o_v, l_v = tf.verify_attn(qv, K, V, kv)
    torch.cuda.synchronize()
    qv_b = host_bits(qv)
    ov, lv = o_v.cpu().double().numpy(), l_v.cpu().double().numpy()
    acc = new_acc()
    for g in (0, W["Hkv"] - 1):
        Kh = oracle.widen(head_bits_gpu(K, lay, 0, g).reshape(-1, 128), "bf16")
        Vh = oracle.widen(head_bits_gpu(V, lay, 0, g).reshape(-1, 128), "bf16")
        for h in range(g * G, (g + 1) * G):
            o, l = oracle.verify_attn(oracle.widen(qv_b[0, h], "bf16"), Kh, Vh, n)
            do, dl = errs(ov[0, h], o, lv[0, h], l, acc)
            assert do <= ATOL and dl <= ATOL
        del Kh, Vh
    report("gqa 512k verify, 512 rows allocated past n", {"verify": acc})
