"""GPU parity of cache maintenance (tf_append_kv, tf_commit_length) with the
oracle's append_full / append_ring / commit_length, bit-exact on the cache
bytes and on the lengths, and end to end: decode loops whose attention and
accept results are compared with the oracle over the logical sequence."""

import numpy as np
import pytest
import torch

import oracle
from hierarchical_speculative_attention_amd import synth, KVDesc
import hierarchical_speculative_attention_amd as tf
from tests.gpu_util import TDT, ATOL, dev, host_bits

pytestmark = pytest.mark.gpu

D = 128


def rows_bits(rng, shape, dtype):
    return synth.to_bits(rng.standard_normal(shape).astype(np.float32), dtype)


def kv_desc(lay, dtype, seq_len):
    return KVDesc(lay.B, lay.H, TDT[dtype], lay.seq_base, lay.seq_cap, seq_len, max(1, int(max(seq_len))), "cuda")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_append_full_matches_oracle(dtype):
    rng = np.random.default_rng(91)
    H, R = 3, 7
    caps = [40, 30, 20, 50, 9]
    lens = [10, 23, 15, -1, 2]          # room / exactly full / no room / bad length / room
    lay = synth.KVLayout.build([max(0, n) for n in lens], H, D, caps=caps)
    K = rows_bits(rng, lay.total_elems, dtype)
    V = rows_bits(rng, lay.total_elems, dtype)
    Kn = rows_bits(rng, (lay.B, H, R, D), dtype)
    Vn = rows_bits(rng, (lay.B, H, R, D), dtype)
    kv = kv_desc(lay, dtype, lens)
    Kd, Vd = dev(K, dtype), dev(V, dtype)
    st = tf.append_kv(dev(Kn, dtype), dev(Vn, dtype), Kd, Vd, kv)
    torch.cuda.synchronize()
    gotK, gotV, got_st = host_bits(Kd), host_bits(Vd), st.cpu().numpy()
    expK, expV = K.copy(), V.copy()
    for b in range(lay.B):
        for h in range(H):
            for src, new, exp in ((K, Kn, expK), (V, Vn, expV)):
                slab = lay.head(src, b, h, rows=caps[b]).astype(np.float64)
                out, s = oracle.append_full(slab, lens[b], new[b, h].astype(np.float64))
                lay.head(exp, b, h, rows=caps[b])[:] = out.astype(np.uint16)
                assert got_st[b] == s, (b, got_st[b], s)
    assert list(got_st) == [oracle.APPEND_OK, oracle.APPEND_OK, oracle.APPEND_NO_ROOM, oracle.APPEND_BAD_LENGTH,
                            oracle.APPEND_OK]
    assert np.array_equal(gotK, expK) and np.array_equal(gotV, expV)
    assert np.array_equal(kv.seq_len.cpu().numpy(), np.array(lens, np.int32))  # lengths are not touched


def test_commit_length_matches_oracle():
    rng = np.random.default_rng(92)
    B = 300
    n = rng.integers(-3, 1000, B).astype(np.int32)
    acc = rng.integers(-2, 10, B).astype(np.int32)
    sl = torch.from_numpy(n.copy()).cuda()
    tf.commit_length(sl, 7)
    tf.commit_length(sl, 0, 6, torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    exp = [oracle.commit_length(oracle.commit_length(int(x), 7), 0, 6, int(a)) for x, a in zip(n, acc)]
    assert sl.cpu().numpy().tolist() == exp


@pytest.mark.parametrize("n_sink,window,slack", [(4, 252, 8), (0, 7, 3), (2, 1, 5)])
def test_ring_decode_loop_matches_oracle(n_sink, window, slack):
    """The drafter appends gamma1 rows one at a time (reserve gamma1), then the
    rejected ones are rolled back; the device ring and length must equal the
    oracle's after every call, and streaming attention over the ring must
    equal the oracle's streaming attention over the logical sequence."""
    rng = np.random.default_rng(93 + window)
    dtype, B, H = "bf16", 2, 2
    cap = n_sink + window + slack
    lay = synth.KVLayout.build([0] * B, H, D, caps=[cap] * B)
    Ks = rows_bits(rng, lay.total_elems, dtype)
    Vs = rows_bits(rng, lay.total_elems, dtype)
    Kd, Vd = dev(Ks, dtype), dev(Vs, dtype)
    kv = kv_desc(lay, dtype, [0] * B)
    ref_K = [[lay.head(Ks, b, h, rows=cap).astype(np.float64) for h in range(H)] for b in range(B)]
    ref_V = [[lay.head(Vs, b, h, rows=cap).astype(np.float64) for h in range(H)] for b in range(B)]
    model_K = [[[] for _ in range(H)] for _ in range(B)]
    model_V = [[[] for _ in range(H)] for _ in range(B)]
    n = [0] * B
    steps = 150
    for step in range(steps):
        g1 = int(rng.integers(1, slack + 1))
        for r in range(g1):
            Kn = rows_bits(rng, (B, H, 1, D), dtype)
            Vn = rows_bits(rng, (B, H, 1, D), dtype)
            st = tf.append_kv(dev(Kn, dtype), dev(Vn, dtype), Kd, Vd, kv, ring=True, n_sink=n_sink, window=window,
                              reserve=g1)
            tf.commit_length(kv.seq_len, 1)
            for b in range(B):
                for h in range(H):
                    ref_K[b][h], s1 = oracle.append_ring(ref_K[b][h], n[b], n_sink, window,
                                                         Kn[b, h].astype(np.float64), reserve=g1)
                    ref_V[b][h], s2 = oracle.append_ring(ref_V[b][h], n[b], n_sink, window,
                                                         Vn[b, h].astype(np.float64), reserve=g1)
                    assert s1 == s2 == oracle.APPEND_OK
                    model_K[b][h].append(Kn[b, h, 0])
                    model_V[b][h].append(Vn[b, h, 0])
                n[b] = oracle.commit_length(n[b], 1)
            assert st.cpu().numpy().tolist() == [oracle.APPEND_OK] * B
        n_acc = rng.integers(0, g1 + 1, B).astype(np.int32)
        tf.commit_length(kv.seq_len, 0, g1, torch.from_numpy(n_acc).cuda())
        for b in range(B):
            n[b] = oracle.commit_length(n[b], 0, g1, int(n_acc[b]))
            for h in range(H):
                model_K[b][h] = model_K[b][h][:n[b]]
                model_V[b][h] = model_V[b][h][:n[b]]
        torch.cuda.synchronize()
        assert kv.seq_len.cpu().numpy().tolist() == n
        gotK, gotV = host_bits(Kd), host_bits(Vd)
        for b in range(B):
            for h in range(H):
                assert np.array_equal(lay.head(gotK, b, h, rows=cap), ref_K[b][h].astype(np.uint16)), (step, b, h)
                assert np.array_equal(lay.head(gotV, b, h, rows=cap), ref_V[b][h].astype(np.uint16)), (step, b, h)
    # streaming attention over the ring = the oracle over the logical sequence
    q = rows_bits(rng, (B, H, 1, D), dtype)
    o, lse = tf.stream_attn(dev(q, dtype).view(B, H, D), Kd, Vd, kv, n_sink, window)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    for b in range(B):
        for h in range(H):
            if n[b] == 0:
                assert np.all(o[b, h] == 0) and np.isneginf(lse[b, h])
                continue
            Kl = oracle.widen(np.array(model_K[b][h]), dtype)
            Vl = oracle.widen(np.array(model_V[b][h]), dtype)
            ro, rl = oracle.stream_attn_masked(oracle.widen(q[b, h, 0], dtype), Kl, Vl, n[b], n_sink, window)
            assert np.abs(o[b, h] - ro).max() <= ATOL and abs(lse[b, h] - rl) <= ATOL


def test_ring_too_small_leaves_ring_untouched():
    rng = np.random.default_rng(94)
    dtype, H, n_sink, window = "fp16", 2, 2, 5
    caps = [n_sink + window + 2, n_sink + window + 3]   # slack 2 and 3
    lay = synth.KVLayout.build([30, 30], H, D, caps=caps)
    Ks = rows_bits(rng, lay.total_elems, dtype)
    Kd, Vd = dev(Ks, dtype), dev(Ks, dtype)
    kv = kv_desc(lay, dtype, [30, 30])
    st = tf.append_kv(dev(rows_bits(rng, (2, H, 3, D), dtype), dtype), dev(rows_bits(rng, (2, H, 3, D), dtype), dtype),
                      Kd, Vd, kv, ring=True, n_sink=n_sink, window=window, reserve=3)
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [oracle.APPEND_RING_TOO_SMALL, oracle.APPEND_OK]
    got = host_bits(Kd)
    for h in range(H):
        assert np.array_equal(lay.head(got, 0, h, rows=caps[0]), lay.head(Ks, 0, h, rows=caps[0]))


def test_full_decode_loop_verify_accept_commit():
    """Target-level loop on the device: append the Q = gamma + 1 drafted rows,
    commit, verify over the full cache, accept, roll the rejected drafts back.
    Each step's verification and accept result equal the oracle's over the
    logical sequence (attention within 2e-3, accept bit-exact)."""
    rng = np.random.default_rng(95)
    dtype, B, H, gamma, vocab = "bf16", 3, 4, 4, 64
    Q = gamma + 1
    n0 = [300, 77, 1]
    cap = 300 + 12 * Q
    lay = synth.KVLayout.build(n0, H, D, caps=[cap] * B)
    K = rows_bits(rng, lay.total_elems, dtype)
    V = rows_bits(rng, lay.total_elems, dtype)
    Kd, Vd = dev(K, dtype), dev(V, dtype)
    kv = kv_desc(lay, dtype, n0)
    kv.max_len = cap
    model_K = [[list(lay.head(K, b, h)) for h in range(H)] for b in range(B)]
    model_V = [[list(lay.head(V, b, h)) for h in range(H)] for b in range(B)]
    n = list(n0)
    for step in range(10):
        Kn = rows_bits(rng, (B, H, Q, D), dtype)
        Vn = rows_bits(rng, (B, H, Q, D), dtype)
        st = tf.append_kv(dev(Kn, dtype), dev(Vn, dtype), Kd, Vd, kv)
        tf.commit_length(kv.seq_len, Q)
        qv = rows_bits(rng, (B, H, Q, D), dtype)
        o, lse = tf.verify_attn(dev(qv, dtype), Kd, Vd, kv)
        a = synth.make_accept_inputs(B=B, gamma=gamma, vocab=vocab, seed=95, layer=step, correlated=step % 2 == 1)
        na, nx = tf.accept(torch.from_numpy(a.target).cuda(), torch.from_numpy(a.draft).cuda(),
                           torch.from_numpy(a.tokens).cuda(), torch.from_numpy(a.uniforms).cuda(), 1.0)
        tf.commit_length(kv.seq_len, 0, gamma, na)
        torch.cuda.synchronize()
        assert st.cpu().numpy().tolist() == [oracle.APPEND_OK] * B
        o, lse, na_h, nx_h = o.cpu().double().numpy(), lse.cpu().double().numpy(), na.cpu().numpy(), nx.cpu().numpy()
        for b in range(B):
            for h in range(H):
                model_K[b][h] += list(Kn[b, h])
                model_V[b][h] += list(Vn[b, h])
                Kl = oracle.widen(np.array(model_K[b][h]), dtype)
                Vl = oracle.widen(np.array(model_V[b][h]), dtype)
                ro, rl = oracle.verify_attn(oracle.widen(qv[b, h], dtype), Kl, Vl, n[b] + Q)
                assert np.abs(o[b, h] - ro).max() <= ATOL and np.abs(lse[b, h] - rl).max() <= ATOL
            rn, rx, margin = oracle.accept(a.target[b], a.draft[b], a.tokens[b], a.uniforms[b], 1.0)
            if margin > 1e-12:
                assert (int(na_h[b]), int(nx_h[b])) == (rn, rx)
            n[b] = oracle.commit_length(oracle.commit_length(n[b], Q), 0, gamma, int(na_h[b]))
            for h in range(H):
                model_K[b][h] = model_K[b][h][:n[b]]
                model_V[b][h] = model_V[b][h][:n[b]]
        assert kv.seq_len.cpu().numpy().tolist() == n
