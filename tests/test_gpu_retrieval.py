"""GPU parity of the retrieval steps: chunk-mean keys, chunk scores and
top-k selection, each fed the same upstream arrays as the oracle."""

import numpy as np
import pytest
import torch

import oracle
from hierarchical_speculative_attention_amd import synth, KVDesc
import hierarchical_speculative_attention_amd as tf
from tests.gpu_util import TDT, desc, dev, host_bits

pytestmark = pytest.mark.gpu


def ck_layout(layout, cs):
    C = [max(1, -(-int(n) // cs)) for n in layout.seq_len]
    return synth.KVLayout.build([-(-int(n) // cs) for n in layout.seq_len], layout.H, layout.d, caps=C)


def run_chunk_keys(inp, cs, out_dtype, chunk_begin=None, max_chunks=None):
    lay = inp.layout
    cl = ck_layout(lay, cs)
    odt = torch.float32 if out_dtype == "fp32" else TDT[out_dtype]
    ck = torch.full((cl.total_elems,), float("nan"), dtype=odt, device="cuda")
    kv = desc(lay, inp.dtype)
    ckd = KVDesc.from_layout(cl, odt, "cuda")
    cb = None if chunk_begin is None else torch.tensor(chunk_begin, dtype=torch.int32, device="cuda")
    tf.build_chunk_keys(dev(inp.K, inp.dtype), kv, cs, ck, ckd, chunk_begin=cb, max_chunks=max_chunks)
    torch.cuda.synchronize()
    return ck, cl, ckd


def check_chunk_keys(inp, ck, cl, cs, out_dtype, only=None):
    lay = inp.layout
    if out_dtype == "fp32":
        got_all = ck.cpu().double().numpy()
    else:
        got_all = oracle.widen(host_bits(ck), out_dtype)
    for b in range(lay.B):
        n = int(lay.seq_len[b])
        for g in range(lay.H):
            ref = oracle.chunk_keys(oracle.widen(lay.head(inp.K, b, g), inp.dtype), n, cs)
            got = cl.head(got_all, b, g)
            rows = range(ref.shape[0]) if only is None else only[b]
            for c in rows:
                r, gv = ref[c], got[c]
                if out_dtype == "fp32":
                    np.testing.assert_allclose(gv, r, rtol=1e-6, atol=1e-6)
                else:
                    # one rounding of the fp64 mean: equal to the correctly rounded value,
                    # except where the mean lies within fp32 rounding of a rounding midpoint
                    exact = oracle.widen(oracle.round_f64_to_bits(r, out_dtype), out_dtype)
                    ulp = np.abs(np.spacing(exact.astype(np.float32 if out_dtype == "bf16" else np.float16)))
                    if out_dtype == "bf16":
                        ulp = np.abs(exact) * 2.0 ** -7 + 1e-40
                    mism = gv != exact
                    if mism.any():
                        assert np.all(np.abs(gv - r)[mism] <= 0.5 * ulp[mism] * (1 + 1e-5) + 1e-7), (b, g, c)
                        assert mism.mean() < 0.01


@pytest.mark.parametrize("dtype,out_dtype", [("bf16", "bf16"), ("bf16", "fp32"), ("fp16", "fp16"), ("fp16", "fp32")])
def test_chunk_keys_parity(dtype, out_dtype):
    inp = synth.make_attn_inputs(lens=[4096, 1003, 1, 17], Hq=4, Hkv=4, dtype=dtype, seed=10, cap_extra=5)
    ck, cl, _ = run_chunk_keys(inp, 8, out_dtype)
    check_chunk_keys(inp, ck, cl, 8, out_dtype)


@pytest.mark.parametrize("cs", [1, 3, 33, 1000, 4096])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_chunk_keys_chunk_sizes(cs, out_dtype):
    # one row per chunk, odd sizes, and chunks longer than a sequence (the
    # only chunk partial); the largest chunk size the C ABI takes
    inp = synth.make_attn_inputs(lens=[5000, 1003, 1, 17], Hq=2, Hkv=2, dtype="bf16", seed=13, cap_extra=5)
    ck, cl, _ = run_chunk_keys(inp, cs, out_dtype)
    check_chunk_keys(inp, ck, cl, cs, out_dtype)


def test_chunk_keys_partial_refresh():
    inp = synth.make_attn_inputs(lens=[1000, 64], Hq=2, Hkv=2, dtype="bf16", seed=11)
    ck, cl, _ = run_chunk_keys(inp, 16, "bf16", chunk_begin=[60, 2], max_chunks=3)
    got = oracle.widen(host_bits(ck), "bf16")
    # chunks [60, 63) of sequence 0 (62 is the partial last chunk) and [2, 4) of sequence 1
    check_chunk_keys(inp, ck, cl, 16, "bf16", only={0: [60, 61, 62], 1: [2, 3]})
    for g in range(2):
        assert np.all(np.isnan(cl.head(got, 0, g)[:60]))
        assert np.all(np.isnan(cl.head(got, 1, g)[:2]))


def run_scores(inp, ck, ckd, c_max):
    q = dev(inp.q_draft, inp.dtype).view(inp.layout.B, inp.Hq, 128)
    s = tf.score_chunks(q, inp.Hq, ck, ckd, c_max)
    torch.cuda.synchronize()
    return s


@pytest.mark.parametrize("Hq,Hkv,ck_dtype,dtype", [(8, 8, "bf16", "bf16"), (8, 2, "bf16", "bf16"), (8, 2, "fp32", "bf16"),
                                                  (4, 4, "fp16", "fp16"), (8, 2, "fp32", "fp16"), (64, 1, "bf16", "bf16"),
                                                  (32, 4, "fp32", "bf16")])
def test_scores_parity(Hq, Hkv, ck_dtype, dtype):
    # keys and queries in bf16 or fp16, chunk keys in the same dtype or fp32,
    # 1 to 64 query heads per KV head
    inp = synth.make_attn_inputs(lens=[4096, 777, 9], Hq=Hq, Hkv=Hkv, dtype=dtype, seed=12,
                                 plant="count", plant_count=4)
    ck, cl, ckd = run_chunk_keys(inp, 8, ck_dtype)
    c_max = 600
    s = run_scores(inp, ck, ckd, c_max).cpu().double().numpy()
    got_ck = ck.cpu().double().numpy() if ck_dtype == "fp32" else oracle.widen(host_bits(ck), ck_dtype)
    G = Hq // Hkv
    for b in range(3):
        C = int(cl.seq_len[b])
        for g in range(Hkv):
            kbar = cl.head(got_ck, b, g)
            qg = oracle.widen(inp.q_draft[b, g * G:(g + 1) * G, 0], dtype)
            ref = oracle.chunk_scores(qg, kbar)
            scale = np.linalg.norm(qg.sum(0)) * np.linalg.norm(kbar, axis=1) + np.abs(qg).sum() * 1e-3
            assert np.all(np.abs(s[b, g, :C] - ref) <= 1e-5 * scale)
            assert np.all(np.isneginf(s[b, g, C:]))


@pytest.mark.parametrize("ck_dtype", ["bf16", "fp16"])
def test_scores_ragged_rows(ck_dtype):
    # 64 rows of a c_max = 8200 score array: more 16-chunk blocks per row than
    # waves in the grid for it, so waves score several blocks, the last round
    # ragged; a row of 3 chunks and an empty one are -inf past their keys
    B, H, c_max = 4, 16, 8200
    C = [8192, 8000, 3, 0]
    lay = synth.KVLayout.build(C, H, 128, caps=[max(c, 1) for c in C])
    g = torch.Generator().manual_seed(21)
    ck_host = torch.randn(lay.total_elems, generator=g).to(TDT[ck_dtype])
    q_host = torch.randn((B, H, 128), generator=g).to(TDT[ck_dtype])
    s = tf.score_chunks(q_host.cuda(), H, ck_host.cuda(), desc(lay, ck_dtype), c_max)
    torch.cuda.synchronize()
    s = s.cpu().double().numpy()
    ck_bits, q_bits = host_bits(ck_host), host_bits(q_host)
    for b in range(B):
        for h in range(H):
            kbar = oracle.widen(lay.head(ck_bits, b, h), ck_dtype)
            qg = oracle.widen(q_bits[b, h:h + 1], ck_dtype)
            ref = oracle.chunk_scores(qg, kbar)
            scale = np.linalg.norm(qg) * np.linalg.norm(kbar, axis=1) + 1e-3
            assert np.all(np.abs(s[b, h, :C[b]] - ref) <= 1e-5 * scale), (b, h)
            assert np.all(np.isneginf(s[b, h, C[b]:])), (b, h)


def run_topk(scores_np, n_chunks, k):
    s = torch.from_numpy(np.ascontiguousarray(scores_np, np.float32)).cuda()
    idx = tf.select_topk(s, torch.tensor(n_chunks, dtype=torch.int32, device="cuda"), k)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def test_topk_bit_exact_on_gpu_scores():
    inp = synth.make_attn_inputs(lens=[4096, 2500], Hq=8, Hkv=8, dtype="bf16", seed=13, plant="count", plant_count=4)
    ck, cl, ckd = run_chunk_keys(inp, 8, "bf16")
    s = run_scores(inp, ck, ckd, 512)
    s_np = s.cpu().numpy()
    for k in [64, 1, 511, 512, 600]:
        idx = run_topk(s_np, [512, 313], k)
        for b, C in enumerate([512, 313]):
            for g in range(8):
                ref = oracle.select_topk(s_np[b, g, :C].astype(np.float64), k)
                assert np.array_equal(idx[b, g], ref), (k, b, g)
    # every planted chunk of the full-length sequence is selected at k = 64
    idx = run_topk(s_np, [512, 313], 64)
    for g in range(8):
        assert set(inp.planted[0].tolist()) <= set(idx[0, g].tolist())


def test_topk_adversarial_rows():
    rng = np.random.default_rng(14)
    rows = []
    C = 1000
    rows.append(np.zeros(C))                                   # all equal
    r = np.zeros(C); r[::2] = -0.0; rows.append(r)             # +-0
    r = rng.standard_normal(C); r[rng.choice(C, 50, replace=False)] = np.inf
    r[rng.choice(C, 50, replace=False)] = -np.inf; rows.append(r)
    r = rng.standard_normal(C); r[rng.choice(C, 300, replace=False)] = np.nan; rows.append(r)
    rows.append(np.round(rng.standard_normal(C) * 2) / 4)     # heavy ties
    rows.append(np.full(C, np.nan))
    rows.append(rng.standard_normal(C) * 1e-38)                # subnormal-range fp32
    scores = np.stack(rows)[None].astype(np.float32)
    for k in [1, 7, 64, 499, 999, 1000, 1500]:
        for n in [C, 937, 65, 64, 1]:
            idx = run_topk(scores, [n], k)
            for g in range(scores.shape[1]):
                ref = oracle.select_topk(scores[0, g, :n].astype(np.float64), k)
                assert np.array_equal(idx[0, g], ref), (k, n, g)


@pytest.mark.parametrize("C,k", [(16384, 512), (16448, 512), (32768, 512), (70000, 3000)])
def test_topk_large_rows(C, k):
    rng = np.random.default_rng(C)
    s = (rng.standard_normal((2, 3, C)) * 5).astype(np.float32)
    s[:, :, rng.choice(C, 100)] = 7.5   # ties near the top
    idx = run_topk(s, [C, C - 11], k)
    for b, n in enumerate([C, C - 11]):
        for g in range(3):
            assert np.array_equal(idx[b, g], oracle.select_topk(s[b, g, :n].astype(np.float64), k))


@pytest.mark.parametrize("C,ks", [(1 << 20, [1, 2048, 100000]), (300001, [4096])])
def test_topk_longest_rows(C, ks):
    # rows past 65536 chunks up to the largest the C ABI takes (2^20): keys
    # re-read from memory each pass; ties near the top, NaNs, a shorter row
    rng = np.random.default_rng(C)
    s = (rng.standard_normal((1, 2, C)) * 4).astype(np.float32)
    s[0, :, rng.choice(C, 5000, replace=False)] = 9.0
    s[0, 1, rng.choice(C, 300, replace=False)] = np.nan
    print(f"top-k longest rows: C={C} ks={ks}", flush=True)
    for k in ks:
        for n in (C, C - 12345):
            idx = run_topk(s, [n], k)
            for g in range(2):
                ref = oracle.select_topk(s[0, g, :n].astype(np.float64), k)
                assert np.array_equal(idx[0, g], ref), (k, n, g)


@pytest.mark.parametrize("C", [1500, 3001, 4096, 5003, 16384, 16448, 20001, 24576, 30000, 40000, 50001])
def test_topk_value_spreads(C):
    """Rows whose k-th key sits in bins of every size: exponents spread so the
    first digit already isolates a small bin, quantised values whose 16-bit
    bins hold exact duplicates, a narrow band that needs all four digits.
    Row lengths cover every keys-per-thread instantiation of the one-launch
    path (2, 4, 8, 16, 20, 24, 32, 48 and 64 keys per thread) with lengths
    that are and are not a multiple of 4."""
    rng = np.random.default_rng(C + 1)
    rows = [
        np.sign(rng.standard_normal(C)) * np.exp2(rng.uniform(-60, 60, C)),     # spread exponents
        np.round(rng.standard_normal(C) * 4 * 1024) / 1024,                     # duplicates in small bins
        1.0 + rng.integers(0, 1 << 12, C) * 2.0 ** -23,                          # one narrow band
        (rng.standard_normal(C) * 4).astype(np.float32),                         # score-like
    ]
    s = np.stack(rows)[None].astype(np.float32)
    for k in [1, 512, 1023, 2049]:
        for n in [C, C - 3]:
            idx = run_topk(s, [n], k)
            for g in range(s.shape[1]):
                ref = oracle.select_topk(s[0, g, :n].astype(np.float64), k)
                assert np.array_equal(idx[0, g], ref), (k, n, g)


@pytest.mark.parametrize("B,rows,C,ks", [(1, 8, 32768, [1, 512, 2048]), (2, 3, 40001, [7, 1000]),
                                         (1, 16, 65536, [1024]), (1, 1, 20000, [64, 1250])])
def test_topk_split_rows(B, rows, C, ks):
    """Few long rows take the slice-and-merge path (a workspace is needed):
    rows whose length leaves slices full, partial (fewer keys than k, all of
    them candidates) or empty, rows with every key tied, NaN rows, row
    lengths that are not a multiple of 4, and the largest slice and merge
    sizes (65536 chunks, 8 x 1024 candidates)."""
    assert all(tf.select_topk_workspace_size(B, rows, C, k) > 0 for k in ks)
    rng = np.random.default_rng(C + rows)
    s = (rng.standard_normal((B, rows, C)) * 3).astype(np.float32)
    s[:, :, rng.choice(C, 200)] = 6.25                   # ties near the top
    s[0, 0, :] = 0.0                                     # every key tied
    if rows > 1:
        s[0, 1, rng.choice(C, C // 3, replace=False)] = np.nan
    if rows > 2:
        s[0, 2, :] = np.round(s[0, 2, :])                # heavy ties in every slice
    for n in [C, C - 3, C // 2 + 1, 4100, 700, ks[-1] + 1, ks[-1], 100, 0]:
        n_b = [n] + [max(0, C - 5 - n)] * (B - 1)
        for k in ks:
            idx = run_topk(s, n_b, k)
            for b in range(B):
                for g in range(rows):
                    ref = oracle.select_topk(s[b, g, :n_b[b]].astype(np.float64), k)
                    assert np.array_equal(idx[b, g], ref), (n_b[b], k, b, g)


def _cluster_row(rng, C, k, m, shared_bits, above, ties=False):
    """A row whose k-th largest score lies in a cluster of m keys that share
    their top `shared_bits` key bits: `above` large scores, the cluster, the
    rest small.  With ties, the cluster holds few distinct values."""
    row = rng.standard_normal(C).astype(np.float32)          # small: |x| < 8 almost surely
    row = np.clip(row, -7.5, 7.5)
    pos = rng.permutation(C)
    row[pos[:above]] = (100.0 + rng.random(above) * 50).astype(np.float32)
    base = np.float32(8.0).view(np.uint32)                   # key bits of positive floats: float bits | 2^31
    span = 1 << (32 - shared_bits)                           # values sharing the top shared_bits key bits
    steps = rng.integers(0, 4 if ties else span, m) if span > 1 else np.zeros(m, np.int64)
    row[pos[above:above + m]] = (base + steps.astype(np.uint32)).view(np.float32)
    return row


def test_topk_headline_shape_adversarial():
    """The benchmark's top-k shape exactly: 32 rows of 16384 chunks, k = 512,
    bit-exact against the oracle, on rows that steer every path of the radix
    selection: GPU-like scores, the k-th key inside a cluster of 63 / 64 / 65 /
    200 keys sharing their top 16, 19 or 24 key bits (with and without ties),
    all equal, NaN-heavy, all NaN, +-0, +-inf at the boundary, heavy ties,
    subnormal-range values."""
    rng = np.random.default_rng(140)
    C, k = 16384, 512
    rows = []
    q = rng.standard_normal(128)
    kb = rng.standard_normal((C, 128)) / np.sqrt(8)
    kb[rng.choice(C, 164, replace=False)] += 0.5 * q
    rows.append((kb @ q).astype(np.float32))                 # scores shaped like the workload's
    for m in (63, 64, 65, 200):
        for bits in (16, 19, 24):
            rows.append(_cluster_row(rng, C, k, m, bits, above=k - min(m, 40)))
    rows.append(_cluster_row(rng, C, k, 64, 16, above=k - 30, ties=True))
    rows.append(_cluster_row(rng, C, k, 300, 24, above=k - 150, ties=True))
    rows.append(np.zeros(C, np.float32))                                        # all equal
    r = np.zeros(C, np.float32); r[::2] = -0.0; rows.append(r)                  # +-0
    r = rng.standard_normal(C).astype(np.float32); r[rng.choice(C, 6000, replace=False)] = np.nan; rows.append(r)
    rows.append(np.full(C, np.nan, np.float32))
    r = rng.standard_normal(C).astype(np.float32); r[rng.choice(C, 511, replace=False)] = np.inf
    r[rng.choice(C, 3000, replace=False)] = -np.inf; rows.append(r)            # +inf just short of k
    rows.append((np.round(rng.standard_normal(C) * 2) / 4).astype(np.float32))  # heavy ties
    rows.append((rng.standard_normal(C) * 1e-38).astype(np.float32))           # subnormal range
    while len(rows) < 32:
        rows.append((rng.standard_normal(C) * rng.uniform(0.1, 50)).astype(np.float32))
    scores = np.stack(rows[:32])[None]
    idx = run_topk(scores, [C], k)
    for g in range(32):
        ref = oracle.select_topk(scores[0, g].astype(np.float64), k)
        assert np.array_equal(idx[0, g], ref), g
