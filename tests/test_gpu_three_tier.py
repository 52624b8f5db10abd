"""The three-tier step driver on the GPU: after every step the device
lengths equal the driver's counts, every level-1 and level-2 decision equals
the oracle's accept on the same inputs, and the candidates Force 3 verifies
are the tokens the Force 2 rounds emitted, in order."""

import numpy as np
import pytest
import torch

import oracle
from hierarchical_speculative_attention_amd import synth, KVDesc
from hierarchical_speculative_attention_amd import three_tier as tt

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def build(n0=3000, H=4, layers=2, d_layers=2, cs=8, k=16, g1=2, g2=5, V=64, S=4, W=28, seed=131, graphs=False):
    g = torch.Generator(device=DEV).manual_seed(seed)
    rnd = lambda *shape: torch.randn(*shape, generator=g, device=DEV).to(torch.bfloat16)
    extra = 64 * (g1 + g2 + 4)
    seq_len = torch.tensor([n0], dtype=torch.int32, device=DEV)
    C = -(-(n0 + extra) // cs)
    ck_len = torch.tensor([-(-n0 // cs)], dtype=torch.int32, device=DEV)
    target = []
    for l in range(layers):
        K, V_, qv, qd, lay, _ = synth.make_layer_torch(lens=[n0], Hq=H, Hkv=H, d=128, dtype="bf16", Q=1, chunk_size=cs,
                                                       plant=None, seed=seed, layer=l, device=DEV, extra_rows=extra)
        kv = KVDesc.from_layout(lay, torch.bfloat16, DEV, max_len=n0 + extra)
        kv.seq_len = seq_len
        ckl = synth.KVLayout.build([C], H, 128, caps=[C])
        ckd = KVDesc.from_layout(ckl, torch.bfloat16, DEV)
        ckd.seq_len = ck_len
        ck = torch.empty(ckl.total_elems, dtype=torch.bfloat16, device=DEV)
        from hierarchical_speculative_attention_amd import build_chunk_keys
        build_chunk_keys(K, kv, cs, ck, ckd)
        target.append(tt.TargetLayer(K, V_, kv, ck, ckd))
    cap = S + W + tt.drafter_reserve(g1, g2)
    d_len = torch.tensor([n0], dtype=torch.int32, device=DEV)
    drafter = []
    for l in range(d_layers):
        lay = synth.KVLayout.build([n0], H, 128, caps=[cap])
        sd = KVDesc.from_layout(lay, torch.bfloat16, DEV)
        sd.seq_len = d_len
        drafter.append(tt.DrafterLayer(rnd(lay.total_elems), rnd(lay.total_elems), sd))
    P = torch.randn((1, g2 + 1, V), generator=g, device=DEV) * 2
    Qr = torch.cat([P[:, :g1 + 1] + torch.randn((1, g1 + 1, V), generator=g, device=DEV) * 0.5], 1)
    R = Qr[:, :g1] + torch.randn((1, g1, V), generator=g, device=DEV) * 0.5
    rng = np.random.default_rng(seed)
    syn = tt.Synthetic(
        draft_q=rnd(1, H, 128), draft_rows=[rnd(1, H, r, 128) for r in (1, 2, 3)],
        r_rows=R.contiguous(), f2_q=rnd(1, H, g1 + 1, 128), f2_rows=rnd(1, H, g1 + 1, 128),
        q_rows=Qr.contiguous(), f3_q=rnd(1, H, g2 + 1, 128), one_row=rnd(1, H, 1, 128), p_rows=P.contiguous(),
        uniforms=torch.from_numpy(synth.open_uniforms(rng, 4096)).to(DEV))
    step = tt.ThreeTierStep(target, drafter, syn, Hq=H, chunk_size=cs, k=k, tail=16, gamma1=g1, gamma2=g2, n_sink=S,
                            window=W, record=True, graphs=graphs)
    return step, syn


@pytest.mark.parametrize("graphs", [False, True], ids=["eager", "graphs"])
def test_three_tier_steps_match_oracle_and_lengths(graphs):
    g1, g2 = 2, 5
    step, syn = build(g1=g1, g2=g2, graphs=graphs)
    R = syn.r_rows.cpu().numpy()[0]
    Qr = syn.q_rows.cpu().numpy()[0]
    P = syn.p_rows.cpu().numpy()[0]
    total_rounds = 0
    for it in range(40):
        n_before = step.n
        emitted = step.step()
        torch.cuda.synchronize()
        # lengths on the device = the driver's counts
        assert int(step.seq_len.item()) == step.n == n_before + emitted
        assert int(step.d_len.item()) == step.n - step.pending and 0 <= step.pending <= 2
        # decisions against the oracle, round by round, then Force 3
        rounds = [e for e in step.log if e[0] == "round"]
        last = step.log[-1]
        assert last[0] == "step"
        chain = []
        for _, drafts, n1, y, u in rounds:
            rn, ry, margin = oracle.accept(Qr, R, drafts, u, 1.0)
            if margin > 1e-12:
                assert (n1, y) == (rn, ry)
            chain += drafts[:n1] + [y]
        _, cand, n2, nxt, u2, cand_q = last
        assert cand == chain[:g2]
        np.testing.assert_array_equal(cand_q, np.stack([Qr[j] for r in rounds for j in range(r[2] + 1)])[:g2])
        rn, rx, margin = oracle.accept(P, cand_q, cand, u2, 1.0)
        if margin > 1e-12:
            assert (n2, nxt) == (rn, rx)
        assert emitted == n2 + 1
        total_rounds += len(rounds)
        step.log.clear()
    assert step.emitted > step.steps     # some candidates were kept
    assert total_rounds > step.steps     # some steps needed more than one round


def test_three_tier_graphs_replay_the_eager_steps():
    """Replayed graphs (with eager work and host reads between replays) take
    every decision of the eager launches and leave the same caches."""
    logs, outs = [], []
    for graphs in (False, True):
        step, _ = build(g1=3, g2=6, seed=77, graphs=graphs)
        entries = []
        for _ in range(30):
            step.step()
            torch.cuda.synchronize()
            entries.append((step.n, step.pending, int(step.seq_len.item()), int(step.d_len.item())))
            for e in step.log:
                entries.append((e[0], e[1], e[2], e[3]))
            step.log.clear()
        logs.append(entries)
        # the written parts: rows below the length (each head), built chunk keys, the whole ring
        n, H = step.n, step.t[0].kv.H
        rows = lambda x, cap, m: x.view(H, cap, 128)[:, :m].cpu()
        outs.append([step.o3.cpu(), step.o2.cpu(), step.o_d.cpu()]
                    + [rows(x.ck, x.ckd.max_len, -(-n // step.cs)) for x in step.t]
                    + [rows(t, x.K.numel() // (H * 128), n) for x in step.t for t in (x.K, x.V)]
                    + [t.cpu() for x in step.dr for t in (x.Ks, x.Vs)])
    assert logs[0] == logs[1]
    for a, b in zip(*outs):
        assert torch.equal(a, b)
