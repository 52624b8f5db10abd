"""The equal-work partition of a batch's verification (host check, no GPU).

The attention kernel gives workgroup g of G the tiles
[floor(g TT / G), floor((g + 1) TT / G)) of the batch's TT 32-token tiles in
(sequence, KV head, tile) order; its part of segment s = b * Hkv + hk goes
to partial slot g + s unless one workgroup holds the whole segment (then it
writes the output); the merge finds a segment's parts as the consecutive
slots from g0 + s, g0 = floor(((x0 + 1) G - 1) / TT) for the segment's first
tile x0.  This mirrors that integer arithmetic and checks, over ragged
batches with empty sequences, that every tile is covered once, slots are
unique and below G + B * Hkv, and the merge sees exactly the parts written.
"""
import numpy as np
import pytest


def wg_of(x, TT, G):
    return ((x + 1) * G - 1) // TT


def partition(tiles_per_head, Hkv, grid):
    B = len(tiles_per_head)
    pre = [0]
    for t in tiles_per_head:
        pre.append(pre[-1] + Hkv * t)
    TT = pre[-1]
    G = min(grid, TT)   # every workgroup below G holds at least one tile
    written = {}   # slot -> (segment, tile lo, tile hi)
    direct = {}    # segment -> (tile lo, tile hi)
    for g in range(G):
        x, xe = g * TT // G, (g + 1) * TT // G
        while x < xe:
            b = max(i for i in range(B) if pre[i] <= x)   # largest b with pre[b] <= x
            T = (pre[b + 1] - pre[b]) // Hkv
            assert T >= 1
            hk = (x - pre[b]) // T
            seg0 = pre[b] + hk * T
            seg1 = seg0 + T
            x1 = min(xe, seg1)
            s = b * Hkv + hk
            if wg_of(seg0, TT, G) == wg_of(seg1 - 1, TT, G):
                assert s not in direct
                direct[s] = (x - seg0, x1 - seg0)
            else:
                slot = g + s
                assert slot not in written, "slot written twice"
                assert 0 <= slot < G + B * Hkv
                written[slot] = (s, x - seg0, x1 - seg0)
            x = x1
    return pre, TT, written, direct


@pytest.mark.parametrize("seed", range(40))
def test_partition_covers_every_tile_once(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(2, 40))
    Hkv = int(rng.choice([1, 2, 8, 32]))
    G = int(rng.choice([1, 7, 64, 512]))
    lens = rng.integers(0, 5000, B)
    lens[rng.random(B) < 0.2] = 0          # empty sequences
    tiles = [int((n + 31) // 32) for n in lens]
    pre, TT, written, direct = partition(tiles, Hkv, G)
    G = min(G, TT)
    for b in range(B):
        T = tiles[b]
        for hk in range(Hkv):
            s = b * Hkv + hk
            if T == 0:
                assert s not in direct
                continue
            seg0 = pre[b] + hk * T
            g0, g1 = wg_of(seg0, TT, G), wg_of(seg0 + T - 1, TT, G)
            if g0 == g1:
                assert direct[s] == (0, T)
                continue
            # what the merge reads: slots g0 + s .. g1 + s, in order, covering [0, T)
            parts = [written[g + s] for g in range(g0, g1 + 1)]
            assert all(p[0] == s for p in parts)
            assert parts[0][1] == 0 and parts[-1][2] == T
            assert all(parts[i][2] == parts[i + 1][1] for i in range(len(parts) - 1))
            assert all(p[1] < p[2] for p in parts)
    # nothing written that the merge does not read
    n_read = 0 if TT == 0 else sum(wg_of(pre[b] + hk * tiles[b] + tiles[b] - 1, TT, G) - wg_of(pre[b] + hk * tiles[b], TT, G) + 1
                 for b in range(B) for hk in range(Hkv)
                 if tiles[b] and wg_of(pre[b] + hk * tiles[b], TT, G) != wg_of(pre[b] + hk * tiles[b] + tiles[b] - 1, TT, G))
    assert n_read == len(written)


def test_partition_balances_the_eight_sequence_batch():
    """The 8-sequence batch (16K-128K, 32 KV heads) on 512 workgroups: every
    workgroup gets 3.69 items' worth of tiles (within one tile)."""
    lens = [16384, 24576, 32768, 49152, 65536, 65536, 98304, 131072]
    tiles = [n // 32 for n in lens]
    G = 512
    TT = 32 * sum(tiles)
    sizes = [(g + 1) * TT // G - g * TT // G for g in range(G)]
    assert max(sizes) - min(sizes) <= 1
    pre, TT2, written, direct = partition(tiles, 32, G)
    assert TT2 == TT
    assert sum(hi - lo for _, lo, hi in written.values()) + sum(hi - lo for lo, hi in direct.values()) == TT


@pytest.mark.parametrize("tiles,Hkv,grid", [([1, 0, 2], 2, 512), ([0, 0, 1], 1, 512), ([3, 5], 8, 7), ([0, 0], 4, 512)])
def test_partition_with_fewer_tiles_than_workgroups(tiles, Hkv, grid):
    pre, TT, written, direct = partition(tiles, Hkv, grid)
    assert sum(hi - lo for _, lo, hi in written.values()) + sum(hi - lo for lo, hi in direct.values()) == TT
    G = min(grid, TT)
    for b, T in enumerate(tiles):
        for hk in range(Hkv if T else 0):
            s = b * Hkv + hk
            seg0 = pre[b] + hk * T
            g0, g1 = wg_of(seg0, TT, G), wg_of(seg0 + T - 1, TT, G)
            if g0 == g1:
                assert direct[s] == (0, T)
            else:
                assert all(g + s in written for g in range(g0, g1 + 1))
