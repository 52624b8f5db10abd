"""The decomposition behind the top-k path for few long rows: selecting each
slice's k best (key descending, index ascending), keeping the candidates in
index order and selecting the k best of them again gives the row's k best,
ties included.  Checked on the host with the oracle's selection, over rows
with heavy ties, NaN and +-inf, slices shorter than k and empty slices."""

import numpy as np
import pytest

import oracle


def sliced_topk(s, k, n_slices):
    L = -(-len(s) // n_slices)
    cand = []
    for z in range(n_slices):
        part = s[z * L:(z + 1) * L]
        if len(part) == 0:
            continue
        sel = oracle.select_topk(part, k)
        cand.extend(z * L + int(i) for i in sel if i >= 0)
    cand = np.array(cand, dtype=np.int64)
    assert np.all(np.diff(cand) > 0)                 # candidates stay in index order
    pick = oracle.select_topk(s[cand], k)
    out = np.full(k, -1, dtype=np.int64)
    got = cand[pick[pick >= 0]]
    out[:len(got)] = got
    return out


@pytest.mark.parametrize("seed", range(6))
def test_slices_then_merge_equal_row_topk(seed):
    rng = np.random.default_rng(seed)
    for C in [37, 64, 200, 1000]:
        rows = [
            rng.standard_normal(C),
            np.round(rng.standard_normal(C) * 2) / 2,     # heavy ties
            np.zeros(C),                                  # all tied
            np.where(rng.random(C) < 0.3, np.nan, rng.standard_normal(C)),
            np.where(rng.random(C) < 0.1, np.inf, np.where(rng.random(C) < 0.1, -np.inf, rng.standard_normal(C))),
        ]
        for s in rows:
            s = s.astype(np.float32).astype(np.float64)
            for k in [1, 3, 8, C // 3 + 1, C - 1, C]:
                for n_slices in [2, 3, 8]:
                    ref = oracle.select_topk(s, k)
                    assert np.array_equal(sliced_topk(s, k, n_slices), ref), (C, k, n_slices)
