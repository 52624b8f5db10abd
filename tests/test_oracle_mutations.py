"""The pins must catch plausible mistakes.  Each case plants one mistake in a
copy of an oracle function (CPU only), runs the pin that should notice it,
and expects that pin to fail."""

import math

import numpy as np
import pytest

import oracle
import oracle.triforce_oracle as T
import tests.test_oracle_pins as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(T, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def verify_off_by_one(qs, K, V, n):
    Q, d = qs.shape
    o, lse = np.zeros((Q, d)), np.zeros(Q)
    for i in range(Q):
        vis = max(0, min(n - Q + i, n))        # mistake: drops the + 1
        o[i], lse[i] = T.attention(qs[i], K[:vis], V[:vis])
    return o, lse


def attention_unscaled(q, K, V):
    if K.shape[0] == 0:
        return np.zeros(q.shape[0]), -math.inf
    logits = K @ q                              # mistake: no 1/sqrt(d)
    w = np.exp(logits - logits.max())
    return (w @ V) / w.sum(), float(logits.max() + math.log(w.sum()))


def chunk_keys_fixed_divisor(K, n, cs):
    C = -(-n // cs) if n > 0 else 0
    out = np.zeros((C, K.shape[1]))
    for c in range(C):
        lo, hi = c * cs, min(n, (c + 1) * cs)
        out[c] = K[lo:hi].sum(axis=0) / cs     # mistake: partial chunk divided by cs
    return out


def topk_ties_high_index(scores, k):
    s = np.array(scores, np.float64)
    s[np.isnan(s)] = -np.inf
    C = len(s)
    order = np.lexsort((-np.arange(C), -s))   # mistake: ties to the higher index
    take = np.sort(order[:min(k, C)])
    out = np.full(k, -1, np.int64)
    out[:len(take)] = take
    return out


def stream_positions_short(n, S, W):
    return np.asarray(list(range(min(S, n))) + list(range(max(S, n - W + 1), n)), np.int64)  # mistake: W - 1 recent


def accept_flipped_residual(target, draft, tokens, uniforms, temperature, probs=False):
    gamma = len(tokens)
    j = gamma
    for i in range(gamma):
        p = T.distribution(target[i], temperature, probs)
        q = T.distribution(draft[i], temperature, probs)
        x = int(tokens[i])
        if p[x] > 0 and (q[x] == 0 or min(1.0, p[x] / q[x]) >= uniforms[i]):
            continue
        j = i
        break
    if j < gamma:
        r = np.maximum(0.0, T.distribution(draft[j], temperature, probs) - T.distribution(target[j], temperature, probs))  # mistake: q - p
        if r.sum() == 0:
            r = T.distribution(target[j], temperature, probs)
    else:
        r = T.distribution(target[gamma], temperature, probs)
    return j, T.inverse_cdf(r, float(uniforms[gamma])), 1.0


def accept_no_bonus(target, draft, tokens, uniforms, temperature, probs=False):
    j, nxt, m = T.accept.__wrapped__(target, draft, tokens, uniforms, temperature, probs) \
        if hasattr(T.accept, "__wrapped__") else ORIG_ACCEPT(target, draft, tokens, uniforms, temperature, probs)
    if j == len(tokens):
        nxt = int(np.argmax(T.distribution(draft[-1], temperature, probs)))  # mistake: bonus from the draft row
    return j, nxt, m


ORIG_ACCEPT = T.accept


def accept_token_index_wraps(target, draft, tokens, uniforms, temperature, probs=False):
    gamma = len(tokens)
    j = gamma
    for i in range(gamma):
        p = T.distribution(target[i], temperature, probs)
        q = T.distribution(draft[i], temperature, probs)
        x = int(tokens[i])
        px, qx = float(p[x]), float(q[x])      # mistake: no range check, -1 reads the last entry
        if px > 0.0 and (qx == 0.0 or min(1.0, px / qx) >= float(uniforms[i])):
            continue
        j = i
        break
    r = (np.maximum(0.0, T.distribution(target[j], temperature, probs) - T.distribution(draft[j], temperature, probs))
         if j < gamma else T.distribution(target[gamma], temperature, probs))
    return j, T.inverse_cdf(r, float(uniforms[gamma])), 1.0


def accept_token_clamped(target, draft, tokens, uniforms, temperature, probs=False):
    V = np.asarray(target).shape[1]
    toks = [min(max(int(x), 0), V - 1) for x in tokens]  # mistake: out-of-vocabulary tokens clamped
    return ORIG_ACCEPT(target, draft, toks, uniforms, temperature, probs)


def round_fp16_via_fp32(x, dtype):
    if dtype == "fp16":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float16).view(np.uint16)  # mistake: rounds twice
    return ORIG_ROUND(x, dtype)


def round_fp16_truncates(x, dtype):
    if dtype == "fp16":
        x = np.asarray(x, np.float64)
        m, e = np.frexp(x)
        r = np.ldexp(np.trunc(np.ldexp(m, 11)), e - 11)   # mistake: truncation, not nearest even
        return r.astype(np.float16).view(np.uint16)
    return ORIG_ROUND(x, dtype)


ORIG_ROUND = T.round_f64_to_bits


def append_ring_short_reserve(slots, n, n_sink, window, new, reserve=None):
    reserve = new.shape[0] if reserve is None else reserve
    return ORIG_APPEND_RING(slots, n, n_sink, window, new, reserve - 1)   # mistake: one slot of slack short


ORIG_APPEND_RING = T.append_ring


def commit_drops_one_more(n, add, gamma=0, n_accepted=None):
    drop = 0 if n_accepted is None else gamma - min(max(int(n_accepted), 0), gamma) + 1  # mistake
    return max(0, n + add - drop)


def ring_slot_one_short(p, n_sink, cap):
    return p if p < n_sink else n_sink + (p - n_sink) % (cap - n_sink - 1)   # mistake: ring one slot short


def _two_level_variant(level1_swap=False, level2_rows="q", shift=0):
    def two_level(p_rows, q_rows, r_rows, w, u1, v1, u2, gamma1, gamma2, temperature, probs=False):
        cand, rounds = [], 0
        while len(cand) < gamma2:
            t0 = len(cand)
            drafts = [T.inverse_cdf(T.distribution(r_rows[t0 + j], temperature, probs), float(w[t0 + j]))
                      for j in range(gamma1)]
            uni = [float(x) for x in u1[t0:t0 + gamma1]] + [float(v1[t0])]
            tgt, drf = (r_rows[t0:t0 + gamma1 + 1], q_rows[t0:t0 + gamma1]) if level1_swap else \
                (q_rows[t0:t0 + gamma1 + 1], r_rows[t0:t0 + gamma1])
            if level1_swap and tgt.shape[0] < gamma1 + 1:
                tgt = np.concatenate([tgt, q_rows[t0 + gamma1:t0 + gamma1 + 1]])
            n1, y, _ = T.accept(tgt, drf, drafts, uni, temperature, probs)
            cand += drafts[:n1] + [y]
            rounds += 1
        cand = cand[:gamma2]
        rows = r_rows if level2_rows == "r" else q_rows
        n2, nxt, _ = T.accept(p_rows[:gamma2 + 1], rows[shift:shift + gamma2], cand, u2, temperature, probs)
        return cand, n2, nxt, rounds
    return two_level


two_level_level1_swapped = _two_level_variant(level1_swap=True)      # mistake: Force 2 tests r against q
two_level_level1_swapped.__name__ = "two_level_level1_swapped"
two_level_draft_rows_r = _two_level_variant(level2_rows="r")          # mistake: level 2 divides by r
two_level_draft_rows_r.__name__ = "two_level_draft_rows_r"
two_level_rows_shifted = _two_level_variant(shift=1)                  # mistake: q rows one position late
two_level_rows_shifted.__name__ = "two_level_rows_shifted"


def tree_masks_no_self(parent):
    out = []
    for i in range(len(parent)):
        m, x = 0, int(parent[i]) if 0 <= int(parent[i]) < i else -1   # mistake: the node itself is left out
        while x >= 0:
            m |= 1 << x
            p = int(parent[x])
            x = p if 0 <= p < x else -1
        out.append(m)
    return out


def verify_tree_base_off_by_one(qs, K, V, n, masks):
    Q, d = qs.shape
    base = n - Q + 1                          # mistake: nodes start one row late
    o, lse = np.zeros((Q, d)), np.zeros(Q)
    for i in range(Q):
        vis = [t for t in range(max(0, n)) if t < base or (int(masks[i]) >> (t - base)) & 1]
        o[i], lse[i] = T.attention(qs[i], K[vis], V[vis])
    return o, lse


def _tree_variant(renormalise=True, update=True):
    def tree_accept(target, draft, tokens, parent, uniforms, temperature, probs=False):
        Q = len(parent)
        children = [[] for _ in range(Q)]
        for c in range(1, Q):
            pc = int(parent[c])
            children[pc if 0 <= pc < c else 0].append(c)
        path, v = [], 0
        while True:
            p = T.distribution(target[v], temperature, probs)
            pr, kept = p, -1
            if children[v]:
                q = T.distribution(draft[v], temperature, probs)
                for c in children[v]:
                    x = int(tokens[c])
                    if 0 <= x < p.shape[0] and pr[x] > 0.0 and uniforms[c - 1] * q[x] <= pr[x]:
                        kept = c
                        break
                    if update:
                        r = np.maximum(0.0, pr - q)
                        pr = (r / r.sum() if r.sum() > 0 else p) if renormalise else r
            if kept < 0:
                return path, T.inverse_cdf(pr, float(uniforms[Q - 1])), 1.0
            path.append(kept)
            v = kept
    return tree_accept


tree_accept_unnormalised = _tree_variant(renormalise=False)   # mistake: residual not renormalised
tree_accept_unnormalised.__name__ = "tree_accept_unnormalised"
tree_accept_no_update = _tree_variant(update=False)           # mistake: siblings tested against p itself
tree_accept_no_update.__name__ = "tree_accept_no_update"


CASES = [
    ("verify_attn", verify_off_by_one, pins.test_verify_rows_are_prefix_attention),
    ("verify_attn", verify_off_by_one, pins.test_verify_alignment_closed_form),
    ("attention", attention_unscaled, pins.test_attention_matches_library_sdpa_and_logsumexp),
    ("chunk_keys", chunk_keys_fixed_divisor, lambda: pins.test_chunk_keys_ramp_closed_form(67, 8)),
    ("select_topk", topk_ties_high_index, pins.test_topk_exhaustive_tie_patterns),
    ("stream_positions", stream_positions_short, lambda: pins.test_stream_ring_equals_mask_and_library(1000, 4, 252)),
    ("accept", accept_flipped_residual, pins.test_accept_hand_examples),
    ("accept", accept_no_bonus, pins.test_accept_hand_examples),
    ("accept", accept_token_index_wraps, pins.test_accept_hand_examples),
    ("accept", accept_token_clamped, pins.test_accept_hand_examples),
    ("round_f64_to_bits", round_fp16_via_fp32, pins.test_round_to_fp16_ties_subnormals_and_library),
    ("round_f64_to_bits", round_fp16_truncates, pins.test_round_to_fp16_ties_subnormals_and_library),
    ("append_ring", append_ring_short_reserve, pins.test_ring_without_slack_refuses_and_would_corrupt),
    ("commit_length", commit_drops_one_more, pins.test_commit_length_closed_forms),
    ("commit_length", commit_drops_one_more, pins.test_full_cache_decode_loop_matches_list_model),
    ("ring_slot_of", ring_slot_one_short, pins.test_ring_slot_hand_table),
    ("tree_masks", tree_masks_no_self, pins.test_tree_masks_hand_table),
    ("tree_accept", tree_accept_unnormalised, pins.test_tree_accept_is_lossless_statistically),
    ("tree_accept", tree_accept_no_update, pins.test_tree_accept_hand_examples),
    ("tree_accept", tree_accept_no_update, pins.test_tree_accept_is_lossless_statistically),
    ("verify_tree_attn", verify_tree_base_off_by_one, pins.test_verify_tree_chain_is_verify_and_rows_match_masked_sdpa),
    ("two_level_accept", two_level_level1_swapped, pins.test_two_level_hand_examples),
    ("two_level_accept", two_level_level1_swapped, pins.test_two_level_is_lossless_statistically),
    ("two_level_accept", two_level_draft_rows_r, pins.test_two_level_is_lossless_statistically),
    ("two_level_accept", two_level_rows_shifted, pins.test_two_level_hand_examples),
    ("two_level_accept", two_level_rows_shifted, pins.test_two_level_is_lossless_statistically),
]


@pytest.mark.parametrize("name,bad,pin", CASES, ids=[f"{c[0]}-{c[1].__name__}" for c in CASES])
def test_pin_catches_planted_mistake(monkeypatch, name, bad, pin):
    _patch(monkeypatch, name, bad)
    with pytest.raises(AssertionError):
        pin()
