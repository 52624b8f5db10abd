"""tf_verify_attn_noalloc (split partials in the library's built-in scratch,
nothing allocated) against tf_verify_attn (caller workspace), through the C
ABI: bitwise-equal outputs on two calls in a row, the second with a smaller
input so that partials left by the first would show; a small case also
against the fp64 oracle; a call too large for the scratch is refused."""

import sys

import numpy as np
import pytest
import torch

from hierarchical_speculative_attention_amd import synth
import hierarchical_speculative_attention_amd as tf
from tests.gpu_util import compare_attn, desc, dev, oracle_verify

pytestmark = pytest.mark.gpu


def both(inp, Q):
    """(out, lse) of tf_verify_attn and of tf_verify_attn_noalloc on inp."""
    kv = desc(inp.layout, inp.dtype)
    q, K, V = dev(inp.q_verify, inp.dtype), dev(inp.K, inp.dtype), dev(inp.V, inp.dtype)
    o_ref, l_ref = tf.verify_attn(q, K, V, kv)
    out = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    tf.verify_attn_noalloc(q, K, V, kv, out, lse)
    torch.cuda.synchronize()
    return (o_ref, l_ref), (out, lse)


def test_noalloc_equals_workspace_call_twice_then_smaller():
    # first call: 32 KV heads of 40000 rows (16 splits, partials in the scratch);
    # second call: GQA 8 x 2 heads of 3000 rows -- fewer splits, fewer rows
    for i, (lens, Hq, Hkv, Q) in enumerate([([40000], 32, 32, 7), ([3000, 2900], 8, 2, 5)]):
        print(f"noalloc call {i}: lens={lens} Hq={Hq} Hkv={Hkv} Q={Q}", flush=True)
        inp = synth.make_attn_inputs(lens=lens, Hq=Hq, Hkv=Hkv, dtype="bf16", Q=Q, seed=60 + i, cap_extra=5)
        (o_ref, l_ref), (out, lse) = both(inp, Q)
        assert torch.equal(out, o_ref), i
        assert torch.equal(lse, l_ref), i


def test_noalloc_matches_oracle_small():
    inp = synth.make_attn_inputs(lens=[700, 4100], Hq=8, Hkv=2, dtype="fp16", Q=5, seed=62, cap_extra=3)
    (_, _), (out, lse) = both(inp, 5)
    compare_attn(out, lse, *oracle_verify(inp, 5))


def test_noalloc_refuses_a_call_beyond_the_scratch():
    cap = tf.verify_attn_noalloc_max_bytes()
    assert cap == 48 << 20
    max_len = 1 << 22   # one sequence: 512 splits per head
    need = tf.verify_attn_workspace_size(1, 32, 32, 7, max_len)
    assert need > cap
    lay = synth.KVLayout.build([64], 32, 128, caps=[64])   # small buffers; max_len sizes the plan
    kv = desc(lay, "bf16", max_len=max_len)
    q = torch.zeros((1, 32, 7, 128), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros(lay.total_elems, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((1, 32, 7, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(tf.TfError) as e:
        tf.verify_attn_noalloc(q, K, K, kv, out)
    assert e.value.status == tf.TF_ERR_WORKSPACE
    assert torch.count_nonzero(out) == 0          # nothing was enqueued
