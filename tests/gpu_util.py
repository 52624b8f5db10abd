"""Helpers for the GPU tests: move generator output to the device and back,
and run the oracle per (sequence, head).  No method arithmetic here beyond
calling the oracle."""

import numpy as np
import torch

import oracle
from hierarchical_speculative_attention_amd import KVDesc

TDT = {"fp16": torch.float16, "bf16": torch.bfloat16}
ATOL = 2e-3  # max abs error bound for attention outputs (fp32 accumulate, 16-bit K/V)


def dev(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """uint16 bit patterns -> device tensor of the 16-bit dtype."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TDT[dtype]).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def desc(layout, dtype: str, device="cuda", seq_len=None, max_len=None) -> KVDesc:
    return KVDesc.from_layout(layout, TDT[dtype], device, seq_len=seq_len, max_len=max_len)


def oracle_verify(inp, Q):
    lay, dt = inp.layout, inp.dtype
    G = inp.Hq // lay.H
    B = lay.B
    o = np.zeros((B, inp.Hq, Q, lay.d))
    lse = np.zeros((B, inp.Hq, Q))
    for b in range(B):
        n = int(lay.seq_len[b])
        for g in range(lay.H):
            K = oracle.widen(lay.head(inp.K, b, g), dt)
            V = oracle.widen(lay.head(inp.V, b, g), dt)
            for j in range(G):
                h = g * G + j
                qs = oracle.widen(inp.q_verify[b, h], dt)
                o[b, h], lse[b, h] = oracle.verify_attn(qs, K, V, n)
    return o, lse


def oracle_sparse(inp, idx, cs):
    lay, dt = inp.layout, inp.dtype
    G = inp.Hq // lay.H
    o = np.zeros((lay.B, inp.Hq, lay.d))
    lse = np.zeros((lay.B, inp.Hq))
    for b in range(lay.B):
        n = int(lay.seq_len[b])
        for g in range(lay.H):
            K = oracle.widen(lay.head(inp.K, b, g), dt)
            V = oracle.widen(lay.head(inp.V, b, g), dt)
            for j in range(G):
                h = g * G + j
                o[b, h], lse[b, h] = oracle.sparse_attn(oracle.widen(inp.q_draft[b, h, 0], dt), K, V, n, idx[b, g], cs)
    return o, lse


def compare_attn(o_gpu, lse_gpu, o_ref, lse_ref, atol=ATOL):
    o_gpu = o_gpu.detach().cpu().double().numpy()
    lse_gpu = lse_gpu.detach().cpu().double().numpy()
    assert o_gpu.shape == o_ref.shape
    err = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    assert err <= atol, f"max abs error {err:.3e} > {atol}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), "lse -inf pattern differs"
    if fin.any():
        lerr = np.abs(lse_gpu[fin] - lse_ref[fin]).max()
        assert lerr <= atol, f"lse max abs error {lerr:.3e}"
    assert np.all(o_gpu[~fin] == 0.0)
    return err
