"""Seeded synthetic inputs for the decode-attention path.

This module only *generates* inputs: random key/value caches, queries, planted
query-correlated chunks, streaming ring-buffer placement, accept-test logits,
draft tokens and uniforms.  It holds none of the method's arithmetic (no chunk
means, no scores, no selection, no softmax, no attention, no acceptance); both
the HIP path and the CPU oracle consume what it produces.

Workload shapes follow the workloads the TriForce pages discuss: the Llama2-7B
128K-context model (32 heads of dimension 128, 32 layers) named in the arXiv
abstract (mlsanity / fugumt pages, "Abstract"), the retrieval budget "top k =
2,048 tokens out of 128k" and the W = 256 streaming window of the aifetchly
blog "TriForce: Hierarchical Speculative Decoding for LLMs", section "1. The
Three Forces of TriForce".  Everything is synthetic: no weights, prompts or
datasets are involved.

Reduced-precision storage: values are drawn in fp32 and rounded once, round to
nearest even, to fp16 or bf16.  bf16 data is carried in numpy as raw uint16 bit
patterns (numpy has no bf16 type); fp16 data also as uint16 bit patterns so both
dtypes share one container.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# Named workloads.  Names say what they are; sizes are the workload's own.
# ---------------------------------------------------------------------------

LLAMA2_RAGGED_LENS = [16384, 24576, 32768, 49152, 65536, 65536, 98304, 131072]

WORKLOADS: Dict[str, dict] = {
    # Small single layer the oracle finishes in seconds.
    "tiny-h8-n4k-fp16": dict(
        B=1, Hq=8, Hkv=8, d=128, lens=[4096], dtype="fp16", layers=1,
        chunk_size=8, budget=512, n_sink=4, window=252, gamma=4, vocab=32000,
        plant="count", plant_count=4),
    # Llama2-7B-128K, one layer (MHA, 32 heads).
    "llama2-7b-128k-1layer": dict(
        B=1, Hq=32, Hkv=32, d=128, lens=[131072], dtype="bf16", layers=1,
        chunk_size=8, budget=4096, n_sink=4, window=252, gamma=6, vocab=32000,
        plant="fraction", plant_fraction=0.01),
    # Llama2-7B-128K, all 32 layers resident (64 GiB of bf16 K/V).
    "llama2-7b-128k-32layers": dict(
        B=1, Hq=32, Hkv=32, d=128, lens=[131072], dtype="bf16", layers=32,
        chunk_size=8, budget=4096, n_sink=4, window=252, gamma=6, vocab=32000,
        plant="fraction", plant_fraction=0.01),
    # Eight sequences of mixed length, one layer.
    "ragged-b8-16k-128k": dict(
        B=8, Hq=32, Hkv=32, d=128, lens=LLAMA2_RAGGED_LENS, dtype="bf16",
        layers=1, chunk_size=8, budget=4096, budgets=[2048, 4096], n_sink=4,
        window=252, gamma=6, gammas=[4, 6, 8], vocab=32000,
        plant="fraction", plant_fraction=0.01),
    # GQA (32 query heads over 8 KV heads), 512K context, 16 layers.
    "gqa-hq32-hkv8-512k-16layers": dict(
        B=1, Hq=32, Hkv=8, d=128, lens=[524288], dtype="bf16", layers=16,
        chunk_size=16, budget=8192, n_sink=4, window=252, gamma=8, vocab=32000,
        plant="zipf", zipf_s=1.1),
}

STREAM_SLACK = 16  # spare ring slots beyond the window (room for gamma appends)
POISON = 1000.0    # finite, exactly representable in fp16 and bf16


# ---------------------------------------------------------------------------
# Rounding of synthetic fp32 data to 16-bit storage (round to nearest even).
# ---------------------------------------------------------------------------

def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 data to fp16/bf16 (nearest even) and return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        lsb = (u >> np.uint64(16)) & np.uint64(1)
        r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
        return r.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype}")


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit storage to fp32 (used only while generating:
    planting needs the rounded query values)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


# ---------------------------------------------------------------------------
# Containers
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class KVLayout:
    """Head-major ragged layout: sequence b, head g, row t lives at element
    seq_base[b] + (g * seq_cap[b] + t) * d of a flat buffer."""
    B: int
    H: int
    d: int
    seq_len: np.ndarray   # int32 [B]
    seq_cap: np.ndarray   # int32 [B]
    seq_base: np.ndarray  # int64 [B]

    @property
    def total_elems(self) -> int:
        return int(sum(int(c) * self.H * self.d for c in self.seq_cap))

    @property
    def max_len(self) -> int:
        return int(self.seq_len.max()) if self.B else 0

    @staticmethod
    def build(lens: Sequence[int], H: int, d: int, caps: Optional[Sequence[int]] = None,
              align_rows: int = 1) -> "KVLayout":
        lens = [int(n) for n in lens]
        if caps is None:
            caps = [max(1, -(-n // align_rows) * align_rows) for n in lens]
        base, off = [], 0
        for c in caps:
            base.append(off)
            off += int(c) * H * d
        return KVLayout(B=len(lens), H=H, d=d,
                        seq_len=np.asarray(lens, np.int32),
                        seq_cap=np.asarray(caps, np.int32),
                        seq_base=np.asarray(base, np.int64))

    def head(self, flat: np.ndarray, b: int, g: int, rows: Optional[int] = None) -> np.ndarray:
        """View of the [rows][d] slab of (b, g); rows defaults to seq_len[b]."""
        n = int(self.seq_len[b]) if rows is None else int(rows)
        start = int(self.seq_base[b]) + g * int(self.seq_cap[b]) * self.d
        return flat[start:start + n * self.d].reshape(n, self.d)


@dataclasses.dataclass
class AttnInputs:
    dtype: str
    layout: KVLayout
    Hq: int
    K: np.ndarray          # uint16 bits, flat
    V: np.ndarray          # uint16 bits, flat
    q_verify: np.ndarray   # uint16 bits [B][Hq][Q][d]; row 0 is the draft query
    q_draft: np.ndarray    # uint16 bits [B][Hq][1][d] (copy of row 0)
    planted: List[np.ndarray]  # per sequence: planted chunk indices (sorted)
    chunk_size: int


# ---------------------------------------------------------------------------
# Seeds: one independent PCG64 stream per tensor.
# ---------------------------------------------------------------------------

_STREAMS = ["K", "V", "q", "qv", "plant_idx", "plant_noise", "zipf_perm", "ring",
            "logits_t", "logits_d", "tokens", "uniforms", "extra"]


def rngs(seed: int, layer: int = 0) -> Dict[str, np.random.Generator]:
    ss = np.random.SeedSequence([int(seed), int(layer)])
    kids = ss.spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(k)) for name, k in zip(_STREAMS, kids)}


def torch_seed(seed: int, layer: int, name: str) -> int:
    idx = _STREAMS.index(name)
    ss = np.random.SeedSequence([int(seed), int(layer), 7919, idx])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


# ---------------------------------------------------------------------------
# Attention inputs on the host (numpy).  Used for everything the oracle checks
# in full; large workloads use the torch generator below with the same recipe.
# ---------------------------------------------------------------------------

def make_attn_inputs(*, lens: Sequence[int], Hq: int, Hkv: int, d: int = 128,
                     dtype: str = "bf16", Q: int = 1, seed: int = 0, layer: int = 0,
                     chunk_size: int = 8, plant: Optional[str] = None,
                     plant_count: int = 0, plant_fraction: float = 0.0,
                     zipf_s: float = 1.1, cap_extra: int = 0,
                     poison_tail: bool = True) -> AttnInputs:
    """K, V ~ N(0, 1); queries ~ N(0, 1); optional planted chunks.

    Planting (count / fraction): chunk indices are drawn without replacement,
    the same for every head; each key row of a planted chunk is
    0.5 * q_h + N(0, sd=0.5), q_h being that head's (rounded) draft query.
    With GQA the mean of the group's draft queries stands in for q_h.
    Zipf planting: per KV head a random permutation ranks the chunks 1..C and
    the rows of the rank-r chunk get 0.5 * r**(-s) * qbar added to N(0, 1).
    Rows in [len, cap) hold POISON so that any read past the end shows up.
    """
    G = Hq // Hkv
    caps = [int(n) + int(cap_extra) for n in lens]
    lay = KVLayout.build(lens, Hkv, d, caps=[max(1, c) for c in caps])
    r = rngs(seed, layer)
    K = r["K"].standard_normal(lay.total_elems, dtype=np.float32)
    V = r["V"].standard_normal(lay.total_elems, dtype=np.float32)
    B = lay.B
    qv = r["qv"].standard_normal((B, Hq, Q, d), dtype=np.float32)
    qd = r["q"].standard_normal((B, Hq, 1, d), dtype=np.float32)
    qv[:, :, 0, :] = qd[:, :, 0, :]
    q_bits = to_bits(qv, dtype)
    q_round = bits_to_f32(q_bits, dtype)  # [B][Hq][Q][d]
    planted: List[np.ndarray] = []
    for b in range(B):
        n = int(lens[b])
        C = -(-n // chunk_size) if n > 0 else 0
        if plant in ("count", "fraction") and C > 0:
            cnt = plant_count if plant == "count" else int(round(plant_fraction * C))
            cnt = min(cnt, C)
            sel = np.sort(r["plant_idx"].choice(C, size=cnt, replace=False)) if cnt else np.zeros(0, np.int64)
            planted.append(sel.astype(np.int64))
            for g in range(Hkv):
                qbar = q_round[b, g * G:(g + 1) * G, 0, :].mean(axis=0)
                rows = lay.head(K, b, g)
                for c in sel:
                    lo, hi = c * chunk_size, min(n, (c + 1) * chunk_size)
                    rows[lo:hi] = 0.5 * qbar + r["plant_noise"].normal(0.0, 0.5, (hi - lo, d)).astype(np.float32)
        elif plant == "zipf" and C > 0:
            planted.append(np.zeros(0, np.int64))
            for g in range(Hkv):
                qbar = q_round[b, g * G:(g + 1) * G, 0, :].mean(axis=0)
                perm = r["zipf_perm"].permutation(C)      # perm[c] = rank-1 of chunk c
                w = 0.5 * (perm.astype(np.float64) + 1.0) ** (-zipf_s)
                rows = lay.head(K, b, g)
                full = (n // chunk_size) * chunk_size
                rows[:full] += (np.repeat(w[:n // chunk_size], chunk_size)[:, None] * qbar[None, :]).astype(np.float32)
                if full < n:
                    rows[full:n] += (w[-1] * qbar[None, :]).astype(np.float32)
        else:
            planted.append(np.zeros(0, np.int64))
        if poison_tail:
            for g in range(Hkv):
                lay.head(K, b, g, rows=int(lay.seq_cap[b]))[n:] = POISON
                lay.head(V, b, g, rows=int(lay.seq_cap[b]))[n:] = POISON
    return AttnInputs(dtype=dtype, layout=lay, Hq=Hq, K=to_bits(K, dtype), V=to_bits(V, dtype),
                      q_verify=q_bits, q_draft=np.ascontiguousarray(q_bits[:, :, :1, :]),
                      planted=planted, chunk_size=chunk_size)


# ---------------------------------------------------------------------------
# Streaming (sink + window) cache, stored as a ring buffer.
# Layout contract: per (sequence, head) the cache has cap >= n_sink + window
# slots; logical position p < n_sink lives in slot p; position p >= n_sink
# lives in slot n_sink + (p - n_sink) mod (cap - n_sink).
# ---------------------------------------------------------------------------

def ring_slot(p: int, n_sink: int, cap: int) -> int:
    return p if p < n_sink else n_sink + (p - n_sink) % (cap - n_sink)


@dataclasses.dataclass
class StreamInputs:
    dtype: str
    layout: KVLayout        # seq_len = logical length n_b, seq_cap = slots
    Hq: int
    n_sink: int
    window: int
    Ks: np.ndarray          # uint16 bits, flat ring buffers
    Vs: np.ndarray
    K_logical: List[np.ndarray]  # per b: uint16 [Hkv][n][d] logical sequence
    V_logical: List[np.ndarray]
    q: np.ndarray           # uint16 bits [B][Hq][1][d]


def make_stream_inputs(*, lens: Sequence[int], Hq: int, Hkv: int, d: int = 128,
                       dtype: str = "bf16", n_sink: int = 4, window: int = 252,
                       slack: int = STREAM_SLACK, seed: int = 0, layer: int = 0) -> StreamInputs:
    """A logical K/V sequence per (b, head) of length n_b ~ N(0, 1), written
    into the ring as an append-only writer would leave it: the sinks and the
    most recent positions that still own a slot.  Slots that no visible
    position owns are filled with POISON."""
    cap = n_sink + window + slack
    lay = KVLayout.build(lens, Hkv, d, caps=[cap] * len(lens))
    r = rngs(seed, layer)
    Ks = np.full(lay.total_elems, POISON, np.float32)
    Vs = np.full(lay.total_elems, POISON, np.float32)
    KL, VL = [], []
    for b, n in enumerate(lens):
        n = int(n)
        kl = r["ring"].standard_normal((Hkv, n, d), dtype=np.float32)
        vl = r["ring"].standard_normal((Hkv, n, d), dtype=np.float32)
        kb, vb = to_bits(kl, dtype), to_bits(vl, dtype)
        KL.append(kb)
        VL.append(vb)
        # Visible positions: sinks, then the last `window` positions.
        vis = list(range(min(n_sink, n))) + list(range(max(n_sink, n - window), n))
        for g in range(Hkv):
            hk = lay.head(Ks, b, g, rows=cap)
            hv = lay.head(Vs, b, g, rows=cap)
            for p in vis:
                s = ring_slot(p, n_sink, cap)
                hk[s] = kl[g, p]
                hv[s] = vl[g, p]
    q = to_bits(r["q"].standard_normal((lay.B, Hq, 1, d), dtype=np.float32), dtype)
    return StreamInputs(dtype=dtype, layout=lay, Hq=Hq, n_sink=n_sink, window=window,
                        Ks=to_bits(Ks, dtype), Vs=to_bits(Vs, dtype),
                        K_logical=KL, V_logical=VL, q=q)


# ---------------------------------------------------------------------------
# Accept-test inputs.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class AcceptInputs:
    target: np.ndarray     # float32 [B][gamma+1][V]
    draft: np.ndarray      # float32 [B][gamma][V]
    tokens: np.ndarray     # int32 [B][gamma]
    uniforms: np.ndarray   # float64 [B][gamma+1], each in (0, 1)


def open_uniforms(g: np.random.Generator, shape) -> np.ndarray:
    u = g.random(shape)
    while np.any(u == 0.0):
        z = u == 0.0
        u[z] = g.random(int(z.sum()))
    return u


def make_accept_inputs(*, B: int, gamma: int, vocab: int = 32000, sd: float = 2.0,
                       correlated: bool = False, seed: int = 0, layer: int = 0) -> AcceptInputs:
    """Target and draft logits i.i.d. N(0, sd) in fp32 (sd is the standard
    deviation); with correlated=True the draft logits are the target's plus
    N(0, 0.5) so that long accepted runs occur.  Draft tokens are uniform over
    the vocabulary here; tests that need tokens drawn from the draft
    distribution draw them themselves."""
    r = rngs(seed, layer)
    t = r["logits_t"].normal(0.0, sd, (B, gamma + 1, vocab)).astype(np.float32)
    if correlated:
        dl = (t[:, :gamma, :] + r["logits_d"].normal(0.0, 0.5, (B, gamma, vocab))).astype(np.float32)
    else:
        dl = r["logits_d"].normal(0.0, sd, (B, gamma, vocab)).astype(np.float32)
    tok = r["tokens"].integers(0, vocab, (B, gamma)).astype(np.int32)
    u = open_uniforms(r["uniforms"], (B, gamma + 1))
    return AcceptInputs(target=t, draft=np.ascontiguousarray(dl), tokens=tok, uniforms=u)


# ---------------------------------------------------------------------------
# Device-side generation for the large workloads (same recipe, torch RNG).
# ---------------------------------------------------------------------------

def make_layer_torch(*, lens: Sequence[int], Hq: int, Hkv: int, d: int, dtype: str,
                     Q: int, chunk_size: int, plant: Optional[str], seed: int, layer: int,
                     device, plant_fraction: float = 0.01, plant_count: int = 0,
                     zipf_s: float = 1.1, K_out=None, V_out=None, extra_rows: int = 0):
    """Generate one layer directly in device memory.

    Returns (K, V, q_verify, q_draft, layout, planted) with K and V flat torch
    tensors of the storage dtype laid out as KVLayout describes; planted[b]
    lists the planted chunk indices (Zipf: the rank-1..3 chunks per KV head).  K_out/V_out
    may be preallocated flat views to fill (so many layers can share one big
    allocation).  The recipe is the one of make_attn_inputs; the random
    streams differ (torch Philox instead of numpy PCG64).  extra_rows adds
    room after every sequence's rows (filled with N(0, 1) values too) for
    rows a decode loop appends."""
    import torch
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    G = Hq // Hkv
    lay = KVLayout.build(lens, Hkv, d, caps=[int(n) + int(extra_rows) for n in lens])
    n_el = lay.total_elems
    gk = torch.Generator(device=device).manual_seed(torch_seed(seed, layer, "K"))
    gv = torch.Generator(device=device).manual_seed(torch_seed(seed, layer, "V"))
    gq = torch.Generator(device=device).manual_seed(torch_seed(seed, layer, "q"))
    K = K_out if K_out is not None else torch.empty(n_el, dtype=tdt, device=device)
    V = V_out if V_out is not None else torch.empty(n_el, dtype=tdt, device=device)
    step = 1 << 26
    for off in range(0, n_el, step):
        m = min(step, n_el - off)
        K[off:off + m] = torch.randn(m, generator=gk, device=device, dtype=torch.float32).to(tdt)
        V[off:off + m] = torch.randn(m, generator=gv, device=device, dtype=torch.float32).to(tdt)
    B = lay.B
    qv = torch.randn((B, Hq, Q, d), generator=gq, device=device, dtype=torch.float32)
    qd = torch.randn((B, Hq, 1, d), generator=gq, device=device, dtype=torch.float32)
    qv[:, :, 0, :] = qd[:, :, 0, :]
    qv = qv.to(tdt)
    q_round = qv.float()
    r = rngs(seed, layer)
    gn = torch.Generator(device=device).manual_seed(torch_seed(seed, layer, "plant_noise"))
    planted = []
    for b in range(B):
        n = int(lens[b])
        C = -(-n // chunk_size)
        base = int(lay.seq_base[b])
        cap = int(lay.seq_cap[b])
        if plant in ("count", "fraction") and C > 0:
            cnt = plant_count if plant == "count" else int(round(plant_fraction * C))
            sel = np.sort(r["plant_idx"].choice(C, size=min(cnt, C), replace=False))
            planted.append(sel.astype(np.int64))
            sel_t = torch.as_tensor(sel, device=device)
            rows = (sel_t[:, None] * chunk_size + torch.arange(chunk_size, device=device)[None, :]).reshape(-1)
            rows = rows[rows < n]
            for g in range(Hkv):
                qbar = q_round[b, g * G:(g + 1) * G, 0, :].mean(dim=0)
                head = K[base + g * cap * d: base + (g + 1) * cap * d].view(cap, d)
                noise = torch.randn((rows.numel(), d), generator=gn, device=device) * 0.5
                head[rows] = (0.5 * qbar[None, :] + noise).to(tdt)
        elif plant == "zipf" and C > 0:
            top = np.zeros((Hkv, 3), np.int64)  # per KV head: chunks of rank 1, 2, 3
            full_chunks = n // chunk_size
            for g in range(Hkv):
                perm_np = r["zipf_perm"].permutation(C)
                top[g] = np.argsort(perm_np)[:3]
                perm = torch.as_tensor(perm_np, device=device)
                w = 0.5 * (perm.double() + 1.0) ** (-zipf_s)
                qbar = q_round[b, g * G:(g + 1) * G, 0, :].mean(dim=0)
                head = K[base + g * cap * d: base + (g + 1) * cap * d].view(cap, d)
                wr = w[:full_chunks].repeat_interleave(chunk_size).float()
                head[:full_chunks * chunk_size] = (head[:full_chunks * chunk_size].float()
                                                   + wr[:, None] * qbar[None, :]).to(tdt)
                if full_chunks * chunk_size < n:
                    t0 = full_chunks * chunk_size
                    head[t0:n] = (head[t0:n].float() + float(w[-1]) * qbar[None, :]).to(tdt)
            planted.append(top)
        else:
            planted.append(np.zeros(0, np.int64))
    return K, V, qv.contiguous(), qv[:, :, :1, :].contiguous(), lay, planted
