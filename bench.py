"""Decode-step benchmark of the TriForce decode-attention path on one MI355X.

One step = for every layer: refresh of the chunk-mean keys the newest rows
fell into, query-to-chunk scores, top-k selection, attention over the
gathered chunks (the sparse draft), sink + window streaming attention (the
small drafter) and full-cache verification of the gamma + 1 draft positions;
then one accept / reject over the vocabulary and the 8-byte-per-sequence
read-back of its result.  Inputs are synthetic, seeded, resident in HBM
before timing starts.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints one JSON line.  Only one GPU is used; --gpus above 1 exits.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn GB/s & % HBM peak, sparse-draft+verify steps/s at 128K ctx"
EXTRA_ROWS = 512  # room after every sequence's rows for the rows the three-tier loop appends
HBM_PEAK_GBPS = 8000.0
WARM_REPLAYS = 5      # untimed replays of each per-kernel graph
KERNEL_REPS = 20      # timed replays of each per-kernel graph
COPY_REPS = 10        # timed 1 GiB device-to-device copies (the secondary peak)
SMALL_REPS = 8        # calls per graph for the once-per-step calls (accept), so the graph launch is amortised
MIN_LAUNCHES = 8      # per-kernel graphs cycle the layers until they hold at least this many launches
CSRC = os.path.join(ROOT, "hierarchical_speculative_attention_amd", "csrc")
VERIFY_SRCS = [os.path.join(CSRC, f) for f in ("attn.hip", "api.hip", "tf_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_attn_llama2-7b-128k_traffic.txt")
DEFAULT_WORKLOAD = "llama2-7b-128k-32layers"  # the shape the committed traffic counters were taken on


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--budget", type=int, default=None, help="override the workload's token budget (retrieval)")
    ap.add_argument("--gamma", type=int, default=None, help="override the workload's draft count (verify rows - 1)")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=16, help="layers the CPU oracle baseline times")
    ap.add_argument("--ck-dtype", default="kv", choices=["kv", "fp32"])
    ap.add_argument("--no-three-tier", action="store_true", help="skip the three-tier step loop")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the per-call timing of sparse verification, tree verification / accept and appends")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the per-kernel figures of the GQA 512K and ragged 8-sequence workloads")
    return ap.parse_args()


def sources_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per verify launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("attn_hip_sha256") != sources_sha(VERIFY_SRCS):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


TRACE_FILE = os.path.join(ROOT, "profiles", "verify_attn_llama2-7b-128k_kernel_trace.txt")


def read_kernel_trace(verify_bytes, sparse_bytes=None):
    """Each verify kernel's own average duration from the committed rocprofv3
    kernel-trace summary (if it was taken on the current kernel source), and
    the fractions of the HBM peak they give: the attention kernel alone, and
    the attention kernel plus the split merge; with sparse_bytes, the same for
    the gathered sparse pass (its own key lines) under "sparse"."""
    if not os.path.exists(TRACE_FILE):
        return None
    kv = {}
    for line in open(TRACE_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("attn_hip_sha256") != sources_sha(VERIFY_SRCS):
        return None
    try:
        a, m = float(kv["attention_kernel_avg_us"]), float(kv["split_merge_kernel_avg_us"])
    except (KeyError, ValueError):
        return None
    out = {"attention_kernel_us": a, "split_merge_kernel_us": m,
           "frac_attention_kernel": round(verify_bytes / (a * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "frac_both_kernels": round(verify_bytes / ((a + m) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "source": os.path.relpath(TRACE_FILE, ROOT)}
    if sparse_bytes is not None and "sparse_kernel_avg_us" in kv:
        try:
            g, sm = float(kv["sparse_kernel_avg_us"]), float(kv["sparse_split_merge_kernel_avg_us"])
        except (KeyError, ValueError):
            return out
        out["sparse"] = {"gather_kernel_us": g, "split_merge_kernel_us": sm,
                         "frac_gather_kernel": round(sparse_bytes / (g * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                         "frac_both_kernels": round(sparse_bytes / ((g + sm) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    return out


class Layer:
    pass


def build_layers(W, layers, Q, ck_dt, tdt, dev, stream):
    """The workload's layers, generated on the device (synth.make_layer_torch):
    full K/V with EXTRA_ROWS of room per sequence, the queries, the chunk-key
    buffer and a sink + window ring per layer."""
    import torch
    import hierarchical_speculative_attention_amd as tf
    from hierarchical_speculative_attention_amd import synth
    B, Hq, Hkv, d, lens, cs = W["B"], W["Hq"], W["Hkv"], W["d"], W["lens"], W["chunk_size"]
    S, Wn = W["n_sink"], W["window"]
    C = [-(-n // cs) for n in lens]
    L = []
    with torch.cuda.stream(stream):
        for l in range(layers):
            K, V, qv, qd, lay, planted = synth.make_layer_torch(
                lens=lens, Hq=Hq, Hkv=Hkv, d=d, dtype=W["dtype"], Q=Q, chunk_size=cs, plant=W["plant"],
                seed=0, layer=l, device=dev, plant_fraction=W.get("plant_fraction", 0.01),
                plant_count=W.get("plant_count", 0), zipf_s=W.get("zipf_s", 1.1), extra_rows=EXTRA_ROWS)
            x = Layer()
            x.K, x.V, x.qv, x.qd = K, V, qv, qd.view(B, Hq, d)
            x.kv = tf.KVDesc.from_layout(lay, tdt, dev)
            ck_lay = synth.KVLayout.build(C, Hkv, d, caps=C)
            x.ckd = tf.KVDesc.from_layout(ck_lay, ck_dt, dev)
            x.ck = torch.empty(ck_lay.total_elems, dtype=ck_dt, device=dev)
            g = torch.Generator(device=dev).manual_seed(synth.torch_seed(0, l, "ring"))
            scap = S + Wn + synth.STREAM_SLACK
            s_lay = synth.KVLayout.build(lens, Hkv, d, caps=[scap] * B)
            x.Ks = torch.randn(s_lay.total_elems, generator=g, device=dev).to(tdt)
            x.Vs = torch.randn(s_lay.total_elems, generator=g, device=dev).to(tdt)
            x.sd = tf.KVDesc.from_layout(s_lay, tdt, dev)
            x.planted = planted
            L.append(x)
    stream.synchronize()
    return L


def step_context(W, budget, gamma, ck_dt, tdt, dev, stream):
    """Buffers one decode step of the workload shares across its layers, and
    the per-layer calls of the step."""
    import torch
    import hierarchical_speculative_attention_amd as tf
    from hierarchical_speculative_attention_amd import synth
    c = Layer()
    c.B, c.Hq, c.Hkv, c.d, c.lens = W["B"], W["Hq"], W["Hkv"], W["d"], W["lens"]
    c.cs, c.budget, c.gamma, c.vocab = W["chunk_size"], budget, gamma, W["vocab"]
    c.S, c.Wn = W["n_sink"], W["window"]
    c.Q, c.k = gamma + 1, budget // c.cs
    c.C = [-(-n // c.cs) for n in c.lens]
    c.c_max = max(c.C)
    B, Hq, Hkv, d, Q, k = c.B, c.Hq, c.Hkv, c.d, c.Q, c.k
    with torch.cuda.stream(stream):
        c.n_chunks = torch.tensor(c.C, dtype=torch.int32, device=dev)
        c.tail_chunk = torch.tensor([max(0, (n - Q) // c.cs) for n in c.lens], dtype=torch.int32, device=dev)
        c.tail_count = (Q + c.cs - 1) // c.cs + 1
        c.scores = torch.empty((B, Hkv, c.c_max), dtype=torch.float32, device=dev)
        c.idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        c.o_sp = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        c.l_sp = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        c.o_st = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        c.l_st = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        c.o_v = torch.empty((B, Hq, Q, d), dtype=torch.float32, device=dev)
        c.l_v = torch.empty((B, Hq, Q), dtype=torch.float32, device=dev)
        c.ws_v = tf.workspace(tf.verify_attn_workspace_size(B, Hq, Hkv, Q, max(c.lens)), dev)
        c.ws_s = tf.workspace(tf.sparse_attn_workspace_size(B, Hq, Hkv, k, c.cs), dev)
        c.ws_t = tf.workspace(tf.select_topk_workspace_size(B, Hkv, c.c_max, k), dev)
        c.ws_a = tf.workspace(tf.accept_workspace_size(B, gamma, c.vocab), dev)
        c.acc_in = synth.make_accept_inputs(B=B, gamma=gamma, vocab=c.vocab, seed=0)
        c.tgt = torch.from_numpy(c.acc_in.target).to(dev)
        c.drf = torch.from_numpy(c.acc_in.draft).to(dev)
        c.tok = torch.from_numpy(c.acc_in.tokens).to(dev)
        c.uni = torch.from_numpy(c.acc_in.uniforms).to(dev)
        c.n_acc = torch.empty(B, dtype=torch.int32, device=dev)
        c.nxt = torch.empty(B, dtype=torch.int32, device=dev)
        c.host_out = torch.empty(2 * B, dtype=torch.int32).pin_memory()
    stream.synchronize()

    def layer_calls(x):
        return [
            ("chunk_refresh", lambda: tf.build_chunk_keys(x.K, x.kv, c.cs, x.ck, x.ckd, chunk_begin=c.tail_chunk,
                                                          max_chunks=c.tail_count, stream=stream)),
            ("score", lambda: tf.score_chunks(x.qd, Hq, x.ck, x.ckd, c.c_max, scores=c.scores, stream=stream)),
            ("topk", lambda: tf.select_topk(c.scores, c.n_chunks, k, idx=c.idx, ws=c.ws_t, stream=stream)),
            ("sparse", lambda: tf.sparse_attn(x.qd, x.K, x.V, x.kv, c.idx, c.cs, out=c.o_sp, lse=c.l_sp, ws=c.ws_s,
                                              stream=stream)),
            ("stream", lambda: tf.stream_attn(x.qd, x.Ks, x.Vs, x.sd, c.S, c.Wn, out=c.o_st, lse=c.l_st,
                                              stream=stream)),
            ("verify", lambda: tf.verify_attn(x.qv, x.K, x.V, x.kv, out=c.o_v, lse=c.l_v, ws=c.ws_v, stream=stream)),
        ]

    def accept_call():
        tf.accept(c.tgt, c.drf, c.tok, c.uni, 1.0, n_accepted=c.n_acc, next_token=c.nxt, ws=c.ws_a, stream=stream)

    def readback():
        c.host_out[:B].copy_(c.n_acc, non_blocking=True)
        c.host_out[B:].copy_(c.nxt, non_blocking=True)
        stream.synchronize()  # the step ends with n_accepted / next_token on the host

    c.layer_calls, c.accept_call, c.readback = layer_calls, accept_call, readback
    return c


def prefill_chunk_keys(L, c, stream):
    """Chunk-mean keys of every layer over the whole cache (a prefill cost,
    timed on its own); returns milliseconds."""
    import torch
    import hierarchical_speculative_attention_amd as tf
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for x in L:
        tf.build_chunk_keys(x.K, x.kv, c.cs, x.ck, x.ckd, stream=stream)
    e1.record(stream)
    stream.synchronize()
    return e0.elapsed_time(e1)


KINDS = ["chunk_refresh", "score", "topk", "sparse", "stream", "verify", "accept"]
BOUND = {"chunk_refresh": "latency", "score": "hbm", "topk": "latency", "sparse": "hbm", "stream": "latency",
         "verify": "hbm", "accept": "latency"}


def time_kinds(L, c, names, stream):
    """One HIP graph per kernel kind with one launch per layer (the layers
    cycled to at least MIN_LAUNCHES launches; SMALL_REPS calls for the accept),
    WARM_REPLAYS untimed replays, then KERNEL_REPS replays between HIP events
    on the launch stream.  Returns (mean us per call, {median, p10, p90})."""
    import torch
    us, dist = {}, {}
    cyc = -(-MIN_LAUNCHES // len(L))  # a graph of fewer launches would be timed with its launch overhead
    Lc = L * cyc
    with torch.cuda.stream(stream):
        for n in names:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                if n == "accept":
                    for _ in range(SMALL_REPS):
                        c.accept_call()
                else:
                    for x in Lc:
                        dict(c.layer_calls(x))[n]()
            for _ in range(WARM_REPLAYS):
                g.replay()
            stream.synchronize()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(KERNEL_REPS + 1)]
            evs[0].record(stream)
            for r in range(KERNEL_REPS):
                g.replay()
                evs[r + 1].record(stream)
            stream.synchronize()
            per = np.array([evs[r].elapsed_time(evs[r + 1]) * 1e3 for r in range(KERNEL_REPS)])
            per /= SMALL_REPS if n == "accept" else len(Lc)    # us per call, one value per replay
            us[n] = float(per.mean())
            dist[n] = {"median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
                       "p90": float(np.percentile(per, 90))}
    return us, dist, cyc


def algorithmic_bytes(c, ckb):
    """Bytes each call must move (no re-read, no avoided work counted)."""
    kvb = 2  # bytes per stored K/V element
    d, Hq, Hkv, B, k, cs, Q = c.d, c.Hq, c.Hkv, c.B, c.k, c.cs, c.Q
    row = d * kvb
    lens = c.lens
    sel_tokens = sum(min(k * cs, n) for n in lens)
    vis_stream = sum(min(c.S, n) + max(0, n - max(c.S, n - c.Wn)) for n in lens)
    return {
        "chunk_refresh": Hkv * B * c.tail_count * (cs * row + d * ckb),
        "score": Hkv * sum(c.C) * d * ckb + B * Hq * row + B * Hkv * c.c_max * 4,
        "topk": B * Hkv * (sum(c.C) // B if B else 0) * 4 + B * Hkv * k * 4,
        "sparse": Hkv * sel_tokens * 2 * row + B * Hkv * k * 4 + B * Hq * (row + d * 4 + 4),
        "stream": Hkv * vis_stream * 2 * row + B * Hq * (row + d * 4 + 4),
        "verify": Hkv * sum(lens) * 2 * row + B * Hq * Q * (row + d * 4 + 4),
        "accept": B * (2 * c.gamma + 1) * c.vocab * 4,
    }


BENCH_LIB = os.path.join(ROOT, "hierarchical_speculative_attention_amd", "libtfbench.so")
CEILING_GRIDS = (256, 512, 1024)


def read_ceiling(L, stream, what="kv", grids=None):
    """How fast HBM serves a pass's bytes when nothing else is done with them:
    a kernel that only reads them (the measurement aid libtfbench.so, verify's
    access shape), timed like the per-kernel graphs (one launch per layer), for
    a few grid sizes.  what = "kv": each layer's K and V (the verification
    pass); "ck": each layer's chunk keys (the score pass), read as two halves;
    "ring": each layer's streaming ring (K and V), where a grid of one
    workgroup per KV head gives each workgroup one head's rows, as the
    streaming kernel does."""
    import ctypes
    import torch
    if not os.path.exists(BENCH_LIB):
        return None
    lib = ctypes.CDLL(BENCH_LIB)
    lib.tfb_read_kv.restype = ctypes.c_int
    lib.tfb_read_kv.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p]
    cyc = -(-MIN_LAUNCHES // len(L))
    Lc = L * cyc
    grids = grids or CEILING_GRIDS
    if what == "kv":
        nbytes = L[0].K.numel() * L[0].K.element_size()
        pairs = [(x.K.data_ptr(), x.V.data_ptr()) for x in Lc]
    elif what == "ring":
        nbytes = L[0].Ks.numel() * L[0].Ks.element_size()
        pairs = [(x.Ks.data_ptr(), x.Vs.data_ptr()) for x in Lc]
    else:
        nbytes = L[0].ck.numel() * L[0].ck.element_size() // 2 // 16 * 16
        pairs = [(x.ck.data_ptr(), x.ck.data_ptr() + nbytes) for x in Lc]
    sink = torch.empty(max(grids) * 4, dtype=torch.int32, device=L[0].K.device)
    out, us = {}, {}
    with torch.cuda.stream(stream):
        for grid in grids:
            def launches():
                for k_ptr, v_ptr in pairs:
                    st = lib.tfb_read_kv(ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), nbytes, grid,
                                         ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
                    if st != 0:
                        raise RuntimeError(f"tfb_read_kv: hip error {st}")
            r = time_graph(launches, stream, len(Lc))
            us[grid] = r["us"]
            out[grid] = 2 * nbytes / (r["us"] * 1e-6) / 1e9
    best = max(out, key=out.get)
    return {"GB_s": round(out[best], 1), "us": us[best], "grid": best, "bytes_per_launch": 2 * nbytes,
            "GB_s_by_grid": {str(g): round(v, 1) for g, v in out.items()},
            "us_by_grid": {str(g): v for g, v in us.items()},
            "what": ("a kernel that only reads each layer's " +
                     {"kv": "K and V", "ck": "chunk keys", "ring": "streaming ring (K and V)"}[what] +
                     " (verify's access shape: 1 KB per wave instruction, nontemporal 16-byte loads, 4 per tensor "
                     "in flight per lane), one launch per layer in a HIP graph; the best grid")}


GATHER_TPW = (128, 256, 512)


def gather_ceiling(L, c, stream, sparse_bytes):
    """How fast one launch can gather the sparse pass's bytes: a kernel that
    only reads the K and V rows of the selected chunks (the measurement aid
    libtfbench.so: chunk indices first, two 32-row tiles per wave in flight, 1
    KB per wave instruction; no attention, no split merge), on the sparse
    call's buffers and indices, timed like the per-kernel graphs (one launch
    per layer), for a few workgroup sizes.  GB/s are over the sparse call's
    algorithmic bytes, so they compare with its figure directly."""
    import ctypes
    import torch
    if not os.path.exists(BENCH_LIB) or c.cs % 4 != 0:
        return None
    lib = ctypes.CDLL(BENCH_LIB)
    if not hasattr(lib, "tfb_gather_kv"):
        return None
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.tfb_gather_kv.restype = i32
    lib.tfb_gather_kv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    cyc = -(-MIN_LAUNCHES // len(L))
    Lc = L * cyc
    splits = -(-(c.k * c.cs) // min(GATHER_TPW))
    sink = torch.empty(splits * c.Hkv * c.B * 4, dtype=torch.int32, device=L[0].K.device)
    out = {}
    with torch.cuda.stream(stream):
        for tpw in GATHER_TPW:
            def launches():
                for x in Lc:
                    st = lib.tfb_gather_kv(vp(x.K.data_ptr()), vp(x.V.data_ptr()), vp(x.kv.seq_base.data_ptr()),
                                           vp(x.kv.seq_cap.data_ptr()), vp(x.kv.seq_len.data_ptr()),
                                           vp(c.idx.data_ptr()), c.B, c.Hkv, c.k, c.cs, tpw, vp(sink.data_ptr()),
                                           vp(stream.cuda_stream))
                    if st != 0:
                        raise RuntimeError(f"tfb_gather_kv: hip error {st}")
            out[tpw] = time_graph(launches, stream, len(Lc))
    best = min(out, key=lambda t: out[t]["us"])
    return {"us": out[best]["us"], "tpw": best,
            "GB_s": round(sparse_bytes / (out[best]["us"] * 1e-6) / 1e9, 1),
            "frac": round(sparse_bytes / (out[best]["us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "us_by_tpw": {str(t): v["us"] for t, v in out.items()},
            "what": "a kernel that only gathers the selected chunks' K and V rows (chunk indices read first, two "
                    "32-row tiles per wave in flight, 1 KB per wave instruction), one launch per layer in a HIP "
                    "graph, on the sparse call's buffers and indices; the best workgroup size; GB/s over the "
                    "sparse call's algorithmic bytes"}


def kernel_table(us, dist, by, names):
    out = {}
    for n in names:
        gbs = by[n] / (us[n] * 1e-6) / 1e9
        out[n] = {"us": round(us[n], 2), "us_median": round(dist[n]["median"], 2),
                  "us_p10": round(dist[n]["p10"], 2), "us_p90": round(dist[n]["p90"], 2),
                  "GB_s": round(gbs, 1), "bytes": int(by[n]), "bound": BOUND[n]}
        if BOUND[n] == "hbm":
            out[n]["frac"] = round(gbs / HBM_PEAK_GBPS, 4)
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path is not sharded "
                                   "across GPUs (it would shard by KV head: every call is independent "
                                   "per sequence and KV head)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from hierarchical_speculative_attention_amd import synth

    W = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)  # default priority
    B, Hq, Hkv, d = W["B"], W["Hq"], W["Hkv"], W["d"]
    lens = W["lens"]
    layers = args.layers or W["layers"]
    cs, budget, gamma, vocab = W["chunk_size"], W["budget"], W["gamma"], W["vocab"]
    if args.budget is not None:
        budget = args.budget
    if args.gamma is not None:
        gamma = args.gamma
    if budget < cs or gamma < 0:
        raise SystemExit(f"budget {budget} must be at least one chunk ({cs}) and gamma >= 0")
    S, Wn = W["n_sink"], W["window"]
    Q = gamma + 1
    k = budget // cs
    tdt = torch.bfloat16 if W["dtype"] == "bf16" else torch.float16
    ck_dt = torch.float32 if args.ck_dtype == "fp32" else tdt
    n_max = max(lens)
    C = [-(-n // cs) for n in lens]
    t_setup = time.perf_counter()

    # ---- inputs, resident in HBM ------------------------------------------
    L = build_layers(W, layers, Q, ck_dt, tdt, dev, stream)
    c = step_context(W, budget, gamma, ck_dt, tdt, dev, stream)
    layer_calls, accept_call, readback = c.layer_calls, c.accept_call, c.readback

    # ---- prefill: chunk-mean keys of every layer (timed on its own) --------
    prefill_ms = prefill_chunk_keys(L, c, stream)
    tokens_total = sum(lens)
    prefill_bytes = layers * Hkv * (tokens_total * d * 2 + sum(C) * d * L[0].ck.element_size())

    # ---- one decode step ----------------------------------------------------
    def step_gpu(verify_events=None):
        for x in L:
            for name, fn in layer_calls(x):
                if name == "verify" and verify_events is not None:
                    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a_.record(stream)
                    fn()
                    b_.record(stream)
                    verify_events.append((a_, b_))
                else:
                    fn()
        accept_call()

    with torch.cuda.stream(stream):
        # eager warm-up, then the step captured once as a HIP graph
        for _ in range(args.warmup):
            step_gpu()
            readback()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step_gpu()
        for _ in range(args.warmup):
            graph.replay()
            readback()
        torch.cuda.synchronize()
        # timed region 1: graph replays (the reported value)
        t0 = time.perf_counter()
        step_t = []
        for _ in range(args.steps):
            ts = time.perf_counter()
            graph.replay()
            readback()
            step_t.append(time.perf_counter() - ts)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        # timed region 2: the same steps launched eagerly, HIP events around
        # every verify launch on the launch stream (roofline of that kernel)
        vev = []
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step_gpu(vev)
            readback()
        torch.cuda.synchronize()
        elapsed_eager = time.perf_counter() - t0
    verify_eager_avg_s = float(np.mean([a_.elapsed_time(b_) for a_, b_ in vev])) / 1e3
    del graph

    # ---- per-kernel breakdown: one graph per kernel kind, one launch per layer
    names = KINDS
    us, dist, cyc = time_kinds(L, c, names, stream)
    with torch.cuda.stream(stream):
        # secondary peak: a 1 GiB device-to-device copy (1 GiB read + 1 GiB written)
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(COPY_REPS):
            dst.copy_(src)
        c1.record(stream)
        stream.synchronize()
        copy_gbps = 2 * src.numel() * src.element_size() * COPY_REPS / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del src, dst
    verify_avg_s = us["verify"] * 1e-6
    ceiling = read_ceiling(L, stream)

    # ---- algorithmic bytes --------------------------------------------------
    by = algorithmic_bytes(c, L[0].ck.element_size())
    kernels = kernel_table(us, dist, by, names)
    # few long rows are selected in slices, then merged (two launches)
    kernels["topk"]["launches"] = 2 if c.ws_t is not None else 1
    step_bytes = layers * sum(by[n] for n in names if n != "accept") + by["accept"]
    verify_bytes = by["verify"]
    achieved = verify_bytes / verify_avg_s / 1e9
    default_shape = args.workload == DEFAULT_WORKLOAD and gamma == W["gamma"] and budget == W["budget"]
    # (the counters and the kernel trace are of the verify launch at the default workload's shape)
    traffic = read_traffic() if default_shape else None
    trace = read_kernel_trace(verify_bytes, by["sparse"]) if default_shape else None
    ck_ceiling = read_ceiling(L, stream, "ck")
    if ck_ceiling:
        # the score pass against a plain read of the chunk keys it streams
        kernels["score"]["read_ceiling"] = ck_ceiling
        kernels["score"]["frac_of_read_ceiling"] = round(ck_ceiling["us"] / kernels["score"]["us"], 4)
    ring_ceiling = read_ceiling(L, stream, "ring", grids=(Hkv * B, 4 * Hkv * B, 16 * Hkv * B))
    if ring_ceiling:
        # streaming attention against a plain read of its ring: with one
        # workgroup per KV head (its own grid) and spread over 4 and 16
        kernels["stream"]["read_ceiling"] = ring_ceiling
        kernels["stream"]["frac_of_one_workgroup_per_head_read"] = round(
            ring_ceiling["us_by_grid"][str(Hkv * B)] / kernels["stream"]["us"], 4)
    gather = gather_ceiling(L, c, stream, by["sparse"])
    if gather:
        # the sparse call against a bare gather of its bytes in one launch
        kernels["sparse"]["gather_ceiling"] = gather
        kernels["sparse"]["frac_of_gather_ceiling"] = round(gather["us"] / kernels["sparse"]["us"], 4)
    if trace and "sparse" in trace:
        # the sparse pass: the call level above (gather kernel + split merge, timed
        # together), each kernel's own traced duration here
        kernels["sparse"]["kernel_trace"] = trace.pop("sparse")
    ms_per_step = elapsed / args.steps * 1e3

    result = {
        "metric": METRIC,
        "value": round(args.steps / elapsed, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "step_ms": {"median": round(float(np.median(step_t)) * 1e3, 3),
                    "p10": round(float(np.percentile(step_t, 10)) * 1e3, 3),
                    "p90": round(float(np.percentile(step_t, 90)) * 1e3, 3)},
        "launch": "HIP graph of the whole step, replayed; n_accepted/next_token read back each step",
        "eager_steps_per_s": round(args.steps / elapsed_eager, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "context": lens if B > 1 else lens[0], "layers": layers, "chunk_size": cs, "budget": budget,
                   "gamma": gamma, "verify_queries": Q, "n_sink": S, "window": Wn, "vocab": vocab,
                   "chunk_key_dtype": str(ck_dt).replace("torch.", ""), "parallelism": "single GPU"},
        "decode_attn_GB_s": round(step_bytes * args.steps / elapsed / 1e9, 1),
        "decode_attn_hbm_frac": round(step_bytes * args.steps / elapsed / 1e9 / HBM_PEAK_GBPS, 4),
        "step_algorithmic_bytes": int(step_bytes),
        "kernels_note": (None if cyc == 1 else
                         f"{layers} layer(s): each per-kernel graph cycles them {cyc} times; inputs under ~256 MB "
                         "are then partly read from the Infinity Cache"),
        "roofline": {"kernel": "verify_attn (attn_kernel + combine_kernel, verify mode)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "frac_basis": "call level: one tf_verify_attn call = the attention kernel, then the split "
                                   "merge kernel, timed together (see avg_launch_us); kernel_trace gives each "
                                   "kernel's own rocprofv3 duration",
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(verify_bytes),
                     "avg_launch_us": round(verify_avg_s * 1e6, 2),
                     "timing": f"HIP events on the launch stream around each of {KERNEL_REPS} replays of a graph "
                               "of the step's verify launches (one per layer, back to back); mean over replays",
                     "eager_avg_launch_us": round(verify_eager_avg_s * 1e6, 2),
                     "kernel_trace": trace,
                     "read_ceiling": ceiling,
                     "frac_of_read_ceiling": (round(achieved / ceiling["GB_s"], 4) if ceiling else None),
                     "copy_GB_s": round(copy_gbps, 1),
                     "frac_of_copy": round(achieved / copy_gbps, 4)},
        "kernels": kernels,
        "kernels_timing": f"per kind: a HIP graph of its launches for every layer ({SMALL_REPS} calls for the "
                          f"accept), {WARM_REPLAYS} warm replays, "
                          f"then {KERNEL_REPS} replays each between HIP events; us = mean per launch, "
                          "median / p10 / p90 over the replays",
        "sparse_draft_pass_us": round(us["score"] + us["topk"] + us["sparse"], 2),
        "prefill_chunk_keys": {"ms_all_layers": round(prefill_ms, 3),
                               "GB_s": round(prefill_bytes / (prefill_ms * 1e-3) / 1e9, 1)},
        "setup_s": round(time.perf_counter() - t_setup, 1),
    }
    idx, acc_in = c.idx, c.acc_in
    if not args.no_next_rows:
        result["next_rows"] = next_rows_leg(L, lens, Hq, Hkv, d, cs, k, S, Wn, gamma, idx, acc_in, dev, stream)
        result["next_rows_timing"] = (f"per call: a HIP graph of one call per layer ({SMALL_REPS} in all for the "
                                      f"tree accept), {WARM_REPLAYS} warm replays, then {KERNEL_REPS} replays "
                                      "each between HIP events; us per call")
    if not args.no_three_tier and B == 1:
        result["three_tier"] = three_tier_leg(L, lens, Hq, Hkv, d, cs, k, S, Wn, gamma, vocab, tdt, ck_dt, dev,
                                              args.steps, args.warmup, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(L[:max(1, min(args.cpu_layers, layers))], lens, Hq, Hkv, d, cs, k, S,
                                              Wn, Q, layers, acc_in, tdt)
        if not args.no_next_rows and B == 1:
            # the same oracle, on the calls the three-tier loop adds (reported beside next_rows)
            result["cpu_baseline"]["next_rows"] = next_rows_cpu_baseline(L[0], lens[0], Hq, Hkv, d, cs, idx, gamma,
                                                                         acc_in, tdt)
        result["cpu_baseline"]["small_layer"] = cpu_baseline_small()
    if not args.no_other_workloads and args.workload == DEFAULT_WORKLOAD:
        # the step's layers leave the GPU before the other workloads are generated
        del L, c, idx
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        others = {}
        for name, b_, g_, cpu in OTHER_WORKLOADS:
            others[f"{name}/budget{b_}/gamma{g_}"] = other_workload(name, b_, g_, args.steps, args.warmup, ck_dt,
                                                                    dev, stream, cpu and not args.no_cpu_baseline)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        result["other_workloads"] = others
        result["other_workloads_timing"] = ("the same per-kernel graphs as kernels (layers cycled to at least "
                                            f"{MIN_LAUNCHES} launches), and for the multi-layer workload the whole "
                                            "step replayed as a HIP graph (steps_per_s)")
    print(json.dumps(result), flush=True)


# The other workloads measured beside the default one: (name, budget, gamma).
OTHER_WORKLOADS = [("gqa-hq32-hkv8-512k-16layers", 8192, 8, True), ("ragged-b8-16k-128k", 4096, 6, True),
                   ("ragged-b8-16k-128k", 2048, 4, False)]   # (name, budget, gamma, time the oracle too)


def other_workload(name, budget, gamma, steps, warmup, ck_dt, dev, stream, cpu=False):
    """Per-kernel figures of another workload at its own shape (and, with
    several layers, the step rate): the same calls and timing as the default
    workload's kernels."""
    import torch
    from hierarchical_speculative_attention_amd import synth
    W = synth.WORKLOADS[name]
    tdt = torch.bfloat16 if W["dtype"] == "bf16" else torch.float16
    layers = W["layers"]
    L = build_layers(W, layers, gamma + 1, ck_dt, tdt, dev, stream)
    c = step_context(W, budget, gamma, ck_dt, tdt, dev, stream)
    prefill_chunk_keys(L, c, stream)
    out = {"batch": W["B"], "q_heads": W["Hq"], "kv_heads": W["Hkv"], "context": W["lens"] if W["B"] > 1 else
           W["lens"][0], "layers": layers, "chunk_size": c.cs, "budget": budget, "gamma": gamma,
           "verify_queries": c.Q, "kv_gib_per_layer": round(c.Hkv * sum(W["lens"]) * c.d * 2 * 2 / 2 ** 30, 2)}
    if layers > 1:
        with torch.cuda.stream(stream):
            def step_gpu():
                for x in L:
                    for _, fn in c.layer_calls(x):
                        fn()
                c.accept_call()
            step_gpu()
            c.readback()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                step_gpu()
            for _ in range(warmup):
                graph.replay()
                c.readback()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                graph.replay()
                c.readback()
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            del graph
        out["steps_per_s"] = round(steps / el, 3)
        out["ms_per_step"] = round(el / steps * 1e3, 3)
    names = KINDS
    us, dist, cyc = time_kinds(L, c, names, stream)
    by = algorithmic_bytes(c, L[0].ck.element_size())
    out["kernels"] = kernel_table(us, dist, by, names)
    out["kernels"]["topk"]["launches"] = 2 if c.ws_t is not None else 1
    out["sparse_draft_pass_us"] = round(us["score"] + us["topk"] + us["sparse"], 2)
    if cyc > 1:
        out["kernels_note"] = (f"{layers} layer(s) cycled {cyc} times per graph; every call here moves more than "
                               "the ~256 MB Infinity Cache except the latency-bound ones")
    if cpu:
        out["cpu_baseline"] = cpu_baseline(L[:1], W["lens"], c.Hq, c.Hkv, c.d, c.cs, c.k, c.S, c.Wn, c.Q, layers,
                                           c.acc_in, tdt)
    del L, c
    return out


def time_graph(fn, stream, per_replay):
    """Mean / median / p10 / p90 microseconds per call of fn (a function that
    enqueues per_replay calls), captured once as a HIP graph and replayed
    between HIP events on the launch stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    for _ in range(WARM_REPLAYS):
        g.replay()
    stream.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(KERNEL_REPS + 1)]
    evs[0].record(stream)
    for r in range(KERNEL_REPS):
        g.replay()
        evs[r + 1].record(stream)
    stream.synchronize()
    per = np.array([evs[r].elapsed_time(evs[r + 1]) * 1e3 for r in range(KERNEL_REPS)]) / per_replay
    return {"us": round(float(per.mean()), 2), "us_median": round(float(np.median(per)), 2),
            "us_p10": round(float(np.percentile(per, 10)), 2), "us_p90": round(float(np.percentile(per, 90)), 2)}


def next_rows_leg(L, lens, Hq, Hkv, d, cs, k, S, Wn, gamma, idx, acc, dev, stream):
    """The calls the three-tier loop adds, each timed on its own over every
    layer (graph of one launch per layer, the layers cycled to at least 8
    launches, like the step's kernels):
    sparse verification of gamma1 + 1 = 3 rows over the selected chunks below
    a 64-row causal tail (Force 2 verifying the drafter), verification over a
    7-node candidate tree, accept over that tree (V = 32000), appending
    gamma + 1 rows to the full cache and one row to the streaming ring, the
    length commit and the tree masks."""
    import torch
    import hierarchical_speculative_attention_amd as tf
    B = len(lens)
    cyc = -(-MIN_LAUNCHES // len(L))
    Lc = L * cyc
    layers = len(Lc)   # launches per graph
    row = d * 2
    g1, tail = 2, 64
    Qt = gamma + 1
    out = {}
    with torch.cuda.stream(stream):
        # sparse verification (the selection of the step's last layer serves every layer)
        q3 = [x.qv[:, :, :g1 + 1].contiguous() for x in Lc]
        ws = tf.workspace(tf.sparse_verify_attn_workspace_size(B, Hq, Hkv, g1 + 1, k, cs, tail), dev)
        o3 = torch.empty((B, Hq, g1 + 1, d), dtype=torch.float32, device=dev)
        l3 = torch.empty((B, Hq, g1 + 1), dtype=torch.float32, device=dev)
        r = time_graph(lambda: [tf.sparse_verify_attn(q, x.K, x.V, x.kv, idx, cs, tail, out=o3, lse=l3, ws=ws,
                                                      stream=stream) for q, x in zip(q3, Lc)], stream, layers)
        sel = idx.cpu().numpy()
        rows = 0
        for b, n in enumerate(lens):
            lo = max(0, n - tail)
            for g in range(Hkv):
                for c in sel[b, g]:
                    if c >= 0:
                        rows += max(0, min(lo, (int(c) + 1) * cs) - int(c) * cs)
                rows += n - lo
        by = rows * 2 * row + B * Hkv * k * 4 + B * Hq * (g1 + 1) * (row + d * 4 + 4)
        out["sparse_verify"] = dict(r, bytes=int(by), GB_s=round(by / (r["us"] * 1e-6) / 1e9, 1), bound="hbm",
                                    shape=f"{g1 + 1} rows x {Hq} heads over {k} chunks x {cs} + a {tail}-row tail")
        # verification over a candidate tree
        parent = torch.tensor([[-1, 0, 0, 1, 1, 2, 2][:Qt] + [-1] * max(0, Qt - 7)] * B, dtype=torch.int32,
                              device=dev)
        tm = tf.tree_masks(parent, stream=stream)
        ws_v = tf.workspace(tf.verify_attn_workspace_size(B, Hq, Hkv, Qt, max(lens)), dev)
        ov = torch.empty((B, Hq, Qt, d), dtype=torch.float32, device=dev)
        lv = torch.empty((B, Hq, Qt), dtype=torch.float32, device=dev)
        r = time_graph(lambda: [tf.verify_tree_attn(x.qv, x.K, x.V, x.kv, tm, out=ov, lse=lv, ws=ws_v,
                                                    stream=stream) for x in Lc], stream, layers)
        by = Hkv * sum(lens) * 2 * row + B * Hq * Qt * (row + d * 4 + 4) + B * Qt * 8
        out["verify_tree"] = dict(r, bytes=int(by), GB_s=round(by / (r["us"] * 1e-6) / 1e9, 1), bound="hbm",
                                  shape=f"{Qt}-node tree (parents {parent[0].tolist()}) x {Hq} heads over the full cache")
        # accept over the tree
        tgt = torch.from_numpy(acc.target).to(dev)
        drf = torch.from_numpy(acc.draft).to(dev)
        V = tgt.shape[-1]
        drf_t = torch.cat([drf, drf[:, :1]], 1)[:, :Qt].contiguous()
        tok = torch.from_numpy(acc.tokens).to(dev)
        tok_t = torch.cat([tok, tok[:, :1]], 1)[:, :Qt].contiguous()
        uni = torch.from_numpy(acc.uniforms).to(dev)[:, :Qt].contiguous()
        ws_t = tf.workspace(tf.tree_accept_workspace_size(B, V), dev)
        r = time_graph(lambda: [tf.tree_accept(tgt, drf_t, tok_t, parent, uni, 1.0, ws=ws_t, stream=stream)
                                for _ in range(SMALL_REPS)], stream, SMALL_REPS)
        by = B * 2 * Qt * V * 4
        out["tree_accept"] = dict(r, bytes=int(by), GB_s=round(by / (r["us"] * 1e-6) / 1e9, 1), bound="latency",
                                  shape=f"{Qt}-node tree, vocabulary {V}, fp64 inside")
        # cache maintenance: rows written past the committed lengths, which stay unchanged
        g = torch.Generator(device=dev).manual_seed(11)
        kn = torch.randn((B, Hkv, Qt, d), generator=g, device=dev).to(L[0].K.dtype)
        vn = torch.randn((B, Hkv, Qt, d), generator=g, device=dev).to(L[0].K.dtype)
        st = torch.empty(B, dtype=torch.int32, device=dev)
        r = time_graph(lambda: [tf.append_kv(kn, vn, x.K, x.V, x.kv, status=st, stream=stream) for x in Lc], stream,
                       layers)
        by = 2 * 2 * B * Hkv * Qt * row
        out["append_full"] = dict(r, bytes=int(by), GB_s=round(by / (r["us"] * 1e-6) / 1e9, 1), bound="latency",
                                  shape=f"{Qt} rows x {Hkv} heads into the full cache")
        k1, v1 = kn[:, :, :1].contiguous(), vn[:, :, :1].contiguous()
        r = time_graph(lambda: [tf.append_kv(k1, v1, x.Ks, x.Vs, x.sd, ring=True, n_sink=S, window=Wn, reserve=1,
                                             status=st, stream=stream) for x in Lc], stream, layers)
        by = 2 * 2 * B * Hkv * row
        out["append_ring"] = dict(r, bytes=int(by), GB_s=round(by / (r["us"] * 1e-6) / 1e9, 1), bound="latency",
                                  shape=f"1 row x {Hkv} heads into the {S} + {Wn} ring")
        ok = bool((st == 0).all().item())
        lens_t = torch.tensor(lens, dtype=torch.int32, device=dev)
        na = torch.zeros(B, dtype=torch.int32, device=dev)
        r = time_graph(lambda: [tf.commit_length(lens_t, 0, 0, na, stream=stream) for _ in range(layers)], stream,
                       layers)
        out["commit_length"] = dict(r, bound="latency", shape=f"{B} sequence length(s)")
        r = time_graph(lambda: [tf.tree_masks(parent, stream=stream) for _ in range(layers)], stream, layers)
        out["tree_masks"] = dict(r, bound="latency", shape=f"{B} tree(s) of {Qt} nodes")
    if not ok:
        raise RuntimeError("append_kv reported a status other than TF_APPEND_OK")
    for v in out.values():
        if v.get("bound") == "hbm":
            v["frac"] = round(v["GB_s"] / HBM_PEAK_GBPS, 4)
    return out


def three_tier_leg(L, lens, Hq, Hkv, d, cs, k, S, Wn, gamma, vocab, tdt, ck_dt, dev, steps, warmup, stream):
    """The three tiers in a loop on the same target caches: a 2-layer drafter
    (the target's head shape) on a sink + window ring drafts gamma1 = 2 tokens
    per Force 2 round, Force 2 rounds on the retrieval cache (tail 64) run
    until gamma2 = gamma candidates exist, Force 3 verifies them on the full
    cache (hierarchical_speculative_attention_amd.three_tier).  Timed twice
    from the same starting state: with the fixed call sequences replayed as
    HIP graphs (the reported rate) and with eager launches; either way the
    host reads back 4 bytes per round and per step (it decides the rounds).
    Logits are synthetic: p ~ N(0, 2); q = p + N(0, 0.5); r = q + N(0, 0.5)."""
    import torch
    import hierarchical_speculative_attention_amd as tf
    from hierarchical_speculative_attention_amd import synth
    from hierarchical_speculative_attention_amd import three_tier as tt
    n0 = lens[0]
    g1, g2 = 2, gamma
    C_cap = -(-(n0 + EXTRA_ROWS) // cs)

    def run(graphs):
        g = torch.Generator(device=dev).manual_seed(synth.torch_seed(0, 0, "extra"))
        rnd = lambda *shape: torch.randn(*shape, generator=g, device=dev).to(tdt)
        with torch.cuda.stream(stream):
            seq_len = torch.tensor([n0], dtype=torch.int32, device=dev)
            ck_len = torch.tensor([-(-n0 // cs)], dtype=torch.int32, device=dev)
            target = []
            for x in L:
                kv = tf.KVDesc(1, Hkv, tdt, x.kv.seq_base, x.kv.seq_cap, seq_len, n0 + EXTRA_ROWS, dev)
                ckl = synth.KVLayout.build([C_cap], Hkv, d, caps=[C_cap])
                ckd = tf.KVDesc(1, Hkv, ck_dt, ckl.seq_base, ckl.seq_cap, ck_len, C_cap, dev)
                ck = torch.empty(ckl.total_elems, dtype=ck_dt, device=dev)
                tf.build_chunk_keys(x.K, kv, cs, ck, ckd, stream=stream)
                target.append(tt.TargetLayer(x.K, x.V, kv, ck, ckd))
            cap = S + Wn + tt.drafter_reserve(g1, g2)
            d_len = torch.tensor([n0], dtype=torch.int32, device=dev)
            drafter = []
            for _ in range(2):
                lay = synth.KVLayout.build([n0], Hkv, d, caps=[cap])
                sd = tf.KVDesc(1, Hkv, tdt, lay.seq_base, lay.seq_cap, d_len, n0, dev)
                drafter.append(tt.DrafterLayer(rnd(lay.total_elems), rnd(lay.total_elems), sd))
            P = torch.randn((1, g2 + 1, vocab), generator=g, device=dev) * 2
            Qr = (P[:, :g1 + 1] + torch.randn((1, g1 + 1, vocab), generator=g, device=dev) * 0.5).contiguous()
            R = (Qr[:, :g1] + torch.randn((1, g1, vocab), generator=g, device=dev) * 0.5).contiguous()
            rng = np.random.default_rng(7)
            syn = tt.Synthetic(draft_q=L[0].qd, draft_rows=[rnd(1, Hkv, r, d) for r in (1, 2, 3)], r_rows=R,
                               f2_q=rnd(1, Hq, g1 + 1, d), f2_rows=rnd(1, Hkv, g1 + 1, d), q_rows=Qr, f3_q=L[0].qv,
                               one_row=rnd(1, Hkv, 1, d), p_rows=P.contiguous(),
                               uniforms=torch.from_numpy(synth.open_uniforms(rng, 1 << 20)).to(dev))
            step = tt.ThreeTierStep(target, drafter, syn, Hq=Hq, chunk_size=cs, k=k, tail=64, gamma1=g1,
                                    gamma2=g2, n_sink=S, window=Wn, stream=stream, graphs=graphs)
            for _ in range(warmup):
                step.step()
            stream.synchronize()
            s0, r0, e0 = step.steps, step.rounds, step.emitted
            t0 = time.perf_counter()
            for _ in range(steps):
                step.step()
            stream.synchronize()
            el = time.perf_counter() - t0
        n_steps, n_rounds, n_tok = step.steps - s0, step.rounds - r0, step.emitted - e0
        return {"steps_per_s": round(n_steps / el, 3), "tokens_per_s": round(n_tok / el, 2),
                "ms_per_step": round(el / n_steps * 1e3, 3), "rounds_per_step": round(n_rounds / n_steps, 3),
                "tokens_per_step": round(n_tok / n_steps, 3), "steps": n_steps}

    res = run(True)
    eager = run(False)
    res.update({"gamma1": g1, "gamma2": g2,
                "drafter": f"2 layers x {Hkv} heads x {d}, ring {S} sinks + {Wn} window",
                "force2": f"sparse verification of gamma1 + 1 rows over {k} chunks x {cs} rows + a 64-row causal tail",
                "launch": "HIP graphs for the retrieval, each round and Force 3; the host reads back 4 bytes per "
                          "Force 2 round and per step",
                "eager": {kk: eager[kk] for kk in ("steps_per_s", "ms_per_step", "rounds_per_step")},
                "logits": "synthetic: p ~ N(0,2), q = p + N(0,0.5), r = q + N(0,0.5)"})
    return res


def next_rows_cpu_baseline(x, n, Hq, Hkv, d, cs, idx, gamma, acc, tdt):
    """The fp64 oracle's versions of the NEXT-row calls, timed on this host on
    a bounded sample and scaled to one call: sparse verification on 4 of the
    KV heads, tree verification on 2 (its row lists are built in Python),
    one tree accept.  Widening the cache to fp64 is not timed."""
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    to_bits = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    dt = "bf16" if tdt == torch.bfloat16 else "fp16"
    G = Hq // Hkv
    Kb, Vb, qv = to_bits(x.K), to_bits(x.V), to_bits(x.qv)
    base, cap = int(x.kv.seq_base[0].item()), int(x.kv.seq_cap[0].item())
    sel = idx.cpu().numpy()
    parent = [-1, 0, 0, 1, 1, 2, 2][:gamma + 1] + [-1] * max(0, gamma + 1 - 7)
    masks = oracle.tree_masks(parent)
    out = {}
    for name, heads in (("sparse_verify", 4), ("verify_tree", 2)):
        t = 0.0
        for g in range(heads):
            off = base + g * cap * d
            K = oracle.widen(Kb[off:off + n * d].reshape(n, d), dt)
            V = oracle.widen(Vb[off:off + n * d].reshape(n, d), dt)
            for j in range(G):
                qs = oracle.widen(qv[0, g * G + j], dt)
                t0 = time.perf_counter()
                if name == "sparse_verify":
                    oracle.sparse_verify_attn(qs[:3], K, V, n, sel[0, g].tolist(), cs, 64)
                else:
                    oracle.verify_tree_attn(qs, K, V, n, masks)
                t += time.perf_counter() - t0
        out[name] = {"us": round(t / heads * Hkv * 1e6, 1), "sample": f"{heads} of {Hkv} KV heads, scaled"}
    Qt = gamma + 1
    drf = np.concatenate([acc.draft, acc.draft[:, :1]], 1)[0, :Qt]
    tok = np.concatenate([acc.tokens, acc.tokens[:, :1]], 1)[0, :Qt]
    t0 = time.perf_counter()
    oracle.tree_accept(acc.target[0], drf, tok, parent, acc.uniforms[0, :Qt], 1.0)
    out["tree_accept"] = {"us": round((time.perf_counter() - t0) * 1e6, 1), "sample": "one call"}
    return {"calls": out, "kind": "oracle", "cores": int(threads), "unit": "us per call"}


def cpu_baseline_small():
    """The oracle over the whole small single layer (8 heads, n = 4096, fp16,
    chunk 8, budget 512, 4 sinks + 252 window, gamma = 4, vocabulary 32000):
    one step (tail refresh, scores, top-k, sparse, streaming and verify
    attention for every head, then one accept) on all cores and on one
    thread.  Inputs come from the same seeded generators, on the host."""
    import oracle
    from hierarchical_speculative_attention_amd import synth
    W = synth.WORKLOADS["tiny-h8-n4k-fp16"]
    n, H, cs, dt = W["lens"][0], W["Hq"], W["chunk_size"], W["dtype"]
    k, Q, S, Wn = W["budget"] // cs, W["gamma"] + 1, W["n_sink"], W["window"]
    inp = synth.make_attn_inputs(lens=[n], Hq=H, Hkv=H, dtype=dt, Q=Q, seed=0, chunk_size=cs,
                                 plant=W["plant"], plant_count=W["plant_count"])
    st = synth.make_stream_inputs(lens=[n], Hq=H, Hkv=H, dtype=dt, n_sink=S, window=Wn, seed=0)
    acc = synth.make_accept_inputs(B=1, gamma=W["gamma"], vocab=W["vocab"], seed=0)
    lay = inp.layout
    heads = []
    for g in range(H):
        K = oracle.widen(lay.head(inp.K, 0, g), dt)
        V = oracle.widen(lay.head(inp.V, 0, g), dt)
        heads.append((K, V, oracle.chunk_keys(K, n, cs),     # prefill: not timed
                      oracle.widen(inp.q_draft[0, g, 0], dt), oracle.widen(inp.q_verify[0, g], dt),
                      oracle.widen(st.K_logical[0][g], dt), oracle.widen(st.V_logical[0][g], dt),
                      oracle.widen(st.q[0, g, 0], dt)))

    def step():
        t0 = time.perf_counter()
        for K, V, ck, qd, qv, Kl, Vl, qs in heads:
            c0 = max(0, (n - Q) // cs)
            ck[c0:] = oracle.chunk_keys(K[c0 * cs:n], n - c0 * cs, cs)
            sel = oracle.select_topk(oracle.chunk_scores(qd[None], ck), k)
            oracle.sparse_attn(qd, K, V, n, sel, cs)
            oracle.stream_attn_masked(qs, Kl, Vl, n, S, Wn)
            oracle.verify_attn(qv, K, V, n)
        oracle.accept(acc.target[0], acc.draft[0], acc.tokens[0], acc.uniforms[0], 1.0)
        return time.perf_counter() - t0

    out = {"workload": "tiny-h8-n4k-fp16 (8 heads, n 4096, fp16, budget 512, gamma 4)", "unit": "steps/s",
           "kind": "oracle", "sample": "the whole step, every head"}
    t = min(step() for _ in range(3))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        out["all_cores"] = {"value": round(1.0 / t, 3), "cores": int(threads), "s_per_step": round(t, 4)}
        with threadpool_limits(limits=1):
            t1 = min(step() for _ in range(3))
        out["single_thread"] = {"value": round(1.0 / t1, 3), "cores": 1, "s_per_step": round(t1, 4)}
    except ImportError:
        out["all_cores"] = {"value": round(1.0 / t, 3), "cores": None, "s_per_step": round(t, 4)}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(sample_layers, lens, Hq, Hkv, d, cs, k, S, Wn, Q, layers, acc_in, tdt):
    """The fp64 oracle timed on this host over a bounded sample of the step:
    the given layers (every head of every sequence) plus one accept, scaled to
    the whole step.  Chunk-key construction over the cache is a prefill cost
    and stays outside the timed region, as on the GPU."""
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    to_bits = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    dt = "bf16" if tdt == torch.bfloat16 else "fp16"
    G = Hq // Hkv

    def heads_of(x, pairs):
        """Oracle time of the step's per-head work for the given (sequence, KV head) pairs of layer x."""
        Kb, Vb = to_bits(x.K), to_bits(x.V)
        qv, qd = to_bits(x.qv), to_bits(x.qd)
        Ksb, Vsb = to_bits(x.Ks), to_bits(x.Vs)
        base = x.kv.seq_base.cpu().numpy()
        cap = x.kv.seq_cap.cpu().numpy()
        scap = int(x.sd.seq_cap[0].item())
        sbase = x.sd.seq_base.cpu().numpy()
        t = 0.0
        for b, g in pairs:
            n = lens[b]
            off = int(base[b]) + g * int(cap[b]) * d
            K = oracle.widen(Kb[off:off + n * d].reshape(n, d), dt)
            V = oracle.widen(Vb[off:off + n * d].reshape(n, d), dt)
            ck = oracle.chunk_keys(K, n, cs)            # prefill: not timed
            soff = int(sbase[b]) + g * scap * d
            Ks = oracle.widen(Ksb[soff:soff + scap * d].reshape(scap, d), dt)
            Vs = oracle.widen(Vsb[soff:soff + scap * d].reshape(scap, d), dt)
            t0 = time.perf_counter()
            c0 = max(0, (n - Q) // cs)
            ck[c0:] = oracle.chunk_keys(K[c0 * cs:n], n - c0 * cs, cs)   # tail refresh
            qg = np.stack([oracle.widen(qd[b, g * G + j], dt) for j in range(G)])
            sel = oracle.select_topk(oracle.chunk_scores(qg, ck), k)
            for j in range(G):
                h = g * G + j
                oracle.sparse_attn(qg[j], K, V, n, sel, cs)
                # streaming positions in ring order; every slot of the ring is resident here
                pos = oracle.stream_positions(n, S, Wn)
                slots = [p if p < S else S + (p - S) % (scap - S) for p in pos]
                oracle.attention(qg[j], Ks[slots], Vs[slots])
                oracle.verify_attn(oracle.widen(qv[b, h], dt), K, V, n)
            t += time.perf_counter() - t0
        return t

    def accepts():
        t0 = time.perf_counter()
        for b in range(acc_in.target.shape[0]):
            oracle.accept(acc_in.target[b], acc_in.draft[b], acc_in.tokens[b], acc_in.uniforms[b], 1.0)
        return time.perf_counter() - t0

    every = [(b, g) for b in range(len(lens)) for g in range(Hkv)]
    t_layers = sum(heads_of(x, every) for x in sample_layers)
    t_acc = accepts()
    nl = len(sample_layers)
    t_step = t_layers / nl * layers + t_acc
    out = {"value": round(1.0 / t_step, 6), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
           "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
           "sample": f"fp64 numpy oracle on {nl} of the {layers} layers (all {Hkv} KV heads x {Hq} query heads, "
                     f"{len(lens)} sequence(s)) + 1 accept, {t_layers + t_acc:.1f} s timed, scaled to "
                     f"{layers} layers ({t_layers / nl:.2f} s per layer); chunk-key prefill untimed",
           "s_per_layer": round(t_layers / nl, 4)}
    # the same oracle on one thread, over a few heads of one layer
    try:
        from threadpoolctl import threadpool_limits
        # four pairs spread over the sequences, scaled by their share of the
        # layer's rows (the work of a pair grows with its sequence's length)
        few = every[::max(1, len(every) // 4)][:4]
        with threadpool_limits(limits=1):
            t1 = heads_of(sample_layers[0], few)
            t1a = accepts()
        rows_all = sum(lens[b] for b, _ in every)
        rows_few = max(1, sum(lens[b] for b, _ in few))
        t1_step = t1 * rows_all / rows_few * layers + t1a
        out["single_thread"] = {"value": round(1.0 / t1_step, 6), "unit": "steps/s", "cores": 1,
                                "sample": f"{len(few)} (sequence, KV head) pairs of one layer + 1 accept on one "
                                          f"thread, {t1 + t1a:.1f} s timed, scaled to the step by rows"}
    except ImportError:
        pass
    return out


if __name__ == "__main__":
    main()
