"""ctypes binding of libtfattn (include/tf_attn.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  torch is used for device memory and for the current stream.
The library is loaded lazily; if it has not been built, or cannot be loaded,
every call raises -- there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtfattn.so")

TF_OK, TF_ERR_INVALID_ARG, TF_ERR_UNSUPPORTED, TF_ERR_WORKSPACE, TF_ERR_HIP = 0, 1, 2, 3, 4
TF_DTYPE_FP16, TF_DTYPE_BF16, TF_DTYPE_FP32 = 1, 2, 3
TF_ACCEPT_PROBS = 1
TF_APPEND_FULL, TF_APPEND_RING = 0, 1
TF_APPEND_OK, TF_APPEND_NO_ROOM, TF_APPEND_RING_TOO_SMALL, TF_APPEND_BAD_LENGTH = 0, 1, 2, 3

EXPORTS = [
    "tf_status_string", "tf_last_error_detail",
    "tf_build_chunk_keys", "tf_score_chunks", "tf_select_topk", "tf_select_topk_workspace_size",
    "tf_sparse_attn", "tf_sparse_attn_workspace_size", "tf_sparse_verify_attn",
    "tf_sparse_verify_attn_workspace_size", "tf_stream_attn",
    "tf_verify_attn", "tf_verify_attn_workspace_size", "tf_accept", "tf_accept_workspace_size",
    "tf_append_kv", "tf_commit_length", "tf_collect_candidates", "tf_verify_tree_attn", "tf_tree_masks",
    "tf_tree_accept", "tf_tree_accept_workspace_size",
    "tf_verify_attn_noalloc", "tf_verify_attn_noalloc_max_bytes",
]


class TfError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {_status_name(status)}: {detail}")


class TfKvDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("seq_base", ctypes.c_void_p),
                ("seq_cap", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("max_len", ctypes.c_int32)]


_lib = None


def _status_name(s: int) -> str:
    return {0: "TF_OK", 1: "TF_ERR_INVALID_ARG", 2: "TF_ERR_UNSUPPORTED",
            3: "TF_ERR_WORKSPACE", 4: "TF_ERR_HIP"}.get(s, f"status {s}")


def lib() -> ctypes.CDLL:
    """Load libtfattn.so (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run hierarchical_speculative_attention_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    dp = ctypes.POINTER(TfKvDesc)
    sig = {
        "tf_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "tf_last_error_detail": (ctypes.c_char_p, []),
        "tf_build_chunk_keys": (ctypes.c_int, [vp, dp, i32, vp, i32, vp, dp, vp]),
        "tf_score_chunks": (ctypes.c_int, [vp, i32, i32, vp, dp, vp, i32, vp]),
        "tf_select_topk": (ctypes.c_int, [vp, i32, i32, i32, vp, i32, vp, vp, sz, vp]),
        "tf_select_topk_workspace_size": (sz, [i32, i32, i32, i32]),
        "tf_sparse_attn": (ctypes.c_int, [vp, i32, vp, vp, dp, vp, i32, i32, vp, vp, vp, sz, vp]),
        "tf_sparse_attn_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "tf_sparse_verify_attn": (ctypes.c_int, [vp, i32, i32, vp, vp, dp, vp, i32, i32, i32, vp, vp, vp, sz, vp]),
        "tf_sparse_verify_attn_workspace_size": (sz, [i32, i32, i32, i32, i32, i32, i32]),
        "tf_stream_attn": (ctypes.c_int, [vp, i32, vp, vp, dp, i32, i32, vp, vp, vp]),
        "tf_verify_attn": (ctypes.c_int, [vp, i32, i32, vp, vp, dp, vp, vp, vp, sz, vp]),
        "tf_verify_attn_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "tf_accept": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, f32, i32, vp, vp, vp, sz, vp]),
        "tf_accept_workspace_size": (sz, [i32, i32, i32]),
        "tf_append_kv": (ctypes.c_int, [vp, vp, i32, vp, vp, dp, i32, i32, i32, i32, vp, vp]),
        "tf_commit_length": (ctypes.c_int, [vp, i32, i32, i32, vp, vp]),
        "tf_collect_candidates": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, i32, vp]),
        "tf_verify_tree_attn": (ctypes.c_int, [vp, i32, i32, vp, vp, dp, vp, vp, vp, vp, sz, vp]),
        "tf_tree_masks": (ctypes.c_int, [vp, i32, i32, vp, vp]),
        "tf_tree_accept": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, f32, i32, vp, vp, vp, vp, sz, vp]),
        "tf_tree_accept_workspace_size": (sz, [i32, i32]),
        "tf_verify_attn_noalloc": (ctypes.c_int, [vp, i32, i32, vp, vp, dp, vp, vp, vp]),
        "tf_verify_attn_noalloc_max_bytes": (sz, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int, fn: str) -> None:
    if status != TF_OK:
        detail = lib().tf_last_error_detail()
        raise TfError(status, fn, detail.decode() if detail else "")


def dtype_code(dt: torch.dtype) -> int:
    return {torch.float16: TF_DTYPE_FP16, torch.bfloat16: TF_DTYPE_BF16, torch.float32: TF_DTYPE_FP32}[dt]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None, device=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


class KVDesc:
    """Head-major ragged layout of a cache buffer: row t of head h of
    sequence b starts at element seq_base[b] + (h * seq_cap[b] + t) * d."""

    def __init__(self, B: int, H: int, dtype: torch.dtype, seq_base, seq_cap, seq_len,
                 max_len: int, device, d: int = 128):
        self.B, self.H, self.d, self.dtype, self.max_len = int(B), int(H), int(d), dtype, int(max_len)
        self.device = torch.device(device)
        self.seq_base = torch.as_tensor(seq_base, dtype=torch.int64).to(self.device).contiguous()
        self.seq_cap = torch.as_tensor(seq_cap, dtype=torch.int32).to(self.device).contiguous()
        self.seq_len = torch.as_tensor(seq_len, dtype=torch.int32).to(self.device).contiguous()

    def c(self) -> TfKvDesc:
        return TfKvDesc(self.B, self.H, self.d, dtype_code(self.dtype), self.seq_base.data_ptr(),
                        self.seq_cap.data_ptr(), self.seq_len.data_ptr(), self.max_len)

    @staticmethod
    def from_layout(layout, dtype: torch.dtype, device, seq_len=None, max_len=None) -> "KVDesc":
        sl = layout.seq_len if seq_len is None else seq_len
        ml = int(max(sl)) if max_len is None and len(sl) else (max_len or 0)
        return KVDesc(layout.B, layout.H, dtype, layout.seq_base, layout.seq_cap, sl, ml, device, layout.d)


# ---------------------------------------------------------------------------
# Workspaces
# ---------------------------------------------------------------------------

def workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A workspace of the size a *_workspace_size() function returned (or
    None when that size is 0).  It needs no initialisation."""
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def verify_attn_workspace_size(B, Hq, H, Q, max_len) -> int:
    return int(lib().tf_verify_attn_workspace_size(B, Hq, H, Q, max_len))


def sparse_attn_workspace_size(B, Hq, H, k, chunk_size) -> int:
    return int(lib().tf_sparse_attn_workspace_size(B, Hq, H, k, chunk_size))


def accept_workspace_size(B, gamma, V) -> int:
    return int(lib().tf_accept_workspace_size(B, gamma, V))


def tree_accept_workspace_size(B, V) -> int:
    return int(lib().tf_tree_accept_workspace_size(B, V))


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------

def build_chunk_keys(K: torch.Tensor, kv: KVDesc, chunk_size: int, ck: torch.Tensor, ckd: KVDesc,
                     chunk_begin: Optional[torch.Tensor] = None, max_chunks: Optional[int] = None,
                     stream=None) -> torch.Tensor:
    _need(K, "K", kv.dtype)
    _need(ck, "ck", ckd.dtype)
    if max_chunks is None:
        max_chunks = max(1, -(-kv.max_len // chunk_size))
    kd, cd = kv.c(), ckd.c()
    _check(lib().tf_build_chunk_keys(_ptr(K), ctypes.byref(kd), chunk_size, _ptr(chunk_begin), int(max_chunks),
                                     _ptr(ck), ctypes.byref(cd), _stream(stream, K.device)), "tf_build_chunk_keys")
    return ck


def score_chunks(q: torch.Tensor, Hq: int, ck: torch.Tensor, ckd: KVDesc, c_max: int,
                 scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _need(q, "q")
    _need(ck, "ck", ckd.dtype)
    if scores is None:
        scores = torch.empty((ckd.B, ckd.H, c_max), dtype=torch.float32, device=q.device)
    _need(scores, "scores", torch.float32)
    cd = ckd.c()
    _check(lib().tf_score_chunks(_ptr(q), dtype_code(q.dtype), Hq, _ptr(ck), ctypes.byref(cd), _ptr(scores),
                                 int(c_max), _stream(stream, q.device)), "tf_score_chunks")
    return scores


def select_topk_workspace_size(B: int, rows: int, c_max: int, k: int) -> int:
    return int(lib().tf_select_topk_workspace_size(B, rows, c_max, k))


def select_topk(scores: torch.Tensor, n_chunks: torch.Tensor, k: int, idx: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _need(scores, "scores", torch.float32)
    _need(n_chunks, "n_chunks", torch.int32)
    B, rows, c_max = scores.shape
    if idx is None:
        idx = torch.empty((B, rows, k), dtype=torch.int32, device=scores.device)
    _need(idx, "idx", torch.int32)
    need = select_topk_workspace_size(B, rows, c_max, k)
    if ws is None and need:
        ws = workspace(need, scores.device)
    wp, wn = (_ptr(ws), ws.numel() * ws.element_size()) if ws is not None else (None, 0)
    _check(lib().tf_select_topk(_ptr(scores), B, rows, c_max, _ptr(n_chunks), int(k), _ptr(idx), wp, wn,
                                _stream(stream, scores.device)), "tf_select_topk")
    return idx


def sparse_attn(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, kv: KVDesc, idx: torch.Tensor,
                chunk_size: int, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None):
    _need(q, "q", kv.dtype)
    _need(K, "K", kv.dtype)
    _need(V, "V", kv.dtype)
    _need(idx, "idx", torch.int32)
    B, Hq = q.shape[0], q.shape[1]
    k = idx.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, kv.d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = sparse_attn_workspace_size(kv.B, Hq, kv.H, k, chunk_size)
    if ws is None:
        ws = workspace(need, q.device)
    kd = kv.c()
    _check(lib().tf_sparse_attn(_ptr(q), Hq, _ptr(K), _ptr(V), ctypes.byref(kd), _ptr(idx), int(k), int(chunk_size),
                                _ptr(out), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream(stream, q.device)), "tf_sparse_attn")
    return out, lse


def sparse_verify_attn_workspace_size(B, Hq, H, Q, k, chunk_size, tail) -> int:
    return int(lib().tf_sparse_verify_attn_workspace_size(B, Hq, H, Q, k, chunk_size, tail))


def sparse_verify_attn(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, kv: KVDesc, idx: torch.Tensor,
                       chunk_size: int, tail: int, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    _need(q, "q", kv.dtype)
    _need(K, "K", kv.dtype)
    _need(V, "V", kv.dtype)
    _need(idx, "idx", torch.int32)
    B, Hq, Q = q.shape[0], q.shape[1], q.shape[2]
    k = idx.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, Q, kv.d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Q), dtype=torch.float32, device=q.device)
    need = sparse_verify_attn_workspace_size(kv.B, Hq, kv.H, Q, k, chunk_size, tail)
    if ws is None:
        ws = workspace(need, q.device)
    kd = kv.c()
    _check(lib().tf_sparse_verify_attn(_ptr(q), Hq, Q, _ptr(K), _ptr(V), ctypes.byref(kd), _ptr(idx), int(k),
                                       int(chunk_size), int(tail), _ptr(out), _ptr(lse), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(stream, q.device)),
           "tf_sparse_verify_attn")
    return out, lse


def stream_attn(q: torch.Tensor, Ks: torch.Tensor, Vs: torch.Tensor, sd: KVDesc, n_sink: int, window: int,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    _need(q, "q", sd.dtype)
    _need(Ks, "Ks", sd.dtype)
    _need(Vs, "Vs", sd.dtype)
    B, Hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((B, Hq, sd.d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    d = sd.c()
    _check(lib().tf_stream_attn(_ptr(q), Hq, _ptr(Ks), _ptr(Vs), ctypes.byref(d), int(n_sink), int(window),
                                _ptr(out), _ptr(lse), _stream(stream, q.device)), "tf_stream_attn")
    return out, lse


def verify_attn(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, kv: KVDesc,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None):
    _need(q, "q", kv.dtype)
    _need(K, "K", kv.dtype)
    _need(V, "V", kv.dtype)
    B, Hq, Q = q.shape[0], q.shape[1], q.shape[2]
    if out is None:
        out = torch.empty((B, Hq, Q, kv.d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Q), dtype=torch.float32, device=q.device)
    need = verify_attn_workspace_size(kv.B, Hq, kv.H, Q, kv.max_len)
    if ws is None:
        ws = workspace(need, q.device)
    kd = kv.c()
    _check(lib().tf_verify_attn(_ptr(q), Hq, Q, _ptr(K), _ptr(V), ctypes.byref(kd), _ptr(out), _ptr(lse),
                                _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream, q.device)),
           "tf_verify_attn")
    return out, lse


def verify_attn_noalloc(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, kv: KVDesc, out: torch.Tensor,
                        lse: Optional[torch.Tensor] = None, stream=None):
    """tf_verify_attn_noalloc: verify attention with the library's built-in
    scratch instead of a workspace.  Nothing is allocated, here either: out
    (fp32 [B][Hq][Q][d]) is the caller's, lse ([B][Hq][Q]) is optional."""
    _need(q, "q", kv.dtype)
    _need(K, "K", kv.dtype)
    _need(V, "V", kv.dtype)
    _need(out, "out", torch.float32)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    Hq, Q = q.shape[1], q.shape[2]
    kd = kv.c()
    _check(lib().tf_verify_attn_noalloc(_ptr(q), Hq, Q, _ptr(K), _ptr(V), ctypes.byref(kd), _ptr(out), _ptr(lse),
                                        _stream(stream, q.device)), "tf_verify_attn_noalloc")
    return out, lse


def verify_attn_noalloc_max_bytes() -> int:
    return int(lib().tf_verify_attn_noalloc_max_bytes())


def accept(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor, uniforms: torch.Tensor,
           temperature: float, probs: bool = False, n_accepted: Optional[torch.Tensor] = None,
           next_token: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    _need(target, "target", torch.float32)
    _need(uniforms, "uniforms", torch.float64)
    B, Qp1, Vv = target.shape
    gamma = Qp1 - 1
    if gamma > 0:
        _need(draft, "draft", torch.float32)
        _need(draft_tokens, "draft_tokens", torch.int32)
    if n_accepted is None:
        n_accepted = torch.empty(B, dtype=torch.int32, device=target.device)
    if next_token is None:
        next_token = torch.empty(B, dtype=torch.int32, device=target.device)
    need = accept_workspace_size(B, gamma, Vv)
    if ws is None:
        ws = workspace(need, target.device)
    _check(lib().tf_accept(_ptr(target), _ptr(draft) if gamma else None, _ptr(draft_tokens) if gamma else None,
                           _ptr(uniforms), B, gamma, Vv, ctypes.c_float(temperature),
                           TF_ACCEPT_PROBS if probs else 0, _ptr(n_accepted), _ptr(next_token), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream, target.device)), "tf_accept")
    return n_accepted, next_token


def append_kv(K_new: torch.Tensor, V_new: torch.Tensor, K: torch.Tensor, V: torch.Tensor, kv: KVDesc,
              ring: bool = False, n_sink: int = 0, window: int = 0, reserve: Optional[int] = None,
              status: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
    """Copy the R new rows per (sequence, head), K_new / V_new [B][H][R][d],
    into the cache at the current lengths (full cache, or streaming ring).
    Returns the per-sequence status array (device int32 [B])."""
    _need(K_new, "K_new", kv.dtype)
    _need(V_new, "V_new", kv.dtype)
    _need(K, "K", kv.dtype)
    _need(V, "V", kv.dtype)
    R = int(K_new.shape[-2]) if K_new.dim() >= 2 else 0
    if tuple(K_new.shape) != (kv.B, kv.H, R, kv.d) or tuple(V_new.shape) != tuple(K_new.shape):
        raise ValueError(f"K_new / V_new must be [{kv.B}][{kv.H}][R][{kv.d}]")
    if status is None:
        status = torch.empty(kv.B, dtype=torch.int32, device=K.device)
    _need(status, "status", torch.int32)
    kd = kv.c()
    _check(lib().tf_append_kv(_ptr(K_new), _ptr(V_new), R, _ptr(K), _ptr(V), ctypes.byref(kd),
                              TF_APPEND_RING if ring else TF_APPEND_FULL, int(n_sink), int(window),
                              int(R if reserve is None else reserve), _ptr(status), _stream(stream, K.device)),
           "tf_append_kv")
    return status


def commit_length(seq_len: torch.Tensor, add: int, gamma: int = 0, n_accepted: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """seq_len[b] += add, minus the gamma - n_accepted[b] rejected drafts
    (device int32 [B], in place)."""
    _need(seq_len, "seq_len", torch.int32)
    if n_accepted is not None:
        _need(n_accepted, "n_accepted", torch.int32)
    _check(lib().tf_commit_length(_ptr(seq_len), int(seq_len.numel()), int(add), int(gamma), _ptr(n_accepted),
                                  _stream(stream, seq_len.device)), "tf_commit_length")
    return seq_len


def collect_candidates(draft_tokens: torch.Tensor, n_accepted: torch.Tensor, next_token: torch.Tensor,
                       q_rows: torch.Tensor, count_in: torch.Tensor, count_out: torch.Tensor,
                       cand: torch.Tensor, cand_q: torch.Tensor, stream=None) -> None:
    """Append one Force 2 round's emitted tokens and their q rows to the
    level-2 candidate chain (cand [B][gamma2], cand_q [B][gamma2][V]);
    count_out[b] = count_in[b] + the tokens taken."""
    B, g1p1, V = q_rows.shape
    gamma2 = cand.shape[1]
    for t, name, dt in ((n_accepted, "n_accepted", torch.int32), (next_token, "next_token", torch.int32),
                        (q_rows, "q_rows", torch.float32), (count_in, "count_in", torch.int32),
                        (count_out, "count_out", torch.int32), (cand, "cand", torch.int32),
                        (cand_q, "cand_q", torch.float32)):
        _need(t, name, dt)
    if g1p1 > 1:
        _need(draft_tokens, "draft_tokens", torch.int32)
    if tuple(cand_q.shape) != (B, gamma2, V):
        raise ValueError("cand_q must be [B][gamma2][V]")
    _check(lib().tf_collect_candidates(_ptr(draft_tokens) if g1p1 > 1 else None, _ptr(n_accepted), _ptr(next_token),
                                       _ptr(q_rows), B, g1p1 - 1, V, _ptr(count_in), _ptr(count_out), _ptr(cand),
                                       _ptr(cand_q), gamma2, _stream(stream, q_rows.device)), "tf_collect_candidates")


def tree_masks(parent: torch.Tensor, stream=None) -> torch.Tensor:
    """Visibility masks (device int64 holding uint64 bits, [B][Q]) of the
    candidate trees given by parent pointers (device int32 [B][Q])."""
    _need(parent, "parent", torch.int32)
    B, Q = parent.shape
    masks = torch.empty((B, Q), dtype=torch.int64, device=parent.device)
    _check(lib().tf_tree_masks(_ptr(parent), B, Q, _ptr(masks), _stream(stream, parent.device)), "tf_tree_masks")
    return masks


def verify_tree_attn(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, kv: KVDesc, tree_mask: torch.Tensor,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, stream=None):
    """Force 3 over a candidate tree: q [B][Hq][Q][d]; tree_mask [B][Q] (int64
    holding the uint64 masks)."""
    _need(q, "q", kv.dtype)
    _need(K, "K", kv.dtype)
    _need(V, "V", kv.dtype)
    _need(tree_mask, "tree_mask", torch.int64)
    B, Hq, Q = q.shape[0], q.shape[1], q.shape[2]
    if tuple(tree_mask.shape) != (B, Q):
        raise ValueError("tree_mask must be [B][Q]")
    if out is None:
        out = torch.empty((B, Hq, Q, kv.d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Q), dtype=torch.float32, device=q.device)
    need = verify_attn_workspace_size(kv.B, Hq, kv.H, Q, kv.max_len)
    if ws is None:
        ws = workspace(need, q.device)
    kd = kv.c()
    _check(lib().tf_verify_tree_attn(_ptr(q), Hq, Q, _ptr(K), _ptr(V), ctypes.byref(kd), _ptr(tree_mask), _ptr(out),
                                     _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream, q.device)),
           "tf_verify_tree_attn")
    return out, lse


def tree_accept(target: torch.Tensor, draft: torch.Tensor, tokens: torch.Tensor, parent: torch.Tensor,
                uniforms: torch.Tensor, temperature: float, probs: bool = False,
                ws: Optional[torch.Tensor] = None, stream=None):
    """Accept / reject over candidate trees: target, draft [B][Q][V] fp32;
    tokens, parent [B][Q] int32; uniforms [B][Q] fp64.  Returns
    (n_accepted [B], path [B][Q-1], next_token [B])."""
    _need(target, "target", torch.float32)
    _need(tokens, "tokens", torch.int32)
    _need(parent, "parent", torch.int32)
    _need(uniforms, "uniforms", torch.float64)
    B, Q, V = target.shape
    if Q > 1:
        _need(draft, "draft", torch.float32)
    n_acc = torch.empty(B, dtype=torch.int32, device=target.device)
    path = torch.empty((B, max(Q - 1, 1)), dtype=torch.int32, device=target.device)
    nxt = torch.empty(B, dtype=torch.int32, device=target.device)
    need = tree_accept_workspace_size(B, V)
    if ws is None:
        ws = workspace(need, target.device)
    _check(lib().tf_tree_accept(_ptr(target), _ptr(draft) if Q > 1 else None, _ptr(tokens), _ptr(parent),
                                _ptr(uniforms), B, Q, V, ctypes.c_float(temperature), TF_ACCEPT_PROBS if probs else 0,
                                _ptr(n_acc), _ptr(path), _ptr(nxt), _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream(stream, target.device)), "tf_tree_accept")
    return n_acc, path[:, :Q - 1], nxt

