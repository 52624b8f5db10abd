"""The C-ABI library loads without a GPU, exports every function the header
declares, and rejects bad arguments on the host before anything is enqueued
(so these calls never reach the GPU: every pointer below is a dummy)."""

import ctypes
import os
import re

import pytest

from hierarchical_speculative_attention_amd import _lib as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tf_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(T.LIB_PATH), reason="libtfattn.so not built")

FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced by a failing call


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tf_[a-z_]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = declared()
    assert len(names) >= 15
    L = T.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(T.EXPORTS) == names


def desc(B=1, H=4, d=128, dtype=T.TF_DTYPE_BF16, max_len=100, arrays=True):
    p = FAKE.value if arrays else None
    return T.TfKvDesc(B, H, d, dtype, p, p, p, max_len)


def call_verify(kv, Hq=4, Q=5, q=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return T.lib().tf_verify_attn(q, Hq, Q, FAKE, FAKE, ctypes.byref(kv), FAKE, None, ws, ws_bytes, None)


def test_status_strings():
    L = T.lib()
    assert L.tf_status_string(0) == b"TF_OK"
    assert L.tf_status_string(3) == b"TF_ERR_WORKSPACE"
    assert L.tf_status_string(99) == b"TF_ERR_UNKNOWN"


@pytest.mark.parametrize("kw,status", [
    (dict(d=64), T.TF_ERR_UNSUPPORTED),
    (dict(dtype=T.TF_DTYPE_FP32), T.TF_ERR_UNSUPPORTED),
    (dict(dtype=7), T.TF_ERR_UNSUPPORTED),
    (dict(H=0), T.TF_ERR_INVALID_ARG),
    (dict(B=-1), T.TF_ERR_INVALID_ARG),
    (dict(max_len=-5), T.TF_ERR_INVALID_ARG),
    (dict(arrays=False), T.TF_ERR_INVALID_ARG),
])
def test_verify_descriptor_errors(kw, status):
    assert call_verify(desc(**kw)) == status
    assert T.lib().tf_last_error_detail()


def test_verify_argument_errors():
    L = T.lib()
    assert call_verify(desc(), Hq=6) == T.TF_ERR_INVALID_ARG           # Hq not a multiple of H
    assert call_verify(desc(), Q=0) == T.TF_ERR_INVALID_ARG
    assert call_verify(desc(H=1), Hq=8, Q=9) == T.TF_ERR_UNSUPPORTED   # 72 rows per KV head
    assert call_verify(desc(), q=None) == T.TF_ERR_INVALID_ARG
    assert call_verify(desc(), q=ctypes.c_void_p(0x10008)) == T.TF_ERR_INVALID_ARG  # misaligned
    need = L.tf_verify_attn_workspace_size(1, 4, 4, 5, 100000)
    assert need > 0
    assert call_verify(desc(max_len=100000), ws=None, ws_bytes=0) == T.TF_ERR_WORKSPACE
    assert call_verify(desc(max_len=100000), ws_bytes=need - 1) == T.TF_ERR_WORKSPACE
    assert call_verify(desc(max_len=100000), ws=ctypes.c_void_p(0x10010)) == T.TF_ERR_INVALID_ARG
    assert b"workspace" in L.tf_last_error_detail()


def test_empty_batch_is_a_no_op():
    assert call_verify(desc(B=0, arrays=False)) == T.TF_OK


def test_other_entry_points_validate():
    L = T.lib()
    kv = desc()
    ckd = desc(dtype=T.TF_DTYPE_FP32)
    assert L.tf_build_chunk_keys(FAKE, ctypes.byref(kv), 0, None, 10, FAKE, ctypes.byref(ckd), None) == T.TF_ERR_INVALID_ARG
    assert L.tf_build_chunk_keys(FAKE, ctypes.byref(kv), 8, None, 0, FAKE, ctypes.byref(ckd), None) == T.TF_ERR_INVALID_ARG
    bad = desc(dtype=T.TF_DTYPE_FP16)
    assert L.tf_build_chunk_keys(FAKE, ctypes.byref(kv), 8, None, 4, FAKE, ctypes.byref(bad), None) == T.TF_ERR_INVALID_ARG
    assert L.tf_score_chunks(FAKE, T.TF_DTYPE_BF16, 6, FAKE, ctypes.byref(kv), FAKE, 200, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_score_chunks(FAKE, T.TF_DTYPE_BF16, 4, FAKE, ctypes.byref(kv), FAKE, 50, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_score_chunks(FAKE, T.TF_DTYPE_FP16, 4, FAKE, ctypes.byref(kv), FAKE, 200, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_score_chunks(FAKE, T.TF_DTYPE_BF16, 4, FAKE, ctypes.byref(kv), FAKE, (1 << 22) + 1, None) == T.TF_ERR_UNSUPPORTED
    assert L.tf_select_topk(FAKE, 1, 4, 100, FAKE, 0, FAKE, None, 0, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_select_topk(FAKE, 1, 4, (1 << 20) + 1, FAKE, 5, FAKE, None, 0, None) == T.TF_ERR_UNSUPPORTED
    assert L.tf_select_topk(None, 1, 4, 100, FAKE, 5, FAKE, None, 0, None) == T.TF_ERR_INVALID_ARG
    # few rows of more than 16384 chunks are selected in 8 slices per row and
    # merged: 8 (key, index) candidates of 8 bytes per slice, row and k
    assert L.tf_select_topk_workspace_size(1, 8, 32768, 512) == 8 * 8 * 512 * 8
    assert L.tf_select_topk_workspace_size(2, 8, 40000, 1023) == 2 * 8 * 8 * 1023 * 8
    assert L.tf_select_topk_workspace_size(1, 32, 16384, 512) == 0     # one workgroup per row
    assert L.tf_select_topk_workspace_size(1, 8, 16384, 512) == 0
    assert L.tf_select_topk_workspace_size(1, 17, 32768, 512) == 0     # enough rows to fill the chip
    assert L.tf_select_topk_workspace_size(1, 8, 32768, 4096) == 0     # slices would not halve the items
    assert L.tf_select_topk_workspace_size(1, 8, 70000, 512) == 0      # rows re-read from memory
    assert L.tf_select_topk(FAKE, 1, 8, 32768, FAKE, 512, FAKE, None, 0, None) == T.TF_ERR_WORKSPACE
    assert L.tf_select_topk(FAKE, 1, 8, 32768, FAKE, 512, FAKE, FAKE, 1000, None) == T.TF_ERR_WORKSPACE
    assert L.tf_sparse_attn(FAKE, 4, FAKE, FAKE, ctypes.byref(kv), FAKE, 0, 8, FAKE, None, None, 0, None) == T.TF_ERR_INVALID_ARG
    need = L.tf_sparse_attn_workspace_size(1, 4, 4, 512, 8)
    assert need > 0
    assert L.tf_sparse_attn(FAKE, 4, FAKE, FAKE, ctypes.byref(kv), FAKE, 512, 8, FAKE, None, None, 0, None) == T.TF_ERR_WORKSPACE
    assert L.tf_stream_attn(FAKE, 4, FAKE, FAKE, ctypes.byref(kv), -1, 252, FAKE, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_stream_attn(FAKE, 3, FAKE, FAKE, ctypes.byref(kv), 4, 252, FAKE, None, None) == T.TF_ERR_INVALID_ARG
    f = ctypes.c_float
    assert L.tf_accept(FAKE, FAKE, FAKE, FAKE, 1, 4, 0, f(1.0), 0, FAKE, FAKE, None, 0, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_accept(FAKE, FAKE, FAKE, FAKE, 1, 4, 100, f(-1.0), 0, FAKE, FAKE, None, 0, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_accept(FAKE, FAKE, FAKE, FAKE, 1, 4, 100, f(float("nan")), 0, FAKE, FAKE, None, 0, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_accept(FAKE, FAKE, FAKE, FAKE, 1, 4, 100, f(1.0), 4, FAKE, FAKE, None, 0, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_accept(FAKE, FAKE, FAKE, ctypes.c_void_p(0x10004), 1, 4, 100, f(1.0), 0, FAKE, FAKE, None, 0, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_accept(FAKE, FAKE, FAKE, FAKE, 1, 4, 70000, f(1.0), 0, FAKE, FAKE, FAKE, 1 << 20, None) == T.TF_ERR_UNSUPPORTED
    assert L.tf_accept(FAKE, FAKE, FAKE, FAKE, 1, 4, 100, f(1.0), 0, FAKE, FAKE, None, 0, None) == T.TF_ERR_WORKSPACE


def test_workspace_sizes_are_deterministic_and_grow_with_length():
    L = T.lib()
    a = L.tf_verify_attn_workspace_size(1, 32, 32, 7, 131072)
    assert a == L.tf_verify_attn_workspace_size(1, 32, 32, 7, 131072)
    assert L.tf_verify_attn_workspace_size(1, 32, 32, 7, 1 << 20) >= a
    assert L.tf_verify_attn_workspace_size(0, 32, 32, 7, 131072) == 0
    assert L.tf_accept_workspace_size(4, 6, 32000) >= 4 * 13 * 8 * 16
    assert L.tf_accept_workspace_size(0, 6, 32000) == 0


def test_cache_maintenance_validates():
    L = T.lib()
    kv = desc()
    assert L.tf_append_kv(FAKE, FAKE, -1, FAKE, FAKE, ctypes.byref(kv), 0, 0, 0, 0, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_append_kv(FAKE, FAKE, 3, FAKE, FAKE, ctypes.byref(kv), 5, 0, 0, 3, None, None) == T.TF_ERR_INVALID_ARG
    # ring: reserve below R, negative sinks or window
    assert L.tf_append_kv(FAKE, FAKE, 3, FAKE, FAKE, ctypes.byref(kv), T.TF_APPEND_RING, 4, 252, 2, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_append_kv(FAKE, FAKE, 3, FAKE, FAKE, ctypes.byref(kv), T.TF_APPEND_RING, -1, 252, 3, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_append_kv(None, FAKE, 3, FAKE, FAKE, ctypes.byref(kv), T.TF_APPEND_FULL, 0, 0, 3, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_append_kv(FAKE, FAKE, 3, ctypes.c_void_p(0x10008), FAKE, ctypes.byref(kv), 0, 0, 0, 3, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_append_kv(FAKE, FAKE, 3, FAKE, FAKE, ctypes.byref(desc(dtype=T.TF_DTYPE_FP32)), 0, 0, 0, 3, None, None) == T.TF_ERR_UNSUPPORTED
    assert L.tf_append_kv(FAKE, FAKE, 0, FAKE, FAKE, ctypes.byref(kv), 0, 0, 0, 0, None, None) == T.TF_OK  # nothing to do
    assert L.tf_commit_length(FAKE, 4, -1, 0, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_commit_length(FAKE, 4, 0, -2, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_commit_length(None, 4, 1, 0, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_commit_length(None, 0, 1, 0, None, None) == T.TF_OK


def test_collect_candidates_validates():
    L = T.lib()
    other = ctypes.c_void_p(0x20000)
    ok_args = lambda **kw: [kw.get(n, d) for n, d in (
        ("draft", FAKE), ("na", FAKE), ("nx", FAKE), ("q", FAKE), ("B", 2), ("g1", 3), ("V", 100),
        ("cin", FAKE), ("cout", other), ("cand", FAKE), ("cq", FAKE), ("g2", 5), ("s", None))]
    assert L.tf_collect_candidates(*ok_args(cout=FAKE)) == T.TF_ERR_INVALID_ARG    # in place: refused
    assert L.tf_collect_candidates(*ok_args(g2=0)) == T.TF_ERR_INVALID_ARG
    assert L.tf_collect_candidates(*ok_args(V=0)) == T.TF_ERR_INVALID_ARG
    assert L.tf_collect_candidates(*ok_args(q=ctypes.c_void_p(0x10004))) == T.TF_ERR_INVALID_ARG
    assert L.tf_collect_candidates(*ok_args(draft=None)) == T.TF_ERR_INVALID_ARG
    assert L.tf_collect_candidates(*ok_args(B=0, draft=None, q=None)) == T.TF_OK


def test_tree_entry_points_validate():
    L = T.lib()
    kv = desc()
    call = lambda Q=5, tm=FAKE, Hq=4: L.tf_verify_tree_attn(FAKE, Hq, Q, FAKE, FAKE, ctypes.byref(kv), tm, FAKE, None,
                                                            FAKE, 1 << 30, None)
    assert call(Q=0) == T.TF_ERR_INVALID_ARG
    assert call(Q=65) == T.TF_ERR_INVALID_ARG
    assert call(Q=17, Hq=16) == T.TF_ERR_UNSUPPORTED          # 4 * 17 rows per KV head
    assert call(tm=None) == T.TF_ERR_INVALID_ARG
    assert call(tm=ctypes.c_void_p(0x10004)) == T.TF_ERR_INVALID_ARG
    assert L.tf_tree_masks(FAKE, 2, 0, FAKE, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_tree_masks(FAKE, 2, 65, FAKE, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_tree_masks(None, 2, 5, FAKE, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_tree_masks(None, 0, 5, None, None) == T.TF_OK


def test_tree_accept_validates():
    L = T.lib()
    f = ctypes.c_float
    call = lambda B=2, Q=5, V=100, t=1.0, flags=0, ws=FAKE, ws_bytes=1 << 30, draft=FAKE: L.tf_tree_accept(
        FAKE, draft, FAKE, FAKE, FAKE, B, Q, V, f(t), flags, FAKE, FAKE, FAKE, ws, ws_bytes, None)
    assert call(Q=0) == T.TF_ERR_INVALID_ARG
    assert call(Q=65) == T.TF_ERR_UNSUPPORTED
    assert call(V=70000) == T.TF_ERR_UNSUPPORTED
    assert call(t=-1.0) == T.TF_ERR_INVALID_ARG
    assert call(flags=8) == T.TF_ERR_INVALID_ARG
    assert call(draft=None) == T.TF_ERR_INVALID_ARG
    assert call(ws=None, ws_bytes=0) == T.TF_ERR_WORKSPACE
    assert L.tf_tree_accept_workspace_size(2, 100) >= 2 * 100 * 8
    assert call(B=0) == T.TF_OK


LOG_PROBE = r"""
import ctypes
from hierarchical_speculative_attention_amd import _lib as T
FAKE = ctypes.c_void_p(0x10000)
kv = T.TfKvDesc(1, 4, 64, T.TF_DTYPE_BF16, FAKE.value, FAKE.value, FAKE.value, 100)
st = T.lib().tf_verify_attn(FAKE, 4, 5, FAKE, FAKE, ctypes.byref(kv), FAKE, None, FAKE, 1 << 30, None)
assert st == T.TF_ERR_UNSUPPORTED, st
"""


@pytest.mark.parametrize("value,logged", [("1", True), ("0", False), (None, False)])
def test_tf_log_prints_rejected_calls(value, logged):
    import subprocess
    import sys
    env = {k: v for k, v in os.environ.items() if k != "TF_LOG"}
    if value is not None:
        env["TF_LOG"] = value
    r = subprocess.run([sys.executable, "-c", LOG_PROBE], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("[tf] ")]
    if logged:
        assert lines == ["[tf] TF_ERR_UNSUPPORTED: kv: head dim 64 (only 128)"], r.stderr
    else:
        assert lines == [], r.stderr


def test_topk_workspace_follows_documented_rule():
    """tf_select_topk needs a workspace exactly when the header says so: at
    most 16 rows of 16385..65536 chunks, k <= 2048 and 2k <= the slice length
    (c_max / 8 rounded up to a multiple of 4); then 8 candidates of 8 bytes per
    row and k."""
    L = T.lib()
    for B, rows in [(1, 1), (1, 8), (2, 8), (1, 16), (4, 4), (1, 17), (3, 6), (1, 32)]:
        for c_max in [16384, 16385, 20001, 32768, 40001, 65536, 65537, 100000]:
            for k in [1, 512, 1250, 2048, 2049, 4096, 5000]:
                sl = ((c_max + 7) // 8 + 3) // 4 * 4
                split = B * rows <= 16 and 16384 < c_max <= 65536 and 2 * k <= sl and k <= 2048
                want = B * rows * 8 * k * 8 if split else 0
                assert L.tf_select_topk_workspace_size(B, rows, c_max, k) == want, (B, rows, c_max, k)


def test_verify_noalloc_validates_before_any_device_call():
    """The entry point that allocates nothing refuses, on the host and before
    any HIP call, arguments tf_verify_attn refuses and a call whose split
    partials exceed its built-in scratch (no GPU is touched here)."""
    L = T.lib()
    cap = L.tf_verify_attn_noalloc_max_bytes()
    assert cap == 48 << 20
    big = desc(B=1, H=32, max_len=1 << 22)  # 512 splits per head
    assert T.lib().tf_verify_attn_workspace_size(1, 32, 32, 7, 1 << 22) > cap
    st = L.tf_verify_attn_noalloc(FAKE, 32, 7, FAKE, FAKE, ctypes.byref(big), FAKE, None, None)
    assert st == T.TF_ERR_WORKSPACE
    assert b"scratch" in L.tf_last_error_detail()
    kv = desc(B=1, H=4, max_len=100)
    assert L.tf_verify_attn_noalloc(FAKE, 6, 5, FAKE, FAKE, ctypes.byref(kv), FAKE, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_verify_attn_noalloc(FAKE, 4, 0, FAKE, FAKE, ctypes.byref(kv), FAKE, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_verify_attn_noalloc(None, 4, 5, FAKE, FAKE, ctypes.byref(kv), FAKE, None, None) == T.TF_ERR_INVALID_ARG
    assert L.tf_verify_attn_noalloc(FAKE, 4, 5, FAKE, FAKE, None, FAKE, None, None) == T.TF_ERR_INVALID_ARG
    empty = desc(B=0, H=4, max_len=0)
    assert L.tf_verify_attn_noalloc(None, 4, 5, None, None, ctypes.byref(empty), None, None, None) == T.TF_OK


def plan_bytes(heads, nsplit, rows):
    """Workspace of a split plan: (max, sum) pairs (rounded up to 256 bytes)
    and 128-float accumulator rows per (head, split, padded query row); none
    with one split."""
    if nsplit <= 1:
        return 0
    parts = heads * nsplit * (-(-rows // 16) * 16)
    return ((parts * 8 + 255) // 256) * 256 + parts * 512


def test_split_counts_of_the_gpu_tests_are_the_librarys():
    """The GPU tests assert which split-plan regime a shape falls in with a
    Python restatement of the plan; the library's workspace sizes for those
    shapes follow from the same split counts."""
    from tests.test_gpu_attn import sparse_plan_tpw, verify_plan_splits
    L = T.lib()
    for Hkv, n in [(128, 300), (128, 400), (64, 600), (64, 1000), (32, 1100), (32, 2100), (16, 4200), (4, 20000)]:
        ns = verify_plan_splits(Hkv, n)
        assert L.tf_verify_attn_workspace_size(1, Hkv, Hkv, 3, n) == plan_bytes(Hkv, ns, 3), (Hkv, n)
    for B, Hkv, G, k, cs in [(1, 128, 1, 125, 8), (1, 64, 1, 162, 8), (1, 32, 1, 375, 8), (2, 4, 2, 300, 8),
                             (1, 16, 1, 1500, 8), (80, 8, 2, 40, 8), (1, 1, 4, 2000, 8), (1, 1, 2, 16500, 8)]:
        ns = -(-(k * cs) // sparse_plan_tpw(B, Hkv, k * cs))
        assert L.tf_sparse_attn_workspace_size(B, G * Hkv, Hkv, k, cs) == plan_bytes(B * Hkv, ns, G), (B, Hkv, k)
