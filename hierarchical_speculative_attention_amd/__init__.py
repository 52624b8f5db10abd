"""MI355X (gfx950) decode-step attention of hierarchical speculative decoding.

The compute path is libtfattn.so (hand-written HIP kernels behind the C ABI of
include/tf_attn.h); this package holds its sources, its build script, a thin
ctypes binding and the seeded input generators.  Importing the package does
not load the library; the first call does, and raises if it is not built.
"""
from ._lib import (  # noqa: F401
    KVDesc, TfError, accept, build_chunk_keys, score_chunks, select_topk, select_topk_workspace_size, sparse_attn,
    sparse_verify_attn, sparse_verify_attn_workspace_size,
    stream_attn, verify_attn, workspace, verify_attn_workspace_size, verify_attn_noalloc,
    verify_attn_noalloc_max_bytes,
    sparse_attn_workspace_size, accept_workspace_size, tree_accept_workspace_size, lib, append_kv, commit_length,
    collect_candidates, tree_masks, verify_tree_attn, tree_accept,
    TF_OK, TF_ERR_INVALID_ARG, TF_ERR_UNSUPPORTED, TF_ERR_WORKSPACE, TF_ERR_HIP,
    TF_APPEND_OK, TF_APPEND_NO_ROOM, TF_APPEND_RING_TOO_SMALL, TF_APPEND_BAD_LENGTH,
)
