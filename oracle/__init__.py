"""fp64 CPU oracle of the decode-attention path (test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the product path)."""
from .triforce_oracle import (  # noqa: F401
    NEG_INF, widen, round_f64_to_bits, chunk_keys, chunk_scores, select_topk,
    attention, sparse_token_positions, sparse_attn, sparse_verify_positions, sparse_verify_attn,
    stream_positions,
    stream_attn_masked, stream_attn_ring, verify_attn, tree_masks, verify_tree_attn, distribution,
    inverse_cdf, accept, tree_accept, two_level_accept,
    APPEND_OK, APPEND_NO_ROOM, APPEND_RING_TOO_SMALL, APPEND_BAD_LENGTH,
    append_full, ring_slot_of, append_ring, ring_visible, commit_length,
)
