"""Host-side checks of the three-tier driver (no GPU): a step that would
append past the full cache, or a drafter ring without room for the rows a
step may roll back, is refused before anything is enqueued -- the append
kernels would otherwise only set a status and write nothing."""

import pytest

from hierarchical_speculative_attention_amd import three_tier as tt


def test_full_cache_room():
    # gamma1 = 2, gamma2 = 6: the deepest row written is n + 7
    tt.check_room(100, 2, 6, 108)
    with pytest.raises(ValueError, match="full cache"):
        tt.check_room(100, 2, 6, 107)
    tt.check_room(0, 1, 1, 2)
    with pytest.raises(ValueError):
        tt.check_room(1, 1, 1, 2)


def test_drafter_ring_room():
    need = 252 + tt.drafter_reserve(2, 6)
    tt.check_ring(need, 252, 2, 6)
    with pytest.raises(ValueError, match="ring has"):
        tt.check_ring(need - 1, 252, 2, 6, layer=1)
