"""The host-side slot-aliasing check (no GPU)."""
import numpy as np
import pytest

from linear_attention_speculative_amd.debug import check_slot_aliasing


def test_distinct_sources_and_in_place_commits_pass():
    check_slot_aliasing(np.array([3, 5, 0, 0, 9]), num_slots=10)
    check_slot_aliasing(np.array([3, 5, 7]), num_slots=10,
                        final_state_indices=np.array([3, 8, 0]),
                        boundary_state_indices=np.array([0, 5, 7]))


def test_duplicate_sources_fail():
    with pytest.raises(ValueError, match="both read slot 5"):
        check_slot_aliasing(np.array([5, 2, 5]), num_slots=8)
    # null and past-pool slots never alias
    check_slot_aliasing(np.array([0, 0, 12, 12]), num_slots=8)


def test_destinations_must_not_hit_other_requests():
    with pytest.raises(ValueError, match="writes slot 5"):
        check_slot_aliasing(np.array([3, 5]), num_slots=8,
                            final_state_indices=np.array([5, 5]))
    with pytest.raises(ValueError, match="writes slot 6"):
        check_slot_aliasing(np.array([3, 5]), num_slots=8,
                            final_state_indices=np.array([6, 5]),
                            boundary_state_indices=np.array([0, 6]))
    # a request that commits nothing writes nothing
    check_slot_aliasing(np.array([3, 5]), num_slots=8,
                        commit_lens=np.array([2, 0]),
                        final_state_indices=np.array([6, 6]))
