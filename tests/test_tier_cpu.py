"""The expert tier's placement policy (moe_vq_tier_plan), on the host: free device
slots first, then the least recently used slot whose expert the step does not select;
selected experts are never evicted, resident ones are not copied again, experts the
host pool does not hold are left absent, and a step selecting more experts than the
tier has slots is refused."""
import pytest

from bit_vector_quantised_amd import _lib


def tier(n_experts=8, n_slots=3, absent=()):
    host = [(e * 256, _lib.FMT_ABSENT if e in absent else _lib.FMT_VQ2) for e in range(n_experts)]
    return _lib.ExpertTier(n_experts, 0, host, [s * 256 for s in range(n_slots)])


def test_free_slots_in_index_order():
    assert _lib.tier_plan(tier(), [5, 1, 3]) == [(5, 0, -1), (1, 1, -1), (3, 2, -1)]


def test_resident_experts_are_not_copied_again():
    t = tier()
    t.set_state([5, -1, 1], [4, 0, 4])
    assert _lib.tier_plan(t, [1, 5, 2]) == [(2, 1, -1)]


def test_least_recently_used_inactive_expert_is_evicted():
    t = tier()
    t.set_state([0, 1, 2], [7, 3, 5])
    # expert 1 holds the oldest stamp and is not selected
    assert _lib.tier_plan(t, [0, 6]) == [(6, 1, 1)]
    # with expert 1 selected, the next oldest (expert 2) goes
    assert _lib.tier_plan(t, [1, 6]) == [(6, 2, 2)]


def test_equal_stamps_evict_the_lower_slot():
    t = tier()
    t.set_state([0, 1, 2], [2, 2, 2])
    assert _lib.tier_plan(t, [7]) == [(7, 0, 0)]


def test_two_misses_take_two_different_slots():
    t = tier()
    t.set_state([0, 1, 2], [1, 2, 3])
    assert _lib.tier_plan(t, [6, 7]) == [(6, 0, 0), (7, 1, 1)]


def test_expert_missing_from_the_host_pool_stays_absent():
    t = tier(absent=(4,))
    assert _lib.tier_plan(t, [4, 2]) == [(2, 0, -1)]


def test_more_selected_experts_than_slots_is_refused():
    t = tier(n_slots=2)
    with pytest.raises(_lib.MoeVqError) as ei:
        _lib.tier_plan(t, [1, 2, 3])
    assert ei.value.status == _lib.ENOSPACE
    # all slots held by selected experts: nothing to evict for a new one
    t.set_state([1, 2], [1, 1])
    with pytest.raises(_lib.MoeVqError) as ei:
        _lib.tier_plan(t, [1, 2, 3])
    assert ei.value.status == _lib.ENOSPACE


def test_bad_expert_id_is_an_argument_error():
    with pytest.raises(_lib.MoeVqError) as ei:
        _lib.tier_plan(tier(), [8])
    assert ei.value.status == _lib.EINVAL
