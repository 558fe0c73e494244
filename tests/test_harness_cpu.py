"""Host-side logic of the trajectory harness that needs no GPU."""

import pytest

from reuse_pab_plan_amd import harness, lib


def test_cache_capacity_check():
    # Host-side sizing of the broadcast cache: two output-sized slots per
    # (block, type); a shortfall raises PAB_ERR_CAPACITY before allocation.
    cfg = harness.CONFIGS["stack28"]
    need = harness.cache_bytes(cfg)
    assert need == 2 * 28 * 3 * 1 * 16 * 48 * 1590 * 72 * 2      # 29.5 GB
    harness.check_capacity(need, need, "cache")
    with pytest.raises(lib.PabError) as e:
        harness.check_capacity(need, need - 1, "cache")
    assert e.value.status == lib.PAB_ERR_CAPACITY
