"""Host: random serving traces through the block manager, with the data
moved and read by the oracle (reshape_and_cache, whole-block copies and the
repack as token moves, the block-table and token-table decodes).  Each
output must equal contiguous attention over the sequence's own K / V in
logical order to fp64 rounding, so a wrong table, slot, prefix hit,
copy-on-write pair or repack tile from the manager fails here without a GPU
(the driver and its checks are in tests/serving_trace.py)."""
import pytest

from tests import serving_trace

pkv = pytest.importorskip("paged_kv_cache_51_amd")


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_serving_trace_host(seed):
    stats = serving_trace.run_trace(seed, pkv, serving_trace.OracleBackend(), log=lambda *a: None)
    assert stats["hit_tokens"] > 0 and stats["steps"] > 5 and stats["evictions"] > 0
    assert stats["cow"] > 0 or stats["forks"] == 0
