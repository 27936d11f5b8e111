"""Host: random serving traces through the block manager, with the data
moved and read by the oracle (reshape_and_cache, whole-block copies and the
repack as token moves, the block-table and token-table decodes).  Each
output must equal contiguous attention over the sequence's own K / V in
logical order to fp64 rounding, so a wrong table, slot, prefix hit,
copy-on-write pair or repack tile from the manager fails here without a GPU
(the driver and its checks are in tests/serving_trace.py)."""
import pytest

import oracle
from tests import serving_trace as st

pkv = pytest.importorskip("paged_kv_cache_51_amd")

CFGS = {"bf16-bs16": st.Cfg(16), "bf16-bs32": st.Cfg(32), "fp8-bs16": st.Cfg(16, oracle.FP8, 0.02, 0.03)}


@pytest.mark.parametrize("name,seed", [("bf16-bs16", 0), ("bf16-bs16", 1), ("bf16-bs16", 2), ("bf16-bs16", 3),
                                       ("bf16-bs32", 4), ("bf16-bs32", 5), ("fp8-bs16", 6), ("fp8-bs16", 7)])
def test_random_serving_trace_host(name, seed):
    cfg = CFGS[name]
    stats = st.run_trace(seed, pkv, st.OracleBackend(cfg), cfg, log=lambda *a: None)
    assert stats["hit_tokens"] > 0 and stats["steps"] > 5 and stats["evictions"] > 0
    assert stats["cow"] > 0 or stats["forks"] == 0
