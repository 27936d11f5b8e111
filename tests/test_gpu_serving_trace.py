"""GPU: random serving traces through the host block manager, the data moved
and read by the library's kernels (reshape_and_cache, copy_blocks,
repack_blocks, the block-table decode, the token-table gather and run-list
decodes, multi-token attention of each prefill chunk), every output checked
against contiguous attention over each
sequence's own K / V (the driver and its checks are in tests/serving_trace.py):
bf16 pools of 16- and 32-token blocks, fp8 pools written from bf16, and
MQA with 20 and 32 query heads."""
import pytest
import torch

import oracle
from tests import serving_trace as st

pkv = pytest.importorskip("paged_kv_cache_51_amd")

pytestmark = pytest.mark.gpu

CFGS = {"bf16-bs16": st.Cfg(16), "bf16-bs32": st.Cfg(32), "fp8-bs16": st.Cfg(16, oracle.FP8, 0.02, 0.03),
        "fp8-bs32": st.Cfg(32, oracle.FP8, 0.02, 0.03),
        # one kv head: 32 query heads (two-tile decode entries), 20 (fp8)
        "mqa32-bf16-bs16": st.Cfg(16, heads=32, kv_heads=1),
        "mqa20-fp8-bs32": st.Cfg(32, oracle.FP8, 0.02, 0.03, heads=20, kv_heads=1)}


def log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name,seed", [("bf16-bs16", 0), ("bf16-bs16", 1), ("bf16-bs16", 2),
                                       ("bf16-bs32", 3), ("fp8-bs16", 4), ("fp8-bs32", 5),
                                       ("mqa32-bf16-bs16", 6), ("mqa20-fp8-bs32", 7)])
def test_random_serving_trace(name, seed):
    cfg = CFGS[name]
    log(f"trace {name} seed {seed}")
    stats = st.run_trace(seed, pkv, st.KernelBackend(pkv, torch, cfg), cfg, log=log)
    assert stats["hit_tokens"] > 0 and stats["steps"] > 5 and stats["evictions"] > 0
