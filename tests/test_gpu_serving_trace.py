"""GPU: random serving traces through the host block manager, the data moved
and read by the library's kernels (reshape_and_cache, copy_blocks,
repack_blocks, the block-table decode, the token-table gather and run-list
decodes), every output checked against contiguous attention over each
sequence's own K / V (the driver and its checks are in tests/serving_trace.py)."""
import pytest
import torch

from tests import serving_trace

pkv = pytest.importorskip("paged_kv_cache_51_amd")

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_serving_trace(seed):
    log(f"trace seed {seed}")
    stats = serving_trace.run_trace(seed, pkv, serving_trace.KernelBackend(pkv, torch), log=log)
    assert stats["hit_tokens"] > 0 and stats["steps"] > 5 and stats["evictions"] > 0
