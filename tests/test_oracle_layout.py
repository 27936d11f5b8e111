"""Pins of the oracle's reading of the pool layout (include/pagedkv.h).

The pages fix no byte layout; the block and tile structure follows "LLM
inference basics and vLLM internals" §4 (16-token blocks, per-request block
tables).  Pins: hand-computed offsets (tests/golden/layout_offsets.txt) and
the bijection property of every sub-tile.
"""
import os

import numpy as np
import pytest

import oracle

G = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_offsets():
    n = 0
    for ln in open(os.path.join(G, "layout_offsets.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        pool, eb, r, k, want = ln.split()
        fn = oracle.k_sub_offset if pool == "K" else oracle.v_sub_offset
        assert fn(int(r), int(k), int(eb)) == int(want), ln
        n += 1
    assert n >= 20


@pytest.mark.parametrize("eb", [1, 2])
@pytest.mark.parametrize("is_v", [0, 1])
def test_subtile_bijection(eb, is_v):
    d = 128
    fn = oracle.v_sub_offset if is_v else oracle.k_sub_offset
    offs = np.array([fn(r, k, eb) for r in range(16) for k in range(d)])
    assert offs.min() == 0 and offs.max() == 16 * d * eb - eb
    assert np.all(offs % eb == 0)
    assert len(np.unique(offs)) == 16 * d


@pytest.mark.parametrize("dtype,bs", [(oracle.BF16, 16), (oracle.FP8, 16), (oracle.BF16, 32)])
def test_pool_offsets_cover_pool_exactly_once(dtype, bs):
    nb, H, d = 3, 2, 128
    eb = oracle.elem_bytes(dtype)
    total = oracle.layer_pool_bytes(nb, H, d, bs, dtype)
    assert total == nb * H * bs * d * eb
    for is_v in (0, 1):
        offs = [oracle.pool_offset(pb, g, t, k, is_v, H, d, bs, dtype)
                for pb in range(nb) for g in range(H) for t in range(bs) for k in range(d)]
        offs = np.array(offs)
        assert len(np.unique(offs)) == offs.size == total // eb
        assert offs.max() == total - eb


def test_tile_base():
    # tile (pb, g) starts at (pb * H_kv + g) * tile_bytes
    H, d, bs = 4, 128, 16
    tile = bs * d * 2
    assert oracle.pool_offset(5, 3, 0, 0, 0, H, d, bs, oracle.BF16) == (5 * H + 3) * tile
    # second 16-token sub-tile of a 32-token block
    assert oracle.pool_offset(1, 0, 16, 0, 1, 1, d, 32, oracle.BF16) == 32 * d * 2 + 16 * d * 2
