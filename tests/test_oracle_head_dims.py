"""Pins of the oracle at head_dim 64 and 256 (the pool layout of
include/pagedkv.h holds for any multiple of 64; the decode path is built
for 64, 128 and 256).

  - hand-computed element offsets from the layout formula;
  - every (row, dim) of a tile maps to its own byte, and the tile is covered;
  - the paged decode equals the contiguous brute force (oracle/brute.py) on
    tiny inputs ("LLM inference basics and vLLM internals" §4: gather
    through the block table; §2: grouped query heads).
"""
import numpy as np
import pytest

import oracle
from oracle import brute
import workloads
from tests import pools


# (head_dim, dtype, is_value, row, dim) -> byte offset inside tile (block 0,
# head 0), worked by hand from the formula in pagedkv.h:
#   K: c = k/8, lane = r + 16(c%4), kk = c/4, e = k%8, n = 2/E,
#      byte = 1024(kk/n) + 16 lane + 8E(kk%n) + E e
#   V: nt = k/16, lane = k%16 + 16(r/4), i = r%4, n = 4/E,
#      byte = 1024(nt/n) + 16 lane + 4E(nt%n) + E i
HAND = [
    (256, oracle.BF16, 0, 3, 200, 1024 * 6 + 16 * 19),          # c=25: lane 19, kk 6
    (256, oracle.BF16, 1, 5, 200, 1024 * 6 + 16 * 24 + 2),      # nt=12: lane 24, i 1
    (256, oracle.FP8, 0, 0, 255, 1024 * 3 + 16 * 48 + 8 + 7),   # c=31: lane 48, kk 7
    (64, oracle.FP8, 0, 15, 63, 1023),                          # last byte of the K sub-tile
    (64, oracle.FP8, 1, 15, 63, 1023),                          # last byte of the V sub-tile
    (64, oracle.BF16, 1, 16, 0, 16 * 64 * 2 + 0),               # row 16: second sub-tile
]


@pytest.mark.parametrize("d,dt,isv,r,k,want", HAND)
def test_hand_offsets(d, dt, isv, r, k, want):
    assert oracle.pool_offset(0, 0, r, k, isv, 1, d, 32, dt) == want


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP8])
@pytest.mark.parametrize("bs", [16, 32])
def test_tile_bijection(d, dt, bs):
    eb = oracle.elem_bytes(dt)
    for isv in (0, 1):
        offs = [oracle.pool_offset(0, 0, r, k, isv, 1, d, bs, dt) for r in range(bs) for k in range(d)]
        assert sorted(offs) == [eb * i for i in range(bs * d)]
    # the second kv head's tile follows the first
    assert oracle.pool_offset(0, 1, 0, 0, 0, 2, d, bs, dt) == bs * d * eb


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("kv,bs", [(oracle.BF16, 16), (oracle.FP8, 32), (oracle.FP16, 16)])
def test_paged_decode_matches_brute_force(d, kv, bs):
    src = oracle.FP16 if kv == oracle.FP16 else oracle.BF16
    lengths = [1, 17, 40, 77]
    H, Hkv = 8, 2
    ks = 0.02 if kv == oracle.FP8 else 1.0
    _, r_perm, _, r_val = workloads.streams(5)
    tabs = workloads.build_tables(lengths, bs, r_perm)
    kb = [workloads.normal_bits(r_val, (c, Hkv, d), src) for c in lengths]
    vb = [workloads.normal_bits(r_val, (c, Hkv, d), src) for c in lengths]
    q = workloads.normal_bits(r_val, (len(lengths), H, d), src)
    kp, vp = pools.write_contiguous(kb, vb, tabs.block_tables, tabs.context_lens, Hkv, d, bs,
                                    tabs.num_blocks, kv, src, ks, ks)
    scale = float(np.float32(1 / np.sqrt(d)))
    got = oracle.paged_decode(q, src, kp, vp, kv, tabs.block_tables, tabs.context_lens, Hkv, bs,
                              scale, ks, ks)

    def values(bits):
        v = oracle.decode_values(bits, src)
        if kv != oracle.FP8:
            return v
        inv = np.float32(1.0) / np.float32(ks)
        codes = oracle.e4m3_encode((v.astype(np.float32) * inv).astype(np.float32))
        return oracle.e4m3_table()[codes] * float(np.float32(ks))

    for s in range(len(lengths)):
        want = brute.attention(oracle.decode_values(q[s], src), values(kb[s]), values(vb[s]), scale)
        np.testing.assert_allclose(got[s], want, rtol=0, atol=1e-12)
