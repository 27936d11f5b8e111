"""Pins of the oracle's paged decode attention.

The oracle gathers K/V through the block table ("LLM inference basics and
vLLM internals" §4; "vLLM internals (2)", "Block table") and runs fp64
softmax attention with GQA head grouping (§2).  It is pinned here to:
  - the contiguous brute force of oracle/brute.py on tiny inputs (the
    textbook attention the paged form must equal; K/V are drawn contiguous
    and scattered into the pool by the test);
  - closed forms: c = 1 gives V_0; q = 0 gives the mean of V; a key equal to
    lambda*q for large lambda selects its value; c = 0 gives zeros;
  - invariants: relabelling physical blocks changes nothing (bitwise);
    sequences sharing prefix blocks (ref_cnt > 1, §4 and "Sharing") match
    private copies bitwise; NaN in the null block, in unused table entries'
    targets and in tail slots of the last block never reaches the output.
"""
import numpy as np
import pytest

import oracle
from oracle import brute
import workloads
from tests import pools

D = 128


def _setup(lengths, H, Hkv, bs, kv_dtype, src_dtype, seed=0, num_blocks=None,
           k_scale=1.0, v_scale=1.0):
    r_len, r_perm, _, r_val = workloads.streams(seed)
    tabs = workloads.build_tables(lengths, bs, r_perm, num_blocks=num_blocks)
    kb = [workloads.normal_bits(r_val, (int(c), Hkv, D), src_dtype) for c in lengths]
    vb = [workloads.normal_bits(r_val, (int(c), Hkv, D), src_dtype) for c in lengths]
    q = workloads.normal_bits(r_val, (len(lengths), H, D), src_dtype)
    kp, vp = pools.write_contiguous(kb, vb, tabs.block_tables, tabs.context_lens, Hkv, D,
                                    bs, tabs.num_blocks, kv_dtype, src_dtype, k_scale,
                                    v_scale)
    return tabs, kb, vb, q, kp, vp


def _values(bits, src_dtype, kv_dtype, scale):
    """Values a correct pool holds for contiguous source bits."""
    v = oracle.decode_values(bits, src_dtype)
    if kv_dtype != oracle.FP8:
        return v
    scale = float(np.float32(scale))              # scales cross the ABI as fp32
    inv = np.float32(1.0) / np.float32(scale)
    codes = oracle.e4m3_encode((v.astype(np.float32) * inv).astype(np.float32))
    return oracle.e4m3_table()[codes] * scale


@pytest.mark.parametrize("kv_dtype,src_dtype,bs", [
    (oracle.BF16, oracle.BF16, 16),
    (oracle.FP16, oracle.FP16, 16),
    (oracle.BF16, oracle.BF16, 32),
    (oracle.FP8, oracle.BF16, 16),
])
def test_matches_contiguous_brute_force(kv_dtype, src_dtype, bs):
    lengths = [1, 17, 64, 200]
    H, Hkv = 12, 2
    ks, vs = (0.02, 0.03) if kv_dtype == oracle.FP8 else (1.0, 1.0)
    tabs, kb, vb, q, kp, vp = _setup(lengths, H, Hkv, bs, kv_dtype, src_dtype,
                                     num_blocks=64 if bs == 16 else 40, k_scale=ks,
                                     v_scale=vs)
    scale = float(np.float32(1 / np.sqrt(D)))
    got = oracle.paged_decode(q, src_dtype, kp, vp, kv_dtype, tabs.block_tables,
                              tabs.context_lens, Hkv, bs, scale, ks, vs)
    for s, c in enumerate(lengths):
        qd = oracle.decode_values(q[s], src_dtype)
        want = brute.attention(qd, _values(kb[s], src_dtype, kv_dtype, ks),
                               _values(vb[s], src_dtype, kv_dtype, vs), scale)
        np.testing.assert_allclose(got[s], want, rtol=0, atol=1e-12)
    assert np.isfinite(got).all()


def test_gather_reads_back_contiguous_values():
    lengths = [5, 40]
    tabs, kb, vb, q, kp, vp = _setup(lengths, 4, 2, 16, oracle.BF16, oracle.BF16)
    for s in range(2):
        k = pools.gather_values(kp, tabs.block_tables, tabs.context_lens, s, 2, D, 16,
                                oracle.BF16, 0)
        v = pools.gather_values(vp, tabs.block_tables, tabs.context_lens, s, 2, D, 16,
                                oracle.BF16, 1)
        assert np.array_equal(k, oracle.decode_values(kb[s], oracle.BF16))
        assert np.array_equal(v, oracle.decode_values(vb[s], oracle.BF16))


def test_closed_forms():
    H, Hkv, bs = 6, 2, 16
    lengths = [1, 33]
    tabs, kb, vb, q, kp, vp = _setup(lengths, H, Hkv, bs, oracle.BF16, oracle.BF16)
    scale = 0.125
    out = oracle.paged_decode(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                              tabs.context_lens, Hkv, bs, scale)
    v0 = oracle.decode_values(vb[0][0], oracle.BF16)          # [Hkv][d]
    for h in range(H):
        assert np.array_equal(out[0, h], v0[h // (H // Hkv)])   # c = 1: exactly V_0
    # q = 0: uniform weights -> mean of V over the context
    qz = np.zeros_like(q)
    out = oracle.paged_decode(qz, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                              tabs.context_lens, Hkv, bs, scale)
    vmean = oracle.decode_values(vb[1], oracle.BF16).mean(axis=0)
    for h in range(H):
        np.testing.assert_allclose(out[1, h], vmean[h // 3], rtol=0, atol=1e-13)


def test_dominant_key_selects_its_value():
    H, Hkv, bs, c, j = 4, 1, 16, 50, 37
    r = np.random.default_rng(3)
    q = workloads.normal_bits(r, (1, H, D), oracle.BF16)
    k = workloads.normal_bits(r, (c, Hkv, D), oracle.BF16) & np.uint16(0x8FFF)  # small keys
    v = workloads.normal_bits(r, (c, Hkv, D), oracle.BF16)
    qd = oracle.decode_values(q[0, 0], oracle.BF16)
    k[j, 0] = workloads.f32_to_bits((qd * 64.0).astype(np.float32), oracle.BF16)
    tabs = workloads.build_tables([c], bs, np.random.default_rng(1))
    kp, vp = pools.write_contiguous([k], [v], tabs.block_tables, tabs.context_lens, Hkv, D,
                                    bs, tabs.num_blocks, oracle.BF16, oracle.BF16)
    out = oracle.paged_decode(q[:, :1], oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                              tabs.context_lens, Hkv, bs, 1.0)
    np.testing.assert_allclose(out[0, 0], oracle.decode_values(v[j, 0], oracle.BF16),
                               atol=1e-9)


def test_zero_context_gives_zeros():
    tabs, kb, vb, q, kp, vp = _setup([0, 3], 4, 2, 16, oracle.BF16, oracle.BF16)
    out = oracle.paged_decode(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                              tabs.context_lens, 2, 16, 0.1)
    assert np.array_equal(out[0], np.zeros((4, D)))
    assert np.isfinite(out[1]).all()


def _relabel(pool, perm, Hkv, bs, eb):
    """Move tile of block b to block perm[b] (whole [H_kv] tiles)."""
    tile = Hkv * bs * D * eb
    nb = len(perm)
    src = pool.reshape(nb, tile)
    out = np.empty_like(src)
    out[perm] = src
    return out.reshape(-1)


@pytest.mark.parametrize("kv_dtype", [oracle.BF16, oracle.FP8])
def test_physical_permutation_invariance(kv_dtype):
    lengths = [3, 31, 70, 128]
    H, Hkv, bs = 8, 2, 16
    tabs, kb, vb, q, kp, vp = _setup(lengths, H, Hkv, bs, kv_dtype, oracle.BF16,
                                     k_scale=0.05, v_scale=0.05)
    base = oracle.paged_decode(q, oracle.BF16, kp, vp, kv_dtype, tabs.block_tables,
                               tabs.context_lens, Hkv, bs, 0.09, 0.05, 0.05)
    nb = tabs.num_blocks
    perm = np.concatenate([[0], 1 + np.random.default_rng(5).permutation(nb - 1)])
    eb = oracle.elem_bytes(kv_dtype)
    kp2, vp2 = _relabel(kp, perm, Hkv, bs, eb), _relabel(vp, perm, Hkv, bs, eb)
    bt2 = perm[tabs.block_tables].astype(np.int32)
    moved = oracle.paged_decode(q, oracle.BF16, kp2, vp2, kv_dtype, bt2, tabs.context_lens,
                                Hkv, bs, 0.09, 0.05, 0.05)
    assert np.array_equal(base, moved)


def test_shared_prefix_blocks_equal_private_copies():
    # seq 0 and 1 hold identical logical K/V; seq 1 reaches its first two
    # blocks through seq 0's physical blocks (ref_cnt 2), seq 2 has copies.
    H, Hkv, bs, c = 4, 1, 16, 45
    r = np.random.default_rng(11)
    k = workloads.normal_bits(r, (c, Hkv, D), oracle.BF16)
    v = workloads.normal_bits(r, (c, Hkv, D), oracle.BF16)
    q1 = workloads.normal_bits(r, (1, H, D), oracle.BF16)
    q = np.concatenate([q1, q1, q1])
    bt = np.array([[3, 8, 5], [3, 8, 9], [2, 6, 7]], np.int32)
    ctx = np.array([c, c, c], np.int32)
    kp, vp = pools.write_contiguous([k, k, k], [v, v, v], bt, ctx, Hkv, D, bs, 12,
                                    oracle.BF16, oracle.BF16)
    out = oracle.paged_decode(q, oracle.BF16, kp, vp, oracle.BF16, bt, ctx, Hkv, bs, 0.1)
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])


def test_nan_poison_never_reaches_output():
    # pools start all-NaN (pools.nan_pool); only context tokens are written.
    # Unused table entries point at the NaN null block 0.
    lengths = [1, 17, 64, 200]
    tabs, kb, vb, q, kp, vp = _setup(lengths, 12, 2, 16, oracle.BF16, oracle.BF16,
                                     num_blocks=64)
    assert (tabs.block_tables[0, 1:] == 0).all()
    out = oracle.paged_decode(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                              tabs.context_lens, 2, 16, 0.088)
    assert np.isfinite(out).all()


@pytest.mark.parametrize("H,Hkv", [(32, 1), (71, 1), (40, 2)])
def test_mqa_and_wide_groups_match_brute_force(H, Hkv):
    """MQA (one kv head for every query head) and groups above 16 query
    heads per kv head ("LLM inference basics and vLLM internals" §2): the
    oracle's head map h -> h / G against the brute force's head expansion."""
    lengths = [1, 17, 64, 130]
    tabs, kb, vb, q, kp, vp = _setup(lengths, H, Hkv, 16, oracle.BF16, oracle.BF16, seed=H)
    scale = float(np.float32(1 / np.sqrt(D)))
    got = oracle.paged_decode(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                              tabs.context_lens, Hkv, 16, scale)
    for s in range(len(lengths)):
        want = brute.attention(oracle.decode_values(q[s], oracle.BF16),
                               oracle.decode_values(kb[s], oracle.BF16),
                               oracle.decode_values(vb[s], oracle.BF16), scale)
        np.testing.assert_allclose(got[s], want, rtol=0, atol=1e-12)
