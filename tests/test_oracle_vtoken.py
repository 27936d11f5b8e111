"""Pins of the token-level virtualisation oracles ("vToken" page: a token
table maps each logical token to its physical place; evicting tokens leaves
survivors where they are; asynchronous repacking moves survivors together so
whole blocks can be freed, keeping the logical order).

  - decode through a token table built from a block table is exactly the
    block-table decode oracle (a separate code path);
  - decode of the survivors of an eviction equals the contiguous textbook
    attention over those tokens;
  - moving tokens and pointing the table at the new slots changes nothing;
    a swap shows every source is read before any destination is written;
  - the block model's repack produces an aligned table, preserves logical
    order and frees exactly the blocks it no longer needs.
"""
import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.blocks import BlockPoolModel
from tests.test_oracle_attention import _setup, _values

D = 128
SCALE = float(np.float32(1 / np.sqrt(D)))


def table_to_slots(block_tables, lengths, bs, width):
    out = np.zeros((len(lengths), width), np.int32)
    for s, c in enumerate(lengths):
        for t in range(int(c)):
            out[s, t] = block_tables[s][t // bs] * bs + t % bs
    return out


@pytest.mark.parametrize("kv,bs", [(oracle.BF16, 16), (oracle.FP8, 32)])
def test_token_table_from_block_table_equals_block_decode(kv, bs):
    lengths = [1, 17, 64, 100]
    ks = vs = 0.03 if kv == oracle.FP8 else 1.0
    tabs, kb, vb, q, kp, vp = _setup(lengths, 8, 2, bs, kv, oracle.BF16, seed=1,
                                     num_blocks=40, k_scale=ks, v_scale=vs)
    slots = table_to_slots(tabs.block_tables, lengths, bs, 128)
    a = oracle.paged_decode_tokens(q, oracle.BF16, kp, vp, kv, slots, tabs.context_lens, 2, bs,
                                   SCALE, ks, vs)
    b = oracle.paged_decode(q, oracle.BF16, kp, vp, kv, tabs.block_tables, tabs.context_lens, 2,
                            bs, SCALE, ks, vs)
    assert np.array_equal(a, b)


def test_survivors_match_contiguous_attention():
    lengths = [40, 90]
    tabs, kb, vb, q, kp, vp = _setup(lengths, 8, 2, 16, oracle.BF16, oracle.BF16, seed=2)
    r = np.random.default_rng(3)
    full = table_to_slots(tabs.block_tables, lengths, 16, 128)
    keep = [np.sort(r.choice(c, size=c // 3, replace=False)) for c in lengths]
    slots = np.zeros((2, 128), np.int32)
    for s in range(2):
        slots[s, :len(keep[s])] = full[s, keep[s]]
    ctx = np.array([len(k) for k in keep], np.int32)
    got = oracle.paged_decode_tokens(q, oracle.BF16, kp, vp, oracle.BF16, slots, ctx, 2, 16, SCALE)
    for s in range(2):
        kk = oracle.decode_values(kb[s][keep[s]], oracle.BF16)
        vv = oracle.decode_values(vb[s][keep[s]], oracle.BF16)
        want = brute.attention(oracle.decode_values(q[s], oracle.BF16), kk, vv, SCALE)
        np.testing.assert_allclose(got[s], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
def test_moving_tokens_and_the_table_changes_nothing(kv):
    lengths = [37]
    bs, nb = 16, 12
    ks = vs = 0.05 if kv == oracle.FP8 else 1.0
    tabs, kb, vb, q, kp, vp = _setup(lengths, 4, 2, bs, kv, oracle.BF16, seed=4, num_blocks=nb,
                                     k_scale=ks, v_scale=vs)
    slots = table_to_slots(tabs.block_tables, lengths, bs, 64)
    used = set(int(x) for x in slots[0, :37])
    free = [x for x in range(bs, nb * bs) if x not in used]
    r = np.random.default_rng(5)
    pick = r.choice(37, 10, replace=False)
    dst = r.choice(free, 10, replace=False)
    moves = [(int(slots[0, t]), int(d)) for t, d in zip(pick, dst)]
    (kp2,), (vp2,) = oracle.move_tokens([kp], [vp], moves, 2, D, bs, kv)
    slots2 = slots.copy()
    for t, d in zip(pick, dst):
        slots2[0, t] = d
    a = oracle.paged_decode_tokens(q, oracle.BF16, kp, vp, kv, slots, [37], 2, bs, SCALE, ks, vs)
    b = oracle.paged_decode_tokens(q, oracle.BF16, kp2, vp2, kv, slots2, [37], 2, bs, SCALE, ks, vs)
    assert np.array_equal(a, b)


def test_move_is_a_swap_safe_copy():
    bs = 16
    tabs, kb, vb, q, kp, vp = _setup([32], 4, 1, bs, oracle.BF16, oracle.BF16, seed=6, num_blocks=4)
    s0 = int(tabs.block_tables[0][0]) * bs + 3
    s1 = int(tabs.block_tables[0][1]) * bs + 9
    (k2,), (v2,) = oracle.move_tokens([kp], [vp], [(s0, s1), (s1, s0)], 1, D, bs, oracle.BF16)
    for pool, new in ((kp, k2), (vp, v2)):
        is_v = pool is vp
        for k in range(D):
            a0 = oracle.pool_offset(s0 // bs, 0, s0 % bs, k, is_v, 1, D, bs, oracle.BF16)
            a1 = oracle.pool_offset(s1 // bs, 0, s1 % bs, k, is_v, 1, D, bs, oracle.BF16)
            assert bytes(new[a0:a0 + 2]) == bytes(pool[a1:a1 + 2])
            assert bytes(new[a1:a1 + 2]) == bytes(pool[a0:a0 + 2])
    changed = np.nonzero(k2 != kp)[0]
    assert len(changed) <= 2 * 2 * D                 # only the two token rows


def test_model_repack_aligns_preserves_order_and_frees_blocks():
    m = BlockPoolModel(32, 16)
    m.add_sequence(1, list(range(100)))              # 7 blocks
    blocks0 = m.block_table(1)
    slots0 = m.token_slots(1)
    keep = [t % 3 == 0 or t > 90 for t in range(100)]
    m.evict_tokens(1, keep)
    surv = [sl for sl, k in zip(slots0, keep) if k]
    assert m.token_slots(1) == surv                  # survivors stay put, in order
    free_before = m.num_free_blocks()
    moves = m.repack(1)
    n = len(surv)
    nb = -(-n // 16)
    assert m.block_table(1) == blocks0[:nb]
    assert m.token_slots(1) == [blocks0[q // 16] * 16 + q % 16 for q in range(n)]
    assert m.num_free_blocks() == free_before + len(blocks0) - nb
    # the moves carry survivor q from its old slot to its aligned slot
    dst_of = dict(moves)
    for q, src in enumerate(surv):
        assert dst_of.get(src, src) == blocks0[q // 16] * 16 + q % 16
    m.evict_tokens(1, [True] * n)                   # a table again: growth needs a repack
    with pytest.raises(ValueError):
        m.append_token(1)
    m.repack(1)
    assert m.append_token(1)[0] == blocks0[n // 16] * 16 + n % 16


def test_model_refuses_eviction_on_shared_blocks():
    m = BlockPoolModel(32, 16)
    m.add_sequence(1, list(range(40)))
    m.fork(1, 2)
    with pytest.raises(ValueError):
        m.evict_tokens(1, [True] * 40)


@pytest.mark.parametrize("H,Hkv", [(32, 1), (40, 2)])
def test_survivors_match_contiguous_attention_wide_groups(H, Hkv):
    """The token-table oracle with MQA / more than 16 query heads per kv
    head ("LLM inference basics and vLLM internals" §2)."""
    lengths = [40, 90]
    tabs, kb, vb, q, kp, vp = _setup(lengths, H, Hkv, 16, oracle.BF16, oracle.BF16, seed=4)
    r = np.random.default_rng(5)
    full = table_to_slots(tabs.block_tables, lengths, 16, 128)
    keep = [np.sort(r.choice(c, size=c // 2, replace=False)) for c in lengths]
    slots = np.zeros((2, 128), np.int32)
    for s in range(2):
        slots[s, :len(keep[s])] = full[s, keep[s]]
    ctx = np.array([len(k) for k in keep], np.int32)
    got = oracle.paged_decode_tokens(q, oracle.BF16, kp, vp, oracle.BF16, slots, ctx, Hkv, 16,
                                     SCALE)
    for s in range(2):
        kk = oracle.decode_values(kb[s][keep[s]], oracle.BF16)
        vv = oracle.decode_values(vb[s][keep[s]], oracle.BF16)
        want = brute.attention(oracle.decode_values(q[s], oracle.BF16), kk, vv, SCALE)
        np.testing.assert_allclose(got[s], want, rtol=0, atol=1e-12)
