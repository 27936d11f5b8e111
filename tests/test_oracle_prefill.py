"""Pins of the oracle's multi-token (causal) paged attention.

The tokens of a prefill chunk, or those left to compute after a prefix-cache
hit ("LLM inference basics and vLLM internals" §5, §6), are the last q_len
tokens of their sequence and attend to every earlier token and themselves.
Pinned to:
  - the contiguous textbook attention of oracle/brute.py, token by token
    over its visible keys (K/V drawn contiguous, scattered into the pool);
  - q_len = 1 everywhere: exactly the oracle's decode (a separate code path);
  - closed forms: the first token of a fresh prefill sees only key 0, so
    its output is V_0; tokens placed before the context start are zero;
  - causality: changing keys after a token's position leaves its output
    unchanged.
"""
import numpy as np
import pytest

import oracle
from oracle import brute
import workloads
from tests import pools
from tests.test_oracle_attention import _setup, _values

D = 128
SCALE = float(np.float32(1 / np.sqrt(D)))


def _chunks(q_lens, H, src_dtype, seed):
    r = np.random.default_rng(seed)
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = workloads.normal_bits(r, (int(qs[-1]), H, D), src_dtype)
    return qs, q


@pytest.mark.parametrize("kv_dtype,src_dtype,bs", [
    (oracle.BF16, oracle.BF16, 16), (oracle.FP16, oracle.FP16, 32), (oracle.FP8, oracle.BF16, 16),
])
def test_matches_contiguous_causal_brute_force(kv_dtype, src_dtype, bs):
    lengths = [5, 17, 64, 130]
    q_lens = [5, 3, 20, 7]                      # the first sequence is a fresh prefill
    H, Hkv = 12, 2
    ks, vs = (0.02, 0.03) if kv_dtype == oracle.FP8 else (1.0, 1.0)
    tabs, kb, vb, _, kp, vp = _setup(lengths, H, Hkv, bs, kv_dtype, src_dtype,
                                     num_blocks=64 if bs == 16 else 40, k_scale=ks, v_scale=vs)
    qs, q = _chunks(q_lens, H, src_dtype, 5)
    got = oracle.paged_prefill(q, src_dtype, kp, vp, kv_dtype, tabs.block_tables,
                               tabs.context_lens, qs, Hkv, bs, SCALE, ks, vs)
    for s in range(len(lengths)):
        qd = oracle.decode_values(q[qs[s]:qs[s + 1]], src_dtype)
        want = brute.causal_chunk(qd, _values(kb[s], src_dtype, kv_dtype, ks),
                                  _values(vb[s], src_dtype, kv_dtype, vs), SCALE)
        np.testing.assert_allclose(got[qs[s]:qs[s + 1]], want, rtol=0, atol=1e-12)
    assert np.isfinite(got).all()


def test_single_token_chunks_equal_decode():
    lengths = [1, 16, 33, 90]
    H, Hkv = 8, 2
    tabs, kb, vb, q, kp, vp = _setup(lengths, H, Hkv, 16, oracle.BF16, oracle.BF16, seed=3)
    qs = np.arange(len(lengths) + 1, dtype=np.int32)
    got = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                               tabs.context_lens, qs, Hkv, 16, SCALE)
    want = oracle.paged_decode(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                               tabs.context_lens, Hkv, 16, SCALE)
    assert np.array_equal(got, want)


def test_first_token_of_fresh_prefill_is_v0_and_early_tokens_are_zero():
    lengths = [24, 3]
    H, Hkv = 4, 2
    tabs, kb, vb, _, kp, vp = _setup(lengths, H, Hkv, 16, oracle.BF16, oracle.BF16, seed=9)
    q_lens = [24, 5]                             # the second: 2 tokens before the context start
    qs, q = _chunks(q_lens, H, oracle.BF16, 1)
    got = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                               tabs.context_lens, qs, Hkv, 16, SCALE)
    v0 = oracle.decode_values(vb[0][0], oracle.BF16)          # [H_kv][d]
    for h in range(H):
        assert np.array_equal(got[0, h], v0[h // (H // Hkv)])
    assert np.array_equal(got[qs[1]:qs[1] + 2], np.zeros((2, H, D)))
    v1 = oracle.decode_values(vb[1][0], oracle.BF16)
    for h in range(H):
        assert np.array_equal(got[qs[1] + 2, h], v1[h // (H // Hkv)])


def test_later_keys_do_not_change_earlier_tokens():
    lengths = [40]
    H, Hkv = 4, 1
    tabs, kb, vb, _, kp, vp = _setup(lengths, H, Hkv, 16, oracle.BF16, oracle.BF16, seed=4)
    qs, q = _chunks([12], H, oracle.BF16, 2)
    a = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                             tabs.context_lens, qs, Hkv, 16, SCALE)
    # overwrite the K/V of the last 6 positions (34..39) with other values
    r = np.random.default_rng(8)
    kb2 = [kb[0].copy()]
    vb2 = [vb[0].copy()]
    kb2[0][34:] = workloads.normal_bits(r, (6, Hkv, D), oracle.BF16)
    vb2[0][34:] = workloads.normal_bits(r, (6, Hkv, D), oracle.BF16)
    kp2, vp2 = pools.write_contiguous(kb2, vb2, tabs.block_tables, tabs.context_lens, Hkv, D,
                                      16, tabs.num_blocks, oracle.BF16, oracle.BF16)
    b = oracle.paged_prefill(q, oracle.BF16, kp2, vp2, oracle.BF16, tabs.block_tables,
                             tabs.context_lens, qs, Hkv, 16, SCALE)
    # chunk tokens sit at positions 28..39: those before 34 are unchanged
    assert np.array_equal(a[:6], b[:6])
    assert not np.array_equal(a[6:], b[6:])


@pytest.mark.parametrize("H,Hkv", [(32, 1), (40, 2)])
def test_mqa_and_wide_groups_match_causal_brute_force(H, Hkv):
    """Multi-token attention with one kv head for all query heads (MQA) or
    more than 16 query heads per kv head ("LLM inference basics and vLLM
    internals" §2)."""
    lengths = [5, 40, 100]
    q_lens = [5, 9, 33]
    tabs, kb, vb, _, kp, vp = _setup(lengths, H, Hkv, 16, oracle.BF16, oracle.BF16, seed=H + 1)
    qs, q = _chunks(q_lens, H, oracle.BF16, 6)
    got = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                               tabs.context_lens, qs, Hkv, 16, SCALE)
    for s in range(len(lengths)):
        qd = oracle.decode_values(q[qs[s]:qs[s + 1]], oracle.BF16)
        want = brute.causal_chunk(qd, oracle.decode_values(kb[s], oracle.BF16),
                                  oracle.decode_values(vb[s], oracle.BF16), SCALE)
        np.testing.assert_allclose(got[qs[s]:qs[s + 1]], want, rtol=0, atol=1e-12)
