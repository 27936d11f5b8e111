"""Test-side construction of paged pools through the CPU oracle.

Pools are NaN-filled, then every context token is written with the oracle's
reshape_and_cache, so only positions a correct decode may read are finite.
The HIP library is never used here: these are oracle-derived inputs.
"""
import numpy as np

import oracle

NAN_BYTES = {oracle.BF16: b"\xc0\x7f", oracle.FP16: b"\x00\x7e", oracle.FP8: b"\x7f"}


def nan_pool(num_blocks, kv_heads, head_dim, block_size, dtype):
    n = oracle.layer_pool_bytes(num_blocks, kv_heads, head_dim, block_size, dtype)
    pat = np.frombuffer(NAN_BYTES[dtype], np.uint8)
    return np.tile(pat, n // len(pat)).copy()


def all_slots(block_tables, context_lens, block_size):
    """(seq, position, slot) for every context token, via the oracle."""
    out = []
    for s, c in enumerate(context_lens):
        for p in range(int(c)):
            out.append((s, p, oracle.slot_of_position(block_tables[s], p, block_size)))
    return out


def write_contiguous(kbits, vbits, block_tables, context_lens, kv_heads, head_dim,
                     block_size, num_blocks, kv_dtype, src_dtype, k_scale=1.0,
                     v_scale=1.0, k_pool=None, v_pool=None):
    """kbits/vbits: list over sequences of [c][H_kv][d] uint16 raw bits.

    Returns (k_pool, v_pool) uint8 arrays with every token written.
    """
    if k_pool is None:
        k_pool = nan_pool(num_blocks, kv_heads, head_dim, block_size, kv_dtype)
    if v_pool is None:
        v_pool = nan_pool(num_blocks, kv_heads, head_dim, block_size, kv_dtype)
    trip = all_slots(block_tables, context_lens, block_size)
    if not trip:
        return k_pool, v_pool
    key = np.stack([kbits[s][p] for s, p, _ in trip])
    val = np.stack([vbits[s][p] for s, p, _ in trip])
    slots = np.array([sl for _, _, sl in trip], np.int64)
    return oracle.reshape_and_cache(key, val, src_dtype, k_pool, v_pool, slots,
                                    block_size, num_blocks, kv_dtype, k_scale, v_scale)


def gather_values(pool, block_tables, context_lens, s, kv_heads, head_dim, block_size,
                  dtype, is_value, scale=1.0):
    """fp64 [c][H_kv][d] values of sequence s read back through the table."""
    c = int(context_lens[s])
    tab = oracle.e4m3_table() if dtype == oracle.FP8 else None
    out = np.zeros((c, kv_heads, head_dim))
    for p in range(c):
        pb = int(block_tables[s][p // block_size])
        for g in range(kv_heads):
            for k in range(head_dim):
                off = oracle.pool_offset(pb, g, p % block_size, k, is_value, kv_heads,
                                         head_dim, block_size, dtype)
                if dtype == oracle.FP8:
                    out[p, g, k] = tab[pool[off]] * scale
                else:
                    bits = int(pool[off]) | (int(pool[off + 1]) << 8)
                    out[p, g, k] = (oracle.bf16_value(bits) if dtype == oracle.BF16
                                    else oracle.fp16_value(bits))
    return out
