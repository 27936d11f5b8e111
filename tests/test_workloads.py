"""Invariants of the seeded input generators (host only).

Block-table structure follows "LLM inference basics and vLLM internals" §4
(block 0 reserved as the null block; blocks assigned one per 16 tokens;
only the last block of a request wastes slots) and "vLLM internals (2)",
"Block table" (waste at most block_size - 1 per request; no external
fragmentation since every block has the same size).
"""
import numpy as np
import pytest

import workloads


@pytest.mark.parametrize("name", ["tiny", "qwen15b", "qwen7b", "qwen72b", "llama7b"])
def test_tables_are_valid(name):
    cfg, tabs, q, _ = workloads.make(name, seed=0)
    bs = cfg.block_size
    bt, ctx = tabs.block_tables, tabs.context_lens
    assert q.shape == (cfg.num_seqs, cfg.num_heads, cfg.head_dim)
    need = -(-ctx // bs)
    used = np.concatenate([bt[s, :need[s]] for s in range(len(ctx))])
    assert used.min() >= 1 and used.max() < tabs.num_blocks       # null block never used
    # only shared-prefix blocks are referenced more than once
    uniq, counts = np.unique(used, return_counts=True)
    assert len(uniq) == tabs.unique_blocks
    shared_refs = int((counts - 1).sum())
    assert shared_refs == sum((len(m) - 1) * k for m, k in tabs.groups)
    # waste per request <= bs - 1
    assert ((need * bs - ctx) <= bs - 1).all()
    # entries past the context are the null block
    for s in range(len(ctx)):
        assert (bt[s, need[s]:] == 0).all()
    if name != "tiny":
        assert tabs.num_blocks == 1 + int(np.ceil(1.1 * tabs.unique_blocks))


def test_config_specifics():
    cfg, tabs, _, _ = workloads.make("tiny")
    assert list(tabs.context_lens) == [1, 17, 64, 200] and tabs.num_blocks == 64
    cfg, tabs, _, _ = workloads.make("qwen7b")
    assert tabs.context_lens.min() >= 1024 and tabs.context_lens.max() <= 8192
    cfg, tabs, _, _ = workloads.make("qwen15b")
    m, k = tabs.groups[0]
    assert m == list(range(8)) and k == 16
    assert (tabs.block_tables[:8, :16] == tabs.block_tables[0, :16]).all()
    assert (tabs.context_lens[:8] >= 257).all()
    cfg, tabs, _, _ = workloads.make("llama7b")
    frac = tabs.shared_logical / float((-(-tabs.context_lens // 16)).sum())
    assert 0.15 <= frac <= 0.21
    cfg, tabs, _, _ = workloads.make("qwen72b")
    assert (tabs.context_lens == 32768).all() and tabs.block_tables.shape == (32, 2048)


def test_seeded_determinism():
    a = workloads.make("qwen15b", seed=3)
    b = workloads.make("qwen15b", seed=3)
    assert np.array_equal(a[1].block_tables, b[1].block_tables)
    assert np.array_equal(a[2], b[2])


def test_unique_kv_tokens_counts_shared_prefix_blocks_once():
    """bench.py's unique-byte numerator: on the 1.5B workload the first 8
    sequences share one 256-token prefix, so the distinct slots read are the
    logical tokens less 7 x 256; without sharing they equal the logical
    tokens; on the grouped-prefix workload every shared block is full, so
    the distinct slots are the logical ones less (refs - 1) x block_size per
    shared block."""
    import bench
    cfg, tabs, _, _ = workloads.make("qwen15b", seed=0)
    ctx = tabs.context_lens
    assert bench.unique_kv_tokens(tabs.block_tables, ctx, cfg.block_size, tabs.num_blocks) == \
        int(ctx.sum()) - 7 * 256
    cfg, tabs, _, _ = workloads.make("qwen7b", seed=0)
    assert bench.unique_kv_tokens(tabs.block_tables, tabs.context_lens, cfg.block_size,
                                  tabs.num_blocks) == int(tabs.context_lens.sum())
    cfg, tabs, _, _ = workloads.make("llama7b", seed=0)
    bs = cfg.block_size
    saved = sum((len(m) - 1) * k * bs for m, k in tabs.groups)
    assert saved > 0
    assert bench.unique_kv_tokens(tabs.block_tables, tabs.context_lens, bs, tabs.num_blocks) == \
        int(tabs.context_lens.sum()) - saved
