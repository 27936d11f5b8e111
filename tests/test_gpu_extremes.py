"""GPU: the decode at the limits of its launch shape, against the oracle.

  - 65,535 sequences, the most one launch takes (the work plan packs the
    sequence index in 16 bits), with short ragged contexts of 1-48 tokens,
    through the decode that writes each sequence's new K / V itself: pools
    bit-identical to reshape_and_cache's, every output row against the
    oracle;
  - one sequence of 262,144 tokens beside a one-token one: the default split
    cuts it into 512 partitions, so the reduce merges that many records per
    head (bf16 and fp8 pools);
  - a fresh 16,384-token prompt as one multi-token chunk (sampled rows).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pkv = pytest.importorskip("paged_kv_cache_51_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {oracle.BF16: 2e-2, oracle.FP16: 2e-2, oracle.FP8: 6e-2}


def log(*a):
    print(*a, flush=True)


def filled_pools(nb, Hkv, D, bs, kv, seed, scale):
    nbytes = pkv.layer_pool_bytes(nb, Hkv, D, bs, kv)
    kpool = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    vpool = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    workloads.device_fill_normal(kpool, kv, seed, scale=scale)
    workloads.device_fill_normal(vpool, kv, seed + 1, scale=scale)
    return kpool, vpool


def test_decode_append_65535_sequences():
    S, H, Hkv, D, bs, kv = 65535, 8, 2, 128, 16, oracle.BF16
    r = np.random.default_rng(65535)
    lengths = r.integers(1, 49, S).astype(np.int32)
    tabs = workloads.build_tables(lengths, bs, r)
    log(f"S={S} tokens={int(lengths.sum())} blocks={tabs.num_blocks}")
    kpool, vpool = filled_pools(tabs.num_blocks, Hkv, D, bs, kv, 31, 1.0)
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    q = torch.randn(S, H, D, generator=g, device=DEV).to(torch.bfloat16)
    newk = torch.randn(S, Hkv, D, generator=g, device=DEV).to(torch.bfloat16)
    newv = torch.randn(S, Hkv, D, generator=g, device=DEV).to(torch.bfloat16)
    bt, cl = torch.from_numpy(tabs.block_tables).to(DEV), torch.from_numpy(lengths).to(DEV)
    mc = int(lengths.max())
    scale = float(np.float32(1.0 / np.sqrt(D)))
    kref, vref = kpool.clone(), vpool.clone()
    pkv.reshape_and_cache(newk, newv, kref, vref, pkv.decode_slot_mapping(bt, cl, bs), bs,
                          tabs.num_blocks, kv)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode_append(out, q, newk, newv, kpool, vpool, bt, cl, mc, Hkv, bs, kv, scale,
                                      num_blocks=tabs.num_blocks)
    torch.cuda.synchronize()
    assert torch.equal(kpool, kref) and torch.equal(vpool, vref), "appended pools differ"
    del kref, vref
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    want = oracle.paged_decode(q.cpu().view(torch.int16).numpy().view(np.uint16), kv,
                               kpool.cpu().numpy(), vpool.cpu().numpy(), kv, tabs.block_tables,
                               lengths, Hkv, bs, scale)
    err = float(np.abs(got - want).max())
    log(f"  max-abs {err:.3e} over all {S} sequences")
    assert err <= TOL[kv]


@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
def test_decode_262144_token_sequence(kv):
    H, Hkv, D, bs = 8, 1, 128, 16
    lengths = np.array([262144, 1], np.int32)
    r = np.random.default_rng(7)
    tabs = workloads.build_tables(lengths, bs, r)
    ks = float(np.float32(8.0 / 448.0)) if kv == oracle.FP8 else 1.0
    kpool, vpool = filled_pools(tabs.num_blocks, Hkv, D, bs, kv, 41, ks)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    q = torch.randn(2, H, D, generator=g, device=DEV).to(torch.bfloat16)
    bt, cl = torch.from_numpy(tabs.block_tables).to(DEV), torch.from_numpy(lengths).to(DEV)
    mc = int(lengths.max())
    part = pkv.default_partition_tokens(2, Hkv, mc, bs)
    log(f"kv={kv}: one sequence of {mc} tokens, partitions of {part} tokens ({-(-mc // part)} of them)")
    assert -(-mc // part) >= 512
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode(out, q, kpool, vpool, bt, cl, mc, Hkv, bs, kv, scale, ks, ks,
                               num_blocks=tabs.num_blocks)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    want = oracle.paged_decode(q.cpu().view(torch.int16).numpy().view(np.uint16), oracle.BF16,
                               kpool.cpu().numpy(), vpool.cpu().numpy(), kv, tabs.block_tables,
                               lengths, Hkv, bs, scale, ks, ks)
    err = float(np.abs(got - want).max())
    log(f"  max-abs {err:.3e}")
    assert err <= TOL[kv]


@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
def test_fresh_prefill_of_16384_tokens(kv):
    """A whole 16,384-token prompt as one chunk (every token new, causal
    from position 0) beside a 3-token one: sampled rows against the oracle
    as one-token chunks at their positions."""
    H, Hkv, D, bs = 28, 4, 128, 16
    lengths = np.array([16384, 3], np.int32)
    q_lens = lengths.copy()
    r = np.random.default_rng(9)
    tabs = workloads.build_tables(lengths, bs, r)
    ks = float(np.float32(8.0 / 448.0)) if kv == oracle.FP8 else 1.0
    kpool, vpool = filled_pools(tabs.num_blocks, Hkv, D, bs, kv, 51, ks)
    T = int(q_lens.sum())
    g = torch.Generator(device=DEV)
    g.manual_seed(13)
    q = torch.randn(T, H, D, generator=g, device=DEV).to(torch.bfloat16)
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    out = torch.full_like(q, float("nan"))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    pkv.paged_attention_prefill(out, q, kpool, vpool, torch.from_numpy(tabs.block_tables).to(DEV),
                                torch.from_numpy(lengths).to(DEV), torch.from_numpy(qs).to(DEV),
                                int(q_lens.max()), int(lengths.max()), Hkv, bs, kv, scale, ks, ks,
                                num_blocks=tabs.num_blocks)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    rows = [(0, j) for j in (0, 1, 15, 16, 4097, 8191, 12000, 16382, 16383)] + [(1, 0), (1, 2)]
    log(f"kv={kv}: rows {rows}")
    qb = q.cpu().view(torch.int16).numpy().view(np.uint16)
    sub_q = qb[[qs[s] + j for s, j in rows]]
    sub_ctx = np.array([j + 1 for _, j in rows], np.int32)       # a fresh prompt: token j at position j
    sub_bt = np.ascontiguousarray(tabs.block_tables[[s for s, _ in rows]])
    want = oracle.paged_prefill(sub_q, oracle.BF16, kpool.cpu().numpy(), vpool.cpu().numpy(), kv, sub_bt,
                                sub_ctx, np.arange(len(rows) + 1, dtype=np.int32), Hkv, bs, scale, ks, ks)
    err = float(np.abs(got[[qs[s] + j for s, j in rows]] - want).max())
    log(f"  max-abs {err:.3e}")
    assert err <= TOL[kv]
