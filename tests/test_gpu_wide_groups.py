"""GPU: more than 16 query heads per kv head, MQA included ("LLM inference
basics and vLLM internals" §2: in MQA every query head shares the one K / V
head; GQA groups them).

A kv head whose group does not fit the columns of one work entry (decode:
two 16-column MFMA tiles at head_dim <= 128, one at 256; the multi-token and
token-table kernels: one) runs as several entry heads, all reading the same
K / V (the last one may hold fewer heads).  Checked here: decode (grid and persistent,
split and unsplit contexts, bf16 / fp8, head_dim 64 / 128 / 256), the decode
with the new token's K / V written inside it, the token-table decode and the
multi-token kernels against the oracle; and, bit for bit, that MQA equals
GQA with replicated K / V where both run the same entries.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import pools

pkv = pytest.importorskip("paged_kv_cache_51_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {oracle.BF16: 2e-2, oracle.FP16: 2e-2, oracle.FP8: 6e-2}


def log(*a):
    print(*a, flush=True)


def dev16(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == oracle.BF16 else torch.float16).to(DEV)


def devi(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def dev8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def values(lengths, H, Hkv, d, src, seed):
    _, r_perm, _, r_val = workloads.streams(seed)
    kb = [workloads.normal_bits(r_val, (int(c), Hkv, d), src) for c in lengths]
    vb = [workloads.normal_bits(r_val, (int(c), Hkv, d), src) for c in lengths]
    q = workloads.normal_bits(r_val, (len(lengths), H, d), src)
    return r_perm, kb, vb, q


def check(got, want, kv, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = float(np.abs(got - want).max())
    log(f"  {what}: max-abs {err:.3e}")
    assert err <= TOL[kv], what


def out_np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("H,Hkv,d", [(32, 1, 128), (28, 1, 128), (40, 2, 128), (17, 1, 128),
                                     (48, 1, 128), (128, 2, 128), (71, 1, 64), (64, 1, 256)])
@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
def test_decode_wide_groups_match_oracle(H, Hkv, d, kv):
    log(f"decode H={H} Hkv={Hkv} d={d} kv={kv}")
    src = oracle.BF16
    ks = float(np.float32(4.0 / 448.0)) if kv == oracle.FP8 else 1.0
    lengths = [1, 17, 64, 200, 333, 2100]
    r_perm, kb, vb, qb = values(lengths, H, Hkv, d, src, H + d)
    tabs = workloads.build_tables(lengths, 16, r_perm)
    kp, vp = pools.write_contiguous(kb, vb, tabs.block_tables, tabs.context_lens, Hkv, d, 16,
                                    tabs.num_blocks, kv, src, ks, ks)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    want = oracle.paged_decode(qb, src, kp, vp, kv, tabs.block_tables, tabs.context_lens, Hkv, 16,
                               scale, ks, ks)
    kd, vd, bt, cl = dev8(kp), dev8(vp), devi(tabs.block_tables), devi(tabs.context_lens)
    q = dev16(qb, src)
    for part, impl in [(0, pkv.IMPL_AUTO), (64, pkv.IMPL_AUTO), (64, pkv.IMPL_MFMA_PERSISTENT),
                       (2048, pkv.IMPL_AUTO), (2048, pkv.IMPL_MFMA)]:
        out = torch.full_like(q, float("nan"))
        pkv.paged_attention_decode(out, q, kd, vd, bt, cl, max(lengths), Hkv, 16, kv, scale, ks, ks,
                                   partition_tokens=part, impl=impl, num_blocks=tabs.num_blocks)
        torch.cuda.synchronize()
        got = out_np(out)
        check(got, want, kv, f"part={part} impl={impl}")
    # c = 1: every head returns V_0 of its kv head (exactly for a 16-bit pool)
    v0 = pools.gather_values(vp, tabs.block_tables, tabs.context_lens, 0, Hkv, d, 16, kv, 1, ks)[0]
    want0 = np.repeat(v0, H // Hkv, axis=0)
    if kv != oracle.FP8:
        assert np.array_equal(got[0], want0)
    else:
        assert np.abs(got[0] - want0).max() <= TOL[kv]


@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
@pytest.mark.parametrize("part", [0, 64])
def test_mqa_equals_gqa_with_replicated_kv_bitwise(kv, part):
    """Entries over the same K / V values compute the same bits wherever the
    values sit.  Decode takes up to 32 query heads per entry at head_dim
    128: MQA with 32 query heads (one 32-column entry) equals each half of
    GQA with 64 query heads over 2 kv heads holding the same K / V (two
    such entries).  The token-table and multi-token kernels take 16 per
    entry: MQA with 32 query heads (two entries) equals GQA with 2 kv
    heads and 32 query heads (two entries)."""
    log(f"MQA vs replicated GQA kv={kv} part={part}")
    src, H, d, bs = oracle.BF16, 32, 128, 16
    ks = float(np.float32(4.0 / 448.0)) if kv == oracle.FP8 else 1.0
    lengths = [1, 30, 64, 500, 1200]
    r_perm, kb, vb, qb = values(lengths, H, 1, d, src, 11)
    tabs = workloads.build_tables(lengths, bs, r_perm)
    rep = lambda xs: [np.repeat(x, 2, axis=1) for x in xs]          # [c][2][d]
    outs = {}
    for Hkv, k_, v_ in [(1, kb, vb), (2, rep(kb), rep(vb))]:
        kp, vp = pools.write_contiguous(k_, v_, tabs.block_tables, tabs.context_lens, Hkv, d, bs,
                                        tabs.num_blocks, kv, src, ks, ks)
        kd, vd, bt, cl = dev8(kp), dev8(vp), devi(tabs.block_tables), devi(tabs.context_lens)
        q = dev16(qb, src)
        # decode: the 32 heads once (MQA), or twice over the two kv heads
        qq = q if Hkv == 1 else torch.cat([q, q], dim=1).contiguous()
        a = torch.full_like(qq, float("nan"))
        pkv.paged_attention_decode(a, qq, kd, vd, bt, cl, max(lengths), Hkv, bs, kv, 0.09, ks, ks,
                                   partition_tokens=part or 2048, num_blocks=tabs.num_blocks)
        if Hkv == 2:
            torch.cuda.synchronize()
            assert torch.equal(a[:, :H].view(torch.int16), a[:, H:].view(torch.int16))
            a = a[:, :H].contiguous()
        slots = np.zeros((len(lengths), max(lengths)), np.int32)
        for s, c in enumerate(lengths):
            slots[s, :c] = [tabs.block_tables[s][t // bs] * bs + t % bs for t in range(c)]
        b = torch.full_like(q, float("nan"))
        pkv.paged_attention_decode_tokens(b, q, kd, vd, devi(slots), cl, Hkv, bs, tabs.num_blocks,
                                          kv, 0.09, ks, ks)
        # the last 40 tokens of each sequence as one chunk (the first as all of its one)
        ql = np.minimum(np.array(lengths), 40)
        qs = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        qp = dev16(workloads.normal_bits(np.random.default_rng(3), (int(qs[-1]), H, d), src), src)
        c_ = torch.full_like(qp, float("nan"))
        pkv.paged_attention_prefill(c_, qp, kd, vd, bt, cl, devi(qs), int(ql.max()), max(lengths),
                                    Hkv, bs, kv, 0.09, ks, ks, num_blocks=tabs.num_blocks)
        torch.cuda.synchronize()
        outs[Hkv] = [t.view(torch.int16).cpu().numpy() for t in (a, b, c_)]
    for name, x, y in zip(("decode", "token table", "multi-token"), outs[1], outs[2]):
        assert np.array_equal(x, y), f"{name}: MQA differs from replicated GQA"


@pytest.mark.parametrize("H,Hkv", [(32, 1), (71, 1)])
@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
def test_decode_append_wide_groups(H, Hkv, kv):
    """Every entry head of a split kv head writes the same new K / V row:
    pools and outputs equal reshape_and_cache followed by the decode."""
    d = 64 if H == 71 else 128
    log(f"decode_append H={H} Hkv={Hkv} d={d} kv={kv}")
    src, bs = oracle.BF16, 16
    ks = float(np.float32(4.0 / 448.0)) if kv == oracle.FP8 else 1.0
    lengths = [1, 16, 17, 300, 1500]
    r_perm, kb, vb, qb = values(lengths, H, Hkv, d, src, 21)
    tabs = workloads.build_tables(lengths, bs, r_perm)
    hist = np.maximum(np.array(lengths) - 1, 0).astype(np.int32)
    kp, vp = pools.write_contiguous([k[:-1] for k in kb], [v[:-1] for v in vb], tabs.block_tables,
                                    hist, Hkv, d, bs, tabs.num_blocks, kv, src, ks, ks)
    newk = np.stack([k[-1] for k in kb])
    newv = np.stack([v[-1] for v in vb])
    scale = float(np.float32(1.0 / np.sqrt(d)))
    bt, cl = devi(tabs.block_tables), devi(tabs.context_lens)
    q = dev16(qb, src)
    res = []
    for fused in (False, True):
        kd, vd = dev8(kp), dev8(vp)
        out = torch.full_like(q, float("nan"))
        if fused:
            pkv.paged_attention_decode_append(out, q, dev16(newk, src), dev16(newv, src), kd, vd, bt,
                                              cl, max(lengths), Hkv, bs, kv, scale, ks, ks,
                                              partition_tokens=512, num_blocks=tabs.num_blocks)
        else:
            sl = pkv.decode_slot_mapping(bt, cl, bs)
            pkv.reshape_and_cache(dev16(newk, src), dev16(newv, src), kd, vd, sl, bs, tabs.num_blocks,
                                  kv, ks, ks)
            pkv.paged_attention_decode(out, q, kd, vd, bt, cl, max(lengths), Hkv, bs, kv, scale, ks, ks,
                                       partition_tokens=512, num_blocks=tabs.num_blocks)
        torch.cuda.synchronize()
        res.append((out.view(torch.int16).cpu().numpy(), kd.cpu().numpy(), vd.cpu().numpy()))
    assert np.array_equal(res[0][1], res[1][1]) and np.array_equal(res[0][2], res[1][2])
    assert np.array_equal(res[0][0], res[1][0])
    want = oracle.paged_decode(qb, src, res[1][1], res[1][2], kv, tabs.block_tables,
                               tabs.context_lens, Hkv, bs, scale, ks, ks)
    got = res[1][0].view(np.uint16)
    check(oracle.decode_values(got, src), want, kv, "fused append")


@pytest.mark.parametrize("H,Hkv", [(32, 1), (40, 2), (17, 1)])
@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
def test_decode_tokens_wide_groups(H, Hkv, kv):
    log(f"token-table decode H={H} Hkv={Hkv} kv={kv}")
    src, d, bs = oracle.BF16, 128, 16
    ks = float(np.float32(4.0 / 448.0)) if kv == oracle.FP8 else 1.0
    lengths = [1, 17, 64, 200, 333]
    r_perm, kb, vb, qb = values(lengths, H, Hkv, d, src, 31)
    tabs = workloads.build_tables(lengths, bs, r_perm)
    kp, vp = pools.write_contiguous(kb, vb, tabs.block_tables, tabs.context_lens, Hkv, d, bs,
                                    tabs.num_blocks, kv, src, ks, ks)
    r = np.random.default_rng(7)
    slots = np.zeros((len(lengths), max(lengths)), np.int32)
    ctx = np.zeros(len(lengths), np.int32)
    for s, c in enumerate(lengths):
        keep = [t for t in range(c) if r.random() < 0.6] or [c - 1]
        slots[s, :len(keep)] = [tabs.block_tables[s][t // bs] * bs + t % bs for t in keep]
        ctx[s] = len(keep)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    want = oracle.paged_decode_tokens(qb, src, kp, vp, kv, slots, ctx, Hkv, bs, scale, ks, ks)
    q = dev16(qb, src)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode_tokens(out, q, dev8(kp), dev8(vp), devi(slots), devi(ctx), Hkv, bs,
                                      tabs.num_blocks, kv, scale, ks, ks)
    torch.cuda.synchronize()
    check(out_np(out), want, kv, "token table")


@pytest.mark.parametrize("H,Hkv", [(32, 1), (40, 2), (17, 1)])
@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
def test_prefill_wide_groups(H, Hkv, kv):
    """Both multi-token forms: chunks of 1-4 tokens (at most four 16-column
    tiles per entry head) and longer ones (the staged form)."""
    log(f"multi-token H={H} Hkv={Hkv} kv={kv}")
    src, d, bs = oracle.BF16, 128, 16
    ks = float(np.float32(4.0 / 448.0)) if kv == oracle.FP8 else 1.0
    for lengths, q_lens in [([5, 40, 300], [1, 3, 4]), ([5, 40, 300, 700], [5, 17, 64, 130])]:
        r_perm, kb, vb, _ = values(lengths, H, Hkv, d, src, 41 + len(q_lens))
        tabs = workloads.build_tables(lengths, bs, r_perm)
        kp, vp = pools.write_contiguous(kb, vb, tabs.block_tables, tabs.context_lens, Hkv, d, bs,
                                        tabs.num_blocks, kv, src, ks, ks)
        qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        qb = workloads.normal_bits(np.random.default_rng(9), (int(qs[-1]), H, d), src)
        scale = float(np.float32(1.0 / np.sqrt(d)))
        want = oracle.paged_prefill(qb, src, kp, vp, kv, tabs.block_tables, tabs.context_lens, qs,
                                    Hkv, bs, scale, ks, ks)
        q = dev16(qb, src)
        out = torch.full_like(q, float("nan"))
        pkv.paged_attention_prefill(out, q, dev8(kp), dev8(vp), devi(tabs.block_tables),
                                    devi(tabs.context_lens), devi(qs), int(max(q_lens)),
                                    max(lengths), Hkv, bs, kv, scale, ks, ks,
                                    num_blocks=tabs.num_blocks)
        torch.cuda.synchronize()
        check(out_np(out), want, kv, f"q_lens={q_lens}")
