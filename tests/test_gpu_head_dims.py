"""GPU parity at head_dim 64 and 256: reshape_and_cache bit-exact (whole
pool) and paged decode within 2e-2 (bf16 / fp16 KV) / 6e-2 (fp8 KV) of the
CPU oracle, across group sizes, block sizes, split and unsplit contexts and
both decode forms (grid and persistent); c = 1 returns V_0 exactly ("LLM
inference basics and vLLM internals" §2 / §4)."""
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


def case(d, lengths, H, Hkv, bs, kv, seed):
    src = oracle.FP16 if kv == oracle.FP16 else oracle.BF16
    ks = float(np.float32(4.0 / 448.0)) if kv == oracle.FP8 else 1.0
    _, r_perm, _, r_val = workloads.streams(seed)
    tabs = workloads.build_tables(lengths, bs, r_perm)
    kb = [workloads.normal_bits(r_val, (int(c), Hkv, d), src) for c in lengths]
    vb = [workloads.normal_bits(r_val, (int(c), Hkv, d), src) for c in lengths]
    q = workloads.normal_bits(r_val, (len(lengths), H, d), src)
    kp, vp = pools.write_contiguous(kb, vb, tabs.block_tables, tabs.context_lens, Hkv, d, bs,
                                    tabs.num_blocks, kv, src, ks, ks)
    return src, ks, tabs, q, kp, vp


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("kv,bs", [(oracle.BF16, 16), (oracle.FP8, 16), (oracle.FP16, 32)])
def test_reshape_and_cache_bit_exact(d, kv, bs):
    log(f"reshape_and_cache d={d} kv={kv} bs={bs}")
    src = oracle.FP16 if kv == oracle.FP16 else oracle.BF16
    Hkv, T, nb = 4, 37, 24
    r = np.random.default_rng(d + kv)
    key = workloads.normal_bits(r, (T, Hkv, d), src)
    val = workloads.normal_bits(r, (T, Hkv, d), src)
    slots = r.permutation(np.arange(bs, nb * bs))[:T].astype(np.int64)
    slots[3] = -1                                   # padding token: skipped
    ks = float(np.float32(0.011)) if kv == oracle.FP8 else 1.0
    base = pools.nan_pool(nb, Hkv, d, bs, kv)
    want_k, want_v = oracle.reshape_and_cache(key, val, src, base, base, slots, bs, nb, kv, ks, ks)
    kd = torch.from_numpy(base.copy()).to(DEV)
    vd = torch.from_numpy(base.copy()).to(DEV)
    pkv.reshape_and_cache(dev16(key, src), dev16(val, src), kd, vd, devi(slots), bs, nb, kv, ks, ks)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().numpy(), want_k)
    assert np.array_equal(vd.cpu().numpy(), want_v)


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("kv,bs", [(oracle.BF16, 16), (oracle.FP8, 16), (oracle.FP16, 32), (oracle.BF16, 32)])
@pytest.mark.parametrize("H,Hkv", [(8, 8), (16, 4), (24, 2)])
@pytest.mark.parametrize("part,impl", [(0, 0), (64, 0), (32, 3), (4096, 0)])
def test_decode_matches_oracle(d, kv, bs, H, Hkv, part, impl):
    if part and part % bs:
        pytest.skip("partition must be a multiple of the block size")
    log(f"decode d={d} kv={kv} bs={bs} H={H}/{Hkv} part={part} impl={impl}")
    lengths = [1, 5, 16, 33, 100, 257, 640]
    src, ks, tabs, qb, kp, vp = case(d, lengths, H, Hkv, bs, kv, seed=d + H)
    q = dev16(qb, src)
    out = torch.full_like(q, float("nan"))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    pkv.paged_attention_decode(out, q, torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV),
                               devi(tabs.block_tables), devi(tabs.context_lens), int(max(lengths)), Hkv,
                               bs, kv, scale, ks, ks, partition_tokens=part, impl=impl,
                               num_blocks=tabs.num_blocks)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want = oracle.paged_decode(qb, src, kp, vp, kv, tabs.block_tables, tabs.context_lens, Hkv, bs,
                               scale, ks, ks)
    err = float(np.abs(got - want).max())
    log(f"  max-abs {err:.3e}")
    assert np.isfinite(got).all() and err <= TOL[kv]
    # c = 1: the output is V_0 rounded to the query dtype, exactly
    v0 = pools.gather_values(vp, tabs.block_tables, tabs.context_lens, 0, Hkv, d, bs, kv, 1, ks)[0]
    want0 = np.repeat(v0, H // Hkv, axis=0)
    if kv != oracle.FP8:
        assert np.array_equal(got[0], want0)         # 16-bit V_0 is representable
    else:
        assert np.abs(got[0] - want0).max() <= TOL[kv]


def test_unsupported_head_dims_rejected():
    q = torch.zeros(1, 2, 96, dtype=torch.bfloat16, device=DEV)
    pool = torch.zeros(pkv.layer_pool_bytes(4, 1, 128, 16, pkv.BF16), dtype=torch.uint8, device=DEV)
    with pytest.raises(Exception):
        pkv.paged_attention_decode(torch.empty_like(q), q, pool, pool, devi([[1]]), devi([1]), 1, 1, 16,
                                   pkv.BF16, 0.1, num_blocks=4)
