"""Seeded synthetic inputs for paged decode attention (shared by tests/bench).

This module only draws random numbers and lays out who owns which physical
block; it holds none of the attention, cache-write, slot or fp8 arithmetic.
Both the HIP path and the CPU oracle receive what it produces.

Workload shapes are five named configurations (the pages'
model shapes: Qwen2.5-1.5B/7B/72B from "LLM inference basics and vLLM
internals" §2's table, and the Llama-2-7B MHA shape from the vToken page's
"KV cache basics").  The pages measure on ShareGPT/Alpaca request traces that
are not available here; the length distributions below stand in for them.

Recipe (all seeded from numpy SeedSequence(seed).spawn(4): lengths,
physical-id permutation, sharing, values):
  - lengths: fixed list (tiny), lognormal(median, sigma=1) rounded and
    clipped, uniform integers, or constant;
  - physical ids: a random permutation of 1..num_blocks-1 (block 0 is the
    null block and is never handed out), consumed in sequence order; shared
    prefix blocks are drawn once and referenced by every member of the group;
  - num_blocks = 1 + ceil(1.1 * unique blocks in use)  (10% free);
  - values: N(0,1) drawn in fp32 and rounded to the storage dtype.
"""
from dataclasses import dataclass, field
import math

import numpy as np

BF16, FP16, FP8 = 0, 1, 2
DTYPE_NAMES = {BF16: "bf16", FP16: "fp16", FP8: "fp8"}


@dataclass
class Config:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: int
    q_dtype: int
    num_layers: int
    lengths: str                    # "fixed" | "lognormal" | "uniform" | "const"
    length_args: tuple
    share: str = "none"             # "none" | "prefix8" | "groups20"
    share_args: tuple = ()
    description: str = ""


CONFIGS = {
    "tiny": Config(
        "tiny", 4, 12, 2, 128, 16, BF16, BF16, 1, "fixed", (1, 17, 64, 200),
        description="Tiny paged decode, 1 layer: 4 seqs, context lens {1,17,64,200}, "
                    "12 q / 2 kv heads, d=128, bs=16, 64-block pool"),
    "qwen15b": Config(
        "qwen15b", 64, 12, 2, 128, 16, BF16, BF16, 1, "lognormal", (512, 1.0, 16, 4096),
        share="prefix8", share_args=(8, 256),
        description="Qwen2.5-1.5B shape, one layer: 64 seqs, 12 q / 2 kv heads, d=128, "
                    "bf16 KV, bs=16, lognormal lengths (median 512), 8 seqs share a "
                    "256-token prefix"),
    "qwen7b": Config(
        "qwen7b", 256, 28, 4, 128, 16, BF16, BF16, 28, "uniform", (1024, 8192),
        description="Qwen2.5-7B shape: 28 layers, 28 q / 4 kv heads, d=128, bf16 KV, "
                    "bs=16, batch 256, context U{1024..8192}"),
    "qwen72b": Config(
        "qwen72b", 32, 64, 8, 128, 16, FP8, BF16, 8, "const", (32768,),
        description="Qwen2.5-72B shape: 64 q / 8 kv heads, d=128, bs=16, batch 32 at "
                    "context 32768, 8 layers, fp8 e4m3 KV (bf16 variant too)"),
    "llama7b": Config(
        "llama7b", 128, 32, 32, 128, 16, FP16, FP16, 1, "lognormal", (2048, 1.0, 16, 4096),
        share="groups20", share_args=(16, 8, 0.2),
        description="Llama-2-7B-style MHA: 32 q / 32 kv heads, d=128, fp16 KV, bs=16 "
                    "(and 32), batch 128, lognormal lengths (median 2048, max 4096), "
                    "20% of logical blocks in group-shared prefixes"),
}


def streams(seed):
    """Four independent generators: lengths, permutation, sharing, values."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(4)]


def draw_lengths(cfg, rng):
    a = cfg.length_args
    if cfg.lengths == "fixed":
        return np.array(a, np.int32)
    if cfg.lengths == "lognormal":
        median, sigma, lo, hi = a
        x = rng.lognormal(mean=math.log(median), sigma=sigma, size=cfg.num_seqs)
        return np.clip(np.rint(x), lo, hi).astype(np.int32)
    if cfg.lengths == "uniform":
        lo, hi = a
        return rng.integers(lo, hi, size=cfg.num_seqs, endpoint=True).astype(np.int32)
    if cfg.lengths == "const":
        return np.full(cfg.num_seqs, a[0], np.int32)
    raise ValueError(cfg.lengths)


def _blocks_for(c, bs):
    return -(-int(c) // bs)


@dataclass
class Tables:
    block_tables: np.ndarray        # [S][max_blocks] int32, unused entries 0
    context_lens: np.ndarray        # [S] int32
    num_blocks: int                 # physical blocks incl. null block 0
    unique_blocks: int              # distinct physical blocks referenced
    shared_logical: int = 0         # logical table entries that point at shared blocks
    groups: list = field(default_factory=list)


def build_tables(lengths, block_size, perm_rng, share="none", share_args=(),
                 share_rng=None, num_blocks=None, extra_free=0.10):
    """Assign physical blocks to every logical block of every sequence.

    share="prefix8": share_args=(n, prefix_tokens): sequences 0..n-1 reference
      the same prefix_tokens/bs physical blocks first (their lengths are raised
      to at least prefix_tokens+1 so each keeps a private token).
    share="groups20": share_args=(groups, size, frac): consecutive groups of
      `size` sequences share floor(frac * mean blocks of the group) prefix
      blocks (capped so every member keeps a private token).
    """
    lengths = np.array(lengths, np.int32).copy()
    S = len(lengths)
    bs = block_size
    shared = {}          # seq -> (list key, count)
    groups = []
    if share == "prefix8":
        n, prefix = share_args
        lengths[:n] = np.maximum(lengths[:n], prefix + 1)
        groups.append((list(range(n)), prefix // bs))
    elif share == "groups20":
        ng, size, frac = share_args
        for gi in range(ng):
            members = list(range(gi * size, min(S, (gi + 1) * size)))
            if not members:
                break
            nb = [_blocks_for(lengths[s], bs) for s in members]
            k = int(math.floor(frac * float(np.mean(nb))))
            k = min(k, min((int(lengths[s]) - 1) // bs for s in members))
            if k > 0:
                groups.append((members, k))
    elif share != "none":
        raise ValueError(share)
    for gi, (members, k) in enumerate(groups):
        for s in members:
            shared[s] = (gi, k)

    need = [_blocks_for(c, bs) for c in lengths]
    unique = sum(need) - sum((len(m) - 1) * k for m, k in groups)
    if num_blocks is None:
        num_blocks = 1 + int(math.ceil((1.0 + extra_free) * unique))
    if num_blocks - 1 < unique:
        raise ValueError("pool too small for the requested lengths")
    ids = perm_rng.permutation(np.arange(1, num_blocks, dtype=np.int64)).astype(np.int32)
    pos = 0
    group_ids = {}
    for gi, (members, k) in enumerate(groups):
        group_ids[gi] = ids[pos:pos + k]
        pos += k
    max_blocks = max(max(need), 1)
    bt = np.zeros((S, max_blocks), np.int32)
    shared_logical = 0
    for s in range(S):
        j0 = 0
        if s in shared:
            gi, k = shared[s]
            bt[s, :k] = group_ids[gi]
            j0 = k
            shared_logical += k
        cnt = need[s] - j0
        bt[s, j0:need[s]] = ids[pos:pos + cnt]
        pos += cnt
    return Tables(bt, lengths, int(num_blocks), int(unique), shared_logical,
                  [(m, k) for m, k in groups])


def normal_bits(rng, shape, dtype):
    """N(0,1) values drawn in fp32, rounded to nearest even in bf16 / fp16,
    returned as raw uint16 bits."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bits(x, dtype)


def f32_to_bits(x, dtype):
    x = np.asarray(x, np.float32)
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def make(cfg_name, seed=0, block_size=None, num_seqs=None):
    """Lengths + block tables + q for a named configuration (host arrays).

    Pool contents are not drawn here (they are large); see fill_pool_* .
    """
    cfg = CONFIGS[cfg_name]
    bs = block_size or cfg.block_size
    r_len, r_perm, r_share, r_val = streams(seed)
    lengths = draw_lengths(cfg, r_len)
    if num_seqs is not None:
        lengths = lengths[:num_seqs]
    if cfg_name == "tiny":
        tables = build_tables(lengths, bs, r_perm, num_blocks=64)
    else:
        tables = build_tables(lengths, bs, r_perm, cfg.share, cfg.share_args, r_share)
    q = normal_bits(r_val, (len(lengths), cfg.num_heads, cfg.head_dim), cfg.q_dtype)
    return cfg, tables, q, r_val


def device_fill_normal(u8_tensor, dtype, seed, scale=1.0):
    """Fill a device byte buffer with N(0,1) values of `dtype`, drawn on the
    device with a seeded torch.Generator (fp8: N(0,1)/scale clamped to +-448
    and cast by torch's float8_e4m3fn conversion)."""
    import torch
    dev = u8_tensor.device
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    n_bytes = u8_tensor.numel()
    chunk = 1 << 28
    if dtype in (BF16, FP16):
        tdt = torch.bfloat16 if dtype == BF16 else torch.float16
        view = u8_tensor.view(tdt)
        for i in range(0, view.numel(), chunk):
            part = view[i:i + chunk]
            part.copy_(torch.randn(part.numel(), generator=g, device=dev,
                                   dtype=torch.float32).to(tdt))
    elif dtype == FP8:
        view = u8_tensor.view(torch.float8_e4m3fn)
        for i in range(0, n_bytes, chunk):
            part = view[i:i + chunk]
            x = torch.randn(part.numel(), generator=g, device=dev, dtype=torch.float32)
            part.copy_((x / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn))
    else:
        raise ValueError(dtype)
