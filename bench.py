#!/usr/bin/env python3
"""Paged decode attention throughput on one MI355X.

A step is one decode step of the whole path for every layer of the
workload: decode slot mapping (once, tables are shared by all layers), then
per layer reshape_and_cache of the batch's new tokens, the partition kernel
and the partition merge.  Inputs are synthetic and resident in HBM before
timing starts (workloads/: seeded lengths and block tables, N(0,1) values).

Output: one JSON line.  `value` is achieved GB/s of algorithmic bytes per
step over step time; bytes per layer = sum_s c_s*2*H_kv*d*b_kv (KV read)
+ S*H*d*(b_q + b_out) (query read, output write) + S*H_kv*d*2*(b_src + b_kv)
(new-token K/V read and written).  `roofline` covers the partition kernel,
timed with HIP events on its launch stream inside the timed region.
`cpu_baseline` times the CPU oracle on a bounded sample of layer 0.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X published HBM3E bandwidth
ROTATE_BYTES = 1 << 30  # K/V read between two uses of one pool copy (>> 256 MB cache)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="qwen7b",
                    choices=["tiny", "qwen15b", "qwen7b", "qwen72b", "llama7b"])
    ap.add_argument("--kv-dtype", default=None, choices=[None, "bf16", "fp16", "fp8"])
    ap.add_argument("--block-size", type=int, default=None, choices=[None, 16, 32])
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--event-every", type=int, default=4,
                    help="decode: HIP events around each launch in every N-th timed step")
    ap.add_argument("--separate-cache-write", action="store_true",
                    help="decode: write the new tokens with reshape_and_cache in a launch of "
                         "their own before each decode launch (default: the decode launch "
                         "writes them, paged_attention_decode_append)")
    ap.add_argument("--head-dim", type=int, default=0, choices=[0, 64, 128, 256],
                    help="decode: override the configuration's head_dim (0 = as configured)")
    ap.add_argument("--heads", type=int, default=0,
                    help="decode: override the query heads (0 = as configured)")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="decode: override the kv heads (0 = as configured; 1 = MQA)")
    ap.add_argument("--impl", default="auto", choices=["auto", "mfma", "vector", "persistent"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (0 disables)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    ap.add_argument("--keep", type=float, default=0.5,
                    help="vtoken: fraction of context tokens an eviction keeps")
    ap.add_argument("--op", default="decode", choices=["decode", "copy_blocks", "prefill", "vtoken"],
                    help="decode: the attention step (default); copy_blocks: copy-on-write "
                         "block copies over the same pool shape; prefill: multi-token causal "
                         "attention (the last --q-len tokens of each sequence are new); vtoken: "
                         "decode through a fragmented token table, repack moves, decode after")
    ap.add_argument("--q-len", type=int, default=512, help="prefill: new tokens per sequence")
    ap.add_argument("--num-seqs", type=int, default=0,
                    help="prefill: sequences (default 16, or the workload's batch if --q-len <= 16)")
    ap.add_argument("--copy-pairs", type=int, default=2048,
                    help="copy_blocks: (src, dst) block pairs per call")
    args = ap.parse_args()
    if args.event_every < 1:
        raise SystemExit("--event-every must be >= 1")
    return args


DECODE_SOURCES = ("decode_core.h", "mfma_math.h", "decode.hip", "pkv_device.h", "cache_write.h")
PREFILL_SOURCES = ("prefill.hip", "decode_core.h", "mfma_math.h", "pkv_device.h", "cache_write.h")
VTOKEN_SOURCES = ("decode_tokens.hip", "decode_core.h", "mfma_math.h", "pkv_device.h")


def kernel_source_hash(files=DECODE_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_cache_51_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config_key, table="decode_traffic.json", files=DECODE_SOURCES):
    """HBM traffic per launch from committed rocprofv3 counter runs, only if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", table)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(config_key)
    if not rec or rec.get("kernel_hash") != kernel_source_hash(files):
        return None
    return rec.get("bytes_per_launch")


def copy_probe(torch, dev, mib):
    """One device-to-device copy of `mib` MiB (reads and writes exactly that
    many bytes): the calibration the counter runs scale FETCH_SIZE /
    WRITE_SIZE by."""
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the library runs on a single GPU; --gpus must be 1"}),
              flush=True)
        sys.exit(2)

    import torch
    import paged_kv_cache_51_amd as pkv
    import workloads

    if args.op == "copy_blocks":
        bench_copy_blocks(args, torch, pkv, workloads)
        return
    if args.op == "prefill":
        bench_prefill(args, torch, pkv, workloads)
        return
    if args.op == "vtoken":
        bench_vtoken(args, torch, pkv, workloads)
        return

    dt_names = {"bf16": pkv.BF16, "fp16": pkv.FP16, "fp8": pkv.FP8_E4M3}
    cfg, tabs, _, _ = workloads.make(args.config, seed=args.seed, block_size=args.block_size)
    if args.head_dim and args.head_dim != cfg.head_dim:
        import dataclasses
        cfg = dataclasses.replace(cfg, head_dim=args.head_dim, description=cfg.description.replace(
            f"d={cfg.head_dim}", f"d={args.head_dim}"))
    if args.heads or args.kv_heads:
        import dataclasses
        h = args.heads or cfg.num_heads
        hkv = args.kv_heads or cfg.num_kv_heads
        if h % hkv:
            raise SystemExit("--heads must be a multiple of --kv-heads")
        cfg = dataclasses.replace(cfg, num_heads=h, num_kv_heads=hkv, description=cfg.description.replace(
            f"{cfg.num_heads} q / {cfg.num_kv_heads} kv heads", f"{h} q / {hkv} kv heads"))
    kv_dtype = dt_names[args.kv_dtype] if args.kv_dtype else cfg.kv_dtype
    q_dtype = cfg.q_dtype
    if kv_dtype in (pkv.BF16, pkv.FP16) and kv_dtype != q_dtype:
        q_dtype = kv_dtype
    bs = args.block_size or cfg.block_size
    L = args.layers or cfg.num_layers
    S, H, Hkv, D = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    impl = {"auto": pkv.IMPL_AUTO, "mfma": pkv.IMPL_MFMA, "vector": pkv.IMPL_VECTOR,
            "persistent": pkv.IMPL_MFMA_PERSISTENT}[args.impl]
    part = args.partition_tokens
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    tq = torch.bfloat16 if q_dtype == pkv.BF16 else torch.float16
    b_kv = 1 if kv_dtype == pkv.FP8_E4M3 else 2
    ctx = tabs.context_lens
    max_ctx = int(ctx.max())
    nb = tabs.num_blocks
    fp8_scale = float(np.float32(8.0 / 448.0))
    ks = vs = fp8_scale if kv_dtype == pkv.FP8_E4M3 else 1.0

    kv_bytes = int(ctx.astype(np.int64).sum()) * 2 * Hkv * D * b_kv
    # Cache hygiene: the MI355X's 256 MB last-level cache (and 4 MB L2 per
    # XCD) would hold a small workload's pools between launches.  Each launch
    # therefore gets its own copy of the layer's pools, queries and outputs,
    # NP copies in rotation with NP * (K/V bytes) >= ROTATE_BYTES, so that
    # at least that much other memory is read between two uses of one copy.
    # A workload of many large layers rotates through its layers as it is.
    NP = max(L, -(-ROTATE_BYTES // max(kv_bytes, 1)))
    print(f"[bench] {cfg.description}; layers={L} kv={kv_dtype} bs={bs} blocks={nb} "
          f"pool copies in rotation={NP}", file=sys.stderr, flush=True)
    t0 = time.time()
    pool_bytes = pkv.layer_pool_bytes(nb, Hkv, D, bs, kv_dtype)
    kpools, vpools = [], []
    if NP > L:
        # one slab per side, sliced into NP pools
        kslab = torch.empty(NP * pool_bytes, dtype=torch.uint8, device=dev)
        vslab = torch.empty(NP * pool_bytes, dtype=torch.uint8, device=dev)
        workloads.device_fill_normal(kslab, kv_dtype, 1000, scale=fp8_scale)
        workloads.device_fill_normal(vslab, kv_dtype, 2000, scale=fp8_scale)
        kpools = [kslab[i * pool_bytes:(i + 1) * pool_bytes] for i in range(NP)]
        vpools = [vslab[i * pool_bytes:(i + 1) * pool_bytes] for i in range(NP)]
    else:
        for layer in range(NP):
            k = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
            v = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
            workloads.device_fill_normal(k, kv_dtype, 1000 + layer, scale=fp8_scale)
            workloads.device_fill_normal(v, kv_dtype, 2000 + layer, scale=fp8_scale)
            kpools.append(k)
            vpools.append(v)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 7)
    qs = [torch.randn(S, H, D, generator=gen, device=dev).to(tq) for _ in range(NP)]
    newk = [torch.randn(S, Hkv, D, generator=gen, device=dev).to(tq) for _ in range(NP)]
    newv = [torch.randn(S, Hkv, D, generator=gen, device=dev).to(tq) for _ in range(NP)]
    outs = [torch.empty(S, H, D, dtype=tq, device=dev) for _ in range(NP)]
    bt = torch.from_numpy(tabs.block_tables).to(dev)
    cl = torch.from_numpy(ctx).to(dev)
    slots = torch.empty(S, dtype=torch.int32, device=dev)
    part_resolved = part or pkv.default_partition_tokens(S, Hkv, max_ctx, bs)
    ws_n = pkv.workspace_bytes(S, H, Hkv, D, max_ctx, bs, part_resolved)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    plan = torch.empty(pkv.plan_bytes(S, Hkv, max_ctx, bs, part_resolved), dtype=torch.uint8,
                       device=dev)
    assert pkv.check_block_tables(bt, cl, bs, nb) == 0
    torch.cuda.synchronize()
    print(f"[bench] inputs resident in {time.time() - t0:.1f}s "
          f"({2 * NP * pool_bytes / 2**30:.1f} GiB of pools)", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    scale = float(np.float32(1.0 / np.sqrt(D)))

    rot = [0]                  # next pool copy in the rotation

    separate = args.separate_cache_write

    def step(ev=None):
        # per-step work shared by all layers: the work plan (and, for separate
        # cache writes, the new tokens' slots)
        if separate:
            pkv.decode_slot_mapping(bt, cl, bs, slot_mapping=slots, stream=stream)
        pkv.build_plan(cl, max_ctx, bt.shape[1], Hkv, bs, part_resolved, plan=plan, stream=stream)
        base = rot[0]
        rot[0] = (base + L) % NP
        for li in range(L):
            layer = (base + li) % NP
            evl = None if ev is None else ev[li]
            if separate:
                pkv.reshape_and_cache(newk[layer], newv[layer], kpools[layer], vpools[layer],
                                      slots, bs, nb, kv_dtype, ks, vs, stream=stream)
            if evl is not None:
                evl[0].record(stream)
            if separate:
                pkv.paged_attention_decode(outs[layer], qs[layer], kpools[layer], vpools[layer],
                                           bt, cl, max_ctx, Hkv, bs, kv_dtype, scale, ks, vs,
                                           workspace=ws, partition_tokens=part_resolved,
                                           impl=impl, stages=pkv.STAGE_PARTITIONS, num_blocks=nb,
                                           plan=plan, stream=stream)
            else:
                # the partition kernel writes each sequence's new K / V itself
                pkv.paged_attention_decode_append(outs[layer], qs[layer], newk[layer], newv[layer],
                                                  kpools[layer], vpools[layer], bt, cl, max_ctx,
                                                  Hkv, bs, kv_dtype, scale, ks, vs, workspace=ws,
                                                  partition_tokens=part_resolved, impl=impl,
                                                  num_blocks=nb, plan=plan, stream=stream,
                                                  stages=pkv.STAGE_PARTITIONS)
            if evl is not None:
                evl[1].record(stream)
            pkv.paged_attention_decode(outs[layer], qs[layer], kpools[layer], vpools[layer], bt,
                                       cl, max_ctx, Hkv, bs, kv_dtype, scale, ks, vs,
                                       workspace=ws, partition_tokens=part_resolved, impl=impl,
                                       stages=pkv.STAGE_REDUCE, num_blocks=nb, plan=plan,
                                       stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)]
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # Per-launch events are recorded in every --event-every-th timed step
    # only: each event pair adds a few microseconds between launches, which
    # would otherwise count against the step throughput.
    timed_steps = [k for k in range(args.steps) if k % args.event_every == 0]
    start.record(stream)
    for k in range(args.steps):
        step(evs[k] if k % args.event_every == 0 else None)
    end.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / args.steps
    dec_ms = [evs[k][layer][0].elapsed_time(evs[k][layer][1])
              for k in timed_steps for layer in range(L)]
    dec_avg_ms = float(np.mean(dec_ms))

    unique_kv_bytes = unique_kv_tokens(tabs.block_tables, ctx, bs, nb) * 2 * Hkv * D * b_kv
    qo_bytes = S * H * D * (2 + 2)
    new_bytes = S * Hkv * D * 2 * (2 + b_kv)
    step_bytes = L * (kv_bytes + qo_bytes + new_bytes)
    gbs = step_bytes / (step_ms * 1e-3) / 1e9
    # the partition kernel's own bytes: K / V, q and out, plus the new
    # tokens' K / V (read, and written to the pool) when it appends them
    launch_bytes = kv_bytes + qo_bytes + (0 if separate else new_bytes)
    achieved = launch_bytes / (dec_avg_ms * 1e-3) / 1e9
    traffic_key = (f"{args.config}-{kv_dtype}-bs{bs}-part{part_resolved}-impl{impl}"
                   + (f"-d{D}" if D != 128 else "")
                   + (f"-h{H}-kv{Hkv}" if args.heads or args.kv_heads else "")
                   + ("-separate" if separate else "-append"))
    traffic = measured_traffic(traffic_key)
    unique_gbs = (unique_kv_bytes + qo_bytes) / (dec_avg_ms * 1e-3) / 1e9
    print(f"[bench] step {step_ms:.3f} ms, {gbs:.0f} GB/s; partition kernel "
          f"{dec_avg_ms * 1e3:.1f} us avg, {achieved:.0f} GB/s ({achieved / PEAK_HBM_GBS:.1%})"
          + (f"; unique K/V {unique_kv_bytes / 1e9:.3f} of {kv_bytes / 1e9:.3f} GB: "
             f"{unique_gbs:.0f} GB/s" if unique_kv_bytes != kv_bytes else ""),
          file=sys.stderr, flush=True)

    # achievable figure: the library's streaming-read probe, one launch over
    # a contiguous buffer of one decode launch's K / V bytes, outside the
    # timed region
    probe_bytes = (launch_bytes + 15) // 16 * 16
    probe_src = torch.full((probe_bytes,), 1, dtype=torch.uint8, device=dev)
    sink = pkv.read_probe(probe_src, stream=stream)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    torch.cuda.synchronize()
    p0.record(stream)
    for _ in range(reps):
        pkv.read_probe(probe_src, sink=sink, stream=stream)
    p1.record(stream)
    torch.cuda.synchronize()
    probe_gbs = probe_bytes * reps / (p0.elapsed_time(p1) * 1e-3) / 1e9
    del sink, probe_src
    print(f"[bench] read-stream probe: {probe_gbs:.0f} GB/s over {probe_bytes / 1e9:.2f} GB "
          f"(decode kernel at {achieved / probe_gbs:.1%} of it)", file=sys.stderr, flush=True)

    if args.copy_probe_mib:
        copy_probe(torch, dev, args.copy_probe_mib)

    clocks = clocks_under_load(torch, step, step_ms)

    cpu = None
    if args.cpu_baseline_seconds > 0:
        cpu = cpu_baseline(args, tabs, kpools[0], vpools[0], qs[0], q_dtype, kv_dtype, Hkv, bs,
                           scale, ks, vs, b_kv, H, D)

    dt_name = {pkv.BF16: "bf16", pkv.FP16: "fp16", pkv.FP8_E4M3: "fp8"}
    rec = {
        "metric": "paged decode attn achieved HBM GB/s (% of MI355X peak) + seq-layers/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name[q_dtype],     # MFMA arithmetic (fp8 K / V widened to it); kv_dtype below
        "data": "synthetic",
        "config": {
            "workload": cfg.description,
            "config": args.config,
            "layers": L,
            "num_seqs": S,
            "num_heads": H,
            "num_kv_heads": Hkv,
            "head_dim": D,
            "block_size": bs,
            "kv_dtype": dt_name[kv_dtype],
            "mean_context": float(ctx.mean()),
            "partition_tokens": part_resolved,
            "impl": args.impl,
            "cache_write": "separate launch (reshape_and_cache)" if separate
                           else "in the decode launch (paged_attention_decode_append)",
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "seq_layers_per_s": round(S * L / (step_ms * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "kernel": {pkv.IMPL_VECTOR: "paged_decode_vector_kernel",
                       pkv.IMPL_MFMA_PERSISTENT: "paged_decode_mfma_persistent"}.get(
                           impl, "paged_decode_mfma_kernel"),
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(dec_avg_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": launch_bytes,
            "launch_timing": f"HIP events on the launch stream around every partition-kernel "
                             f"launch of {len(timed_steps)} of the {args.steps} timed steps "
                             f"({len(dec_ms)} launches)",
        },
        "unique_bytes": {
            "kv_bytes_per_launch": unique_kv_bytes,
            "gbs": round(unique_gbs, 1),
            "note": "shared blocks counted once (equal to the logical bytes without sharing)",
        },
        "achievable": {
            "kind": "read-stream probe (pkv_read_probe: non-temporal 16-byte loads, one contiguous "
                    "slice per workgroup, two workgroups per CU), one launch over a contiguous "
                    "buffer of one decode launch's bytes",
            "gbs": round(probe_gbs, 1),
            "bytes": probe_bytes,
            "decode_frac_of_probe": round(achieved / probe_gbs, 4),
        },
        "cache_hygiene": {
            "pool_copies_in_rotation": NP,
            "kv_bytes_read_between_reuse": int(NP - 1) * kv_bytes if NP > 1 else 0,
            "note": "each launch reads its own copy of the layer's pools, q and out; "
                    f"copies rotate so that >= {ROTATE_BYTES / 1e9:.0f} GB of other K/V is "
                    "read between two uses of one copy (256 MB last-level cache)"
                    if NP > L else "layers are distinct pools larger than the caches",
        },
        "clocks": clocks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def bench_prefill(args, torch, pkv, workloads):
    """Multi-token causal paged attention over the workload's contexts: the
    last --q-len tokens of each of --num-seqs sequences are new (a chunked
    prefill step, or a few tokens per sequence after prefix-cache hits).  A
    step is one paged_attention_prefill call per layer.  Reported: TFLOP/s
    (4 * d flops per (query row, head, visible key)) and the unique KV +
    query / output bytes per second; the roofline takes whichever bound
    the step's intensity puts it under."""
    dt_names = {"bf16": pkv.BF16, "fp16": pkv.FP16, "fp8": pkv.FP8_E4M3}
    cfg, tabs_all, _, _ = workloads.make(args.config, seed=args.seed, block_size=args.block_size)
    kv = dt_names[args.kv_dtype] if args.kv_dtype else cfg.kv_dtype
    q_dtype = cfg.q_dtype if kv == pkv.FP8_E4M3 else kv
    bs = args.block_size or cfg.block_size
    L = args.layers or min(cfg.num_layers, 4)
    H, Hkv, D = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    qlen = args.q_len
    S = args.num_seqs or (cfg.num_seqs if qlen <= 16 else min(16, cfg.num_seqs))
    ctx = tabs_all.context_lens[:S].astype(np.int64)
    if (ctx < qlen).any():
        raise SystemExit(f"--q-len {qlen} exceeds a context length ({int(ctx.min())})")
    bt_np = tabs_all.block_tables[:S]
    nb = tabs_all.num_blocks
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    pool_bytes = pkv.layer_pool_bytes(nb, Hkv, D, bs, kv)
    fp8_scale = float(np.float32(8.0 / 448.0))
    ks = vs = fp8_scale if kv == pkv.FP8_E4M3 else 1.0
    kpools = [torch.empty(pool_bytes, dtype=torch.uint8, device=dev) for _ in range(L)]
    vpools = [torch.empty(pool_bytes, dtype=torch.uint8, device=dev) for _ in range(L)]
    for i in range(L):
        workloads.device_fill_normal(kpools[i], kv, 1000 + i, scale=fp8_scale)
        workloads.device_fill_normal(vpools[i], kv, 2000 + i, scale=fp8_scale)
    tq = torch.bfloat16 if q_dtype == pkv.BF16 else torch.float16
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 17)
    T = S * qlen
    qs = [torch.randn(T, H, D, generator=gen, device=dev).to(tq) for _ in range(L)]
    outs = [torch.empty(T, H, D, dtype=tq, device=dev) for _ in range(L)]
    bt = torch.from_numpy(np.ascontiguousarray(bt_np)).to(dev)
    cl = torch.from_numpy(ctx.astype(np.int32)).to(dev)
    qsl = torch.arange(0, T + 1, qlen, dtype=torch.int32, device=dev)
    mc = int(ctx.max())
    scale = float(np.float32(1.0 / np.sqrt(D)))
    stream = torch.cuda.current_stream()

    def step(ev=None):
        for layer in range(L):
            if ev is not None:
                ev[layer][0].record(stream)
            pkv.paged_attention_prefill(outs[layer], qs[layer], kpools[layer], vpools[layer], bt,
                                        cl, qsl, qlen, mc, Hkv, bs, kv, scale, ks, vs,
                                        stream=stream)
            if ev is not None:
                ev[layer][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)]
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    end.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / args.steps
    launch_ms = float(np.mean([evs[k][l][0].elapsed_time(evs[k][l][1])
                               for k in range(args.steps) for l in range(L)]))
    b_kv = 1 if kv == pkv.FP8_E4M3 else 2
    # visible keys of token j (position c - qlen + j): c - qlen + j + 1
    keys = int(sum(qlen * (c - qlen) + qlen * (qlen + 1) // 2 for c in ctx))
    flops = 4 * D * H * keys
    nbytes = int(ctx.sum()) * 2 * Hkv * D * b_kv + T * H * D * 4
    tflops = flops / (launch_ms * 1e-3) / 1e12
    gbs = nbytes / (launch_ms * 1e-3) / 1e9
    peak_tf = {pkv.BF16: 2500.0, pkv.FP16: 2500.0}.get(q_dtype, 2500.0)
    ridge = peak_tf * 1e12 / (PEAK_HBM_GBS * 1e9)
    mfma_bound = flops / nbytes > ridge
    print(f"[bench] prefill: {S} seqs x {qlen} new tokens, contexts {int(ctx.min())}-{int(ctx.max())}; "
          f"{launch_ms * 1e3:.1f} us per layer, {tflops:.1f} TFLOP/s, {gbs:.0f} GB/s; "
          f"intensity {flops / nbytes:.0f} flop/B", file=sys.stderr, flush=True)
    if args.copy_probe_mib:
        copy_probe(torch, dev, args.copy_probe_mib)
    clocks = clocks_under_load(torch, step, step_ms)
    kv_name = {pkv.BF16: "bf16", pkv.FP16: "fp16", pkv.FP8_E4M3: "fp8"}[kv]
    traffic = measured_traffic(f"prefill-{args.config}-{kv_name}-bs{bs}-q{qlen}-s{S}",
                               "prefill_traffic.json", PREFILL_SOURCES)
    cpu = None
    if args.cpu_baseline_seconds > 0:
        cpu = cpu_sample(args, "prefill", lambda n: _prefill_oracle_sample(
            n, kpools[0], vpools[0], qs[0], bt_np, ctx, qlen, q_dtype, kv, Hkv, bs, scale, ks, vs),
            lambda n: 4 * D * H * sum(int(ctx[0]) - qlen + j + 1 for j in range(qlen - n, qlen)),
            "TFLOP/s", 1e12,
            "layer 0, sequence 0: its last n new tokens (one-token chunks at their positions), "
            "fp64 C oracle, OpenMP over (row, head)", min(qlen, 256))
    dt_name = {pkv.BF16: "bf16", pkv.FP16: "fp16", pkv.FP8_E4M3: "fp8"}
    print(json.dumps({
        "metric": "paged multi-token attention TFLOP/s" if mfma_bound
                  else "paged multi-token attention HBM GB/s",
        "value": round(tflops if mfma_bound else gbs, 2 if mfma_bound else 1),
        "unit": "TFLOP/s" if mfma_bound else "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": dt_name[q_dtype], "data": "synthetic",
        "config": {"workload": f"{cfg.description.split(':')[0]}: {S} sequences, the last {qlen} "
                               f"of {int(ctx.min())}-{int(ctx.max())} context tokens new, {L} layers",
                   "num_seqs": S, "q_len": qlen, "layers": L, "num_heads": H,
                   "num_kv_heads": Hkv, "kv_dtype": dt_name[kv], "block_size": bs,
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 2), "gbs": round(gbs, 1),
        "roofline": {"bound": "mfma" if mfma_bound else "hbm", "kernel": "paged_prefill_staged_kernel" if -(-qlen // (16 // (H // Hkv))) > 4 else "paged_prefill_mfma_kernel",
                     "achieved": round(tflops if mfma_bound else gbs, 2),
                     "peak": peak_tf if mfma_bound else PEAK_HBM_GBS,
                     "unit": "TFLOP/s" if mfma_bound else "GB/s",
                     "frac": round((tflops / peak_tf) if mfma_bound else (gbs / PEAK_HBM_GBS), 4),
                     "traffic": traffic, "avg_launch_us": round(launch_ms * 1e3, 2),
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes},
        "clocks": clocks,
        "cpu_baseline": cpu,
    }), flush=True)


def bench_vtoken(args, torch, pkv, workloads):
    """Token-level virtualisation on the workload: every sequence keeps a
    random --keep fraction of its context (an eviction); time (1) decode
    through the fragmented token table, per token (the gather) and over run
    lists (whole sub-tiles, rows masked; the list built once per step: the
    step and `value`), (2) the repack moves over all layers, (3) the
    block-table decode of the repacked sequences.  Bytes: surviving K/V +
    q/out for the decodes; moved token rows read + written for the
    repack."""
    cfg, tabs, _, _ = workloads.make(args.config, seed=args.seed, block_size=args.block_size)
    dt_names = {"bf16": pkv.BF16, "fp16": pkv.FP16, "fp8": pkv.FP8_E4M3}
    kv = dt_names[args.kv_dtype] if args.kv_dtype else cfg.kv_dtype
    q_dtype = cfg.q_dtype if kv == pkv.FP8_E4M3 else kv
    bs = args.block_size or cfg.block_size
    L = args.layers or min(cfg.num_layers, 4)
    S, H, Hkv, D = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    ctx = tabs.context_lens.astype(np.int64)
    nb = tabs.num_blocks
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    # the block manager owns the pool: one sequence per row, blocks as allocated
    bm = pkv.BlockManager(nb, bs)
    for s in range(S):
        bm.add_sequence(s, [0] * int(ctx[s]))
    r = np.random.default_rng(args.seed + 5)
    for s in range(S):
        keep = r.random(int(ctx[s])) < args.keep
        keep[-1] = True
        bm.evict_tokens(s, keep.tolist())
    width = int(ctx.max())
    n_keep = np.array([bm.num_tokens(s) for s in range(S)], np.int64)
    slots = torch.tensor([bm.token_slots(s, width) for s in range(S)], dtype=torch.int32, device=dev)
    cl = torch.from_numpy(n_keep.astype(np.int32)).to(dev)
    pool_bytes = pkv.layer_pool_bytes(nb, Hkv, D, bs, kv)
    fp8_scale = float(np.float32(8.0 / 448.0))
    ks = vs = fp8_scale if kv == pkv.FP8_E4M3 else 1.0
    kpools = [torch.empty(pool_bytes, dtype=torch.uint8, device=dev) for _ in range(L)]
    vpools = [torch.empty(pool_bytes, dtype=torch.uint8, device=dev) for _ in range(L)]
    for i in range(L):
        workloads.device_fill_normal(kpools[i], kv, 1000 + i, scale=fp8_scale)
        workloads.device_fill_normal(vpools[i], kv, 2000 + i, scale=fp8_scale)
    tq = torch.bfloat16 if q_dtype == pkv.BF16 else torch.float16
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 9)
    qs = [torch.randn(S, H, D, generator=gen, device=dev).to(tq) for _ in range(L)]
    outs = [torch.empty(S, H, D, dtype=tq, device=dev) for _ in range(L)]
    scale = float(np.float32(1.0 / np.sqrt(D)))
    stream = torch.cuda.current_stream()
    b_kv = 1 if kv == pkv.FP8_E4M3 else 2
    dec_bytes = int(n_keep.sum()) * 2 * Hkv * D * b_kv + S * H * D * 4

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    cpu = None
    if args.cpu_baseline_seconds > 0:
        slots_np = slots.cpu().numpy()
        cpu = cpu_sample(args, "vtoken", lambda n: _tokens_oracle_sample(
            n, kpools[0], vpools[0], qs[0], slots_np, n_keep, q_dtype, kv, Hkv, bs, scale, ks, vs),
            lambda n: int(n_keep[:n].sum()) * 2 * Hkv * D * b_kv + n * H * D * 4, "GB/s", 1e9,
            "layer 0, first n sequences through the fragmented token table, fp64 C oracle, "
            "OpenMP over (seq, head)", S)

    def frag_step():
        for l in range(L):
            pkv.paged_attention_decode_tokens(outs[l], qs[l], kpools[l], vpools[l], slots, cl, Hkv, bs,
                                              nb, kv, scale, ks, vs, stream=stream)
    frag_ms = timed(frag_step, args.steps) / L
    # the same attention over run lists: the table as pool sub-tiles with
    # row masks, built once per step (the table is shared by all layers)
    runs = torch.empty(pkv.token_runs_bytes(S, width), dtype=torch.uint8, device=dev)
    runs_build_ms = timed(lambda: pkv.token_runs(slots, cl, bs, nb, runs=runs, stream=stream), args.steps)
    counts = runs[:4 * S].view(torch.int32).cpu().numpy()
    n_entries = int(counts[counts >= 0].sum())         # sub-tiles the run lists read
    n_marked = int((counts < 0).sum())                  # sequences left to the token gather

    def runs_layers():
        for l in range(L):
            pkv.paged_attention_decode_runs(outs[l], qs[l], kpools[l], vpools[l], runs, width, Hkv, bs, nb,
                                            kv, scale, ks, vs, token_slots=slots, context_lens=cl,
                                            stream=stream)
    runs_ms = timed(runs_layers, args.steps) / L

    def runs_step():
        pkv.token_runs(slots, cl, bs, nb, runs=runs, stream=stream)
        runs_layers()
    runs_step_ms = timed(runs_step, args.steps)
    # the repack, both ways: whole-block rebuild (pkv_repack_blocks, one
    # chain per sequence) and the same rows as generic token moves
    tiles, offsets = [], [0]
    for s in range(S):
        tiles += bm.repack_tiles(s)
        offsets.append(len(tiles))
    moves = [(src, blk * bs + i) for blk, srcs in tiles for i, src in enumerate(srcs)
             if src != blk * bs + i]
    mv = torch.tensor(moves, dtype=torch.int32, device=dev).reshape(-1, 2)
    tl = torch.tensor([[blk] + list(srcs) for blk, srcs in tiles], dtype=torch.int32,
                      device=dev).reshape(-1, 1 + bs)
    to = torch.tensor(offsets, dtype=torch.int32, device=dev)
    need = pkv.lib().pkv_move_tokens_scratch_bytes(L, mv.shape[0], Hkv, D, kv)
    scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    # repeated for timing (the values the synthetic pools end up with do
    # not matter here; the decode below only needs the same bytes moved)
    move_ms = timed(lambda: pkv.move_tokens(kpools, vpools, mv, nb, Hkv, D, bs, kv,
                                            scratch=scratch, stream=stream), max(1, args.steps // 2))
    tile_ms = timed(lambda: pkv.repack_blocks(kpools, vpools, tl, to, nb, Hkv, D, bs, kv,
                                              stream=stream), max(1, args.steps // 2))
    move_bytes = mv.shape[0] * L * 2 * Hkv * D * b_kv * 2
    tile_bytes = tl.shape[0] * bs * L * 2 * Hkv * D * b_kv * 2
    mb = -(-width // bs)
    bt = torch.tensor([bm.block_table(s, mb) for s in range(S)], dtype=torch.int32, device=dev)
    mc = int(n_keep.max())

    def block_step():
        for l in range(L):
            pkv.paged_attention_decode(outs[l], qs[l], kpools[l], vpools[l], bt, cl, mc, Hkv, bs, kv,
                                       scale, ks, vs, num_blocks=nb, stream=stream)
    block_ms = timed(block_step, args.steps) / L
    if args.copy_probe_mib:
        copy_probe(torch, dev, args.copy_probe_mib)
    kv_name = {pkv.BF16: "bf16", pkv.FP16: "fp16", pkv.FP8_E4M3: "fp8"}[kv]
    traffic = measured_traffic(f"vtoken-{args.config}-{kv_name}-bs{bs}-keep{args.keep:.2f}",
                               "vtoken_traffic.json", VTOKEN_SOURCES)
    runs_traffic = measured_traffic(f"vtoken-runs-{args.config}-{kv_name}-bs{bs}-keep{args.keep:.2f}",
                                    "vtoken_traffic.json", VTOKEN_SOURCES)
    frag_gbs = dec_bytes / (frag_ms * 1e-3) / 1e9
    runs_gbs = dec_bytes / (runs_ms * 1e-3) / 1e9
    runs_step_gbs = dec_bytes * L / (runs_step_ms * 1e-3) / 1e9
    # bytes of the sub-tiles the run lists read (each entry one 16-token
    # sub-tile of K and of V per kv head) + q / out
    sub_bytes = n_entries * 2 * Hkv * 16 * D * b_kv + S * H * D * 4
    block_gbs = dec_bytes / (block_ms * 1e-3) / 1e9
    move_gbs = move_bytes / (move_ms * 1e-3) / 1e9
    tile_gbs = tile_bytes / (tile_ms * 1e-3) / 1e9
    print(f"[bench] vtoken: keep {args.keep:.2f} ({int(n_keep.sum())} of {int(ctx.sum())} tokens); "
          f"fragmented-table decode {frag_ms * 1e3:.1f} us/layer ({frag_gbs:.0f} GB/s); repack x {L} "
          f"layers: {tl.shape[0]} whole blocks rebuilt {tile_ms * 1e3:.1f} us ({tile_gbs:.0f} GB/s "
          f"read + written), as {mv.shape[0]} token moves {move_ms * 1e3:.1f} us ({move_gbs:.0f} GB/s); "
          f"block decode after {block_ms * 1e3:.1f} us/layer ({block_gbs:.0f} GB/s)",
          file=sys.stderr, flush=True)
    print(f"[bench] vtoken run lists: {n_entries} sub-tiles ({sub_bytes / 1e9:.2f} GB read per layer), "
          f"{n_marked} of {S} sequences token by token (fewer than {pkv.RUNS_MIN_KEYS} keys per sub-tile); "
          f"build {runs_build_ms * 1e3:.1f} us per step, decode {runs_ms * 1e3:.1f} us/layer ({runs_gbs:.0f} "
          f"GB/s surviving, {sub_bytes / (runs_ms * 1e-3) / 1e9:.0f} GB/s of sub-tiles read); step of "
          f"{L} layers {runs_step_ms * 1e3:.1f} us ({runs_step_gbs:.0f} GB/s)", file=sys.stderr, flush=True)
    dt_name = {pkv.BF16: "bf16", pkv.FP16: "fp16", pkv.FP8_E4M3: "fp8"}
    print(json.dumps({
        "metric": "token-table decode HBM GB/s (surviving K/V + q/out)",
        "value": round(runs_step_gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(runs_step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": dt_name[q_dtype], "data": "synthetic",
        "config": {"workload": f"{cfg.description.split(':')[0]}: each sequence keeps a random "
                               f"{args.keep:.0%} of its context, {L} layers",
                   "keep": args.keep, "layers": L, "num_seqs": S, "parallelism": "single GPU"},
        "repack": {"tiles": int(tl.shape[0]), "tiles_us": round(tile_ms * 1e3, 1),
                   "tiles_gbs_read_plus_write": round(tile_gbs, 1),
                   "moves": int(mv.shape[0]), "moves_us": round(move_ms * 1e3, 1),
                   "moves_gbs_read_plus_write": round(move_gbs, 1)},
        "after_repack_block_decode": {"us_per_layer": round(block_ms * 1e3, 1),
                                      "gbs": round(block_gbs, 1)},
        "step": "run lists built once (pkv_token_runs), then paged_attention_decode_runs per layer",
        "run_lists": {"entries": n_entries, "sub_tile_bytes_per_layer": sub_bytes,
                      "sequences_token_by_token": n_marked, "min_keys_per_entry": pkv.RUNS_MIN_KEYS,
                      "build_us_per_step": round(runs_build_ms * 1e3, 2),
                      "sub_tile_gbs": round(sub_bytes / (runs_ms * 1e-3) / 1e9, 1)},
        "token_gather_decode": {"kernel": "paged_decode_tokens_kernel",
                                "us_per_layer": round(frag_ms * 1e3, 1), "gbs": round(frag_gbs, 1),
                                "traffic": traffic},
        "roofline": {"bound": "hbm", "kernel": "paged_decode_runs_kernel",
                     "achieved": round(runs_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(runs_gbs / PEAK_HBM_GBS, 4), "traffic": runs_traffic,
                     "avg_launch_us": round(runs_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": dec_bytes},
        "cpu_baseline": cpu,
    }), flush=True)


def bench_copy_blocks(args, torch, pkv, workloads):
    """Copy-on-write block copies: one call copies `--copy-pairs` random
    (src, dst) blocks in every layer's K and V pool of the workload's pool
    shape.  A step is one call; bytes = pairs x layers x 2 pools x block
    bytes, read and written."""
    dt_names = {"bf16": pkv.BF16, "fp16": pkv.FP16, "fp8": pkv.FP8_E4M3}
    cfg = workloads.CONFIGS[args.config]
    kv = dt_names[args.kv_dtype] if args.kv_dtype else cfg.kv_dtype
    bs = args.block_size or cfg.block_size
    L = args.layers or cfg.num_layers
    Hkv, D = cfg.num_kv_heads, cfg.head_dim
    npairs = args.copy_pairs
    nb = 1 + 4 * npairs                       # room for disjoint sources and destinations
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    pool_bytes = pkv.layer_pool_bytes(nb, Hkv, D, bs, kv)
    block = pool_bytes // nb
    ks = [torch.empty(pool_bytes, dtype=torch.uint8, device=dev) for _ in range(L)]
    vs = [torch.empty(pool_bytes, dtype=torch.uint8, device=dev) for _ in range(L)]
    for i, t in enumerate(ks + vs):
        workloads.device_fill_normal(t, kv, 3000 + i, scale=8.0 / 448.0)
    r = np.random.default_rng(args.seed)
    perm = r.permutation(np.arange(1, nb))
    pairs_np = np.stack([perm[:npairs], perm[npairs:2 * npairs]], 1).astype(np.int32)
    pairs = torch.from_numpy(pairs_np).to(dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pkv.copy_blocks(ks, vs, pairs, nb, Hkv, D, bs, kv, stream=stream)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(args.steps):
        evs[k][0].record(stream)
        pkv.copy_blocks(ks, vs, pairs, nb, Hkv, D, bs, kv, stream=stream)
        evs[k][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / args.steps
    launch_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    nbytes = npairs * L * 2 * block * 2
    gbs = nbytes / (step_ms * 1e-3) / 1e9
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    print(f"[bench] copy_blocks: {npairs} pairs x {L} layers x K,V, block {block} B; "
          f"{launch_ms * 1e3:.1f} us per call, {achieved:.0f} GB/s", file=sys.stderr, flush=True)
    cpu = None
    if args.cpu_baseline_seconds > 0:
        import oracle.blocks as ob
        hk = [ks[0].cpu().numpy()]
        hv = [vs[0].cpu().numpy()]
        n = min(npairs, 256)
        t0 = time.time()
        ob.copy_blocks(hk, hv, pairs_np[:n].tolist(), block)
        dt = time.time() - t0
        cpu = {"value": round(n * 2 * block * 2 / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"layer 0, first {n} of {npairs} pairs, numpy slice copies"}
    dt_name = {pkv.BF16: "bf16", pkv.FP16: "fp16", pkv.FP8_E4M3: "fp8"}
    print(json.dumps({
        "metric": "copy_blocks HBM GB/s (bytes read + written)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"copy-on-write copies: {npairs} random block pairs x {L} layers "
                               f"x K and V, {cfg.description.split(':')[0]} pool shape "
                               f"({Hkv} kv heads, d={D}, {dt_name[kv]}, bs={bs})",
                   "pairs": npairs, "layers": L, "block_bytes": block,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "copy_blocks_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None, "avg_launch_us": round(launch_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
    }), flush=True)


def clocks_under_load(torch, step, step_ms, seconds=1.5):
    """GPU clocks and power while this workload runs: about `seconds` of
    steps are queued (after the timed region, outside every timing) and
    rocm-smi is read while they execute; then once more when the GPU is idle
    again."""
    n_load = int(min(20000, max(1, seconds * 1e3 / max(step_ms, 1e-3))))
    for _ in range(n_load):
        step()
    clocks = {"under_load": gpu_clocks(), "load_steps": n_load}
    torch.cuda.synchronize()
    clocks["idle_after"] = gpu_clocks()
    return clocks


def gpu_clocks():
    """Current GPU clocks and power as rocm-smi reports them (a child
    process, after the timed region), or the reason they are missing."""
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        # under the profiler a child process may not start another program
        return {"error": "not read under rocprofv3"}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"],
                           capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout[r.stdout.index("{"):])
    except Exception as e:            # tool missing, no JSON, timeout
        return {"error": f"rocm-smi: {type(e).__name__}: {e}"[:200]}
    out = {}
    for card, vals in data.items():
        if isinstance(vals, dict):
            out[card] = {k.strip(" :"): v for k, v in vals.items()
                         if any(w in k.lower() for w in ("clk", "clock", "power"))}
    return out or {"raw": r.stdout[:400]}


def host_info():
    """The CPU the oracle ran on: model, logical CPUs, and this process's
    affinity mask."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
    runs, start = [], None
    for c in aff + [None]:
        if start is None:
            start = prev = c
        elif c is None or c != prev + 1:
            runs.append(f"{start}-{prev}" if prev != start else f"{start}")
            start = prev = c
        else:
            prev = c
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": ",".join(runs),
            "affinity_cpus": len(aff)}


def median3(run, n):
    """Median of three timings of run(n)."""
    return float(np.median([run(n) for _ in range(3)]))


_PKV2ORC = {0: 0, 1: 1, 2: 2}      # library dtype codes -> oracle dtype codes (same values)


def cpu_sample(args, what, run, work_of, unit, unit_scale, sample_desc, n_max):
    """Time run(n) (the oracle on a sample of n units) with n grown until it
    takes about --cpu-baseline-seconds; report work_of(n) / time."""
    import oracle
    run(1)                                       # pulls pools to the host, builds caches
    t = time.time()
    run(1)
    t1 = max(time.time() - t, 1e-6)
    n = int(min(n_max, max(1, args.cpu_baseline_seconds / 3 / t1)))

    def timed(k):
        t = time.time()
        run(k)
        return time.time() - t

    tn = median3(timed, n)
    print(f"[bench] cpu oracle ({what}): n={n} in {tn:.1f}s (median of 3) on "
          f"{oracle.max_threads()} threads", file=sys.stderr, flush=True)
    return {"value": round(work_of(n) / tn / unit_scale, 6), "unit": unit,
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": sample_desc.replace(" n ", f" {n} ").replace("first n", f"first {n}")
                                 .replace("last n", f"last {n}"),
            "seconds": round(tn, 2), "timing": "median of 3 runs of the sample",
            "host": host_info()}


_HOST = {}


def _host(t):
    key = t.data_ptr()
    if key not in _HOST:
        _HOST[key] = t.cpu().numpy()
    return _HOST[key]


def _prefill_oracle_sample(n, kpool, vpool, q, bt, ctx, qlen, q_dtype, kv, Hkv, bs, scale, ks, vs):
    import oracle
    import torch
    qb = q.cpu().view(torch.int16).numpy().view(np.uint16)
    c0 = int(ctx[0])
    rows = list(range(qlen - n, qlen))
    sub_q = qb[rows]
    sub_ctx = np.array([c0 - qlen + j + 1 for j in rows], np.int32)   # one-token chunks
    sub_bt = np.repeat(bt[:1], len(rows), axis=0)
    oracle.paged_prefill(sub_q, _PKV2ORC[q_dtype], _host(kpool), _host(vpool), _PKV2ORC[kv], sub_bt,
                         sub_ctx, np.arange(len(rows) + 1, dtype=np.int32), Hkv, bs, scale, ks, vs)


def _tokens_oracle_sample(n, kpool, vpool, q, slots, n_keep, q_dtype, kv, Hkv, bs, scale, ks, vs):
    import oracle
    import torch
    qb = q[:n].cpu().view(torch.int16).numpy().view(np.uint16)
    oracle.paged_decode_tokens(qb, _PKV2ORC[q_dtype], _host(kpool), _host(vpool), _PKV2ORC[kv],
                               slots[:n], n_keep[:n].astype(np.int32), Hkv, bs, scale, ks, vs)


def unique_kv_tokens(block_tables, ctx, bs, num_blocks):
    """Distinct pool slots a decode over these tables reads: a physical block
    referenced by several sequences (a shared prefix) counts once, with the
    most tokens any of them uses in it."""
    ids, toks = [], []
    for s, c in enumerate(np.asarray(ctx, dtype=np.int64)):
        nblk = -(-int(c) // bs)
        ids.append(block_tables[s, :nblk].astype(np.int64))
        toks.append(np.minimum(bs, int(c) - bs * np.arange(nblk, dtype=np.int64)))
    used = np.zeros(num_blocks, dtype=np.int64)
    if ids:
        np.maximum.at(used, np.concatenate(ids), np.concatenate(toks))
    return int(used.sum())


def cpu_baseline(args, tabs, kpool, vpool, q, q_dtype, kv_dtype, Hkv, bs, scale, ks, vs, b_kv,
                 H, D):
    """The oracle as it stands, on a bounded sample of layer 0."""
    import oracle
    t0 = time.time()
    kp = kpool.cpu().numpy()
    vp = vpool.cpu().numpy()
    qb = q.cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    ctx = tabs.context_lens
    bt = tabs.block_tables
    odt = {0: oracle.BF16, 1: oracle.FP16, 2: oracle.FP8}
    threads = oracle.max_threads()

    def run(n):
        t = time.time()
        oracle.paged_decode(qb[:n], odt[q_dtype], kp, vp, odt[kv_dtype], bt[:n], ctx[:n], Hkv,
                            bs, scale, ks, vs)
        return time.time() - t

    t1 = run(1)
    n = int(min(len(ctx), max(1, args.cpu_baseline_seconds / 3 / max(t1, 1e-6))))
    tn = median3(run, n)
    kv = int(ctx[:n].astype(np.int64).sum()) * 2 * Hkv * D * b_kv
    qo = n * H * D * 4
    print(f"[bench] cpu oracle: {n} seqs in {tn:.1f}s (median of 3) on {threads} threads",
          file=sys.stderr, flush=True)
    # the same oracle on one core, over a sample of about a third of the time
    oracle.set_threads(1)
    try:
        s1 = run(1)
        n1 = int(min(n, max(1, args.cpu_baseline_seconds / 9 / max(s1, 1e-6))))
        sn = median3(run, n1)
    finally:
        oracle.set_threads(threads)
    kv1 = int(ctx[:n1].astype(np.int64).sum()) * 2 * Hkv * D * b_kv
    print(f"[bench] cpu oracle, one core: {n1} seqs in {sn:.1f}s", file=sys.stderr, flush=True)
    return {
        "value": round((kv + qo) / tn / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"layer 0, first {n} of {len(ctx)} sequences ({int(ctx[:n].sum())} "
                  f"context tokens), fp64 C oracle, OpenMP over (seq, head)",
        "seq_layers_per_s": round(n / tn, 3),
        "seconds": round(tn, 2),
        "timing": "median of 3 runs of the sample",
        "host": host_info(),
        "single_core": {
            "value": round((kv1 + n1 * H * D * 4) / sn / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "sample": f"layer 0, first {n1} sequences ({int(ctx[:n1].sum())} context tokens)",
            "seq_layers_per_s": round(n1 / sn, 3),
            "seconds": round(sn, 2),
        },
    }


if __name__ == "__main__":
    main()
