"""A random serving trace driven through the host block manager.

The block manager (prefix cache on) serves a random mix of requests — new
prompts, half of them sharing a prefix with an earlier prompt ("LLM
inference basics and vLLM internals" §5: whole-block prefix hits), prefilled
in random chunks (§6: chunked prefill; a block becomes a hit only once the
chunk that fills it is marked computed, so later prompts, and prompts freed
half-way, exercise that rule), decode steps (appends, with copy-on-write
after forks, §4), forks, frees, and token evictions followed by a repack
(the "vToken" page).  A backend moves the data the manager's answers call
for — it writes only the tokens a prompt did not hit, runs the copy-on-write
copies before the step's writes, repacks evicted sequences — and attends.
Each chunk's tokens attend causally over everything written so far
(multi-token attention); after every completed prompt, decode step,
eviction and repack, every sequence's decode output is compared too, each
against textbook attention over that sequence's own K / V in logical order
(oracle/brute.py), so tables, hits, copies, writes, repacks and the
attention are checked together.

A token's K / V is a fixed function of the tokens up to it (a chained key
seeds its values), so a prompt that hits cached blocks finds exactly the
values it would have written itself.

Two backends: OracleBackend (numpy pools and the oracle's data movement and
attention, for the host logic on the CPU) and KernelBackend (the library's
kernels on the GPU).
"""
import numpy as np

import oracle
from oracle import brute
import workloads

D, L, NB = 128, 2, 700
SCALE = float(np.float32(1.0 / np.sqrt(D)))
NAN_BF16 = 0x7FC0
NAN_E4M3 = 0x7F
MAX_LIVE = 9


class Cfg:
    """Pool block size, kv dtype (bf16, or fp8 e4m3 written from bf16 with
    per-tensor scales) and head counts; queries are bf16."""

    def __init__(self, block_size=16, kv_dtype=oracle.BF16, k_scale=1.0, v_scale=1.0, heads=8, kv_heads=2):
        self.bs, self.kv = block_size, kv_dtype
        self.ks, self.vs = float(np.float32(k_scale)), float(np.float32(v_scale))
        self.h, self.hkv = heads, kv_heads

    def __repr__(self):
        return f"bs={self.bs} kv={'fp8' if self.kv == oracle.FP8 else 'bf16'} heads={self.h}/{self.hkv}"


def bf16_f64(bits):
    """Exact values of bf16 bits (the upper half of an fp32)."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def chain(key, tok):
    return hash((key, tok)) & ((1 << 62) - 1)


def stored_values(bits, kv, scale):
    """What the pool holds for bf16 source bits, as exact values: the bf16
    values, or the fp8 e4m3 code of fp32(x) * fp32(1 / scale) (the oracle's
    encoder) decoded and times the scale."""
    x = bf16_f64(bits)
    if kv == oracle.BF16:
        return x
    inv = np.float32(1.0) / np.float32(scale)
    codes = oracle.e4m3_encode(x.astype(np.float32) * inv)
    return oracle.e4m3_table()[codes.astype(np.int64)] * scale


class Truth:
    """The K / V of a token, a fixed function of its chained key: source
    bits ([L][H_kv][d] bf16) and the exact values the pool holds."""

    def __init__(self, cfg):
        self.cfg = cfg
        self.cache = {}

    def kv(self, key):
        if key not in self.cache:
            r = np.random.default_rng(key)
            kb = workloads.normal_bits(r, (L, self.cfg.hkv, D), oracle.BF16)
            vb = workloads.normal_bits(r, (L, self.cfg.hkv, D), oracle.BF16)
            c = self.cfg
            self.cache[key] = (kb, vb, stored_values(kb, c.kv, c.ks), stored_values(vb, c.kv, c.vs))
        return self.cache[key]


def poisoned_pool(cfg):
    n = oracle.layer_pool_bytes(NB, cfg.hkv, D, cfg.bs, cfg.kv)
    if cfg.kv == oracle.FP8:
        return np.full(n, NAN_E4M3, np.uint8)
    return np.full(n // 2, NAN_BF16, np.uint16).view(np.uint8)


class OracleBackend:
    """Pools as numpy bytes, moved and read by the oracle."""

    def __init__(self, cfg):
        self.c = cfg
        self.tol = 1e-9
        self.k = [poisoned_pool(cfg) for _ in range(L)]
        self.v = [poisoned_pool(cfg) for _ in range(L)]

    def write(self, layer, kb, vb, slots):
        c = self.c
        self.k[layer], self.v[layer] = oracle.reshape_and_cache(
            kb, vb, oracle.BF16, self.k[layer], self.v[layer], np.asarray(slots, np.int64), c.bs, NB, c.kv,
            c.ks, c.vs)

    def copy_blocks(self, pairs):
        bs = self.c.bs
        moves = [(s * bs + r, d * bs + r) for s, d in pairs for r in range(bs)]
        self.k, self.v = oracle.move_tokens(self.k, self.v, moves, self.c.hkv, D, bs, self.c.kv)

    def repack(self, tiles):
        bs = self.c.bs
        moves = [(src, blk * bs + r) for blk, srcs in tiles for r, src in enumerate(srcs)]
        self.k, self.v = oracle.move_tokens(self.k, self.v, moves, self.c.hkv, D, bs, self.c.kv)

    def decode(self, layer, q, tables, lens):
        c = self.c
        return oracle.paged_decode(q, oracle.BF16, self.k[layer], self.v[layer], c.kv, np.asarray(tables, np.int32),
                                   np.asarray(lens, np.int32), self.c.hkv, c.bs, SCALE, c.ks, c.vs)

    def prefill(self, layer, q, table, ctx):
        c = self.c
        n = q.shape[0]
        return oracle.paged_prefill(q, oracle.BF16, self.k[layer], self.v[layer], c.kv, np.asarray([table], np.int32),
                                    np.asarray([ctx], np.int32), np.asarray([0, n], np.int32), c.hkv, c.bs,
                                    SCALE, c.ks, c.vs)

    def decode_tokens(self, layer, q, table, lens):
        c = self.c
        return {"table": oracle.paged_decode_tokens(q, oracle.BF16, self.k[layer], self.v[layer], c.kv,
                                                    np.asarray(table, np.int32), np.asarray(lens, np.int32),
                                                    self.c.hkv, c.bs, SCALE, c.ks, c.vs)}


class KernelBackend:
    """Pools on the GPU, moved and read by the library's kernels (every call
    through the C ABI; outputs start as NaN)."""

    def __init__(self, pkv, torch, cfg):
        self.pkv, self.torch, self.c = pkv, torch, cfg
        self.tol = 6e-2 if cfg.kv == oracle.FP8 else 2e-2
        self.dt = pkv.FP8_E4M3 if cfg.kv == oracle.FP8 else pkv.BF16
        self.k = [torch.from_numpy(poisoned_pool(cfg)).to("cuda") for _ in range(L)]
        self.v = [torch.from_numpy(poisoned_pool(cfg)).to("cuda") for _ in range(L)]

    def _bf16(self, bits):
        t = self.torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(self.torch.bfloat16).to("cuda")

    def _i32(self, a):
        return self.torch.tensor(np.asarray(a, np.int32), dtype=self.torch.int32, device="cuda")

    def _out(self, S):
        return self.torch.full((S, self.c.h, D), float("nan"), dtype=self.torch.bfloat16, device="cuda")

    def _host(self, out):
        self.torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)

    def write(self, layer, kb, vb, slots):
        c = self.c
        self.pkv.reshape_and_cache(self._bf16(kb), self._bf16(vb), self.k[layer], self.v[layer],
                                   self._i32(slots), c.bs, NB, self.dt, c.ks, c.vs)

    def copy_blocks(self, pairs):
        self.pkv.copy_blocks(self.k, self.v, self._i32(pairs), NB, self.c.hkv, D, self.c.bs, self.dt)

    def repack(self, tiles):
        flat = self._i32([[blk] + list(srcs) for blk, srcs in tiles])
        self.pkv.repack_blocks(self.k, self.v, flat, self._i32([0, len(tiles)]), NB, self.c.hkv, D, self.c.bs,
                               self.dt)

    def decode(self, layer, q, tables, lens):
        c = self.c
        out = self._out(len(lens))
        self.pkv.paged_attention_decode(out, self._bf16(q), self.k[layer], self.v[layer], self._i32(tables),
                                        self._i32(lens), int(max(lens)), c.hkv, c.bs, self.dt, SCALE, c.ks, c.vs,
                                        num_blocks=NB, partition_tokens=4 * c.bs)
        return self._host(out)

    def prefill(self, layer, q, table, ctx):
        c = self.c
        n = q.shape[0]
        out = self.torch.full((n, self.c.h, D), float("nan"), dtype=self.torch.bfloat16, device="cuda")
        self.pkv.paged_attention_prefill(out, self._bf16(q), self.k[layer], self.v[layer], self._i32([table]),
                                         self._i32([ctx]), self._i32([0, n]), n, ctx, c.hkv, c.bs, self.dt,
                                         SCALE, c.ks, c.vs, num_blocks=NB)
        return self._host(out)

    def decode_tokens(self, layer, q, table, lens):
        pkv, c = self.pkv, self.c
        tt, cl, qt = self._i32(table), self._i32(lens), self._bf16(q)
        width = tt.shape[1]
        res = {}
        out = self._out(len(lens))
        pkv.paged_attention_decode_tokens(out, qt, self.k[layer], self.v[layer], tt, cl, c.hkv, c.bs, NB, self.dt,
                                          SCALE, c.ks, c.vs)
        res["gather"] = self._host(out)
        for min_keys in (0, pkv.RUNS_MIN_KEYS):
            runs = pkv.token_runs(tt, cl, c.bs, NB, min_keys_per_entry=min_keys)
            out = self._out(len(lens))
            pkv.paged_attention_decode_runs(out, qt, self.k[layer], self.v[layer], runs, width, c.hkv, c.bs, NB,
                                            self.dt, SCALE, c.ks, c.vs, token_slots=tt, context_lens=cl)
            res[f"runs (min keys {min_keys})"] = self._host(out)
        return res


def check(got, q, seqs, sids, layer, tol, label):
    """Each sequence's output against contiguous attention over its own
    tokens' K / V in logical order."""
    for i, sid in enumerate(sids):
        kv = seqs[sid]["kv"]
        k = np.stack([t[2][layer] for t in kv])
        v = np.stack([t[3][layer] for t in kv])
        want = brute.attention(bf16_f64(q[i]), k, v, SCALE)
        err = float(np.abs(got[i] - want).max())
        assert err <= tol, f"{label} layer {layer}: sequence {sid} ({len(kv)} tokens) max-abs {err}"


def run_trace(seed, pkv, dev, cfg, num_ops=70, log=print):
    """Drive num_ops random requests; returns counts of what ran."""
    r = np.random.default_rng(seed)
    truth = Truth(cfg)
    BS = cfg.bs
    bm = pkv.BlockManager(NB, BS, prefix_caching=True)
    # sid -> {"keys": chained key per token, "kv": Truth.kv per token,
    #         "done": tokens whose K / V are written, "evicted"}
    seqs = {}
    prompts = []              # prompts seen so far (prefix sources)
    next_sid = 0
    stats = dict(prompts=0, hit_tokens=0, chunks=0, steps=0, cow=0, forks=0, frees=0, evictions=0,
                 repacked_tiles=0, freed_mid_prefill=0)

    def write(triples):
        """(sid, position, slot) triples: their K / V into every layer."""
        if not triples:
            return
        slots = [sl for _, _, sl in triples]
        for layer in range(L):
            kb = np.stack([seqs[s]["kv"][p][0][layer] for s, p, _ in triples])
            vb = np.stack([seqs[s]["kv"][p][1][layer] for s, p, _ in triples])
            dev.write(layer, kb, vb, slots)

    def decode_all(sids, label):
        maxb = max(-(-bm.num_tokens(s) // BS) for s in sids)
        tables = [bm.block_table(s, maxb) for s in sids]
        lens = [bm.num_tokens(s) for s in sids]
        assert lens == [len(seqs[s]["kv"]) for s in sids]
        for layer in range(L):
            q = workloads.normal_bits(r, (len(sids), cfg.h, D), oracle.BF16)
            check(dev.decode(layer, q, tables, lens), q, seqs, sids, layer, dev.tol, label)

    def prefill_chunk(sid, label):
        """Write the next chunk of a prompt (the whole rest, or a random
        part), attend with its tokens as queries over everything written so
        far (multi-token causal attention), then mark it computed."""
        s = seqs[sid]
        p0, n_all = s["done"], len(s["kv"])
        n = n_all - p0 if r.random() < 0.4 else int(r.integers(1, n_all - p0 + 1))
        p1 = p0 + n
        write([(sid, p0 + i, sl) for i, sl in enumerate(bm.slots(sid, p0, n))])
        table = bm.block_table(sid, -(-n_all // BS))
        for layer in range(L):
            q = workloads.normal_bits(r, (n, cfg.h, D), oracle.BF16)
            got = dev.prefill(layer, q, table, p1)
            k = np.stack([t[2][layer] for t in s["kv"][:p1]])
            v = np.stack([t[3][layer] for t in s["kv"][:p1]])
            want = brute.causal_chunk(bf16_f64(q), k, v, SCALE)
            err = float(np.abs(got - want).max())
            assert err <= dev.tol, f"{label} layer {layer}: chunk {p0}..{p1} of sequence {sid} max-abs {err}"
        bm.mark_computed(sid, p1)
        s["done"] = p1
        stats["chunks"] += 1
        if p1 == n_all:
            decode_all([sid], f"{label}, prompt complete")

    for op_i in range(num_ops):
        live = list(seqs)
        growable = [s for s in live if not seqs[s]["evicted"] and seqs[s]["done"] == len(seqs[s]["kv"])]
        prefilling = [s for s in live if seqs[s]["done"] < len(seqs[s]["kv"])]
        u = r.random()
        if u < 0.25 or not live:
            if len(live) >= MAX_LIVE:
                continue
            n = int(r.integers(20, 260))
            if prompts and r.random() < 0.5:
                src = prompts[int(r.integers(len(prompts)))]
                k = int(r.integers(1, len(src) + 1))
                toks = list(src[:k]) + [int(x) for x in r.integers(0, 1000, max(0, n - k))]
            else:
                toks = [int(x) for x in r.integers(0, 1000, n)]
            sid = next_sid
            next_sid += 1
            hit = bm.add_sequence(sid, toks)
            assert hit % BS == 0 and 0 <= hit <= len(toks)
            keys, key = [], seed
            for t in toks:
                key = chain(key, t)
                keys.append(key)
            assert hit < len(toks)                 # the last token is always computed
            seqs[sid] = {"keys": keys, "kv": [truth.kv(kk) for kk in keys], "done": hit, "evicted": False}
            prompts.append(toks)
            stats["prompts"] += 1
            stats["hit_tokens"] += hit
            prefill_chunk(sid, f"op {op_i} prompt ({hit} of {len(toks)} tokens hit)")
        elif u < 0.35 and prefilling:
            sid = int(r.choice(prefilling))
            prefill_chunk(sid, f"op {op_i} next chunk")
        elif u < 0.65 and growable:
            # one decode step for a random subset: copy-on-write copies, then
            # the new tokens' K / V, then attention
            batch = sorted(set(int(x) for x in r.choice(growable, int(r.integers(1, len(growable) + 1)))))
            pairs, writes = [], []
            for sid in batch:
                tok = int(r.integers(0, 1000))
                slot, src, dst = bm.append_token(sid, tok)
                s = seqs[sid]
                key = chain(s["keys"][-1], tok)
                s["keys"].append(key)
                s["kv"].append(truth.kv(key))
                s["done"] += 1                     # the step writes it
                if src >= 0:
                    pairs.append((src, dst))
                writes.append((sid, len(s["kv"]) - 1, slot))
            if pairs:
                dev.copy_blocks(pairs)
                stats["cow"] += len(pairs)
            write(writes)
            decode_all(batch, f"op {op_i} decode step")
            stats["steps"] += 1
        elif u < 0.75 and growable:
            parent = int(r.choice(growable))
            child = next_sid
            next_sid += 1
            bm.fork(parent, child)
            p = seqs[parent]
            seqs[child] = {"keys": list(p["keys"]), "kv": list(p["kv"]), "done": p["done"], "evicted": False}
            stats["forks"] += 1
        elif u < 0.85 and live:
            sid = int(r.choice(live))
            bm.free_sequence(sid)
            stats["freed_mid_prefill"] += sid in prefilling
            del seqs[sid]
            stats["frees"] += 1
        else:
            # drop about half of a sequence's tokens (it must own its blocks
            # alone), attend through the token table, repack, attend through
            # the block table
            alone = [s for s in growable
                     if all(bm.ref_count(b) == 1 for b in bm.block_table(s, -(-bm.num_tokens(s) // BS)))]
            if not alone:
                continue
            sid = int(r.choice(alone))
            s = seqs[sid]
            keep = [bool(x) for x in (r.random(len(s["kv"])) < float(r.choice([0.2, 0.5, 0.9])))]
            keep[-1] = True
            bm.evict_tokens(sid, keep)
            s["kv"] = [kv for kv, k in zip(s["kv"], keep) if k]
            s["done"] = len(s["kv"])
            s["keys"] = [kk for kk, k in zip(s["keys"], keep) if k]
            m = len(s["kv"])
            table = [bm.token_slots(sid, m)]
            for layer in range(L):
                q = workloads.normal_bits(r, (1, cfg.h, D), oracle.BF16)
                for path, got in dev.decode_tokens(layer, q, table, [m]).items():
                    check(got, q, seqs, [sid], layer, dev.tol, f"op {op_i} evicted, {path}")
            tiles = bm.repack_tiles(sid)
            if tiles:
                dev.repack(tiles)
            stats["repacked_tiles"] += len(tiles)
            decode_all([sid], f"op {op_i} after repack")
            stats["evictions"] += 1
    log(f"seed {seed} {cfg}: {stats}")
    return stats
