"""Reference model of the block pool — TEST INFRASTRUCTURE ONLY (same rule
as the rest of oracle/: imported by tests/ only).

A plain, slow model of what the block manager computes, written from the
pages, sharing no code with the library:

  [P1] "LLM inference basics and vLLM internals" (ttlab.hopto.org),
       §4 PagedAttention and block management: blocks of 16 tokens handed
       out one at a time, a per-request table from logical to physical
       blocks, waste only in a request's last block, one physical block
       shared by equal prefixes (reference count, copy-on-write), a free
       queue, block 0 reserved as the null block.
       §5 prefix cache: a block's hash comes from its parent's hash, its
       tokens and extra keys, so only prefixes match; only full blocks are
       cached, hits are whole blocks, the last prompt token is always
       recomputed; a finished request gives its blocks back with their
       content, the queue front is reused first (least recently used), and
       a request gives its blocks back last block first.
       §9 / §10: the LRU experiment and the block-level model of it.
  [P2] "vLLM internals (2)" (youngju.dev), "Sharing".

Readings (where the pages leave it open):
  - free blocks that hold no reusable content (never used, or a partial
    block, which has no hash) are handed out before any cached block is
    evicted — the block model of [P1] §10 does this, and it is the reading
    under which that model prints 0 / 0 / 21,488;
  - content keys are exact: key(block j) = (key(block j-1), its tokens),
    rooted at the extra key.  A hash of that chain, as the pages describe,
    matches exactly these keys up to collisions;
  - "only full blocks are cached" (§5) is read together with §6's chunked
    prefill, where a prompt's K/V is computed over several steps: a block
    counts as full once the K/V of its last token is computed.  So a
    block becomes findable only when the caller marks the tokens up to its
    end computed (mark_computed); a prompt's hit blocks are computed from
    the start, and a token appended to a sequence whose every token is
    computed counts as computed at once (the decode step that appends it
    writes its K/V).  A block freed before it was computed was never
    findable and goes back as a clean block.  Content already cached under
    the same key is not published twice.
"""


class BlockPoolModel:
    """One block pool.  Block ids 1..num_blocks-1 are usable; 0 is null."""

    def __init__(self, num_blocks, block_size, prefix_caching=False):
        self.bs = block_size
        self.prefix = prefix_caching
        self.ref = [0] * num_blocks
        self.ref[0] = 1                              # the null block stays taken
        self.clean = list(range(1, num_blocks))      # free, nothing cached; front first
        self.cached = []                             # free, cached content; front = least recently freed
        self.key_of = {}                             # block -> content key
        self.block_of = {}                           # content key -> block
        self.seqs = {}                               # id -> {"blocks", "tokens", "keys", "root"}

    # -- pool ([P1] §4 free queue; §5 reuse order) --------------------------
    def free_count(self):
        return len(self.clean) + len(self.cached)

    num_free_blocks = free_count

    def num_cached_free_blocks(self):
        return len(self.cached)

    def ref_count(self, b):
        return self.ref[b]

    def _take(self):
        if self.clean:
            b = self.clean.pop(0)
        else:
            b = self.cached.pop(0)                   # evict: its content is gone
            del self.block_of[self.key_of.pop(b)]
        self.ref[b] = 1
        return b

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            (self.cached if b in self.key_of else self.clean).append(b)

    def _publish(self, b, key):
        if key not in self.block_of:
            self.block_of[key] = b
            self.key_of[b] = key

    # -- requests -------------------------------------------------------------
    def add_sequence(self, sid, tokens, extra_key=0):
        """Blocks for a prompt; returns the number of tokens served from the
        prefix cache ([P1] §5)."""
        assert sid not in self.seqs
        bs, n = self.bs, len(tokens)
        nblk = -(-n // bs)
        root = ("root", extra_key)
        keys, k = [], root
        for j in range(n // bs):
            k = (k, tuple(tokens[j * bs:(j + 1) * bs]))
            keys.append(k)
        hits = []
        if self.prefix:
            for j, k in enumerate(keys):
                if (j + 1) * bs > n - 1 or k not in self.block_of:
                    break
                hits.append(self.block_of[k])
        free_hits = sum(1 for b in hits if self.ref[b] == 0)
        need = nblk - len(hits)
        if need > self.free_count() - free_hits:
            raise MemoryError("not enough free blocks")
        blocks = []
        for b in hits:
            if self.ref[b] == 0:
                self.cached.remove(b)
            self.ref[b] += 1
            blocks.append(b)
        for j in range(len(hits), nblk):
            blocks.append(self._take())
        self.seqs[sid] = {"blocks": blocks, "tokens": list(tokens), "keys": keys, "root": root,
                          "computed": len(hits) * bs}
        return len(hits) * bs

    def mark_computed(self, sid, n):
        """The K/V of the sequence's first n tokens are written: full blocks
        inside them become findable ([P1] §5, read with §6)."""
        s = self.seqs[sid]
        if not 0 <= n <= len(s["tokens"]):
            raise ValueError("computed count outside the sequence")
        old = s["computed"]
        if n <= old:
            return
        s["computed"] = n
        if not self.prefix or s.get("evicted"):
            return
        bs = self.bs
        for j in range(len(s["keys"])):
            if old < (j + 1) * bs <= n:
                self._publish(s["blocks"][j], s["keys"][j])

    def num_computed_tokens(self, sid):
        return self.seqs[sid]["computed"]

    def append_token(self, sid, token=0):
        """Returns (slot, cow_src, cow_dst) ([P1] §4; copy-on-write)."""
        s = self.seqs[sid]
        if "slots" in s:
            raise ValueError("evicted tokens: repack first")
        bs = self.bs
        pos = len(s["tokens"])
        j, off = divmod(pos, bs)
        src = dst = -1
        if off == 0:
            if self.free_count() < 1:
                raise MemoryError("no free block")
            s["blocks"].append(self._take())
        elif self.ref[s["blocks"][j]] > 1:
            if self.free_count() < 1:
                raise MemoryError("no free block for copy-on-write")
            src = s["blocks"][j]
            dst = self._take()
            self._release(src)
            s["blocks"][j] = dst
        done = s["computed"] == len(s["tokens"])
        s["tokens"].append(token)
        if off == bs - 1 and not s.get("evicted"):
            parent = s["keys"][j - 1] if j else s["root"]
            s["keys"].append((parent, tuple(s["tokens"][j * bs:(j + 1) * bs])))
        if done:                                     # a decode step writes the token it appends
            self.mark_computed(sid, len(s["tokens"]))
        return s["blocks"][j] * bs + off, src, dst

    def fork(self, parent, child):
        assert child not in self.seqs
        p = self.seqs[parent]
        if "slots" in p:
            raise ValueError("evicted tokens: repack first")
        self.seqs[child] = {"blocks": list(p["blocks"]), "tokens": list(p["tokens"]),
                            "keys": list(p["keys"]), "root": p["root"],
                            "computed": p["computed"]}
        if p.get("evicted"):
            self.seqs[child]["evicted"] = True
        for b in p["blocks"]:
            self.ref[b] += 1

    def free_sequence(self, sid):
        s = self.seqs.pop(sid)
        for b in reversed(s["blocks"]):              # last block first ([P1] §5)
            self._release(b)

    def block_table(self, sid):
        return list(self.seqs[sid]["blocks"])

    # -- token-level virtualisation ("vToken" page) ---------------------------
    # A sequence's logical tokens each have a physical slot; normally slot(t)
    # = blocks[t // bs] * bs + t % bs.  Evicting tokens leaves the survivors
    # where they are (their slots in logical order form the token table);
    # repacking moves them so that the table is block-aligned again and the
    # emptied blocks can be freed.  Readings: a sequence whose blocks are
    # shared cannot evict (its blocks would change under other readers);
    # evicted content is no longer the hashed prefix, so the blocks lose
    # their cached content, and the sequence never publishes content again
    # (the K/V of its later tokens were computed with the evicted ones in
    # context, so they match no prompt); repacking fills the sequence's own blocks in
    # order (all sources are read before any destination is written), frees
    # the blocks it no longer needs last block first, and a sequence must be
    # repacked before it grows again.
    def token_slots(self, sid):
        s = self.seqs[sid]
        if "slots" in s:
            return list(s["slots"])
        bs = self.bs
        return [s["blocks"][t // bs] * bs + t % bs for t in range(len(s["tokens"]))]

    def evict_tokens(self, sid, keep):
        s = self.seqs[sid]
        assert len(keep) == len(s["tokens"])
        if any(self.ref[b] != 1 for b in s["blocks"]):
            raise ValueError("shared blocks")
        slots = self.token_slots(sid)
        s["slots"] = [sl for sl, k in zip(slots, keep) if k]
        s["tokens"] = [t for t, k in zip(s["tokens"], keep) if k]
        s["keys"] = []
        s["computed"] = len(s["tokens"])
        s["evicted"] = True      # its K/V no longer match any prompt: never published again
        for b in s["blocks"]:
            if b in self.key_of:
                del self.block_of[self.key_of.pop(b)]

    def repack(self, sid):
        """Returns the (src_slot, dst_slot) moves that make the table aligned."""
        s = self.seqs[sid]
        bs = self.bs
        cur = self.token_slots(sid)
        n = len(cur)
        keep_blocks = -(-n // bs)
        moves = []
        for q, src in enumerate(cur):
            dst = s["blocks"][q // bs] * bs + q % bs
            if src != dst:
                moves.append((src, dst))
        for b in reversed(s["blocks"][keep_blocks:]):
            self._release(b)
        s["blocks"] = s["blocks"][:keep_blocks]
        s.pop("slots", None)
        return moves

    def repack_tiles(self, sid):
        """The same repack as repack(), as whole blocks: [(block, [source
        slot of each row])] for every remaining block that receives a moved
        token, in block order; rows that keep their token or lie past the
        last survivor name their own slot."""
        s = self.seqs[sid]
        bs = self.bs
        cur = self.token_slots(sid)
        n = len(cur)
        tiles = []
        for j in range(-(-n // bs)):
            b = s["blocks"][j]
            src = [cur[j * bs + i] if j * bs + i < n else b * bs + i for i in range(bs)]
            if any(x != b * bs + i for i, x in enumerate(src)):
                tiles.append((b, src))
        self.repack(sid)
        return tiles

    def slots(self, sid, first, count):
        bl = self.seqs[sid]["blocks"]
        return [bl[p // self.bs] * self.bs + p % self.bs for p in range(first, first + count)]


def copy_blocks(k_pools, v_pools, pairs, block_bytes):
    """Copy-on-write copies ([P1] §4): for every (src, dst) pair, the bytes
    of physical block src (all kv heads) in every layer's K and V pool
    (numpy uint8 arrays, modified in place) replace those of block dst.
    Pairs naming block 0, a block outside the pool, or src == dst are
    skipped."""
    for pool in list(k_pools) + list(v_pools):
        nb = len(pool) // block_bytes
        for src, dst in pairs:
            if 1 <= src < nb and 1 <= dst < nb and src != dst:
                pool[dst * block_bytes:(dst + 1) * block_bytes] = \
                    pool[src * block_bytes:(src + 1) * block_bytes]
