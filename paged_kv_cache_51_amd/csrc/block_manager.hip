// block_manager.hip — the block pool that produces the block tables and slot
// mappings the decode path consumes, with reference counts, copy-on-write,
// and the prefix cache; plus the copy_blocks kernel that performs the
// copies copy-on-write asks for.
//
// What is modelled ("LLM inference basics and vLLM internals" §4 and §5,
// "vLLM internals (2)" "Sharing"):
//   - the pool hands out fixed-size physical blocks one at a time as a
//     request grows; block 0 is reserved as the null block and never handed
//     out;
//   - a request's logical block j maps to a physical block through its
//     block table; requests with the same prefix can point at one physical
//     block, which then carries a reference count > 1; writing into a shared,
//     partly filled block first copies it to a private block
//     (copy-on-write);
//   - prefix cache: every full block gets a hash chained from its parent
//     block's hash, its tokens and an extra key (LoRA id, salt, ...), so a
//     block only matches when everything before it matches too; only full
//     blocks are cached, so hits come in whole blocks, and a prompt always
//     recomputes at least its last token.  A finished request returns its
//     blocks with their content kept; blocks are reused least recently freed
//     first, and a request returns its blocks last-block first, so the tail
//     of a cached prompt is given up before its head.
//
// "Only full blocks are cached" is read together with chunked prefill (§6),
// which computes a prompt's K/V over several steps: a block counts as full
// once the K/V of its last token is computed.  A block therefore becomes
// findable only when the caller marks the tokens up to its end computed
// (pkv_bm_mark_computed, once the step that writes them is enqueued); a
// prompt's hit blocks are computed from the start, and a token appended to a
// sequence whose every token is computed counts as computed at once (the
// decode step that appends it writes its K/V).  A block freed before it was
// computed was never findable and returns as a clean block.
//
// Reading where the pages leave the order open (their own block-level model
// of the LRU experiment in §10 takes it): a free block that holds no cached
// content (never used, or a partial block, which has no hash) is handed out
// before any cached block is evicted.  With that reading the model of §9/§10
// (1,344 usable blocks, ten 5,033-token documents read in order, again in
// order, then reversed) gives 0 / 0 / 21,488 hit tokens, the figures the
// pages print; a single first-in-first-out queue for all free blocks gives
// 21,376 for the third pass.
//
// Host-side state, single-threaded: a pkv_block_manager must not be used by
// two threads at once.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kClean = 0;    // free, no cached content
constexpr int kCached = 1;   // free, holds a full block's cached content
constexpr int kInUse = 2;

// 64-bit FNV-1a (Fowler-Noll-Vo) over the bytes of the values fed to it.
struct Fnv1a {
    uint64_t h = 0xcbf29ce484222325ull;
    void bytes(const void* p, size_t n) {
        const unsigned char* c = static_cast<const unsigned char*>(p);
        for (size_t i = 0; i < n; ++i) {
            h ^= c[i];
            h *= 0x100000001b3ull;
        }
    }
};

uint64_t chain_seed(uint64_t extra_key) {
    Fnv1a f;
    const char tag[] = "pkv-prefix-root";
    f.bytes(tag, sizeof tag);
    f.bytes(&extra_key, sizeof extra_key);
    return f.h;
}

uint64_t block_hash(uint64_t parent, const int32_t* tokens, int n) {
    Fnv1a f;
    f.bytes(&parent, sizeof parent);
    f.bytes(tokens, sizeof(int32_t) * (size_t)n);
    return f.h;
}

struct Sequence {
    std::vector<int32_t> blocks;   // block table
    std::vector<int32_t> tokens;   // kept only with the prefix cache
    std::vector<uint64_t> chain;   // content hash of each full block so far
    std::vector<int32_t> slots;    // per-token slots after an eviction (else empty)
    bool fragmented = false;       // tokens evicted and not yet repacked
    bool evicted = false;          // ever lost tokens: its K/V match no prompt, never published
    int32_t num_tokens = 0;
    int32_t num_computed = 0;      // leading tokens whose K/V are written
    uint64_t seed = 0;
};

}  // namespace

struct BlockManager {
    int32_t num_blocks = 0, block_size = 0;
    bool prefix_cache = false;
    std::vector<int32_t> ref;
    // two intrusive doubly-linked queues of free blocks (kClean, kCached)
    std::vector<int32_t> prev, next;
    std::vector<uint8_t> state;
    int32_t head[2] = {-1, -1}, tail[2] = {-1, -1}, count[2] = {0, 0};
    // cached content of a block: its hash, its parent's hash, its tokens
    std::vector<uint8_t> hashed;
    std::vector<uint64_t> hash, parent;
    std::vector<int32_t> content;
    std::unordered_map<uint64_t, int32_t> by_hash;
    std::unordered_map<int64_t, Sequence> seqs;

    void push_back(int q, int32_t b) {
        state[b] = (uint8_t)q;
        prev[b] = tail[q];
        next[b] = -1;
        if (tail[q] >= 0) next[tail[q]] = b; else head[q] = b;
        tail[q] = b;
        ++count[q];
    }
    void unlink(int32_t b) {
        const int q = state[b];
        if (prev[b] >= 0) next[prev[b]] = next[b]; else head[q] = next[b];
        if (next[b] >= 0) prev[next[b]] = prev[b]; else tail[q] = prev[b];
        prev[b] = next[b] = -1;
        --count[q];
        state[b] = kInUse;
    }
    void drop_content(int32_t b) {
        if (!hashed[b]) return;
        auto it = by_hash.find(hash[b]);
        if (it != by_hash.end() && it->second == b) by_hash.erase(it);
        hashed[b] = 0;
    }
    // A free block for new content: clean ones first, else evict the least
    // recently freed cached one.  Caller checked availability.
    int32_t take() {
        const int q = count[kClean] > 0 ? kClean : kCached;
        const int32_t b = head[q];
        unlink(b);
        drop_content(b);
        ref[b] = 1;
        return b;
    }
    int32_t available() const { return count[kClean] + count[kCached]; }
    void release(int32_t b) {
        if (--ref[b] == 0) push_back(hashed[b] ? kCached : kClean, b);
    }
    // Block b (exclusively owned, full) now holds the tokens of a full block
    // with content hash h and parent hash p: make it findable, unless the
    // same content is cached already.
    void publish(int32_t b, uint64_t h, uint64_t p, const int32_t* toks) {
        if (by_hash.count(h)) return;
        hashed[b] = 1;
        hash[b] = h;
        parent[b] = p;
        std::memcpy(&content[(size_t)b * block_size], toks, sizeof(int32_t) * (size_t)block_size);
        by_hash.emplace(h, b);
    }
    // The K/V of the sequence's first n tokens are written: publish its full
    // blocks that end inside them and did not end inside the old count.
    void mark_computed(Sequence& sq, int32_t n) {
        const int32_t old = sq.num_computed;
        if (n <= old) return;
        sq.num_computed = n;
        if (!prefix_cache || sq.evicted) return;
        const int32_t bs = block_size;
        for (int32_t j = old / bs; j < (int32_t)sq.chain.size() && (j + 1) * bs <= n; ++j)
            publish(sq.blocks[j], sq.chain[j], j ? sq.chain[j - 1] : sq.seed, &sq.tokens[(size_t)j * bs]);
    }
    // The cached block holding (h, p, toks), or -1.
    int32_t lookup(uint64_t h, uint64_t p, const int32_t* toks) const {
        auto it = by_hash.find(h);
        if (it == by_hash.end()) return -1;
        const int32_t b = it->second;
        if (!hashed[b] || parent[b] != p ||
            std::memcmp(&content[(size_t)b * block_size], toks, sizeof(int32_t) * (size_t)block_size))
            return -1;
        return b;
    }
};

}  // namespace pkv

struct pkv_block_manager {
    pkv::BlockManager m;
};

using pkv::fail;
using pkv::ok;

namespace {
pkv::Sequence* find_seq(pkv_block_manager* bm, int64_t id) {
    auto it = bm->m.seqs.find(id);
    return it == bm->m.seqs.end() ? nullptr : &it->second;
}
}  // namespace

extern "C" {

int32_t pkv_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching,
                      pkv_block_manager** out) {
    if (!out) return fail(PKV_ERR_ARG, "null output handle");
    *out = nullptr;
    if (num_blocks < 1 || block_size <= 0 || block_size > 4096)
        return fail(PKV_ERR_ARG, "need num_blocks >= 1 and 0 < block_size <= 4096");
    pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
    if (!bm) return fail(PKV_ERR_SIZE, "out of host memory");
    pkv::BlockManager& m = bm->m;
    try {
        m.num_blocks = num_blocks;
        m.block_size = block_size;
        m.prefix_cache = prefix_caching != 0;
        m.ref.assign(num_blocks, 0);
        m.prev.assign(num_blocks, -1);
        m.next.assign(num_blocks, -1);
        m.state.assign(num_blocks, pkv::kInUse);
        m.hashed.assign(num_blocks, 0);
        m.hash.assign(num_blocks, 0);
        m.parent.assign(num_blocks, 0);
        if (m.prefix_cache) m.content.assign((size_t)num_blocks * block_size, 0);
    } catch (...) {
        delete bm;
        return fail(PKV_ERR_SIZE, "out of host memory");
    }
    // block 0 is the null block: permanently referenced, never free
    m.ref[0] = 1;
    for (int32_t b = 1; b < num_blocks; ++b) m.push_back(pkv::kClean, b);
    *out = bm;
    return ok();
}

int32_t pkv_bm_destroy(pkv_block_manager* bm) {
    delete bm;
    return ok();
}

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) {
    if (!bm) return fail(PKV_ERR_ARG, "null handle");
    return bm->m.available();
}

int32_t pkv_bm_num_cached_free_blocks(const pkv_block_manager* bm) {
    if (!bm) return fail(PKV_ERR_ARG, "null handle");
    return bm->m.count[pkv::kCached];
}

int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block) {
    if (!bm) return fail(PKV_ERR_ARG, "null handle");
    if (block < 0 || block >= bm->m.num_blocks) return fail(PKV_ERR_ARG, "block %d out of range", block);
    return bm->m.ref[block];
}

int32_t pkv_bm_num_tokens(const pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return fail(PKV_ERR_ARG, "null handle");
    const pkv::Sequence* sq = find_seq(const_cast<pkv_block_manager*>(bm), seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    return sq->num_tokens;
}

int32_t pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                            int32_t num_tokens, uint64_t extra_key, int32_t* num_cached_tokens) {
    if (!bm || (num_tokens > 0 && !tokens)) return fail(PKV_ERR_ARG, "null pointer");
    if (num_tokens < 0) return fail(PKV_ERR_ARG, "negative token count");
    if (find_seq(bm, seq_id)) return fail(PKV_ERR_ARG, "sequence %lld exists", (long long)seq_id);
    pkv::BlockManager& m = bm->m;
    const int bs = m.block_size;
    const int32_t nblk = (num_tokens + bs - 1) / bs;
    const int32_t nfull = num_tokens / bs;
    const uint64_t seed = pkv::chain_seed(extra_key);

    // content hashes of the full blocks, and the longest cached prefix of
    // them that still leaves the last prompt token to compute
    std::vector<uint64_t> chain;
    std::vector<int32_t> hits;
    if (m.prefix_cache) {
        uint64_t p = seed;
        chain.reserve(nfull);
        for (int32_t j = 0; j < nfull; ++j) {
            const uint64_t h = pkv::block_hash(p, tokens + (int64_t)j * bs, bs);
            if ((int32_t)hits.size() == j && (int64_t)(j + 1) * bs <= (int64_t)num_tokens - 1) {
                const int32_t b = m.lookup(h, p, tokens + (int64_t)j * bs);
                if (b >= 0) hits.push_back(b);
            }
            chain.push_back(h);
            p = h;
        }
    }
    int32_t hit_free = 0;   // hit blocks now free (they leave the free queue)
    for (int32_t b : hits) hit_free += m.ref[b] == 0;
    const int32_t need = nblk - (int32_t)hits.size();
    if (need > m.available() - hit_free)
        return fail(PKV_ERR_SIZE, "need %d free blocks, %d available", need, m.available() - hit_free);

    pkv::Sequence sq;
    try {
        sq.blocks.reserve(nblk);
        if (m.prefix_cache) sq.tokens.assign(tokens, tokens + num_tokens);
    } catch (...) {
        return fail(PKV_ERR_SIZE, "out of host memory");
    }
    for (int32_t b : hits) {
        if (m.ref[b] == 0) m.unlink(b);
        ++m.ref[b];
        sq.blocks.push_back(b);
    }
    for (int32_t j = (int32_t)hits.size(); j < nblk; ++j) sq.blocks.push_back(m.take());
    sq.chain = std::move(chain);
    sq.num_tokens = num_tokens;
    sq.num_computed = (int32_t)hits.size() * bs;   // the hit blocks hold their K/V already
    sq.seed = seed;
    m.seqs.emplace(seq_id, std::move(sq));
    if (num_cached_tokens) *num_cached_tokens = (int32_t)hits.size() * bs;
    return ok();
}

int32_t pkv_bm_append_token(pkv_block_manager* bm, int64_t seq_id, int32_t token, int32_t* slot,
                            int32_t* cow_src, int32_t* cow_dst) {
    if (!bm || !slot) return fail(PKV_ERR_ARG, "null pointer");
    pkv::Sequence* sq = find_seq(bm, seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    if (sq->fragmented) return fail(PKV_ERR_ARG, "sequence %lld has evicted tokens: repack it first", (long long)seq_id);
    pkv::BlockManager& m = bm->m;
    const int bs = m.block_size;
    const int32_t pos = sq->num_tokens;
    const int32_t j = pos / bs, off = pos % bs;
    int32_t src = -1, dst = -1;
    if (off == 0) {
        if (m.available() < 1) return fail(PKV_ERR_SIZE, "no free block");
        sq->blocks.push_back(m.take());
    } else if (m.ref[sq->blocks[j]] > 1) {
        // shared partial block: write into a private copy
        if (m.available() < 1) return fail(PKV_ERR_SIZE, "no free block for copy-on-write");
        src = sq->blocks[j];
        dst = m.take();
        m.release(src);
        sq->blocks[j] = dst;
    }
    if (m.prefix_cache && !sq->evicted) {
        sq->tokens.push_back(token);
        if (off == bs - 1) {
            const uint64_t p = j ? sq->chain[j - 1] : sq->seed;
            sq->chain.push_back(pkv::block_hash(p, &sq->tokens[(size_t)j * bs], bs));
        }
    }
    const bool all_computed = sq->num_computed == sq->num_tokens;
    ++sq->num_tokens;
    if (all_computed) m.mark_computed(*sq, sq->num_tokens);   // a decode step writes it
    *slot = sq->blocks[j] * bs + off;
    if (cow_src) *cow_src = src;
    if (cow_dst) *cow_dst = dst;
    return ok();
}

int32_t pkv_bm_mark_computed(pkv_block_manager* bm, int64_t seq_id, int32_t num_computed_tokens) {
    if (!bm) return fail(PKV_ERR_ARG, "null handle");
    pkv::Sequence* sq = find_seq(bm, seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    if (num_computed_tokens < 0 || num_computed_tokens > sq->num_tokens)
        return fail(PKV_ERR_ARG, "computed count %d outside the sequence's %d tokens", num_computed_tokens,
                    sq->num_tokens);
    bm->m.mark_computed(*sq, num_computed_tokens);
    return ok();
}

int32_t pkv_bm_num_computed_tokens(const pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return fail(PKV_ERR_ARG, "null handle");
    const pkv::Sequence* sq = find_seq(const_cast<pkv_block_manager*>(bm), seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    return sq->num_computed;
}

int32_t pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id) {
    if (!bm) return fail(PKV_ERR_ARG, "null handle");
    pkv::Sequence* par = find_seq(bm, parent_id);
    if (!par) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)parent_id);
    if (par->fragmented) return fail(PKV_ERR_ARG, "sequence %lld has evicted tokens: repack it first", (long long)parent_id);
    if (find_seq(bm, child_id)) return fail(PKV_ERR_ARG, "sequence %lld exists", (long long)child_id);
    pkv::Sequence copy;
    try {
        copy = *par;
    } catch (...) {
        return fail(PKV_ERR_SIZE, "out of host memory");
    }
    for (int32_t b : copy.blocks) ++bm->m.ref[b];
    bm->m.seqs.emplace(child_id, std::move(copy));
    return ok();
}

int32_t pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return fail(PKV_ERR_ARG, "null handle");
    auto it = bm->m.seqs.find(seq_id);
    if (it == bm->m.seqs.end()) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    const std::vector<int32_t>& bl = it->second.blocks;
    for (size_t i = bl.size(); i-- > 0;) bm->m.release(bl[i]);   // last block first
    bm->m.seqs.erase(it);
    return ok();
}

int32_t pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* table,
                           int32_t max_blocks, int32_t* num_blocks) {
    if (!bm || (max_blocks > 0 && !table)) return fail(PKV_ERR_ARG, "null pointer");
    const pkv::Sequence* sq = find_seq(const_cast<pkv_block_manager*>(bm), seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    const int32_t n = (int32_t)sq->blocks.size();
    if (num_blocks) *num_blocks = n;
    if (n > max_blocks) return fail(PKV_ERR_SIZE, "table holds %d blocks, row has %d", n, max_blocks);
    for (int32_t j = 0; j < max_blocks; ++j) table[j] = j < n ? sq->blocks[j] : 0;
    return ok();
}

int32_t pkv_bm_slots(const pkv_block_manager* bm, int64_t seq_id, int32_t first_pos,
                     int32_t count, int32_t* slots) {
    if (!bm || (count > 0 && !slots)) return fail(PKV_ERR_ARG, "null pointer");
    const pkv::Sequence* sq = find_seq(const_cast<pkv_block_manager*>(bm), seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    if (first_pos < 0 || count < 0 || (int64_t)first_pos + count > sq->num_tokens)
        return fail(PKV_ERR_ARG, "positions [%d, %d) outside the sequence's %d tokens", first_pos,
                    first_pos + count, sq->num_tokens);
    const int bs = bm->m.block_size;
    for (int32_t i = 0; i < count; ++i) {
        const int32_t p = first_pos + i;
        slots[i] = sq->fragmented ? sq->slots[p] : sq->blocks[p / bs] * bs + p % bs;
    }
    return ok();
}

// ---- token-level virtualisation ("vToken" page): eviction leaves the
// survivors where they are (the per-token table lists their slots in
// logical order); repacking moves them into the sequence's own blocks in
// order, frees the blocks no longer needed (last first) and makes the table
// block-aligned again.

int32_t pkv_bm_evict_tokens(pkv_block_manager* bm, int64_t seq_id, const uint8_t* keep,
                            int32_t num_tokens) {
    if (!bm || (num_tokens > 0 && !keep)) return fail(PKV_ERR_ARG, "null pointer");
    pkv::Sequence* sq = find_seq(bm, seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    if (num_tokens != sq->num_tokens)
        return fail(PKV_ERR_ARG, "keep mask covers %d tokens, the sequence holds %d", num_tokens, sq->num_tokens);
    pkv::BlockManager& m = bm->m;
    for (int32_t b : sq->blocks)
        if (m.ref[b] != 1) return fail(PKV_ERR_ARG, "block %d is shared: a shared block cannot lose tokens", b);
    const int bs = m.block_size;
    std::vector<int32_t> slots;
    try {
        slots.reserve(num_tokens);
        for (int32_t t = 0; t < num_tokens; ++t)
            if (keep[t]) slots.push_back(sq->fragmented ? sq->slots[t] : sq->blocks[t / bs] * bs + t % bs);
    } catch (...) {
        return fail(PKV_ERR_SIZE, "out of host memory");
    }
    // the blocks no longer hold the hashed token runs
    for (int32_t b : sq->blocks) m.drop_content(b);
    sq->slots = std::move(slots);
    sq->tokens.clear();            // only needed to publish, which an evicted sequence never does
    sq->chain.clear();
    sq->num_tokens = (int32_t)sq->slots.size();
    sq->num_computed = sq->num_tokens;
    sq->fragmented = true;
    sq->evicted = true;
    return ok();
}

int32_t pkv_bm_repack(pkv_block_manager* bm, int64_t seq_id, int32_t* moves, int32_t max_moves,
                      int32_t* num_moves) {
    if (!bm || !num_moves || (max_moves > 0 && !moves)) return fail(PKV_ERR_ARG, "null pointer");
    pkv::Sequence* sq = find_seq(bm, seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    pkv::BlockManager& m = bm->m;
    const int bs = m.block_size;
    const int32_t n = sq->num_tokens;
    int32_t cnt = 0;
    if (sq->fragmented)
        for (int32_t q = 0; q < n; ++q) cnt += sq->slots[q] != sq->blocks[q / bs] * bs + q % bs;
    *num_moves = cnt;
    if (cnt > max_moves) return fail(PKV_ERR_SIZE, "%d moves, room for %d", cnt, max_moves);
    if (sq->fragmented) {
        int32_t i = 0;
        for (int32_t q = 0; q < n; ++q) {
            const int32_t dst = sq->blocks[q / bs] * bs + q % bs;
            if (sq->slots[q] != dst) {
                moves[2 * i] = sq->slots[q];
                moves[2 * i + 1] = dst;
                ++i;
            }
        }
    }
    const size_t need = (size_t)((n + bs - 1) / bs);
    for (size_t i = sq->blocks.size(); i-- > need;) m.release(sq->blocks[i]);   // last block first
    sq->blocks.resize(need);
    sq->slots.clear();
    sq->fragmented = false;
    return ok();
}

// The same repack as tiles: for each of the sequence's first ceil(n / bs)
// blocks that receives at least one moved token, the block id and the
// source slot of each of its bs rows (a row that keeps its token, or lies
// past the last survivor, names its own slot).  Tiles come in block order,
// which is the order pkv_repack_blocks needs: every source sits at or after
// the row it moves to.
int32_t pkv_bm_repack_tiles(pkv_block_manager* bm, int64_t seq_id, int32_t* tiles, int32_t max_tiles,
                            int32_t* num_tiles) {
    if (!bm || !num_tiles || (max_tiles > 0 && !tiles)) return fail(PKV_ERR_ARG, "null pointer");
    pkv::Sequence* sq = find_seq(bm, seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    pkv::BlockManager& m = bm->m;
    const int bs = m.block_size;
    const int32_t n = sq->num_tokens;
    const int32_t need = (n + bs - 1) / bs;
    auto src_of = [&](int32_t j, int32_t i) {
        const int32_t q = j * bs + i;
        return q < n ? sq->slots[q] : sq->blocks[j] * bs + i;
    };
    int32_t cnt = 0;
    if (sq->fragmented)
        for (int32_t j = 0; j < need; ++j)
            for (int32_t i = 0; i < bs; ++i)
                if (src_of(j, i) != sq->blocks[j] * bs + i) {
                    ++cnt;
                    break;
                }
    *num_tiles = cnt;
    if (cnt > max_tiles) return fail(PKV_ERR_SIZE, "%d tiles, room for %d", cnt, max_tiles);
    if (sq->fragmented) {
        int32_t k = 0;
        for (int32_t j = 0; j < need; ++j) {
            bool moved = false;
            for (int32_t i = 0; i < bs && !moved; ++i) moved = src_of(j, i) != sq->blocks[j] * bs + i;
            if (!moved) continue;
            int32_t* t = tiles + (int64_t)k * (1 + bs);
            t[0] = sq->blocks[j];
            for (int32_t i = 0; i < bs; ++i) t[1 + i] = src_of(j, i);
            ++k;
        }
    }
    for (size_t i = sq->blocks.size(); i-- > (size_t)need;) m.release(sq->blocks[i]);   // last block first
    sq->blocks.resize(need);
    sq->slots.clear();
    sq->fragmented = false;
    return ok();
}

int32_t pkv_bm_token_slots(const pkv_block_manager* bm, int64_t seq_id, int32_t* slots,
                           int32_t max_tokens, int32_t* num_tokens) {
    if (!bm || (max_tokens > 0 && !slots)) return fail(PKV_ERR_ARG, "null pointer");
    const pkv::Sequence* sq = find_seq(const_cast<pkv_block_manager*>(bm), seq_id);
    if (!sq) return fail(PKV_ERR_ARG, "unknown sequence %lld", (long long)seq_id);
    if (num_tokens) *num_tokens = sq->num_tokens;
    if (sq->num_tokens > max_tokens)
        return fail(PKV_ERR_SIZE, "%d tokens, row has %d", sq->num_tokens, max_tokens);
    const int bs = bm->m.block_size;
    for (int32_t t = 0; t < max_tokens; ++t)
        slots[t] = t >= sq->num_tokens ? 0
                   : sq->fragmented ? sq->slots[t] : sq->blocks[t / bs] * bs + t % bs;
    return ok();
}

}  // extern "C"

// ------------------------------------------------------------ copy_blocks --

namespace pkv {

constexpr int kCopyThreads = 256;
constexpr int kCopyLayers = 64;   // layers per launch (kernel-argument array)

struct CopyArgs {
    uint8_t* k[kCopyLayers];
    uint8_t* v[kCopyLayers];
    const int32_t* pairs;   // [n][2] (src, dst)
    int64_t block_bytes;    // bytes of one block (all kv heads) in one pool
    int32_t num_blocks;
};

// Workgroup (pair, layer, K or V): copy one block's bytes, 16 per thread
// per load; each thread issues kCopyUnroll loads before its stores so that
// several are in flight.  Pairs naming a block outside [1, num_blocks) are
// skipped.
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(const CopyArgs a) {
    const int pair = blockIdx.x, layer = blockIdx.y;
    const int32_t src = a.pairs[2 * pair], dst = a.pairs[2 * pair + 1];
    if (src < 1 || src >= a.num_blocks || dst < 1 || dst >= a.num_blocks || src == dst) return;
    uint8_t* base = blockIdx.z ? a.v[layer] : a.k[layer];
    const uint4* from = reinterpret_cast<const uint4*>(base + (int64_t)src * a.block_bytes);
    uint4* to = reinterpret_cast<uint4*>(base + (int64_t)dst * a.block_bytes);
    const int64_t n = a.block_bytes / 16;
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += kCopyUnroll * kCopyThreads) {
        uint4 r[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = i0 + u * kCopyThreads;
            if (i < n) r[u] = from[i];
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = i0 + u * kCopyThreads;
            if (i < n) to[i] = r[u];
        }
    }
}

}  // namespace pkv

extern "C" int32_t pkv_copy_blocks(void* const* k_layers, void* const* v_layers,
                                   int32_t num_layers, int32_t num_blocks, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t kv_dtype,
                                   const int32_t* pairs, int32_t num_pairs, pkv_stream_t stream) {
    if (num_layers < 0 || num_pairs < 0 || num_blocks < 1 || num_kv_heads <= 0)
        return fail(PKV_ERR_ARG, "bad copy_blocks sizes");
    const int64_t tile = pkv_tile_bytes(head_dim, block_size, kv_dtype);
    if (tile <= 0) return fail(PKV_ERR_ARG, "bad head_dim / block_size / kv_dtype");
    if (num_pairs == 0 || num_layers == 0) return ok();
    if (!k_layers || !v_layers || !pairs) return fail(PKV_ERR_ARG, "null pointer");
    if (num_pairs > 65535 * 64) return fail(PKV_ERR_UNSUPPORTED, "too many pairs per call");
    pkv::CopyArgs a{};
    a.pairs = pairs;
    a.block_bytes = tile * num_kv_heads;
    a.num_blocks = num_blocks;
    (void)hipGetLastError();
    for (int32_t l0 = 0; l0 < num_layers; l0 += pkv::kCopyLayers) {
        const int32_t nl = num_layers - l0 < pkv::kCopyLayers ? num_layers - l0 : pkv::kCopyLayers;
        for (int32_t i = 0; i < nl; ++i) {
            if (!k_layers[l0 + i] || !v_layers[l0 + i]) return fail(PKV_ERR_ARG, "null layer pointer");
            a.k[i] = static_cast<uint8_t*>(k_layers[l0 + i]);
            a.v[i] = static_cast<uint8_t*>(v_layers[l0 + i]);
        }
        hipLaunchKernelGGL(pkv::copy_blocks_kernel, dim3(num_pairs, nl, 2), dim3(pkv::kCopyThreads), 0,
                           (hipStream_t)stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return pkv::hip_fail(e, "copy_blocks launch");
    }
    return ok();
}
