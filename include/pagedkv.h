/*
 * pagedkv.h — C ABI of libpagedkv.so: paged KV cache + PagedAttention decode
 * for AMD Instinct MI355X (gfx950 / CDNA4).
 *
 * Sources (the web pages this library is built from):
 *   [P1] "LLM inference basics and vLLM internals: KV cache, PagedAttention,
 *        scheduler" (ttlab.hopto.org), §1 arithmetic intensity, §2 KV cache
 *        and the size formula, §4 PagedAttention and block management.
 *   [P2] "vLLM internals (2): why PagedAttention pages the KV cache"
 *        (youngju.dev), sections "Block table: logically contiguous,
 *        physically scattered", "Block size tradeoff", "Sharing".
 *   [P4] "vToken: token-level virtualization of the KV cache"
 *        (gotosocial.chinng-lab-srv.dev), "KV cache basics" and
 *        "PagedAttention: block management learned from OS virtual memory".
 *
 * What is computed (the operation this ABI exposes):
 *   The KV cache holds, per layer, the key and value vector of every past
 *   token; a decode step adds only the new token's K/V and attends over all
 *   of them ([P1] §2, [P4] "KV cache basics").  The cache is cut into
 *   fixed-size blocks (16 tokens by default); each request owns a block table
 *   mapping its logical block j to a physical block id, so a request's blocks
 *   may sit anywhere in the pool and several requests may point at the same
 *   physical block ([P1] §4 and its diagram, [P2] "Block table", "Sharing").
 *   Query heads are grouped: all G = num_heads / num_kv_heads query heads of
 *   a group read the same K/V head ([P1] §2, MQA/GQA paragraph).
 *
 *   For sequence s with context length c (which already counts the token
 *   being decoded), query head h, kv head g = h / G:
 *     K_t = dequant(k_cache tile(block_tables[s][t / bs], g), row t % bs)
 *     out[s,h,:] = sum_t softmax_t(scale * q[s,h,:] . K_t) * V_t,  t < c
 *   (V_t likewise).  Block size and block-table semantics follow [P1] §4;
 *   the per-token byte count 2*L*H_kv*d*b follows [P1] §2's formula.
 *
 * Conventions shared by every entry point
 *   - All pointers are device pointers unless stated; all buffers are owned
 *     by the caller.  The library keeps no pointer beyond a call except inside
 *     a pkv_pool handle (which only records them).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream) and never synchronise the host, except pkv_check_block_tables.
 *   - Return 0 on success, a negative PKV_ERR_* code otherwise; the message
 *     is then available from pkv_last_error() (thread-local).  Nothing is
 *     launched when an argument check fails.  No C++ exception crosses the ABI.
 *   - Per-step data (block tables, context lengths, slot mappings) is device
 *     data; the launch shape depends only on host scalars, so a decode step
 *     can be captured into a HIP graph.
 *
 * ----------------------------------------------------------------------------
 * KV pool layout (frozen; the oracle reads the pool through this formula)
 * ----------------------------------------------------------------------------
 * One layer has one K pool and one V pool, each an array of
 *     [num_blocks][num_kv_heads] tiles,  tile = block_size tokens x head_dim.
 * Tile (pb, g) starts at byte  ((int64)pb * num_kv_heads + g) * tile_bytes,
 *     tile_bytes = block_size * head_dim * E,   E = element bytes (2 or 1).
 * A tile is block_size/16 sub-tiles of 16 tokens; token t of the block lives
 * in sub-tile u = t / 16 (byte u * 16 * head_dim * E), as row r = t % 16.
 * A sub-tile is a sequence of 1 KiB "rows": 64 lanes x 16 bytes, so one
 * wave-wide 16-byte-per-lane load reads one row, fully contiguous.
 *
 *   K element (r, k), 0<=r<16, 0<=k<head_dim:
 *       c = k / 8,  lane = r + 16 * (c % 4),  kk = c / 4,  e = k % 8,
 *       n = 2 / E   (8-element groups per 16-byte lane slot),
 *       byte = 1024*(kk / n) + 16*lane + 8*E*(kk % n) + E*e
 *   V element (r, k):
 *       nt = k / 16,  lane = (k % 16) + 16 * (r / 4),  i = r % 4,
 *       n = 4 / E   (4-element groups per 16-byte lane slot),
 *       byte = 1024*(nt / n) + 16*lane + 4*E*(nt % n) + E*i
 *
 * Why: in K, lane L of a row holds 8 consecutive dims of token L%16 — exactly
 * the A operand of a 16x16x32 matrix-core product S^T = K.Q^T.  In V, lane L
 * holds 4 consecutive tokens of dim L%16 — the A operand of a 16x16x16
 * product O^T = V^T.P^T, whose B operand (P) is in the same lane order as the
 * S^T result.  head_dim must be a multiple of 64; the cache write and the
 * block-table decode are built for 64, 128 and 256, every other kernel for
 * 128.  block_size 16 or 32.  Element encodings: bf16 / fp16 bit patterns
 * unchanged; fp8 = OCP OFP8 E4M3 ("e4m3fn": bias 7, max 448, no infinities,
 * S.1111.111 = NaN) holding round-to-nearest-even(x / scale) saturated to
 * +-448, and dequantised as code * scale.
 * Block 0 is the null block ([P1] §4: the block pool reserves block 0); no
 * kernel reads it unless a block table points at it.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q / out / key / value / KV pool. */
typedef enum {
    PKV_BF16 = 0,      /* bfloat16 */
    PKV_FP16 = 1,      /* IEEE binary16 */
    PKV_FP8_E4M3 = 2   /* OCP E4M3 with per-tensor fp32 scale (KV pool only) */
} pkv_dtype;

enum {
    PKV_OK = 0,
    PKV_ERR_ARG = -1,          /* null pointer, bad size, inconsistent heads */
    PKV_ERR_SIZE = -2,         /* workspace / pool / buffer too small */
    PKV_ERR_HIP = -3,          /* a HIP runtime call or launch failed */
    PKV_ERR_UNSUPPORTED = -4   /* valid but not built: head_dim, dtype pair */
};

/* Opaque stream type: a hipStream_t passed through unchanged. */
typedef void* pkv_stream_t;

/* ---------------------------------------------------------------- errors -- */

/* Message for the last nonzero return on this thread ("" if none).  The
 * string is owned by the library and valid until the next call.  (The pages
 * define no error channel; this one is the library's.) */
const char* pkv_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t pkv_version(void);

/* ------------------------------------------------------------ pool sizes -- */

/* Bytes of KV per token over all layers: 2 * L * H_kv * d * b ([P1] §2 size
 * formula; b = 2 for bf16/fp16, 1 for fp8 — [P1] §2 notes that FP8 KV makes
 * b = 1).  Returns a negative PKV_ERR_* code on a bad argument.
 * Example: L=28, H_kv=2, d=128, bf16 -> 28672. */
int64_t pkv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads,
                            int32_t head_dim, int32_t kv_dtype);

/* Bytes of one tile (block_size x head_dim elements) and of one layer's K
 * (equivalently V) pool of num_blocks blocks.  Negative on a bad argument. */
int64_t pkv_tile_bytes(int32_t head_dim, int32_t block_size, int32_t kv_dtype);
int64_t pkv_layer_pool_bytes(int32_t num_blocks, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size,
                             int32_t kv_dtype);

/* ------------------------------------------------------------- KV pool -- */

typedef struct {
    int32_t num_layers;
    int32_t num_blocks;     /* physical blocks per layer, block 0 = null */
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;     /* tokens per block: 16 or 32 */
    int32_t kv_dtype;       /* pkv_dtype */
} pkv_pool_desc;

typedef struct pkv_pool pkv_pool;

/* pkv_bytes_per_token of a pool descriptor (its num_layers, num_kv_heads,
 * head_dim, kv_dtype): the KV bytes one token occupies in that pool over all
 * layers.  Negative PKV_ERR_ARG for a null descriptor or bad fields. */
int64_t kv_pool_bytes_per_token(const pkv_pool_desc* desc);

/* Bind caller-allocated device memory as a paged KV pool ([P1] §4 block
 * pool; layout above).  k_layers / v_layers are host arrays of num_layers
 * device pointers, each at least bytes_each bytes, which must be at least
 * pkv_layer_pool_bytes(desc).  The handle records the pointers; it allocates
 * no device memory.  Errors: PKV_ERR_ARG (null, bad descriptor),
 * PKV_ERR_SIZE (bytes_each too small), PKV_ERR_UNSUPPORTED. */
int32_t kv_pool_create(const pkv_pool_desc* desc, void* const* k_layers,
                       void* const* v_layers, int64_t bytes_each,
                       pkv_pool** out);
/* Release a handle made by kv_pool_create (NULL is allowed).  The device
 * memory stays the caller's.  The pages define no such call: it only frees
 * the handle's host record. */
int32_t kv_pool_destroy(pkv_pool* pool);
int32_t kv_pool_get_desc(const pkv_pool* pool, pkv_pool_desc* out);
/* Device pointers of layer `layer`'s K and V pools. */
int32_t kv_pool_layer(const pkv_pool* pool, int32_t layer, void** k_cache,
                      void** v_cache);
/* Fill the null block (block 0) of every layer's K and V pool with a NaN
 * pattern of the pool's dtype, so that a stray read of it shows in the
 * output.  Asynchronous on `stream`. */
int32_t kv_pool_poison_null_block(const pkv_pool* pool, pkv_stream_t stream);

/* ---------------------------------------------------------- cache write -- */

/* Slot of each sequence's newest token: the token at position c-1 sits in
 * logical block (c-1)/bs at offset (c-1)%bs, so
 *     slot_mapping[s] = block_tables[s][(c-1)/bs] * bs + (c-1) % bs
 * ([P1] §4 diagram: request A's tokens 32-37 live in the block that logical
 * B2 maps to; [P2] "Block table").  c = context_lens[s] already counts the
 * new token; c <= 0 or c > max_blocks_per_seq*bs gives slot -1 (no write).
 * block_tables: [num_seqs][max_blocks_per_seq] int32, row-major. */
int32_t pkv_decode_slot_mapping(const int32_t* block_tables,
                                int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t block_size, int32_t* slot_mapping,
                                pkv_stream_t stream);

/* reshape_and_cache: write the new tokens' K and V into the pool.
 * key, value: [num_tokens][num_kv_heads][head_dim] of src_dtype (bf16/fp16),
 * contiguous.  For token t with slot = slot_mapping[t] >= 0, block
 * pb = slot / block_size, row = slot % block_size, every head g and dim k:
 *     k_cache element (pb, g, row, k) <- encode(key[t][g][k])
 * and likewise for V (only new tokens' K/V are added: [P4] "KV cache basics";
 * [P1] §2).  encode is the identity on bits when kv_dtype == src_dtype; for
 * fp8 it is e4m3(RNE_satfinite(float(x) * inv)) with inv = 1.0f / k_scale
 * (resp. v_scale) rounded to fp32 on the host.  Slots < 0 or >= num_blocks *
 * block_size are skipped (padding tokens).  Tokens must have distinct slots.
 * Errors: PKV_ERR_ARG, PKV_ERR_UNSUPPORTED (kv bf16/fp16 must equal
 * src_dtype; head_dim not 64, 128 or 256), PKV_ERR_HIP. */
int32_t reshape_and_cache(const void* key, const void* value,
                          int32_t src_dtype, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int32_t num_tokens,
                          int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks,
                          int32_t kv_dtype, float k_scale, float v_scale,
                          pkv_stream_t stream);

/* --------------------------------------------------------------- decode -- */

/* Implementation selector for paged_attention_decode_ex. */
enum {
    PKV_IMPL_AUTO = 0,    /* matrix-core kernel, waves per workgroup chosen
                             per workload: eight for 16-bit pools with
                             head_dim <= 128, at most 16 query heads per
                             kv head and partitions of >= 2048 tokens,
                             else four */
    PKV_IMPL_MFMA = 1,    /* GQA group on 16x16 MFMA tiles, one workgroup
                             of four waves per (item, kv head) of the plan,
                             the heads of an item on one XCD: the form whose
                             results paged_attention_prefill with one-token
                             chunks and paged_attention_decode_tokens with
                             an aligned table reproduce bit for bit */
    PKV_IMPL_VECTOR = 2,  /* same plan, layout and merge with the per-unit
                             math on the vector ALU (dot2), for comparison;
                             G <= 8, else PKV_ERR_UNSUPPORTED */
    PKV_IMPL_MFMA_PERSISTENT = 3  /* MFMA, resident workgroups claiming
                             plan entries from an atomic counter in the
                             plan header; a plan must then not be shared
                             by launches that run concurrently */
};

/* Which kernels one call launches (bit mask; default both). */
enum {
    PKV_STAGE_PARTITIONS = 1,  /* per-partition attention (+ direct output
                                  for single-partition sequences) */
    PKV_STAGE_REDUCE = 2       /* partial-softmax merge of multi-partition
                                  sequences */
};

typedef struct {
    int32_t partition_tokens; /* context split size; 0 = the library default
                                 (pkv_default_partition_tokens); must be a
                                 multiple of block_size */
    int32_t impl;             /* PKV_IMPL_* */
    int32_t stages;           /* PKV_STAGE_* mask; 0 = both */
    int32_t num_blocks;       /* pool size for id clamping; 0 = unchecked */
    const void* plan;         /* device plan from paged_attention_plan built
                                 for the same context_lens, max_context_len,
                                 max_blocks_per_seq, num_kv_heads, block_size
                                 and partition_tokens; NULL = build one in
                                 the workspace */
} pkv_decode_opts;

/* Default context split.  A sequence's context is cut into partitions of
 * this many tokens only as far as needed to give the GPU about four
 * workgroups per compute unit in total (num_seqs * num_kv_heads *
 * partitions); partial results written while the KV stream is being read
 * cost far more than their size, so larger partitions are preferred.
 * Depends on the current device's CU count.  Negative on a bad argument. */
int32_t pkv_default_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                     int32_t max_context_len,
                                     int32_t block_size);

/* Workspace bytes for a decode call: the work plan, plus — when a sequence
 * can span several partitions (P = ceil(max_context_len / partition) > 1)
 * — per (sequence, kv head, partition) the group's head_dim fp32 partial
 * outputs and one 128-byte line of maxima and normalisers.  With a caller
 * plan (opts->plan) the plan part is not used.  The default split size is
 * resolved from max_context_len here and in the decode call alike, so this
 * size always suffices for a decode with the same arguments (the decode may
 * need less when max_blocks_per_seq * block_size < max_context_len).  The
 * pages define no workspace: it is this library's split-context scratch. */
int64_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_context_len,
                                        int32_t block_size,
                                        int32_t partition_tokens);

/* Work plan: the list of (sequence, partition) items of a decode, longest
 * first, so that workgroups dispatched in order form a longest-first
 * schedule.  Built on the device from context_lens (no host sync); a plan
 * stays valid while context_lens and the sizes below are unchanged, so one
 * plan serves every layer of a decode step.  plan: device memory of at
 * least paged_attention_plan_bytes(...) bytes. */
int64_t paged_attention_plan_bytes(int32_t num_seqs, int32_t num_kv_heads,
                                   int32_t max_context_len, int32_t block_size,
                                   int32_t partition_tokens);
int32_t paged_attention_plan(const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_context_len,
                             int32_t max_blocks_per_seq, int32_t num_kv_heads,
                             int32_t block_size, int32_t partition_tokens,
                             void* plan, int64_t plan_bytes,
                             pkv_stream_t stream);

/* paged_attention_decode: one query token per sequence attends over its
 * whole context through the block table (operation above; [P1] §4, [P2]
 * "Block table").
 *   out, q       : [num_seqs][num_heads][head_dim] of q_dtype (bf16 / fp16),
 *                  contiguous; out rounded to nearest even.
 *   k_cache,
 *   v_cache      : one layer's pools, layout above, kv_dtype.  bf16/fp16 KV
 *                  must equal q_dtype; fp8 KV works with either q_dtype.
 *   block_tables : [num_seqs][max_blocks_per_seq] int32; entries at or past
 *                  ceil(c/bs) are never read.
 *   context_lens : [num_seqs] int32, c >= 0 (c = 0 gives a zero output).
 *                  c is clamped to min(max_context_len, max_blocks_per_seq *
 *                  block_size) so the kernel never reads past the table.
 *   scale        : logit scale (1/sqrt(head_dim) usually).
 *   k_scale,
 *   v_scale      : fp8 dequantisation scales (ignored unless kv fp8).
 *   workspace    : >= paged_attention_workspace_bytes(...) bytes of device
 *                  memory.
 * num_heads must be a multiple of num_kv_heads; G = num_heads /
 * num_kv_heads may be anything from 1 (MHA) to num_heads (MQA, one kv head
 * for all query heads: [P1] §2).  Query heads h = g*G .. g*G + G - 1 read kv
 * head g.  A work entry holds up to 32 query heads of one kv head (two
 * 16-column MFMA tiles; 16 at head_dim 256); a larger group runs as several
 * entries, all reading the same K / V (sharing it in the XCD's L2 when they
 * run together).  Errors: PKV_ERR_ARG, PKV_ERR_SIZE (workspace),
 * PKV_ERR_UNSUPPORTED (head_dim not 64, 128 or 256 — 128 only with
 * PKV_IMPL_VECTOR —, dtype pair), PKV_ERR_HIP. */
int32_t paged_attention_decode(void* out, const void* q, int32_t q_dtype,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables,
                               int32_t max_blocks_per_seq,
                               const int32_t* context_lens,
                               int32_t max_context_len, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, float scale,
                               int32_t block_size, int32_t kv_dtype,
                               float k_scale, float v_scale, void* workspace,
                               int64_t workspace_bytes, pkv_stream_t stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same operation, arguments and kernels as
 * paged_attention_decode, without the workspace arguments: the work plan and
 * partition partials live in a static device array of
 * PKV_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends.  Allocates nothing and calls no allocating
 * routine.  A call whose workspace (paged_attention_workspace_bytes with the
 * default split) exceeds that size fails with PKV_ERR_SIZE before anything
 * is launched.  All calls on one GPU share its array and each fully rewrites
 * what it reads: calls that overlap on one GPU (concurrent streams, or
 * threads) race and must be serialised by the caller.  Errors: as
 * paged_attention_decode. */
#define PKV_NOALLOC_SCRATCH_BYTES (16ll << 20)
int32_t paged_attention_decode_noalloc(void* out, const void* q, int32_t q_dtype,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables,
                                       int32_t max_blocks_per_seq,
                                       const int32_t* context_lens,
                                       int32_t max_context_len, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, float scale,
                                       int32_t block_size, int32_t kv_dtype,
                                       float k_scale, float v_scale,
                                       pkv_stream_t stream);

/* Same as paged_attention_decode with explicit options (NULL = defaults).
 * With opts->num_blocks > 0, block ids outside [0, num_blocks) are read as
 * the null block 0 instead of faulting. */
int32_t paged_attention_decode_ex(void* out, const void* q, int32_t q_dtype,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables,
                                  int32_t max_blocks_per_seq,
                                  const int32_t* context_lens,
                                  int32_t max_context_len, int32_t num_seqs,
                                  int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, float scale,
                                  int32_t block_size, int32_t kv_dtype,
                                  float k_scale, float v_scale,
                                  void* workspace, int64_t workspace_bytes,
                                  const pkv_decode_opts* opts,
                                  pkv_stream_t stream);

/* paged_attention_decode_append: reshape_and_cache of each sequence's new
 * token followed by paged_attention_decode_ex, in one launch.  Each decode
 * step appends only the new token's key and value, and attention then sees
 * every token including it (vToken page, "KV cache basics"): c counts the
 * new token, which sits at position c - 1.  The workgroup whose partition holds position c - 1 of
 * (sequence, kv head) writes the token's K / V row to slot
 * block_tables[s][(c-1) / block_size] * block_size + (c-1) % block_size
 * exactly as reshape_and_cache would (bit for bit), then reads the pool.
 *   key, value : [num_seqs][num_kv_heads][head_dim] of q_dtype, the new
 *                token's K and V (post-RoPE), device memory.
 *   k_cache,
 *   v_cache    : one layer's pools, written and read.
 *   opts       : required, with opts->num_blocks > 0 (the pool size): a
 *                table entry at or past it gets no write (and is read as
 *                the null block, as in paged_attention_decode_ex).
 * Other arguments as paged_attention_decode_ex.  No write happens for a
 * sequence with c <= 0 or c > min(max_context_len, max_blocks_per_seq *
 * block_size).  The block receiving the token must not be read by another
 * sequence of the same call (copy-on-write, [P1] §4, guarantees it: only
 * unshared blocks are written); otherwise that sequence may see the slot
 * before or after the write.  Errors: as paged_attention_decode_ex, plus
 * PKV_ERR_ARG for missing opts / num_blocks, key or value, non-positive fp8
 * scales, or a stages mask without PKV_STAGE_PARTITIONS. */
int32_t paged_attention_decode_append(void* out, const void* q, int32_t q_dtype,
                                      const void* key, const void* value,
                                      void* k_cache, void* v_cache,
                                      const int32_t* block_tables,
                                      int32_t max_blocks_per_seq,
                                      const int32_t* context_lens,
                                      int32_t max_context_len, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, float scale,
                                      int32_t block_size, int32_t kv_dtype,
                                      float k_scale, float v_scale,
                                      void* workspace, int64_t workspace_bytes,
                                      const pkv_decode_opts* opts,
                                      pkv_stream_t stream);

/* ------------------------------------------------------- multi-token --
 *
 * paged_attention_prefill: several new tokens per sequence (a chunk of a
 * chunked prefill, or the tokens left to compute after a prefix-cache hit,
 * [P1] §5 / §6) attend causally over their paged context: the q_len(s) =
 * query_start_loc[s+1] - query_start_loc[s] tokens of sequence s are its
 * last ones, token j at position p = c - q_len(s) + j (c = context_lens[s],
 * which counts them; their K/V are already in the cache), and
 *     out[row, h, :] = sum_{t <= p} softmax_t(scale * q[row,h,:] . K_t) V_t,
 *     row = query_start_loc[s] + j,
 * with K_t, V_t read through the block table as for decode.  With q_len = 1
 * for every sequence this is paged_attention_decode.
 *   q, out          : [num_query_tokens][num_heads][head_dim] q_dtype rows,
 *                     sequences packed in order.
 *   query_start_loc : device int32[num_seqs + 1], non-decreasing, from 0;
 *                     max_query_len >= every q_len(s) (host scalar: grid).
 *   max_query_len   : host scalar that sizes the grid; it must be at least
 *                     every q_len(s).  The rows of a sequence past the first
 *                     max_query_len are not written (their contents stay
 *                     undefined): the caller passes the true maximum.
 *   num_blocks      : pool size; block ids outside [0, num_blocks) are read
 *                     as the null block 0 instead of faulting (0 =
 *                     unchecked).
 * Other arguments as paged_attention_decode; no workspace.  A token whose
 * position would be < 0 (c < q_len) gets a zero output row.  q and the
 * context's K / V are expected finite: a NaN or infinity in a query row, or
 * in a key or value a row can see, gives an undefined result in that row
 * (this kernel is built with the compiler's finite-math assumption for its
 * min / max; positions a row cannot see may hold anything).  Errors:
 * PKV_ERR_ARG, PKV_ERR_UNSUPPORTED (head_dim != 128, dtype pair),
 * PKV_ERR_HIP. */
int32_t paged_attention_prefill(void* out, const void* q, int32_t q_dtype,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_tables,
                                int32_t max_blocks_per_seq,
                                const int32_t* context_lens,
                                const int32_t* query_start_loc,
                                int32_t max_query_len, int32_t max_context_len,
                                int32_t num_seqs, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                float scale, int32_t block_size, int32_t num_blocks,
                                int32_t kv_dtype, float k_scale, float v_scale,
                                pkv_stream_t stream);

/* ------------------------------------------------------------ validation -- */

/* Count block-table entries that a decode of these context lengths would
 * read and that fall outside [1, num_blocks) (the null block 0 counts as
 * invalid), plus context lengths < 0 or > max_blocks_per_seq * block_size.
 * Synchronous: waits for `stream`, writes the count to *bad_count (host).
 * Uses 4 bytes of caller scratch device memory `scratch_dev`. */
int32_t pkv_check_block_tables(const int32_t* block_tables,
                               int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t block_size, int32_t num_blocks,
                               int32_t* scratch_dev, int64_t* bad_count,
                               pkv_stream_t stream);

/* ------------------------------------------------------------- measurement --
 *
 * Read-stream probe: the HBM read rate a plain stream reaches on this
 * device, reported beside the decode kernel's rate as the achievable figure
 * (the 8 TB/s peak is the vendor's).  Not part of the attention path.
 *
 * pkv_read_probe_sink_bytes: bytes of the sink buffer pkv_read_probe needs
 * on the current device (one 16-byte word per probe thread).
 *
 * pkv_read_probe: reads the `bytes` bytes at device pointer `src` once
 * (16-byte words, non-temporal loads, one contiguous slice per workgroup)
 * and writes the XOR of each thread's words to device buffer `sink`; the
 * XOR of all sink words equals the XOR of all source words.  bytes: a
 * multiple of 16 (0: nothing runs); src and sink 16-byte aligned,
 * caller-owned.  Asynchronous on `stream`.  Errors: PKV_ERR_ARG (null,
 * alignment, bytes), PKV_ERR_SIZE (sink_bytes below the required size),
 * PKV_ERR_HIP. */
int64_t pkv_read_probe_sink_bytes(void);
int32_t pkv_read_probe(const void* src, int64_t bytes, void* sink, int64_t sink_bytes,
                       pkv_stream_t stream);

/* ---------------------------------------------------------- block manager --
 *
 * Host-side block pool that produces the block tables and slots the calls
 * above consume ([P1] §4: blocks handed out one at a time as a request
 * grows, block 0 reserved as the null block, a doubly linked queue of free
 * blocks, reference counts and copy-on-write for shared blocks; [P2]
 * "Sharing"; [P1] §5 prefix cache: a full block's hash chains its parent's
 * hash, its tokens and an extra key, only full blocks are cached, a prompt
 * recomputes at least its last token, freed blocks keep their content and
 * are reused least recently freed first, a request returns its blocks last
 * block first).  Where the order of reuse is open, free blocks holding no
 * cached content are handed out before a cached block is evicted (the
 * reading under which [P1] §10's block model prints 0 / 0 / 21,488 hits for
 * its §9 experiment).
 *
 * Sequences are named by caller ids.  Slots are block * block_size +
 * offset, as pkv_decode_slot_mapping computes them.  Not thread-safe: one
 * handle, one thread at a time.  Host memory only; no GPU call is made.
 * Errors: PKV_ERR_ARG (null, unknown or duplicate sequence id, range),
 * PKV_ERR_SIZE (not enough free blocks: the state is left unchanged). */
typedef struct pkv_block_manager pkv_block_manager;

/* num_blocks includes the null block (so num_blocks - 1 are usable);
 * prefix_caching != 0 keeps and reuses the content of full blocks. */
int32_t pkv_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching,
                      pkv_block_manager** out);
int32_t pkv_bm_destroy(pkv_block_manager* bm);
/* Free blocks (no cached content + cached content), and the cached ones. */
int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);
int32_t pkv_bm_num_cached_free_blocks(const pkv_block_manager* bm);
/* Reference count of a block (the null block reports 1). */
int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block);
int32_t pkv_bm_num_tokens(const pkv_block_manager* bm, int64_t seq_id);
/* New sequence with a prompt of num_tokens tokens (host array): blocks for
 * all of them; with the prefix cache, the longest cached run of leading
 * full blocks is shared instead (*num_cached_tokens, a multiple of
 * block_size, always < num_tokens).  Those hit tokens count as computed;
 * the prompt's other blocks become findable by later prompts only once
 * pkv_bm_mark_computed covers them.  extra_key separates otherwise equal
 * prompts (salt, adapter). */
int32_t pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                            int32_t num_tokens, uint64_t extra_key,
                            int32_t* num_cached_tokens);
/* Append one token: *slot receives its cache slot.  If the last block is
 * shared and partly filled, it is replaced by a private block first and
 * (*cow_src, *cow_dst) name the copy to run (pkv_copy_blocks) before the
 * token is written; otherwise both are -1. */
int32_t pkv_bm_append_token(pkv_block_manager* bm, int64_t seq_id, int32_t token,
                            int32_t* slot, int32_t* cow_src, int32_t* cow_dst);
/* The K/V of the sequence's first num_computed_tokens tokens are written, or
 * are written by work already enqueued on the stream ahead of any later
 * reader (a prefill chunk's reshape_and_cache).  With the prefix cache, every
 * full block that ends inside them becomes findable by later prompts: [P1] §5
 * caches only full blocks, and with chunked prefill ([P1] §6) a prompt's
 * blocks fill over several steps, so a block counts as full once its last
 * token's K/V is computed.  Counts never go back (a smaller value is a no-op);
 * PKV_ERR_ARG if num_computed_tokens exceeds the sequence's tokens.  A token
 * appended to a sequence whose every token is computed counts as computed at
 * once (the decode step that appends it writes its K/V); a block freed before
 * it was computed is never findable. */
int32_t pkv_bm_mark_computed(pkv_block_manager* bm, int64_t seq_id, int32_t num_computed_tokens);
int32_t pkv_bm_num_computed_tokens(const pkv_block_manager* bm, int64_t seq_id);
/* child shares every block of parent (reference counts + 1). */
int32_t pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id);
/* Drop the sequence; its blocks lose a reference, last block first. */
int32_t pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);
/* The block table as a row of max_blocks ids (host array), padded with the
 * null block 0; *num_blocks = blocks in use (PKV_ERR_SIZE if > max_blocks). */
int32_t pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* table,
                           int32_t max_blocks, int32_t* num_blocks);
/* Slots of positions [first_pos, first_pos + count) (host array). */
int32_t pkv_bm_slots(const pkv_block_manager* bm, int64_t seq_id, int32_t first_pos,
                     int32_t count, int32_t* slots);

/* Token-level virtualisation ([P4] "vToken": a token table maps each
 * logical token to its physical place; tokens dropped by an eviction
 * policy leave holes; repacking moves survivors so whole blocks can be
 * freed, keeping the logical order).
 * pkv_bm_evict_tokens: keep[t] != 0 keeps logical token t (host array of
 *   num_tokens = the sequence's token count).  Survivors keep their slots,
 *   in logical order; the sequence must own every block alone
 *   (PKV_ERR_ARG otherwise); its blocks lose any cached prefix content.
 *   Until repacked, the sequence cannot grow or fork, and attention must
 *   read it through pkv_bm_token_slots / paged_attention_decode_tokens.
 * pkv_bm_repack: host array moves[max_moves][2] receives the (src, dst)
 *   slot moves that put survivor q at block q / bs, row q % bs of the
 *   sequence's own blocks; *num_moves = their count (PKV_ERR_SIZE, state
 *   unchanged, if more than max_moves).  The blocks past the survivors are
 *   freed at once (last first): run pkv_move_tokens on the stream before
 *   anything else writes to them.
 * pkv_bm_token_slots: slot of every logical token (host array of
 *   max_tokens, padded with 0). */
int32_t pkv_bm_evict_tokens(pkv_block_manager* bm, int64_t seq_id, const uint8_t* keep,
                            int32_t num_tokens);
int32_t pkv_bm_repack(pkv_block_manager* bm, int64_t seq_id, int32_t* moves, int32_t max_moves,
                      int32_t* num_moves);
int32_t pkv_bm_token_slots(const pkv_block_manager* bm, int64_t seq_id, int32_t* slots,
                           int32_t max_tokens, int32_t* num_tokens);

/* pkv_bm_repack_tiles: the same repack as pkv_bm_repack (same state change,
 * same freed blocks), returned as whole blocks for pkv_repack_blocks: host
 * array tiles[max_tiles][1 + block_size] receives, for each of the
 * sequence's remaining blocks that gets at least one moved token, in block
 * order, the block id followed by the source slot of each of its rows (a
 * row that keeps its token, or lies past the last survivor, names its own
 * slot); *num_tiles = their count (PKV_ERR_SIZE, state unchanged, if more
 * than max_tiles). */
int32_t pkv_bm_repack_tiles(pkv_block_manager* bm, int64_t seq_id, int32_t* tiles, int32_t max_tiles,
                            int32_t* num_tiles);

/* Decode through a per-token table ([P4] "vToken"): logical token t of
 * sequence s is read from physical slot token_slots[s][t] (device int32
 * [num_seqs][max_tokens_per_seq]; block slot / block_size, row slot %
 * block_size), for t < min(context_lens[s], max_tokens_per_seq).  Otherwise
 * as paged_attention_decode (no split, no workspace).  Slots outside
 * [block_size, num_blocks * block_size) are read as slot block_size.  A
 * block-aligned table gives exactly the block-table result; a fragmented
 * one costs element-wise V loads (V lanes of the pool layout interleave four
 * tokens per 16 bytes).  Errors: as
 * paged_attention_decode. */
int32_t paged_attention_decode_tokens(void* out, const void* q, int32_t q_dtype,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* token_slots, int32_t max_tokens_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float scale, int32_t block_size, int32_t num_blocks,
                                      int32_t kv_dtype, float k_scale, float v_scale,
                                      pkv_stream_t stream);

/* The same decode over a run list ([P4] "vToken": attention reads every
 * surviving token through the table; here each pool sub-tile that holds
 * survivors is read whole and the rows that are not the sequence's keys are
 * skipped).  Survivors of a random eviction sit in nearly every line of
 * every tile, so paged_attention_decode_tokens fetches about the whole pool
 * anyway; a run list fetches the same lines with the block path's whole-row
 * loads.
 *
 * pkv_token_runs_bytes: bytes of the run list of num_seqs sequences of
 *   at most max_tokens_per_seq table entries (negative on a bad argument).
 * pkv_token_runs: builds the run list of a token table (arguments as
 *   paged_attention_decode_tokens; num_seqs <= 65535, max_tokens_per_seq <
 *   2^27) into `runs` (device memory of at least pkv_token_runs_bytes,
 *   8-byte aligned; PKV_ERR_SIZE if smaller).  Layout (int32, each area on
 *   256 bytes): [num_seqs counts n_s][num_seqs lengths 16 n_s][the decode's
 *   work plan: sequences by decreasing n_s][num_seqs x max_tokens_per_seq
 *   entries of two int32: (sub-tile, row mask)] (the entries end the
 *   buffer); entry e < n_s of sequence s holds the pool sub-tile slot / 16
 *   and a 16-bit mask of its rows that are keys.  An entry takes table
 *   entries t, t + 1,
 *   ... (t < min(context_lens[s], max_tokens_per_seq)) while they lie in one
 *   16-token sub-tile at strictly increasing rows; any other step opens a
 *   new entry, so the entries list every table entry exactly once (a slot
 *   listed twice counts twice).  Slots outside [block_size, num_blocks *
 *   block_size) read as slot block_size.  Built once per step: the table is
 *   shared by all layers.  min_keys_per_entry (0..16): a sequence whose
 *   list holds fewer keys than this per entry on average (sparse survivors,
 *   whole sub-tiles mostly skipped) is marked for the token gather instead
 *   (count -1 - n_s); 0 marks none.  Measured crossover on the Qwen2.5-7B
 *   decode shape: about 5 (10 % of tokens kept: gather 212 us / layer, run
 *   list 308 us; 25 %: 353 / 373 us; 50 %: 463 / 376 us).
 * paged_attention_decode_runs: attention of each sequence over the keys of
 *   its run list (`runs`, runs_bytes long, from pkv_token_runs with the same
 *   num_seqs, max_tokens_per_seq, block_size and num_blocks; PKV_ERR_SIZE if
 *   runs_bytes < pkv_token_runs_bytes), and of the sequences the list marked
 *   for the gather token by token through token_slots / context_lens (the
 *   table the list was built from; a second launch, in which the workgroups
 *   of unmarked sequences leave at once: 4-9 us on the Qwen2.5-7B decode
 *   shape when none is marked).  Pass both as NULL only for a list built
 *   with min_keys_per_entry = 0 (marked sequences are then left unwritten):
 *   a caller that knows its survivors are dense skips the second launch
 *   that way.  Otherwise as
 *   paged_attention_decode_tokens, whose result it equals within rounding
 *   (the softmax visits the same keys in sub-tile units), and for a
 *   block-aligned table the block-table decode's on one partition with the
 *   same waves per workgroup bit for bit (PKV_IMPL_AUTO with partitions of
 *   >= 2048 tokens: eight waves for 16-bit pools, four for fp8).  Sub-tile
 *   ids past the pool read block 0.
 *   Errors: as paged_attention_decode_tokens. */
int64_t pkv_token_runs_bytes(int32_t num_seqs, int32_t max_tokens_per_seq);
int32_t pkv_token_runs(const int32_t* token_slots, int32_t max_tokens_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                       int32_t num_blocks, int32_t min_keys_per_entry, void* runs,
                       int64_t runs_bytes, pkv_stream_t stream);
int32_t paged_attention_decode_runs(void* out, const void* q, int32_t q_dtype,
                                    const void* k_cache, const void* v_cache, const void* runs,
                                    int64_t runs_bytes, const int32_t* token_slots,
                                    const int32_t* context_lens, int32_t max_tokens_per_seq,
                                    int32_t num_seqs, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, float scale,
                                    int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                                    float k_scale, float v_scale, pkv_stream_t stream);

/* Rebuild whole blocks after an eviction ([P4] "vToken", asynchronous
 * repacking): for every tile t (device int32 tiles[t][1 + block_size]: the
 * destination block, then the source slot of each of its rows), in every
 * layer, K and V of every kv head, row i of block tiles[t][0] receives the
 * token at slot tiles[t][1 + i].  Tiles are grouped in chains (device int32
 * chain_offsets[num_chains + 1]: chain c is tiles chain_offsets[c] ..
 * chain_offsets[c + 1] - 1) and a chain's tiles are rebuilt in order,
 * 16-row sub-tile by sub-tile.  Requirement (what pkv_bm_repack_tiles
 * produces, one chain per sequence): no source of a sub-tile lies in rows
 * an earlier sub-tile of its chain writes, and the chains write disjoint
 * blocks that no other chain reads.  Then every source is read before it is
 * overwritten and the result equals pkv_move_tokens with the moves (source,
 * destination) of all rows, without its scratch.  Sub-tiles are stored
 * whole (no partial writes).  A source slot outside [block_size,
 * num_blocks * block_size) leaves its row unchanged; a destination block
 * outside [1, num_blocks) skips its tile.  Errors: PKV_ERR_ARG (null
 * pointers, bad sizes), PKV_ERR_UNSUPPORTED (head_dim), PKV_ERR_HIP. */
int32_t pkv_repack_blocks(void* const* k_layers, void* const* v_layers, int32_t num_layers,
                          int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t kv_dtype, const int32_t* tiles,
                          const int32_t* chain_offsets, int32_t num_chains, pkv_stream_t stream);

/* Move whole tokens (K and V rows of every kv head, every layer) from slot
 * moves[i][0] to slot moves[i][1] ([P4] "vToken" repacking); moves is a
 * device int32 [num_moves][2].  Every source is read before any
 * destination is written (through `scratch`, device memory of at least
 * pkv_move_tokens_scratch_bytes(...) bytes), so moves may chain or swap.
 * A move naming a slot outside [block_size, num_blocks * block_size) is
 * skipped; two moves must not share a destination.  Errors: PKV_ERR_ARG,
 * PKV_ERR_SIZE (scratch), PKV_ERR_UNSUPPORTED (head_dim), PKV_ERR_HIP. */
int64_t pkv_move_tokens_scratch_bytes(int32_t num_layers, int32_t num_moves,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t kv_dtype);
int32_t pkv_move_tokens(void* const* k_layers, void* const* v_layers, int32_t num_layers,
                        int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t kv_dtype, const int32_t* moves,
                        int32_t num_moves, void* scratch, int64_t scratch_bytes,
                        pkv_stream_t stream);

/* Copy whole blocks (all kv heads, K and V, every layer) from pairs[i][0]
 * to pairs[i][1] ([P1] §4 copy-on-write): pairs is a device int32 array of
 * num_pairs (src, dst); k_layers / v_layers are host arrays of num_layers
 * device pool pointers (layout above).  A pair naming a block outside
 * [1, num_blocks), or src == dst, is skipped.  Destinations must be distinct
 * and must not be sources of other pairs in the same call.  Errors:
 * PKV_ERR_ARG, PKV_ERR_HIP. */
int32_t pkv_copy_blocks(void* const* k_layers, void* const* v_layers, int32_t num_layers,
                        int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t kv_dtype, const int32_t* pairs,
                        int32_t num_pairs, pkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
