// api.hip — the extern "C" boundary declared in include/pagedkv.h:
// argument checks, workspace sizing, kernel selection, error reporting.
// Every computation runs in the kernels of cache_ops.hip / decode*.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/pagedkv.h"
#include "pkv_launch.h"

namespace pkv {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int32_t ok() {
    g_err.clear();
    return PKV_OK;
}

int32_t hip_fail(hipError_t e, const char* what) {
    return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

const char* last_error() { return g_err.c_str(); }

}  // namespace pkv

namespace {

using pkv::fail;
using pkv::hip_fail;
using pkv::ok;

bool valid_dtype(int32_t dt) { return dt == PKV_BF16 || dt == PKV_FP16 || dt == PKV_FP8_E4M3; }
int32_t elem_size(int32_t dt) { return dt == PKV_FP8_E4M3 ? 1 : 2; }
bool valid_block_size(int32_t bs) { return bs == 16 || bs == 32; }

constexpr int32_t kBuiltHeadDim = 128;
// head_dim of the cache write and the block-table decode (matrix-core
// kernels); every other kernel is built for kBuiltHeadDim only
bool decode_head_dim(int32_t d) { return d == 64 || d == 128 || d == 256; }
constexpr int64_t kWorkgroupsPerCu = 4;   // default split target: 4 workgroups per CU

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

int32_t ctx_cap_of(int32_t max_context_len, int32_t max_blocks, int32_t block_size) {
    const int64_t table_tokens = (int64_t)max_blocks * block_size;
    return (int32_t)(table_tokens < max_context_len ? table_tokens : max_context_len);
}

// Split the context only as far as parallelism needs: about
// kWorkgroupsPerCu workgroups per CU in total.  Partial results written in
// the middle of the KV read stream are expensive, so larger is better once
// the GPU is full; the longest-first plan balances what remains.
int32_t resolve_partition(int32_t requested, int32_t num_seqs, int32_t num_kv_heads,
                          int32_t ctx_cap, int32_t block_size) {
    if (requested > 0) return requested;
    const int64_t items = std::max<int64_t>(1, (int64_t)num_seqs * num_kv_heads);
    const int64_t target = kWorkgroupsPerCu * device_cu_count();
    const int64_t splits = (target + items - 1) / items;
    int64_t part = (ctx_cap + splits - 1) / splits;
    part = std::max<int64_t>(block_size, (part + block_size - 1) / block_size * block_size);
    while ((ctx_cap + part - 1) / part > 65535) part *= 2;
    return (int32_t)std::min<int64_t>(part, 1 << 30);
}

int64_t num_parts_of(int32_t ctx_cap, int32_t part) { return std::max<int64_t>(1, (ctx_cap + part - 1) / part); }

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int64_t plan_bytes_of(int32_t num_seqs, int64_t P) { return align256(4 * (4 + (int64_t)num_seqs * P)); }

// Workspace: [partial outputs][partial max/normaliser][plan]; the partial
// areas exist only when some sequence can span several partitions.  Records
// are per entry head (pkv::set_heads): group rows of D floats each, and a
// line of ml_line(group) floats of maxima and normalisers.
struct WsLayout { int64_t o_bytes, ml_bytes, plan_off, total; };
WsLayout ws_layout(int32_t S, int32_t H, int32_t Hkv, int32_t D, int64_t P) {
    WsLayout w{};
    if (P > 1) {
        pkv::DecodeArgs e{};
        pkv::set_heads(e, H, Hkv, pkv::decode_max_cols(D));
        w.o_bytes = align256((int64_t)S * e.num_kv_heads * e.group * P * D * 4);
        w.ml_bytes = align256((int64_t)S * e.num_kv_heads * P * pkv::ml_line(e.group) * 4);
    }
    w.plan_off = w.o_bytes + w.ml_bytes;
    w.total = w.plan_off + plan_bytes_of(S, P);
    return w;
}

// Kernels are built for head_dim 128; layout sizes accept any multiple of 64.
int32_t check_layout_args(int32_t head_dim, int32_t block_size, int32_t kv_dtype) {
    if (!valid_dtype(kv_dtype)) return fail(PKV_ERR_ARG, "kv_dtype %d is not a pkv_dtype", kv_dtype);
    if (head_dim <= 0 || head_dim % 64) return fail(PKV_ERR_ARG, "head_dim %d is not a positive multiple of 64", head_dim);
    if (!valid_block_size(block_size)) return fail(PKV_ERR_ARG, "block_size %d must be 16 or 32", block_size);
    return PKV_OK;
}

}  // namespace

struct pkv_pool {
    pkv_pool_desc desc;
    std::vector<void*> k;
    std::vector<void*> v;
    int64_t bytes_each;
};

extern "C" {

const char* pkv_last_error(void) { return pkv::last_error(); }

int32_t pkv_version(void) { return 100; }

int64_t pkv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                            int32_t kv_dtype) {
    if (num_layers <= 0 || num_kv_heads <= 0 || head_dim <= 0)
        return fail(PKV_ERR_ARG, "layers, kv heads and head_dim must be positive");
    if (!valid_dtype(kv_dtype)) return fail(PKV_ERR_ARG, "kv_dtype %d is not a pkv_dtype", kv_dtype);
    ok();
    return 2LL * num_layers * num_kv_heads * head_dim * elem_size(kv_dtype);
}

int64_t kv_pool_bytes_per_token(const pkv_pool_desc* desc) {
    if (!desc) return fail(PKV_ERR_ARG, "null descriptor");
    return pkv_bytes_per_token(desc->num_layers, desc->num_kv_heads, desc->head_dim, desc->kv_dtype);
}

int64_t pkv_tile_bytes(int32_t head_dim, int32_t block_size, int32_t kv_dtype) {
    if (int32_t e = check_layout_args(head_dim, block_size, kv_dtype)) return e;
    ok();
    return (int64_t)block_size * head_dim * elem_size(kv_dtype);
}

int64_t pkv_layer_pool_bytes(int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t kv_dtype) {
    if (int32_t e = check_layout_args(head_dim, block_size, kv_dtype)) return e;
    if (num_blocks <= 0 || num_kv_heads <= 0)
        return fail(PKV_ERR_ARG, "num_blocks and num_kv_heads must be positive");
    if ((int64_t)num_blocks * block_size >= (1LL << 31))
        return fail(PKV_ERR_ARG, "num_blocks * block_size must stay below 2^31 (slot numbers are int32)");
    ok();
    return (int64_t)num_blocks * num_kv_heads * block_size * head_dim * elem_size(kv_dtype);
}

int32_t kv_pool_create(const pkv_pool_desc* desc, void* const* k_layers, void* const* v_layers,
                       int64_t bytes_each, pkv_pool** out) {
    if (!desc || !k_layers || !v_layers || !out) return fail(PKV_ERR_ARG, "null argument");
    *out = nullptr;
    if (desc->num_layers <= 0) return fail(PKV_ERR_ARG, "num_layers must be positive");
    const int64_t need = pkv_layer_pool_bytes(desc->num_blocks, desc->num_kv_heads, desc->head_dim,
                                              desc->block_size, desc->kv_dtype);
    if (need < 0) return (int32_t)need;
    if (bytes_each < need)
        return fail(PKV_ERR_SIZE, "each layer pool needs %lld bytes, got %lld", (long long)need,
                    (long long)bytes_each);
    for (int32_t i = 0; i < desc->num_layers; ++i)
        if (!k_layers[i] || !v_layers[i]) return fail(PKV_ERR_ARG, "layer %d pointer is null", i);
    pkv_pool* p = new (std::nothrow) pkv_pool;
    if (!p) return fail(PKV_ERR_ARG, "out of host memory");
    p->desc = *desc;
    p->k.assign(k_layers, k_layers + desc->num_layers);
    p->v.assign(v_layers, v_layers + desc->num_layers);
    p->bytes_each = bytes_each;
    *out = p;
    return ok();
}

int32_t kv_pool_destroy(pkv_pool* pool) {
    delete pool;
    return ok();
}

int32_t kv_pool_get_desc(const pkv_pool* pool, pkv_pool_desc* out) {
    if (!pool || !out) return fail(PKV_ERR_ARG, "null argument");
    *out = pool->desc;
    return ok();
}

int32_t kv_pool_layer(const pkv_pool* pool, int32_t layer, void** k_cache, void** v_cache) {
    if (!pool || !k_cache || !v_cache) return fail(PKV_ERR_ARG, "null argument");
    if (layer < 0 || layer >= pool->desc.num_layers)
        return fail(PKV_ERR_ARG, "layer %d outside [0, %d)", layer, pool->desc.num_layers);
    *k_cache = pool->k[layer];
    *v_cache = pool->v[layer];
    return ok();
}

int32_t kv_pool_poison_null_block(const pkv_pool* pool, pkv_stream_t stream) {
    if (!pool) return fail(PKV_ERR_ARG, "null pool");
    const pkv_pool_desc& d = pool->desc;
    const int64_t bytes = (int64_t)d.num_kv_heads * d.block_size * d.head_dim * elem_size(d.kv_dtype);
    uint32_t pattern = d.kv_dtype == PKV_BF16 ? 0x7fc0u : (d.kv_dtype == PKV_FP16 ? 0x7e00u : 0x7fu);
    const int pattern_bytes = elem_size(d.kv_dtype);
    hipStream_t st = (hipStream_t)stream;
    for (int32_t i = 0; i < d.num_layers; ++i) {
        hipError_t e = pkv::launch_fill_pattern(pool->k[i], bytes, pattern, pattern_bytes, st);
        if (e == hipSuccess) e = pkv::launch_fill_pattern(pool->v[i], bytes, pattern, pattern_bytes, st);
        if (e != hipSuccess) return hip_fail(e, "null-block fill");
    }
    return ok();
}

int32_t pkv_decode_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                                int32_t* slot_mapping, pkv_stream_t stream) {
    if (num_seqs < 0 || max_blocks_per_seq < 0) return fail(PKV_ERR_ARG, "negative size");
    if (!valid_block_size(block_size)) return fail(PKV_ERR_ARG, "block_size %d must be 16 or 32", block_size);
    if (num_seqs > 0 && (!block_tables || !context_lens || !slot_mapping))
        return fail(PKV_ERR_ARG, "null pointer");
    (void)hipGetLastError();
    hipError_t e = pkv::launch_decode_slot_mapping(block_tables, max_blocks_per_seq, context_lens,
                                                   num_seqs, block_size, slot_mapping,
                                                   (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode_slot_mapping launch");
    return ok();
}

int32_t reshape_and_cache(const void* key, const void* value, int32_t src_dtype, void* k_cache,
                          void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, int32_t kv_dtype, float k_scale, float v_scale,
                          pkv_stream_t stream) {
    if (int32_t e = check_layout_args(head_dim, block_size, kv_dtype)) return e;
    if (src_dtype != PKV_BF16 && src_dtype != PKV_FP16)
        return fail(PKV_ERR_ARG, "src_dtype must be bf16 or fp16");
    if (num_kv_heads > 65535) return fail(PKV_ERR_UNSUPPORTED, "num_kv_heads must be <= 65535 (grid limit)");
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_ARG, "num_tokens >= 0, num_kv_heads > 0 and num_blocks > 0 required");
    if ((int64_t)num_blocks * block_size >= (1LL << 31))
        return fail(PKV_ERR_ARG, "num_blocks * block_size must stay below 2^31");
    if (!decode_head_dim(head_dim))
        return fail(PKV_ERR_UNSUPPORTED, "reshape_and_cache is built for head_dim 64, 128 and 256, got %d", head_dim);
    if (kv_dtype != PKV_FP8_E4M3 && kv_dtype != src_dtype)
        return fail(PKV_ERR_UNSUPPORTED, "a 16-bit pool must have the source dtype");
    if (num_tokens > 0 && (!key || !value || !k_cache || !v_cache || !slot_mapping))
        return fail(PKV_ERR_ARG, "null pointer");
    float k_inv = 1.0f, v_inv = 1.0f;
    if (kv_dtype == PKV_FP8_E4M3) {
        if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
            return fail(PKV_ERR_ARG, "fp8 scales must be finite and positive");
        k_inv = 1.0f / k_scale;   // IEEE fp32 division, correctly rounded
        v_inv = 1.0f / v_scale;
    }
    pkv::RacArgs a{key, value, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                   block_size, num_blocks, src_dtype, kv_dtype, k_inv, v_inv};
    (void)hipGetLastError();
    hipError_t e = pkv::launch_reshape_and_cache(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "reshape_and_cache launch");
    return ok();
}

int32_t pkv_default_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                     int32_t max_context_len, int32_t block_size) {
    if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0 || !valid_block_size(block_size))
        return fail(PKV_ERR_ARG, "bad partition query");
    ok();
    return resolve_partition(0, num_seqs, num_kv_heads, max_context_len, block_size);
}

int64_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_context_len,
                                        int32_t block_size, int32_t partition_tokens) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_context_len < 0 || partition_tokens < 0 || !valid_block_size(block_size) ||
        num_heads % num_kv_heads)
        return fail(PKV_ERR_ARG, "bad workspace query");
    const int32_t part = resolve_partition(partition_tokens, num_seqs, num_kv_heads, max_context_len, block_size);
    ok();
    return ws_layout(num_seqs, num_heads, num_kv_heads, head_dim, num_parts_of(max_context_len, part)).total;
}

int64_t paged_attention_plan_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                   int32_t block_size, int32_t partition_tokens) {
    if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0 || partition_tokens < 0 ||
        !valid_block_size(block_size))
        return fail(PKV_ERR_ARG, "bad plan query");
    const int32_t part = resolve_partition(partition_tokens, num_seqs, num_kv_heads, max_context_len, block_size);
    ok();
    return plan_bytes_of(num_seqs, num_parts_of(max_context_len, part));
}

int32_t paged_attention_plan(const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                             int32_t max_blocks_per_seq, int32_t num_kv_heads, int32_t block_size,
                             int32_t partition_tokens, void* plan, int64_t plan_bytes,
                             pkv_stream_t stream) {
    if (num_seqs < 0 || num_seqs > 65535 || num_kv_heads <= 0 || max_context_len < 0 ||
        max_blocks_per_seq < 0 || partition_tokens < 0 || !valid_block_size(block_size))
        return fail(PKV_ERR_ARG, "bad plan arguments");
    if (!plan || (num_seqs > 0 && !context_lens)) return fail(PKV_ERR_ARG, "null pointer");
    const int32_t ctx_cap = ctx_cap_of(max_context_len, max_blocks_per_seq, block_size);
    // the split size comes from max_context_len alone, as in the size queries
    const int32_t part = resolve_partition(partition_tokens, num_seqs, num_kv_heads, max_context_len, block_size);
    if (part % block_size) return fail(PKV_ERR_ARG, "partition_tokens %d is not a multiple of block_size %d", part, block_size);
    const int64_t need = plan_bytes_of(num_seqs, num_parts_of(ctx_cap, part));
    if (plan_bytes < need) return fail(PKV_ERR_SIZE, "plan needs %lld bytes, got %lld", (long long)need, (long long)plan_bytes);
    (void)hipGetLastError();
    hipError_t e = pkv::launch_plan(context_lens, num_seqs, ctx_cap, block_size, part / block_size,
                                    (int32_t*)plan, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    return ok();
}

// The decode behind paged_attention_decode_ex and _append: `append` (may be
// null) carries the new token's K / V rows and the inverse fp8 scales.
struct AppendRows {
    const void* key;
    const void* value;
    float k_inv, v_inv;
};

static int32_t decode_impl(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                           const void* v_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, float scale, int32_t block_size,
                           int32_t kv_dtype, float k_scale, float v_scale, void* workspace,
                           int64_t workspace_bytes, const pkv_decode_opts* opts,
                           const AppendRows* append, pkv_stream_t stream) {
    pkv_decode_opts o{0, PKV_IMPL_AUTO, 0, 0, nullptr};
    if (opts) o = *opts;
    if (int32_t e = check_layout_args(head_dim, block_size, kv_dtype)) return e;
    if (q_dtype != PKV_BF16 && q_dtype != PKV_FP16) return fail(PKV_ERR_ARG, "q_dtype must be bf16 or fp16");
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 || max_blocks_per_seq < 0)
        return fail(PKV_ERR_ARG, "bad sizes");
    if (num_heads % num_kv_heads) return fail(PKV_ERR_ARG, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
    const int32_t G = num_heads / num_kv_heads;
    pkv::DecodeArgs a{};
    // entry heads: column groups of <= 32 query heads (<= 16 at head_dim 256)
    pkv::set_heads(a, num_heads, num_kv_heads, pkv::decode_max_cols(head_dim));
    if ((int64_t)num_seqs * a.num_kv_heads > 0x7fffffff || num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "num_seqs must be <= 65535 and num_seqs * num_kv_heads < 2^31 (grid limits)");
    if (!decode_head_dim(head_dim))
        return fail(PKV_ERR_UNSUPPORTED, "decode is built for head_dim 64, 128 and 256, got %d", head_dim);
    if (kv_dtype != PKV_FP8_E4M3 && kv_dtype != q_dtype)
        return fail(PKV_ERR_UNSUPPORTED, "a 16-bit KV pool must have the query dtype");
    if (!std::isfinite(scale)) return fail(PKV_ERR_ARG, "scale must be finite");
    if (kv_dtype == PKV_FP8_E4M3 && !(std::isfinite(k_scale) && std::isfinite(v_scale)))
        return fail(PKV_ERR_ARG, "fp8 scales must be finite");
    if (o.impl < 0 || o.impl > 3) return fail(PKV_ERR_ARG, "impl %d unknown", o.impl);
    if (o.impl == PKV_IMPL_VECTOR && head_dim != kBuiltHeadDim)
        return fail(PKV_ERR_UNSUPPORTED, "the vector kernel is built for head_dim 128");
    if (o.impl == PKV_IMPL_VECTOR && G > 8) return fail(PKV_ERR_UNSUPPORTED, "vector kernel supports at most 8 query heads per kv head");
    const int32_t stages = o.stages ? o.stages : (PKV_STAGE_PARTITIONS | PKV_STAGE_REDUCE);
    if (stages & ~(PKV_STAGE_PARTITIONS | PKV_STAGE_REDUCE)) return fail(PKV_ERR_ARG, "bad stages mask");
    if (o.partition_tokens < 0) return fail(PKV_ERR_ARG, "partition_tokens < 0");
    if (o.num_blocks < 0) return fail(PKV_ERR_ARG, "num_blocks < 0");
    if (num_seqs > 0 && (!out || !q || !k_cache || !v_cache || !context_lens || (max_blocks_per_seq > 0 && !block_tables)))
        return fail(PKV_ERR_ARG, "null pointer");

    const int32_t ctx_cap = ctx_cap_of(max_context_len, max_blocks_per_seq, block_size);
    // The split size comes from max_context_len alone, as in
    // paged_attention_workspace_bytes / _plan_bytes; the partition count from
    // the (possibly smaller) clamped context, so it never exceeds theirs.
    const int32_t part_tokens = resolve_partition(o.partition_tokens, num_seqs, num_kv_heads, max_context_len, block_size);
    if (part_tokens < block_size || part_tokens % block_size)
        return fail(PKV_ERR_ARG, "partition_tokens %d must be a positive multiple of block_size %d", part_tokens, block_size);
    const int64_t num_parts = num_parts_of(ctx_cap, part_tokens);
    if (num_parts > 65535) return fail(PKV_ERR_UNSUPPORTED, "more than 65535 partitions (raise partition_tokens)");
    if ((int64_t)num_seqs * a.num_kv_heads * num_parts > 0x7fffffff)
        return fail(PKV_ERR_UNSUPPORTED, "too many workgroups (raise partition_tokens)");
    const WsLayout wl = ws_layout(num_seqs, num_heads, num_kv_heads, head_dim, num_parts);
    const int64_t need = o.plan ? wl.plan_off : wl.total;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PKV_ERR_SIZE, "workspace needs %lld bytes, got %lld", (long long)need, (long long)workspace_bytes);

    a.out = out;
    a.q = q;
    a.k_cache = (const uint8_t*)k_cache;
    a.v_cache = (const uint8_t*)v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.ws_out = (float*)workspace;
    a.ws_ml = wl.ml_bytes ? (float*)((char*)workspace + wl.o_bytes) : nullptr;
    a.plan = o.plan ? (const int32_t*)o.plan : (const int32_t*)((char*)workspace + wl.plan_off);
    a.max_blocks = max_blocks_per_seq;
    a.ctx_cap = ctx_cap;
    a.num_seqs = num_seqs;
    a.part_blocks = part_tokens / block_size;
    a.num_parts = (int32_t)num_parts;
    a.num_blocks = o.num_blocks;
    a.head_dim = head_dim;
    const float ks = kv_dtype == PKV_FP8_E4M3 ? k_scale : 1.0f;
    a.qk_scale_log2 = (float)((double)scale * (double)ks * 1.4426950408889634);
    a.out_scale = kv_dtype == PKV_FP8_E4M3 ? v_scale : 1.0f;
    if (append) {
        a.new_key = append->key;
        a.new_value = append->value;
        a.k_inv = append->k_inv;
        a.v_inv = append->v_inv;
    }

    hipStream_t st = (hipStream_t)stream;
    (void)hipGetLastError();
    if ((stages & PKV_STAGE_PARTITIONS) && !o.plan && num_seqs > 0) {
        hipError_t e = pkv::launch_plan(context_lens, num_seqs, ctx_cap, block_size, a.part_blocks,
                                        (int32_t*)a.plan, st);
        if (e != hipSuccess) return hip_fail(e, "plan launch");
    }
    if (stages & PKV_STAGE_PARTITIONS) {
        hipError_t e = pkv::launch_decode_partitions(a, q_dtype, kv_dtype, block_size, o.impl, st);
        if (e != hipSuccess) return hip_fail(e, "paged decode launch");
    }
    if ((stages & PKV_STAGE_REDUCE) && num_parts > 1) {
        hipError_t e = pkv::launch_decode_reduce(a, q_dtype, block_size, st);
        if (e != hipSuccess) return hip_fail(e, "partition reduce launch");
    }
    return ok();
}

int32_t paged_attention_decode_ex(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, float scale,
                                  int32_t block_size, int32_t kv_dtype, float k_scale,
                                  float v_scale, void* workspace, int64_t workspace_bytes,
                                  const pkv_decode_opts* opts, pkv_stream_t stream) {
    return decode_impl(out, q, q_dtype, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, num_seqs, num_heads, num_kv_heads, head_dim,
                       scale, block_size, kv_dtype, k_scale, v_scale, workspace, workspace_bytes,
                       opts, nullptr, stream);
}

int32_t paged_attention_decode_append(void* out, const void* q, int32_t q_dtype, const void* key,
                                      const void* value, void* k_cache, void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t max_context_len,
                                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, float scale, int32_t block_size,
                                      int32_t kv_dtype, float k_scale, float v_scale,
                                      void* workspace, int64_t workspace_bytes,
                                      const pkv_decode_opts* opts, pkv_stream_t stream) {
    if (!opts || opts->num_blocks <= 0)
        return fail(PKV_ERR_ARG, "decode_append needs opts->num_blocks > 0 (the pool size bounds the write)");
    if (opts->stages && !(opts->stages & PKV_STAGE_PARTITIONS))
        return fail(PKV_ERR_ARG, "decode_append writes in the partition stage; it cannot be left out");
    if (valid_block_size(block_size) && (int64_t)opts->num_blocks * block_size >= (1LL << 31))
        return fail(PKV_ERR_ARG, "num_blocks * block_size must stay below 2^31");
    if (num_seqs > 0 && (!key || !value)) return fail(PKV_ERR_ARG, "null pointer");
    AppendRows ap{key, value, 1.0f, 1.0f};
    if (kv_dtype == PKV_FP8_E4M3) {
        if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
            return fail(PKV_ERR_ARG, "fp8 scales must be finite and positive");
        ap.k_inv = 1.0f / k_scale;   // as reshape_and_cache
        ap.v_inv = 1.0f / v_scale;
    }
    return decode_impl(out, q, q_dtype, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, num_seqs, num_heads, num_kv_heads, head_dim,
                       scale, block_size, kv_dtype, k_scale, v_scale, workspace, workspace_bytes,
                       opts, &ap, stream);
}

int32_t paged_attention_prefill(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                const int32_t* query_start_loc, int32_t max_query_len,
                                int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, float scale,
                                int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                                float k_scale, float v_scale, pkv_stream_t stream) {
    if (int32_t e = check_layout_args(head_dim, block_size, kv_dtype)) return e;
    if (q_dtype != PKV_BF16 && q_dtype != PKV_FP16) return fail(PKV_ERR_ARG, "q_dtype must be bf16 or fp16");
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
        max_blocks_per_seq < 0 || max_query_len < 0 || num_blocks < 0)
        return fail(PKV_ERR_ARG, "bad sizes");
    if (num_heads % num_kv_heads) return fail(PKV_ERR_ARG, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
    if (head_dim != kBuiltHeadDim) return fail(PKV_ERR_UNSUPPORTED, "kernels are built for head_dim 128, got %d", head_dim);
    if (kv_dtype != PKV_FP8_E4M3 && kv_dtype != q_dtype)
        return fail(PKV_ERR_UNSUPPORTED, "a 16-bit KV pool must have the query dtype");
    if (!std::isfinite(scale)) return fail(PKV_ERR_ARG, "scale must be finite");
    if (kv_dtype == PKV_FP8_E4M3 && !(std::isfinite(k_scale) && std::isfinite(v_scale)))
        return fail(PKV_ERR_ARG, "fp8 scales must be finite");
    if (num_seqs > 0 && (!out || !q || !k_cache || !v_cache || !context_lens || !query_start_loc ||
                         (max_blocks_per_seq > 0 && !block_tables)))
        return fail(PKV_ERR_ARG, "null pointer");
    pkv::DecodeArgs a{};
    pkv::set_heads(a, num_heads, num_kv_heads);   // entry heads: column groups of <= 16 query heads
    const int32_t tile_tokens = 16 / a.group;
    const int64_t max_tiles = ((int64_t)max_query_len + tile_tokens - 1) / tile_tokens;
    if ((int64_t)num_seqs * max_tiles * a.num_kv_heads > 0x7fffffff)
        return fail(PKV_ERR_UNSUPPORTED, "too many workgroups");
    a.out = out;
    a.q = q;
    a.k_cache = (const uint8_t*)k_cache;
    a.v_cache = (const uint8_t*)v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.max_blocks = max_blocks_per_seq;
    a.ctx_cap = ctx_cap_of(max_context_len, max_blocks_per_seq, block_size);
    a.num_seqs = num_seqs;
    a.part_blocks = std::max(1, max_blocks_per_seq);   // one partition: the whole context
    a.num_parts = 1;
    a.num_blocks = num_blocks;
    a.head_dim = head_dim;
    const float ks = kv_dtype == PKV_FP8_E4M3 ? k_scale : 1.0f;
    a.qk_scale_log2 = (float)((double)scale * (double)ks * 1.4426950408889634);
    a.out_scale = kv_dtype == PKV_FP8_E4M3 ? v_scale : 1.0f;
    (void)hipGetLastError();
    hipError_t e = pkv::launch_prefill(a, q_dtype, kv_dtype, block_size, query_start_loc, tile_tokens,
                                       (int)max_tiles, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "paged prefill launch");
    return ok();
}

// Checks shared by the token-table decodes; fills the launch arguments.
// `table` is the token table or the run list (what max_tokens_per_seq
// sizes).
static int32_t token_decode_args(pkv::DecodeArgs& a, void* out, const void* q, int32_t q_dtype,
                                 const void* k_cache, const void* v_cache, const void* table,
                                 int32_t max_tokens_per_seq, const int32_t* context_lens,
                                 bool need_context_lens, int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim, float scale, int32_t block_size,
                                 int32_t num_blocks, int32_t kv_dtype, float k_scale, float v_scale) {
    if (int32_t e = check_layout_args(head_dim, block_size, kv_dtype)) return e;
    if (q_dtype != PKV_BF16 && q_dtype != PKV_FP16) return fail(PKV_ERR_ARG, "q_dtype must be bf16 or fp16");
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_tokens_per_seq < 0 || num_blocks < 2)
        return fail(PKV_ERR_ARG, "bad sizes (num_blocks must count the null block and at least one more)");
    if ((int64_t)num_blocks * block_size >= (1LL << 31)) return fail(PKV_ERR_ARG, "slots must fit int32");
    if (num_heads % num_kv_heads) return fail(PKV_ERR_ARG, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
    if (head_dim != kBuiltHeadDim) return fail(PKV_ERR_UNSUPPORTED, "kernels are built for head_dim 128, got %d", head_dim);
    if (kv_dtype != PKV_FP8_E4M3 && kv_dtype != q_dtype)
        return fail(PKV_ERR_UNSUPPORTED, "a 16-bit KV pool must have the query dtype");
    if (!std::isfinite(scale)) return fail(PKV_ERR_ARG, "scale must be finite");
    if (kv_dtype == PKV_FP8_E4M3 && !(std::isfinite(k_scale) && std::isfinite(v_scale)))
        return fail(PKV_ERR_ARG, "fp8 scales must be finite");
    pkv::set_heads(a, num_heads, num_kv_heads);   // entry heads: column groups of <= 16 query heads
    if ((int64_t)num_seqs * a.num_kv_heads > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "too many workgroups");
    if (num_seqs > 0 && (!out || !q || !k_cache || !v_cache || (need_context_lens && !context_lens) ||
                         (max_tokens_per_seq > 0 && !table)))
        return fail(PKV_ERR_ARG, "null pointer");
    a.out = out;
    a.q = q;
    a.k_cache = (const uint8_t*)k_cache;
    a.v_cache = (const uint8_t*)v_cache;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.part_blocks = 1;
    a.num_parts = 1;
    a.num_blocks = num_blocks;
    a.head_dim = head_dim;
    const float ks = kv_dtype == PKV_FP8_E4M3 ? k_scale : 1.0f;
    a.qk_scale_log2 = (float)((double)scale * (double)ks * 1.4426950408889634);
    a.out_scale = kv_dtype == PKV_FP8_E4M3 ? v_scale : 1.0f;
    return PKV_OK;
}

int32_t paged_attention_decode_tokens(void* out, const void* q, int32_t q_dtype,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* token_slots, int32_t max_tokens_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float scale, int32_t block_size, int32_t num_blocks,
                                      int32_t kv_dtype, float k_scale, float v_scale,
                                      pkv_stream_t stream) {
    pkv::DecodeArgs a{};
    if (int32_t e = token_decode_args(a, out, q, q_dtype, k_cache, v_cache, token_slots, max_tokens_per_seq,
                                      context_lens, true, num_seqs, num_heads, num_kv_heads, head_dim, scale,
                                      block_size, num_blocks, kv_dtype, k_scale, v_scale))
        return e;
    (void)hipGetLastError();
    hipError_t e = pkv::launch_decode_tokens(a, q_dtype, kv_dtype, block_size, token_slots,
                                             max_tokens_per_seq, nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "token-table decode launch");
    return ok();
}

// Run list: [counts: num_seqs int32][lengths in tokens, 16 x counts][plan
// of the decode: one item per sequence, longest first][entries: num_seqs x
// max_tokens_per_seq pairs of int32]; each area starts on 256 bytes.
struct RunsLayout { int64_t lens16, plan, entries, total; };
static RunsLayout runs_layout(int32_t num_seqs, int32_t max_tokens_per_seq) {
    RunsLayout r{};
    r.lens16 = align256(4LL * num_seqs);
    r.plan = r.lens16 + align256(4LL * num_seqs);
    r.entries = r.plan + plan_bytes_of(num_seqs, 1);
    r.total = r.entries + 8LL * num_seqs * max_tokens_per_seq;
    return r;
}
// the plan sizes items in tokens: 16 per table entry at most
constexpr int32_t kMaxRunTokens = (1 << 27) - 1;

int64_t pkv_token_runs_bytes(int32_t num_seqs, int32_t max_tokens_per_seq) {
    if (num_seqs < 0 || max_tokens_per_seq < 0 || max_tokens_per_seq > kMaxRunTokens)
        return fail(PKV_ERR_ARG, "bad sizes");
    ok();
    return runs_layout(num_seqs, max_tokens_per_seq).total;
}

int32_t pkv_token_runs(const int32_t* token_slots, int32_t max_tokens_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                       int32_t num_blocks, int32_t min_keys_per_entry, void* runs, int64_t runs_bytes,
                       pkv_stream_t stream) {
    if (!valid_block_size(block_size)) return fail(PKV_ERR_ARG, "block_size must be 16 or 32");
    if (min_keys_per_entry < 0 || min_keys_per_entry > 16) return fail(PKV_ERR_ARG, "min_keys_per_entry must be 0..16");
    if (num_seqs < 0 || num_seqs > 65535 || max_tokens_per_seq < 0 || max_tokens_per_seq > kMaxRunTokens ||
        num_blocks < 2)
        return fail(PKV_ERR_ARG, "bad sizes (num_seqs <= 65535, max_tokens_per_seq < 2^27, num_blocks must "
                                 "count the null block and at least one more)");
    if ((int64_t)num_blocks * block_size >= (1LL << 31)) return fail(PKV_ERR_ARG, "slots must fit int32");
    if (num_seqs == 0) return ok();
    if (!runs || !context_lens || (max_tokens_per_seq > 0 && !token_slots)) return fail(PKV_ERR_ARG, "null pointer");
    const RunsLayout rl = runs_layout(num_seqs, max_tokens_per_seq);
    if (runs_bytes < rl.total)
        return fail(PKV_ERR_SIZE, "run list needs %lld bytes, got %lld", (long long)rl.total, (long long)runs_bytes);
    if ((uintptr_t)runs % 8) return fail(PKV_ERR_ARG, "run list must be 8-byte aligned");
    (void)hipGetLastError();
    char* rb = (char*)runs;
    hipError_t e = pkv::launch_token_runs(token_slots, max_tokens_per_seq, context_lens, num_seqs, block_size,
                                          num_blocks, min_keys_per_entry, (int32_t*)rb, (int32_t*)(rb + rl.lens16),
                                          (int32_t*)(rb + rl.plan), (int2*)(rb + rl.entries), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "run-list launch");
    return ok();
}

int32_t paged_attention_decode_runs(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                                    const void* v_cache, const void* runs, int64_t runs_bytes,
                                    const int32_t* token_slots, const int32_t* context_lens,
                                    int32_t max_tokens_per_seq, int32_t num_seqs, int32_t num_heads,
                                    int32_t num_kv_heads,
                                    int32_t head_dim, float scale, int32_t block_size, int32_t num_blocks,
                                    int32_t kv_dtype, float k_scale, float v_scale, pkv_stream_t stream) {
    pkv::DecodeArgs a{};
    if (int32_t e = token_decode_args(a, out, q, q_dtype, k_cache, v_cache, runs, max_tokens_per_seq, nullptr,
                                      false, num_seqs, num_heads, num_kv_heads, head_dim, scale, block_size,
                                      num_blocks, kv_dtype, k_scale, v_scale))
        return e;
    if ((token_slots == nullptr) != (context_lens == nullptr))
        return fail(PKV_ERR_ARG, "token_slots and context_lens go together (both or neither)");
    if (num_seqs > 0 && !runs) return fail(PKV_ERR_ARG, "null pointer");
    if ((uintptr_t)runs % 8) return fail(PKV_ERR_ARG, "run list must be 8-byte aligned");
    if (num_seqs > 65535 || max_tokens_per_seq > kMaxRunTokens)
        return fail(PKV_ERR_ARG, "num_seqs <= 65535 and max_tokens_per_seq < 2^27");
    const RunsLayout rl = runs_layout(num_seqs, max_tokens_per_seq);
    if (num_seqs > 0 && runs_bytes < rl.total)
        return fail(PKV_ERR_SIZE, "run list of %lld bytes, needs %lld", (long long)runs_bytes, (long long)rl.total);
    const char* rb = (const char*)runs;
    a.plan = (const int32_t*)(rb + rl.plan);
    (void)hipGetLastError();
    hipError_t e = pkv::launch_decode_runs(a, q_dtype, kv_dtype, block_size, (const int32_t*)rb,
                                           (const int2*)(rb + rl.entries), max_tokens_per_seq,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "run-list decode launch");
    if (token_slots) {
        // the sequences the run list marked for the token gather
        a.context_lens = context_lens;
        e = pkv::launch_decode_tokens(a, q_dtype, kv_dtype, block_size, token_slots, max_tokens_per_seq,
                                      (const int32_t*)rb, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "token-table decode launch");
    }
    return ok();
}

int64_t pkv_move_tokens_scratch_bytes(int32_t num_layers, int32_t num_moves,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t kv_dtype) {
    if (!valid_dtype(kv_dtype) || num_layers < 0 || num_moves < 0 || num_kv_heads <= 0 || head_dim <= 0)
        return fail(PKV_ERR_ARG, "bad sizes");
    ok();
    return (int64_t)num_moves * num_layers * 2 * num_kv_heads * head_dim * elem_size(kv_dtype);
}

int32_t pkv_move_tokens(void* const* k_layers, void* const* v_layers, int32_t num_layers,
                        int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t kv_dtype, const int32_t* moves,
                        int32_t num_moves, void* scratch, int64_t scratch_bytes,
                        pkv_stream_t stream) {
    if (int32_t e = check_layout_args(head_dim, block_size, kv_dtype)) return e;
    if (head_dim != kBuiltHeadDim) return fail(PKV_ERR_UNSUPPORTED, "kernels are built for head_dim 128, got %d", head_dim);
    if (num_layers < 0 || num_moves < 0 || num_kv_heads <= 0 || num_blocks < 1)
        return fail(PKV_ERR_ARG, "bad sizes");
    if ((int64_t)num_blocks * block_size >= (1LL << 31)) return fail(PKV_ERR_ARG, "slots must fit int32");
    if (num_moves == 0 || num_layers == 0) return ok();
    if (!k_layers || !v_layers || !moves) return fail(PKV_ERR_ARG, "null pointer");
    for (int32_t l = 0; l < num_layers; ++l)
        if (!k_layers[l] || !v_layers[l]) return fail(PKV_ERR_ARG, "null layer pointer");
    const int64_t need = (int64_t)num_moves * num_layers * 2 * num_kv_heads * head_dim * elem_size(kv_dtype);
    if (!scratch || scratch_bytes < need)
        return fail(PKV_ERR_SIZE, "scratch needs %lld bytes, got %lld", (long long)need, (long long)scratch_bytes);
    (void)hipGetLastError();
    hipError_t e = pkv::launch_move_tokens(k_layers, v_layers, num_layers, num_blocks, num_kv_heads,
                                           block_size, kv_dtype, moves, num_moves, scratch,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "move_tokens launch");
    return ok();
}

int32_t pkv_repack_blocks(void* const* k_layers, void* const* v_layers, int32_t num_layers,
                          int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t kv_dtype, const int32_t* tiles,
                          const int32_t* chain_offsets, int32_t num_chains, pkv_stream_t stream) {
    if (int32_t e = check_layout_args(head_dim, block_size, kv_dtype)) return e;
    if (head_dim != kBuiltHeadDim) return fail(PKV_ERR_UNSUPPORTED, "kernels are built for head_dim 128, got %d", head_dim);
    if (num_layers < 0 || num_chains < 0 || num_kv_heads <= 0 || num_blocks < 1)
        return fail(PKV_ERR_ARG, "bad sizes");
    if (num_kv_heads > 65535) return fail(PKV_ERR_UNSUPPORTED, "num_kv_heads must be <= 65535 (grid limit)");
    if ((int64_t)num_blocks * block_size >= (1LL << 31)) return fail(PKV_ERR_ARG, "slots must fit int32");
    if (num_chains == 0 || num_layers == 0) return ok();
    if (!k_layers || !v_layers || !tiles || !chain_offsets) return fail(PKV_ERR_ARG, "null pointer");
    for (int32_t l = 0; l < num_layers; ++l)
        if (!k_layers[l] || !v_layers[l]) return fail(PKV_ERR_ARG, "null layer pointer");
    (void)hipGetLastError();
    hipError_t e = pkv::launch_repack_blocks(k_layers, v_layers, num_layers, num_blocks, num_kv_heads,
                                             block_size, kv_dtype, tiles, chain_offsets, num_chains,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "repack_blocks launch");
    return ok();
}

int32_t paged_attention_decode(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, float scale,
                               int32_t block_size, int32_t kv_dtype, float k_scale, float v_scale,
                               void* workspace, int64_t workspace_bytes, pkv_stream_t stream) {
    return paged_attention_decode_ex(out, q, q_dtype, k_cache, v_cache, block_tables,
                                     max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                                     num_heads, num_kv_heads, head_dim, scale, block_size,
                                     kv_dtype, k_scale, v_scale, workspace, workspace_bytes,
                                     nullptr, stream);
}

int32_t pkv_check_block_tables(const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                               int32_t num_blocks, int32_t* scratch_dev, int64_t* bad_count,
                               pkv_stream_t stream) {
    if (!bad_count || !scratch_dev) return fail(PKV_ERR_ARG, "null pointer");
    if (num_seqs < 0 || max_blocks_per_seq < 0 || num_blocks <= 0) return fail(PKV_ERR_ARG, "bad sizes");
    if (!valid_block_size(block_size)) return fail(PKV_ERR_ARG, "block_size %d must be 16 or 32", block_size);
    if (num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !block_tables)))
        return fail(PKV_ERR_ARG, "null pointer");
    hipStream_t st = (hipStream_t)stream;
    (void)hipGetLastError();
    hipError_t e = pkv::launch_check_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                            block_size, num_blocks, scratch_dev, st);
    if (e != hipSuccess) return hip_fail(e, "table check launch");
    int32_t host = 0;
    e = hipMemcpyAsync(&host, scratch_dev, sizeof host, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "table check readback");
    *bad_count = host;
    return ok();
}

int64_t pkv_read_probe_sink_bytes(void) { return pkv::read_probe_sink_bytes(); }

int32_t pkv_read_probe(const void* src, int64_t bytes, void* sink, int64_t sink_bytes, pkv_stream_t stream) {
    if (bytes < 0 || bytes % 16 != 0) return fail(PKV_ERR_ARG, "bytes %lld must be a non-negative multiple of 16",
                                                  (long long)bytes);
    if (bytes == 0) return ok();
    if (!src || !sink) return fail(PKV_ERR_ARG, "null pointer");
    if (((uintptr_t)src | (uintptr_t)sink) % 16 != 0) return fail(PKV_ERR_ARG, "src and sink must be 16-byte aligned");
    const int64_t need = pkv::read_probe_sink_bytes();
    if (sink_bytes < need)
        return fail(PKV_ERR_SIZE, "sink holds %lld bytes, the probe needs %lld", (long long)sink_bytes,
                    (long long)need);
    (void)hipGetLastError();
    hipError_t e = pkv::launch_read_probe(src, bytes / 16, sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "read probe launch");
    return ok();
}

}  // extern "C"
