// pkv_launch.h — host-side launchers between the C ABI (api.hip) and the
// kernels.  Argument checking happens in api.hip; launchers assume valid
// arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct RacArgs {
    const void* key;
    const void* value;
    void* k_cache;
    void* v_cache;
    const int32_t* slot_mapping;
    int32_t num_tokens;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t num_blocks;
    int32_t src_dtype;
    int32_t kv_dtype;
    float k_inv;
    float v_inv;
};

struct DecodeArgs {
    void* out;
    const void* q;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* ws_out;         // [S][num_kv_heads][P][group][head_dim] partial outputs (normalised)
    float* ws_ml;          // [S][num_kv_heads][P][ml_line(group)] (max in log2 units, normaliser per column)
    const int32_t* plan;   // work plan (plan.hip): count, then (seq << 16 | part)
    int32_t max_blocks;    // block-table row length
    int32_t ctx_cap;       // context clamp: min(max_context_len, max_blocks*bs)
    int32_t num_seqs;
    int32_t num_heads;
    // Entry heads.  A pool kv head whose query heads fit the columns one
    // work entry holds (16: one MFMA tile; the decode partition kernel takes
    // 32, two tiles, at head_dim <= 128) is one entry head (kv_split = 1,
    // group = its query heads).  A larger group (MQA, or GQA with many query
    // heads per kv head) is split into kv_split entry heads of `group`
    // columns each, the last one possibly fewer; all of them read the same
    // K / V.  Set by set_heads().
    int32_t num_kv_heads;  // entry heads: pool_kv_heads * kv_split
    int32_t group;         // query-head columns per entry head (<= 16, or <= 32 in decode)
    int32_t kv_split;      // entry heads per pool kv head
    int32_t group_all;     // query heads per pool kv head (num_heads / pool_kv_heads)
    int32_t pool_kv_heads; // kv heads of the pool
    int32_t part_blocks;   // blocks per partition
    int32_t num_parts;     // partitions launched per (seq, kv head)
    int32_t num_blocks;    // pool size for id clamping (0 = unchecked)
    int32_t head_dim;      // 64, 128 or 256 (decode); 128 elsewhere
    float qk_scale_log2;   // scale * k_scale * log2(e)
    float out_scale;       // v_scale for fp8 pools, else 1
    // Append (decode only; null = off): the new token's K and V rows
    // [num_seqs][num_kv_heads][head_dim] in the query dtype, written to the
    // slot of position c - 1 by the workgroup whose partition holds it,
    // before that workgroup reads the pool.  The pools are then written
    // through k_cache / v_cache.
    const void* new_key;
    const void* new_value;
    float k_inv;           // 1 / k_scale for fp8 pools, else 1
    float v_inv;
};

// Entry heads of a (num_heads, num_kv_heads) layout: the fewest entry heads
// per kv head whose columns fit max_cols, columns spread evenly.
inline void set_heads(DecodeArgs& a, int32_t num_heads, int32_t num_kv_heads, int32_t max_cols = 16) {
    const int32_t g_all = num_heads / num_kv_heads;
    const int32_t split = (g_all + max_cols - 1) / max_cols;
    a.num_heads = num_heads;
    a.pool_kv_heads = num_kv_heads;
    a.group_all = g_all;
    a.kv_split = split;
    a.group = (g_all + split - 1) / split;
    a.num_kv_heads = num_kv_heads * split;
}

// Columns of a decode work entry at head_dim d: two 16-column MFMA tiles up
// to d = 128, one at 256 (the accumulators of two would not fit).
inline int32_t decode_max_cols(int32_t head_dim) { return head_dim <= 128 ? 32 : 16; }

// Floats of one partition record's line of maxima and normalisers: 16 + 16
// for entries of at most 16 columns, 32 + 32 above.
__host__ __device__ inline int ml_line(int group) { return group > 16 ? 64 : 32; }

// Error reporting shared by the extern "C" entry points (api.hip): set the
// thread-local message and return the code.
int32_t fail(int32_t code, const char* fmt, ...);
int32_t ok();
int32_t hip_fail(hipError_t e, const char* what);

hipError_t launch_reshape_and_cache(const RacArgs& a, hipStream_t st);
hipError_t launch_decode_slot_mapping(const int32_t* bt, int32_t max_blocks, const int32_t* ctx,
                                      int32_t num_seqs, int32_t bs, int32_t* slots,
                                      hipStream_t st);
hipError_t launch_check_tables(const int32_t* bt, int32_t max_blocks, const int32_t* ctx,
                               int32_t num_seqs, int32_t bs, int32_t num_blocks, int32_t* bad,
                               hipStream_t st);
hipError_t launch_plan(const int32_t* context_lens, int32_t num_seqs, int32_t ctx_cap,
                       int32_t block_size, int32_t part_blocks, int32_t* plan, hipStream_t st);
hipError_t launch_fill_pattern(void* p, int64_t n_bytes, uint32_t pattern, int pattern_bytes,
                               hipStream_t st);
// Read-stream probe: sink holds read_probe_sink_bytes() bytes.
int64_t read_probe_sink_bytes();
hipError_t launch_read_probe(const void* src, int64_t n16, void* sink, hipStream_t st);

// Partition kernel (matrix-core or vector implementation) and the merge.
hipError_t launch_decode_partitions(const DecodeArgs& a, int q_dtype, int kv_dtype,
                                    int block_size, int impl, hipStream_t st);
hipError_t launch_decode_reduce(const DecodeArgs& a, int q_dtype, int block_size,
                                hipStream_t st);
// Decode through a per-token slot table; token moves between slots
// (decode_tokens.hip).
hipError_t launch_decode_tokens(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                                const int32_t* token_slots, int max_tokens, const int32_t* only_marked,
                                hipStream_t st);
// Run lists of a token table, and decode through them (decode_tokens.hip).
hipError_t launch_token_runs(const int32_t* token_slots, int max_tokens, const int32_t* context_lens,
                             int num_seqs, int block_size, int num_blocks, int min_keys, int32_t* counts,
                             int32_t* lens16, int32_t* plan, int2* entries, hipStream_t st);
hipError_t launch_decode_runs(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                              const int32_t* counts, const int2* entries, int max_tokens, hipStream_t st);
hipError_t launch_repack_blocks(void* const* k_layers, void* const* v_layers, int num_layers,
                                int num_blocks, int num_kv_heads, int block_size, int kv_dtype,
                                const int32_t* tiles, const int32_t* chain_offsets, int num_chains,
                                hipStream_t st);
hipError_t launch_move_tokens(void* const* k_layers, void* const* v_layers, int num_layers,
                              int num_blocks, int num_kv_heads, int block_size, int kv_dtype,
                              const int32_t* moves, int num_moves, void* scratch, hipStream_t st);

// Multi-token attention (query tiles of tile_tokens tokens, causal).
hipError_t launch_prefill(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                          const int32_t* query_start, int tile_tokens, int max_tiles,
                          hipStream_t st);

}  // namespace pkv
