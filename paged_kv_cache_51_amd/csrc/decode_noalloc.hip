// decode_noalloc.hip — paged_attention_decode for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops or
// harnesses that forbid allocation): the decode's workspace (work plan and
// partition partials) lives in a file-scope device array instead of
// caller memory.  The kernels are paged_attention_decode's.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pagedkv.h"
#include "pkv_launch.h"

// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in): its device address is looked up once per
// device, with that device current, and that address is what the kernels
// receive.
static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int32_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return pkv::hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return pkv::fail(PKV_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return pkv::hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return pkv::fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return PKV_OK;
}

}  // namespace

extern "C" int32_t paged_attention_decode_noalloc(
    void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t max_context_len, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t block_size, int32_t kv_dtype, float k_scale,
    float v_scale, pkv_stream_t stream) {
    // the workspace this decode needs, checked before anything is set up
    const int64_t need = paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                         max_context_len, block_size, 0);
    if (need < 0) return (int32_t)need;
    if (need > PKV_NOALLOC_SCRATCH_BYTES)
        return pkv::fail(PKV_ERR_SIZE,
                         "this decode needs %lld bytes of workspace; the static scratch of "
                         "paged_attention_decode_noalloc holds %lld (use paged_attention_decode)",
                         (long long)need, (long long)PKV_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (int32_t e = scratch_address(&ws)) return e;
    // Every scratch byte the kernels read is written earlier in the same
    // call (the plan kernel writes the plan and its counters, the partition
    // kernel the partials the reduce reads), so nothing needs clearing.
    return paged_attention_decode_ex(out, q, q_dtype, k_cache, v_cache, block_tables,
                                     max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                                     num_heads, num_kv_heads, head_dim, scale, block_size, kv_dtype,
                                     k_scale, v_scale, ws, PKV_NOALLOC_SCRATCH_BYTES, nullptr, stream);
}
