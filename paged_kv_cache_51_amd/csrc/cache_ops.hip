// cache_ops.hip — writing new tokens into the paged pool, and the small
// indexing kernels around it.
//
// Pages: "LLM inference basics and vLLM internals" (ttlab.hopto.org) §4 —
// tokens live in fixed 16-token blocks reached through a per-request block
// table, block 0 is reserved as the null block; vToken page
// (gotosocial.chinng-lab-srv.dev) "KV cache basics" — each decode step only
// appends the new token's key and value.
#include "cache_write.h"
#include "pkv_launch.h"

namespace pkv {

// One wave per (token, kv head); the row layout is TokenRow's.
template <int SRC, int KVT, int BS, int D>
__global__ __launch_bounds__(64) void reshape_and_cache_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int32_t num_kv_heads,
    int64_t num_slots, float k_inv, float v_inv) {
    const int t = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t src = ((int64_t)t * num_kv_heads + g) * D;
    TokenRow<D> row;
    row.load(key + src, value + src, lane);
    row.template store<SRC, KVT, BS>(k_cache, v_cache, slot, num_kv_heads, g, lane, k_inv, v_inv);
}

// slot of the newest token (position c-1) of every sequence.
__global__ __launch_bounds__(256) void decode_slot_mapping_kernel(
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t block_size,
    int32_t* __restrict__ slot_mapping) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= num_seqs) return;
    const int c = context_lens[s];
    if (c <= 0 || (int64_t)c > (int64_t)max_blocks * block_size) {
        slot_mapping[s] = -1;
        return;
    }
    const int pos = c - 1;
    const int32_t pb = block_tables[(int64_t)s * max_blocks + pos / block_size];
    slot_mapping[s] = pb * block_size + pos % block_size;
}

// Count table entries a decode would read that are outside [1, num_blocks),
// and context lengths outside [0, max_blocks * block_size].
__global__ __launch_bounds__(256) void check_tables_kernel(
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t block_size, int32_t num_blocks,
    int32_t* __restrict__ bad) {
    const int s = blockIdx.y;
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    const int c = context_lens[s];
    int nbad = 0;
    if (j == 0 && (c < 0 || (int64_t)c > (int64_t)max_blocks * block_size)) nbad++;
    const int cc = c < 0 ? 0 : (c > max_blocks * block_size ? max_blocks * block_size : c);
    const int nblk = (cc + block_size - 1) / block_size;
    if (j < nblk) {
        const int32_t id = block_tables[(int64_t)s * max_blocks + j];
        if (id < 1 || id >= num_blocks) nbad++;
    }
    if (nbad) atomicAdd(bad, nbad);
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = 0;
}

// Fill n 16-bit (or n 8-bit when pattern_bytes == 1) elements with a pattern.
__global__ __launch_bounds__(256) void fill_pattern_kernel(uint8_t* __restrict__ p, int64_t n_bytes,
                                                           uint32_t pattern, int pattern_bytes) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_bytes) return;
    const int byte_in = (int)(i % pattern_bytes);
    p[i] = (uint8_t)(pattern >> (8 * byte_in));
}

// ----------------------------------------------------------------- launch --

template <int SRC, int KVT, int BS, int D>
static hipError_t launch_rac(const RacArgs& a, hipStream_t st) {
    dim3 grid(a.num_tokens, a.num_kv_heads);
    hipLaunchKernelGGL((reshape_and_cache_kernel<SRC, KVT, BS, D>), grid, dim3(64), 0, st,
                       (const uint16_t*)a.key, (const uint16_t*)a.value, (uint8_t*)a.k_cache,
                       (uint8_t*)a.v_cache, a.slot_mapping, a.num_kv_heads,
                       (int64_t)a.num_blocks * BS, a.k_inv, a.v_inv);
    return hipGetLastError();
}

template <int SRC, int KVT, int D>
static hipError_t launch_rac_d(const RacArgs& a, hipStream_t st) {
    return a.block_size == 16 ? launch_rac<SRC, KVT, 16, D>(a, st) : launch_rac<SRC, KVT, 32, D>(a, st);
}

template <int SRC, int KVT>
static hipError_t launch_rac_bs(const RacArgs& a, hipStream_t st) {
    if (a.head_dim == 64) return launch_rac_d<SRC, KVT, 64>(a, st);
    if (a.head_dim == 256) return launch_rac_d<SRC, KVT, 256>(a, st);
    return launch_rac_d<SRC, KVT, 128>(a, st);
}

hipError_t launch_reshape_and_cache(const RacArgs& a, hipStream_t st) {
    if (a.num_tokens == 0) return hipSuccess;
    if (a.src_dtype == DT_BF16) {
        if (a.kv_dtype == DT_BF16) return launch_rac_bs<DT_BF16, DT_BF16>(a, st);
        return launch_rac_bs<DT_BF16, DT_FP8>(a, st);
    }
    if (a.kv_dtype == DT_FP16) return launch_rac_bs<DT_FP16, DT_FP16>(a, st);
    return launch_rac_bs<DT_FP16, DT_FP8>(a, st);
}

hipError_t launch_decode_slot_mapping(const int32_t* bt, int32_t max_blocks, const int32_t* ctx,
                                      int32_t num_seqs, int32_t bs, int32_t* slots,
                                      hipStream_t st) {
    if (num_seqs == 0) return hipSuccess;
    hipLaunchKernelGGL(decode_slot_mapping_kernel, dim3((num_seqs + 255) / 256), dim3(256), 0, st,
                       bt, max_blocks, ctx, num_seqs, bs, slots);
    return hipGetLastError();
}

hipError_t launch_check_tables(const int32_t* bt, int32_t max_blocks, const int32_t* ctx,
                               int32_t num_seqs, int32_t bs, int32_t num_blocks, int32_t* bad,
                               hipStream_t st) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, st, bad);
    if (num_seqs > 0 && max_blocks > 0) {
        dim3 grid((max_blocks + 255) / 256, num_seqs);
        hipLaunchKernelGGL(check_tables_kernel, grid, dim3(256), 0, st, bt, max_blocks, ctx, bs,
                           num_blocks, bad);
    }
    return hipGetLastError();
}

// Read-stream probe (measurement aid, no part of the attention path): the
// HBM read rate a plain stream reaches on this device, the figure the
// decode kernel's K / V stream is compared against.  Workgroup g reads the
// 16-byte words [g * per, min((g + 1) * per, n)) of one contiguous slice,
// four non-temporal loads in flight per lane, and XORs them into one word
// per thread (so every word is read exactly once and the XOR of the sink is
// the XOR of the source).  Two workgroups per CU of 256 threads measured
// best: 6.9 TB/s over 2.5 GB, against 6.0-6.2 TB/s with cache-allocating
// loads or a grid-stride walk.
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* __restrict__ src, int64_t n,
                                                                   int64_t per, u32x4_t* __restrict__ sink) {
    u32x4_t acc = {0u, 0u, 0u, 0u};
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n ? b0 + per : n;
    int64_t i = b0 + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < b1; i += kProbeUnroll * kProbeThreads) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
    }
    for (; i < b1; i += kProbeThreads) acc ^= __builtin_nontemporal_load(src + i);
    sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

int read_probe_groups() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return 2 * cus;
}

int64_t read_probe_sink_bytes() { return (int64_t)read_probe_groups() * kProbeThreads * 16; }

hipError_t launch_read_probe(const void* src, int64_t n16, void* sink, hipStream_t st) {
    if (n16 <= 0) return hipSuccess;
    const int groups = read_probe_groups();
    const int64_t per = (n16 + groups - 1) / groups;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)groups), dim3(kProbeThreads), 0, st,
                       (const u32x4_t*)src, n16, per, (u32x4_t*)sink);
    return hipGetLastError();
}

hipError_t launch_fill_pattern(void* p, int64_t n_bytes, uint32_t pattern, int pattern_bytes,
                               hipStream_t st) {
    if (n_bytes <= 0) return hipSuccess;
    const int64_t blocks = (n_bytes + 255) / 256;
    hipLaunchKernelGGL(fill_pattern_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       (uint8_t*)p, n_bytes, pattern, pattern_bytes);
    return hipGetLastError();
}

}  // namespace pkv
