// prefill.hip — multi-token paged attention on gfx950 matrix cores: the
// new tokens of a chunk (chunked prefill, or the suffix after a prefix-cache
// hit) attend causally to their sequence's paged context.
//
// What is computed ("LLM inference basics and vLLM internals" §5, prefix
// cache, and §6, chunked prefill; the block-table lookup of §4): token j of a
// chunk of q_len new tokens sits at position ctx - q_len + j and sees keys
// 0..ctx - q_len + j, read through the block table exactly as in decode.
// The per-unit arithmetic is the decode kernel's (decode_core.h,
// mfma_math.h) with the query columns (token, head) pairs.
#include "decode_core.h"
#include "mfma_math.h"

namespace pkv {

// Multi-token form: workgroup (sequence s, query tile, kv head) attends the
// tile's tokens to the paged context, causally: token j of a chunk of
// q_len new tokens sits at position ctx - q_len + j and sees keys up to it.
// Tiles hold tile_tokens = 16 / G tokens (so the tile's (token, head) pairs
// fill the 16 MFMA columns), and the last tiles of a chunk, which see the
// most keys, are dispatched first.  No context split: the tiles give the
// parallelism.  With q_len = 1 a tile is exactly a decode entry.
template <int KVT, int QT, int BS, int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU)))
void paged_prefill_mfma_kernel(const DecodeArgs a, const int32_t* __restrict__ query_start,
                               int tile_tokens, int max_tiles) {
    extern __shared__ float pkv_smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kvh = blockIdx.x % a.num_kv_heads;
    const int rest = blockIdx.x / a.num_kv_heads;
    const int tile = max_tiles - 1 - rest / a.num_seqs;
    const int s = rest % a.num_seqs;
    const int q0 = query_start[s];
    const int q_len = query_start[s + 1] - q0;
    const int j0 = tile * tile_tokens;
    if (j0 >= q_len) return;
    decode_entry<MfmaMath<KVT, QT>, KVT, QT, BS, NW, DEPTH>(
        a, pkv_smem, s, 0, kvh, lane, w,
        QueryTile{(int64_t)q0 + j0, min(tile_tokens, q_len - j0), q_len - j0});
}

// Wave-per-tile form for longer chunks: workgroup (sequence s, group of NW
// query tiles, kv head); wave w takes tile NW*group + w and walks all of the
// keys it sees alone (units in order), so the NW waves read the same K / V
// units at about the same time and share them through the CU's L1 instead
// of each tile fetching them from L2.  A tile here holds 32 / G tokens (two
// 16-column MFMA tiles sharing each unit's K / V fragments).  Each wave
// merges nothing but itself, in its own LDS area.
#ifndef PKV_PREFILL_WAVES_PER_EU
#define PKV_PREFILL_WAVES_PER_EU 2
#endif

// (two waves per SIMD: the register budget is kept at 256 per lane)
template <int KVT, int QT, int BS, int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PKV_PREFILL_WAVES_PER_EU)))
void paged_prefill_wave_kernel(const DecodeArgs a, const int32_t* __restrict__ query_start,
                               int tile_tokens, int max_groups, int lds_per_wave) {
    extern __shared__ float pkv_smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kvh = blockIdx.x % a.num_kv_heads;
    const int rest = blockIdx.x / a.num_kv_heads;
    const int grp = max_groups - 1 - rest / a.num_seqs;
    const int s = rest % a.num_seqs;
    const int q0 = query_start[s];
    const int q_len = query_start[s + 1] - q0;
    const int j0 = (grp * NW + w) * tile_tokens;
    if (j0 >= q_len) return;
    decode_entry<MfmaMath<KVT, QT, 2>, KVT, QT, BS, 1, DEPTH>(
        a, pkv_smem + w * lds_per_wave, s, 0, kvh, lane, 0,
        QueryTile{(int64_t)q0 + j0, min(tile_tokens, q_len - j0), q_len - j0});
}

#ifndef PKV_PREFILL_DEPTH
#define PKV_PREFILL_DEPTH 2
#endif

template <int KVT, int QT, int BS>
static hipError_t launch_prefill_t(const DecodeArgs& a, const int32_t* query_start, int tile_tokens,
                                   int max_tiles, hipStream_t st) {
    if (max_tiles > kWavesPerGroup) {
        // two 16-column tiles per wave
        const int tt = 2 * tile_tokens;
        const int wave_tiles = (max_tiles * tile_tokens + tt - 1) / tt;
        const int per_wave = merge_lds_floats(1, tt * a.group, 32);
        const int groups = (wave_tiles + kWavesPerGroup - 1) / kWavesPerGroup;
        const size_t lds = sizeof(float) * per_wave * kWavesPerGroup;
        const dim3 grid((unsigned)((int64_t)a.num_seqs * groups * a.num_kv_heads));
        hipLaunchKernelGGL((paged_prefill_wave_kernel<KVT, QT, BS, kWavesPerGroup, PKV_PREFILL_DEPTH>), grid,
                           dim3(kWavesPerGroup * kWave), lds, st, a, query_start, tt, groups,
                           per_wave);
        return hipGetLastError();
    }
    const size_t lds = sizeof(float) * merge_lds_floats(kWavesPerGroup, tile_tokens * a.group);
    const dim3 grid((unsigned)((int64_t)a.num_seqs * max_tiles * a.num_kv_heads));
    hipLaunchKernelGGL((paged_prefill_mfma_kernel<KVT, QT, BS, kWavesPerGroup, kDepth>), grid,
                       dim3(kWavesPerGroup * kWave), lds, st, a, query_start, tile_tokens, max_tiles);
    return hipGetLastError();
}

template <int KVT, int QT>
static hipError_t launch_prefill_bs(const DecodeArgs& a, int bs, const int32_t* query_start,
                                    int tile_tokens, int max_tiles, hipStream_t st) {
    return bs == 16 ? launch_prefill_t<KVT, QT, 16>(a, query_start, tile_tokens, max_tiles, st)
                    : launch_prefill_t<KVT, QT, 32>(a, query_start, tile_tokens, max_tiles, st);
}

hipError_t launch_prefill(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                          const int32_t* query_start, int tile_tokens, int max_tiles,
                          hipStream_t st) {
    if (a.num_seqs == 0 || max_tiles == 0) return hipSuccess;
    if (q_dtype == DT_BF16) {
        if (kv_dtype == DT_BF16)
            return launch_prefill_bs<DT_BF16, DT_BF16>(a, block_size, query_start, tile_tokens, max_tiles, st);
        return launch_prefill_bs<DT_FP8, DT_BF16>(a, block_size, query_start, tile_tokens, max_tiles, st);
    }
    if (kv_dtype == DT_FP16)
        return launch_prefill_bs<DT_FP16, DT_FP16>(a, block_size, query_start, tile_tokens, max_tiles, st);
    return launch_prefill_bs<DT_FP8, DT_FP16>(a, block_size, query_start, tile_tokens, max_tiles, st);
}

}  // namespace pkv
