// decode.hip — PagedAttention decode on gfx950 matrix cores, plus the
// split-context merge.
//
// What is computed ("LLM inference basics and vLLM internals" §4 and "vLLM
// internals (2)", "Block table"): for each sequence, its one new query token
// attends over all c context tokens, whose K/V rows are found by looking up
// the physical block of logical block t / block_size in the request's block
// table.  GQA ("LLM inference basics..." §2): the G query heads of a group
// share one K/V head, so one pass over a K/V tile serves all G of them.
//
// Work decomposition (one workgroup of NW waves per (sequence, kv head,
// partition) from the work plan of plan.hip):
//   - a partition is part_blocks consecutive logical blocks; the workgroup
//     walks its 16-token sub-tiles ("units"), wave w taking units w, w+NW, ...
//   - per unit a wave loads the K and V sub-tiles (4 + 4 rows of 1 KiB for
//     16-bit KV, 2 + 2 for fp8) straight into registers: the pool stores them
//     in MFMA operand order, so no LDS staging and no shuffles are needed;
//   - S^T = K . Q^T on four 16x16x32 MFMAs (rows = 16 tokens, columns = the
//     G query heads padded to 16), online softmax in fp32 in the log2 domain,
//     then O^T += V^T . P^T on eight 16x16x16 MFMAs whose B operand is the
//     S^T result in place (same lane order);
//   - the next DEPTH-1 units' loads are in flight while a unit is computed
//     (a ring of register sets);
//   - waves park their partial results in LDS and the last wave to finish
//     merges them (no barrier wait); a sequence that fits one partition gets
//     its output directly, otherwise (max, normaliser, normalised output) per
//     partition go to the workspace for decode_reduce_kernel.
#include "decode_core.h"
#include "mfma_math.h"

#include <algorithm>

namespace pkv {

// Grid form (see grid_entry).  D = head_dim; PLAIN: cache-allocating K / V
// loads (load_unit), for kv heads split over several entry heads; NT: 16-
// column MFMA tiles per entry (2 for entries of 17-32 query heads).
template <int KVT, int QT, int BS, int NW, int DEPTH, int D = kHeadDim, bool PLAIN = false, int NT = 1>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU)))
void paged_decode_mfma_kernel(const DecodeArgs a) {
    extern __shared__ float pkv_smem[];
    grid_entry<MfmaMath<KVT, QT, NT, D>, KVT, QT, BS, NW, DEPTH, PLAIN>(a, pkv_smem);
}

// Persistent form: as many workgroups as fit on the GPU at once, each
// claiming the next work entry of the longest-first plan from an atomic
// counter until the plan is exhausted.  CUs (and XCDs) that run faster
// simply take more entries.  The counters live in the plan header
// (zeroed by the planner); the last workgroup to leave resets them, so
// the plan can serve the next launch on the same stream.
template <int KVT, int QT, int BS, int NW, int DEPTH, int D = kHeadDim, bool PLAIN = false, int NT = 1>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU)))
void paged_decode_mfma_persistent(const DecodeArgs a) {
    extern __shared__ float pkv_smem[];
    int* sm_entry = reinterpret_cast<int*>(pkv_smem) + 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int32_t* counters = const_cast<int32_t*>(a.plan) + 1;   // [0] next entry, [1] workgroups done
    const int total = a.plan[0] * a.num_kv_heads;
    for (;;) {
        if (threadIdx.x == 0) *sm_entry = atomicAdd(&counters[0], 1);
        __syncthreads();
        const int k = __builtin_amdgcn_readfirstlane(*sm_entry);
        __syncthreads();
        if (k >= total) break;
        const int item = k / a.num_kv_heads;
        const int kvh = k - item * a.num_kv_heads;
        const uint32_t packed = (uint32_t)a.plan[kPlanHeader + item];
        const int s = (int)(packed >> 16);
        decode_entry<MfmaMath<KVT, QT, NT, D>, KVT, QT, BS, NW, DEPTH, PLAIN>(a, pkv_smem, s, (int)(packed & 0xffffu),
                                                                               kvh, lane, w, QueryTile{s, 1, 1});
    }
    if (threadIdx.x == 0) {
        __threadfence();
        if (atomicAdd(&counters[1], 1) == (int)gridDim.x - 1) {
            atomicExch(&counters[0], 0);
            atomicExch(&counters[1], 0);
        }
    }
}

// Merge the partitions of every multi-partition sequence: with per-partition
// max m_p (log2 units), normaliser l_p and normalised output o_p,
//   out = sum_p 2^(m_p - M) l_p o_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// One wave per (query head, sequence); lane owns dims e, e + 1 for
// e = 2 lane + 128 i (D = head_dim).  Partitions are summed in order p = 0,
// 1, ... in chunks of kReduceChunk whose records are loaded together; the
// first chunk's loads are issued with the pass that forms M (they do not
// depend on it), so a launch of at most kReduceChunk partitions per sequence
// waits for one memory round trip after the context length.
constexpr int kReduceChunk = 8;
template <int QT, int BS, int D = kHeadDim>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(const DecodeArgs a) {
    const int hq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
    int ctx = a.context_lens[s];
    ctx = ctx < a.ctx_cap ? ctx : a.ctx_cap;
    if (ctx <= 0) return;
    const int nblk = (ctx + BS - 1) / BS;
    const int np = (nblk + a.part_blocks - 1) / a.part_blocks;
    if (np <= 1) return;
    // query head hq -> its entry head kvh and column h in that entry
    const int G = a.group, ph = hq / a.group_all, r = hq - ph * a.group_all;
    const int cg = r / G, h = r - cg * G, kvh = ph * a.kv_split + cg;
    const int64_t base = ((int64_t)s * a.num_kv_heads + kvh) * a.num_parts;
    const int ML = ml_line(G);
    constexpr int NE = (D + 2 * kWave - 1) / (2 * kWave);   // dim pairs per lane
    // one chunk of records: maxima, normalisers and this lane's output dims
    // (indices clamped to the last partition; entries past it are not summed)
    float cm[kReduceChunk], cl[kReduceChunk];
    float2 co[kReduceChunk][NE];
    auto load_chunk = [&](int p0) {
#pragma unroll
        for (int j = 0; j < kReduceChunk; ++j) {
            const int64_t rec = base + min(p0 + j, np - 1);
            cm[j] = a.ws_ml[rec * ML + h];
            cl[j] = a.ws_ml[rec * ML + ML / 2 + h];
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int e = min(2 * lane + 2 * kWave * i, D - 2);
                co[j][i] = *reinterpret_cast<const float2*>(a.ws_out + (rec * G + h) * D + e);
            }
        }
    };
    load_chunk(0);
    float M = -INFINITY;
    for (int p = lane; p < np; p += kWave) M = fmaxf(M, a.ws_ml[(base + p) * ML + h]);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) M = fmaxf(M, xor_shfl(M, d));
    float L = 0.f, o0[NE], o1[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) o0[i] = o1[i] = 0.f;
    for (int p0 = 0; p0 < np; p0 += kReduceChunk) {
        if (p0 > 0) load_chunk(p0);
#pragma unroll
        for (int j = 0; j < kReduceChunk; ++j) {
            if (p0 + j < np) {
                const float fct = fast_exp2(cm[j] - M) * cl[j];
                L += fct;
#pragma unroll
                for (int i = 0; i < NE; ++i) {
                    o0[i] += fct * co[j][i].x;
                    o1[i] += fct * co[j][i].y;
                }
            }
        }
    }
    const float sc = a.out_scale / L;
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)s * a.num_heads + hq) * D;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int e = 2 * lane + 2 * kWave * i;
        if (e < D)
            *reinterpret_cast<uint32_t*>(out + e) =
                (uint32_t)f32_to_bits<QT>(o0[i] * sc) | ((uint32_t)f32_to_bits<QT>(o1[i] * sc) << 16);
    }
}

// ----------------------------------------------------------------- launch --

// Waves per workgroup and units in flight per wave of the partition kernel.
// 16-bit pools: eight waves, so a workgroup streams its item twice as fast
// and the end of a launch, when few items are left, is shorter (7B shape
// 381.9 -> 378.5 us, Llama MHA 722.6 -> 712.4 us per layer, interleaved in
// one process), as long as partitions are long (>= 2048 tokens: with the
// 512-token partitions of a small batch, 1.5B shape, eight waves were 10 %
// slower, each wave holding only a few units), the eight waves' merge area
// stays within 64 KiB of LDS and head_dim <= 128; fp8 pools: four waves with
// one unit in flight (72B fp8 334.8 -> 329.6 us; eight waves were 0.6 %
// slower there).
template <int KVT, int QT, int BS, int D, int NW, int DEPTH, bool PLAIN, int NT = 1>
static hipError_t launch_mfma_nw_t(const DecodeArgs& a, bool persistent, hipStream_t st) {
    const size_t lds = sizeof(float) * merge_lds_floats(NW, a.group, 16 * NT, D);
    const dim3 block(NW * kWave);
    if (!persistent) {
        const dim3 grid((unsigned)grid_workgroups(a));
        hipLaunchKernelGGL((paged_decode_mfma_kernel<KVT, QT, BS, NW, DEPTH, D, PLAIN, NT>), grid, block, lds, st, a);
        return hipGetLastError();
    }
    // as many workgroups as can be resident at once (never more than entries)
    static int per_cu[16 * NT + 1] = {};      // cache by group size (LDS use)
    int& occ = per_cu[a.group];
    if (!occ) {
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ, reinterpret_cast<const void*>(&paged_decode_mfma_persistent<KVT, QT, BS, NW, DEPTH, D, PLAIN, NT>),
            block.x, lds);
        if (e != hipSuccess || occ <= 0) occ = 1;
    }
    int dev = 0, cus = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t entries = (int64_t)a.num_seqs * a.num_kv_heads * a.num_parts;
    const dim3 grid((unsigned)std::min<int64_t>(entries, (int64_t)occ * cus));
    hipLaunchKernelGGL((paged_decode_mfma_persistent<KVT, QT, BS, NW, DEPTH, D, PLAIN, NT>), grid, block, lds, st, a);
    return hipGetLastError();
}

// Cache-allocating K / V loads when a kv head is read by several entry
// heads (more than 16 query heads per kv head), non-temporal ones otherwise.
template <int KVT, int QT, int BS, int D, int NW, int DEPTH>
static hipError_t launch_mfma_nw(const DecodeArgs& a, bool persistent, hipStream_t st) {
    return a.kv_split > 1 ? launch_mfma_nw_t<KVT, QT, BS, D, NW, DEPTH, true>(a, persistent, st)
                          : launch_mfma_nw_t<KVT, QT, BS, D, NW, DEPTH, false>(a, persistent, st);
}

// four_waves: the four-wave form whatever the workload (PKV_IMPL_MFMA), the
// one whose results the multi-token and token-table kernels, which run the
// same per-wave code with four waves, reproduce bit for bit.
template <int KVT, int QT, int BS, int D>
static hipError_t launch_mfma(const DecodeArgs& a, bool persistent, bool four_waves, hipStream_t st) {
    constexpr int NW8 = 2 * kWavesPerGroup;
    constexpr int DP = KVT == DT_FP8 ? 1 : kDepth;
    if constexpr (D <= 128) {
        // Entries of 17-32 query heads (MQA, wide GQA groups): two MFMA
        // tiles per wave over one read of the K / V, four waves, one unit in
        // flight (217 VGPRs, two waves per SIMD; with two units in flight
        // 265, one wave per SIMD).  One kv head, 256 sequences of 1K-8K
        // tokens, against 16-column entries sharing the K / V in L2:
        // 24 heads 172 -> 131 us, 32 heads 142 -> 143 us, 48 heads 171 ->
        // 162 us, 64 heads 199 -> 179 us, 96 heads 254 -> 224 us.
        if (a.group > 16)
            return a.kv_split > 1 ? launch_mfma_nw_t<KVT, QT, BS, D, kWavesPerGroup, 1, true, 2>(a, persistent, st)
                                  : launch_mfma_nw_t<KVT, QT, BS, D, kWavesPerGroup, 1, false, 2>(a, persistent, st);
    }
    if (four_waves) return launch_mfma_nw<KVT, QT, BS, D, kWavesPerGroup, DP>(a, persistent, st);
    if constexpr (KVT == DT_FP8) {
        return launch_mfma_nw<KVT, QT, BS, D, kWavesPerGroup, 1>(a, persistent, st);
    } else if constexpr (D <= 128) {
        if ((int64_t)a.part_blocks * BS >= 2048 && sizeof(float) * merge_lds_floats(NW8, a.group, 16, D) <= 65536)
            return launch_mfma_nw<KVT, QT, BS, D, NW8, kDepth>(a, persistent, st);
        return launch_mfma_nw<KVT, QT, BS, D, kWavesPerGroup, kDepth>(a, persistent, st);
    } else {
        // head_dim 256: eight waves would spill (256 VGPRs at most)
        return launch_mfma_nw<KVT, QT, BS, D, kWavesPerGroup, kDepth>(a, persistent, st);
    }
}

template <int KVT, int QT, int D>
static hipError_t launch_mfma_d(const DecodeArgs& a, int bs, bool persistent, bool four, hipStream_t st) {
    return bs == 16 ? launch_mfma<KVT, QT, 16, D>(a, persistent, four, st)
                    : launch_mfma<KVT, QT, 32, D>(a, persistent, four, st);
}

template <int KVT, int QT>
static hipError_t launch_mfma_bs(const DecodeArgs& a, int bs, bool persistent, bool four, hipStream_t st) {
    if (a.head_dim == 64) return launch_mfma_d<KVT, QT, 64>(a, bs, persistent, four, st);
    if (a.head_dim == 256) return launch_mfma_d<KVT, QT, 256>(a, bs, persistent, four, st);
    return launch_mfma_d<KVT, QT, 128>(a, bs, persistent, four, st);
}

hipError_t launch_decode_vector(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                                hipStream_t st);

hipError_t launch_decode_partitions(const DecodeArgs& a, int q_dtype, int kv_dtype,
                                    int block_size, int impl, hipStream_t st) {
    if (a.num_seqs == 0 || a.num_parts == 0) return hipSuccess;
    if (impl == 2) return launch_decode_vector(a, q_dtype, kv_dtype, block_size, st);
    const bool persistent = impl == 3;
    const bool four = impl == 1;
    if (q_dtype == DT_BF16) {
        if (kv_dtype == DT_BF16) return launch_mfma_bs<DT_BF16, DT_BF16>(a, block_size, persistent, four, st);
        return launch_mfma_bs<DT_FP8, DT_BF16>(a, block_size, persistent, four, st);
    }
    if (kv_dtype == DT_FP16) return launch_mfma_bs<DT_FP16, DT_FP16>(a, block_size, persistent, four, st);
    return launch_mfma_bs<DT_FP8, DT_FP16>(a, block_size, persistent, four, st);
}

template <int QT, int D>
static void launch_reduce_t(const DecodeArgs& a, int block_size, dim3 grid, hipStream_t st) {
    if (block_size == 16)
        hipLaunchKernelGGL((decode_reduce_kernel<QT, 16, D>), grid, dim3(kWave), 0, st, a);
    else
        hipLaunchKernelGGL((decode_reduce_kernel<QT, 32, D>), grid, dim3(kWave), 0, st, a);
}

template <int QT>
static void launch_reduce_q(const DecodeArgs& a, int block_size, dim3 grid, hipStream_t st) {
    if (a.head_dim == 64) launch_reduce_t<QT, 64>(a, block_size, grid, st);
    else if (a.head_dim == 256) launch_reduce_t<QT, 256>(a, block_size, grid, st);
    else launch_reduce_t<QT, 128>(a, block_size, grid, st);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, int q_dtype, int block_size,
                                hipStream_t st) {
    if (a.num_seqs == 0 || a.num_parts <= 1) return hipSuccess;
    dim3 grid(a.num_heads, a.num_seqs);
    if (q_dtype == DT_BF16) launch_reduce_q<DT_BF16>(a, block_size, grid, st);
    else launch_reduce_q<DT_FP16>(a, block_size, grid, st);
    return hipGetLastError();
}

}  // namespace pkv
