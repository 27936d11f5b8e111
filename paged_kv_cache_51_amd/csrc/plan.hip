// plan.hip — work plan for the partition kernel: which (sequence,
// partition) each workgroup decodes, longest first.
//
// Workgroups are dispatched in launch order to whichever CU frees up first,
// so ordering the work items by decreasing size makes the dispatcher run a
// longest-processing-time-first schedule: the short items fill in at the
// end instead of a long one starting last.  Each item is expanded over the
// kv heads with the head fastest, so the heads of one item land on
// consecutive XCDs (workgroups go to the 8 XCDs round-robin).
//
// Plan layout (int32): [0] item count, [1] next work entry and [2] finished
// workgroups of the persistent decode (zeroed here, reset by the last
// workgroup of each launch), [3] reserved, [4 + i] item i as
// (sequence << 16) | partition.  Built by one workgroup with a counting sort
// on the item size in 16-token units (sizes above kMaxBucket share the top
// bucket).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kPlanThreads = 1024;
constexpr int kMaxBucket = 4095;

__device__ __forceinline__ int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ context_lens,
                                                           int32_t num_seqs, int32_t ctx_cap,
                                                           int32_t block_size, int32_t part_blocks,
                                                           int32_t* __restrict__ plan) {
    constexpr int kWaves = kPlanThreads / kWave;
    __shared__ int hist[kMaxBucket + 1];
    __shared__ int wave_total[kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    const int part_units = part_blocks * (block_size / kSubTokens);
    const int nbucket = min(part_units, kMaxBucket) + 1;
    // The length of this thread's first sequence, read once for both passes
    // below (every sequence, when there are at most kPlanThreads of them).
    const int c_first = tid < num_seqs ? context_lens[tid] : 0;
    for (int b = tid; b < nbucket; b += kPlanThreads) hist[b] = 0;
    __syncthreads();

    // Item (s, p) covers units [p*part_units, min((p+1)*part_units, n_units));
    // a sequence with no context still gets one (empty) item so that its
    // output is written (zeros).
    auto items_of = [&](int s, int& n_units) {
        const int c = clamp_ctx(s == tid ? c_first : context_lens[s], ctx_cap);
        n_units = (c + kSubTokens - 1) / kSubTokens;
        const int nblk = (c + block_size - 1) / block_size;
        return c <= 0 ? 1 : (nblk + part_blocks - 1) / part_blocks;
    };
    auto bucket_of = [&](int n_units, int p) {
        const int sz = min(part_units, n_units - p * part_units);
        return min(max(sz, 0), kMaxBucket);
    };

    for (int s = tid; s < num_seqs; s += kPlanThreads) {
        int n_units;
        const int P = items_of(s, n_units);
        for (int p = 0; p < P; ++p) atomicAdd(&hist[bucket_of(n_units, p)], 1);
    }
    __syncthreads();

    // Exclusive scan over buckets in decreasing size: bucket b's first slot
    // is the number of items larger than b.  Thread t owns a contiguous run
    // of buckets taken from the top; the runs' sums are scanned in thread
    // order by shuffles within each wave and the waves' totals in LDS.
    const int per = (nbucket + kPlanThreads - 1) / kPlanThreads;
    int local = 0;
    for (int j = 0; j < per; ++j) {
        const int b = nbucket - 1 - (tid * per + j);
        if (b >= 0) local += hist[b];
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    if (lane == kWave - 1) wave_total[wid] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int t = wave_total[w];
        before += w < wid ? t : 0;
        total += t;
    }
    int run = before + incl - local;          // exclusive prefix of this thread's run
    for (int j = 0; j < per; ++j) {
        const int b = nbucket - 1 - (tid * per + j);
        if (b >= 0) {
            const int cnt = hist[b];
            hist[b] = run;                    // becomes the bucket's next free slot
            run += cnt;
        }
    }
    if (tid == 0) {
        plan[0] = total;
        plan[1] = 0;   // persistent decode: next entry to claim
        plan[2] = 0;   // persistent decode: workgroups finished
        plan[3] = 0;
    }
    __syncthreads();

    for (int s = tid; s < num_seqs; s += kPlanThreads) {
        int n_units;
        const int P = items_of(s, n_units);
        for (int p = 0; p < P; ++p) {
            const int pos = atomicAdd(&hist[bucket_of(n_units, p)], 1);
            plan[4 + pos] = (s << 16) | p;
        }
    }
}

hipError_t launch_plan(const int32_t* context_lens, int32_t num_seqs, int32_t ctx_cap,
                       int32_t block_size, int32_t part_blocks, int32_t* plan, hipStream_t st) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, context_lens, num_seqs,
                       ctx_cap, block_size, part_blocks, plan);
    return hipGetLastError();
}

}  // namespace pkv
