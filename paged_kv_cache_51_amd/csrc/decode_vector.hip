// decode_vector.hip — the partition kernel with its per-unit math on the
// vector ALU instead of the matrix cores: same pool layout, same register
// fragments, same work plan, ring and merge (decode_core.h), same
// arithmetic order within a unit up to the summation order of the logits.
// It exists to measure what the matrix cores buy on an HBM-bound decode.
#include "decode_core.h"

namespace pkv {

// Groups of up to 8 query heads per kv head.  Lane l holds token l & 15 and
// dims 8*((l>>4) + 4kk)..+7 of a unit's K (the MFMA A-operand order), so a
// head's logit is 16 dot2 per lane plus a sum over the four 16-lane rows,
// which leaves every row with all 16 logits.  The weights then move to the
// V order (tokens 4*(l>>4)..+3 of dim 16nt + (l & 15)) with two lane reads
// per head, and PV is 16 dot2 per head.  The queries sit in LDS and are read
// as broadcasts, which leaves the registers to 8 heads of accumulators.  The
// running max m is the same in every lane; l (per token lane) and the
// partial outputs (per row) are reduced over lanes when parked.
template <int KVT, int QT>
struct VectorMath {
    static constexpr int kMaxGroup = 8;
    static constexpr int kCols = 16;
    static constexpr int kD = kHeadDim;       // built for head_dim 128
    __host__ __device__ static constexpr int query_lds_floats(int g) { return g * kHeadDim / 2; }

    float acc[kMaxGroup][8];  // dim 16nt + (lane & 15), over this row's tokens
    float m[kMaxGroup], l[kMaxGroup];
    u32x4_t qreg;             // this thread's 16-byte share of the group's queries
    const u32x4_t* qlds;      // [head][16] chunks of 8 dims
    int G;

    // decode only: one query token per entry (columns = the G heads)
    __device__ __forceinline__ void load_q(const DecodeArgs& a, const QueryTile& qt, int kvh, int) {
        G = a.group;
        const int tid = threadIdx.x;
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.q) +
                             (qt.row0 * a.num_heads + (int64_t)first_head(a, kvh)) * (kHeadDim / 8);
        const u32x4_t z = {0u, 0u, 0u, 0u};
        qreg = tid < G * (kHeadDim / 8) ? src[tid] : z;
    }
    // one token at the end of the context: it sees every key (unit() masks
    // at the context length)
    __device__ __forceinline__ void limit(int, int, int) {}
    __device__ __forceinline__ void stage_q(float* lds, int tid) {
        u32x4_t* q = reinterpret_cast<u32x4_t*>(lds);
        if (tid < G * (kHeadDim / 8)) q[tid] = qreg;
        qlds = q;
    }

    __device__ __forceinline__ void begin() {
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.f;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[h][nt] = 0.f;
        }
    }

    __device__ __forceinline__ void unit(const UnitRegs<KVT>& u, int tok0, int ctx, float cs, int lane) {
        const int row = lane >> 4;
        const bool valid = tok0 + (lane & 15) < ctx;
        u32x4_t kf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kf[kk] = k_frag<KVT, QT>(u, kk);
        float t[kMaxGroup], bm[kMaxGroup];
        bool jump = false;
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            if (h < G) {
                float d = 0.f;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const u32x4_t q4 = qlds[h * (kHeadDim / 8) + row + 4 * kk];
#pragma unroll
                    for (int j = 0; j < 4; ++j) d = dot2<QT>(kf[kk][j], q4[j], d);
                }
                d += xor_shfl(d, 16);
                d += xor_shfl(d, 32);
                t[h] = valid ? d * cs : -INFINITY;
                float b = t[h];
                b = fmaxf(b, xor_shfl(b, 1));
                b = fmaxf(b, xor_shfl(b, 2));
                b = fmaxf(b, xor_shfl(b, 4));
                b = fmaxf(b, xor_shfl(b, 8));   // unit max: finite, the unit holds a valid token
                bm[h] = b;
                jump |= b > m[h] + kRescaleSlack;
            }
        }
        if (__builtin_amdgcn_ballot_w64(jump)) {
            // Some head's max jumped: move every head's reference to its max.
#pragma unroll
            for (int h = 0; h < kMaxGroup; ++h) {
                if (h < G) {
                    const float mn = fmaxf(m[h], bm[h]);
                    const float alpha = (m[h] == -INFINITY) ? 0.f : fast_exp2(m[h] - mn);
                    l[h] *= alpha;
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) acc[h][nt] *= alpha;
                    m[h] = mn;
                }
            }
        }
        u32x2_t vf[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) vf[nt] = v_frag<KVT, QT>(u, nt);
        if (tok0 + kSubTokens > ctx) {
            // Last unit of the context: zero V rows past it (0 x NaN = NaN).
            const int tb = tok0 + 4 * row;
            u32x2_t vm;
            vm[0] = (tb + 0 < ctx ? 0x0000ffffu : 0u) | (tb + 1 < ctx ? 0xffff0000u : 0u);
            vm[1] = (tb + 2 < ctx ? 0x0000ffffu : 0u) | (tb + 3 < ctx ? 0xffff0000u : 0u);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) vf[nt] &= vm;
        }
        const int src = 4 * row;   // lane holding token 4*row (rows are copies)
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            if (h < G) {
                const float p = valid ? fast_exp2(t[h] - m[h]) : 0.f;
                const uint32_t pb = f32_to_bits<QT>(p);
                l[h] += bits_to_f32<QT>(pb);    // normalise with the rounded weights
                // even token lanes hold the pair (t, t+1), low half first
                const uint32_t pair = pb | (lane_fetch(pb, lane ^ 1) << 16);
                const uint32_t p01 = lane_fetch(pair, src);
                const uint32_t p23 = lane_fetch(pair, src + 2);
#pragma unroll
                for (int nt = 0; nt < 8; ++nt)
                    acc[h][nt] = dot2<QT>(vf[nt][1], p23, dot2<QT>(vf[nt][0], p01, acc[h][nt]));
            }
        }
    }

    __device__ __forceinline__ void park(float* sm_m, float* sm_l, float* sm_acc, int w, int,
                                         int lane) {
        const int row = lane >> 4, c = lane & 15;
        float mv = -INFINITY, lv = 0.f;
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
            if (h < G) {
                float x = l[h];          // the 16 tokens of a row (the rows are copies)
                x += xor_shfl(x, 1);
                x += xor_shfl(x, 2);
                x += xor_shfl(x, 4);
                x += xor_shfl(x, 8);
                if (c == h) {
                    mv = m[h];
                    lv = x;
                }
                float* dst = sm_acc + (w * G + h) * kMergeRow + c;
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    float y = acc[h][nt];
                    y += xor_shfl(y, 16);
                    y += xor_shfl(y, 32);
                    if ((nt >> 1) == row) dst[16 * nt] = y;   // row r stores tiles 2r, 2r+1
                }
            }
        }
        if (lane < 16) {
            sm_m[w * 16 + lane] = mv;
            sm_l[w * 16 + lane] = lv;
        }
    }
};

template <int KVT, int QT, int BS, int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU)))
void paged_decode_vector_kernel(const DecodeArgs a) {
    extern __shared__ float pkv_smem[];
    grid_entry<VectorMath<KVT, QT>, KVT, QT, BS, NW, DEPTH>(a, pkv_smem);
}

template <int KVT, int QT, int BS>
static hipError_t launch_vector(const DecodeArgs& a, hipStream_t st) {
    if (a.group > VectorMath<KVT, QT>::kMaxGroup) return hipErrorNotSupported;
    const size_t lds = sizeof(float) * (merge_lds_floats(kWavesPerGroup, a.group) +
                                        VectorMath<KVT, QT>::query_lds_floats(a.group));
    const dim3 grid((unsigned)grid_workgroups(a));
    hipLaunchKernelGGL((paged_decode_vector_kernel<KVT, QT, BS, kWavesPerGroup, kDepth>), grid,
                       dim3(kWavesPerGroup * kWave), lds, st, a);
    return hipGetLastError();
}

template <int KVT, int QT>
static hipError_t launch_vector_bs(const DecodeArgs& a, int bs, hipStream_t st) {
    return bs == 16 ? launch_vector<KVT, QT, 16>(a, st) : launch_vector<KVT, QT, 32>(a, st);
}

hipError_t launch_decode_vector(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                                hipStream_t st) {
    if (q_dtype == DT_BF16) {
        if (kv_dtype == DT_BF16) return launch_vector_bs<DT_BF16, DT_BF16>(a, block_size, st);
        return launch_vector_bs<DT_FP8, DT_BF16>(a, block_size, st);
    }
    if (kv_dtype == DT_FP16) return launch_vector_bs<DT_FP16, DT_FP16>(a, block_size, st);
    return launch_vector_bs<DT_FP8, DT_FP16>(a, block_size, st);
}

}  // namespace pkv
