// mfma_math.h — the matrix-core per-unit math of the partition kernels
// (the policy decode_core.h's entry bodies call): logits, online softmax
// and PV for one 16-token unit, and the park into the merge area.
#pragma once
#include "decode_core.h"

namespace pkv {

// MFMA policy: S^T = K . Q^T on four 16x16x32 MFMAs (rows = 16 tokens,
// columns = the tile's (query token, head) pairs padded to 16; for decode
// the G heads), then O^T += V^T . P^T on eight 16x16x16 MFMAs whose B
// operand is S^T's lane order.  Lane l holds column l & 15 for the softmax
// state and rows 4*(l>>4)..+3 of each 16-row tile.
template <int KVT, int QT>
struct MfmaMath {
    static constexpr int kMaxGroup = 16;
    __host__ __device__ static constexpr int query_lds_floats(int) { return 0; }

    u32x4_t qf[4];            // Q^T fragments: 8 dims per kk of column lane & 15
    f32x4_t acc[8];
    float m, l;
    int col;                  // lane & 15: column (token col / G, head col % G)
    bool cvalid;              // the column holds a real (token, head)
    int lim;                  // the column sees keys at positions < lim

    __device__ __forceinline__ void load_q(const DecodeArgs& a, const QueryTile& qt, int kvh,
                                           int lane) {
        const int G = a.group;
        col = lane & 15;
        cvalid = col < qt.ntok * G;
        const int j = cvalid ? col / G : 0;
        const int h = cvalid ? col - j * G : 0;
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                              ((qt.row0 + j) * a.num_heads + (int64_t)kvh * G + h) * (kHeadDim * 2);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const u32x4_t z = {0u, 0u, 0u, 0u};
            qf[kk] = cvalid ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * ((lane >> 4) + 4 * kk))
                            : z;
        }
    }
    // pos0 = position of the tile's first token: token j sees keys <= pos0 + j
    __device__ __forceinline__ void limit(int pos0, int G, int) {
        lim = cvalid ? pos0 + col / G + 1 : 0;
    }
    __device__ __forceinline__ void stage_q(float*, int) {}

    __device__ __forceinline__ void begin() {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[nt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        l = 0.f;
    }

    // tok0 = logical position of the unit's first token; ctx = context
    // length; cs = scale * k_scale * log2(e).
    __device__ __forceinline__ void unit(const UnitRegs<KVT>& u, int tok0, int ctx, float cs, int lane) {
        f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) st = mfma_16x16x32<QT>(k_frag<KVT, QT>(u, kk), qf[kk], st);

        const int tb = tok0 + 4 * (lane >> 4);
        float t[4];
        bool valid[4];            // key visible to this lane's column
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            valid[i] = (tb + i) < lim;
            t[i] = valid[i] ? st[i] * cs : -INFINITY;
        }
        float bm = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
        bm = fmaxf(bm, xor_shfl(bm, 16));
        bm = fmaxf(bm, xor_shfl(bm, 32));     // max of the unit for column lane&15
        if (__builtin_amdgcn_ballot_w64(bm > m + kRescaleSlack)) {
            // Some column's max jumped: move every column's reference to its
            // max (a column that sees no key of this unit keeps its own).
            const float mn = fmaxf(m, bm);
            const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
            l *= alpha;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[nt] *= alpha;
            m = mn;
        }
        uint32_t pbits[4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = valid[i] ? fast_exp2(t[i] - m) : 0.f;
            pbits[i] = f32_to_bits<QT>(p);
            psum += bits_to_f32<QT>(pbits[i]);   // normalise with the rounded weights
        }
        l += psum;
        u32x2_t pf;
        pf[0] = pbits[0] | (pbits[1] << 16);
        pf[1] = pbits[2] | (pbits[3] << 16);
        if (tok0 + kSubTokens <= ctx) {
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                acc[nt] = mfma_16x16x16<QT>(v_frag<KVT, QT>(u, nt), pf, acc[nt]);
        } else {
            // Last unit of the context: rows past the context hold whatever
            // the slot last held (NaN or stale data); a zero weight times NaN
            // would still poison the sum, so zero those V elements too.
            bool row[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) row[i] = (tb + i) < ctx;
            u32x2_t vm;
            vm[0] = (row[0] ? 0x0000ffffu : 0u) | (row[1] ? 0xffff0000u : 0u);
            vm[1] = (row[2] ? 0x0000ffffu : 0u) | (row[3] ? 0xffff0000u : 0u);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                acc[nt] = mfma_16x16x16<QT>(v_frag<KVT, QT>(u, nt) & vm, pf, acc[nt]);
        }
    }

    __device__ __forceinline__ void park(float* sm_m, float* sm_l, float* sm_acc, int w, int ncols,
                                         int lane) {
        // normaliser of column lane & 15: sum the four lanes sharing it
        l += xor_shfl(l, 16);
        l += xor_shfl(l, 32);
        if (lane < 16) {
            sm_m[w * 16 + lane] = m;
            sm_l[w * 16 + lane] = l;
        }
        if (cvalid) {
            float* row = sm_acc + (w * ncols + col) * kMergeRow + 4 * (lane >> 4);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) *reinterpret_cast<f32x4_t*>(row + 16 * nt) = acc[nt];
        }
    }
};

}  // namespace pkv
