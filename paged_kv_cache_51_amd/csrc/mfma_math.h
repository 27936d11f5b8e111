// mfma_math.h — the matrix-core per-unit math of the partition kernels
// (the policy decode_core.h's entry bodies call): logits, online softmax
// and PV for one 16-token unit, and the park into the merge area.
#pragma once
#include "decode_core.h"

namespace pkv {

// MFMA policy: S^T = K . Q^T on four 16x16x32 MFMAs per 16-column tile
// (rows = 16 tokens, columns = the entry's (query token, head) pairs padded
// to 16 per tile; for decode the G heads), then O^T += V^T . P^T on eight
// 16x16x16 MFMAs per tile whose B operand is S^T's lane order.  Lane l holds
// column 16t + (l & 15) of tile t for the softmax state and rows
// 4*(l>>4)..+3 of each 16-row tile.  NT tiles (1 for the partition
// kernels, 2 for the multi-token wave kernel) share the unit's K and V
// fragments and the loop around them.
template <int KVT, int QT, int NT = 1, int D = kHeadDim>
struct MfmaMath {
    static constexpr int kMaxGroup = 16;
    static constexpr int kCols = 16 * NT;     // columns of one entry at most
    static constexpr int kD = D;              // head_dim
    static constexpr int KD = D / 32;         // k steps of the logits (32 dims each)
    static constexpr int NV = D / 16;         // 16-dim tiles of the output
    __host__ __device__ static constexpr int query_lds_floats(int) { return 0; }

    u32x4_t qf[NT][KD];       // Q^T fragments: 8 dims per kk of this lane's columns
    f32x4_t acc[NT][NV];
    float m[NT], l[NT];
    int col;                  // lane & 15; tile t's column is 16t + col
    bool cvalid[NT];          // the column holds a real (token, head)
    int lim[NT];              // the column sees keys at positions < lim

    __device__ __forceinline__ void load_q(const DecodeArgs& a, const QueryTile& qt, int kvh,
                                           int lane) {
        const int G = a.group;
        const int hq0 = first_head(a, kvh), nh = heads_of(a, kvh);
        col = lane & 15;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int c = 16 * t + col;
            // column c = (token c / G, head c % G); heads past nh pad the
            // last column group of a split kv head
            cvalid[t] = c < qt.ntok * G && c % G < nh;
            const int j = cvalid[t] ? c / G : 0;
            const int h = cvalid[t] ? c - j * G : 0;
            const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                                  ((qt.row0 + j) * a.num_heads + hq0 + h) * (D * 2);
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                const u32x4_t z = {0u, 0u, 0u, 0u};
                qf[t][kk] = cvalid[t] ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * ((lane >> 4) + 4 * kk))
                                      : z;
            }
        }
    }
    // pos0 = position of the entry's first token: token j sees keys <= pos0 + j
    __device__ __forceinline__ void limit(int pos0, int G, int) {
#pragma unroll
        for (int t = 0; t < NT; ++t) lim[t] = cvalid[t] ? pos0 + (16 * t + col) / G + 1 : 0;
    }
    __device__ __forceinline__ void stage_q(float*, int) {}

    __device__ __forceinline__ void begin() {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int nt = 0; nt < NV; ++nt) acc[t][nt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            m[t] = -INFINITY;
            l[t] = 0.f;
        }
    }

    // tok0 = logical position of the unit's first token; ctx = context
    // length; cs = scale * k_scale * log2(e).
    __device__ __forceinline__ void unit(const UnitRegs<KVT, D>& u, int tok0, int ctx, float cs, int lane) {
        unit_impl<false>(u, tok0, ctx, 0xffffu, cs, lane);
    }
    // A pool sub-tile of which only some rows hold keys of the sequence:
    // row r is a key when bit r of the wave-uniform rows16 is set, and is
    // skipped otherwise (weight 0, V zeroed: the row may hold anything).
    // Every real column sees every key.  With all 16 bits set the result
    // is unit()'s on a unit wholly inside the context, bit for bit.
    __device__ __forceinline__ void unit_rows(const UnitRegs<KVT, D>& u, uint32_t rows16, float cs, int lane) {
        unit_impl<true>(u, 0, 0, rows16, cs, lane);
    }

    template <bool ROWS>
    __device__ __forceinline__ void unit_impl(const UnitRegs<KVT, D>& u, int tok0, int ctx, uint32_t rows16,
                                              float cs, int lane) {
        f32x4_t st[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) st[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            const u32x4_t kf = k_frag<KVT, QT>(u, kk);
#pragma unroll
            for (int t = 0; t < NT; ++t) st[t] = mfma_16x16x32<QT>(kf, qf[t][kk], st[t]);
        }

        const int tb = tok0 + 4 * (lane >> 4);
        const uint32_t rows4 = (rows16 >> (4 * (lane >> 4))) & 0xfu;   // this lane's rows (ROWS)
        float x[NT][4];
        bool valid[NT][4];        // key visible to this lane's column
        float bm[NT];
        bool jump = false;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (ROWS) valid[t][i] = cvalid[t] && ((rows4 >> i) & 1u);
                else valid[t][i] = (tb + i) < lim[t];
                x[t][i] = valid[t][i] ? st[t][i] * cs : -INFINITY;
            }
            bm[t] = fmaxf(fmaxf(x[t][0], x[t][1]), fmaxf(x[t][2], x[t][3]));
            bm[t] = fmaxf(bm[t], xor_shfl(bm[t], 16));
            bm[t] = fmaxf(bm[t], xor_shfl(bm[t], 32));     // max of the unit for the column
            jump |= bm[t] > m[t] + kRescaleSlack;
        }
        if (__builtin_amdgcn_ballot_w64(jump)) {
            // Some column's max jumped: move every column's reference to its
            // max (a column that sees no key of this unit keeps its own).
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float mn = fmaxf(m[t], bm[t]);
                const float alpha = (m[t] == -INFINITY) ? 0.f : fast_exp2(m[t] - mn);
                l[t] *= alpha;
#pragma unroll
                for (int nt = 0; nt < NV; ++nt) acc[t][nt] *= alpha;
                m[t] = mn;
            }
        }
        u32x2_t pf[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            uint32_t pbits[4];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = valid[t][i] ? fast_exp2(x[t][i] - m[t]) : 0.f;
                pbits[i] = f32_to_bits<QT>(p);
                psum += bits_to_f32<QT>(pbits[i]);   // normalise with the rounded weights
            }
            l[t] += psum;
            pf[t][0] = pbits[0] | (pbits[1] << 16);
            pf[t][1] = pbits[2] | (pbits[3] << 16);
        }
        if (ROWS ? rows16 == 0xffffu : tok0 + kSubTokens <= ctx) {
#pragma unroll
            for (int nt = 0; nt < NV; ++nt) {
                const u32x2_t vf = v_frag<KVT, QT>(u, nt);
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t][nt] = mfma_16x16x16<QT>(vf, pf[t], acc[t][nt]);
            }
        } else {
            // Last unit of the context: rows past the context hold whatever
            // the slot last held (NaN or stale data); a zero weight times NaN
            // would still poison the sum, so zero those V elements too.
            // (ROWS: rows whose bit is clear, which another token may hold)
            bool row[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) row[i] = ROWS ? ((rows4 >> i) & 1u) != 0 : (tb + i) < ctx;
            u32x2_t vm;
            vm[0] = (row[0] ? 0x0000ffffu : 0u) | (row[1] ? 0xffff0000u : 0u);
            vm[1] = (row[2] ? 0x0000ffffu : 0u) | (row[3] ? 0xffff0000u : 0u);
#pragma unroll
            for (int nt = 0; nt < NV; ++nt) {
                const u32x2_t vf = v_frag<KVT, QT>(u, nt) & vm;
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t][nt] = mfma_16x16x16<QT>(vf, pf[t], acc[t][nt]);
            }
        }
    }

    __device__ __forceinline__ void park(float* sm_m, float* sm_l, float* sm_acc, int w, int ncols,
                                         int lane) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // normaliser of the column: sum the four lanes sharing it
            float lt = l[t];
            lt += xor_shfl(lt, 16);
            lt += xor_shfl(lt, 32);
            if (lane < 16) {
                sm_m[w * kCols + 16 * t + lane] = m[t];
                sm_l[w * kCols + 16 * t + lane] = lt;
            }
            if (cvalid[t]) {
                float* row = sm_acc + (w * ncols + 16 * t + col) * merge_row(D) + 4 * (lane >> 4);
#pragma unroll
                for (int nt = 0; nt < NV; ++nt) *reinterpret_cast<f32x4_t*>(row + 16 * nt) = acc[t][nt];
            }
        }
    }
};

}  // namespace pkv
