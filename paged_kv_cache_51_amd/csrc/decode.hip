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
#include "pkv_device.h"
#include "pkv_launch.h"

#include <algorithm>

namespace pkv {

template <int KVT>
struct UnitRegs {
    static constexpr int R = rows_per_sub(KVT);
    u32x4_t k[R];
    u32x4_t v[R];
};

template <int KVT>
__device__ __forceinline__ void load_unit(UnitRegs<KVT>& u, const uint8_t* kbase,
                                          const uint8_t* vbase, int lane) {
    const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(kbase) + lane;
    const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(vbase) + lane;
#pragma unroll
    for (int r = 0; r < UnitRegs<KVT>::R; ++r) u.k[r] = kp[kWave * r];
#pragma unroll
    for (int r = 0; r < UnitRegs<KVT>::R; ++r) u.v[r] = vp[kWave * r];
}

// K fragment kk (dims 8*((lane>>4) + 4kk) .. +7 of token lane&15).
template <int KVT, int QT>
__device__ __forceinline__ u32x4_t k_frag(const UnitRegs<KVT>& u, int kk) {
    if constexpr (KVT == DT_FP8) {
        const u32x4_t row = u.k[kk >> 1];
        return (kk & 1) ? e4m3x8_to_16<QT>(row[2], row[3]) : e4m3x8_to_16<QT>(row[0], row[1]);
    } else {
        return u.k[kk];
    }
}

// V fragment nt (tokens 4*(lane>>4) .. +3 of dim 16*nt + (lane&15)).
template <int KVT, int QT>
__device__ __forceinline__ u32x2_t v_frag(const UnitRegs<KVT>& u, int nt) {
    if constexpr (KVT == DT_FP8) {
        return e4m3x4_to_16<QT>(u.v[nt >> 2][nt & 3]);
    } else {
        const u32x4_t row = u.v[nt >> 1];
        u32x2_t r;
        r[0] = (nt & 1) ? row[2] : row[0];
        r[1] = (nt & 1) ? row[3] : row[1];
        return r;
    }
}

// Rescale threshold (log2 units): the reference max m of a head only moves
// when a unit's max exceeds it by more than this, so weights stay <= 2^8
// (exact math for any reference; fp32 / bf16 / fp16 hold 2^8 easily) and the
// 32 accumulators are rescaled only on such rare jumps.
constexpr float kRescaleSlack = 8.0f;

// Row stride (floats) of a head's partial output in the merge area: 128
// dims plus 4 floats of padding to spread heads over LDS banks.
constexpr int kMergeRow = kHeadDim + 4;

// Plan header ints before the item list: [count][next entry][done][reserved].
constexpr int kPlanHeader = 4;

__host__ __device__ constexpr int merge_lds_floats(int nw, int g) { return 4 + 32 * nw + nw * g * kMergeRow; }

// One 16-token unit: logits, online-softmax update, PV accumulation.
// tok0 = logical position of the unit's first token; ctx = context length;
// cs = scale * k_scale * log2(e).  m (log2 units) is the head's reference.
template <int KVT, int QT>
__device__ __forceinline__ void process_unit(const UnitRegs<KVT>& u, const u32x4_t (&qf)[4],
                                             f32x4_t (&acc)[8], float& m, float& l, int tok0,
                                             int ctx, float cs, int lane) {
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) st = mfma_16x16x32<QT>(k_frag<KVT, QT>(u, kk), qf[kk], st);

    const int tb = tok0 + 4 * (lane >> 4);
    float t[4];
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        valid[i] = (tb + i) < ctx;
        t[i] = valid[i] ? st[i] * cs : -INFINITY;
    }
    float bm = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
    bm = fmaxf(bm, xor_shfl(bm, 16));
    bm = fmaxf(bm, xor_shfl(bm, 32));     // max of the unit for head lane&15
    if (__builtin_amdgcn_ballot_w64(bm > m + kRescaleSlack)) {
        // Some head's max jumped: move every head's reference to its max.
        const float mn = fmaxf(m, bm);     // finite: every unit holds a valid token
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
        // Last unit of the context: rows past the context hold whatever the
        // slot last held (NaN or stale data); a zero weight times NaN would
        // still poison the sum, so zero those V elements too.
        u32x2_t vm;
        vm[0] = (valid[0] ? 0x0000ffffu : 0u) | (valid[1] ? 0xffff0000u : 0u);
        vm[1] = (valid[2] ? 0x0000ffffu : 0u) | (valid[3] ? 0xffff0000u : 0u);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            acc[nt] = mfma_16x16x16<QT>(v_frag<KVT, QT>(u, nt) & vm, pf, acc[nt]);
    }
}

#ifndef PKV_WAVES_PER_EU
#define PKV_WAVES_PER_EU 1
#endif
// Decode one work entry: kv head `kvh` of plan item (sequence s,
// partition part), by the NW waves of the calling workgroup.  Every exit
// before the LDS counter barrier depends only on (s, part), so all waves of
// the workgroup take it together.
template <int KVT, int QT, int BS, int NW, int DEPTH>
__device__ __forceinline__ void decode_entry(const DecodeArgs& a, float* pkv_smem, int s, int part,
                                             int kvh, int lane, int w) {
    constexpr int NSUB = BS / kSubTokens;
    constexpr int64_t SUB = sub_tile_bytes(KVT);
    constexpr int64_t TILE = SUB * NSUB;
    const int G = a.group;
    const int units_per_part = a.part_blocks * NSUB;
    const int u0 = part * units_per_part;
    const int first = u0 + w;                 // this wave's first unit
    const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks;

    // Issue every load that does not need the context length at once: the
    // block ids of this wave's first 64 units (index clamped into the table
    // row; ids past the context are never used) and the query fragments.
    // Only one memory round trip then precedes the first K/V unit.
    int ids0 = 0;
    if (a.max_blocks > 0) ids0 = bt_row[min(first + NW * lane, a.max_blocks * NSUB - 1) / NSUB];

    // Q^T fragments: lane holds head (lane & 15) of the group, 8 dims per kk.
    const int hl = lane & 15;
    const bool hvalid = hl < G;
    u32x4_t qf[4];
    {
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                              ((int64_t)s * a.num_heads + (int64_t)kvh * G + (hvalid ? hl : 0)) *
                                  (kHeadDim * 2);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const u32x4_t z = {0u, 0u, 0u, 0u};
            qf[kk] = hvalid ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * ((lane >> 4) + 4 * kk))
                            : z;
        }
    }

    int ctx = a.context_lens[s];
    ctx = ctx < a.ctx_cap ? ctx : a.ctx_cap;
    if (ctx <= 0) {
        if (part == 0) {
            uint16_t* out = reinterpret_cast<uint16_t*>(a.out) +
                            ((int64_t)s * a.num_heads + (int64_t)kvh * G) * kHeadDim;
            for (int e = threadIdx.x; e < G * kHeadDim; e += NW * kWave) out[e] = 0;
        }
        return;
    }
    const int n_units = (ctx + kSubTokens - 1) / kSubTokens;
    if (u0 >= n_units) return;
    const int u1 = min(u0 + units_per_part, n_units);
    const int nblk = (ctx + BS - 1) / BS;
    const bool single = nblk <= a.part_blocks;
    int* done = reinterpret_cast<int*>(pkv_smem);
    if (threadIdx.x == 0) *done = 0;
    __syncthreads();

    f32x4_t acc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    const int n_my = first < u1 ? (u1 - first + NW - 1) / NW : 0;
    if (n_my > 0) {
        const uint8_t* kpool = a.k_cache + (int64_t)kvh * TILE;
        const uint8_t* vpool = a.v_cache + (int64_t)kvh * TILE;
        const int64_t head_stride = (int64_t)a.num_kv_heads * TILE;
        auto load_ids = [&](int i0) -> int {
            const int i = i0 + lane;
            return i < n_my ? bt_row[(first + NW * i) / NSUB] : 0;
        };
        auto unit_offset = [&](int ids, int c0, int j) -> int64_t {
            int pb = __builtin_amdgcn_readlane(ids, j);
            if (a.num_blocks > 0 && (unsigned)pb >= (unsigned)a.num_blocks) pb = 0;
            return (int64_t)pb * head_stride + ((first + NW * (c0 + j)) % NSUB) * SUB;
        };
        // Units in chunks of 64 per wave: lane j of `ids` holds the block
        // id of the chunk's unit j (read back with readlane).  Within a chunk
        // a ring of DEPTH register buffers keeps DEPTH units in flight.  The
        // steady state only runs while every refill is a real unit, so its
        // loads are unconditional and their counters static; the drain
        // refills what is left, so no load is issued past the last unit
        // (except prologue repeats when the wave has fewer than DEPTH units).
        for (int c0 = 0; c0 < n_my; c0 += kWave) {
            const int nc = min(kWave, n_my - c0);
            const int ids = c0 == 0 ? ids0 : load_ids(c0);
            UnitRegs<KVT> buf[DEPTH];
            // Unconditional prologue: a conditional load here would make the
            // compiler's load-counter analysis assume the ring may be half
            // empty and wait for every outstanding load inside the loop.  With
            // fewer than DEPTH units the extra slots repeat the last unit.
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int64_t off = unit_offset(ids, c0, min(d, nc - 1));
                load_unit<KVT>(buf[d], kpool + off, vpool + off, lane);
            }
            auto tok_of = [&](int j) { return (first + NW * (c0 + j)) * kSubTokens; };
            int i = 0;
            for (; i + 2 * DEPTH <= nc; i += DEPTH) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    process_unit<KVT, QT>(buf[d], qf, acc, m, l, tok_of(i + d), ctx,
                                          a.qk_scale_log2, lane);
                    const int64_t off = unit_offset(ids, c0, i + d + DEPTH);
                    load_unit<KVT>(buf[d], kpool + off, vpool + off, lane);
                }
            }
            // drain: units i .. nc-1 (at most 2*DEPTH-1 of them)
            const int refills = nc - i - DEPTH;   // < DEPTH; may be negative
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                if (i + d < nc) {
                    process_unit<KVT, QT>(buf[d], qf, acc, m, l, tok_of(i + d), ctx,
                                          a.qk_scale_log2, lane);
                    if (d < refills) {
                        const int64_t off = unit_offset(ids, c0, i + d + DEPTH);
                        load_unit<KVT>(buf[d], kpool + off, vpool + off, lane);
                    }
                }
            }
#pragma unroll
            for (int d = 0; d < DEPTH - 1; ++d) {
                if (d < refills)
                    process_unit<KVT, QT>(buf[d], qf, acc, m, l, tok_of(i + DEPTH + d), ctx,
                                          a.qk_scale_log2, lane);
            }
        }
    }
    // Normaliser of head (lane & 15): sum the four lanes sharing the head.
    l += xor_shfl(l, 16);
    l += xor_shfl(l, 32);

    // ---- merge the NW waves: every wave parks its partial (m, l, O for the
    // G real heads) in LDS and leaves; the last wave to arrive merges them
    // and writes whole output rows.  No wave waits at a barrier for the
    // slowest one, so early finishers free their registers at once.
    float* sm_m = pkv_smem + 4;
    float* sm_l = sm_m + NW * 16;
    float* sm_acc = sm_l + NW * 16;
    if (lane < 16) {
        sm_m[w * 16 + lane] = m;
        sm_l[w * 16 + lane] = l;
    }
    if (hvalid) {
        float* row = sm_acc + (w * G + hl) * kMergeRow + 4 * (lane >> 4);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) *reinterpret_cast<f32x4_t*>(row + 16 * nt) = acc[nt];
    }
    __threadfence_block();
    int prev = 0;
    if (lane == 0) prev = atomicAdd(done, 1);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != NW - 1) return;
    __threadfence_block();

    for (int h = 0; h < G; ++h) {
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww * 16 + h]);
        float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = sm_m[ww * 16 + h];
            const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            const float2 ov = *reinterpret_cast<const float2*>(sm_acc + (ww * G + h) * kMergeRow + 2 * lane);
            L += f * sm_l[ww * 16 + h];
            o0 += f * ov.x;
            o1 += f * ov.y;
        }
        const float invL = 1.0f / L;
        const int hq = kvh * G + h;
        if (single) {
            const float sc = invL * a.out_scale;
            uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)s * a.num_heads + hq) * kHeadDim;
            *reinterpret_cast<uint32_t*>(out + 2 * lane) =
                (uint32_t)f32_to_bits<QT>(o0 * sc) | ((uint32_t)f32_to_bits<QT>(o1 * sc) << 16);
        } else {
            // record (s, kvh, part): G rows of head_dim floats, contiguous
            const int64_t rec = ((int64_t)s * a.num_kv_heads + kvh) * a.num_parts + part;
            *reinterpret_cast<float2*>(a.ws_out + (rec * G + h) * kHeadDim + 2 * lane) =
                make_float2(o0 * invL, o1 * invL);
        }
    }
    if (!single && lane < 32) {
        // one full 128-byte line per record: maxima of the G heads at [0, 16),
        // normalisers at [16, 32)
        const int h = lane & 15;
        float M = -INFINITY, L = 0.f;
        if (h < G) {
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww * 16 + h]);
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const float mw = sm_m[ww * 16 + h];
                L += ((mw == -INFINITY) ? 0.f : fast_exp2(mw - M)) * sm_l[ww * 16 + h];
            }
        }
        const int64_t rec = ((int64_t)s * a.num_kv_heads + kvh) * a.num_parts + part;
        a.ws_ml[rec * 32 + lane] = (h < G) ? (lane < 16 ? M : L) : 0.f;
    }
}

// One workgroup per work entry (plan item x kv head, head fastest): the
// plan lists items longest first, so the dispatcher's greedy in-order
// placement runs long work first and the heads of an item spread over
// consecutive XCDs.
template <int KVT, int QT, int BS, int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU)))
void paged_decode_mfma_kernel(const DecodeArgs a) {
    // Dynamic LDS (merge_lds_floats): [counters 4][m NW*16][l NW*16]
    // [acc NW*G rows of kMergeRow floats].
    extern __shared__ float pkv_smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int item = blockIdx.x / a.num_kv_heads;
    const int kvh = blockIdx.x - item * a.num_kv_heads;
    const int n_items = a.plan[0];
    const uint32_t packed = (uint32_t)a.plan[kPlanHeader + item];   // in bounds; valid if item < n_items
    if (item >= n_items) return;
    decode_entry<KVT, QT, BS, NW, DEPTH>(a, pkv_smem, (int)(packed >> 16), (int)(packed & 0xffffu),
                                          kvh, lane, w);
}

// Persistent form: as many workgroups as fit on the GPU at once, each
// claiming the next work entry of the longest-first plan from an atomic
// counter until the plan is exhausted.  CUs (and XCDs) that run faster
// simply take more entries.  The counters live in the plan header
// (zeroed by the planner); the last workgroup to leave resets them, so
// the plan can serve the next launch on the same stream.
template <int KVT, int QT, int BS, int NW, int DEPTH>
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
        decode_entry<KVT, QT, BS, NW, DEPTH>(a, pkv_smem, (int)(packed >> 16),
                                              (int)(packed & 0xffffu), kvh, lane, w);
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
// One wave per (query head, sequence); lane owns dims 2*lane, 2*lane+1.
template <int QT, int BS>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(const DecodeArgs a) {
    const int hq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
    int ctx = a.context_lens[s];
    ctx = ctx < a.ctx_cap ? ctx : a.ctx_cap;
    if (ctx <= 0) return;
    const int nblk = (ctx + BS - 1) / BS;
    const int np = (nblk + a.part_blocks - 1) / a.part_blocks;
    if (np <= 1) return;
    const int G = a.group, kvh = hq / G, h = hq - kvh * G;
    const int64_t base = ((int64_t)s * a.num_kv_heads + kvh) * a.num_parts;
    float M = -INFINITY;
    for (int p = lane; p < np; p += kWave) M = fmaxf(M, a.ws_ml[(base + p) * 32 + h]);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) M = fmaxf(M, xor_shfl(M, d));
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    for (int p = 0; p < np; ++p) {
        const float mp = a.ws_ml[(base + p) * 32 + h];
        const float lp = a.ws_ml[(base + p) * 32 + 16 + h];
        const float fct = fast_exp2(mp - M) * lp;
        const float2 op = *reinterpret_cast<const float2*>(a.ws_out + ((base + p) * G + h) * kHeadDim + 2 * lane);
        L += fct;
        o0 += fct * op.x;
        o1 += fct * op.y;
    }
    const float sc = a.out_scale / L;
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)s * a.num_heads + hq) * kHeadDim;
    const uint32_t packed = (uint32_t)f32_to_bits<QT>(o0 * sc) | ((uint32_t)f32_to_bits<QT>(o1 * sc) << 16);
    *reinterpret_cast<uint32_t*>(out + 2 * lane) = packed;
}

// ----------------------------------------------------------------- launch --

#ifndef PKV_WAVES_PER_GROUP
#define PKV_WAVES_PER_GROUP 4
#endif
#ifndef PKV_PIPELINE_DEPTH
#define PKV_PIPELINE_DEPTH 2
#endif
constexpr int kWavesPerGroup = PKV_WAVES_PER_GROUP;
constexpr int kDepth = PKV_PIPELINE_DEPTH;

template <int KVT, int QT, int BS>
static hipError_t launch_mfma(const DecodeArgs& a, bool persistent, hipStream_t st) {
    const size_t lds = sizeof(float) * merge_lds_floats(kWavesPerGroup, a.group);
    const dim3 block(kWavesPerGroup * kWave);
    if (!persistent) {
        const dim3 grid(a.num_seqs * a.num_kv_heads * a.num_parts);
        hipLaunchKernelGGL((paged_decode_mfma_kernel<KVT, QT, BS, kWavesPerGroup, kDepth>), grid,
                           block, lds, st, a);
        return hipGetLastError();
    }
    // as many workgroups as can be resident at once (never more than entries)
    static int per_cu[17] = {0};              // cache by group size (LDS use)
    int& occ = per_cu[a.group];
    if (!occ) {
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ, reinterpret_cast<const void*>(&paged_decode_mfma_persistent<KVT, QT, BS, kWavesPerGroup, kDepth>),
            block.x, lds);
        if (e != hipSuccess || occ <= 0) occ = 1;
    }
    int dev = 0, cus = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t entries = (int64_t)a.num_seqs * a.num_kv_heads * a.num_parts;
    const dim3 grid((unsigned)std::min<int64_t>(entries, (int64_t)occ * cus));
    hipLaunchKernelGGL((paged_decode_mfma_persistent<KVT, QT, BS, kWavesPerGroup, kDepth>), grid, block,
                       lds, st, a);
    return hipGetLastError();
}

template <int KVT, int QT>
static hipError_t launch_mfma_bs(const DecodeArgs& a, int bs, bool persistent, hipStream_t st) {
    return bs == 16 ? launch_mfma<KVT, QT, 16>(a, persistent, st)
                    : launch_mfma<KVT, QT, 32>(a, persistent, st);
}

hipError_t launch_decode_vector(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                                hipStream_t st);

hipError_t launch_decode_partitions(const DecodeArgs& a, int q_dtype, int kv_dtype,
                                    int block_size, int impl, hipStream_t st) {
    if (a.num_seqs == 0 || a.num_parts == 0) return hipSuccess;
    if (impl == 2) return launch_decode_vector(a, q_dtype, kv_dtype, block_size, st);
    const bool persistent = impl == 3;
    if (q_dtype == DT_BF16) {
        if (kv_dtype == DT_BF16) return launch_mfma_bs<DT_BF16, DT_BF16>(a, block_size, persistent, st);
        return launch_mfma_bs<DT_FP8, DT_BF16>(a, block_size, persistent, st);
    }
    if (kv_dtype == DT_FP16) return launch_mfma_bs<DT_FP16, DT_FP16>(a, block_size, persistent, st);
    return launch_mfma_bs<DT_FP8, DT_FP16>(a, block_size, persistent, st);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, int q_dtype, int block_size,
                                hipStream_t st) {
    if (a.num_seqs == 0 || a.num_parts <= 1) return hipSuccess;
    dim3 grid(a.num_heads, a.num_seqs);
    if (q_dtype == DT_BF16) {
        if (block_size == 16)
            hipLaunchKernelGGL((decode_reduce_kernel<DT_BF16, 16>), grid, dim3(kWave), 0, st, a);
        else
            hipLaunchKernelGGL((decode_reduce_kernel<DT_BF16, 32>), grid, dim3(kWave), 0, st, a);
    } else {
        if (block_size == 16)
            hipLaunchKernelGGL((decode_reduce_kernel<DT_FP16, 16>), grid, dim3(kWave), 0, st, a);
        else
            hipLaunchKernelGGL((decode_reduce_kernel<DT_FP16, 32>), grid, dim3(kWave), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace pkv
