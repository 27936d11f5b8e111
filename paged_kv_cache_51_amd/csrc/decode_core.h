// decode_core.h — body shared by the partition kernels: register layout of
// a 16-token unit, the walk over a work entry's units with a ring of loads
// in flight, and the merge of a workgroup's waves.  The per-unit math is a
// policy (matrix cores in decode.hip, vector ALU in decode_vector.hip).
#pragma once
#include "cache_write.h"
#include "pkv_launch.h"

namespace pkv {

// Entry head kvh of DecodeArgs (a pool kv head, or one column group of a
// pool kv head with more query heads than one work entry holds): its pool
// kv head, its first query head and its number of query heads.  "LLM inference basics and
// vLLM internals" §2: query heads share a kv head in contiguous groups
// (GQA), all of them in MQA.
__device__ __forceinline__ int pool_head(const DecodeArgs& a, int kvh) {
    return a.kv_split == 1 ? kvh : kvh / a.kv_split;
}
__device__ __forceinline__ int first_head(const DecodeArgs& a, int kvh) {
    const int p = pool_head(a, kvh);
    return p * a.group_all + (kvh - p * a.kv_split) * a.group;
}
__device__ __forceinline__ int heads_of(const DecodeArgs& a, int kvh) {
    const int p = pool_head(a, kvh);
    return min(a.group, a.group_all - (kvh - p * a.kv_split) * a.group);
}

// One 16-token unit of one kv head in registers: R pool rows of K and of V
// (D = head_dim).
template <int KVT, int D = kHeadDim>
struct UnitRegs {
    static constexpr int R = rows_per_sub(KVT, D);
    u32x4_t k[R];
    u32x4_t v[R];
};

// PLAIN = false: non-temporal loads ("nt"): every K / V byte is read once
// per launch, so it should not displace anything from the caches.  Measured
// on the 7B shape: 424 -> 380 us per layer (the cache-allocating stream tops
// out near 6.3 TB/s).  PLAIN = true: cache-allocating loads, for kv heads
// read by several entry heads, which then find each other's K / V in L2.
// Measured with 16-column entries (one kv head, 256 sequences of 1K-8K
// tokens): 32 query heads 172 -> 142 us, 64 query heads 279 -> 200 us (16
// query heads, one entry: 119 us with nt loads, 135 without).
template <int KVT, int D, bool PLAIN = false>
__device__ __forceinline__ void load_unit(UnitRegs<KVT, D>& u, const uint8_t* kbase,
                                          const uint8_t* vbase, int lane) {
    const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(kbase) + lane;
    const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(vbase) + lane;
    if constexpr (PLAIN) {
#pragma unroll
        for (int r = 0; r < UnitRegs<KVT, D>::R; ++r) u.k[r] = kp[kWave * r];
#pragma unroll
        for (int r = 0; r < UnitRegs<KVT, D>::R; ++r) u.v[r] = vp[kWave * r];
    } else {
#pragma unroll
        for (int r = 0; r < UnitRegs<KVT, D>::R; ++r) u.k[r] = __builtin_nontemporal_load(kp + kWave * r);
#pragma unroll
        for (int r = 0; r < UnitRegs<KVT, D>::R; ++r) u.v[r] = __builtin_nontemporal_load(vp + kWave * r);
    }
}

// K fragment kk (dims 8*((lane>>4) + 4kk) .. +7 of token lane&15).
template <int KVT, int QT, int D>
__device__ __forceinline__ u32x4_t k_frag(const UnitRegs<KVT, D>& u, int kk) {
    if constexpr (KVT == DT_FP8) {
        const u32x4_t row = u.k[kk >> 1];
        return (kk & 1) ? e4m3x8_to_16<QT>(row[2], row[3]) : e4m3x8_to_16<QT>(row[0], row[1]);
    } else {
        return u.k[kk];
    }
}

// V fragment nt (tokens 4*(lane>>4) .. +3 of dim 16*nt + (lane&15)).
template <int KVT, int QT, int D>
__device__ __forceinline__ u32x2_t v_frag(const UnitRegs<KVT, D>& u, int nt) {
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

// Row stride (floats) of a head's partial output in the merge area: d dims
// plus 4 floats of padding to spread heads over LDS banks.
__host__ __device__ constexpr int merge_row(int d = kHeadDim) { return d + 4; }
constexpr int kMergeRow = merge_row();

// Plan header ints before the item list: [count][next entry][done][reserved].
constexpr int kPlanHeader = 4;

// Merge area of NW waves: [counters 4][m: NW x kcols][l: NW x kcols]
// [partial outputs: NW x ncols rows of kMergeRow floats]; kcols = the
// policy's column capacity (16 per tile).
__host__ __device__ constexpr int merge_lds_floats(int nw, int ncols, int kcols = 16, int d = kHeadDim) {
    return 4 + 2 * nw * kcols + nw * ncols * merge_row(d);
}

// The query side of a work entry: ntok consecutive query tokens of one
// sequence (1 for decode), stored at rows row0 .. row0 + ntok - 1 of q /
// out, the first of them at logical position ctx - back (ctx = the
// sequence's context length, which counts these tokens).  The 16 matrix
// columns of the entry are the pairs (token j, head h), column c = j*G + h,
// ncols = ntok * G <= 16; token j attends to keys t <= ctx - back + j.
struct QueryTile {
    int64_t row0;
    int ntok;
    int back;
};

// ---------------------------------------------------------------------------
// Per-unit math.  A policy holds one wave's running state for the columns
// of its entry (running max m in log2 units, normaliser l, partial output)
// and provides:
//   load_q   issue the query loads (before the context length is known),
//   limit    set each column's key limit (first key position it must not
//            see) once the context length is known,
//   stage_q  make the queries usable (after the workgroup's exits, before
//            the workgroup barrier),
//   begin    reset the running state,
//   unit     one 16-token unit: logits, online-softmax update, PV,
//   park     reduce over lanes and store (m, l, O) in the merge area.
// Both policies follow the same arithmetic: fp32 logits, log2-domain
// softmax with a lazy rescale, weights rounded to the query type and the
// normaliser summed from the rounded weights.

#ifndef PKV_WAVES_PER_EU
#define PKV_WAVES_PER_EU 1
#endif
#ifndef PKV_WAVES_PER_GROUP
#define PKV_WAVES_PER_GROUP 4
#endif
#ifndef PKV_PIPELINE_DEPTH
#define PKV_PIPELINE_DEPTH 2
#endif
constexpr int kWavesPerGroup = PKV_WAVES_PER_GROUP;
constexpr int kDepth = PKV_PIPELINE_DEPTH;

// Merge the NW waves of a work entry and store its result: every wave
// parks its partial (m, l, O for the entry's columns) in LDS and leaves; the
// last wave to arrive merges them and writes whole output rows (or, for a
// split context, the partition's record).  No wave waits at a barrier for
// the slowest one, so early finishers free their registers at once.
template <class Math, int QT, int NW>
__device__ __forceinline__ void park_and_store(const DecodeArgs& a, float* pkv_smem, Math& mt, int s,
                                               int part, int kvh, int lane, int w,
                                               const QueryTile& qt, int ncols, bool single) {
    const int G = a.group;
    const int hq0 = first_head(a, kvh), nh = heads_of(a, kvh);
    constexpr int KC = Math::kCols;
    constexpr int D = Math::kD;
    constexpr int MR = merge_row(D);
    int* done = reinterpret_cast<int*>(pkv_smem);   // zeroed before the workgroup barrier
    float* sm_m = pkv_smem + 4;
    float* sm_l = sm_m + NW * KC;
    float* sm_acc = sm_l + NW * KC;
    mt.park(sm_m, sm_l, sm_acc, w, ncols, lane);
    __threadfence_block();
    int prev = 0;
    if (lane == 0) prev = atomicAdd(done, 1);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != NW - 1) return;
    __threadfence_block();

    for (int c = 0; c < ncols; ++c) {
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww * KC + c]);
        float f[NW];
        float L = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = sm_m[ww * KC + c];
            f[ww] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            L += f[ww] * sm_l[ww * KC + c];
        }
        // L = 0 only for a token placed before the start of the context
        const float invL = L > 0.f ? 1.0f / L : 0.f;
        const int h = c % G;
        if (h >= nh) continue;                    // padding column of a split group
        const int hq = hq0 + h;
        // lane owns dims e, e + 1 for e = 2 lane + 128 i
#pragma unroll
        for (int e = 2 * lane; e < D; e += 2 * kWave) {
            float o0 = 0.f, o1 = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const float2 ov = *reinterpret_cast<const float2*>(sm_acc + (ww * ncols + c) * MR + e);
                o0 += f[ww] * ov.x;
                o1 += f[ww] * ov.y;
            }
            if (single) {
                const float sc = invL * a.out_scale;
                uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((qt.row0 + c / G) * a.num_heads + hq) * D;
                *reinterpret_cast<uint32_t*>(out + e) =
                    (uint32_t)f32_to_bits<QT>(o0 * sc) | ((uint32_t)f32_to_bits<QT>(o1 * sc) << 16);
            } else {
                // (split contexts are decode only: one token, column c = head h)
                // record (s, kvh, part): G rows of head_dim floats, contiguous
                const int64_t rec = ((int64_t)s * a.num_kv_heads + kvh) * a.num_parts + part;
                *reinterpret_cast<float2*>(a.ws_out + (rec * G + h) * D + e) = make_float2(o0 * invL, o1 * invL);
            }
        }
    }
    const int ML = ml_line(G);                // (the launch gives KC >= ML / 2)
    if (!single && lane < ML) {
        // one line per record: maxima of the columns at [0, ML / 2),
        // normalisers at [ML / 2, ML) (entries of <= 16 columns: one
        // 128-byte line)
        const int h = lane % (ML / 2);
        float M = -INFINITY, L = 0.f;
        if (h < G) {
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww * KC + h]);
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const float mw = sm_m[ww * KC + h];
                L += ((mw == -INFINITY) ? 0.f : fast_exp2(mw - M)) * sm_l[ww * KC + h];
            }
        }
        const int64_t rec = ((int64_t)s * a.num_kv_heads + kvh) * a.num_parts + part;
        a.ws_ml[rec * ML + lane] = (h < G) ? (lane < ML / 2 ? M : L) : 0.f;
    }
}

// Decode one work entry: kv head `kvh` of (sequence s, partition part) for
// the query tile qt, by the NW waves of the calling workgroup.  Every exit
// before the LDS counter barrier depends only on (s, part, qt), so all
// waves of the workgroup take it together.  With NW = 1 the calling wave
// works alone (its own entry and its own LDS area, no workgroup barrier),
// so the waves of one workgroup can run different entries.  PLAIN: K / V
// with cache-allocating loads (load_unit).
template <class Math, int KVT, int QT, int BS, int NW, int DEPTH, bool PLAIN = false>
__device__ __forceinline__ void decode_entry(const DecodeArgs& a, float* pkv_smem, int s, int part,
                                             int kvh, int lane, int w, const QueryTile& qt) {
    constexpr int NSUB = BS / kSubTokens;
    constexpr int D = Math::kD;
    constexpr int64_t SUB = sub_tile_bytes(KVT, D);
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

    const int ncols = qt.ntok * G;
    Math mt;
    mt.load_q(a, qt, kvh, lane);

    const int c_full = a.context_lens[s];
    const int ctx = c_full < a.ctx_cap ? c_full : a.ctx_cap;
    // Append, first half: wave 0 fetches the new token's K / V row and the
    // block id of position c - 1 now, beside the query loads, so the write
    // below adds no memory round trip of its own.  Every partition's wave 0
    // fetches (512 bytes); only the one holding position c - 1 writes.
    const bool append = a.new_key != nullptr && qt.ntok == 1 && w == 0;
    const int ph = pool_head(a, kvh);
    TokenRow<D> new_row;
    int32_t new_pb = -1;
    if (append) {
        const int64_t row = ((int64_t)s * a.pool_kv_heads + ph) * D;
        new_row.load(reinterpret_cast<const uint16_t*>(a.new_key) + row,
                     reinterpret_cast<const uint16_t*>(a.new_value) + row, lane);
        // only when the context is not clamped (the table and
        // max_context_len cover position c - 1)
        if (c_full > 0 && c_full == ctx) new_pb = bt_row[(c_full - 1) / BS];
    }
    // keys this tile may see: positions < kv_end (its last token's + 1)
    const int kv_end = min(ctx, ctx - qt.back + qt.ntok);
    if (kv_end <= 0) {
        if (part == 0) {
            // no key at all: zero output (empty context, or tokens placed
            // before the start of the context)
            const int hq0 = first_head(a, kvh), nh = heads_of(a, kvh);
            for (int e = (NW == 1 ? lane : (int)threadIdx.x); e < ncols * D; e += NW * kWave) {
                const int c = e / D;
                if (c % G >= nh) continue;
                uint16_t* out = reinterpret_cast<uint16_t*>(a.out) +
                                ((qt.row0 + c / G) * a.num_heads + hq0 + c % G) * D;
                out[e % D] = 0;
            }
        }
        return;
    }
    mt.limit(ctx - qt.back, G, lane);
    const int n_units = (kv_end + kSubTokens - 1) / kSubTokens;
    if (u0 >= n_units) return;
    const int u1 = min(u0 + units_per_part, n_units);
    const int nblk = (kv_end + BS - 1) / BS;
    const bool single = nblk <= a.part_blocks;
    int* done = reinterpret_cast<int*>(pkv_smem);
    const int ltid = NW == 1 ? lane : (int)threadIdx.x;
    if (ltid == 0) *done = 0;
    if (append && u1 == n_units && (unsigned)new_pb < (unsigned)a.num_blocks) {
        // Append, second half: this workgroup's partition holds position
        // ctx - 1, the new token, so it writes the token's K / V into its
        // slot (as reshape_and_cache would) before any wave loads that unit;
        // the barrier below orders the stores before those loads (waves of
        // one workgroup share the CU's write-through L1).  Every entry head
        // of a split pool head writes the same bytes, so each one reads its
        // own store.
        new_row.template store<QT, KVT, BS>(const_cast<uint8_t*>(a.k_cache),
                                            const_cast<uint8_t*>(a.v_cache),
                                            (int64_t)new_pb * BS + (ctx - 1) % BS, a.pool_kv_heads,
                                            ph, lane, a.k_inv, a.v_inv);
        if constexpr (NW == 1) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    }
    mt.stage_q(pkv_smem + merge_lds_floats(NW, ncols, Math::kCols, D), ltid);
    if constexpr (NW > 1) __syncthreads();
    // With an append, no wave's pool load may be moved above the barrier by
    // the compiler (plain loads have been seen sunk below workgroup
    // barriers; the asm's memory clobber pins them on this side).  The
    // hardware side needs no wait: waves of one workgroup share the CU's
    // vector memory path, and the workgroup-scope release of the barrier
    // orders the stores before the other waves' later loads.
    if (a.new_key != nullptr) asm volatile("" ::: "memory");
    mt.begin();

    const int n_my = first < u1 ? (u1 - first + NW - 1) / NW : 0;
    if (n_my > 0) {
        const uint8_t* kpool = a.k_cache + (int64_t)ph * TILE;
        const uint8_t* vpool = a.v_cache + (int64_t)ph * TILE;
        const int64_t head_stride = (int64_t)a.pool_kv_heads * TILE;
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
            UnitRegs<KVT, D> buf[DEPTH];
            // Unconditional prologue: a conditional load here would make the
            // compiler's load-counter analysis assume the ring may be half
            // empty and wait for every outstanding load inside the loop.  With
            // fewer than DEPTH units the extra slots repeat the last unit.
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int64_t off = unit_offset(ids, c0, min(d, nc - 1));
                load_unit<KVT, D, PLAIN>(buf[d], kpool + off, vpool + off, lane);
            }
            auto tok_of = [&](int j) { return (first + NW * (c0 + j)) * kSubTokens; };
            int i = 0;
            for (; i + 2 * DEPTH <= nc; i += DEPTH) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    mt.unit(buf[d], tok_of(i + d), ctx, a.qk_scale_log2, lane);
                    const int64_t off = unit_offset(ids, c0, i + d + DEPTH);
                    load_unit<KVT, D, PLAIN>(buf[d], kpool + off, vpool + off, lane);
                }
            }
            // drain: units i .. nc-1 (at most 2*DEPTH-1 of them)
            const int refills = nc - i - DEPTH;   // < DEPTH; may be negative
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                if (i + d < nc) {
                    mt.unit(buf[d], tok_of(i + d), ctx, a.qk_scale_log2, lane);
                    if (d < refills) {
                        const int64_t off = unit_offset(ids, c0, i + d + DEPTH);
                        load_unit<KVT, D, PLAIN>(buf[d], kpool + off, vpool + off, lane);
                    }
                }
            }
#pragma unroll
            for (int d = 0; d < DEPTH - 1; ++d) {
                if (d < refills)
                    mt.unit(buf[d], tok_of(i + DEPTH + d), ctx, a.qk_scale_log2, lane);
            }
        }
    }
    park_and_store<Math, QT, NW>(a, pkv_smem, mt, s, part, kvh, lane, w, qt, ncols, single);
}

// Workgroups of the grid form: the plan's items in groups of 8, each group
// expanded over the kv heads (8 x Hkv workgroups per group).
__host__ __device__ inline int64_t grid_workgroups(const DecodeArgs& a) {
    const int64_t groups = ((int64_t)a.num_seqs * a.num_parts + 7) / 8;
    return groups * 8 * a.num_kv_heads;
}

// Grid form: one workgroup per work entry (plan item x kv head).  Workgroup
// b is dispatched to XCD b % 8, so within each group of 8 * Hkv workgroups
// the 8 items take one XCD each and b / 8 picks the head: all heads of an
// item run on one XCD at the same time.  Their K / V tiles of a physical
// block are adjacent in the pool, and reading them together is measurably
// faster than spreading them out (spreading the heads of a sequence over
// other times costs about 10%; one XCD instead of four gains about 1%).
// The plan lists items longest first, so the dispatcher's greedy in-order
// placement runs long work first.  Dynamic LDS: [counters 4][m NW*16]
// [l NW*16][acc NW*G rows of kMergeRow floats][policy's query area].
template <class Math, int KVT, int QT, int BS, int NW, int DEPTH, bool PLAIN = false>
__device__ __forceinline__ void grid_entry(const DecodeArgs& a, float* pkv_smem) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int per_group = 8 * a.num_kv_heads;
    const int grp = blockIdx.x / per_group;
    const int rem = blockIdx.x - grp * per_group;
    const int item = grp * 8 + (rem & 7);
    const int kvh = rem >> 3;
    const int n_items = a.plan[0];
    // loaded along with the count (index clamped into the list); valid if
    // item < n_items
    const uint32_t packed = (uint32_t)a.plan[kPlanHeader + min(item, a.num_seqs * a.num_parts - 1)];
    if (item >= n_items) return;
    const int s = (int)(packed >> 16);
    decode_entry<Math, KVT, QT, BS, NW, DEPTH, PLAIN>(a, pkv_smem, s, (int)(packed & 0xffffu), kvh, lane, w,
                                                       QueryTile{s, 1, 1});
}

}  // namespace pkv
