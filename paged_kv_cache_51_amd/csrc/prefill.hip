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

// Workgroup form (chunks of at most four 16-column tiles): workgroup
// (sequence s, query tile, kv head) attends the tile's tokens to the paged
// context, causally: token j of a chunk of q_len new tokens sits at position
// ctx - q_len + j and sees keys up to it.  The decode entry body serves it.
// Tiles hold tile_tokens = 16 / G tokens (so the tile's (token, head) pairs
// fill the 16 MFMA columns), and the last tiles of a chunk, which see the
// most keys, are dispatched first, sequences in the staged form's order
// (longest context first, XCD bands).  No context split: the tiles give the
// parallelism.  With q_len = 1 a tile is exactly a decode entry.
#ifndef PKV_PREFILL_WG_NT2
#define PKV_PREFILL_WG_NT2 1
#endif

// Sequences ranked above this count keep their own order (the ranking costs
// each workgroup num_seqs^2 / 256 LDS reads).
constexpr int kRankSeqsMax = 512;

// Rank of the sequence at slot j (0 <= j < bw) of band `band` (bands of P
// sequences, bw of them in this band).  Slot j's workgroups all go to the
// same XCDs; the slots alternate direction from band to band so that no XCD
// gets the longer sequence of every band (with slot j = rank offset j,
// XCDs 0-3 carried 12 % more work than XCDs 4-7 on 1-8K contexts and
// finished 90 us later).
__device__ __forceinline__ int band_rank(int band, int j, int P, int bw) {
    return band * P + ((band & 1) ? bw - 1 - j : j);
}

// The sequence of rank `rank` when the sequences are ordered by descending
// context length (ties by index).  Whole-workgroup call (barriers); `lds`
// holds kRankSeqsMax + 1 ints and is free again on return.
__device__ __forceinline__ int seq_of_rank(const DecodeArgs& a, int rank, int* lds) {
    const int S = a.num_seqs;
    if (S > kRankSeqsMax) return rank;
    for (int i = threadIdx.x; i < S; i += blockDim.x) lds[i] = min(a.context_lens[i], a.ctx_cap);
    __syncthreads();
    for (int i = threadIdx.x; i < S; i += blockDim.x) {
        const int ci = lds[i];
        int r = 0;
        for (int j = 0; j < S; ++j) {
            const int cj = lds[j];
            r += (cj > ci) | ((cj == ci) & (j < i));
        }
        if (r == rank) lds[kRankSeqsMax] = i;        // ranks are a permutation
    }
    __syncthreads();
    // the same word in every lane: a scalar, so that every quantity derived
    // from the sequence (its lengths, block-table row, loop bounds) is one
    const int s = __builtin_amdgcn_readfirstlane(lds[kRankSeqsMax]);
    __syncthreads();
    return s;
}

// Two-tile workgroups over 16-bit pools: one unit in flight per wave and two
// waves per SIMD (247-256 VGPRs instead of 277 at one wave): 3-5 % faster on
// 4- and 8-token chunks.  fp8 pools keep two units in flight at one wave per
// SIMD (one unit in flight was 59 % slower for them).
template <int KVT, int NT>
__host__ __device__ constexpr int small_chunk_waves_per_eu() {
    return (NT == 2 && KVT != DT_FP8) ? 2 : PKV_WAVES_PER_EU;
}
template <int KVT, int NT>
__host__ __device__ constexpr int small_chunk_depth() {
    return (NT == 2 && KVT != DT_FP8) ? 1 : kDepth;
}

// PLAIN: cache-allocating K / V loads, for kv heads split over several
// entry heads (they share the K / V in L2; load_unit in decode_core.h).
template <int KVT, int QT, int BS, int NW, int DEPTH, int NT, bool PLAIN = false>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(small_chunk_waves_per_eu<KVT, NT>())))
void paged_prefill_mfma_kernel(const DecodeArgs a, const int32_t* __restrict__ query_start,
                               int tile_tokens, int max_tiles) {
    extern __shared__ float pkv_smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int Hkv = a.num_kv_heads;
    const int kvh = blockIdx.x % Hkv;
    const int item = blockIdx.x / Hkv;               // (sequence rank, tile) item
    const int P = (Hkv < 8 && 8 % Hkv == 0) ? 8 / Hkv : 1;
    const int band = item / (P * max_tiles);
    const int in_band = item - band * P * max_tiles;
    const int bw = min(P, a.num_seqs - band * P);    // sequences in this band
    const int tile = max_tiles - 1 - in_band / bw;
    const int s = seq_of_rank(a, band_rank(band, in_band % bw, P, bw), reinterpret_cast<int*>(pkv_smem));
    const int q0 = query_start[s];
    const int q_len = query_start[s + 1] - q0;
    const int j0 = tile * tile_tokens;
    if (j0 >= q_len) return;
    decode_entry<MfmaMath<KVT, QT, NT>, KVT, QT, BS, NW, DEPTH, PLAIN>(
        a, pkv_smem, s, 0, kvh, lane, w,
        QueryTile{(int64_t)q0 + j0, min(tile_tokens, q_len - j0), q_len - j0});
}

// Max over the four 16-lane rows of the wave, the result in every lane.
// permlane16_swap(v, v) returns rows (0, 0, 2, 2) and (1, 1, 3, 3) of v;
// permlane32_swap(x, x) returns rows (0, 1, 0, 1) and (2, 3, 2, 3) of x.
// (Every operation here is visible to the compiler: it must place the wait
// states between a matrix-core result and the vector instructions reading
// it, which it cannot do for inline assembly.)
__device__ __forceinline__ float rows_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Two fp32 values -> a packed pair of the query type (RNE), low first.
template <int QT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    if constexpr (QT == DT_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// 1.0 in both halves of a packed pair of the query type.
template <int QT>
__device__ __forceinline__ constexpr uint32_t ones2() {
    return QT == DT_BF16 ? 0x3f803f80u : 0x3c003c00u;
}

// ---------------------------------------------------------------------------
// Staged form, for chunks of more than four 16-column tiles.  Workgroup =
// (sequence, four consecutive 32-column query tiles, kv head): wave w owns
// tile w (32 / G tokens, two 16-column MFMA tiles) and the four waves walk
// the keys together, two 16-token units ("a pair") at a time, sharing every
// K / V byte through LDS (reading the units into each wave separately
// moves four times the bytes through the L1 return path, which then bounds
// the kernel: 405 against 463 TFLOP/s on 16 x 512-token chunks).
//   - wave w fetches one quarter of each pair (K of unit A / K of unit B /
//     V of A / V of B for w = 0..3), 16 bytes per lane per 1 KiB pool row,
//     one pair ahead in registers, and writes it to one of two LDS stages:
//     K rows as in the pool, V straight in PV operand order (entry [nt][lane]
//     = the unit A then unit B halves of dim tile nt; fp8 pools are widened
//     to the query type here); one workgroup barrier per pair;
//   - three waves per SIMD (168 VGPRs): the PV operands are read from LDS
//     right before the PV MFMAs, and except over widened fp8 stages the
//     query fragments of k steps 2 and 3 live in an LDS area of the wave's
//     own; occupancy is what hides each wave's latencies (one wave per SIMD
//     ran 35-55 % slower, three waves 4-14 % faster than two);
//   - PV runs on 16x16x32 MFMAs whose 32-long contraction covers both units
//     (16x16x16 runs at half the matrix rate on gfx950): lane group
//     g = lane >> 4 contributes tokens 4g..4g+3 of unit A and of unit B to
//     its eight k slots, in V (A operand) and P (B operand) alike;
//   - pairs that every real column of the wave sees in full (all but the
//     last one or two on the diagonal) skip the per-key causal and context
//     masks; the logit scale is applied to the row maxima (max(s) * cs =
//     max(s * cs) for cs > 0; a negative scale flips the query's signs) and
//     folded into the exponent as one fused multiply-add, p = 2^(s*cs - m),
//     with the running max m kept on scaled values; row maxima are reduced over
//     the four 16-lane rows with the gfx950 permlane swaps (VALU, no LDS
//     round trip); the normaliser is summed from the rounded weights with
//     packed dot instructions;
//   - waves whose tile sees fewer keys, or that have no tile, keep fetching
//     and meeting the barriers; a wave's result needs no merge: it
//     normalises its columns in registers and writes them out;
//   - work order: longest first.  A workgroup's time is about its
//     sequence's context length, so the sequences are taken by descending
//     context (each workgroup ranks them itself from context_lens) and,
//     within one, the query tiles that see the most keys first; in the
//     launch order of the grid's (sequence, group) items a band of 8 / H_kv
//     sequences shares the groups round-robin, so that every workgroup of
//     one (sequence, kv head) lands on the same XCD and its K / V stays in
//     that XCD's L2 (blocks go to the XCDs in turn); successive bands run
//     in alternating directions to even out the XCDs' work.  Ordered by group
//     first, as before, contexts of 1-8K left most of the chip idle while
//     the last long sequences ran (1.2-1.5x the balanced time).
// Same arithmetic as decode otherwise: fp32 logits, log2-domain online
// softmax with the lazy rescale, weights rounded to the query type.

// LDS bytes of one stage: K [2 units][R rows][64 lanes] x 16 B, V 8 dim
// tiles x 64 lanes x 16 B (16-bit pools) or [2][R][64] x 16 B raw (fp8).
__host__ __device__ constexpr int stage_bytes(int kvt) {
    return 2 * rows_per_sub(kvt) * 1024 + (kvt == DT_FP8 ? 2 * rows_per_sub(kvt) * 1024 : 8 * 1024);
}
static_assert(2 * stage_bytes(DT_FP8) >= 4 * (kRankSeqsMax + 1), "the ranking borrows the stage area");

// Type of the staged kernel's LDS stages: an fp8 pool is widened to the
// query type by the stage writer (each wave converts its quarter of a pair
// once, instead of every wave converting the whole pair for its MFMAs; on
// the three-wave packed-column kernel that was faster or equal on every
// shape measured, 7B 16 x 512 624 -> 573 us, 72B fp8 8 x 512 4637 -> 4397
// us, against fp8 stages widened by each wave).
__host__ __device__ constexpr int staged_kvt(int kvt, int qt) {
    return kvt == DT_FP8 ? qt : kvt;
}

// Running maximum of a staged-kernel column that has seen no key yet: finite,
// so that the exponent subtracts it with no select (-inf would need one to
// avoid -inf - -inf).  Every finite scaled logit passes it plus the rescale
// slack, so the first key a column sees replaces it, with alpha =
// 2^(-FLT_MAX - m) = 0 for the empty sums.
constexpr float kNoKeyMax = -3.402823466e38f;
// Logit of a key a column must not see (causal limit, context end): finite,
// so that kMaskedLogit * cs is finite or -inf for every cs >= 0 (cs = 0
// included) and never NaN; its weight is set to 0 by a select.  No real
// logit of finite 16-bit inputs is this value.
constexpr float kMaskedLogit = -3.402823466e38f;

// One unit pair of a stage: logits, online softmax and PV for the wave's two
// column tiles.  masked (uniform): apply each column's causal limit; pairs
// every real column sees in full skip it.  V rows at or past the context
// end arrive zeroed from the stage writer, so no V mask is needed here.
// One code path: the branch covers only the logit select (a second copy of
// the whole pair made the compiler copy the 64 accumulators every pair).
// KVT here is the type the stage holds: 16-bit (fp8 pools are widened to
// the query type by the stage writer).
//
// LATE_V: read the PV operands right before the PV MFMAs instead of before
// the softmax (fewer registers live through the softmax: what lets the
// staged form run three waves per SIMD).  QLDS: this lane's query
// fragments of k steps 2 and 3 come from LDS (entry [t][kk - 2] at
// qhi[(2t + kk - 2) * 64]) instead of registers.  PRIO: raise the wave's
// issue priority over its two MFMA chains, so that of the waves sharing a
// SIMD the one with matrix work ready issues it while the others run their
// softmax (bit-identical; 2-5 % faster on 16-token blocks, 3-6 % on 32-token
// blocks of 16-bit pools; with fp8 pools in 32-token blocks it left a
// spill inside the loop and was 1-4 % slower, so it is off there).
template <int KVT, int QT, bool LATE_V, bool QLDS, bool PRIO, class Math>
__device__ __forceinline__ void staged_pair(Math& mt, const uint8_t* stage, int tok0,
                                            bool masked, float cs, int lane, const u32x4_t* qhi) {
    static_assert(KVT != DT_FP8, "stages hold 16-bit K / V");
    constexpr int R = rows_per_sub(KVT);
    constexpr int NT = Math::kCols / 16;           // 16-column tiles of the wave
    const u32x4_t* kl = reinterpret_cast<const u32x4_t*>(stage) + lane;
    const u32x4_t* vl = reinterpret_cast<const u32x4_t*>(stage + 2 * R * 1024) + lane;
    // logits
    f32x4_t st[2][NT];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) st[u][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        u32x4_t k[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) k[u] = kl[(u * R + kk) * kWave];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            u32x4_t qv;
            if constexpr (QLDS) qv = kk >= 2 ? qhi[(2 * t + kk - 2) * kWave] : mt.qf[t][kk];
            else qv = mt.qf[t][kk];
            st[0][t] = mfma_16x16x32<QT>(k[0], qv, st[0][t]);
            st[1][t] = mfma_16x16x32<QT>(k[1], qv, st[1][t]);
        }
    }
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    // PV operands, read before the softmax so their LDS latency hides behind
    // it (the rescale branch below ends the scheduler's region)
    auto read_v = [&](u32x4_t (&vop)[8]) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) vop[nt] = vl[nt * kWave];
    };
    u32x4_t vop[8];
    if constexpr (!LATE_V) read_v(vop);
    // raw logits; the scale (cs >= 0) goes into the maxima and into the
    // exponent's fused multiply-add; keys a column must not see hold the
    // finite kMaskedLogit for the max and get weight 0 below (finite, so
    // that no product with cs = 0 is ever a NaN: this file is built assuming
    // none occurs)
    float y[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) y[t][4 * u + i] = st[u][t][i];
    if (masked) {
        const int ta = tok0 + 4 * (lane >> 4);   // this lane's keys: ta..ta+3, ta+16..ta+19
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[t][4 * u + i] = (ta + 16 * u + i) < mt.lim[t] ? y[t][4 * u + i] : kMaskedLogit;
    }
    // The rescale test needs only this lane's own maximum: a column's scaled
    // maximum passes m + slack exactly when one of its lanes' does (cs >= 0
    // and rounding keep the order).  A lane whose keys are all masked may
    // pass once, while its column has seen no key (kMaskedLogit * cs >
    // kNoKeyMax for cs < 1); that rescale multiplies empty sums by 0 and is
    // harmless.  The column maximum across lanes is formed only inside the
    // rare rescale branch.
    float mx[NT];
    bool jump = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        mx[t] = fmaxf(fmaxf(fmaxf(y[t][0], y[t][1]), fmaxf(y[t][2], y[t][3])),
                      fmaxf(fmaxf(y[t][4], y[t][5]), fmaxf(y[t][6], y[t][7])));
        jump |= mx[t] * cs > mt.m[t] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(jump)) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float rm = rows_max(mx[t]);
            const float mn = fmaxf(mt.m[t], rm * cs);
            const float alpha = fast_exp2(mt.m[t] - mn);   // 0 when leaving kNoKeyMax
            mt.l[t] *= alpha;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) mt.acc[t][nt] *= alpha;
            mt.m[t] = mn;
        }
    }
    u32x4_t pf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        // masked keys: the select below gives them weight 0 (their exponent
        // is finite or -inf, never NaN); m is finite
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(fmaf(y[t][j], cs, -mt.m[t]));
        if (masked) {
#pragma unroll
            for (int j = 0; j < 8; ++j) pv[j] = y[t][j] == kMaskedLogit ? 0.f : pv[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) pf[t][j] = pack2<QT>(pv[2 * j], pv[2 * j + 1]);
        float lt = mt.l[t];
#pragma unroll
        for (int j = 0; j < 4; ++j) lt = dot2<QT>(pf[t][j], ones2<QT>(), lt);
        mt.l[t] = lt;
    }
    // PV
    if constexpr (LATE_V) read_v(vop);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int t = 0; t < NT; ++t) mt.acc[t][nt] = mfma_16x16x32<QT>(vop[nt], pf[t], mt.acc[t][nt]);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
}

// Columns packed across token boundaries (the staged form): local column c
// of the wave holds the (token, head) pair number h0 + c counted from head 0
// of query row row0, for c < ncols; the rest are padding.  Sets the query
// fragments, the column validity and each column's causal limit (keys at
// positions < lim; pos0 = position of row0).
template <class Math>
__device__ __forceinline__ void load_q_cols(Math& mt, const DecodeArgs& a, int64_t row0, int h0, int ncols,
                                            int kvh, int lane) {
    constexpr int NT = Math::kCols / 16;
    const int G = a.group;
    const int hq0 = first_head(a, kvh), nh = heads_of(a, kvh);
    mt.col = lane & 15;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int c = 16 * t + mt.col;
        // heads past nh pad the last column group of a split kv head
        mt.cvalid[t] = c < ncols && (c + h0) % G < nh;
        const int cl = mt.cvalid[t] ? c + h0 : 0;
        const int j = cl / G;
        const int h = cl - j * G;
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                              ((row0 + j) * a.num_heads + hq0 + h) * (kHeadDim * 2);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const u32x4_t z = {0u, 0u, 0u, 0u};
            mt.qf[t][kk] = mt.cvalid[t] ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * ((lane >> 4) + 4 * kk)) : z;
        }
    }
}
template <class Math>
__device__ __forceinline__ void limit_cols(Math& mt, int pos0, int h0, int G) {
    constexpr int NT = Math::kCols / 16;
#pragma unroll
    for (int t = 0; t < NT; ++t) mt.lim[t] = mt.cvalid[t] ? pos0 + (16 * t + mt.col + h0) / G + 1 : 0;
}

// 16-column tiles per wave of the staged form: 2 (two waves per SIMD).  4
// tiles (64 columns, half the LDS reads and barriers per MFMA) need 333
// VGPRs, one wave per SIMD, and measured 35-55 % slower on the multi-token
// workloads: the second wave is what hides each wave's latencies.
#ifndef PKV_PREFILL_TILES_PER_WAVE
#define PKV_PREFILL_TILES_PER_WAVE 2
#endif

// (two waves per SIMD: the register budget is kept at 256 per lane)
#ifndef PKV_PREFILL_WAVES_PER_EU
#define PKV_PREFILL_WAVES_PER_EU 2
#endif

// Waves per SIMD of the staged form: three (168 VGPRs), with the PV
// operands read late and a one-pair fetch ring; 16-bit pools (twice the
// fetch registers of fp8) also keep half of the query fragments in LDS.
#ifndef PKV_PREFILL_THREE_WAVES_16BIT
#define PKV_PREFILL_THREE_WAVES_16BIT 1
#endif
template <int KVT, int NT>
__host__ __device__ constexpr int staged_waves_per_eu() {
    return NT != 2 ? 1 : ((KVT == DT_FP8 || PKV_PREFILL_THREE_WAVES_16BIT) ? 3 : PKV_PREFILL_WAVES_PER_EU);
}
// query fragments of k steps 2, 3 in LDS at three waves, except for fp8
// pools (168 VGPRs with up to 5 spilled without it, but 2-4 % faster than
// with it)
template <int KVT, int NT>
__host__ __device__ constexpr bool staged_q_in_lds() {
    return staged_waves_per_eu<KVT, NT>() == 3 && KVT != DT_FP8;
}
// LDS bytes of the staged form: two stages, then per wave its query half
// (two tiles x two k steps x 64 lanes x 16 B)
template <int KVT, int QT, int NT>
__host__ __device__ constexpr int staged_lds_bytes(int nw) {
    return 2 * stage_bytes(staged_kvt(KVT, QT)) + (staged_q_in_lds<KVT, NT>() ? nw * NT * 2 * 1024 : 0);
}

template <int KVT, int QT, int BS, int NW, int NT>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(staged_waves_per_eu<KVT, NT>())))
void paged_prefill_staged_kernel(const DecodeArgs a, const int32_t* __restrict__ query_start,
                                 int max_groups) {
    static_assert(NW == 4, "one pool-row quarter of a unit pair per wave");
    constexpr int NSUB = BS / kSubTokens;
    constexpr int R = rows_per_sub(KVT);
    constexpr int64_t SUB = sub_tile_bytes(KVT);
    constexpr int64_t TILE = SUB * NSUB;
    constexpr int SKVT = staged_kvt(KVT, QT);         // what the stages hold
    constexpr bool kThree = staged_waves_per_eu<KVT, NT>() == 3;
    constexpr bool kQLds = staged_q_in_lds<KVT, NT>();
    constexpr int SR = rows_per_sub(SKVT);
    constexpr int SB = stage_bytes(SKVT);
    using Math = MfmaMath<KVT, QT, NT>;
    extern __shared__ float pkv_smem[];
    uint8_t* stages = reinterpret_cast<uint8_t*>(pkv_smem);
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int Hkv = a.num_kv_heads;
    const int kvh = blockIdx.x % Hkv;
    const int item = blockIdx.x / Hkv;               // (sequence rank, group) item
    const int P = (Hkv < 8 && 8 % Hkv == 0) ? 8 / Hkv : 1;
    const int band = item / (P * max_groups);
    const int in_band = item - band * P * max_groups;
    const int bw = min(P, a.num_seqs - band * P);    // sequences in this band
    const int grp = max_groups - 1 - in_band / bw;
    const int s = seq_of_rank(a, band_rank(band, in_band % bw, P, bw), reinterpret_cast<int*>(pkv_smem));
    // the sequence's bounds as scalars (vector loads, since the kernel
    // writes global memory; without this the pair loop and its block-table
    // indexing run as per-lane arithmetic)
    const int q0 = __builtin_amdgcn_readfirstlane(query_start[s]);
    const int q_len = __builtin_amdgcn_readfirstlane(query_start[s + 1]) - q0;
    // Columns: the chunk's (token, head) pairs in order, c = j * G + h, cut
    // into CW-column waves and NW-wave workgroups across token boundaries
    // (no padding columns except at the chunk's end)
    constexpr int CW = 16 * NT;
    const int G = a.group;
    const int ncs = q_len * G;
    const int cg0 = grp * NW * CW;                   // the workgroup's first column
    if (cg0 >= ncs) return;                          // (whole workgroup)
    int ctx = __builtin_amdgcn_readfirstlane(a.context_lens[s]);
    ctx = ctx < a.ctx_cap ? ctx : a.ctx_cap;
    // keys of the workgroup: up to its last column's token
    const int kv_end_g = min(ctx, ctx - q_len + (min(ncs, cg0 + NW * CW) - 1) / G + 1);

    // this wave's columns (it may have none): pairs h0 .. h0 + ncw - 1
    // counted from head 0 of chunk token j0
    const int c0w = cg0 + w * CW;
    const bool has_tile = c0w < ncs;
    const int j0 = has_tile ? c0w / G : 0;
    const int h0 = has_tile ? c0w - j0 * G : 0;
    const int ncw = has_tile ? min(CW, ncs - c0w) : 0;
    const int64_t row0 = (int64_t)q0 + j0;
    Math mt;
    if (has_tile) load_q_cols(mt, a, row0, h0, ncw, kvh, lane);
    const int pos0 = ctx - (q_len - j0);             // position of token j0
    const int kv_end = has_tile ? min(ctx, pos0 + (h0 + ncw - 1) / G + 1) : 0;
    limit_cols(mt, pos0, h0, G);
    mt.begin();
#pragma unroll
    for (int t = 0; t < NT; ++t) mt.m[t] = kNoKeyMax;
    // the scale is applied after the max, which needs it positive: a
    // negative one flips the sign of every query element instead (exact)
    float cs = a.qk_scale_log2;
    if (cs < 0.f) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) mt.qf[t][kk] ^= 0x80008000u;
        cs = -cs;
    }
    // query fragments of k steps 2, 3 to this wave's LDS area (same wave
    // writes and reads them: no barrier)
    const u32x4_t* qhi = nullptr;
    if constexpr (kQLds) {
        u32x4_t* qa = reinterpret_cast<u32x4_t*>(stages + 2 * SB) + w * (NT * 2 * kWave) + lane;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 2; ++j) qa[(2 * t + j) * kWave] = mt.qf[t][2 + j];
        qhi = qa;
    }
    // loop bounds as scalars (the divisions by G above are vector code)
    const int n_pairs_w = __builtin_amdgcn_readfirstlane(kv_end > 0 ? (kv_end + 2 * kSubTokens - 1) / (2 * kSubTokens) : 0);
    const int n_free = __builtin_amdgcn_readfirstlane(pos0 + 1 >= kSubTokens ? (pos0 + 1) / kSubTokens : 0);

    if (kv_end_g > 0) {
        const int n_units = __builtin_amdgcn_readfirstlane((kv_end_g + kSubTokens - 1) / kSubTokens);
        const int n_pairs = (n_units + 1) / 2;
        const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks;
        // wave w fetches K (w < 2) or V (w >= 2) rows of unit A (w even) or B
        const uint8_t* pool = ((w >> 1) ? a.v_cache : a.k_cache) + (int64_t)pool_head(a, kvh) * TILE;
        const int64_t head_stride = (int64_t)a.pool_kv_heads * TILE;
        // unit fetched by this wave for pair p (indices past the last pair
        // repeat it; a missing second unit repeats the last unit)
        auto unit_of = [&](int p) { return min(2 * min(p, n_pairs - 1) + (w & 1), n_units - 1); };
        auto fetch_at = [&](u32x4_t (&r)[R], int p, int pb) {
            if (a.num_blocks > 0 && (unsigned)pb >= (unsigned)a.num_blocks) pb = 0;
            const int u = unit_of(p);
            const u32x4_t* g = reinterpret_cast<const u32x4_t*>(pool + (int64_t)pb * head_stride + (u % NSUB) * SUB) + lane;
#pragma unroll
            for (int i = 0; i < R; ++i) r[i] = g[kWave * i];
        };
        auto fetch = [&](u32x4_t (&r)[R], int p) { fetch_at(r, p, bt_row[unit_of(p) / NSUB]); };
        // block id of pair p as a vector load issued two fetches ahead (a
        // scalar load would be waited for at once, next to its use)
        auto id_load = [&](int p) {
            int z = 0;
            asm volatile("" : "+v"(z));
            return bt_row[unit_of(p) / NSUB + z];
        };
        // store this wave's quarter of pair p into a stage; V rows of tokens
        // at or past the context end are zeroed (they may hold anything, and
        // a zero weight times NaN would still poison the PV sum)
        auto stage_write = [&](u32x4_t (&r)[R], int st, int p) {
            if (w >= 2) {
                const int t0 = kSubTokens * unit_of(p);
                if (t0 + kSubTokens > ctx) {
                    // lane (dim, group g) holds tokens 4g..4g+3 per dim tile
                    const int tb = t0 + 4 * (lane >> 4);
                    if constexpr (KVT == DT_FP8) {
                        const uint32_t mk = (tb + 0 < ctx ? 0x000000ffu : 0u) | (tb + 1 < ctx ? 0x0000ff00u : 0u) |
                                            (tb + 2 < ctx ? 0x00ff0000u : 0u) | (tb + 3 < ctx ? 0xff000000u : 0u);
#pragma unroll
                        for (int i = 0; i < R; ++i) r[i] &= mk;
                    } else {
                        const uint32_t m01 = (tb + 0 < ctx ? 0x0000ffffu : 0u) | (tb + 1 < ctx ? 0xffff0000u : 0u);
                        const uint32_t m23 = (tb + 2 < ctx ? 0x0000ffffu : 0u) | (tb + 3 < ctx ? 0xffff0000u : 0u);
                        const u32x4_t mk = {m01, m23, m01, m23};
#pragma unroll
                        for (int i = 0; i < R; ++i) r[i] &= mk;
                    }
                }
            }
            uint8_t* base = stages + st * SB;
            if constexpr (SKVT != KVT) {
                // fp8 pool widened here, once per pair: row i of K gives
                // 16-bit rows 2i (its dims 0..7 per lane) and 2i + 1; dword d
                // of V row i is dim tile 4i + d, stored as the 16-bit V path
                // stores it
                if (w < 2) {
                    u32x4_t* d = reinterpret_cast<u32x4_t*>(base + (w & 1) * SR * 1024) + lane;
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        d[kWave * (2 * i)] = e4m3x8_to_16<QT>(r[i][0], r[i][1]);
                        d[kWave * (2 * i + 1)] = e4m3x8_to_16<QT>(r[i][2], r[i][3]);
                    }
                } else {
                    u32x2_t* d = reinterpret_cast<u32x2_t*>(base + 2 * SR * 1024) + 2 * lane + (w & 1);
#pragma unroll
                    for (int i = 0; i < R; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q) d[2 * kWave * (4 * i + q)] = e4m3x4_to_16<QT>(r[i][q]);
                }
            } else if (w < 2) {
                // K rows as in the pool: [unit][row][lane]
                u32x4_t* d = reinterpret_cast<u32x4_t*>(base + (w >> 1) * 2 * R * 1024 + (w & 1) * R * 1024) + lane;
#pragma unroll
                for (int i = 0; i < R; ++i) d[kWave * i] = r[i];
            } else {
                // 16-bit V: row i holds dim tiles 2i (dwords 0, 1) and 2i+1
                // (dwords 2, 3); unit A fills the low halves, B the high
                u32x2_t* d = reinterpret_cast<u32x2_t*>(base + 2 * R * 1024) + 2 * lane + (w & 1);
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    d[2 * kWave * (2 * i)] = (u32x2_t){r[i][0], r[i][1]};
                    d[2 * kWave * (2 * i + 1)] = (u32x2_t){r[i][2], r[i][3]};
                }
            }
        };
        auto compute = [&](int p, int st) {
            if (p < n_pairs_w)
                staged_pair<SKVT, QT, kThree, kQLds, !(KVT == DT_FP8 && BS == 32)>(
                    mt, stages + st * SB, 2 * p * kSubTokens, 2 * p + 2 > n_free, cs, lane, qhi);
        };

        // Fetches, stage writes and barriers are unconditional (indices past
        // the last pair repeat it; compute skips pairs the wave does not
        // see), so the load counters the compiler waits on stay static: a
        // stage write waits only for its own pair, not for the one behind.
        if constexpr (kThree) {
            // one pair in flight in registers (three waves per SIMD hide
            // the shorter lead)
            u32x4_t r0[R];
            fetch(r0, 0);
            int id2 = id_load(2);
            stage_write(r0, 0, 0);
            fetch(r0, 1);
            __syncthreads();
            for (int p = 0; p < n_pairs; ++p) {
                compute(p, p & 1);
                stage_write(r0, (p + 1) & 1, p + 1);
                fetch_at(r0, p + 2, __builtin_amdgcn_readfirstlane(id2));
                id2 = id_load(p + 3);
                __syncthreads();
            }
        } else {
            // two pairs in flight in registers
            u32x4_t r0[R], r1[R];
            fetch(r0, 0);
            fetch(r1, 1);
            int id3 = id_load(3), id4 = id_load(4);
            stage_write(r0, 0, 0);
            fetch(r0, 2);
            __syncthreads();
            for (int p = 0; p < n_pairs; p += 2) {
                compute(p, 0);
                stage_write(r1, 1, p + 1);
                fetch_at(r1, p + 3, __builtin_amdgcn_readfirstlane(id3));
                id3 = id_load(p + 5);
                __syncthreads();
                compute(p + 1, 1);
                stage_write(r0, 0, p + 2);
                fetch_at(r0, p + 4, __builtin_amdgcn_readfirstlane(id4));
                id4 = id_load(p + 6);
                __syncthreads();
            }
        }
    }
    if (!has_tile) return;
    // normalise and store this wave's columns (column 16t + (lane & 15) of
    // tile t; lane group g holds dims 16nt + 4g .. +3)
    const int g = lane >> 4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float L = mt.l[t];
        {
            const auto a16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(L), __float_as_uint(L), false, false);
            const float x = __uint_as_float(a16[0]) + __uint_as_float(a16[1]);
            const auto a32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            L = __uint_as_float(a32[0]) + __uint_as_float(a32[1]);
        }
        if (!mt.cvalid[t]) continue;
        // L = 0 only for a token placed before the start of the context
        const float sc = (L > 0.f ? 1.0f / L : 0.f) * a.out_scale;
        const int cl = 16 * t + (lane & 15) + h0;
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out) +
                        ((row0 + cl / G) * a.num_heads + first_head(a, kvh) + cl % G) * kHeadDim + 4 * g;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const f32x4_t o = mt.acc[t][nt];
            const u32x2_t v = {pack2<QT>(o[0] * sc, o[1] * sc), pack2<QT>(o[2] * sc, o[3] * sc)};
            *reinterpret_cast<u32x2_t*>(out + 16 * nt) = v;
        }
    }
}

template <int KVT, int QT, int BS>
static hipError_t launch_prefill_t(const DecodeArgs& a, const int32_t* query_start, int tile_tokens,
                                   int max_tiles, hipStream_t st) {
    if (max_tiles > kWavesPerGroup) {
        // staged form: 16 * NT columns (NT 16-column tiles) per wave, four
        // waves; columns packed across tokens (max_tiles * tile_tokens bounds
        // the longest chunk)
        constexpr int NW = 4;
        constexpr int NT = PKV_PREFILL_TILES_PER_WAVE;
        const int64_t max_cols = (int64_t)max_tiles * tile_tokens * a.group;
        const int groups = (int)((max_cols + NW * 16 * NT - 1) / (NW * 16 * NT));
        const dim3 grid((unsigned)((int64_t)a.num_seqs * groups * a.num_kv_heads));
        hipLaunchKernelGGL((paged_prefill_staged_kernel<KVT, QT, BS, NW, NT>), grid, dim3(NW * kWave),
                           (staged_lds_bytes<KVT, QT, NT>(NW)), st, a, query_start, groups);
        return hipGetLastError();
    }
    if (PKV_PREFILL_WG_NT2 && max_tiles >= 2) {
        // two 16-column tiles per workgroup: its K / V is read once for both
        const int tt = 2 * tile_tokens;
        const int tiles2 = (max_tiles + 1) / 2;
        const size_t lds = std::max(sizeof(float) * merge_lds_floats(kWavesPerGroup, tt * a.group, 32),
                                    sizeof(int) * (kRankSeqsMax + 1));
        const dim3 grid((unsigned)((int64_t)a.num_seqs * tiles2 * a.num_kv_heads));
        if (a.kv_split > 1)
            hipLaunchKernelGGL((paged_prefill_mfma_kernel<KVT, QT, BS, kWavesPerGroup, small_chunk_depth<KVT, 2>(), 2, true>),
                               grid, dim3(kWavesPerGroup * kWave), lds, st, a, query_start, tt, tiles2);
        else
            hipLaunchKernelGGL((paged_prefill_mfma_kernel<KVT, QT, BS, kWavesPerGroup, small_chunk_depth<KVT, 2>(), 2>),
                               grid, dim3(kWavesPerGroup * kWave), lds, st, a, query_start, tt, tiles2);
        return hipGetLastError();
    }
    const size_t lds = std::max(sizeof(float) * merge_lds_floats(kWavesPerGroup, tile_tokens * a.group),
                                sizeof(int) * (kRankSeqsMax + 1));
    const dim3 grid((unsigned)((int64_t)a.num_seqs * max_tiles * a.num_kv_heads));
    if (a.kv_split > 1)
        hipLaunchKernelGGL((paged_prefill_mfma_kernel<KVT, QT, BS, kWavesPerGroup, kDepth, 1, true>), grid,
                           dim3(kWavesPerGroup * kWave), lds, st, a, query_start, tile_tokens, max_tiles);
    else
        hipLaunchKernelGGL((paged_prefill_mfma_kernel<KVT, QT, BS, kWavesPerGroup, kDepth, 1>), grid,
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
