// decode_tokens.hip — token-level virtualisation ("vToken" page, "the core
// idea: token-level virtualisation" and "asynchronous repacking"):
//   - decode through a per-token table: logical token t of sequence s sits
//     at physical slot token_slots[s][t] (block slot / bs, row slot % bs),
//     so tokens evicted from a block leave holes that the table skips;
//   - moving whole tokens between slots (the repacking copy), so survivors
//     can be packed into fewer blocks and the emptied blocks freed, while
//     the table keeps the logical order.
//
// The decode reuses the MFMA math and the wave merge of the block path
// (decode_core.h); only the loads differ: each lane computes the address
// of its own token instead of taking a whole 16-token sub-tile.  K lanes
// hold 16 contiguous bytes of one token (the pool layout's K rows), so a K
// fragment is still four 16-byte loads per lane; V lanes hold 4 tokens of
// one dim, so a lane loads the 16-byte chunk holding each of its 4 tokens'
// values per pool row (16 loads per unit) and picks the token's bytes out
// with byte permutes.  When the table is block-aligned the addresses
// coincide with the block path's.  Repacking exists to return the table to
// that state.  The run-list form below reads whole pool sub-tiles instead
// and skips the rows that are not keys.
#include "decode_core.h"
#include "mfma_math.h"

namespace pkv {

// Byte offset, inside one (block, kv head) tile, of K / V element (row r
// of the block, dim k) — the layout frozen in pagedkv.h.
template <int KVT>
__device__ __forceinline__ int tile_offset_k(int r, int k) {
    constexpr int E = elem_bytes(KVT), n = 2 / E;
    const int c = k >> 3, lane = (r & 15) + 16 * (c & 3), kk = c >> 2, e = k & 7;
    return (r >> 4) * sub_tile_bytes(KVT) + 1024 * (kk / n) + 16 * lane + 8 * E * (kk % n) + E * e;
}
template <int KVT>
__device__ __forceinline__ int tile_offset_v(int r, int k) {
    constexpr int E = elem_bytes(KVT), n = 4 / E;
    const int nt = k >> 4, lane = (k & 15) + 16 * ((r & 15) >> 2), i = r & 3;
    return (r >> 4) * sub_tile_bytes(KVT) + 1024 * (nt / n) + 16 * lane + 4 * E * (nt % n) + E * i;
}

// Load logical unit j of a chunk (tokens 16*unit .. +15) into the block
// path's register fragments.  slot_l: lane l holds the slot of token
// (l & 15) of chunk unit (l >> 4).
template <int KVT, int BS>
__device__ __forceinline__ void gather_unit(UnitRegs<KVT>& u, const uint8_t* kpool,
                                            const uint8_t* vpool, int64_t head_stride,
                                            int32_t slot_l, int j, int lane) {
    constexpr int E = elem_bytes(KVT);
    constexpr int R = rows_per_sub(KVT);
    const int g = lane >> 4;
    // K: this lane's token row, 16 bytes per 1 KiB row
    {
        const int32_t slot = (int32_t)lane_fetch((uint32_t)slot_l, 16 * j + (lane & 15));
        const int32_t pb = slot / BS, rp = slot - pb * BS;
        const uint8_t* base = kpool + (int64_t)pb * head_stride + (rp >> 4) * sub_tile_bytes(KVT) +
                              16 * ((rp & 15) + 16 * g);
#pragma unroll
        for (int r = 0; r < R; ++r) u.k[r] = *reinterpret_cast<const u32x4_t*>(base + 1024 * r);
    }
    // V: tokens 4g .. 4g+3 of dim d = lane & 15 for each dim tile nt.  A
    // source token's values for dim d sit in one 16-byte chunk per pool row
    // (row nt / n, lane d + 16 (row-in-block % 16) / 4), shared with the
    // three other tokens of its group of 4: load that chunk whole for each
    // of the 4 tokens and row, then pick the token's bytes out of it.
    const int d = lane & 15;
    const u32x4_t* vc[4];
    int sub[4];                                   // token's place in its group of 4
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t slot = (int32_t)lane_fetch((uint32_t)slot_l, 16 * j + 4 * g + i);
        const int32_t pb = slot / BS, rp = slot - pb * BS;
        vc[i] = reinterpret_cast<const u32x4_t*>(vpool + (int64_t)pb * head_stride + (rp >> 4) * sub_tile_bytes(KVT) +
                                                 16 * (d + 16 * ((rp & 15) >> 2)));
        sub[i] = rp & 3;
    }
    u32x4_t c[4][R];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) c[i][r] = vc[i][kWave * r];
    if constexpr (E == 2) {
        // chunk dwords: (nt even: tokens 0,1 | 2,3), (nt odd: 0,1 | 2,3);
        // token i's value is half sub & 1 of dword sub >> 1 (+ 2 if odd)
        uint32_t sel[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t a0 = 2 * (sub[2 * h] & 1), a1 = 4 + 2 * (sub[2 * h + 1] & 1);
            sel[h] = a0 | ((a0 + 1) << 8) | (a1 << 16) | ((a1 + 1) << 24);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int odd = 0; odd < 2; ++odd)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t lo = (sub[2 * h] >> 1) ? c[2 * h][r][2 * odd + 1] : c[2 * h][r][2 * odd];
                    const uint32_t hi = (sub[2 * h + 1] >> 1) ? c[2 * h + 1][r][2 * odd + 1] : c[2 * h + 1][r][2 * odd];
                    u.v[r][2 * odd + h] = __builtin_amdgcn_perm(hi, lo, sel[h]);
                }
    } else {
        // fp8: dword q of a chunk is dim tile 4 row + q, byte = token
        const uint32_t s01 = sub[0] | ((4 + sub[1]) << 8) | (0x0c0cu << 16);   // bytes 2, 3: zero
        const uint32_t s23 = (0x0c0cu) | (sub[2] << 16) | ((4 + sub[3]) << 24);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                u.v[r][q] = __builtin_amdgcn_perm(c[1][r][q], c[0][r][q], s01) |
                            __builtin_amdgcn_perm(c[3][r][q], c[2][r][q], s23);
    }
}

// One workgroup per (sequence, kv head); wave w takes units w, w + NW, ...
// in chunks of 4 (one slot load per lane per chunk, then four units of
// loads in flight), no context split.
// only_marked (a run list's counts, or null): decode only the sequences
// the run list marked for the gather (negative count), leave the others to
// the run-list decode.
template <int KVT, int QT, int BS, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU)))
void paged_decode_tokens_kernel(const DecodeArgs a, const int32_t* __restrict__ token_slots,
                                int max_tokens, const int32_t* __restrict__ only_marked) {
    extern __shared__ float pkv_smem[];
    constexpr int CH = 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = blockIdx.x / a.num_kv_heads;
    const int kvh = blockIdx.x - s * a.num_kv_heads;
    if (only_marked != nullptr && only_marked[s] >= 0) return;
    const int G = a.group;
    const QueryTile qt{s, 1, 1};
    MfmaMath<KVT, QT> mt;
    mt.load_q(a, qt, kvh, lane);
    int ctx = a.context_lens[s];
    ctx = ctx < max_tokens ? ctx : max_tokens;
    if (ctx <= 0) {
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)s * a.num_heads + first_head(a, kvh)) * kHeadDim;
        for (int e = threadIdx.x; e < heads_of(a, kvh) * kHeadDim; e += NW * kWave) out[e] = 0;
        return;
    }
    mt.limit(ctx - 1, G, lane);
    const int n_units = (ctx + kSubTokens - 1) / kSubTokens;
    int* done = reinterpret_cast<int*>(pkv_smem);
    if (threadIdx.x == 0) *done = 0;
    __syncthreads();
    mt.begin();

    constexpr int64_t TILE = (int64_t)sub_tile_bytes(KVT) * (BS / kSubTokens);
    const uint8_t* kpool = a.k_cache + (int64_t)pool_head(a, kvh) * TILE;
    const uint8_t* vpool = a.v_cache + (int64_t)pool_head(a, kvh) * TILE;
    const int64_t head_stride = (int64_t)a.pool_kv_heads * TILE;
    const int32_t* row = token_slots + (int64_t)s * max_tokens;
    const int32_t slot_cap = a.num_blocks * BS;   // slots in [BS, slot_cap) are real
    const int n_my = w < n_units ? (n_units - w + NW - 1) / NW : 0;
    for (int c0 = 0; c0 < n_my; c0 += CH) {
        const int nc = min(CH, n_my - c0);
        // lane l: slot of token (l & 15) of chunk unit min(l >> 4, nc - 1);
        // tokens past the context read the last token (masked later)
        const int ul = w + NW * (c0 + min(lane >> 4, nc - 1));
        const int tok = min(16 * ul + (lane & 15), ctx - 1);
        int32_t slot = row[tok];
        if ((unsigned)(slot - BS) >= (unsigned)(slot_cap - BS)) slot = BS;   // outside the pool: block 1, row 0
        UnitRegs<KVT> buf[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j)
            gather_unit<KVT, BS>(buf[j], kpool, vpool, head_stride, slot, min(j, nc - 1), lane);
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (j < nc)
                mt.unit(buf[j], (w + NW * (c0 + j)) * kSubTokens, ctx, a.qk_scale_log2, lane);
    }
    park_and_store<MfmaMath<KVT, QT>, QT, NW>(a, pkv_smem, mt, s, 0, kvh, lane, w, qt, G, true);
}

template <int KVT, int QT, int BS>
static hipError_t launch_tokens_t(const DecodeArgs& a, const int32_t* token_slots, int max_tokens,
                                  const int32_t* only_marked, hipStream_t st) {
    const size_t lds = sizeof(float) * merge_lds_floats(kWavesPerGroup, a.group);
    hipLaunchKernelGGL((paged_decode_tokens_kernel<KVT, QT, BS, kWavesPerGroup>),
                       dim3(a.num_seqs * a.num_kv_heads), dim3(kWavesPerGroup * kWave), lds, st, a,
                       token_slots, max_tokens, only_marked);
    return hipGetLastError();
}

template <int KVT, int QT>
static hipError_t launch_tokens_bs(const DecodeArgs& a, int bs, const int32_t* ts, int mt,
                                   const int32_t* om, hipStream_t st) {
    return bs == 16 ? launch_tokens_t<KVT, QT, 16>(a, ts, mt, om, st)
                    : launch_tokens_t<KVT, QT, 32>(a, ts, mt, om, st);
}

hipError_t launch_decode_tokens(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                                const int32_t* token_slots, int max_tokens, const int32_t* only_marked,
                                hipStream_t st) {
    if (a.num_seqs == 0) return hipSuccess;
    const int32_t* om = only_marked;
    if (q_dtype == DT_BF16) {
        if (kv_dtype == DT_BF16) return launch_tokens_bs<DT_BF16, DT_BF16>(a, block_size, token_slots, max_tokens, om, st);
        return launch_tokens_bs<DT_FP8, DT_BF16>(a, block_size, token_slots, max_tokens, om, st);
    }
    if (kv_dtype == DT_FP16) return launch_tokens_bs<DT_FP16, DT_FP16>(a, block_size, token_slots, max_tokens, om, st);
    return launch_tokens_bs<DT_FP8, DT_FP16>(a, block_size, token_slots, max_tokens, om, st);
}

// ------------------------------------------------------------ run lists --
// The same attention over the pool's sub-tiles instead of single tokens.
// Tokens evicted at random leave survivors in nearly every 64-byte line of
// every tile, so the token gather above fetches about the whole pool
// anyway, with 20 loads per lane and unit where the block path issues 8.
// A run list reads each sub-tile that holds survivors whole, with the
// block path's loads, and skips the rows that are not the sequence's keys
// (their weight is 0 and their V zeroed, as for the tail of a context).
//
// Run list of sequence s: entries e = 0 .. n_s - 1, each a pool sub-tile
// (global index slot / 16: block slot / BS, sub-tile (slot % BS) / 16) and
// a 16-bit mask of the rows that are keys.  An entry takes consecutive
// table entries t, t + 1, ... while they lie in one sub-tile at strictly
// increasing rows (at most 16); any other step starts a new entry, so a
// slot listed twice counts twice, as in the table.  Table entries outside
// [BS, num_blocks * BS) read slot BS (block 1, row 0), as the token gather
// does.
//
// One workgroup per sequence walks its table in tiles of kRunTile entries:
// each thread flags which of its kRunPer entries start an entry, a
// workgroup scan numbers the starts, every entry ORs its row bit into its
// entry's mask in LDS, and the starts write their entries.  The tile's last
// entry may go on in the next tile: it stays open (sub-tile and mask in
// registers) until a later start or the end closes it.  Also writes
// lens16[s] = 16 n_s, the run list's length in tokens, from which the plan
// kernel orders the decode longest first.  With min_keys > 0, a sequence
// whose list holds fewer than min_keys keys per entry on average (sparse
// survivors: whole sub-tiles would be mostly skipped rows) is marked for
// the token gather instead: counts[s] = -1 - n_s, lens16[s] = 0.
constexpr int kRunThreads = 256;
constexpr int kRunPer = 4;
constexpr int kRunTile = kRunThreads * kRunPer;

__global__ __launch_bounds__(kRunThreads) void token_runs_kernel(const int32_t* __restrict__ token_slots,
                                                                 int max_tokens,
                                                                 const int32_t* __restrict__ context_lens,
                                                                 int block_size, int num_blocks, int min_keys,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ lens16,
                                                                 int2* __restrict__ entries) {
    constexpr int kWaves = kRunThreads / kWave;
    __shared__ uint32_t tmask[kRunTile + 1];      // [0]: the entry open from earlier tiles
    __shared__ int wave_total[kWaves];
    __shared__ int last_sub;
    const int s = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    int ctx = context_lens[s];
    ctx = ctx < 0 ? 0 : (ctx < max_tokens ? ctx : max_tokens);
    const int32_t* row = token_slots + (int64_t)s * max_tokens;
    int2* out = entries + (int64_t)s * max_tokens;
    const int32_t cap = num_blocks * block_size;
    auto slot_at = [&](int t) {
        const int32_t v = row[t];
        return (unsigned)(v - block_size) >= (unsigned)(cap - block_size) ? block_size : v;
    };
    // uniform state: entries written so far; the open entry (index n_done)
    int n_done = 0, open_sub = 0;
    uint32_t open_mask = 0;
    bool open = false;
    for (int t0 = 0; t0 < ctx; t0 += kRunTile) {
        const bool last = t0 + kRunTile >= ctx;
        const int tb = t0 + kRunPer * tid;
        int32_t v[kRunPer];
        bool st[kRunPer];
        int32_t prev = (tb > 0 && tb <= ctx) ? slot_at(tb - 1) : 0;
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < kRunPer; ++k) {
            const int t = tb + k;
            const bool valid = t < ctx;
            v[k] = valid ? slot_at(t) : 0;
            st[k] = valid && (t == 0 || (v[k] >> 4) != (prev >> 4) || (v[k] & 15) <= (prev & 15));
            prev = v[k];
            cnt += st[k] ? 1 : 0;
        }
        // starts before this thread's (thread order = table order) and in all
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane == kWave - 1) wave_total[wid] = incl;
        __syncthreads();
        int before = incl - cnt, T = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int x = wave_total[w];
            before += w < wid ? x : 0;
            T += x;
        }
        for (int j = tid; j <= T; j += kRunThreads) tmask[j] = (j == 0 && open) ? open_mask : 0u;
        __syncthreads();
        // entry of each table entry, counted in the tile: -1 = the open one
        int local = before - 1;
#pragma unroll
        for (int k = 0; k < kRunPer; ++k) {
            if (st[k]) ++local;
            if (tb + k < ctx) atomicOr(&tmask[local + 1], 1u << (v[k] & 15));
        }
        __syncthreads();
        const int base_idx = n_done + (open ? 1 : 0);
        local = before - 1;
#pragma unroll
        for (int k = 0; k < kRunPer; ++k) {
            if (st[k]) {
                ++local;
                // closed by a later start in the tile, or by the end
                if (local < T - 1 || last) out[base_idx + local] = make_int2(v[k] >> 4, (int)tmask[local + 1]);
                if (local == T - 1) last_sub = v[k] >> 4;
            }
        }
        if (tid == 0 && open && (T > 0 || last)) out[n_done] = make_int2(open_sub, (int)tmask[0]);
        __syncthreads();
        if (T > 0) {
            open_sub = last_sub;
            open_mask = tmask[T];
            n_done = base_idx + T - 1;
            open = true;
        } else {
            open_mask = tmask[0];
        }
        __syncthreads();                          // tmask and last_sub are reused
    }
    if (tid == 0) {
        const int n = open ? n_done + 1 : 0;
        const bool sparse = min_keys > 0 && n > 0 && (int64_t)ctx < (int64_t)min_keys * n;
        counts[s] = sparse ? -1 - n : n;
        lens16[s] = sparse ? 0 : 16 * n;
    }
}

hipError_t launch_token_runs(const int32_t* token_slots, int max_tokens, const int32_t* context_lens,
                             int num_seqs, int block_size, int num_blocks, int min_keys, int32_t* counts,
                             int32_t* lens16, int32_t* plan, int2* entries, hipStream_t st) {
    if (num_seqs == 0) return hipSuccess;
    hipLaunchKernelGGL(token_runs_kernel, dim3(num_seqs), dim3(kRunThreads), 0, st, token_slots, max_tokens,
                       context_lens, block_size, num_blocks, min_keys, counts, lens16, entries);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // longest run list first: one item per sequence (a partition as long
    // as the longest list), sized in 16-token units
    return launch_plan(lens16, num_seqs, 16 * max_tokens, kSubTokens, max_tokens > 0 ? max_tokens : 1, plan, st);
}

// Attention over a run list: one workgroup per (sequence, entry head); wave
// w takes entries w, w + NW, ... with the block path's ring of whole
// sub-tile loads, DEPTH in flight.  A block-aligned table gives the block
// path's result bit for bit (four waves, unsplit context).  PLAIN:
// cache-allocating loads, for kv heads split over several entry heads.
template <int KVT, int QT, int BS, int NW, int DEPTH, bool PLAIN>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU)))
void paged_decode_runs_kernel(const DecodeArgs a, const int32_t* __restrict__ counts,
                              const int2* __restrict__ entries, int max_tokens) {
    extern __shared__ float pkv_smem[];
    constexpr int NSUB = BS / kSubTokens;
    constexpr int64_t SUB = sub_tile_bytes(KVT);
    constexpr int64_t TILE = SUB * NSUB;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the plan's sequences (longest run list first) in groups of 8, each
    // group expanded over the entry heads with the heads of a sequence on
    // one XCD, as the block path's grid form
    const int per_group = 8 * a.num_kv_heads;
    const int grp = blockIdx.x / per_group;
    const int rem = blockIdx.x - grp * per_group;
    const int item = grp * 8 + (rem & 7);
    const int kvh = rem >> 3;
    if (item >= a.num_seqs) return;
    const int s = (int)((uint32_t)a.plan[kPlanHeader + item] >> 16);
    if (s >= a.num_seqs) return;              // a list built for other sizes
    const QueryTile qt{s, 1, 1};
    // entry i of this sequence as one 64-bit load: (sub-tile, rows)
    const uint64_t* ent = reinterpret_cast<const uint64_t*>(entries) + (int64_t)s * max_tokens;
    auto entry = [&](int i) -> uint64_t { return max_tokens > 0 ? ent[min(i, max_tokens - 1)] : 0ull; };
    // this wave's first 64 entries load beside the queries and the count
    const uint64_t e0 = entry(w + NW * lane);
    MfmaMath<KVT, QT> mt;
    mt.load_q(a, qt, kvh, lane);
    const int n_units = __builtin_amdgcn_readfirstlane(counts[s]);
    if (n_units < 0) return;                  // marked for the token gather
    if (n_units == 0) {
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)s * a.num_heads + first_head(a, kvh)) * kHeadDim;
        for (int e = threadIdx.x; e < heads_of(a, kvh) * kHeadDim; e += NW * kWave) out[e] = 0;
        return;
    }
    int* done = reinterpret_cast<int*>(pkv_smem);
    if (threadIdx.x == 0) *done = 0;
    __syncthreads();
    mt.begin();

    const uint8_t* kpool = a.k_cache + (int64_t)pool_head(a, kvh) * TILE;
    const uint8_t* vpool = a.v_cache + (int64_t)pool_head(a, kvh) * TILE;
    const int64_t head_stride = (int64_t)a.pool_kv_heads * TILE;
    const int n_my = w < n_units ? (n_units - w + NW - 1) / NW : 0;
    for (int c0 = 0; c0 < n_my; c0 += kWave) {
        const int nc = min(kWave, n_my - c0);
        const uint64_t e = c0 == 0 ? e0 : entry(w + NW * (c0 + lane));
        const int e_sub = (int)(uint32_t)e, e_rows = (int)(uint32_t)(e >> 32);
        auto unit_offset = [&](int j) -> int64_t {
            const int sub = __builtin_amdgcn_readlane(e_sub, j);
            int pb = sub / NSUB;
            if ((unsigned)pb >= (unsigned)a.num_blocks) pb = 0;
            return (int64_t)pb * head_stride + (sub - (sub / NSUB) * NSUB) * SUB;
        };
        auto rows_of = [&](int j) { return (uint32_t)__builtin_amdgcn_readlane(e_rows, j); };
        UnitRegs<KVT> buf[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int64_t off = unit_offset(min(d, nc - 1));
            load_unit<KVT, kHeadDim, PLAIN>(buf[d], kpool + off, vpool + off, lane);
        }
        int i = 0;
        for (; i + 2 * DEPTH <= nc; i += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                mt.unit_rows(buf[d], rows_of(i + d), a.qk_scale_log2, lane);
                const int64_t off = unit_offset(i + d + DEPTH);
                load_unit<KVT, kHeadDim, PLAIN>(buf[d], kpool + off, vpool + off, lane);
            }
        }
        const int refills = nc - i - DEPTH;       // < DEPTH; may be negative
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            if (i + d < nc) {
                mt.unit_rows(buf[d], rows_of(i + d), a.qk_scale_log2, lane);
                if (d < refills) {
                    const int64_t off = unit_offset(i + d + DEPTH);
                    load_unit<KVT, kHeadDim, PLAIN>(buf[d], kpool + off, vpool + off, lane);
                }
            }
        }
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d)
            if (d < refills) mt.unit_rows(buf[d], rows_of(i + DEPTH + d), a.qk_scale_log2, lane);
    }
    park_and_store<MfmaMath<KVT, QT>, QT, NW>(a, pkv_smem, mt, s, 0, kvh, lane, w, qt, a.group, true);
}

template <int KVT, int QT, int BS, int NW, int DP>
static hipError_t launch_runs_nw(const DecodeArgs& a, const int32_t* counts, const int2* entries,
                                 int max_tokens, hipStream_t st) {
    const size_t lds = sizeof(float) * merge_lds_floats(NW, a.group);
    const dim3 grid((unsigned)(((int64_t)a.num_seqs + 7) / 8 * 8 * a.num_kv_heads)), block(NW * kWave);
    if (a.kv_split > 1)
        hipLaunchKernelGGL((paged_decode_runs_kernel<KVT, QT, BS, NW, DP, true>), grid, block, lds,
                           st, a, counts, entries, max_tokens);
    else
        hipLaunchKernelGGL((paged_decode_runs_kernel<KVT, QT, BS, NW, DP, false>), grid, block, lds,
                           st, a, counts, entries, max_tokens);
    return hipGetLastError();
}

// Waves per workgroup as the block path's partition kernel on unsplit
// contexts: eight for 16-bit pools (a sequence's list streams in half the
// time, so the end of the launch is shorter), four with one sub-tile in
// flight for fp8.
template <int KVT, int QT, int BS>
static hipError_t launch_runs_t(const DecodeArgs& a, const int32_t* counts, const int2* entries,
                                int max_tokens, hipStream_t st) {
    if constexpr (KVT == DT_FP8)
        return launch_runs_nw<KVT, QT, BS, kWavesPerGroup, 1>(a, counts, entries, max_tokens, st);
    else
        return launch_runs_nw<KVT, QT, BS, 2 * kWavesPerGroup, kDepth>(a, counts, entries, max_tokens, st);
}

template <int KVT, int QT>
static hipError_t launch_runs_bs(const DecodeArgs& a, int bs, const int32_t* c, const int2* e, int mt,
                                 hipStream_t st) {
    return bs == 16 ? launch_runs_t<KVT, QT, 16>(a, c, e, mt, st) : launch_runs_t<KVT, QT, 32>(a, c, e, mt, st);
}

hipError_t launch_decode_runs(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                              const int32_t* counts, const int2* entries, int max_tokens, hipStream_t st) {
    if (a.num_seqs == 0) return hipSuccess;
    if (q_dtype == DT_BF16) {
        if (kv_dtype == DT_BF16) return launch_runs_bs<DT_BF16, DT_BF16>(a, block_size, counts, entries, max_tokens, st);
        return launch_runs_bs<DT_FP8, DT_BF16>(a, block_size, counts, entries, max_tokens, st);
    }
    if (kv_dtype == DT_FP16) return launch_runs_bs<DT_FP16, DT_FP16>(a, block_size, counts, entries, max_tokens, st);
    return launch_runs_bs<DT_FP8, DT_FP16>(a, block_size, counts, entries, max_tokens, st);
}

// ------------------------------------------------------------ move tokens --
// Two passes so that every source is read before any destination is
// written (moves may chain or swap): gather each moved token's K and V rows
// (all kv heads) of every layer into scratch, then scatter them.  Workgroup
// (move, layer, K or V); a thread per element.  A move naming a slot outside
// [BS, num_blocks * BS) is skipped by both passes.

constexpr int kMoveThreads = 256;
constexpr int kMoveLayers = 64;

struct MoveArgs {
    uint8_t* k[kMoveLayers];
    uint8_t* v[kMoveLayers];
    const int32_t* moves;
    uint8_t* scratch;        // [move][layer][K,V][H_kv * 128 elements]
    int32_t num_moves;
    int32_t num_layers;      // layers in this launch
    int32_t layer0;          // first layer of this launch (scratch index)
    int32_t total_layers;
    int32_t num_kv_heads;
    int32_t num_blocks;
};

template <int KVT, int BS, bool SCATTER>
__global__ __launch_bounds__(kMoveThreads) void move_tokens_kernel(const MoveArgs a) {
    constexpr int E = elem_bytes(KVT);
    constexpr int64_t TILE = (int64_t)sub_tile_bytes(KVT) * (BS / kSubTokens);
    const int mv = blockIdx.x, layer = blockIdx.y, is_v = blockIdx.z;
    const int32_t src = a.moves[2 * mv], dst = a.moves[2 * mv + 1];
    const int32_t cap = a.num_blocks * BS;
    if ((unsigned)(src - BS) >= (unsigned)(cap - BS) || (unsigned)(dst - BS) >= (unsigned)(cap - BS)) return;
    const int32_t slot = SCATTER ? dst : src;
    const int32_t pb = slot / BS, r = slot - pb * BS;
    uint8_t* pool = is_v ? a.v[layer] : a.k[layer];
    const int per = a.num_kv_heads * kHeadDim;
    uint8_t* tmp = a.scratch + (((int64_t)mv * a.total_layers + a.layer0 + layer) * 2 + is_v) * per * E;
    for (int e = threadIdx.x; e < per; e += kMoveThreads) {
        const int g = e / kHeadDim, k = e - g * kHeadDim;
        const int64_t off = ((int64_t)pb * a.num_kv_heads + g) * TILE +
                            (is_v ? tile_offset_v<KVT>(r, k) : tile_offset_k<KVT>(r, k));
        if constexpr (E == 2) {
            uint16_t* p = reinterpret_cast<uint16_t*>(pool + off);
            uint16_t* t = reinterpret_cast<uint16_t*>(tmp) + e;
            if (SCATTER) *p = *t; else *t = *p;
        } else {
            if (SCATTER) pool[off] = tmp[e]; else tmp[e] = pool[off];
        }
    }
}

template <int KVT, int BS>
static hipError_t launch_moves_t(MoveArgs a, void* const* kl, void* const* vl, hipStream_t st) {
    for (int pass = 0; pass < 2; ++pass) {
        for (int l0 = 0; l0 < a.total_layers; l0 += kMoveLayers) {
            const int nl = a.total_layers - l0 < kMoveLayers ? a.total_layers - l0 : kMoveLayers;
            for (int i = 0; i < nl; ++i) {
                a.k[i] = static_cast<uint8_t*>(kl[l0 + i]);
                a.v[i] = static_cast<uint8_t*>(vl[l0 + i]);
            }
            a.layer0 = l0;
            a.num_layers = nl;
            const dim3 grid(a.num_moves, nl, 2);
            if (pass == 0)
                hipLaunchKernelGGL((move_tokens_kernel<KVT, BS, false>), grid, dim3(kMoveThreads), 0, st, a);
            else
                hipLaunchKernelGGL((move_tokens_kernel<KVT, BS, true>), grid, dim3(kMoveThreads), 0, st, a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// ---------------------------------------------------------- repack blocks --
// Whole-block rebuild after an eviction: destination unit (16 rows of a
// tile's block) gets its K and V sub-tiles assembled from the rows' source
// slots with the same per-token gather as the token-table decode, then
// stored whole (16-byte stores of complete pool rows: no partial writes).
// A repack is a compaction: the survivor that lands in row q comes from a
// position >= q, so the sources of a unit never lie in rows that an earlier
// unit of the chain writes, but they may lie in rows a later unit writes.
// Workgroup (chain, layer, kv head): its four waves take the chain's units in
// rounds of 4 x CH (wave w gathers units w CH .. w CH + CH - 1 of the round
// into registers), waits for them and meets the barrier, then every wave
// stores its units: every store follows the gathers of all units up to its
// own.  The chains of one call touch disjoint blocks.

struct RepackArgs {
    uint8_t* k[kMoveLayers];
    uint8_t* v[kMoveLayers];
    const int32_t* tiles;          // [tile][1 + bs]: destination block, source slot per row
    const int32_t* chain_offsets;  // [num_chains + 1]
    int32_t num_kv_heads;
    int32_t num_blocks;
};

#ifndef PKV_REPACK_UNITS
#define PKV_REPACK_UNITS 4
#endif

template <int KVT, int BS>
__global__ __launch_bounds__(kMoveThreads) void repack_blocks_kernel(const RepackArgs a) {
    constexpr int NSUB = BS / kSubTokens;
    constexpr int R = rows_per_sub(KVT);
    constexpr int64_t SUB = sub_tile_bytes(KVT);
    constexpr int64_t TILE = SUB * NSUB;
    constexpr int CH = PKV_REPACK_UNITS;   // units one wave gathers per round
    constexpr int NW = kMoveThreads / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int layer = blockIdx.y;
    const int h = blockIdx.z;
    const int t0 = a.chain_offsets[blockIdx.x];
    const int n_units = (a.chain_offsets[blockIdx.x + 1] - t0) * NSUB;
    if (n_units <= 0) return;                      // (whole workgroup)
    const int32_t cap = a.num_blocks * BS;
    const int64_t head_stride = (int64_t)a.num_kv_heads * TILE;
    const uint8_t* kp = a.k[layer] + (int64_t)h * TILE;
    const uint8_t* vp = a.v[layer] + (int64_t)h * TILE;
    for (int r0 = 0; r0 < n_units; r0 += NW * CH) {
        const int c0 = r0 + w * CH;                // this wave's first unit
        const int nc = max(0, min(CH, n_units - c0));
        // lane l: row l % 16 of unit c0 + min(l / 16, nc - 1) (lanes past the
        // wave's units repeat its last one; a wave with none repeats the
        // chain's last unit); a source outside the pool leaves the row as it
        // is (reads its own slot)
        const int un = nc > 0 ? c0 + min(lane >> 4, nc - 1) : n_units - 1;
        const int32_t* tile = a.tiles + (int64_t)(t0 + un / NSUB) * (1 + BS);
        const int32_t dst_block = tile[0];
        const int row = (un % NSUB) * kSubTokens + (lane & 15);
        int32_t slot = tile[1 + row];
        if ((unsigned)(slot - BS) >= (unsigned)(cap - BS)) slot = dst_block * BS + row;
        const bool dst_ok = (unsigned)(dst_block - 1) < (unsigned)(a.num_blocks - 1);
        if (!dst_ok) slot = BS;   // (unit skipped below; any valid slot)
        UnitRegs<KVT> buf[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j)
            gather_unit<KVT, BS>(buf[j], kp, vp, head_stride, slot, max(0, min(j, nc - 1)), lane);
        // Every gather of the round complete (data in registers) before any
        // wave stores.  The empty asm ties each gathered register, so the
        // loads can neither stay outstanding at the barrier nor be sunk
        // below it into the store branch (the compiler did sink them there,
        // racing with the other waves' stores, without this).
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
            for (int r = 0; r < R; ++r) asm volatile("" : "+v"(buf[j].k[r]), "+v"(buf[j].v[r]));
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if (j >= nc) continue;
            const int uj = c0 + j;
            const int32_t db = __builtin_amdgcn_readlane(dst_block, 16 * j);
            if ((unsigned)(db - 1) >= (unsigned)(a.num_blocks - 1)) continue;
            const int64_t off = (int64_t)db * head_stride + (int64_t)h * TILE + (uj % NSUB) * SUB + 16 * lane;
            u32x4_t* kd = reinterpret_cast<u32x4_t*>(a.k[layer] + off);
            u32x4_t* vd = reinterpret_cast<u32x4_t*>(a.v[layer] + off);
            // non-temporal: the rebuilt rows are not read again here
#pragma unroll
            for (int r = 0; r < R; ++r) __builtin_nontemporal_store(buf[j].k[r], kd + kWave * r);
#pragma unroll
            for (int r = 0; r < R; ++r) __builtin_nontemporal_store(buf[j].v[r], vd + kWave * r);
        }
        // no barrier here: the next round's sources lie at or past its own
        // rows, beyond every row this round writes
    }
}

template <int KVT, int BS>
static hipError_t launch_repack_t(RepackArgs a, void* const* kl, void* const* vl, int num_layers,
                                  int num_chains, hipStream_t st) {
    for (int l0 = 0; l0 < num_layers; l0 += kMoveLayers) {
        const int nl = num_layers - l0 < kMoveLayers ? num_layers - l0 : kMoveLayers;
        for (int i = 0; i < nl; ++i) {
            a.k[i] = static_cast<uint8_t*>(kl[l0 + i]);
            a.v[i] = static_cast<uint8_t*>(vl[l0 + i]);
        }
        hipLaunchKernelGGL((repack_blocks_kernel<KVT, BS>), dim3(num_chains, nl, a.num_kv_heads),
                           dim3(kMoveThreads), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_repack_blocks(void* const* k_layers, void* const* v_layers, int num_layers,
                                int num_blocks, int num_kv_heads, int block_size, int kv_dtype,
                                const int32_t* tiles, const int32_t* chain_offsets, int num_chains,
                                hipStream_t st) {
    if (num_chains == 0 || num_layers == 0) return hipSuccess;
    RepackArgs a{};
    a.tiles = tiles;
    a.chain_offsets = chain_offsets;
    a.num_kv_heads = num_kv_heads;
    a.num_blocks = num_blocks;
    if (kv_dtype == DT_FP8)
        return block_size == 16 ? launch_repack_t<DT_FP8, 16>(a, k_layers, v_layers, num_layers, num_chains, st)
                                : launch_repack_t<DT_FP8, 32>(a, k_layers, v_layers, num_layers, num_chains, st);
    return block_size == 16 ? launch_repack_t<DT_BF16, 16>(a, k_layers, v_layers, num_layers, num_chains, st)
                            : launch_repack_t<DT_BF16, 32>(a, k_layers, v_layers, num_layers, num_chains, st);
}

hipError_t launch_move_tokens(void* const* k_layers, void* const* v_layers, int num_layers,
                              int num_blocks, int num_kv_heads, int block_size, int kv_dtype,
                              const int32_t* moves, int num_moves, void* scratch, hipStream_t st) {
    if (num_moves == 0 || num_layers == 0) return hipSuccess;
    MoveArgs a{};
    a.moves = moves;
    a.scratch = static_cast<uint8_t*>(scratch);
    a.num_moves = num_moves;
    a.total_layers = num_layers;
    a.num_kv_heads = num_kv_heads;
    a.num_blocks = num_blocks;
    if (kv_dtype == DT_FP8)
        return block_size == 16 ? launch_moves_t<DT_FP8, 16>(a, k_layers, v_layers, st)
                                : launch_moves_t<DT_FP8, 32>(a, k_layers, v_layers, st);
    return block_size == 16 ? launch_moves_t<DT_BF16, 16>(a, k_layers, v_layers, st)
                            : launch_moves_t<DT_BF16, 32>(a, k_layers, v_layers, st);
}

}  // namespace pkv
