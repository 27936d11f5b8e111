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
// that state.
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
template <int KVT, int QT, int BS, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PKV_WAVES_PER_EU)))
void paged_decode_tokens_kernel(const DecodeArgs a, const int32_t* __restrict__ token_slots,
                                int max_tokens) {
    extern __shared__ float pkv_smem[];
    constexpr int CH = 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = blockIdx.x / a.num_kv_heads;
    const int kvh = blockIdx.x - s * a.num_kv_heads;
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
                                  hipStream_t st) {
    const size_t lds = sizeof(float) * merge_lds_floats(kWavesPerGroup, a.group);
    hipLaunchKernelGGL((paged_decode_tokens_kernel<KVT, QT, BS, kWavesPerGroup>),
                       dim3(a.num_seqs * a.num_kv_heads), dim3(kWavesPerGroup * kWave), lds, st, a,
                       token_slots, max_tokens);
    return hipGetLastError();
}

template <int KVT, int QT>
static hipError_t launch_tokens_bs(const DecodeArgs& a, int bs, const int32_t* ts, int mt,
                                   hipStream_t st) {
    return bs == 16 ? launch_tokens_t<KVT, QT, 16>(a, ts, mt, st) : launch_tokens_t<KVT, QT, 32>(a, ts, mt, st);
}

hipError_t launch_decode_tokens(const DecodeArgs& a, int q_dtype, int kv_dtype, int block_size,
                                const int32_t* token_slots, int max_tokens, hipStream_t st) {
    if (a.num_seqs == 0) return hipSuccess;
    if (q_dtype == DT_BF16) {
        if (kv_dtype == DT_BF16) return launch_tokens_bs<DT_BF16, DT_BF16>(a, block_size, token_slots, max_tokens, st);
        return launch_tokens_bs<DT_FP8, DT_BF16>(a, block_size, token_slots, max_tokens, st);
    }
    if (kv_dtype == DT_FP16) return launch_tokens_bs<DT_FP16, DT_FP16>(a, block_size, token_slots, max_tokens, st);
    return launch_tokens_bs<DT_FP8, DT_FP16>(a, block_size, token_slots, max_tokens, st);
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
