// cache_write.h — writing one token's K and V row of one kv head into its
// pool slot: the body of reshape_and_cache, shared with the decode kernels
// that append the new token themselves.
//
// Pages: vToken page (gotosocial.chinng-lab-srv.dev) "KV cache basics" —
// each decode step appends only the new token's key and value; "LLM
// inference basics and vLLM internals" §4 — a token's slot is its physical
// block times block_size plus its offset in the block.
#pragma once
#include "pkv_device.h"

namespace pkv {

// One token's K and V row of one kv head (D elements of the source type),
// held by one wave: lane l owns dims k0 = 2l + 128 i and k0 + 1, as two
// packed 16-bit values per row and i.
template <int D>
struct TokenRow {
    static constexpr int N = (D + 2 * kWave - 1) / (2 * kWave);
    uint32_t kw[N];
    uint32_t vw[N];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ key,
                                         const uint16_t* __restrict__ value, int lane) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int k0 = 2 * lane + 2 * kWave * i;
            if (k0 < D) {
                kw[i] = *reinterpret_cast<const uint32_t*>(key + k0);
                vw[i] = *reinterpret_cast<const uint32_t*>(value + k0);
            }
        }
    }

    // Into slot `slot` of the pools at kv head g.  K: dims k0, k0 + 1 are
    // adjacent inside one 8-dim group, so one 4-byte (16-bit types) or 2-byte
    // (fp8) store.  V: the two dims live in neighbouring lanes of the V row,
    // so two element stores.  fp8 pools store RNE-satfinite E4M3 of
    // x * inv (inv = 1 / scale).
    template <int SRC, int KVT, int BS>
    __device__ __forceinline__ void store(uint8_t* __restrict__ k_cache,
                                          uint8_t* __restrict__ v_cache, int64_t slot,
                                          int num_kv_heads, int g, int lane, float k_inv,
                                          float v_inv) const {
        constexpr int EB = elem_bytes(KVT);
        constexpr int64_t SUB = sub_tile_bytes(KVT, D);
        constexpr int64_t TILE = SUB * (BS / kSubTokens);
        const int64_t pb = slot / BS;
        const int row = (int)(slot % BS);
        const int r = row % kSubTokens;
        const int64_t base = (pb * num_kv_heads + g) * TILE + (row / kSubTokens) * SUB;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int k0 = 2 * lane + 2 * kWave * i;
            if (k0 >= D) continue;
            // K position of (r, k0): group c = k0/8 -> lane r + 16*(c%4), row c/4.
            const int kc = k0 / 8, kkk = kc / 4;
            const int k_lane = r + 16 * (kc % 4);
            const int k_per = 2 / EB;
            const int64_t k_off = 1024 * (kkk / k_per) + 16 * k_lane + 8 * EB * (kkk % k_per) + EB * (k0 % 8);
            // V position of (r, k) for k = k0, k0+1: tile nt = k/16, lane k%16 + 16*(r/4).
            const int v_per = 4 / EB;
            const int nt = k0 / 16;
            const int64_t v_off0 = 1024 * (nt / v_per) + 16 * ((k0 % 16) + 16 * (r / 4)) +
                                   4 * EB * (nt % v_per) + EB * (r % 4);
            const int64_t v_off1 = v_off0 + 16;   // next dim = next lane
            if constexpr (KVT == DT_FP8) {
                const float k_lo = bits_to_f32<SRC>(kw[i] & 0xffffu) * k_inv;
                const float k_hi = bits_to_f32<SRC>(kw[i] >> 16) * k_inv;
                const float v_lo = bits_to_f32<SRC>(vw[i] & 0xffffu) * v_inv;
                const float v_hi = bits_to_f32<SRC>(vw[i] >> 16) * v_inv;
                const uint16_t kcode = (uint16_t)(f32_to_e4m3(k_lo) | (f32_to_e4m3(k_hi) << 8));
                *reinterpret_cast<uint16_t*>(k_cache + base + k_off) = kcode;
                v_cache[base + v_off0] = (uint8_t)f32_to_e4m3(v_lo);
                v_cache[base + v_off1] = (uint8_t)f32_to_e4m3(v_hi);
            } else {
                *reinterpret_cast<uint32_t*>(k_cache + base + k_off) = kw[i];
                *reinterpret_cast<uint16_t*>(v_cache + base + v_off0) = (uint16_t)(vw[i] & 0xffffu);
                *reinterpret_cast<uint16_t*>(v_cache + base + v_off1) = (uint16_t)(vw[i] >> 16);
            }
        }
    }
};

}  // namespace pkv
