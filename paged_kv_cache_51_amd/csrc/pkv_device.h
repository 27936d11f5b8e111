// pkv_device.h — device-side types and helpers shared by the gfx950 kernels.
//
// Pool layout (tile order, 1 KiB rows of 64 lanes x 16 bytes, K lanes holding
// 8 dims of one token, V lanes holding 4 tokens of one dim) is defined in
// include/pagedkv.h; the constants here restate it (head_dim 128 unless a
// template says otherwise).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum : int { DT_BF16 = 0, DT_FP16 = 1, DT_FP8 = 2 };

constexpr int kHeadDim = 128;
constexpr int kWave = 64;
constexpr int kSubTokens = 16;   // tokens per sub-tile (one MFMA M/N edge)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int elem_bytes(int dt) { return dt == DT_FP8 ? 1 : 2; }

// Bytes of one 16-token sub-tile of one pool (K or V) at head_dim d (a
// multiple of 64; the kernels are built for 64, 128 and 256).
__host__ __device__ constexpr int sub_tile_bytes(int dt, int d = kHeadDim) { return kSubTokens * d * elem_bytes(dt); }

// 1 KiB rows per sub-tile: d / 32 for 16-bit elements (4 at d = 128), d / 64
// for fp8.
__host__ __device__ constexpr int rows_per_sub(int dt, int d = kHeadDim) { return sub_tile_bytes(dt, d) / 1024; }

// ---------------------------------------------------------------- scalars --

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;                      // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    _Float16 h = (_Float16)x;                  // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

template <int DT>
__device__ __forceinline__ uint16_t f32_to_bits(float x) {
    if constexpr (DT == DT_BF16) return f32_to_bf16_bits(x);
    else return f32_to_f16_bits(x);
}

template <int DT>
__device__ __forceinline__ float bits_to_f32(uint32_t bits16) {
    if constexpr (DT == DT_BF16) return bf16_bits_to_f32(bits16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// fp32 -> OCP E4M3 (e4m3fn), round to nearest even, saturating to +-448,
// NaN -> 0x7F (sign kept), sign kept on underflow.  Integer formulation:
// subnormal range (|x| < 2^-6) rounds |x| * 2^9 to an integer (exact scaling
// by a power of two, then v_rndne); the normal range rounds the fp32
// mantissa to 3 bits at bit 20 with ties to even.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;           // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;          // >= 448 (and inf)
    if (a < 0x3c800000u) {                              // < 2^-6
        float f = __uint_as_float(a) * 512.0f;
        return sign | (uint32_t)__builtin_rintf(f);      // 0..8 (8 = 2^-6)
    }
    uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);       // RNE at bit 20
    uint32_t e = (r >> 23) - 120u;                      // rebias 127 -> 7
    return sign | (e << 3) | ((r >> 20) & 7u);
}

// ------------------------------------------------------------ MFMA wraps --

// 16x16x32: A (16 x 32) and B (32 x 16) as 8 16-bit elements per lane.
template <int QT>
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
    if constexpr (QT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// 16x16x16: A (16 x 16) and B (16 x 16) as 4 16-bit elements per lane.
template <int QT>
__device__ __forceinline__ f32x4_t mfma_16x16x16(u32x2_t a, u32x2_t b, f32x4_t c) {
    if constexpr (QT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                         __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// Two E4M3 codes (bytes 2*hi, 2*hi+1 of w) -> two 16-bit values of type QT,
// packed low element first.  Exact: every E4M3 value is representable.
template <int QT, bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_16(uint32_t w) {
    if constexpr (QT == DT_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Eight E4M3 codes (two dwords) -> eight 16-bit values (four dwords).
template <int QT>
__device__ __forceinline__ u32x4_t e4m3x8_to_16(uint32_t lo, uint32_t hi) {
    u32x4_t r;
    r[0] = e4m3x2_to_16<QT, false>(lo);
    r[1] = e4m3x2_to_16<QT, true>(lo);
    r[2] = e4m3x2_to_16<QT, false>(hi);
    r[3] = e4m3x2_to_16<QT, true>(hi);
    return r;
}

// Four E4M3 codes (one dword) -> four 16-bit values (two dwords).
template <int QT>
__device__ __forceinline__ u32x2_t e4m3x4_to_16(uint32_t w) {
    u32x2_t r;
    r[0] = e4m3x2_to_16<QT, false>(w);
    r[1] = e4m3x2_to_16<QT, true>(w);
    return r;
}

// Cross-lane xor shuffle of a float within the wave (ds_bpermute).
__device__ __forceinline__ float xor_shfl(float v, int mask) {
    int lane = __lane_id();
    int src = (lane ^ mask) << 2;
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Dword of lane `src` (any lane of the wave), read by every lane.
__device__ __forceinline__ uint32_t lane_fetch(uint32_t v, int src) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}

// a.x * b.x + a.y * b.y + c on two packed 16-bit pairs of type DT (vector
// ALU dot instruction, fp32 accumulate).
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == DT_BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                      c, false);
}

}  // namespace pkv
