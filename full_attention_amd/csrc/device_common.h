// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pakv_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = 16;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// The same rounding (to nearest even) in one instruction, v_cvt_pk_bf16_f32;
// a NaN comes out as a quiet NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

// 16x16x32 bf16 MFMA: C[16x16] += A[16x32] * B[32x16].  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, each with the 8 contraction indices
// of group l / 16; it receives C rows 4*(l/16) .. +3 of column l % 16.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x16 bf16 MFMA: as above with 4 contraction indices per lane.
__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Lanes l, l^16, l^32, l^48 hold the same column.  v_permlane16_swap trades
// odd 16-lane rows of its first operand with even rows of its second, and
// v_permlane32_swap the upper half of the first with the lower half of the
// second; given the same register twice, the two results hold, in every lane,
// the lane's own value and its partner's (16, then 32 lanes away), without
// the round trip through LDS that a shuffle takes.
__device__ __forceinline__ float wave_max_across_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The sum of the four lanes, added in the same order in every lane (row 0 + row 1, row 2 + row 3,
// then the two), so all four hold the same bits.
__device__ __forceinline__ float wave_sum_across_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// acc + lo^2 + hi^2 for the bf16 pair of a word (v_dot2c_f32_bf16: the
// products are exact in float32, the sum rounds as float32 does).
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_dot;
__device__ __forceinline__ float sq_sum_bf16x2(uint32_t word, float acc) {
    const bf16x2_dot v = __builtin_bit_cast(bf16x2_dot, word);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

__device__ __forceinline__ int32_t clamp_i32(int32_t x, int32_t lo, int32_t hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

// int8 code pair -> bf16 pair bits (exact: |code| <= 128 has an 8-bit significand).
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t word, int byte_lo) {
    float a = (float)(int8_t)((word >> (8 * byte_lo)) & 0xffu);
    float b = (float)(int8_t)((word >> (8 * (byte_lo + 1))) & 0xffu);
    return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// fp8 (OCP E4M3) code pair -> bf16 pair bits: bytes 0, 1 (byte_lo 0) or 2, 3
// (byte_lo 2) of word, in one gfx950 instruction (v_cvt_scalef32_pk_bf16_fp8
// with scale 1).  Exact: every E4M3 value, subnormals included, has a bf16
// twin (3 mantissa bits, exponents 2^-9 .. 2^8).  (Through float32 and a
// pack it took two instructions per pair; the fp8 long-context full layer
// went from ~216 to ~191 us.)
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t word, int byte_lo) {
    const bf16x2_cvt v = byte_lo == 2 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)word, 1.0f, true)
                                      : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)word, 1.0f, false);
    return __builtin_bit_cast(uint32_t, v);
}

// Transposing LDS read (ds_read_b64_tr_b16, gfx950).  Each lane gives the LDS
// byte address of 4 consecutive 16-bit elements, a row of a 16 x 4 block per
// 16-lane group; lane (a = i % 16 / 4, k = i % 4) of the group receives
// element k of the rows a, a + 4, a + 8, a + 12 (measured on the device).  So
// if lane j of group g addresses row 4 g + j / 4, elements 4 (j % 4) .. + 3
// of a token-major tile, lane i receives one element column (the i-th of the
// four groups' 16) for the four tokens 4 g .. 4 g + 3: the operand a value
// product wants from keys stored token-major.
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_tr;
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
    auto* lp = (__attribute__((address_space(3))) bf16x4_tr*)(uintptr_t)p;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

// Page-table entries outside the pool (or positions past a table's width)
// are read as page 0, or dropped by a store, in every build.  A build with
// PAKV_DEBUG_BOUNDS also counts them, per kind of call, in the library's
// counter array (`bad` is its device address; null in other builds).
constexpr int kBadIdPlan = 0, kBadIdStore = 1, kBadIdExtend = 2;
__device__ __forceinline__ void note_bad_id(uint32_t* bad, int kind) {
#ifdef PAKV_DEBUG_BOUNDS
    if (bad) __hip_atomic_fetch_add(bad + kind, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
    (void)bad;
    (void)kind;
#endif
}

}  // namespace pakv_dev
