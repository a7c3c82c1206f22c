// Device helpers shared by the gfx950 attention kernels.
//
// MFMA lane layout used throughout (v_mfma_f32_16x16x4_f32, one wave of 64
// lanes, lane l = 16*g + i with i = l % 16 and g = l / 16):
//   A (16x4, M x K): lane l holds A[m = i][k = g]
//   B (4x16, K x N): lane l holds B[k = g][n = i]
//   C (16x16):       lane l, register r holds C[m = 4*g + r][n = i]
// so a C tile keeps its column index in i and spreads its rows over (g, r).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 2^x and log2(x) on the hardware transcendental unit (v_exp_f32, v_log_f32).
// exp(y) is evaluated as 2^(y * log2 e); the log2(e) factor is folded into the
// score scale by the callers.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Both values {x[l], x[l ^ 16]} / {x[l], x[l ^ 32]} at every lane, through the
// gfx950 row-swap permutes (no LDS traffic).  Only symmetric combinations of the
// pair are used, so which element is which does not matter.
__device__ __forceinline__ void pair_xor16(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair_xor32(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Exchanges between two registers (gfx950 v_permlane16_swap / v_permlane32_swap):
//   swap_rows16(a, b): the odd 16-lane rows of a trade places with the even rows of b,
//     i.e. a = [a0, b0, a2, b2], b = [a1, b1, a3, b3] in 16-lane rows;
//   swap_rows32(a, b): the upper half of a trades places with the lower half of b,
//     i.e. a = [a0, a1, b0, b1], b = [a2, a3, b2, b3].
__device__ __forceinline__ void swap_rows16(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap_rows32(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Reductions over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows),
// i.e. over g for a fixed i.  Every lane of the group ends with the same bits.
__device__ __forceinline__ float rows4_max(float x) {
    float a, b;
    pair_xor16(x, a, b);
    x = fmaxf(a, b);
    pair_xor32(x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float rows4_sum(float x) {
    float a, b;
    pair_xor16(x, a, b);
    x = a + b;
    pair_xor32(x, a, b);
    return a + b;
}

// Data-parallel-primitive lane moves (VALU, no LDS): CTRL is the DPP control.
//   0xB1 quad_perm [1,0,3,2] = lane ^ 1        0x4E quad_perm [2,3,0,1] = lane ^ 2
//   0x124 row_ror:4, 0x128 row_ror:8 (rotate inside a 16-lane row; lane % 4 kept)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppRor4 = 0x124;
constexpr int kDppRor8 = 0x128;
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <- lane 7 - i inside each 8-lane half-row

// sum / max over the 4 lanes of a quad (lanes 4k .. 4k+3)
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp_mov<kDppXor1>(x);
    return x + dpp_mov<kDppXor2>(x);
}
__device__ __forceinline__ float quad_max(float x) {
    x = fmaxf(x, dpp_mov<kDppXor1>(x));
    return fmaxf(x, dpp_mov<kDppXor2>(x));
}
// sum / max over the 4 lanes of a 16-lane row that share lane % 4
__device__ __forceinline__ float row_stride4_sum(float x) {
    x += dpp_mov<kDppRor4>(x);
    return x + dpp_mov<kDppRor8>(x);
}
__device__ __forceinline__ float row_stride4_max(float x) {
    x = fmaxf(x, dpp_mov<kDppRor4>(x));
    return fmaxf(x, dpp_mov<kDppRor8>(x));
}
// whole-wave reductions
__device__ __forceinline__ float wave_sum(float x) { return rows4_sum(row_stride4_sum(quad_sum(x))); }
__device__ __forceinline__ float wave_max(float x) { return rows4_max(row_stride4_max(quad_max(x))); }

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Inclusive prefix sum over the 64 lanes of a wave on DPP moves (no LDS): shifted
// adds inside each 16-lane row (a lane whose source is outside its row adds 0), then
// row 0's total into row 1 and row 2's into row 3 (row_bcast:15), then the total of
// rows 0-1 into rows 2 and 3 (row_bcast:31).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add(int x) {
    return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
    x = dpp_add<0x111, 0xF>(x);  // row_shr:1
    x = dpp_add<0x112, 0xF>(x);  // row_shr:2
    x = dpp_add<0x114, 0xF>(x);  // row_shr:4
    x = dpp_add<0x118, 0xF>(x);  // row_shr:8
    x = dpp_add<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x = dpp_add<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

}  // namespace attn
