// moe_device.h -- device-side helpers shared by the gfx950 kernels of the
// fused mixture-of-experts forward (wave reductions, number formats, vector
// types).  CDNA4: 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;  // 16 bytes, kept in VGPRs

// Index of the calling thread's wave in its block, as a wave-uniform
// (scalar) value.  Conditions built from it then compile to scalar branches:
// an MFMA ignores EXEC, so an MFMA placed under a lane-mask branch would run
// for the whole wave with stale operands.
__device__ __forceinline__ int wave_index(int tid) {
    return __builtin_amdgcn_readfirstlane(tid / kWave);
}

// Order-preserving map of an fp32 value onto uint32 (larger float -> larger
// integer; -inf maps above 0, so 0 is below every real key).  -0 and +0 are
// equal values and get one key, so they tie like any other equal keys (and
// a selection then takes the lower index).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave reductions on DPP (no LDS): lane shifts by 1, 2, 4 and 8 inside each
// 16-lane row, then the row-15 and lane-31 broadcasts, leave op over all 64
// lanes in lane 63 (an inclusive scan; lanes without a source take the
// identity); readlane makes the result wave-uniform.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t identity, uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(identity), static_cast<int>(v),
                                                             CTRL, ROW_MASK, 0xF, false));
}

// One step: every lane combines its value with the value DPP control CTRL
// brings (32-bit words moved separately, so any trivially copyable T).
template <int CTRL, int ROW_MASK, class T, class Op>
__device__ __forceinline__ T dpp_step(T v, T identity, Op op) {
    static_assert(sizeof(T) % 4 == 0, "32-bit words");
    constexpr int W = sizeof(T) / 4;
    struct Words { uint32_t w[W]; };
    const Words a = __builtin_bit_cast(Words, v), id = __builtin_bit_cast(Words, identity);
    Words b;
#pragma unroll
    for (int i = 0; i < W; ++i) b.w[i] = dpp_u32<CTRL, ROW_MASK>(id.w[i], a.w[i]);
    return op(v, __builtin_bit_cast(T, b));
}

template <class T, class Op>
__device__ __forceinline__ T wave_reduce_to_lane63(T v, T identity, Op op) {
    v = dpp_step<0x111, 0xF>(v, identity, op);  // row_shr:1
    v = dpp_step<0x112, 0xF>(v, identity, op);  // row_shr:2
    v = dpp_step<0x114, 0xF>(v, identity, op);  // row_shr:4
    v = dpp_step<0x118, 0xF>(v, identity, op);  // row_shr:8
    v = dpp_step<0x142, 0xA>(v, identity, op);  // row_bcast:15 into rows 1 and 3
    v = dpp_step<0x143, 0xC>(v, identity, op);  // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = wave_reduce_to_lane63(v, uint64_t{0}, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
    return (static_cast<uint64_t>(readlane_u32(static_cast<uint32_t>(v >> 32), 63)) << 32) |
           readlane_u32(static_cast<uint32_t>(v), 63);
}

__device__ __forceinline__ float wave_max_f32(float v) {
    v = wave_reduce_to_lane63(v, -__builtin_huge_valf(), [](float a, float b) { return fmaxf(a, b); });
    return __uint_as_float(readlane_u32(__float_as_uint(v), 63));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    v = wave_reduce_to_lane63(v, 0.0f, [](float a, float b) { return a + b; });
    return __uint_as_float(readlane_u32(__float_as_uint(v), 63));
}

// Inclusive prefix sum across the wave: the reduction steps above leave
// lane i holding lanes 0..i (each step combines disjoint lane ranges).
__device__ __forceinline__ int32_t wave_inclusive_sum_i32(int32_t v) {
    return wave_reduce_to_lane63(v, int32_t{0}, [](int32_t a, int32_t b) { return a + b; });
}

// Exclusive prefix sum of v over the NT threads of a block (NT a multiple of
// 64, at most 64 waves); `wave_sums` is LDS scratch of NT/64 ints.  Every
// thread of the block must call it; *total receives the block sum.
template <int NT>
__device__ __forceinline__ int32_t block_exclusive_sum_i32(int32_t v, int32_t* wave_sums, int32_t* total) {
    static_assert(NT % 64 == 0 && NT / 64 <= 64, "whole waves");
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = wave_index(threadIdx.x);
    const int32_t incl = wave_inclusive_sum_i32(v);
    if (lane == 63) wave_sums[w] = incl;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int32_t t = wave_sums[i];
        before += i < w ? t : 0;
        all += t;
    }
    __syncthreads();  // wave_sums may be reused after the call
    *total = all;
    return before + incl - v;
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> OCP e4m3 code, round to nearest even, saturated to +-448 first
// (the hardware conversion on gfx950 produces the OCP format).
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
    x = fminf(fmaxf(x, -448.0f), 448.0f);
    return static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false) & 0xFF);
}


}  // namespace moe
