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
// integer; -inf maps above 0, so 0 is below every real key).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint64_t w = __shfl_xor(v, o, kWave);
        v = v > w ? v : w;
    }
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
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
