// moe_quant.hip -- per-token-group-128 fp8 quantisation of the layer input,
// computed once and shared by the routed and the shared experts (SGLang page
// "srt/models/deepseek_v2.py", DeepseekV2MoE._maybe_quant_moe_input_once:
// one fp32 scale per 128 consecutive values of a token row).
//   scale = max(amax, 1e-10) / 448,  code = e4m3(x / scale)   (fp32, RNE)
// A group of 128 bf16 values is 16 lanes x 8 values (16-byte loads); the
// group amax is a 4-step shuffle reduction inside the 16 lanes.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                        int H, uint8_t* __restrict__ q,
                                                        float* __restrict__ s) {
    const int64_t t = blockIdx.x;
    if (t >= T) return;
    const int ngroups = H / 128;
    const int l16 = threadIdx.x % 16;
    for (int g = threadIdx.x / 16; g < ngroups; g += blockDim.x / 16) {
        const int64_t base = t * H + static_cast<int64_t>(g) * 128 + l16 * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(x + base);
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(v[i] << 16);
            f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
        const float scale = fmaxf(amax, 1e-10f) / 448.0f;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= static_cast<uint32_t>(f32_to_e4m3(f[i] / scale)) << (8 * i);
            hi |= static_cast<uint32_t>(f32_to_e4m3(f[4 + i] / scale)) << (8 * i);
        }
        *reinterpret_cast<uint2*>(q + base) = make_uint2(lo, hi);
        if (l16 == 0) s[t * ngroups + g] = scale;
    }
}

hipError_t launch_quant_fp8(const void* hidden, int64_t T, int H, uint8_t* q, float* scale,
                            hipStream_t stream) {
    quant_fp8_kernel<<<static_cast<unsigned>(T), 256, 0, stream>>>(
        static_cast<const uint16_t*>(hidden), T, H, q, scale);
    return hipGetLastError();
}

}  // namespace moe
