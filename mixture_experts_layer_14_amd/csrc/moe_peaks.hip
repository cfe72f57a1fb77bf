// moe_peaks.hip -- measurement helpers, not steps of the layer: a bf16 MFMA
// loop and an HBM read stream, so that a benchmark can print the peaks this
// particular MI355X reaches (at its sustained clock) beside the published
// ones.
#include "../../include/moe.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

// Each wave runs `iters` rounds of 8 independent 32x32x16 bf16 MFMAs (8
// accumulators, so the matrix core never waits on a dependency); the sums
// go to `sink` so nothing is optimised away.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int64_t iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & (kWave - 1);
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(0.001f * (lane + i));
        b[i] = static_cast<__bf16>(0.002f * (lane - i));
    }
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// Each block reads its own contiguous share of the `n16` 16-byte words, 256
// threads striding by 256 with U loads in flight per thread; the xor of
// everything read goes to `sink`.
template <int U>
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          int64_t per_block, unsigned* __restrict__ sink) {
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * per_block;
    const int64_t n = begin >= n16 ? 0 : (n16 - begin < per_block ? n16 - begin : per_block);
    const u32x4* p = src + begin;
    u32x4 x = {0u, 0u, 0u, 0u};
    for (int64_t i = threadIdx.x; i < n; i += 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = i + u * 256 < n ? p[i + u * 256] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u];
    }
    sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_peak_mfma_bf16(int64_t iters, int32_t blocks, float* sink, void* stream) {
    if (iters < 1 || blocks < 1 || !sink) return MOE_ERR_INVALID;
    moe::mfma_loop_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_peak_read(const void* buf, int64_t bytes, int32_t blocks, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes < 16 || blocks < 1 || (bytes & 15) ||
        (reinterpret_cast<uintptr_t>(buf) & 15))
        return MOE_ERR_INVALID;
    const int64_t n16 = bytes / 16;
    moe::read_stream_kernel<16><<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const moe::u32x4*>(buf), n16, (n16 + blocks - 1) / blocks, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
