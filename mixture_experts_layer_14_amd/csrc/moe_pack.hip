// moe_pack.hip -- weight re-layout for the gfx950 GEMM kernels.
//
// A row-major matrix of `rows` rows x `row_bytes` bytes becomes
// [rows/16][row_bytes/64][16][64]: the 64-byte pieces of 16 consecutive rows
// over the same k range form one contiguous KiB.  The tile kernels copy 16
// rows x 64 bytes (or 8 rows x 128 bytes) per instruction and the
// weight-streaming kernel reads 16 rows x 64 bytes per MFMA step, so every
// such access becomes one sequential burst instead of 16 pieces one row
// pitch apart.  A pure byte permutation: values are copied bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

// one thread per 16 output bytes; consecutive threads write consecutive bytes
__global__ __launch_bounds__(256) void pack_rows_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t rows,
                                                        int64_t row_bytes, int64_t total16) {
    const int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (o >= total16) return;
    const int64_t per_matrix = rows * row_bytes / 16;
    const int64_t m = o / per_matrix;
    int64_t w = o - m * per_matrix;
    const int64_t chunks = row_bytes / 64;
    const int piece = static_cast<int>(w & 3);         // 16-byte piece of the 64 bytes
    const int r16 = static_cast<int>((w >> 2) & 15);   // row within the 16-row group
    w >>= 6;                                           // (group, chunk) index
    const int64_t c = w % chunks, group = w / chunks;
    const int64_t row = group * 16 + r16;
    dst[o] = src[m * per_matrix + (row * row_bytes + c * 64 + piece * 16) / 16];
}

}  // namespace

hipError_t launch_pack_weights(const void* src, void* dst, int64_t matrices, int64_t rows,
                               int64_t row_bytes, hipStream_t stream) {
    const int64_t total16 = matrices * rows * row_bytes / 16;
    if (total16 == 0) return hipSuccess;
    const int64_t blocks = (total16 + 255) / 256;
    pack_rows_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
        static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), rows, row_bytes, total16);
    return hipGetLastError();
}

}  // namespace moe
