// moe_topk.hip -- router: top-k selection and routing weights, one 64-lane
// wavefront per token (the per-token selection is topk_row in moe_topk.h,
// which states the operation and cites the pages).
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {

template <int VPL, int PB>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= a.T) return;  // wave-uniform exit
    topk_row<VPL, PB>(a, t, lane);
}

template <int VPL>
static void launch_topk_vpl(const TopkArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
    if (a.parts <= 8)
        topk_kernel<VPL, topk_part_batch(VPL, 8)><<<grid, block, 0, stream>>>(a);
    else
        topk_kernel<VPL, topk_part_batch(VPL, 32)><<<grid, block, 0, stream>>>(a);
}

hipError_t launch_topk(const float* logits, int parts, float* logits_out, const float* bias,
                       int64_t T, int E, int K, int scoring, int renorm, int G, int TG, float rsf,
                       int32_t* ids, float* weights, hipStream_t stream) {
    const TopkArgs a{logits, parts, T * E, logits_out, bias, T, E, K, scoring, renorm, G, TG, rsf, ids, weights};
    const int waves_per_block = 4;
    const dim3 block(kWave * waves_per_block);
    const dim3 grid(static_cast<unsigned>((T + waves_per_block - 1) / waves_per_block));
    const int vpl = (E + kWave - 1) / kWave;
    if (vpl <= 1)
        launch_topk_vpl<1>(a, grid, block, stream);
    else if (vpl <= 2)
        launch_topk_vpl<2>(a, grid, block, stream);
    else if (vpl <= 4)
        launch_topk_vpl<4>(a, grid, block, stream);
    else
        launch_topk_vpl<8>(a, grid, block, stream);
    return hipGetLastError();
}

}  // namespace moe
