// moe_topk.hip -- router: top-k selection and routing weights, one 64-lane
// wavefront per token.
//
// Operation (vLLM docs page "vllm.model_executor.layers.fused_moe.layer",
// FusedMoE.select_experts; SGLang page "srt/models/deepseek_v2.py",
// DeepseekV2MoE grouped top-k arguments and MoEGate correction bias):
//   softmax: score = softmax(logits), selection key = logit (same order);
//   sigmoid: score = sigmoid(logit), key = score + e_score_correction_bias;
//   grouped: experts split into G contiguous groups; a group scores the sum
//            of its two largest keys (with a bias) or its largest key; the TG
//            best groups stay eligible;
//   select K keys, descending, exact ties to the lower index;
//   weight = score (renormalised over the K selected if asked) * rsf.
//
// Layout: lane l holds experts e = l + 64*v, v < VPL, so every row load is
// a run of coalesced 256-byte wave accesses.  A selection round is one wave
// arg-max over packed (ordered key bits << 32 | ~expert) 64-bit values.
//
// The logits may come as `parts` partial sums (the router gate GEMM with H
// split into parts, parts * T * E floats): the kernel adds them in part
// order, the order of router_reduce_kernel, so routing the router GEMM's
// output through moe_router_gemm + moe_topk or through moe_router_topk gives
// the same bits; with logits_out the summed logits are stored as well.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ logits, int parts, int64_t part_stride, float* __restrict__ logits_out,
    const float* __restrict__ bias, int64_t T, int E, int K, int scoring, int renorm, int G, int TG,
    float rsf, int32_t* __restrict__ ids, float* __restrict__ weights) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;  // wave-uniform exit
    const float* row = logits + t * E;

    float key[VPL], score[VPL];
    bool cand[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = lane + kWave * v;
        cand[v] = e < E;
        key[v] = cand[v] ? row[e] : -INFINITY;
    }
    // the other parts, added in part order; the loads of 8 parts are issued
    // before their adds, so a long split is not a chain of dependent loads
    constexpr int PB = 8;
    for (int p0 = 1; p0 < parts; p0 += PB) {
        float pl[PB][VPL];
#pragma unroll
        for (int q = 0; q < PB; ++q)
#pragma unroll
            for (int v = 0; v < VPL; ++v)
                pl[q][v] = (p0 + q < parts && cand[v]) ? row[(p0 + q) * part_stride + lane + kWave * v] : 0.0f;
#pragma unroll
        for (int q = 0; q < PB; ++q)
#pragma unroll
            for (int v = 0; v < VPL; ++v)
                if (p0 + q < parts) key[v] += pl[q][v];
    }
    if (logits_out) {
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (cand[v]) logits_out[t * E + lane + kWave * v] = key[v];
    }

    float softmax_sum = 0.0f, softmax_max = 0.0f;
    if (scoring == 0) {
        float m = -INFINITY;
#pragma unroll
        for (int v = 0; v < VPL; ++v) m = fmaxf(m, key[v]);
        m = wave_max_f32(m);
        float s = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            score[v] = cand[v] ? expf(key[v] - m) : 0.0f;  // unnormalised
            s += score[v];
        }
        softmax_sum = wave_sum_f32(s);
        softmax_max = m;
    } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int e = lane + kWave * v;
            score[v] = cand[v] ? 1.0f / (1.0f + expf(-key[v])) : 0.0f;
            key[v] = cand[v] ? score[v] + (bias ? bias[e] : 0.0f) : -INFINITY;
        }
    }
    (void)softmax_max;

    if (G > 1) {
        const int per = E / G;
        int grp[VPL];  // group of each of the lane's experts (one division each)
#pragma unroll
        for (int v = 0; v < VPL; ++v) grp[v] = (lane + kWave * v) / per;
        float my_gscore = -INFINITY;
        for (int g = 0; g < G; ++g) {
            float2 top{-INFINITY, -INFINITY};  // the lane's two largest keys of group g
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                if (cand[v] && grp[v] == g) {
                    const float k = key[v];
                    if (k > top.x) { top.y = top.x; top.x = k; } else if (k > top.y) { top.y = k; }
                }
            }
            // merge of two (largest, second largest) pairs, over the wave
            top = wave_reduce_to_lane63(top, float2{-INFINITY, -INFINITY}, [](float2 a, float2 b) {
                return float2{fmaxf(a.x, b.x), fmaxf(fminf(a.x, b.x), fmaxf(a.y, b.y))};
            });
            const float b1 = __uint_as_float(readlane_u32(__float_as_uint(top.x), 63));
            const float b2 = __uint_as_float(readlane_u32(__float_as_uint(top.y), 63));
            const float gs = (bias != nullptr && per >= 2) ? b1 + b2 : b1;
            if (lane == g) my_gscore = gs;
        }
        uint64_t keep = 0;
        for (int r = 0; r < TG; ++r) {
            uint64_t packed = 0;
            if (lane < G && !((keep >> lane) & 1ull))
                packed = (static_cast<uint64_t>(ordered_bits(my_gscore)) << 32) |
                         static_cast<uint32_t>(~static_cast<uint32_t>(lane));
            packed = wave_max_u64(packed);
            keep |= 1ull << (~static_cast<uint32_t>(packed));
        }
#pragma unroll
        for (int v = 0; v < VPL; ++v) cand[v] = cand[v] && ((keep >> grp[v]) & 1ull);
    }

    int my_id = 0;
    float my_w = 0.0f, sel_sum = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int e = lane + kWave * v;
            if (cand[v]) {
                const uint64_t p = (static_cast<uint64_t>(ordered_bits(key[v])) << 32) |
                                   static_cast<uint32_t>(~static_cast<uint32_t>(e));
                best = p > best ? p : best;
            }
        }
        best = wave_max_u64(best);
        const int e_sel = static_cast<int>(~static_cast<uint32_t>(best));
        const int owner = e_sel & (kWave - 1);
        const int v_sel = e_sel / kWave;
        float s_mine = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            if (v == v_sel) {
                s_mine = score[v];
                if (lane == owner) cand[v] = false;
            }
        }
        const float s_sel = __uint_as_float(readlane_u32(__float_as_uint(s_mine), owner));
        sel_sum += s_sel;
        if (lane == k) {
            my_id = e_sel;
            my_w = s_sel;
        }
    }

    if (lane < K) {
        float w;
        if (renorm)
            w = my_w / sel_sum;
        else
            w = scoring == 0 ? my_w / softmax_sum : my_w;
        ids[t * K + lane] = my_id;
        weights[t * K + lane] = w * rsf;
    }
}

hipError_t launch_topk(const float* logits, int parts, float* logits_out, const float* bias,
                       int64_t T, int E, int K, int scoring, int renorm, int G, int TG, float rsf,
                       int32_t* ids, float* weights, hipStream_t stream) {
    const int waves_per_block = 4;
    const dim3 block(kWave * waves_per_block);
    const dim3 grid(static_cast<unsigned>((T + waves_per_block - 1) / waves_per_block));
    const int vpl = (E + kWave - 1) / kWave;
    const int64_t ps = T * E;
#define MOE_TOPK_LAUNCH(V)                                                                          \
    topk_kernel<V><<<grid, block, 0, stream>>>(logits, parts, ps, logits_out, bias, T, E, K, scoring, \
                                               renorm, G, TG, rsf, ids, weights)
    if (vpl <= 1)
        MOE_TOPK_LAUNCH(1);
    else if (vpl <= 2)
        MOE_TOPK_LAUNCH(2);
    else if (vpl <= 4)
        MOE_TOPK_LAUNCH(4);
    else
        MOE_TOPK_LAUNCH(8);
#undef MOE_TOPK_LAUNCH
    return hipGetLastError();
}

}  // namespace moe
