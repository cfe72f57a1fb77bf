// moe_topk.h -- router top-k of one token on one 64-lane wavefront, shared by
// the top-k kernel and the router kernel that runs the top-k itself.
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
// a run of coalesced 256-byte wave accesses.  A selection round is a DPP
// max of the order-preserving 32-bit keys, then one ballot per v for the
// lowest index holding it.  Groups of a power-of-two size up to 64 are whole
// lane segments of one v: their two largest keys come from one segmented
// DPP reduction for all groups at once.
//
// The logits may come as `parts` partial sums (the router gate GEMM with H
// split into parts, parts * T * E floats): they are added in part order, the
// order of the router's reduce kernel, so the separate calls and the fused
// one give the same bits.
#pragma once

#include "moe_device.h"

namespace moe {

struct TopkArgs {
    const float* logits;  // `parts` arrays of T x E partial logits, part_stride floats apart
    int parts;
    int64_t part_stride;
    float* logits_out;  // the summed logits, or null
    const float* bias;  // per-expert selection bias (sigmoid scoring), or null
    int64_t T;
    int E, K, scoring, renorm, G, TG;
    float rsf;
    int32_t* ids;
    float* weights;
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = wave_reduce_to_lane63(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
    return readlane_u32(v, 63);
}

// Index (64 v + lane) of the largest okey among the candidates `ok`, exact
// ties to the lower index; the winner stops being a candidate.  -1 when no
// candidate is left (the parameter checks rule that out).
template <int VPL>
__device__ __forceinline__ int take_first_max(const uint32_t (&okey)[VPL], bool (&ok)[VPL], int lane) {
    uint32_t m = 0;
#pragma unroll
    for (int v = 0; v < VPL; ++v) m = ok[v] && okey[v] > m ? okey[v] : m;
    m = wave_max_u32(m);
    int sel = -1;
#pragma unroll
    for (int v = VPL - 1; v >= 0; --v) {
        const uint64_t b = __ballot(ok[v] && okey[v] == m);
        if (b) sel = v * kWave + __builtin_ctzll(b);
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) ok[v] = ok[v] && v * kWave + lane != sel;
    return sel;
}

// Top-k of token t (its wave calls it; `lane` = lane in the wave).  PB part
// loads are issued before their adds.
template <int VPL, int PB>
__device__ __forceinline__ void topk_row(const TopkArgs& a, int64_t t, int lane) {
    const int E = a.E;
    const float* row = a.logits + t * E;
    float key[VPL], score[VPL];
    bool cand[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = lane + kWave * v;
        cand[v] = e < E;
        key[v] = cand[v] ? row[e] : -INFINITY;
    }
    for (int p0 = 1; p0 < a.parts; p0 += PB) {
        float pl[PB][VPL];
#pragma unroll
        for (int q = 0; q < PB; ++q)
#pragma unroll
            for (int v = 0; v < VPL; ++v)
                pl[q][v] = (p0 + q < a.parts && cand[v]) ? row[(p0 + q) * a.part_stride + lane + kWave * v] : 0.0f;
#pragma unroll
        for (int q = 0; q < PB; ++q)
#pragma unroll
            for (int v = 0; v < VPL; ++v)
                if (p0 + q < a.parts) key[v] += pl[q][v];
    }
    if (a.logits_out) {
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (cand[v]) a.logits_out[t * E + lane + kWave * v] = key[v];
    }

    float softmax_sum = 0.0f;
    if (a.scoring == 0) {
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
    } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int e = lane + kWave * v;
            score[v] = cand[v] ? 1.0f / (1.0f + expf(-key[v])) : 0.0f;
            key[v] = cand[v] ? score[v] + (a.bias ? a.bias[e] : 0.0f) : -INFINITY;
        }
    }

    if (a.G > 1) {
        const int per = E / a.G;
        const bool two = a.bias != nullptr && per >= 2;  // group score: two largest keys, or the largest
        // (largest, second largest) of two disjoint sets
        auto merge = [](float2 x, float2 y) {
            return float2{fmaxf(x.x, y.x), fmaxf(fminf(x.x, y.x), fmaxf(x.y, y.y))};
        };
        const float2 none{-INFINITY, -INFINITY};
        if (per <= kWave && (per & (per - 1)) == 0) {
            // every group is the lane segment [j*per, (j+1)*per) of one v: the
            // row shifts and broadcasts of a wave reduction, stopped at the
            // segment size, leave each group's pair in the segment's last lane
            float2 top[VPL];
#pragma unroll
            for (int v = 0; v < VPL; ++v) top[v] = cand[v] ? float2{key[v], -INFINITY} : none;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                if (per >= 2) top[v] = dpp_step<0x111, 0xF>(top[v], none, merge);  // row_shr:1
                if (per >= 4) top[v] = dpp_step<0x112, 0xF>(top[v], none, merge);  // row_shr:2
                if (per >= 8) top[v] = dpp_step<0x114, 0xF>(top[v], none, merge);  // row_shr:4
                if (per >= 16) top[v] = dpp_step<0x118, 0xF>(top[v], none, merge); // row_shr:8
                if (per >= 32) top[v] = dpp_step<0x142, 0xA>(top[v], none, merge); // row_bcast:15
                if (per >= 64) top[v] = dpp_step<0x143, 0xC>(top[v], none, merge); // row_bcast:31
            }
            const bool last = (lane & (per - 1)) == per - 1;
            uint32_t gkey[VPL];
            bool gok[VPL];
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                gok[v] = last && (v * kWave + lane) / per < a.G;
                gkey[v] = ordered_bits(two ? top[v].x + top[v].y : top[v].x);
            }
            // the TG best groups (ties to the lower group, i.e. the lower
            // segment end), then every lane of a kept segment stays eligible
            uint64_t kept[VPL];
#pragma unroll
            for (int v = 0; v < VPL; ++v) kept[v] = 0;
            for (int r = 0; r < a.TG; ++r) {
                const int sel = take_first_max(gkey, gok, lane);
#pragma unroll
                for (int v = 0; v < VPL; ++v)
                    if (v == sel / kWave) kept[v] |= 1ull << (sel & (kWave - 1));
            }
#pragma unroll
            for (int v = 0; v < VPL; ++v) cand[v] = cand[v] && ((kept[v] >> (lane | (per - 1))) & 1ull);
        } else {
            // other group sizes: one wave reduction per group; group g's score
            // lands in lane g (G <= 64)
            int grp[VPL];
#pragma unroll
            for (int v = 0; v < VPL; ++v) grp[v] = (lane + kWave * v) / per;
            float my_gscore = -INFINITY;
            for (int g = 0; g < a.G; ++g) {
                float2 top = none;
#pragma unroll
                for (int v = 0; v < VPL; ++v)
                    if (cand[v] && grp[v] == g) top = merge(top, float2{key[v], -INFINITY});
                top = wave_reduce_to_lane63(top, none, merge);
                const float b1 = __uint_as_float(readlane_u32(__float_as_uint(top.x), 63));
                const float b2 = __uint_as_float(readlane_u32(__float_as_uint(top.y), 63));
                if (lane == g) my_gscore = two ? b1 + b2 : b1;
            }
            uint32_t gkey[1] = {ordered_bits(my_gscore)};
            bool gok[1] = {lane < a.G};
            uint64_t keep = 0;
            for (int r = 0; r < a.TG; ++r) {
                const int sel = take_first_max(gkey, gok, lane);
                if (sel >= 0) keep |= 1ull << sel;
            }
#pragma unroll
            for (int v = 0; v < VPL; ++v) cand[v] = cand[v] && ((keep >> grp[v]) & 1ull);
        }
    }

    uint32_t okey[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) okey[v] = ordered_bits(key[v]);
    int my_id = 0;
    float my_w = 0.0f, sel_sum = 0.0f;
    for (int k = 0; k < a.K; ++k) {
        const int e_sel = take_first_max(okey, cand, lane);
        const int owner = e_sel & (kWave - 1);
        const int v_sel = e_sel / kWave;
        float s_mine = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (v == v_sel) s_mine = score[v];
        const float s_sel = __uint_as_float(readlane_u32(__float_as_uint(s_mine), owner));
        sel_sum += s_sel;
        if (lane == k) {
            my_id = e_sel;
            my_w = s_sel;
        }
    }

    if (lane < a.K) {
        float w;
        if (a.renorm)
            w = my_w / sel_sum;
        else
            w = a.scoring == 0 ? my_w / softmax_sum : my_w;
        a.ids[t * a.K + lane] = my_id;
        a.weights[t * a.K + lane] = w * a.rsf;
    }
}

// Parts loaded per batch: all of a decode split (up to 32) at once where the
// registers allow.
constexpr int topk_part_batch(int vpl, int parts) { return parts <= 8 ? 8 : (vpl <= 4 ? 32 : 16); }

}  // namespace moe
