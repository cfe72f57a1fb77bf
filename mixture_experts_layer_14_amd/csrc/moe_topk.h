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
// Layout: lane l holds the VPL consecutive experts e = VPL*l + v, so a row
// (or a part of it) is one vector load per lane and the wave reads it as one
// contiguous run.  A selection round is a DPP max of the order-preserving
// 32-bit keys, then one ballot per v and the lowest index holding the max.
// When a group is a whole number of lanes (a power of two up to 64 of them),
// the two largest keys of every group come from the lane's own values plus
// one segmented DPP reduction, for all groups at once.  (A group smaller
// than a lane's run cannot occur: VPL is the smallest of 1, 2, 4, 8 with
// 64*VPL >= E, so E/G < VPL would need more than 64 groups.)
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

// Index (VPL*lane + v) of the largest okey among the candidates `ok`,
// exact ties to the lower index; the winner stops being a candidate.  -1
// when no candidate is left (the parameter checks rule that out).
template <int VPL>
__device__ __forceinline__ int take_first_max(const uint32_t (&okey)[VPL], bool (&ok)[VPL], int lane) {
    uint32_t m = 0;
#pragma unroll
    for (int v = 0; v < VPL; ++v) m = ok[v] && okey[v] > m ? okey[v] : m;
    m = wave_max_u32(m);
    int sel = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const uint64_t b = __ballot(ok[v] && okey[v] == m);
        const int i = b ? __builtin_ctzll(b) * VPL + v : 0x7fffffff;
        sel = i < sel ? i : sel;
    }
    sel = sel == 0x7fffffff ? -1 : sel;
#pragma unroll
    for (int v = 0; v < VPL; ++v) ok[v] = ok[v] && VPL * lane + v != sel;
    return sel;
}

// VPL consecutive floats of `src` from element VPL*lane (VEC: as vector
// loads, the caller having checked that n is a multiple of VPL and `src`
// aligned to the vector), elements at or past n reading `fill`.  No branch:
// a lane past n loads an element below n and discards it, so a batch of
// these loads stays in flight together.
template <int VPL, bool VEC>
__device__ __forceinline__ void load_run(const float* src, int lane, int n, float fill, float (&out)[VPL]) {
    const int e0 = VPL * lane;
    if constexpr (VEC && VPL == 2) {
        const float2 x = *reinterpret_cast<const float2*>(src + (e0 < n ? e0 : 0));
        out[0] = e0 < n ? x.x : fill;
        out[1] = e0 < n ? x.y : fill;
    } else if constexpr (VEC && VPL % 4 == 0) {
#pragma unroll
        for (int h = 0; h < VPL / 4; ++h) {
            const float4 x = *reinterpret_cast<const float4*>(src + (e0 < n ? e0 + 4 * h : 0));
            out[4 * h] = e0 < n ? x.x : fill;
            out[4 * h + 1] = e0 < n ? x.y : fill;
            out[4 * h + 2] = e0 < n ? x.z : fill;
            out[4 * h + 3] = e0 < n ? x.w : fill;
        }
    } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const float x = src[e0 + v < n ? e0 + v : n - 1];
            out[v] = e0 + v < n ? x : fill;
        }
    }
}

// Whether runs of VPL floats at `p` may be loaded as vectors (see load_run).
template <int VPL>
__device__ __forceinline__ bool vec_ok(const void* p, int n) {
    constexpr uintptr_t kAlign = VPL == 2 ? 8 : 16;
    return VPL > 1 && n % VPL == 0 && (reinterpret_cast<uintptr_t>(p) & (kAlign - 1)) == 0;
}

// The logits of token t, summed over the parts in part order; PB part loads
// are issued before their adds (parts past the last load the last part
// again and are not added).
template <int VPL, int PB, bool VEC>
__device__ __forceinline__ void load_logits(const TopkArgs& a, int64_t t, int lane, float (&key)[VPL]) {
    const float* row = a.logits + t * a.E;
    load_run<VPL, VEC>(row, lane, a.E, -INFINITY, key);
    for (int p0 = 1; p0 < a.parts; p0 += PB) {
        float pl[PB][VPL];
#pragma unroll
        for (int q = 0; q < PB; ++q) {
            const int p = p0 + q < a.parts ? p0 + q : a.parts - 1;
            load_run<VPL, VEC>(row + p * a.part_stride, lane, a.E, 0.0f, pl[q]);
        }
#pragma unroll
        for (int q = 0; q < PB; ++q)
#pragma unroll
            for (int v = 0; v < VPL; ++v)
                if (p0 + q < a.parts) key[v] += pl[q][v];
    }
}

// (largest, second largest) of two disjoint sets
__device__ __forceinline__ float2 merge_top2(float2 x, float2 y) {
    return float2{fmaxf(x.x, y.x), fmaxf(fminf(x.x, y.x), fmaxf(x.y, y.y))};
}

// Top-k of token t (its wave calls it; `lane` = lane in the wave).  PB part
// loads are issued before their adds.
template <int VPL, int PB>
__device__ __forceinline__ void topk_row(const TopkArgs& a, int64_t t, int lane) {
    static_assert(VPL == 1 || VPL == 2 || VPL % 4 == 0, "vector runs of 1, 2 or 4k floats");
    const int E = a.E;
    float key[VPL], score[VPL];
    bool cand[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) cand[v] = VPL * lane + v < E;
    // rows start at multiples of E floats from `logits`, parts at multiples
    // of T*E: vector loads when the base allows them
    if (vec_ok<VPL>(a.logits, E))
        load_logits<VPL, PB, true>(a, t, lane, key);
    else
        load_logits<VPL, PB, false>(a, t, lane, key);
    if (a.logits_out) {
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (cand[v]) a.logits_out[t * E + VPL * lane + v] = key[v];
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
        float bias[VPL];
        if (a.bias && vec_ok<VPL>(a.bias, E))
            load_run<VPL, true>(a.bias, lane, E, 0.0f, bias);
        else if (a.bias)
            load_run<VPL, false>(a.bias, lane, E, 0.0f, bias);
        else
#pragma unroll
            for (int v = 0; v < VPL; ++v) bias[v] = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            score[v] = cand[v] ? 1.0f / (1.0f + expf(-key[v])) : 0.0f;
            key[v] = cand[v] ? score[v] + bias[v] : -INFINITY;
        }
    }

    if (a.G > 1) {
        const int per = E / a.G;
        const bool two = a.bias != nullptr && per >= 2;  // group score: two largest keys, or the largest
        const float2 none{-INFINITY, -INFINITY};
        const int seg = per / VPL;  // lanes per group, when a group is whole lanes
        if (per % VPL == 0 && seg <= kWave && (seg & (seg - 1)) == 0) {
            // the lane's (largest, second) pair, then a segmented reduction
            // over the group's `seg` lanes leaves the group's pair in its
            // last lane
            float2 p = none;
#pragma unroll
            for (int v = 0; v < VPL; ++v)
                if (cand[v]) p = merge_top2(p, float2{key[v], -INFINITY});
            if (seg >= 2) p = dpp_step<0x111, 0xF>(p, none, merge_top2);   // row_shr:1
            if (seg >= 4) p = dpp_step<0x112, 0xF>(p, none, merge_top2);   // row_shr:2
            if (seg >= 8) p = dpp_step<0x114, 0xF>(p, none, merge_top2);   // row_shr:4
            if (seg >= 16) p = dpp_step<0x118, 0xF>(p, none, merge_top2);  // row_shr:8
            if (seg >= 32) p = dpp_step<0x142, 0xA>(p, none, merge_top2);  // row_bcast:15
            if (seg >= 64) p = dpp_step<0x143, 0xC>(p, none, merge_top2);  // row_bcast:31
            // the TG best groups, each named by its last lane (in group order)
            uint32_t gkey[1] = {ordered_bits(two ? p.x + p.y : p.x)};
            bool gok[1] = {(lane & (seg - 1)) == seg - 1 && VPL * lane < E};
            const bool was_end = gok[0];
            for (int r = 0; r < a.TG; ++r) take_first_max(gkey, gok, lane);
            // selected: a group end that is no longer a candidate
            const uint64_t kept = __ballot(was_end && !gok[0]);
            const bool mine = (kept >> (lane | (seg - 1))) & 1ull;
#pragma unroll
            for (int v = 0; v < VPL; ++v) cand[v] = cand[v] && mine;
        } else {
            // other group sizes: one wave reduction per group; group g's score
            // lands in lane g (G <= 64)
            int grp[VPL];
#pragma unroll
            for (int v = 0; v < VPL; ++v) grp[v] = (VPL * lane + v) / per;
            float my_gscore = -INFINITY;
            for (int g = 0; g < a.G; ++g) {
                float2 top = none;
#pragma unroll
                for (int v = 0; v < VPL; ++v)
                    if (cand[v] && grp[v] == g) top = merge_top2(top, float2{key[v], -INFINITY});
                top = wave_reduce_to_lane63(top, none, merge_top2);
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
        const int owner = e_sel / VPL;
        const int v_sel = e_sel - owner * VPL;
        float s_mine = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (v == v_sel) s_mine = score[v];
        const float s_sel = __uint_as_float(readlane_u32(__float_as_uint(s_mine), owner & (kWave - 1)));
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
